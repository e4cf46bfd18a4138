// Launch parameters shared by the host dispatcher and the attention kernels.
#pragma once

#include <stdint.h>

namespace fa {

// Rows per workgroup of the 16-bit kernel of fa_fwd16.h: four 64-lane waves of 32 query rows each.
constexpr int kBlockRows = 128;
constexpr int kWaveRows = 32;
constexpr int kThreads = 256;
// fp32 kernel for head dims up to 128 (fa_fwd32.h): 64 rows per workgroup, four waves of 16 rows
constexpr int kF32Rows = 64;
constexpr int kF32SplitRows = 32;   // fp32 workgroups whose key range is split in two halves
// The key-split form is not built for masked head-dim-128 problems (it would spill registers at
// three waves per SIMD).
constexpr bool fwd32_split_built(int dp, bool masked) { return !(masked && dp > 64); }
// fp32 kernel for head dims 129..384 (fa_fwd32w.h): 64 rows per workgroup, eight waves
constexpr int kWideRows = 64;
constexpr int kWideThreads = 512;

// Lazy rescaling threshold, in log2 units: the running row maximum is only moved when a
// new score exceeds it by more than this, so unnormalised probabilities stay <= 2^8.
constexpr float kRescaleLog2 = 8.0f;
// The speculative softmax of the ring kernel lets weights grow to 2^14 against a stale running
// maximum before it moves the maximum (a lane's sum of 16 weights above kSpecBound); 2^14 keeps
// every weight finite in f16 (largest finite value 65504) and in fp32 sums.
constexpr float kSpecBound = 16384.0f;
// Largest exponent offset |m k| the speculative softmax folds into one multiply-add (its rounding
// error, at most 2^12 * 2^-24, is negligible); rows beyond it take the exact fix-up.
constexpr float kSpecOffsetMax = 4096.0f;

struct FwdParams {
    const void* q;               // [batch, heads, sq, dim]
    const void* k;               // [batch, kv_heads, kv_capacity, dim]
    const void* v;               // [batch, kv_heads, kv_capacity, dim]
    const void* mask;            // [mask_planes, sq, sk] or null
    const int32_t* total_lengths;
    const int32_t* past_lengths;
    void* out;
    int batch, heads, kv_heads, sq, sk, dim, group;
    int causal, window, mask_planes;
    int q_tiles;                 // ceil(sq / rows per workgroup of the kernel)
    int pairs;                   // batch * q_tiles: (batch, query tile) pairs
    int xcd_groups;              // 1: group-major workgroup order (see decode_work)
    int items_per_xcd;           // work items per XCD (the non-persistent grid / 8)
    int vec_kv;                  // q/k/v rows move in 16-byte pieces (dim and pointers allow it)
    int vec_mask;                // mask rows move in 16-byte pieces
    int vec_out;                 // output rows move in 4-element pieces
    int raw_scores;              // 1: scores stay raw dot products, scale folded into kfac
    int mask_in_acc;             // 1: Q is pre-multiplied by the (power-of-two) scale and the
                                 //    ring kernel's Q.K products start from the mask values
    float scale;
    float softcap;
    float cap_y;                 // scale / softcap: dot product -> tanh argument
    float kfac;                  // log2(e) per unit of the tracked score
    // softcap without a mask: the base-2 exponent kfac * tanh(cap_y * s) of a dot product s as
    // s (tc_b1 + s^2 (tc_b3 + tc_b5 s^2)), the odd series of tanh to fifth order, for |s| < tc_slim
    float tc_b1, tc_b3, tc_b5, tc_slim;
    int64_t kv_capacity;
    int64_t o_stride_b, o_stride_h, o_stride_i;  // output strides in elements
};

// Split-key (decode) launches: the workspace and how the key range is cut (fa_splitkv.h).
struct SplitParams {
    float* ws_o;     // [num_splits][batch * kv_heads][32][dim] unnormalised outputs
    float* ws_m;     // [num_splits][batch * kv_heads][32] running maxima (tracked units; -inf: no key)
    float* ws_l;     // [num_splits][batch * kv_heads][32] denominators
    int num_splits;  // a multiple of 4 (one span per wave, four waves per workgroup)
    int span;        // keys per span, a multiple of 32
    int rows;        // query rows per (batch, KV head) group: (heads / kv_heads) * sq <= 32
};

}  // namespace fa
