// Parameters and launch of the sparse index-selection kernels (dsa_select.hip).
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>

namespace dsa {

struct DsaParams {
    const void* query;     // [batch, q_seq, heads, head_dim] of the input dtype
    const void* key;       // [batch, key_seq, head_dim]
    const void* weights;   // [batch, q_seq, heads]
    const float* bias;     // [batch, 1, q_seq, key_seq]
    uint32_t* keys;        // workspace: [batch * q_seq, key_seq] order keys (0 = removed)
    int* aux;              // workspace, after the keys: [batch * q_seq, kAuxInts] per-row words
    int* counts;           // workspace, after aux: [batch * q_seq, chunks] per-chunk counts
    int* cand;             // workspace, after the counts: [batch * q_seq, 2, key_seq] candidates
    int64_t* out;          // [batch, 1, q_seq, top_k]
    int64_t batch, q_seq, heads, head_dim, key_seq, top_k;
    float scale, weights_scale;
};

// Selection chunks and per-row workspace words (see dsa_select.hip): the workspace holds the
// keys (4 bytes per cell), then kAuxInts words per row, then one word per chunk of
// kSelChunkKeys positions of every row, then two words per cell (candidate keys and positions).
constexpr int kAuxInts = 4104;
constexpr int kSelChunkKeys = 2048;

// dtype 0 f32, 1 f16, 2 bf16; head_dim <= 128.  Enqueues the scoring kernel (when key_seq > 0)
// and the selection kernels (when there is a row).
hipError_t launch_index_select(const DsaParams& p, int dtype, hipStream_t s);

}  // namespace dsa
