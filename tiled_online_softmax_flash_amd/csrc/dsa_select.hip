// Sparse index selection on gfx950: the operation of the onnx-runtime-ep-cuda page
// `src/kernels/dsa_index_select.rs` (module documentation; "Determinism / bit-parity").
//
// Two kernels on the caller's stream:
//   * dsa_score_kernel: one thread per (query row, key position) cell.  It keeps its key row in
//     registers as float32 and forms, for every head in ascending order, the dot product over
//     the head dim in ascending order with every product and sum rounded on its own (no fused
//     multiply-add: the page fixes this order so that the device and the CPU reference agree bit
//     for bit), then ReLU(scale * dot) * (weight * weights_scale) summed over heads, plus the
//     bias.  A NaN result becomes the canonical quiet NaN.  It writes one 32-bit key per cell:
//     0 for a position the bias removes (bias <= -1e30), otherwise the score mapped to an
//     unsigned integer whose order is the IEEE-754 total order (never 0 for a canonical score).
//     A workgroup covers 256 positions of one query row, so the row's query and weights are
//     wave-uniform and come through scalar loads.
//   * dsa_select_kernel: one workgroup per query row.  keep = min(#allowed, top_k).  The keep-th
//     largest key is found exactly by four 8-bit radix passes (LDS histogram, block-wide
//     descending prefix over the 256 digits).  Positions are then compacted in ascending order,
//     256 at a time with ballot prefix counts: every key above the threshold, and the first
//     keys equal to it, as many as the rank left over (ties go to the lower position).  The
//     rest of the row is -1.
// The kernels compute in float32 like the page's; the selection is integer-exact.
#include <hip/hip_runtime.h>
#include <hip/hip_bf16.h>
#include <hip/hip_fp16.h>

#include <cstdint>

#include "dsa_kernels.h"

namespace dsa {

constexpr int kScoreThreads = 256;
constexpr int kSelectThreads = 256;

template <typename T>
__device__ __forceinline__ float to_f32(T x);
template <>
__device__ __forceinline__ float to_f32<float>(float x) { return x; }
template <>
__device__ __forceinline__ float to_f32<_Float16>(_Float16 x) { return (float)x; }
template <>
__device__ __forceinline__ float to_f32<uint16_t>(uint16_t x) {   // bfloat16 bits
    return __uint_as_float((uint32_t)x << 16);
}

__device__ __forceinline__ uint32_t order_key(float x) {
    const uint32_t u = __float_as_uint(x);
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// DMAX: head dims up to DMAX (32, 64 or 128) held in registers.
// The file is compiled with -ffp-contract=off, and the pragma keeps the kernel's products and
// sums apart even where that flag is missing.
template <typename T, int DMAX>
__global__ void __launch_bounds__(kScoreThreads) dsa_score_kernel(const DsaParams p) {
#pragma clang fp contract(off)
    const int64_t tiles = (p.key_seq + kScoreThreads - 1) / kScoreThreads;
    const int64_t row = (int64_t)blockIdx.x / tiles;
    const int64_t t = ((int64_t)blockIdx.x - row * tiles) * kScoreThreads + threadIdx.x;
    if (t >= p.key_seq) return;
    const int64_t cell = row * p.key_seq + t;
    const float bias = p.bias[cell];
    if (!(bias > -1e30f)) {
        p.keys[cell] = 0u;
        return;
    }
    const int64_t b = row / p.q_seq;
    const int D = (int)p.head_dim;
    const T* krow = (const T*)p.key + (b * p.key_seq + t) * p.head_dim;
    float kv[DMAX];
#pragma unroll
    for (int d = 0; d < DMAX; ++d) kv[d] = d < D ? to_f32<T>(krow[d]) : 0.0f;
    const T* qrow = (const T*)p.query + row * p.heads * p.head_dim;
    const T* wrow = (const T*)p.weights + row * p.heads;
    float total = 0.0f;
    for (int64_t h = 0; h < p.heads; ++h) {
        const T* qh = qrow + h * p.head_dim;
        float dot = 0.0f;
#pragma unroll
        for (int d = 0; d < DMAX; ++d) {
            if (d < D) {
                const float prod = to_f32<T>(qh[d]) * kv[d];
                dot = dot + prod;
            }
        }
        const float scaled = p.scale * dot;
        const float relu = scaled > 0.0f ? scaled : 0.0f;   // NaN gives 0
        const float wgt = to_f32<T>(wrow[h]) * p.weights_scale;
        total = total + relu * wgt;
    }
    float score = total + bias;
    if (score != score) score = __uint_as_float(0x7fc00000u);
    p.keys[cell] = order_key(score);
}

__device__ __forceinline__ int lane_id() { return __builtin_amdgcn_mbcnt_hi(~0u, __builtin_amdgcn_mbcnt_lo(~0u, 0u)); }

// number of set bits of a 64-lane ballot below this lane
__device__ __forceinline__ int prefix_below(uint64_t mask) {
    return (int)__builtin_amdgcn_mbcnt_hi((uint32_t)(mask >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)mask, 0u));
}

// Inclusive prefix sum over the 256 threads of the workgroup (thread order); `tot` gets the
// total.  `wsum` is 4 ints of LDS.  Contains barriers: every thread must call it.
__device__ __forceinline__ int block_inclusive_sum(int v, int* wsum, int* tot) {
    const int lane = lane_id();
    const int wave = threadIdx.x >> 6;
    int x = v;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
        const int y = __shfl_up(x, off, 64);
        if (lane >= off) x += y;
    }
    if (lane == 63) wsum[wave] = x;
    __syncthreads();
    int before = 0;
    for (int w = 0; w < wave; ++w) before += wsum[w];
    const int all = wsum[0] + wsum[1] + wsum[2] + wsum[3];
    __syncthreads();
    *tot = all;
    return before + x;
}

// Exclusive count of `flag` over lower threads of the workgroup; `tot` gets the total.
__device__ __forceinline__ int block_exclusive_count(bool flag, int* wsum, int* tot) {
    const int wave = threadIdx.x >> 6;
    const uint64_t m = __ballot(flag);
    if (lane_id() == 0) wsum[wave] = __popcll(m);
    __syncthreads();
    int before = 0;
    for (int w = 0; w < wave; ++w) before += wsum[w];
    const int all = wsum[0] + wsum[1] + wsum[2] + wsum[3];
    __syncthreads();
    *tot = all;
    return before + prefix_below(m);
}

__global__ void __launch_bounds__(kSelectThreads) dsa_select_kernel(const DsaParams p) {
    __shared__ int hist[256];
    __shared__ int wsum[4];
    __shared__ int pick[2];
    const int tid = threadIdx.x;
    const int64_t row = blockIdx.x;
    const int64_t T = p.key_seq;
    const uint32_t* keys = p.keys + row * T;
    int64_t* out = p.out + row * p.top_k;

    // allowed positions of the row
    int local = 0;
    for (int64_t t = tid; t < T; t += kSelectThreads) local += keys[t] != 0u;
    int n_allowed;
    block_inclusive_sum(local, wsum, &n_allowed);
    const int64_t keep = (int64_t)n_allowed < p.top_k ? (int64_t)n_allowed : p.top_k;
    for (int64_t s = keep + tid; s < p.top_k; s += kSelectThreads) out[s] = -1;
    if (keep == 0) return;

    // the keep-th largest key: four passes over 8-bit digits, most significant first.  Keys of
    // removed positions are 0, below every allowed key, and keep <= #allowed, so they never
    // reach the threshold.
    uint32_t prefix = 0u;
    int rank = (int)keep;   // 1-based rank among the keys that match `prefix`, largest first
#pragma unroll 1
    for (int pass = 0; pass < 4; ++pass) {
        const int shift = 24 - 8 * pass;
        const uint32_t hi_mask = pass == 0 ? 0u : (0xffffffffu << (shift + 8));
        hist[tid] = 0;
        __syncthreads();
        for (int64_t t = tid; t < T; t += kSelectThreads) {
            const uint32_t k = keys[t];
            if ((k & hi_mask) == prefix) atomicAdd(&hist[(k >> shift) & 255u], 1);
        }
        __syncthreads();
        // thread i holds digit 255 - i: an inclusive prefix in thread order is the count of
        // keys with this digit or a larger one
        const int cnt = hist[255 - tid];
        int total;
        const int cum = block_inclusive_sum(cnt, wsum, &total);
        // exactly one digit (from the top) has a cumulative count that first reaches `rank`
        // (the keys that match `prefix` number at least `rank`)
        if (cum >= rank && cum - cnt < rank) {
            pick[0] = 255 - tid;
            pick[1] = cum - cnt;   // keys with a larger digit
        }
        __syncthreads();
        const uint32_t digit = (uint32_t)pick[0];
        rank -= pick[1];
        prefix |= digit << shift;
        __syncthreads();
    }
    const uint32_t thr = prefix;
    const int ties_needed = rank;   // keys equal to the threshold to take, lowest positions first

    // ascending compaction, 256 positions at a time
    int64_t written = 0;
    int ties_taken = 0;
    for (int64_t base = 0; base < T && written < keep; base += kSelectThreads) {
        const int64_t t = base + tid;
        const uint32_t k = t < T ? keys[t] : 0u;
        const bool gt = k > thr;
        const bool eq = k == thr && t < T;
        int eq_total;
        const int eq_before = block_exclusive_count(eq, wsum, &eq_total);
        const bool take = gt || (eq && ties_taken + eq_before < ties_needed);
        int sel_total;
        const int sel_before = block_exclusive_count(take, wsum, &sel_total);
        if (take && written + sel_before < keep) out[written + sel_before] = t;   // exactly keep are taken
        written += sel_total;
        ties_taken += eq_total;
    }
}

template <typename T>
hipError_t launch_score(const DsaParams& p, hipStream_t s) {
    const int64_t tiles = (p.key_seq + kScoreThreads - 1) / kScoreThreads;
    const unsigned grid = (unsigned)(p.q_seq * p.batch * tiles);
    if (p.head_dim <= 32)
        hipLaunchKernelGGL((dsa_score_kernel<T, 32>), dim3(grid), dim3(kScoreThreads), 0, s, p);
    else if (p.head_dim <= 64)
        hipLaunchKernelGGL((dsa_score_kernel<T, 64>), dim3(grid), dim3(kScoreThreads), 0, s, p);
    else
        hipLaunchKernelGGL((dsa_score_kernel<T, 128>), dim3(grid), dim3(kScoreThreads), 0, s, p);
    return hipGetLastError();
}

hipError_t launch_index_select(const DsaParams& p, int dtype, hipStream_t s) {
    const int64_t rows = p.batch * p.q_seq;
    if (rows == 0) return hipSuccess;
    if (p.key_seq > 0) {
        hipError_t e = dtype == 0 ? launch_score<float>(p, s)
                                  : (dtype == 1 ? launch_score<_Float16>(p, s) : launch_score<uint16_t>(p, s));
        if (e != hipSuccess) return e;
    }
    hipLaunchKernelGGL(dsa_select_kernel, dim3((unsigned)rows), dim3(kSelectThreads), 0, s, p);
    return hipGetLastError();
}

}  // namespace dsa
