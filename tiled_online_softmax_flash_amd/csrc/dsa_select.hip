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
//     A workgroup covers 256 positions of one query row; the row's query is staged in LDS as
//     float32 and read by broadcast loads.
//   * dsa_select_kernel: one 1024-thread workgroup per query row, the row's keys cached in LDS
//     (up to 32768 positions).  keep = min(#allowed, top_k).  The keep-th largest key is found
//     exactly by four 8-bit radix passes (LDS histogram, block-wide descending prefix over the
//     256 digits).  Positions are then compacted in ascending order, each thread owning a
//     contiguous run of positions and two block prefix sums placing its winners: every key
//     above the threshold, and the first keys equal to it, as many as the rank left over (ties
//     go to the lower position).  The rest of the row is -1.
// The kernels compute in float32 like the page's; the selection is integer-exact.
#include <hip/hip_runtime.h>

#include <cstdint>

#include "dsa_kernels.h"

namespace dsa {

constexpr int kScoreThreads = 256;
constexpr int kSelectThreads = 1024;

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

// Head chunk staged in LDS: the query rows of up to kQStage / DMAX heads as float32.
constexpr int kQStage = 8192;

// The file is compiled with -ffp-contract=off, and the pragma keeps the kernel's products and
// sums apart even where that flag is missing.  DMAX (32, 64 or 128) bounds the head dim held in
// registers.
//
// Dims d >= head_dim are padded with zeros on both sides, which leaves every sum bit-identical:
// a dot product starts at +0 and can never become -0 (x + -x is +0 under round-to-nearest), so
// adding the +0 products of the padding changes nothing, NaN and infinities included.
template <typename T, int DMAX>
__global__ void __launch_bounds__(kScoreThreads) dsa_score_kernel(const DsaParams p) {
#pragma clang fp contract(off)
    __shared__ __attribute__((aligned(16))) float qs[kQStage];
    __shared__ float wq[kQStage / DMAX];
    constexpr int HC = kQStage / DMAX;   // heads per staged chunk
    const int64_t tiles = (p.key_seq + kScoreThreads - 1) / kScoreThreads;
    const int64_t row = (int64_t)blockIdx.x / tiles;
    const int64_t t = ((int64_t)blockIdx.x - row * tiles) * kScoreThreads + threadIdx.x;
    const bool inside = t < p.key_seq;
    const int64_t cell = row * p.key_seq + (inside ? t : 0);
    const float bias = inside ? p.bias[cell] : 0.0f;
    const bool active = inside && bias > -1e30f;
    const int D = (int)p.head_dim;
    const int64_t b = row / p.q_seq;
    const T* krow = (const T*)p.key + (b * p.key_seq + (inside ? t : 0)) * p.head_dim;
    // the key row into registers, all loads in flight together: 16-byte loads when the rows are
    // 16-byte aligned and exactly DMAX long, else element loads at clamped (in-range) indices
    float kv[DMAX];
#pragma unroll
    for (int d = 0; d < DMAX; ++d) kv[d] = 0.0f;
    // (no heads: the score is the bias alone and key may be NULL, so nothing is loaded)
    const bool load = active && p.heads > 0;
    const bool vec = D == DMAX && ((uintptr_t)p.key % 16) == 0 && (DMAX * sizeof(T)) % 16 == 0;
    if (load && vec) {
        constexpr int PER = 16 / (int)sizeof(T);   // elements per 16-byte load
        uint4 raw[DMAX / PER];
#pragma unroll
        for (int c = 0; c < DMAX / PER; ++c) raw[c] = *(const uint4*)(krow + c * PER);
#pragma unroll
        for (int c = 0; c < DMAX / PER; ++c) {
            const T* e = (const T*)&raw[c];
#pragma unroll
            for (int j = 0; j < PER; ++j) kv[c * PER + j] = to_f32<T>(e[j]);
        }
    } else if (load && D > 0) {
        T raw[DMAX];
#pragma unroll
        for (int d = 0; d < DMAX; ++d) raw[d] = krow[d < D ? d : D - 1];
#pragma unroll
        for (int d = 0; d < DMAX; ++d) kv[d] = d < D ? to_f32<T>(raw[d]) : 0.0f;
    }
    const T* qrow = (const T*)p.query + row * p.heads * p.head_dim;
    const T* wrow = (const T*)p.weights + row * p.heads;
    float total = 0.0f;
    for (int64_t h0 = 0; h0 < p.heads; h0 += HC) {
        const int nh = (int)(p.heads - h0 < HC ? p.heads - h0 : HC);
        __syncthreads();   // the previous chunk's reads are done
        // all of this thread's loads in flight together, at clamped (in-range) indices
        constexpr int PER_T = kQStage / kScoreThreads;
        T raw[PER_T];
        if (D > 0) {
#pragma unroll
            for (int j = 0; j < PER_T; ++j) {
                const int i = (int)threadIdx.x + j * kScoreThreads;
                const int hh = i / DMAX, dd = i - hh * DMAX;
                const int64_t idx = (hh < nh && dd < D) ? (h0 + hh) * p.head_dim + dd : 0;
                raw[j] = qrow[idx];
            }
        } else {
#pragma unroll
            for (int j = 0; j < PER_T; ++j) raw[j] = (T)0;
        }
#pragma unroll
        for (int j = 0; j < PER_T; ++j) {
            const int i = (int)threadIdx.x + j * kScoreThreads;
            const int hh = i / DMAX, dd = i - hh * DMAX;
            qs[i] = (hh < nh && dd < D) ? to_f32<T>(raw[j]) : 0.0f;
        }
        for (int i = threadIdx.x; i < nh; i += kScoreThreads)
            wq[i] = to_f32<T>(wrow[h0 + i]) * p.weights_scale;   // weight times weights_scale
        __syncthreads();
        if (active) {
            for (int hh = 0; hh < nh; ++hh) {
                const float* qh = qs + hh * DMAX;
                float dot = 0.0f;
                // query reads (same address on every lane) requested two groups ahead of use
                float4 qa = *(const float4*)(qh);
                float4 qb = *(const float4*)(qh + 4);
#pragma unroll
                for (int d = 0; d < DMAX; d += 4) {
                    const float4 q4 = qa;
                    qa = qb;
                    if (d + 8 < DMAX) qb = *(const float4*)(qh + d + 8);
                    dot = dot + q4.x * kv[d];
                    dot = dot + q4.y * kv[d + 1];
                    dot = dot + q4.z * kv[d + 2];
                    dot = dot + q4.w * kv[d + 3];
                }
                const float scaled = p.scale * dot;
                const float relu = scaled > 0.0f ? scaled : 0.0f;   // NaN gives 0
                total = total + relu * wq[hh];
            }
        }
    }
    if (!inside) return;
    float score = total + bias;
    if (score != score) score = __uint_as_float(0x7fc00000u);
    p.keys[cell] = active ? order_key(score) : 0u;
}

__device__ __forceinline__ int lane_id() { return __builtin_amdgcn_mbcnt_hi(~0u, __builtin_amdgcn_mbcnt_lo(~0u, 0u)); }

// Inclusive prefix sum over the NT threads of the workgroup (thread order); `tot` gets the
// total.  `wsum` is NT / 64 ints of LDS.  Contains barriers: every thread must call it.
template <int NT>
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
    int before = 0, all = 0;
#pragma unroll
    for (int w = 0; w < NT / 64; ++w) {
        before += w < wave ? wsum[w] : 0;
        all += wsum[w];
    }
    __syncthreads();
    *tot = all;
    return before + x;
}

// Rows of at most kKeyCache positions are read from the workspace once and kept in LDS for
// the radix passes and the compaction, with one padding word after every 32 keys so that
// threads walking contiguous 32-key runs hit distinct banks.
constexpr int kKeyCache = 32768;
__device__ __forceinline__ int64_t cache_index(int64_t t) { return t + (t >> 5); }

template <bool CACHE>
__global__ void __launch_bounds__(kSelectThreads) dsa_select_kernel(const DsaParams p) {
    constexpr int NT = kSelectThreads;
    __shared__ uint32_t kc[CACHE ? kKeyCache + kKeyCache / 32 : 1];
    __shared__ int hist[256];
    __shared__ int wsum[NT / 64];
    __shared__ int pick[2];
    const int tid = threadIdx.x;
    const int64_t row = blockIdx.x;
    const int64_t T = p.key_seq;
    const uint32_t* gkeys = p.keys + row * T;
    int64_t* out = p.out + row * p.top_k;
    auto key_at = [&](int64_t t) -> uint32_t { return CACHE ? kc[cache_index(t)] : gkeys[t]; };

    // allowed positions of the row (and the row into LDS)
    int local = 0;
#pragma unroll 4
    for (int64_t t = tid; t < T; t += NT) {
        const uint32_t k = gkeys[t];
        if (CACHE) kc[cache_index(t)] = k;
        local += k != 0u;
    }
    int n_allowed;
    block_inclusive_sum<NT>(local, wsum, &n_allowed);   // its barriers also publish kc
    const int64_t keep = (int64_t)n_allowed < p.top_k ? (int64_t)n_allowed : p.top_k;
    for (int64_t s = keep + tid; s < p.top_k; s += NT) out[s] = -1;
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
        if (tid < 256) hist[tid] = 0;
        __syncthreads();
#pragma unroll 4
        for (int64_t t = tid; t < T; t += NT) {
            const uint32_t k = key_at(t);
            if ((k & hi_mask) == prefix) atomicAdd(&hist[(k >> shift) & 255u], 1);
        }
        __syncthreads();
        // thread i < 256 holds digit 255 - i: an inclusive prefix in thread order is the count
        // of keys with this digit or a larger one
        const int cnt = tid < 256 ? hist[255 - tid] : 0;
        int total;
        const int cum = block_inclusive_sum<NT>(cnt, wsum, &total);
        // exactly one digit (from the top) has a cumulative count that first reaches `rank`
        // (the keys that match `prefix` number at least `rank`)
        if (tid < 256 && cum >= rank && cum - cnt < rank) {
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

    // ascending compaction: thread i owns the contiguous positions [i C, (i + 1) C).  It counts
    // its keys above and equal to the threshold; block prefix sums give it the ties it may take
    // (the lowest positions first) and its first output slot; it then writes its winners in
    // position order.
    const int64_t C = (T + NT - 1) / NT;
    const int64_t c0 = (int64_t)tid * C;
    const int64_t c1 = c0 + C < T ? c0 + C : T;
    int gt_n = 0, eq_n = 0;
    for (int64_t t = c0; t < c1; ++t) {
        const uint32_t k = key_at(t);
        gt_n += k > thr;
        eq_n += k == thr;
    }
    int total;
    const int eq_before = block_inclusive_sum<NT>(eq_n, wsum, &total) - eq_n;
    int my_ties = ties_needed - eq_before;
    my_ties = my_ties < 0 ? 0 : (my_ties > eq_n ? eq_n : my_ties);
    const int sel = gt_n + my_ties;
    int64_t slot = block_inclusive_sum<NT>(sel, wsum, &total) - sel;
    int ties_taken = 0;
    for (int64_t t = c0; t < c1; ++t) {
        const uint32_t k = key_at(t);
        bool take = k > thr;
        if (k == thr && ties_taken < my_ties) {
            take = true;
            ++ties_taken;
        }
        if (take) {
            if (slot < keep) out[slot] = t;   // exactly keep are taken
            ++slot;
        }
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
    if (p.key_seq <= kKeyCache)
        hipLaunchKernelGGL(dsa_select_kernel<true>, dim3((unsigned)rows), dim3(kSelectThreads), 0, s, p);
    else
        hipLaunchKernelGGL(dsa_select_kernel<false>, dim3((unsigned)rows), dim3(kSelectThreads), 0, s, p);
    return hipGetLastError();
}

}  // namespace dsa
