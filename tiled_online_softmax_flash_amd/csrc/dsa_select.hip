// Sparse index selection on gfx950: the operation of the onnx-runtime-ep-cuda page
// `src/kernels/dsa_index_select.rs` (module documentation; "Determinism / bit-parity").
//
// Kernels on the caller's stream:
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
//   * selection, in a row's chunks of 2048 positions, one 256-thread workgroup per chunk, so
//     that a decode step's few rows still spread over the chip.  keep = min(#allowed, top_k).
//     The keep-th largest key is found exactly by three radix passes (digits of 11, 11 and 10
//     bits), one kernel each:
//     every workgroup adds its chunk's histogram of the current digit (keys that match the
//     digits found so far) into the row's histogram in the workspace, and the next pass's
//     workgroups each read the finished histograms back to find the digits so far.  A count
//     kernel then gives every chunk its keys above and equal to the threshold, and a write
//     kernel places them: every key above the threshold, and the first keys equal to it, as
//     many as the rank left over (ties go to the lower position), in ascending position order,
//     each chunk's slots following from the counts of the chunks before it.  The rest of the
//     row is -1.  The scoring kernel clears the row's histograms, so a call needs no memset.
// The kernels compute in float32 like the page's; the selection is integer-exact.
#include <hip/hip_runtime.h>

#include <cstdint>

#include "dsa_kernels.h"

namespace dsa {

constexpr int kScoreThreads = 256;

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
    // the row's selection histograms and counters start from zero (the first tile clears them;
    // the selection kernels run after this kernel)
    if ((int64_t)blockIdx.x == row * tiles)
        for (int i = threadIdx.x; i < kAuxInts; i += kScoreThreads) p.aux[row * kAuxInts + i] = 0;
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

// ---- selection, split over chunks of a row
constexpr int kSelThreads = 256;
constexpr int kSelChunk = kSelChunkKeys;          // positions per workgroup: 8 per thread
constexpr int kKeysPerThread = kSelChunk / kSelThreads;

// The key is found in three radix passes over digits of 11, 11 and 10 bits (most significant
// first).  Per-row auxiliary words after the keys in the workspace (kAuxInts per row): the three
// passes' histograms (2048, 2048 and 1024 words), then the allowed count, the threshold key and
// the ties to take.  Then per chunk of every row: its keys above and equal to the threshold.
constexpr int kPasses = 3;
constexpr int kMaxBins = 2048;
__host__ __device__ constexpr int pass_bits(int q) { return q < 2 ? 11 : 10; }
__host__ __device__ constexpr int pass_shift(int q) { return q == 0 ? 21 : (q == 1 ? 10 : 0); }
__host__ __device__ constexpr int pass_hist(int q) { return q == 0 ? 0 : (q == 1 ? 2048 : 4096); }
constexpr int kAuxAllowed = 5120, kAuxThr = 5121, kAuxTies = 5122;
static_assert(kAuxTies < kAuxInts, "per-row words");

__host__ __device__ __forceinline__ int64_t sel_chunks(int64_t T) { return (T + kSelChunk - 1) / kSelChunk; }

// The digit of pass q that holds the rank-th largest key (rank >= 1, among the keys that the
// histogram counts): the largest digit whose count of keys with this digit or a larger one
// reaches rank.  *above gets the count of keys with a larger digit.  Thread i sums digits
// nb-1-DPT*i down to nb-DPT*(i+1); a prefix over the threads finds the thread whose run holds
// the crossing, which walks its digits.  All 256 threads call it (barriers); every thread gets
// the result.
__device__ __forceinline__ int find_digit(const int* hist, int nb, int rank, int* wsum, int* pick, int* above) {
    const int tid = threadIdx.x;
    const int dpt = nb / kSelThreads;
    const int hi = nb - 1 - dpt * tid;
    int c[kMaxBins / kSelThreads];
    int cnt = 0;
#pragma unroll
    for (int j = 0; j < kMaxBins / kSelThreads; ++j) {
        c[j] = j < dpt ? hist[hi - j] : 0;
        cnt += c[j];
    }
    int total;
    const int cum = block_inclusive_sum<kSelThreads>(cnt, wsum, &total);
    if (cum >= rank && cum - cnt < rank) {
        int run = cum - cnt;
#pragma unroll
        for (int j = 0; j < kMaxBins / kSelThreads; ++j) {
            if (j < dpt && run < rank && run + c[j] >= rank) {
                pick[0] = hi - j;
                pick[1] = run;
            }
            run += c[j];
        }
    }
    __syncthreads();
    const int digit = pick[0];
    *above = pick[1];
    __syncthreads();
    return digit;
}

// Keys found so far: the digits of passes 0 .. npass-1 (in their bits of *prefix) and the rank
// left among the keys that match them.  Returns keep (0: nothing is selected).
__device__ __forceinline__ int64_t sel_state(const DsaParams& p, const int* aux, int npass, uint32_t* prefix,
                                             int* rank, int* wsum, int* pick) {
    const int64_t allowed = aux[kAuxAllowed];
    const int64_t keep = allowed < p.top_k ? allowed : p.top_k;
    *prefix = 0u;
    *rank = (int)keep;
    if (keep == 0) return 0;
    for (int q = 0; q < npass; ++q) {
        int above;
        const int digit = find_digit(aux + pass_hist(q), 1 << pass_bits(q), *rank, wsum, pick, &above);
        *rank -= above;
        *prefix |= (uint32_t)digit << pass_shift(q);
    }
    return keep;
}

// Radix pass PASS over one chunk: the chunk's histogram of digit PASS among the keys that match
// the digits found so far, added into the row's histogram.  Pass 0 also counts the allowed
// positions (keys of removed positions are 0, below every allowed key; keep <= #allowed, so they
// never reach the threshold).
template <int PASS>
__global__ void __launch_bounds__(kSelThreads) dsa_pass_kernel(const DsaParams p) {
    constexpr int NB = 1 << pass_bits(PASS);
    constexpr int shift = pass_shift(PASS);
    constexpr uint32_t hi_mask = PASS == 0 ? 0u : (0xffffffffu << ((shift + pass_bits(PASS)) & 31));
    __shared__ int hist[NB];
    __shared__ int wsum[kSelThreads / 64];
    __shared__ int pick[2];
    const int tid = threadIdx.x;
    const int64_t T = p.key_seq;
    const int64_t nch = sel_chunks(T);
    const int64_t row = (int64_t)blockIdx.x / nch;
    const int64_t ch = (int64_t)blockIdx.x - row * nch;
    int* aux = p.aux + row * kAuxInts;
    const uint32_t* keys = p.keys + row * T;
    // the chunk's keys are requested first, so that their latency overlaps the histogram reads
    uint32_t kk[kKeysPerThread];
#pragma unroll
    for (int j = 0; j < kKeysPerThread; ++j) {
        const int64_t t = ch * kSelChunk + j * kSelThreads + tid;
        kk[j] = t < T ? keys[t] : 0u;
    }
    uint32_t prefix = 0u;
    int rank = 0;
    if (PASS > 0 && sel_state(p, aux, PASS, &prefix, &rank, wsum, pick) == 0) return;
#pragma unroll
    for (int i = tid; i < NB; i += kSelThreads) hist[i] = 0;
    __syncthreads();
    int allowed = 0;
#pragma unroll
    for (int j = 0; j < kKeysPerThread; ++j) {
        if (ch * kSelChunk + j * kSelThreads + tid < T) {
            const uint32_t k = kk[j];
            if (PASS == 0) allowed += k != 0u;
            if ((k & hi_mask) == prefix) atomicAdd(&hist[(k >> shift) & (uint32_t)(NB - 1)], 1);
        }
    }
    __syncthreads();
#pragma unroll
    for (int i = tid; i < NB; i += kSelThreads)
        if (hist[i] != 0) atomicAdd(&aux[pass_hist(PASS) + i], hist[i]);
    if (PASS == 0) {
        int total;
        block_inclusive_sum<kSelThreads>(allowed, wsum, &total);
        if (tid == 0 && total != 0) atomicAdd(&aux[kAuxAllowed], total);
    }
}

// The threshold (the keep-th largest key) and the ties to take from the three finished
// histograms; each chunk's keys above and equal to it.
__global__ void __launch_bounds__(kSelThreads) dsa_count_kernel(const DsaParams p) {
    __shared__ int wsum[kSelThreads / 64];
    __shared__ int pick[2];
    const int tid = threadIdx.x;
    const int64_t T = p.key_seq;
    const int64_t nch = sel_chunks(T);
    const int64_t row = (int64_t)blockIdx.x / nch;
    const int64_t ch = (int64_t)blockIdx.x - row * nch;
    int* aux = p.aux + row * kAuxInts;
    const uint32_t* keys = p.keys + row * T;
    uint32_t kk[kKeysPerThread];   // requested before the histograms are read
#pragma unroll
    for (int j = 0; j < kKeysPerThread; ++j) {
        const int64_t t = ch * kSelChunk + j * kSelThreads + tid;
        kk[j] = t < T ? keys[t] : 0u;
    }
    uint32_t thr;
    int ties;
    if (sel_state(p, aux, kPasses, &thr, &ties, wsum, pick) == 0) return;
    // (positions past T hold 0 here, which is below the threshold, an allowed key)
    int gt = 0, eq = 0;
#pragma unroll
    for (int j = 0; j < kKeysPerThread; ++j) {
        gt += kk[j] > thr;
        eq += kk[j] == thr;
    }
    int gt_all, eq_all;
    block_inclusive_sum<kSelThreads>(gt, wsum, &gt_all);
    block_inclusive_sum<kSelThreads>(eq, wsum, &eq_all);
    if (tid == 0) {
        p.counts[2 * (row * nch + ch)] = gt_all;
        p.counts[2 * (row * nch + ch) + 1] = eq_all;
        if (ch == 0) {
            aux[kAuxThr] = (int)thr;
            aux[kAuxTies] = ties;
        }
    }
}

// Output of one chunk: thread i owns positions [8 i, 8 i + 8) of the chunk.  The chunks before
// it give the chunk's first output slot and the ties left for it; block prefix sums give each
// thread the ties it may take (the lowest positions first) and its first slot; it writes its
// winners in position order.  The slots past keep are -1 (spread over the row's chunks).
__global__ void __launch_bounds__(kSelThreads) dsa_write_kernel(const DsaParams p) {
    __shared__ int wsum[kSelThreads / 64];
    const int tid = threadIdx.x;
    const int64_t T = p.key_seq;
    const int64_t nch = sel_chunks(T);
    const int64_t row = (int64_t)blockIdx.x / nch;
    const int64_t ch = (int64_t)blockIdx.x - row * nch;
    const int* aux = p.aux + row * kAuxInts;
    const uint32_t* keys = p.keys + row * T;
    int64_t* out = p.out + row * p.top_k;
    // the chunk's keys are requested before the row's words and counts are read
    const int64_t t0 = ch * kSelChunk + (int64_t)tid * kKeysPerThread;
    uint32_t k8[kKeysPerThread];
#pragma unroll
    for (int j = 0; j < kKeysPerThread; ++j) k8[j] = t0 + j < T ? keys[t0 + j] : 0u;
    const int64_t allowed = aux[kAuxAllowed];
    const int64_t keep = allowed < p.top_k ? allowed : p.top_k;
    for (int64_t s = keep + ch * kSelThreads + tid; s < p.top_k; s += nch * kSelThreads) out[s] = -1;
    if (keep == 0) return;
    const uint32_t thr = (uint32_t)aux[kAuxThr];
    const int ties_needed = aux[kAuxTies];
    // keys above and equal to the threshold in the chunks before this one
    int gt_b = 0, eq_b = 0;
    for (int64_t c = tid; c < ch; c += kSelThreads) {
        gt_b += p.counts[2 * (row * nch + c)];
        eq_b += p.counts[2 * (row * nch + c) + 1];
    }
    int gt_before, eq_before;
    block_inclusive_sum<kSelThreads>(gt_b, wsum, &gt_before);
    block_inclusive_sum<kSelThreads>(eq_b, wsum, &eq_before);
    const int ties_left = ties_needed - eq_before;   // ties this chunk and later ones may take
    const int64_t slot0 = (int64_t)gt_before + (eq_before < ties_needed ? eq_before : ties_needed);
    int gt_n = 0, eq_n = 0;
#pragma unroll
    for (int j = 0; j < kKeysPerThread; ++j) {
        gt_n += k8[j] > thr;
        eq_n += k8[j] == thr;
    }
    int total;
    const int eq_in = block_inclusive_sum<kSelThreads>(eq_n, wsum, &total) - eq_n;
    int my_ties = ties_left - eq_in;
    my_ties = my_ties < 0 ? 0 : (my_ties > eq_n ? eq_n : my_ties);
    const int sel = gt_n + my_ties;
    int64_t slot = slot0 + block_inclusive_sum<kSelThreads>(sel, wsum, &total) - sel;
    int ties_taken = 0;
#pragma unroll
    for (int j = 0; j < kKeysPerThread; ++j) {
        bool take = k8[j] > thr;
        if (k8[j] == thr && ties_taken < my_ties) {
            take = true;
            ++ties_taken;
        }
        if (take) {
            if (slot < keep) out[slot] = t0 + j;   // exactly keep are taken
            ++slot;
        }
    }
}

// key_seq == 0: every row is -1.
__global__ void __launch_bounds__(kSelThreads) dsa_fill_kernel(const DsaParams p) {
    int64_t* out = p.out + (int64_t)blockIdx.x * p.top_k;
    for (int64_t s = threadIdx.x; s < p.top_k; s += kSelThreads) out[s] = -1;
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
    if (p.key_seq == 0) {
        hipLaunchKernelGGL(dsa_fill_kernel, dim3((unsigned)rows), dim3(kSelThreads), 0, s, p);
        return hipGetLastError();
    }
    hipError_t e = dtype == 0 ? launch_score<float>(p, s)
                              : (dtype == 1 ? launch_score<_Float16>(p, s) : launch_score<uint16_t>(p, s));
    if (e != hipSuccess) return e;
    const dim3 grid((unsigned)(rows * sel_chunks(p.key_seq)));
    static_assert(kPasses == 3, "one launch per pass");
    hipLaunchKernelGGL(dsa_pass_kernel<0>, grid, dim3(kSelThreads), 0, s, p);
    hipLaunchKernelGGL(dsa_pass_kernel<1>, grid, dim3(kSelThreads), 0, s, p);
    hipLaunchKernelGGL(dsa_pass_kernel<2>, grid, dim3(kSelThreads), 0, s, p);
    hipLaunchKernelGGL(dsa_count_kernel, grid, dim3(kSelThreads), 0, s, p);
    hipLaunchKernelGGL(dsa_write_kernel, grid, dim3(kSelThreads), 0, s, p);
    return hipGetLastError();
}

}  // namespace dsa
