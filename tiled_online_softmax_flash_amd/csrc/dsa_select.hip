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
//     The keep-th largest key (the threshold) is found exactly from its digits of 11, 11 and 10
//     bits, in three kernels:
//       dsa_hist_kernel: every chunk adds its histogram of the top digit into the row's (and
//         its allowed count);
//       dsa_cand_kernel: every chunk reads the finished histogram back, finds the threshold's
//         top digit d0, stores its count of keys with a larger top digit, and appends its keys
//         with top digit d0 (the candidates, with their positions) to the row's list, counting
//         their second digits into the row's second histogram;
//       dsa_write_kernel: every chunk finds the threshold's second digit from that histogram and
//         its third among the row's candidates by itself, and from the stored counts and the
//         candidates' positions the keys above and equal to the threshold in the chunks before
//         it; it then places its winners: every key above the threshold, and the first keys
//         equal to it, as many as the rank left over (ties go to the lower position), in
//         ascending position order.
//     The rest of the row is -1.  The scoring kernel clears the row's histograms and counters,
//     so a call needs no memset.
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

// Inclusive prefix sum over the 64 lanes of a wave (all lanes active), with DPP moves: within
// each row of 16 lanes by shifts of 1, 2, 4 and 8 (lanes shifted in from outside the row read 0),
// then the last lane of row 0 added into row 1 and of row 2 into row 3 (row_bcast:15), then
// lane 31 into rows 2 and 3 (row_bcast:31).
__device__ __forceinline__ int wave_inclusive_sum(int x) {
    x += __builtin_amdgcn_update_dpp(0, x, 0x111, 0xf, 0xf, true);   // row_shr:1
    x += __builtin_amdgcn_update_dpp(0, x, 0x112, 0xf, 0xf, true);   // row_shr:2
    x += __builtin_amdgcn_update_dpp(0, x, 0x114, 0xf, 0xf, true);   // row_shr:4
    x += __builtin_amdgcn_update_dpp(0, x, 0x118, 0xf, 0xf, true);   // row_shr:8
    x += __builtin_amdgcn_update_dpp(0, x, 0x142, 0xa, 0xf, true);   // row_bcast:15, rows 1 and 3
    x += __builtin_amdgcn_update_dpp(0, x, 0x143, 0xc, 0xf, true);   // row_bcast:31, rows 2 and 3
    return x;
}

// Inclusive prefix sum over the NT threads of the workgroup (thread order); `tot` gets the
// total.  `wsum` is NT / 64 ints of LDS.  Contains barriers: every thread must call it.
template <int NT>
__device__ __forceinline__ int block_inclusive_sum(int v, int* wsum, int* tot) {
    const int lane = lane_id();
    const int wave = threadIdx.x >> 6;
    const int x = wave_inclusive_sum(v);
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

// Two inclusive prefix sums over the NT threads with one exchange between the waves; `w2` is
// NT / 64 pairs of ints of LDS.  Contains barriers: every thread must call it.
template <int NT>
__device__ __forceinline__ void block_inclusive_sum2(int a, int b, int (*w2)[2], int* pa, int* pb, int* ta, int* tb) {
    const int lane = lane_id();
    const int wave = threadIdx.x >> 6;
    const int xa = wave_inclusive_sum(a), xb = wave_inclusive_sum(b);
    if (lane == 63) {
        w2[wave][0] = xa;
        w2[wave][1] = xb;
    }
    __syncthreads();
    int ba = 0, bb = 0, aa = 0, ab = 0;
#pragma unroll
    for (int w = 0; w < NT / 64; ++w) {
        if (w < wave) {
            ba += w2[w][0];
            bb += w2[w][1];
        }
        aa += w2[w][0];
        ab += w2[w][1];
    }
    __syncthreads();
    *pa = ba + xa;
    *pb = bb + xb;
    *ta = aa;
    *tb = ab;
}

// ---- selection, split over chunks of a row
constexpr int kSelThreads = 256;
constexpr int kSelChunk = kSelChunkKeys;          // positions per workgroup: 8 per thread
constexpr int kKeysPerThread = kSelChunk / kSelThreads;

// The threshold key is found by digits of 11, 11 and 10 bits (most significant first).  Per-row
// auxiliary words after the keys in the workspace (kAuxInts per row): the histogram of the top
// digit (2048 words), then the allowed count, the candidate count, and the row's top digit,
// the rank left among the candidates and keep, as the candidate kernel found them, and from
// word kAuxH1 the histogram of the candidates' second digit (2048 words).  Then per
// chunk of every row: its keys with a larger top digit.  Then per row up to key_seq candidates
// (keys whose top digit is the threshold's) and, after them, their positions.
constexpr int kMaxBins = 2048;
__host__ __device__ constexpr int pass_bits(int q) { return q < 2 ? 11 : 10; }
__host__ __device__ constexpr int pass_shift(int q) { return q == 0 ? 21 : (q == 1 ? 10 : 0); }
constexpr int kAuxAllowed = 2048, kAuxCand = 2049, kAuxD0 = 2050, kAuxRank = 2051, kAuxKeep = 2052;
constexpr int kAuxH1 = 2056;
static_assert(kAuxKeep < kAuxH1 && kAuxH1 + (1 << 11) <= kAuxInts, "per-row words");

__host__ __device__ __forceinline__ int64_t sel_chunks(int64_t T) { return (T + kSelChunk - 1) / kSelChunk; }

// The digit of pass q that holds the rank-th largest key (rank >= 1, among the keys that the
// histogram counts): the largest digit whose count of keys with this digit or a larger one
// reaches rank.  *above gets the count of keys with a larger digit.  Thread i sums digits
// nb-1-DPT*i down to nb-DPT*(i+1); a prefix over the threads finds the thread whose run holds
// the crossing, which walks its digits.  All 256 threads call it (barriers); every thread gets
// the result.
// find_digit_counts takes thread i's counts c[j] = hist[nb - 1 - DPT*i - j] (0 for j >= DPT)
// already loaded.
__device__ __forceinline__ int find_digit_counts(const int (&c)[kMaxBins / kSelThreads], int nb, int rank, int* wsum,
                                                 int* pick, int* above) {
    const int tid = threadIdx.x;
    const int dpt = nb / kSelThreads;
    const int hi = nb - 1 - dpt * tid;
    int cnt = 0;
#pragma unroll
    for (int j = 0; j < kMaxBins / kSelThreads; ++j) cnt += c[j];
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
__device__ __forceinline__ int find_digit(const int* hist, int nb, int rank, int* wsum, int* pick, int* above) {
    const int dpt = nb / kSelThreads;
    const int hi = nb - 1 - dpt * (int)threadIdx.x;
    int c[kMaxBins / kSelThreads];
#pragma unroll
    for (int j = 0; j < kMaxBins / kSelThreads; ++j) c[j] = j < dpt ? hist[hi - j] : 0;
    return find_digit_counts(c, nb, rank, wsum, pick, above);
}

// Histogram of the top digit over one chunk, added into the row's; the allowed positions are
// counted too (keys of removed positions are 0, below every allowed key, whose top digit is
// never 0; keep <= #allowed, so they never reach the threshold).
__global__ void __launch_bounds__(kSelThreads) dsa_hist_kernel(const DsaParams p) {
    constexpr int NB = 1 << pass_bits(0);
    constexpr int shift = pass_shift(0);
    __shared__ int hist[NB];
    const int tid = threadIdx.x;
    const int64_t T = p.key_seq;
    const int64_t nch = sel_chunks(T);
    const int64_t row = (int64_t)blockIdx.x / nch;
    const int64_t ch = (int64_t)blockIdx.x - row * nch;
    int* aux = p.aux + row * kAuxInts;
    const uint32_t* keys = p.keys + row * T;
    uint32_t kk[kKeysPerThread];
#pragma unroll
    for (int j = 0; j < kKeysPerThread; ++j) {
        const int64_t t = ch * kSelChunk + j * kSelThreads + tid;
        kk[j] = t < T ? keys[t] : 0u;
    }
#pragma unroll
    for (int i = tid; i < NB; i += kSelThreads) hist[i] = 0;
    __syncthreads();
    int allowed = 0;
#pragma unroll
    for (int j = 0; j < kKeysPerThread; ++j) {
        if (ch * kSelChunk + j * kSelThreads + tid < T) {
            allowed += kk[j] != 0u;
            atomicAdd(&hist[kk[j] >> shift], 1);
        }
    }
    __syncthreads();
#pragma unroll
    for (int i = tid; i < NB; i += kSelThreads)
        if (hist[i] != 0) atomicAdd(&aux[i], hist[i]);
    // each wave adds its allowed count
    const int wave_allowed = wave_inclusive_sum(allowed);
    if (lane_id() == 63 && wave_allowed != 0) atomicAdd(&aux[kAuxAllowed], wave_allowed);
}

// Each chunk finds, from the row's finished histogram, keep, the top digit d0 of the keep-th
// largest key and the rank left among the keys with that digit; stores its own count of keys
// with a larger top digit; and appends its keys with top digit d0 (the candidates) and their
// positions to the row's list, and counts their second digits into the row's second histogram.
// Chunk 0 records d0, the rank and keep.  The slots past keep are set to -1 here (spread over the
// row's chunks).
__global__ void __launch_bounds__(kSelThreads) dsa_cand_kernel(const DsaParams p) {
    __shared__ int wsum[kSelThreads / 64];
    __shared__ int w2[kSelThreads / 64][2];
    __shared__ int pick[2];
    const int tid = threadIdx.x;
    const int64_t T = p.key_seq;
    const int64_t nch = sel_chunks(T);
    const int64_t row = (int64_t)blockIdx.x / nch;
    const int64_t ch = (int64_t)blockIdx.x - row * nch;
    int* aux = p.aux + row * kAuxInts;
    const uint32_t* keys = p.keys + row * T;
    int* cand_key = p.cand + row * 2 * T;
    int* cand_pos = cand_key + T;
    int64_t* out = p.out + row * p.top_k;
    const int64_t t0 = ch * kSelChunk + (int64_t)tid * kKeysPerThread;
    uint32_t k8[kKeysPerThread];   // requested before the histogram is read; past T: 0
#pragma unroll
    for (int j = 0; j < kKeysPerThread; ++j) k8[j] = t0 + j < T ? keys[t0 + j] : 0u;
    const int64_t allowed = aux[kAuxAllowed];
    const int64_t keep = allowed < p.top_k ? allowed : p.top_k;
    for (int64_t s = keep + ch * kSelThreads + tid; s < p.top_k; s += nch * kSelThreads) out[s] = -1;
    if (keep == 0) return;
    int above;
    const int d0 = find_digit(aux, 1 << pass_bits(0), (int)keep, wsum, pick, &above);
    int gt_n = 0, c_n = 0;
#pragma unroll
    for (int j = 0; j < kKeysPerThread; ++j) {
        const int dg = (int)(k8[j] >> pass_shift(0));
        gt_n += dg > d0;
        c_n += dg == d0;
    }
    int gt_all, c_all, gt_in, c_in;
    block_inclusive_sum2<kSelThreads>(gt_n, c_n, w2, &gt_in, &c_in, &gt_all, &c_all);
    const int c_at = c_in - c_n;
    if (tid == 0) {
        p.counts[row * nch + ch] = gt_all;
        pick[0] = c_all != 0 ? atomicAdd(&aux[kAuxCand], c_all) : 0;
        if (ch == 0) {
            aux[kAuxD0] = d0;
            aux[kAuxRank] = (int)keep - above;
            aux[kAuxKeep] = (int)keep;
        }
    }
    __syncthreads();
    int at = pick[0] + c_at;
#pragma unroll
    for (int j = 0; j < kKeysPerThread; ++j) {
        if ((int)(k8[j] >> pass_shift(0)) == d0) {
            cand_key[at] = (int)k8[j];
            cand_pos[at] = (int)(t0 + j);
            ++at;
            atomicAdd(&aux[kAuxH1 + ((k8[j] >> pass_shift(1)) & ((1u << pass_bits(1)) - 1u))], 1);
        }
    }
}

// Digit q (1 or 2) of the rank-th largest among the row's n candidates that match `prefix` in
// the digits above it: a histogram of this workgroup alone (LDS, zeroed and visible to every
// thread on entry), then find_digit.  The candidate keys are read from `cand_key` (LDS or the
// workspace).
template <int Q, typename KeyPtr>
__device__ __forceinline__ int cand_digit(KeyPtr cand_key, int n, uint32_t prefix, int rank, int* hist, int* wsum,
                                          int* pick, int* above) {
    constexpr int NB = 1 << pass_bits(Q);
    constexpr int shift = pass_shift(Q);
    constexpr uint32_t hi_mask = 0xffffffffu << ((shift + pass_bits(Q)) & 31);
    for (int i = threadIdx.x; i < n; i += kSelThreads) {
        const uint32_t k = (uint32_t)cand_key[i];
        if ((k & hi_mask) == prefix) atomicAdd(&hist[(k >> shift) & (uint32_t)(NB - 1)], 1);
    }
    __syncthreads();
    return find_digit(hist, NB, rank, wsum, pick, above);
}

// Output of one chunk: thread i owns positions [8 i, 8 i + 8) of the chunk.  The threshold (the
// keep-th largest key) and the ties to take come from the row's candidates (the other two
// digits, found by this workgroup alone); the chunks before this one give its first output
// slot and the ties left for it: their stored counts of keys with a larger top digit, and their
// candidates above and equal to the threshold.  Block prefix sums give each thread the ties it
// may take (the lowest positions first) and its first slot; it writes its winners in position
// order.
constexpr int kCandLds = 2048;   // candidates the write kernel keeps in LDS (8 per thread)

__global__ void __launch_bounds__(kSelThreads) dsa_write_kernel(const DsaParams p) {
    __shared__ int hist2[1 << pass_bits(2)];
    __shared__ uint32_t ck[kCandLds];
    __shared__ int cp[kCandLds];
    __shared__ int wsum[kSelThreads / 64];
    __shared__ int w4[kSelThreads / 64][4];
    __shared__ int pick[2];
    const int tid = threadIdx.x;
    const int64_t T = p.key_seq;
    const int64_t nch = sel_chunks(T);
    const int64_t row = (int64_t)blockIdx.x / nch;
    const int64_t ch = (int64_t)blockIdx.x - row * nch;
    const int* aux = p.aux + row * kAuxInts;
    const int* cand_key = p.cand + row * 2 * T;
    const int* cand_pos = cand_key + T;
    const uint32_t* keys = p.keys + row * T;
    int64_t* out = p.out + row * p.top_k;
    // The chunk's keys, and the first kCandLds entries of the row's candidate list whatever the
    // candidate count (entries past it are ignored), are requested before the row's words are
    // read, so that the three loads share one round trip.
    const int64_t t0 = ch * kSelChunk + (int64_t)tid * kKeysPerThread;
    uint32_t k8[kKeysPerThread];
#pragma unroll
    for (int j = 0; j < kKeysPerThread; ++j) k8[j] = t0 + j < T ? keys[t0 + j] : 0u;
    constexpr int CPT = kCandLds / kSelThreads;
    uint32_t ckr[CPT];
    int cpr[CPT];
#pragma unroll
    for (int j = 0; j < CPT; ++j) {
        const int i = j * kSelThreads + tid;
        ckr[j] = i < T ? (uint32_t)cand_key[i] : 0u;
        cpr[j] = i < T ? cand_pos[i] : 0;
    }
    // the candidates' second-digit histogram, this thread's run of find_digit_counts
    constexpr int DPT1 = (1 << pass_bits(1)) / kSelThreads;
    int c1[kMaxBins / kSelThreads];
#pragma unroll
    for (int j = 0; j < kMaxBins / kSelThreads; ++j)
        c1[j] = j < DPT1 ? aux[kAuxH1 + (1 << pass_bits(1)) - 1 - DPT1 * tid - j] : 0;
    int gt_b = 0, eq_b = 0;   // keys above (then also equal to) the threshold before this chunk
    for (int64_t c = tid; c < ch; c += kSelThreads) gt_b += p.counts[row * nch + c];
    const int64_t allowed = aux[kAuxAllowed];
    const int64_t keep = allowed < p.top_k ? allowed : p.top_k;
    if (keep == 0) return;
    const int n = aux[kAuxCand];
    int rank = aux[kAuxRank];
    uint32_t prefix = (uint32_t)aux[kAuxD0] << pass_shift(0);
    const bool in_lds = n <= kCandLds;
#pragma unroll
    for (int j = 0; j < CPT; ++j) {
        ck[j * kSelThreads + tid] = ckr[j];
        cp[j * kSelThreads + tid] = cpr[j];
    }
    for (int i = tid; i < (1 << pass_bits(2)); i += kSelThreads) hist2[i] = 0;
    __syncthreads();
    // the threshold's other two digits, and the candidates above and equal to it before this chunk
    int above;
    uint32_t thr;
    const int64_t lim = ch * kSelChunk;
    prefix |= (uint32_t)find_digit_counts(c1, 1 << pass_bits(1), rank, wsum, pick, &above) << pass_shift(1);
    rank -= above;
    if (in_lds) {
        thr = prefix | (uint32_t)cand_digit<2>(ck, n, prefix, rank, hist2, wsum, pick, &above);
        for (int i = tid; i < n; i += kSelThreads) {
            if (cp[i] < lim) {
                gt_b += ck[i] > thr;
                eq_b += ck[i] == thr;
            }
        }
    } else {
        thr = prefix | (uint32_t)cand_digit<2>(cand_key, n, prefix, rank, hist2, wsum, pick, &above);
        for (int i = tid; i < n; i += kSelThreads) {
            if (cand_pos[i] < lim) {
                const uint32_t k = (uint32_t)cand_key[i];
                gt_b += k > thr;
                eq_b += k == thr;
            }
        }
    }
    const int ties_needed = rank - above;   // keys equal to the threshold that are taken
    // One exchange between the waves gives the totals of gt_b and eq_b (the chunks before this
    // one: gt_before, eq_before) and the exclusive prefixes of this chunk's own counts over the
    // threads.  Ties go to the lowest positions: the chunk may take ties_left = ties_needed -
    // eq_before of its own, thread i the first ones after the eq_excl ties of the threads
    // before it, so the threads before it take min(ties_left, eq_excl) ties in all.
    int gt_n = 0, eq_n = 0;
#pragma unroll
    for (int j = 0; j < kKeysPerThread; ++j) {
        gt_n += k8[j] > thr;
        eq_n += k8[j] == thr;
    }
    const int lane = lane_id();
    const int wave = tid >> 6;
    const int xg = wave_inclusive_sum(gt_n), xe = wave_inclusive_sum(eq_n);
    const int sg = wave_inclusive_sum(gt_b), se = wave_inclusive_sum(eq_b);
    if (lane == 63) {
        w4[wave][0] = xg;
        w4[wave][1] = xe;
        w4[wave][2] = sg;
        w4[wave][3] = se;
    }
    __syncthreads();
    int gt_excl = xg - gt_n, eq_excl = xe - eq_n, gt_before = 0, eq_before = 0;
#pragma unroll
    for (int w = 0; w < kSelThreads / 64; ++w) {
        if (w < wave) {
            gt_excl += w4[w][0];
            eq_excl += w4[w][1];
        }
        gt_before += w4[w][2];
        eq_before += w4[w][3];
    }
    const int ties_left = ties_needed - eq_before > 0 ? ties_needed - eq_before : 0;
    const int64_t slot0 = (int64_t)gt_before + (eq_before < ties_needed ? eq_before : ties_needed);
    int my_ties = ties_left - eq_excl;
    my_ties = my_ties < 0 ? 0 : (my_ties > eq_n ? eq_n : my_ties);
    int64_t slot = slot0 + gt_excl + (ties_left < eq_excl ? ties_left : eq_excl);
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
    hipLaunchKernelGGL(dsa_hist_kernel, grid, dim3(kSelThreads), 0, s, p);
    hipLaunchKernelGGL(dsa_cand_kernel, grid, dim3(kSelThreads), 0, s, p);
    hipLaunchKernelGGL(dsa_write_kernel, grid, dim3(kSelThreads), 0, s, p);
    return hipGetLastError();
}

}  // namespace dsa
