// Tiled online-softmax attention forward for fp32 inputs with head dims up to 128 on gfx950.
//
// Every value stays in fp32, as the pictor-kernels page `src/gpu_backend/cuda_imagen_attn_kernels.rs`
// requires of its parity-first path (no reduced-precision staging of Q, K, V, S or P).  The
// contractions run on v_mfma_f32_16x16x4_f32 (full fp32 products, fp32 accumulation), so a wave
// owns 16 query rows and a workgroup of four waves 64 rows.  fp32 problems are small in rows per
// flop: at 32 rows per wave a 24-head, 1536-row problem makes 1152 waves for 1024 SIMDs, and
// most SIMDs run a single wave that cannot hide its own latency; 16-row waves double the count.
//
// Lane l = 16 s + r of a wave stands for query row r of the wave and k-slot s (0..3):
//   * S^T = K Q^T, one MFMA per 4 dims: lane (r, s) supplies K[key r][dim s DP/4 + c] and
//     Q[row r][dim s DP/4 + c] at step c, and ends with the scores of keys 4s..4s+3 of row r.
//   * O^T += V^T P^T, one MFMA per 4 keys and 16 dims: lane (r, s) supplies V[key 4s+v][dim]
//     and its own weight P[row r][key 4s+v] at step v, and accumulates O[row r][16 db + 4s + i].
// A row's statistics are reduced over its four lanes r, r+16, r+32, r+48 with permlane swaps.
// Tiles of 16 keys are staged in LDS through registers (K row-major, V transposed so that a
// lane's four keys of one dim are one 16-byte read), double-buffered with one barrier per tile.
//
// On gfx950 an fp32 MFMA and the vector instructions of other waves on the same SIMD do not
// overlap (measured: every vector instruction adds its own issue time to the MFMA time), so the
// loop keeps vector work per tile small: tile loads go through buffer descriptors (no address or
// bounds arithmetic per tile), tile classification is scalar, the loop is unrolled twice so that
// LDS addresses are constants, and the softmax takes the weights against the running maximum
// as it stands, without a per-tile row maximum, redoing a tile exactly only when its weights
// grow too large (see compute_tile).
#pragma once

#include <type_traits>

#include "fa_device.h"

namespace fa {

// max / sum over the four lanes r, r + 16, r + 32, r + 48 (every lane gets the result).
__device__ __forceinline__ float row4_max(float x) {
    const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return half_swap_max(__builtin_fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1])));
}
__device__ __forceinline__ float row4_sum(float x) {
    const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return half_swap_sum(__uint_as_float(a[0]) + __uint_as_float(a[1]));
}

// A buffer offset beyond every descriptor's range: loads through it return 0.
constexpr uint32_t kOutOfRange = 0x7ffffff0u;

// RAW: no mask, no softcap and scale > 0 (scale folded into the base-2 exponent factor).
// SPLIT: a workgroup takes 32 rows (two 16-row groups) and its key range in two halves: wave w
// covers row group w % 2 over key half w / 2, each half with its own (single) K/V tile buffer in
// LDS, and the two waves of a row group merge their results at the end.  A problem of n 64-row
// tiles then makes 2n half-size workgroups, which spread evenly over the CUs where n does not
// (n = 2.25 per CU leaves a quarter of the CUs a third workgroup; 4.5 half-size ones do not).
template <int DP, bool MASKED, bool SOFTCAP, bool RAW, bool SPLIT>
__global__ void __attribute__((amdgpu_flat_work_group_size(kThreads, kThreads), amdgpu_waves_per_eu(3)))
fwd32_kernel(const FwdParams p) {
    constexpr int BN = 16;              // keys per tile
    constexpr int WR = 16;              // query rows per wave
    constexpr int KP = DP + 4;          // K tile row pitch (floats): 16-byte pad
    constexpr int VP = BN + 4;          // V^T tile row pitch (floats): 16-byte pad
    constexpr int KSZ = BN * KP;
    constexpr int VSZ = DP * VP;
    constexpr int QS = DP / 4;          // dims of one k-slot
    constexpr int NQ = DP / 16;         // 16-byte pieces of a k-slot
    constexpr int NDB = DP / 16;        // 16-dim output blocks
    constexpr int CPR = DP / 4;         // 16-byte chunks per K/V row
    constexpr int NCH = BN * CPR;       // chunks per K (or V) tile
    constexpr int NTH = SPLIT ? kThreads / 2 : kThreads;   // threads that load one tile
    constexpr int NLD = (NCH + NTH - 1) / NTH;
    constexpr int ROWS = SPLIT ? kF32SplitRows : kF32Rows;  // query rows per workgroup
    static_assert(DP % 32 == 0 && DP <= 128, "padded head dim");
    static_assert(kF32Rows == 4 * WR && kF32SplitRows == 2 * WR && kThreads == 256, "four 16-row waves");

    __shared__ __attribute__((aligned(16))) float lds[2 * (KSZ + VSZ)];

    const WorkItem w = decode_work(p, blockIdx.x);
    if (!w.valid) return;
    const int b = w.b, h = w.h;
    const int kvh = h / p.group;
    const int tid = threadIdx.x;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform: keep in SGPRs
    const int rg = SPLIT ? (wave & 1) : wave;                    // the wave's row group
    const int kh = SPLIT ? (wave >> 1) : 0;                      // SPLIT: the wave's key half
    const int th = SPLIT ? tid - kh * NTH : tid;                 // thread among its tile's loaders
    const int lane = tid & 63;
    const int r = lane & 15;
    const int s = lane >> 4;
    const int D = p.dim;

    const KeyRule rule = make_rule(p, b);
    const int Lk = (int)rule.L;         // keys < sk <= INT32_MAX
    const int64_t q0 = (int64_t)w.qt * ROWS;
    const int64_t q_last = (q0 + ROWS < p.sq ? q0 + ROWS : p.sq) - 1;
    const int64_t wr0 = q0 + rg * WR;
    const bool wave_has_rows = wr0 < p.sq;
    const int64_t wr1 = (wr0 + WR - 1 < p.sq ? wr0 + WR - 1 : p.sq - 1);
    const int64_t row = wr0 + r;
    const bool row_valid = row < p.sq;
    const int64_t my_lo = row_valid ? rule.lo(row) : 1;
    const int64_t my_hi = row_valid ? rule.hi(row) : 0;
    // 32-bit copies for the per-element test on partial tiles: keys are < sk <= INT32_MAX, so a
    // lower bound above INT32_MAX or an upper bound below -1 leaves the row just as empty.
    const int my_lo32 = (int)(my_lo < 0x7fffffffLL ? my_lo : 0x7fffffffLL);
    const int my_hi32 = (int)(my_hi > -1 ? my_hi : -1);
    const int64_t w_lo_min = rule.lo(wr0), w_lo_max = rule.lo(wr1);
    const int64_t w_hi_min = rule.hi(wr0), w_hi_max = rule.hi(wr1);

    const int64_t lo_wg = rule.lo(q0), hi_wg = rule.hi(q_last);
    const int kt_begin = hi_wg >= lo_wg ? (int)(lo_wg / BN) : 0;
    const int n_tiles = hi_wg >= lo_wg ? (int)(hi_wg / BN) - kt_begin + 1 : 0;

    const float* __restrict__ kg = (const float*)p.k + ((int64_t)b * p.kv_heads + kvh) * p.kv_capacity * D;
    const float* __restrict__ vg = (const float*)p.v + ((int64_t)b * p.kv_heads + kvh) * p.kv_capacity * D;

    // ---- Q: lane (r, s) holds Q[row][s*QS + 4c + e] in qf[c][e]
    f32x4 qf[NQ];
    {
        const float* qrow = (const float*)p.q + (((int64_t)b * p.heads + h) * p.sq + (row_valid ? row : 0)) * D;
#pragma unroll
        for (int c = 0; c < NQ; ++c) {
            const int d0 = s * QS + 4 * c;
            f32x4 val = f32x4(0.0f);
            if (row_valid && p.vec_kv && d0 < D) {
                val = *(const f32x4*)(qrow + d0);
            } else {
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    if (row_valid && d0 + e < D) val[e] = qrow[d0 + e];
            }
            qf[c] = val;
        }
    }

    // ---- mask rows of this workgroup: one descriptor per tile (its base moves with the tile),
    // per-lane byte offsets; rows past sq and keys past the rows' end read as 0.  Keys past sk
    // of a row read the next row's values, which only ever meet keys the key rule excludes.
    const char* mbase = nullptr;
    int64_t mask_bytes = 0;
    uint32_t mask_off = kOutOfRange;
    if constexpr (MASKED) {
        mbase = (const char*)p.mask + ((mask_plane(p, b, h) * p.sq + q0) * (int64_t)p.sk) * 4;
        mask_bytes = (q_last - q0 + 1) * (int64_t)p.sk * 4;   // < 2 GiB (checked by the host)
        if (row_valid) mask_off = (uint32_t)((row - q0) * (int64_t)p.sk * 4) + 16u * (uint32_t)s;
    }

    f32x4 o[NDB];
#pragma unroll
    for (int i = 0; i < NDB; ++i) o[i] = f32x4(0.0f);
    // Running state of the row.  nmk = -m_run * kfac while the multiply-add form of the weights
    // may be used (m_run finite and |m_run kfac| <= kSpecOffsetMax); NaN otherwise, which sends
    // every tile of the row through the exact softmax.
    float m_run = neg_inf();
    float nmk = __builtin_nanf("");
    float l_run = 0.0f;  // this lane's share (keys 4s..4s+3 of every tile) of the row's sum
    const float kfac = p.kfac;
    const float th_x = kRescaleLog2 / kfac;

    // ---- tile ranges of this wave (wave-uniform, 32-bit): tiles holding a key some row of the
    // wave attends, and tiles whose every key every row of the wave attends
    int wt_first = 0, wt_last = -1, wf_first = 0, wf_last = -1;
    if (wave_has_rows && w_lo_min <= w_hi_max) {
        wt_first = (int)(w_lo_min / BN);
        wt_last = (int)(w_hi_max / BN);
        wf_first = (int)((w_lo_max + BN - 1) / BN);
        wf_last = w_hi_min >= BN - 1 ? (int)((w_hi_min + 1) / BN) - 1 : -1;
    }

    // ---- per-thread tile layout, fixed for the whole loop.  Chunk u (16 bytes) of K is key
    // u / CPR, dims 4 (u % CPR)..; chunk u of V is key u % BN, dims 4 (u / BN).. (key-fastest,
    // so that the transposed LDS writes of a half-wave fall in 32 different banks).  Each tile is
    // read through a descriptor that ends at key L (or the tile end): keys past L read as 0, and
    // chunks past the head dim take an offset beyond any descriptor.
    uint32_t k_off[NLD], v_off[NLD];
    int k_cnt[NLD], v_cnt[NLD];   // valid floats of the chunk (0..4)
    int k_lds[NLD], v_lds[NLD];
#pragma unroll
    for (int n = 0; n < NLD; ++n) {
        const int u = th + NTH * n;
        const bool in = NCH % NTH == 0 || u < NCH;
        const int kr = u / CPR, kc = (u % CPR) * 4;
        const int vr = u % BN, vc = (u / BN) * 4;
        k_cnt[n] = in ? (D - kc < 0 ? 0 : (D - kc > 4 ? 4 : D - kc)) : 0;
        v_cnt[n] = in ? (D - vc < 0 ? 0 : (D - vc > 4 ? 4 : D - vc)) : 0;
        k_off[n] = k_cnt[n] > 0 ? (uint32_t)(kr * D + kc) * 4u : kOutOfRange;
        v_off[n] = v_cnt[n] > 0 ? (uint32_t)(vr * D + vc) * 4u : kOutOfRange;
        k_lds[n] = in ? kr * KP + kc : 0;
        v_lds[n] = in ? vc * VP + vr : 0;
    }

    f32x4 kreg[NLD], vreg[NLD];
    auto tile_rsrc = [&](const float* base, int kt) {
        const int k0 = kt * BN;
        const int keys = Lk - k0 < BN ? Lk - k0 : BN;   // >= 1 for every loaded tile
        return make_rsrc(base + (int64_t)k0 * D, keys * D * 4);
    };
    // VEC: rows move in 16-byte pieces (D a multiple of 4, aligned pointers); else one float at
    // a time, floats past the head dim reading as 0.
    auto load_tile = [&](auto vec_tag, int kt) {
        const __amdgpu_buffer_rsrc_t rk = tile_rsrc(kg, kt);
        const __amdgpu_buffer_rsrc_t rv = tile_rsrc(vg, kt);
#pragma unroll
        for (int n = 0; n < NLD; ++n) {
            if constexpr (decltype(vec_tag)::value) {
                kreg[n] = __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(rk, k_off[n], 0, 0));
                vreg[n] = __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(rv, v_off[n], 0, 0));
            } else {
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    kreg[n][e] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(
                        rk, e < k_cnt[n] ? k_off[n] + 4u * e : kOutOfRange, 0, 0));
                    vreg[n][e] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(
                        rv, e < v_cnt[n] ? v_off[n] + 4u * e : kOutOfRange, 0, 0));
                }
            }
        }
    };

    auto store_tile = [&](float* kl) {
        float* vl = kl + KSZ;
#pragma unroll
        for (int n = 0; n < NLD; ++n) {
            if (NCH % NTH != 0 && th + NTH * n >= NCH) continue;
            *(f32x4*)(kl + k_lds[n]) = kreg[n];
#pragma unroll
            for (int e = 0; e < 4; ++e) vl[v_lds[n] + e * VP] = vreg[n][e];
        }
    };

    // mask[row][keys 4s..4s+3 of tile kt]
    auto load_mask = [&](int kt) -> f32x4 {
        const int64_t k0b = (int64_t)kt * BN * 4;
        const __amdgpu_buffer_rsrc_t rm = make_rsrc(mbase + k0b, (int)(mask_bytes - k0b));
        if (p.vec_mask)
            return __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(rm, mask_off, 0, 0));
        f32x4 val;
#pragma unroll
        for (int e = 0; e < 4; ++e)
            val[e] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(
                rm, mask_off == kOutOfRange ? kOutOfRange : mask_off + 4u * e, 0, 0));
        return val;
    };

    auto compute_tile = [&](const float* kl, int kt, const f32x4& mval) {
        const float* vl = kl + KSZ;

        // S^T = K Q^T, in two interleaved chains (even and odd steps) so that consecutive
        // MFMAs do not wait on each other's results
        f32x4 sc = f32x4(0.0f), sc_odd = f32x4(0.0f);
#pragma unroll
        for (int c = 0; c < NQ; ++c) {
            const f32x4 a = *(const f32x4*)(kl + r * KP + s * QS + 4 * c);
#pragma unroll
            for (int e = 0; e < 4; e += 2) {
                sc = __builtin_amdgcn_mfma_f32_16x16x4f32(a[e], qf[c][e], sc, 0, 0, 0);
                sc_odd = __builtin_amdgcn_mfma_f32_16x16x4f32(a[e + 1], qf[c][e + 1], sc_odd, 0, 0, 0);
            }
        }
        sc += sc_odd;

        auto epi = [&](float sv, float mv) -> float {
            if constexpr (SOFTCAP) {
                const float th = tanh_fast(sv * p.cap_y);
                return MASKED ? __builtin_fmaf(p.softcap, th, mv) : th;
            } else if constexpr (MASKED) {
                return __builtin_fmaf(sv, p.scale, mv);
            } else {
                return RAW ? sv : sv * p.scale;
            }
        };
        if (kt >= wf_first && kt <= wf_last) {
#pragma unroll
            for (int i = 0; i < 4; ++i) sc[i] = epi(sc[i], MASKED ? mval[i] : 0.0f);
        } else {
            const int base = kt * BN + 4 * s;
            const int lo_rel = my_lo32 - base;
            const int hi_rel = my_hi32 - base;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const float x = epi(sc[i], MASKED ? mval[i] : 0.0f);
                sc[i] = (i >= lo_rel && i <= hi_rel) ? x : neg_inf();
            }
        }

        // Weights against the running maximum as it stands.  The tile is redone exactly when
        // a lane's four weights sum past kSpecBound (or are not finite, or the row has no usable
        // maximum yet, nmk = NaN): the row maximum of the tile is taken, the running maximum
        // moved if the tile's exceeds it by more than kRescaleLog2 (base 2), the row's output
        // and sum rescaled, and the weights recomputed.
        float pv[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) pv[i] = exp2_hw(__builtin_fmaf(sc[i], kfac, nmk));
        float psum = (pv[0] + pv[1]) + (pv[2] + pv[3]);
        if (wave_any(!(psum <= kSpecBound))) {
            float mt = __builtin_fmaxf(__builtin_fmaxf(sc[0], sc[1]), __builtin_fmaxf(sc[2], sc[3]));
            mt = row4_max(mt);
            const bool need = mt > m_run + th_x;
            if (wave_any(need)) {
                const float m_new = need ? mt : m_run;
                const float alpha = need ? exp2_hw((m_run - m_new) * kfac) : 1.0f;
#pragma unroll
                for (int i = 0; i < NDB; ++i) o[i] *= alpha;
                l_run *= alpha;
                m_run = m_new;
            }
            const float mk = m_run * kfac;
            const bool fma_form = m_run == neg_inf() || __builtin_fabsf(mk) <= kSpecOffsetMax;
            nmk = (m_run != neg_inf() && fma_form) ? -mk : __builtin_nanf("");
            if (!wave_any(!fma_form)) {
                const float nm = (m_run == neg_inf()) ? 0.0f : -mk;
#pragma unroll
                for (int i = 0; i < 4; ++i) pv[i] = exp2_hw(__builtin_fmaf(sc[i], kfac, nm));
            } else {
                // large offsets: subtract before scaling, so that the rounding of m k does not
                // weigh this row's keys differently from its earlier ones
                const float mr = (m_run == neg_inf()) ? 0.0f : m_run;
#pragma unroll
                for (int i = 0; i < 4; ++i) pv[i] = exp2_hw((sc[i] - mr) * kfac);
            }
            psum = (pv[0] + pv[1]) + (pv[2] + pv[3]);
        }
        l_run += psum;

        // O^T += V^T P^T
#pragma unroll
        for (int db = 0; db < NDB; ++db) {
            const f32x4 a = *(const f32x4*)(vl + (16 * db + r) * VP + 4 * s);
#pragma unroll
            for (int v = 0; v < 4; ++v)
                o[db] = __builtin_amdgcn_mfma_f32_16x16x4f32(a[v], pv[v], o[db], 0, 0, 0);
        }
    };

    auto wave_needs = [&](int kt) { return kt >= wt_first && kt <= wt_last; };
    auto main_loop = [&](auto vec_tag) {
        f32x4 mcur = f32x4(0.0f);
        if (MASKED && wave_needs(kt_begin)) mcur = load_mask(kt_begin);
        load_tile(vec_tag, kt_begin);
        store_tile(lds);
        __syncthreads();
        // tile t sits in buffer t % 2; two tiles per trip so that the buffer is a constant
        auto step = [&](auto buf_tag, int t) {
            constexpr int BUF = decltype(buf_tag)::value;
            const int kt = kt_begin + t;
            const bool more = t + 1 < n_tiles;
            f32x4 mnext = f32x4(0.0f);
            if (more) {
                load_tile(vec_tag, kt + 1);
                if (MASKED && wave_needs(kt + 1)) mnext = load_mask(kt + 1);
            }
            if (wave_needs(kt)) compute_tile(lds + BUF * (KSZ + VSZ), kt, mcur);
            if (more) store_tile(lds + (BUF ^ 1) * (KSZ + VSZ));
            __syncthreads();
            mcur = mnext;
        };
        for (int t = 0; t < n_tiles; t += 2) {
            step(std::integral_constant<int, 0>{}, t);
            if (t + 1 < n_tiles) step(std::integral_constant<int, 1>{}, t + 1);
        }
    };
    // SPLIT: key half kh takes tiles [kt_begin + kh n0, ...): n0 = ceil(n_tiles / 2) of them for
    // half 0, the rest for half 1, each through its own buffer (the next tile is loaded into
    // registers under this one's products, stored after a barrier).  Both halves run n0 trips
    // so that every wave reaches every barrier.
    const int n0 = (n_tiles + 1) / 2;
    auto split_loop = [&](auto vec_tag) {
        const int first = kt_begin + kh * n0;
        const int mine = kh ? n_tiles - n0 : n0;
        float* const buf = lds + kh * (KSZ + VSZ);
        f32x4 mcur = f32x4(0.0f);
        if (mine > 0) {
            if (MASKED && wave_needs(first)) mcur = load_mask(first);
            load_tile(vec_tag, first);
            store_tile(buf);
        }
        __syncthreads();
        for (int t = 0; t < n0; ++t) {
            const int kt = first + t;
            const bool more = t + 1 < mine;
            f32x4 mnext = f32x4(0.0f);
            if (more) {
                load_tile(vec_tag, kt + 1);
                if (MASKED && wave_needs(kt + 1)) mnext = load_mask(kt + 1);
            }
            if (t < mine && wave_needs(kt)) compute_tile(buf, kt, mcur);
            __syncthreads();   // the tile's products are done in both halves
            if (more) store_tile(buf);
            __syncthreads();   // the next tile visible
            mcur = mnext;
        }
    };
    if (n_tiles > 0) {
        if constexpr (SPLIT) {
            if (p.vec_kv) split_loop(std::true_type{});
            else split_loop(std::false_type{});
        } else {
            if (p.vec_kv) main_loop(std::true_type{});
            else main_loop(std::false_type{});
        }
    }

    if constexpr (SPLIT) {
        // the key-half-1 wave of each row group hands its running maximum, sum share and O to
        // the key-half-0 wave (lane by lane: both hold the same rows and k-slots), which merges
        // them: both parts are rescaled to the larger maximum (a part with no maximum yet adds 0)
        constexpr int MW = 2 + 4 * NDB;      // words per lane
        static_assert(2 * 64 * MW <= 2 * (KSZ + VSZ), "merge area inside the tile buffers");
        float* const mb = lds + rg * 64 * MW + lane;
        __syncthreads();   // (n_tiles == 0: no loop barrier) the tile buffers are free
        if (kh == 1) {
            mb[0] = m_run;
            mb[64] = l_run;
#pragma unroll
            for (int db = 0; db < NDB; ++db)
#pragma unroll
                for (int i = 0; i < 4; ++i) mb[64 * (2 + 4 * db + i)] = o[db][i];
        }
        __syncthreads();
        if (kh == 1) return;   // no barrier follows
        const float m1 = mb[0];
        const float mm = __builtin_fmaxf(m_run, m1);
        const float a0 = m_run == neg_inf() ? 0.0f : exp2_hw((m_run - mm) * kfac);
        const float a1 = m1 == neg_inf() ? 0.0f : exp2_hw((m1 - mm) * kfac);
        l_run = l_run * a0 + mb[64] * a1;
#pragma unroll
        for (int db = 0; db < NDB; ++db)
#pragma unroll
            for (int i = 0; i < 4; ++i) o[db][i] = o[db][i] * a0 + mb[64 * (2 + 4 * db + i)] * a1;
    }

    // every lane takes part in the row sums before the invalid rows leave
    const float l = row4_sum(l_run);
    if (!row_valid) return;
    const float inv = l > 0.0f ? 1.0f / l : 0.0f;
    float* orow = (float*)p.out + (int64_t)b * p.o_stride_b + (int64_t)h * p.o_stride_h + row * p.o_stride_i;
#pragma unroll
    for (int db = 0; db < NDB; ++db) {
        const int d = 16 * db + 4 * s;
        if (d >= D) continue;
        const f32x4 val = o[db] * inv;
        if (p.vec_out) {
            *(f32x4*)(orow + d) = val;
        } else {
#pragma unroll
            for (int c = 0; c < 4; ++c)
                if (d + c < D) orow[d + c] = val[c];
        }
    }
}

template <int DP, bool MASKED, bool SOFTCAP, bool RAW>
hipError_t launch_fwd32_one(const FwdParams& p, int grid, bool split, hipStream_t stream) {
    if constexpr (fwd32_split_built(DP, MASKED)) {
        if (split) {
            hipLaunchKernelGGL((fwd32_kernel<DP, MASKED, SOFTCAP, RAW, true>), dim3(grid), dim3(kThreads), 0,
                               stream, p);
            return hipGetLastError();
        }
    } else {
        if (split) return hipErrorInvalidValue;
    }
    hipLaunchKernelGGL((fwd32_kernel<DP, MASKED, SOFTCAP, RAW, false>), dim3(grid), dim3(kThreads), 0, stream, p);
    return hipGetLastError();
}

template <int DP>
hipError_t launch_fwd32_dp(const FwdParams& p, int grid, bool masked, bool softcap, bool split, hipStream_t s) {
    if (softcap) return masked ? launch_fwd32_one<DP, true, true, false>(p, grid, split, s)
                               : launch_fwd32_one<DP, false, true, false>(p, grid, split, s);
    if (masked) return launch_fwd32_one<DP, true, false, false>(p, grid, split, s);
    return p.raw_scores ? launch_fwd32_one<DP, false, false, true>(p, grid, split, s)
                        : launch_fwd32_one<DP, false, false, false>(p, grid, split, s);
}

// Head dims 65..96 take the 128-dim build (dims past D are zero): a 96-dim build needs more
// registers than three waves per SIMD allow.  split: 32-row workgroups with the key range in two
// halves (the grid and p.q_tiles counted in 32-row tiles).
inline hipError_t launch_fwd32(const FwdParams& p, int dp, int grid, bool masked, bool softcap, bool split,
                               hipStream_t s) {
    switch (dp) {
        case 32: return launch_fwd32_dp<32>(p, grid, masked, softcap, split, s);
        case 64: return launch_fwd32_dp<64>(p, grid, masked, softcap, split, s);
        default: return launch_fwd32_dp<128>(p, grid, masked, softcap, split, s);
    }
}

}  // namespace fa
