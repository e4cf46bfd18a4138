// Tiled online-softmax attention forward for fp32 inputs with head dims 129..384 on gfx950.
//
// The pictor-kernels page (`src/gpu_backend/cuda_imagen_attn_kernels.rs`) builds its fp32
// joint-attention kernel a second time with a head-dim bound of 384, for the image decoder's
// attention (96 KiB of K/V per block there).  Same method and fp32 arithmetic as fa_fwd32.h
// (full fp32 products on v_mfma_f32_32x32x2_f32, fp32 accumulation, no reduced-precision
// staging of Q, K, V, S or P); the head dim is split into four 96-dim groups so that each wave
// keeps few registers:
//   * 8 waves: row block rb (32 query rows; 2 per workgroup) x dim group g (96 dims), two waves
//     per SIMD (with three groups, six waves left two SIMDs with one wave and two with two).
//   * A 32-key K/V tile of all 384 dims sits in LDS (K row-permuted, V as [key quad][dim][4
//     keys]; 97 KB), single-buffered, filled by buffer-to-LDS loads that run under the other
//     half of the tile's work: the next K tile under the softmax and P.V, the next V tile under
//     the next Q.K.  Two barriers a tile.
//   * Wave (rb, g) takes the scores' partial sums over its dims, S_g = K_g Q_g^T.  The four
//     partials of a row block meet in LDS and every wave of the row block adds them in the
//     order g = 0, 1, 2, 3, so the four hold identical scores and run an identical softmax; each
//     then adds P V_g to its own 96 dims of O.
#pragma once

#include "fa_device.h"

namespace fa {

template <bool MASKED, bool SOFTCAP, bool RAW>
__global__ void __attribute__((amdgpu_flat_work_group_size(kWideThreads, kWideThreads)))
fwd32w_kernel(const FwdParams p) {
    constexpr int DP = 384, GD = 96, NG = 4, RBW = kWideRows / kWaveRows, BN = 32, NT = kWideThreads;
    constexpr int KP = DP + 4;          // K tile row pitch (floats): 16-byte pad
    constexpr int VQ = DP * 4;          // floats of one key quad of the V tile ([dim][4 keys])
    constexpr int KSZ = BN * KP;
    constexpr int VSZ = (BN / 4) * VQ;
    constexpr int NQC = GD / 8;         // 8-dim chunks of a group's part of the QK reduction
    constexpr int NDB = GD / 32;        // 32-dim output blocks of a group
    constexpr int SPART = 64 * 16;      // floats of one wave's partial scores
    static_assert(RBW * NG * 64 == NT, "one wave per (row block, dim group)");
    static_assert(NT / 64 * 4 == BN, "each wave loads four keys of a tile");
    static_assert(GD % 32 == 0 && GD * NG == DP, "dim groups of whole 32-dim blocks");

    __shared__ __attribute__((aligned(16))) float lds[KSZ + VSZ + RBW * NG * SPART];
    float* const kl = lds;
    float* const vl = lds + KSZ;
    float* const part = lds + KSZ + VSZ;

    const WorkItem w = decode_work(p, blockIdx.x);
    if (!w.valid) return;
    const int b = w.b, h = w.h;
    const int kvh = h / p.group;
    const int tid = threadIdx.x;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int g = wave % NG, rbw = wave / NG;
    const int lane = tid & 63;
    const int lr = lane & 31;
    const int hh = lane >> 5;
    const int D = p.dim;

    const KeyRule rule = make_rule(p, b);
    const int64_t q0 = (int64_t)w.qt * kWideRows;
    const int64_t q_last = (q0 + kWideRows < p.sq ? q0 + kWideRows : p.sq) - 1;
    const int64_t wr0 = q0 + rbw * kWaveRows;
    const bool wave_has_rows = wr0 < p.sq;
    const int64_t wr1 = (wr0 + kWaveRows - 1 < p.sq ? wr0 + kWaveRows - 1 : p.sq - 1);
    const int64_t row = wr0 + lr;
    const bool row_valid = row < p.sq;
    const int64_t my_lo = row_valid ? rule.lo(row) : 1;
    const int64_t my_hi = row_valid ? rule.hi(row) : 0;
    // 32-bit copies for the per-element test on partial tiles (keys are < sk <= INT32_MAX)
    const int my_lo32 = (int)(my_lo < 0x7fffffffLL ? my_lo : 0x7fffffffLL);
    const int my_hi32 = (int)(my_hi > -1 ? my_hi : -1);
    const int64_t w_lo_min = rule.lo(wr0), w_lo_max = rule.lo(wr1);
    const int64_t w_hi_min = rule.hi(wr0), w_hi_max = rule.hi(wr1);

    const int64_t lo_wg = rule.lo(q0), hi_wg = rule.hi(q_last);
    const int kt_begin = hi_wg >= lo_wg ? (int)(lo_wg / BN) : 0;
    const int n_tiles = hi_wg >= lo_wg ? (int)(hi_wg / BN) - kt_begin + 1 : 0;

    const float* __restrict__ kg = (const float*)p.k + ((int64_t)b * p.kv_heads + kvh) * p.kv_capacity * D;
    const float* __restrict__ vg = (const float*)p.v + ((int64_t)b * p.kv_heads + kvh) * p.kv_capacity * D;

    // ---- Q: lane (m, hh) holds Q[row][GD g + 8c + 4hh + e], e = 0..3 (k-slot hh of step 4c+e)
    f32x4 qf[NQC];
    {
        const float* qrow = (const float*)p.q + (((int64_t)b * p.heads + h) * p.sq + (row_valid ? row : 0)) * D;
#pragma unroll
        for (int c = 0; c < NQC; ++c) {
            const int d0 = GD * g + 8 * c + 4 * hh;
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

    const float* mrow = nullptr;
    if (MASKED)
        mrow = (const float*)p.mask + (mask_plane(p, b, h) * p.sq + (row_valid ? row : 0)) * (int64_t)p.sk;

    f32x16 o[NDB];
#pragma unroll
    for (int i = 0; i < NDB; ++i) o[i] = f32x16(0.0f);
    float m_run = neg_inf();
    float l_run = 0.0f;
    const float kfac = p.kfac;
    const float th_x = kRescaleLog2 / kfac;

    // K/V tile kt into LDS by buffer-to-LDS loads (4 bytes a lane, 256 bytes an instruction), no
    // registers in between.  Wave w loads keys 4w..4w+3 of the tile: K in 64-dim runs of one key,
    // V in 16-dim x 4-key blocks (lane l: key 4w + l%4, dim 16m + l/4), which puts V in LDS as
    // [key quad][dim][4 keys].  Rows past the cache length read as zeros (the tile's buffer ends
    // at the last valid row); lanes past the head dim take an offset past any buffer (zeros).
    const int kfull = D >> 6, vfull = D >> 4;           // whole 64-dim K runs, 16-dim V blocks
    const bool kpart = (D & 63) != 0, vpart = (D & 15) != 0;
    uint32_t kvo[4], kvo_p[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        kvo[i] = (uint32_t)(((4 * wave + i) * D + lane) * 4);
        kvo_p[i] = lane < D - 64 * kfull ? kvo[i] : kOutOfRange;
    }
    const uint32_t vvo = (uint32_t)(((4 * wave + (lane & 3)) * D + (lane >> 2)) * 4);
    const uint32_t vvo_p = 16 * vfull + (lane >> 2) < D ? vvo : kOutOfRange;
    const uint32_t kl_base = lds_addr(kl), vl_base = lds_addr(vl) + (uint32_t)(wave * VQ * 4);
    auto tile_rows = [&](int kt) -> int {
        const int64_t left = rule.L - (int64_t)kt * BN;
        return left >= BN ? BN : left > 0 ? (int)left : 0;
    };
    // Head dim 384 (every run and block whole) issues straight-line code; other head dims loop.
    auto issue_k = [&](int kt) {
        const u32x4 rk = make_rsrc_words(kg + (int64_t)kt * BN * D, tile_rows(kt) * D * 4);
        // opaque copy: the LDS addresses are formed here, per tile, instead of being hoisted out
        // of the tile loop into scalar registers (which then spill)
        uint32_t kb = kl_base;
        asm volatile("" : "+s"(kb));
        if (kfull == DP / 64) {
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const uint32_t dst = kb + (uint32_t)(lds_row_of_key(4 * wave + i) * KP * 4);
#pragma unroll
                for (int c = 0; c < DP / 64; ++c) dma_lds4(rk, dst + 256 * c, kvo[i], 256 * c);
            }
        } else {
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                uint32_t dst = kb + (uint32_t)(lds_row_of_key(4 * wave + i) * KP * 4);
                uint32_t so = 0;
#pragma unroll 1
                for (int c = 0; c < kfull; ++c, dst += 256, so += 256) dma_lds4(rk, dst, kvo[i], so);
                if (kpart) dma_lds4(rk, dst, kvo_p[i], so);
            }
        }
    };
    auto issue_v = [&](int kt) {
        const u32x4 rv = make_rsrc_words(vg + (int64_t)kt * BN * D, tile_rows(kt) * D * 4);
        uint32_t vb = vl_base;
        asm volatile("" : "+s"(vb));
        if (vfull == DP / 16) {
#pragma unroll
            for (int m = 0; m < DP / 16; ++m) dma_lds4(rv, vb + 256 * m, vvo, 64 * m);
        } else {
            uint32_t so = 0;
#pragma unroll 1
            for (int m = 0; m < vfull; ++m, vb += 256, so += 64) dma_lds4(rv, vb, vvo, so);
            if (vpart) dma_lds4(rv, vb, vvo_p, so);
        }
    };
    // K dims past the last 64-dim run are never loaded: zero them once (Q is zero there too)
    {
        const int z0 = 64 * (kfull + (kpart ? 1 : 0));
        const int zw = DP - z0;
        for (int idx = tid; idx < BN * zw; idx += NT) kl[(idx / zw) * KP + z0 + idx % zw] = 0.0f;
    }

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

    float* const my_part = part + (rbw * NG + g) * SPART;
    if (n_tiles > 0) {
        issue_k(kt_begin);
        issue_v(kt_begin);
        dma_wait<0>();
    }
    __syncthreads();   // tile 0 and the zeroed K dims visible to every wave
    for (int t = 0; t < n_tiles; ++t) {
        const int kt = kt_begin + t;
        const int64_t k0 = (int64_t)kt * BN;
        const int64_t k1 = k0 + BN - 1;
        const bool more = t + 1 < n_tiles;
        // the four waves of a row block decide alike; every wave reaches every barrier
        const bool act = wave_has_rows && !(k0 > w_hi_max || k1 < w_lo_min || w_lo_min > w_hi_max);
        if (act) {
            // partial S^T = K_g Q_g^T over this group's dims
            f32x16 s = f32x16(0.0f);
#pragma unroll
            for (int c = 0; c < NQC; ++c) {
                const f32x4 a = *(const f32x4*)(kl + lr * KP + GD * g + 8 * c + 4 * hh);
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    s = __builtin_amdgcn_mfma_f32_32x32x2f32(a[e], qf[c][e], s, 0, 0, 0);
            }
#pragma unroll
            for (int c = 0; c < 4; ++c)
                *(f32x4*)(my_part + (c * 64 + lane) * 4) = f32x4{s[4 * c], s[4 * c + 1], s[4 * c + 2], s[4 * c + 3]};
        }
        dma_wait<0>();     // this wave's V loads of the tile landed
        __syncthreads();   // Q.K done everywhere (K's LDS is free); the whole V tile visible
        if (!MASKED && more) issue_k(kt + 1);
        if (act) {
            f32x16 s;
#pragma unroll
            for (int gg = 0; gg < NG; ++gg) {
                const float* src = part + (rbw * NG + gg) * SPART;
#pragma unroll
                for (int c = 0; c < 4; ++c) {
                    const f32x4 v = *(const f32x4*)(src + (c * 64 + lane) * 4);
#pragma unroll
                    for (int e = 0; e < 4; ++e) s[4 * c + e] = gg == 0 ? v[e] : s[4 * c + e] + v[e];
                }
            }

            const bool full = k0 >= w_lo_max && k1 <= w_hi_min;
            float mval[16];
            if (MASKED) {
                const int64_t jb = k0 + 16 * hh;
#pragma unroll
                for (int c = 0; c < 4; ++c) {
                    const int64_t j = jb + 4 * c;
                    f32x4 val = f32x4(0.0f);
                    if (row_valid) {
                        if (p.vec_mask && j + 3 < p.sk) {
                            val = *(const f32x4*)(mrow + j);
                        } else {
#pragma unroll
                            for (int e = 0; e < 4; ++e)
                                if (j + e < p.sk) val[e] = mrow[j + e];
                        }
                    }
#pragma unroll
                    for (int e = 0; e < 4; ++e) mval[4 * c + e] = val[e];
                }
            }
            float mt = neg_inf();
            if (full) {
#pragma unroll
                for (int v = 0; v < 16; ++v) {
                    const float x = epi(s[v], MASKED ? mval[v] : 0.0f);
                    s[v] = x;
                    mt = __builtin_fmaxf(mt, x);
                }
            } else {
                const int base = (int)k0 + 16 * hh;
                const int lo_rel = my_lo32 - base;
                const int hi_rel = my_hi32 - base;
#pragma unroll
                for (int v = 0; v < 16; ++v) {
                    float x = epi(s[v], MASKED ? mval[v] : 0.0f);
                    x = (v >= lo_rel && v <= hi_rel) ? x : neg_inf();
                    s[v] = x;
                    mt = __builtin_fmaxf(mt, x);
                }
            }
            mt = __builtin_fmaxf(mt, __shfl_xor(mt, 32));

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
            const bool slow = (mk == neg_inf() || mk == -neg_inf()) && m_run != neg_inf();
            float pv[16];
            if (!wave_any(slow)) {
                const float nmk = (m_run == neg_inf()) ? 0.0f : -mk;
#pragma unroll
                for (int v = 0; v < 16; ++v) {
                    pv[v] = exp2_hw(__builtin_fmaf(s[v], kfac, nmk));
                    l_run += pv[v];
                }
            } else {
                const float mr = (m_run == neg_inf()) ? 0.0f : m_run;
#pragma unroll
                for (int v = 0; v < 16; ++v) {
                    pv[v] = exp2_hw((s[v] - mr) * kfac);
                    l_run += pv[v];
                }
            }

            // masked builds start the next K tile only now: their mask loads would wait on it
            if (MASKED && more) issue_k(kt + 1);

            // O_g^T += V_g^T P^T : step t uses key 16*hh + t in k-slot hh
#pragma unroll
            for (int db = 0; db < NDB; ++db) {
#pragma unroll
                for (int q4 = 0; q4 < 4; ++q4) {
                    const f32x4 a = *(const f32x4*)(vl + (4 * hh + q4) * VQ + (GD * g + 32 * db + lr) * 4);
#pragma unroll
                    for (int e = 0; e < 4; ++e)
                        o[db] = __builtin_amdgcn_mfma_f32_32x32x2f32(a[e], pv[4 * q4 + e], o[db], 0, 0, 0);
                }
            }
        }
        if (MASKED && more && !act) issue_k(kt + 1);
        dma_wait<0>();     // this wave's K loads of the next tile landed
        __syncthreads();   // P.V done everywhere (V and the partial scores are free), next K visible
        if (more) issue_v(kt + 1);
    }

    if (!row_valid) return;
    const float l = l_run + __shfl_xor(l_run, 32);
    const float inv = l > 0.0f ? 1.0f / l : 0.0f;
    float* orow = (float*)p.out + (int64_t)b * p.o_stride_b + (int64_t)h * p.o_stride_h + row * p.o_stride_i;
#pragma unroll
    for (int db = 0; db < NDB; ++db) {
#pragma unroll
        for (int a = 0; a < 4; ++a) {
            const int d = GD * g + 32 * db + 8 * a + 4 * hh;
            if (d >= D) continue;
            f32x4 val;
#pragma unroll
            for (int c = 0; c < 4; ++c) val[c] = o[db][4 * a + c] * inv;
            if (p.vec_out) {
                *(f32x4*)(orow + d) = val;
            } else {
#pragma unroll
                for (int c = 0; c < 4; ++c)
                    if (d + c < D) orow[d + c] = val[c];
            }
        }
    }
}

template <bool MASKED, bool SOFTCAP, bool RAW>
hipError_t launch_fwd32w_one(const FwdParams& p, int grid, hipStream_t stream) {
    hipLaunchKernelGGL((fwd32w_kernel<MASKED, SOFTCAP, RAW>), dim3(grid), dim3(kWideThreads), 0, stream, p);
    return hipGetLastError();
}

inline hipError_t launch_fwd32w(const FwdParams& p, int grid, bool masked, bool softcap, hipStream_t s) {
    if (softcap) return masked ? launch_fwd32w_one<true, true, false>(p, grid, s)
                               : launch_fwd32w_one<false, true, false>(p, grid, s);
    if (masked) return launch_fwd32w_one<true, false, false>(p, grid, s);
    return p.raw_scores ? launch_fwd32w_one<false, false, true>(p, grid, s)
                        : launch_fwd32w_one<false, false, false>(p, grid, s);
}

}  // namespace fa
