// Tiled online-softmax attention forward for fp32 inputs on gfx950.
//
// Same structure as the 16-bit kernel (fa_fwd16.h), with every value kept in fp32 as the
// pictor-kernels page `src/gpu_backend/cuda_imagen_attn_kernels.rs` requires of its
// parity-first path (no reduced-precision staging of Q, K, V, S or P).  The contractions run
// on v_mfma_f32_32x32x2_f32 (full fp32 products, fp32 accumulation); K/V tiles of 32 keys
// are staged in LDS (K row-permuted, V transposed), double-buffered.
#pragma once

#include "fa_device.h"

namespace fa {

// RAW: no mask, no softcap and scale > 0 (scale folded into the base-2 exponent factor).
template <int DP, bool MASKED, bool SOFTCAP, bool RAW>
__global__ void __attribute__((amdgpu_flat_work_group_size(256, 256), amdgpu_waves_per_eu(2, 2)))
fwd32_kernel(const FwdParams p) {
    constexpr int BN = 32;
    constexpr int KP = DP + 4;          // K tile row pitch (floats): 16-byte pad
    constexpr int VP = BN + 4;          // V^T tile row pitch (floats): 16-byte pad
    constexpr int KSZ = BN * KP;
    constexpr int VSZ = DP * VP;
    constexpr int NQC = DP / 8;         // 8-dim chunks of the QK reduction
    constexpr int NDB = DP / 32;
    constexpr int CPR = DP / 4;         // 16-byte chunks per K row
    constexpr int NKC = BN * CPR / 256;
    constexpr int NVBLK = (BN / 4) * (DP / 4);
    constexpr int NVB = (NVBLK + 255) / 256;
    static_assert(DP % 32 == 0 && DP <= 128, "padded head dim");

    __shared__ __attribute__((aligned(16))) float lds[2 * (KSZ + VSZ)];

    const WorkItem w = decode_work(p, blockIdx.x);
    if (!w.valid) return;
    const int b = w.b, h = w.h;
    const int kvh = h / p.group;
    const int tid = threadIdx.x;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform: keep in SGPRs
    const int lane = tid & 63;
    const int lr = lane & 31;
    const int hh = lane >> 5;
    const int D = p.dim;

    const KeyRule rule = make_rule(p, b);
    const int64_t q0 = (int64_t)w.qt * kBlockRows;
    const int64_t q_last = (q0 + kBlockRows < p.sq ? q0 + kBlockRows : p.sq) - 1;
    const int64_t wr0 = q0 + wave * kWaveRows;
    const bool wave_has_rows = wr0 < p.sq;
    const int64_t wr1 = (wr0 + kWaveRows - 1 < p.sq ? wr0 + kWaveRows - 1 : p.sq - 1);
    const int64_t row = wr0 + lr;
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

    // ---- Q: lane (m, hh) holds Q[row][8*c + 4*hh + e], e = 0..3 (k-slot hh of step 4c+e)
    f32x4 qf[NQC];
    {
        const float* qrow = (const float*)p.q + (((int64_t)b * p.heads + h) * p.sq + (row_valid ? row : 0)) * D;
#pragma unroll
        for (int c = 0; c < NQC; ++c) {
            const int d0 = 8 * c + 4 * hh;
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

    f32x4 kreg[NKC];
    f32x4 vreg[NVB][4];

    auto load_tile = [&](int kt) {
        const int64_t k0 = (int64_t)kt * BN;
#pragma unroll
        for (int n = 0; n < NKC; ++n) {
            const int c = tid + 256 * n;
            const int krow = c / CPR;
            const int kcol = (c % CPR) * 4;
            const int64_t j = k0 + krow;
            f32x4 val = f32x4(0.0f);
            if (j < rule.L && kcol < D) {
                const float* src = kg + j * D + kcol;
                if (p.vec_kv) {
                    val = *(const f32x4*)src;
                } else {
#pragma unroll
                    for (int e = 0; e < 4; ++e)
                        if (kcol + e < D) val[e] = src[e];
                }
            }
            kreg[n] = val;
        }
#pragma unroll
        for (int n = 0; n < NVB; ++n) {
            const int blk = tid + 256 * n;
            const int kq = blk & 7;
            const int dq = blk >> 3;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int64_t j = k0 + 4 * kq + e;
                f32x4 val = f32x4(0.0f);
                if ((NVBLK % 256 == 0 || blk < NVBLK) && j < rule.L && 4 * dq < D) {
                    const float* src = vg + j * D + 4 * dq;
                    if (p.vec_kv) {
                        val = *(const f32x4*)src;
                    } else {
#pragma unroll
                        for (int x = 0; x < 4; ++x)
                            if (4 * dq + x < D) val[x] = src[x];
                    }
                }
                vreg[n][e] = val;
            }
        }
    };

    auto store_tile = [&](int buf) {
        float* kl = lds + buf * (KSZ + VSZ);
        float* vl = kl + KSZ;
#pragma unroll
        for (int n = 0; n < NKC; ++n) {
            const int c = tid + 256 * n;
            const int krow = c / CPR;
            const int kcol = (c % CPR) * 4;
            *(f32x4*)(kl + lds_row_of_key(krow) * KP + kcol) = kreg[n];
        }
#pragma unroll
        for (int n = 0; n < NVB; ++n) {
            const int blk = tid + 256 * n;
            if (NVBLK % 256 == 0 || blk < NVBLK) {
                const int kq = blk & 7;
                const int dq = blk >> 3;
#pragma unroll
                for (int c = 0; c < 4; ++c)
                    *(f32x4*)(vl + (4 * dq + c) * VP + 4 * kq) =
                        f32x4{vreg[n][0][c], vreg[n][1][c], vreg[n][2][c], vreg[n][3][c]};
            }
        }
    };

    auto compute_tile = [&](int buf, int kt) {
        const int64_t k0 = (int64_t)kt * BN;
        const int64_t k1 = k0 + BN - 1;
        if (!wave_has_rows || k0 > w_hi_max || k1 < w_lo_min || w_lo_min > w_hi_max) return;
        const bool full = k0 >= w_lo_max && k1 <= w_hi_min;
        const float* kl = lds + buf * (KSZ + VSZ);
        const float* vl = kl + KSZ;

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

        // S^T = K Q^T
        f32x16 s = f32x16(0.0f);
#pragma unroll
        for (int c = 0; c < NQC; ++c) {
            const f32x4 a = *(const f32x4*)(kl + lr * KP + 8 * c + 4 * hh);
#pragma unroll
            for (int e = 0; e < 4; ++e)
                s = __builtin_amdgcn_mfma_f32_32x32x2f32(a[e], qf[c][e], s, 0, 0, 0);
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

        // O^T += V^T P^T : step t uses key 16*hh + t in k-slot hh
#pragma unroll
        for (int db = 0; db < NDB; ++db) {
#pragma unroll
            for (int q4 = 0; q4 < 4; ++q4) {
                const f32x4 a = *(const f32x4*)(vl + (32 * db + lr) * VP + 16 * hh + 4 * q4);
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    o[db] = __builtin_amdgcn_mfma_f32_32x32x2f32(a[e], pv[4 * q4 + e], o[db], 0, 0, 0);
            }
        }
    };

    if (n_tiles > 0) {
        load_tile(kt_begin);
        store_tile(0);
        __syncthreads();
        for (int t = 0; t < n_tiles; ++t) {
            const int cur = t & 1;
            if (t + 1 < n_tiles) load_tile(kt_begin + t + 1);
            compute_tile(cur, kt_begin + t);
            if (t + 1 < n_tiles) store_tile(cur ^ 1);
            __syncthreads();
        }
    }

    if (!row_valid) return;
    const float l = l_run + __shfl_xor(l_run, 32);
    const float inv = l > 0.0f ? 1.0f / l : 0.0f;
    float* orow = (float*)p.out + (int64_t)b * p.o_stride_b + (int64_t)h * p.o_stride_h + row * p.o_stride_i;
#pragma unroll
    for (int db = 0; db < NDB; ++db) {
#pragma unroll
        for (int a = 0; a < 4; ++a) {
            const int d = 32 * db + 8 * a + 4 * hh;
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

template <int DP, bool MASKED, bool SOFTCAP, bool RAW>
hipError_t launch_fwd32_one(const FwdParams& p, int grid, hipStream_t stream) {
    hipLaunchKernelGGL((fwd32_kernel<DP, MASKED, SOFTCAP, RAW>), dim3(grid), dim3(kThreads), 0, stream, p);
    return hipGetLastError();
}

template <int DP>
hipError_t launch_fwd32_dp(const FwdParams& p, int grid, bool masked, bool softcap, hipStream_t s) {
    if (softcap) return masked ? launch_fwd32_one<DP, true, true, false>(p, grid, s)
                               : launch_fwd32_one<DP, false, true, false>(p, grid, s);
    if (masked) return launch_fwd32_one<DP, true, false, false>(p, grid, s);
    return p.raw_scores ? launch_fwd32_one<DP, false, false, true>(p, grid, s)
                        : launch_fwd32_one<DP, false, false, false>(p, grid, s);
}

inline hipError_t launch_fwd32(const FwdParams& p, int dp, int grid, bool masked, bool softcap, hipStream_t s) {
    switch (dp) {
        case 32: return launch_fwd32_dp<32>(p, grid, masked, softcap, s);
        case 64: return launch_fwd32_dp<64>(p, grid, masked, softcap, s);
        case 96: return launch_fwd32_dp<96>(p, grid, masked, softcap, s);
        default: return launch_fwd32_dp<128>(p, grid, masked, softcap, s);
    }
}

}  // namespace fa
