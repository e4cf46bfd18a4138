// Tiled online-softmax attention forward for 16-bit inputs (bf16 / f16) on gfx950.
//
// The algorithm is the tile-granular online softmax of the onnx-runtime-ep-cuda page
// `src/kernels/flash_attention.rs` (`flash_attention_body` and `flash_attention_f16_tc`):
// K/V tiles staged in on-chip memory and reused by a block of query rows, a running row
// maximum and denominator, and an output numerator rescaled whenever the maximum moves.
// The layout of the work is CDNA4's own:
//
//   * A workgroup owns 128 query rows of one (batch, head): four waves of 32 rows.  Q stays in
//     registers for the whole key loop.
//   * K/V tiles of 64 keys move HBM -> registers -> LDS, double-buffered: the next tile's
//     global loads are in flight while the current one is consumed, one barrier per tile.
//     K is stored row-major (rows permuted, see lds_row_of_key); V is stored transposed
//     (V^T[d][key]) so that each MFMA operand is one 16-byte LDS read.
//   * S^T = K Q^T and O^T += V^T P^T run on v_mfma_f32_32x32x16_{bf16,f16} with fp32
//     accumulators.  Computing the transposed products makes every accumulator value of a
//     lane belong to the lane's own query row (m = lane % 32): the running maximum, the
//     denominator and the rescale of O are per-lane scalars, and P leaves the S accumulator
//     already in the B-operand layout of the P.V product; no LDS round trip, no shuffles.
//   * The two lanes sharing a row (lane, lane ^ 32) combine their row maxima with one
//     cross-half exchange per tile; the denominators are combined once at the end.
//   * Softmax arithmetic is base 2: p = 2^(x*k - m*k) with log2(e) folded into k.  The maximum
//     is moved lazily (only when a tile raises it by more than 2^8), so O is rarely rescaled.
//   * Only the key tiles that intersect the workgroup's attended range are visited; tiles
//     entirely inside every row's range skip the per-element structural mask.
//   * The epilogue writes O / l rounded to nearest even, or 0 for rows with no attended key
//     (the `denominator > 0` rule of the pages' final store).
#pragma once

#include "fa_device.h"

namespace fa {

struct TraitsBF16 {
    typedef __bf16 vec8 __attribute__((ext_vector_type(8)));
    typedef __bf16 vec4 __attribute__((ext_vector_type(4)));
    typedef __bf16 scalar;
    __device__ __forceinline__ static f32x16 mfma(vec8 a, vec8 b, f32x16 c) {
        return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
    }
};

struct TraitsF16 {
    typedef _Float16 vec8 __attribute__((ext_vector_type(8)));
    typedef _Float16 vec4 __attribute__((ext_vector_type(4)));
    typedef _Float16 scalar;
    __device__ __forceinline__ static f32x16 mfma(vec8 a, vec8 b, f32x16 c) {
        return __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0);
    }
};

// Mask element kinds: none, fp32, or the input's own 16-bit type.
enum MaskKind { kMaskNone = 0, kMaskF32 = 1, kMaskT = 2 };

template <typename Tr, int DP, int MASKK, bool SOFTCAP>
__global__ void __attribute__((amdgpu_flat_work_group_size(256, 256), amdgpu_waves_per_eu(2, 2)))
fwd16_kernel(const FwdParams p) {
    using vec8 = typename Tr::vec8;
    using vec4 = typename Tr::vec4;
    using scalar = typename Tr::scalar;
    constexpr int BN = 64;              // keys per tile
    constexpr int KP = DP + 8;          // K tile row pitch (elements): 16-byte pad
    constexpr int VP = BN + 8;          // V^T tile row pitch (elements): 16-byte pad
    constexpr int KSZ = BN * KP;
    constexpr int VSZ = DP * VP;
    constexpr int NKS = DP / 16;        // k-steps of S^T = K Q^T
    constexpr int NDB = DP / 32;        // 32-row d blocks of O^T
    constexpr int CPR = DP / 8;         // 16-byte chunks per K row
    constexpr int NKC = BN * CPR / 256; // K chunks per thread
    constexpr int NVBLK = (BN / 4) * (DP / 4);          // 4 keys x 4 dims blocks of V
    constexpr int NVB = (NVBLK + 255) / 256;            // V blocks per thread
    static_assert(DP % 32 == 0 && DP <= 128, "padded head dim");

    __shared__ __attribute__((aligned(16))) uint16_t lds[2 * (KSZ + VSZ)];

    const WorkItem w = decode_work(p, blockIdx.x);
    if (!w.valid) return;
    const int b = w.b, h = w.h;
    const int kvh = h / p.group;
    const int tid = threadIdx.x;
    const int wave = tid >> 6;
    const int lane = tid & 63;
    const int lr = lane & 31;   // query row within the wave / A-operand row
    const int hh = lane >> 5;   // which half of the wave
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
    const int64_t w_lo_min = rule.lo(wr0), w_lo_max = rule.lo(wr1);
    const int64_t w_hi_min = rule.hi(wr0), w_hi_max = rule.hi(wr1);

    // workgroup key-tile range
    const int64_t lo_wg = rule.lo(q0), hi_wg = rule.hi(q_last);
    const int kt_begin = hi_wg >= lo_wg ? (int)(lo_wg / BN) : 0;
    const int n_tiles = hi_wg >= lo_wg ? (int)(hi_wg / BN) - kt_begin + 1 : 0;

    const scalar* __restrict__ qg = (const scalar*)p.q;
    const uint16_t* __restrict__ kg = (const uint16_t*)p.k + ((int64_t)b * p.kv_heads + kvh) * p.kv_capacity * D;
    const uint16_t* __restrict__ vg = (const uint16_t*)p.v + ((int64_t)b * p.kv_heads + kvh) * p.kv_capacity * D;

    // ---- Q fragments: lane (m, hh) holds Q[row][16*ks + 8*hh .. +7]
    vec8 qf[NKS];
    {
        const scalar* qrow = qg + (((int64_t)b * p.heads + h) * p.sq + (row_valid ? row : 0)) * D;
#pragma unroll
        for (int ks = 0; ks < NKS; ++ks) {
            const int d0 = 16 * ks + 8 * hh;
            vec8 val;
            if (row_valid && p.vec_kv && d0 < D) {
                val = *(const vec8*)(qrow + d0);
            } else {
#pragma unroll
                for (int e = 0; e < 8; ++e)
                    val[e] = (row_valid && d0 + e < D) ? qrow[d0 + e] : (scalar)0.0f;
            }
            qf[ks] = val;
        }
    }

    // ---- mask row pointer (per lane)
    const float* mrow32 = nullptr;
    const scalar* mrow16 = nullptr;
    if (MASKK != kMaskNone) {
        const int64_t off = (mask_plane(p, b, h) * p.sq + (row_valid ? row : 0)) * (int64_t)p.sk;
        if (MASKK == kMaskF32) mrow32 = (const float*)p.mask + off;
        else mrow16 = (const scalar*)p.mask + off;
    }

    // ---- running state
    f32x16 o[NDB];
#pragma unroll
    for (int i = 0; i < NDB; ++i) o[i] = f32x16(0.0f);
    float m_run = neg_inf();
    float l_run = 0.0f;
    const float kfac = p.kfac;
    const float th_x = kRescaleLog2 / kfac;

    // ---- tile staging registers
    u32x4 kreg[NKC];
    u32x2 vreg[NVB][4];

    auto load_tile = [&](int kt) {
        const int64_t k0 = (int64_t)kt * BN;
#pragma unroll
        for (int n = 0; n < NKC; ++n) {
            const int c = tid + 256 * n;
            const int krow = c / CPR;
            const int kcol = (c % CPR) * 8;
            const int64_t j = k0 + krow;
            u32x4 val = u32x4(0u);
            if (j < rule.L && kcol < D) {
                const uint16_t* src = kg + j * D + kcol;
                if (p.vec_kv) {
                    val = *(const u32x4*)src;
                } else {
                    uint32_t t[4] = {0u, 0u, 0u, 0u};
#pragma unroll
                    for (int e = 0; e < 8; ++e)
                        if (kcol + e < D) t[e >> 1] |= (uint32_t)src[e] << (16 * (e & 1));
                    val = u32x4{t[0], t[1], t[2], t[3]};
                }
            }
            kreg[n] = val;
        }
#pragma unroll
        for (int n = 0; n < NVB; ++n) {
            const int blk = tid + 256 * n;
            const int kq = (blk / 8 / (DP / 4)) * 8 + (blk & 7);
            const int dq = (blk / 8) % (DP / 4);
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int64_t j = k0 + 4 * kq + e;
                u32x2 val = u32x2(0u);
                if ((NVBLK % 256 == 0 || blk < NVBLK) && j < rule.L && 4 * dq < D) {
                    const uint16_t* src = vg + j * D + 4 * dq;
                    if (p.vec_kv) {
                        val = *(const u32x2*)src;
                    } else {
                        uint32_t t[2] = {0u, 0u};
#pragma unroll
                        for (int x = 0; x < 4; ++x)
                            if (4 * dq + x < D) t[x >> 1] |= (uint32_t)src[x] << (16 * (x & 1));
                        val = u32x2{t[0], t[1]};
                    }
                }
                vreg[n][e] = val;
            }
        }
    };

    auto store_tile = [&](int buf) {
        uint16_t* kl = lds + buf * (KSZ + VSZ);
        uint16_t* vl = kl + KSZ;
#pragma unroll
        for (int n = 0; n < NKC; ++n) {
            const int c = tid + 256 * n;
            const int krow = c / CPR;
            const int kcol = (c % CPR) * 8;
            const int lrow = (krow & ~31) + lds_row_of_key(krow & 31);
            *(u32x4*)(kl + lrow * KP + kcol) = kreg[n];
        }
#pragma unroll
        for (int n = 0; n < NVB; ++n) {
            const int blk = tid + 256 * n;
            if (NVBLK % 256 == 0 || blk < NVBLK) {
                const int kq = (blk / 8 / (DP / 4)) * 8 + (blk & 7);
                const int dq = (blk / 8) % (DP / 4);
                // 4x4 transpose of 16-bit elements: vreg[n][e] holds key e, dims 0..3
#pragma unroll
                for (int c = 0; c < 4; ++c) {
                    const int word = c >> 1;
                    const int sh = 16 * (c & 1);
                    const uint32_t k0v = (vreg[n][0][word] >> sh) & 0xffffu;
                    const uint32_t k1v = (vreg[n][1][word] >> sh) & 0xffffu;
                    const uint32_t k2v = (vreg[n][2][word] >> sh) & 0xffffu;
                    const uint32_t k3v = (vreg[n][3][word] >> sh) & 0xffffu;
                    *(u32x2*)(vl + (4 * dq + c) * VP + 4 * kq) = u32x2{k0v | (k1v << 16), k2v | (k3v << 16)};
                }
            }
        }
    };

    auto compute_tile = [&](int buf, int kt) {
        const int64_t k0 = (int64_t)kt * BN;
        const int64_t k1 = k0 + BN - 1;
        if (!wave_has_rows || k0 > w_hi_max || k1 < w_lo_min || w_lo_min > w_hi_max) return;
        const bool full = k0 >= w_lo_max && k1 <= w_hi_min;
        const uint16_t* kl = lds + buf * (KSZ + VSZ);
        const uint16_t* vl = kl + KSZ;

        // additive mask values for this lane's 32 keys: k0 + 32*sb + 16*hh + v
        float mval[2][16];
        if (MASKK != kMaskNone) {
#pragma unroll
            for (int sb = 0; sb < 2; ++sb) {
                const int64_t jb = k0 + 32 * sb + 16 * hh;
#pragma unroll
                for (int c = 0; c < 4; ++c) {
                    const int64_t j = jb + 4 * c;
                    if (MASKK == kMaskF32) {
                        f32x4 val = f32x4(0.0f);
                        if (row_valid) {
                            if (p.vec_mask && j + 3 < p.sk) {
                                val = *(const f32x4*)(mrow32 + j);
                            } else {
#pragma unroll
                                for (int e = 0; e < 4; ++e)
                                    if (j + e < p.sk) val[e] = mrow32[j + e];
                            }
                        }
#pragma unroll
                        for (int e = 0; e < 4; ++e) mval[sb][4 * c + e] = val[e];
                    } else {
                        vec4 val = vec4((scalar)0.0f);
                        if (row_valid) {
                            if (p.vec_mask && j + 3 < p.sk) {
                                val = *(const vec4*)(mrow16 + j);
                            } else {
#pragma unroll
                                for (int e = 0; e < 4; ++e)
                                    if (j + e < p.sk) val[e] = mrow16[j + e];
                            }
                        }
#pragma unroll
                        for (int e = 0; e < 4; ++e) mval[sb][4 * c + e] = (float)val[e];
                    }
                }
            }
        }

        // S^T = K Q^T : two 32-key blocks
        f32x16 s[2];
        s[0] = f32x16(0.0f);
        s[1] = f32x16(0.0f);
#pragma unroll
        for (int ks = 0; ks < NKS; ++ks) {
#pragma unroll
            for (int sb = 0; sb < 2; ++sb) {
                const vec8 a = *(const vec8*)(kl + (32 * sb + lr) * KP + 16 * ks + 8 * hh);
                s[sb] = Tr::mfma(a, qf[ks], s[sb]);
            }
        }

        // score epilogue -> x (tracked units), tile maximum
        float mt = neg_inf();
#pragma unroll
        for (int sb = 0; sb < 2; ++sb) {
#pragma unroll
            for (int v = 0; v < 16; ++v) {
                float x = s[sb][v];
                if (SOFTCAP) {
                    const float th = tanh_fast(x * p.cap_y);
                    x = (MASKK != kMaskNone) ? __builtin_fmaf(p.softcap, th, mval[sb][v]) : th;
                } else if (MASKK != kMaskNone) {
                    x = __builtin_fmaf(x, p.scale, mval[sb][v]);
                } else if (!p.raw_scores) {
                    x = x * p.scale;
                }
                if (!full) {
                    const int64_t j = k0 + 32 * sb + 16 * hh + v;
                    x = (j >= my_lo && j <= my_hi) ? x : neg_inf();
                }
                s[sb][v] = x;
                mt = __builtin_fmaxf(mt, x);
            }
        }
        mt = __builtin_fmaxf(mt, __shfl_xor(mt, 32));

        // lazy move of the running maximum
        const bool need = mt > m_run + th_x;
        if (wave_any(need)) {
            const float m_new = need ? mt : m_run;
            const float alpha = need ? exp2_hw((m_run - m_new) * kfac) : 1.0f;
#pragma unroll
            for (int i = 0; i < NDB; ++i) o[i] *= alpha;
            l_run *= alpha;
            m_run = m_new;
        }

        // probabilities (unnormalised, <= 2^8) and their 16-bit copies for P.V
        const float mk = m_run * kfac;
        const bool slow = (mk == neg_inf() || mk == -neg_inf()) && m_run != neg_inf();
        vec8 pf[2][2];
        if (!wave_any(slow)) {
            const float nmk = (m_run == neg_inf()) ? 0.0f : -mk;
#pragma unroll
            for (int sb = 0; sb < 2; ++sb) {
                f32x8 lo8, hi8;
#pragma unroll
                for (int v = 0; v < 8; ++v) {
                    lo8[v] = exp2_hw(__builtin_fmaf(s[sb][v], kfac, nmk));
                    hi8[v] = exp2_hw(__builtin_fmaf(s[sb][v + 8], kfac, nmk));
                    l_run += lo8[v] + hi8[v];
                }
                pf[sb][0] = __builtin_convertvector(lo8, vec8);
                pf[sb][1] = __builtin_convertvector(hi8, vec8);
            }
        } else {
            // a row maximum beyond fp32 range once scaled by kfac: subtract first
            const float mr = (m_run == neg_inf()) ? 0.0f : m_run;
#pragma unroll
            for (int sb = 0; sb < 2; ++sb) {
                f32x8 lo8, hi8;
#pragma unroll
                for (int v = 0; v < 8; ++v) {
                    lo8[v] = exp2_hw((s[sb][v] - mr) * kfac);
                    hi8[v] = exp2_hw((s[sb][v + 8] - mr) * kfac);
                    l_run += lo8[v] + hi8[v];
                }
                pf[sb][0] = __builtin_convertvector(lo8, vec8);
                pf[sb][1] = __builtin_convertvector(hi8, vec8);
            }
        }

        // O^T += V^T P^T : k-slot 8*hh + i of step (sb, u) is key 32*sb + 16*hh + 8*u + i
#pragma unroll
        for (int db = 0; db < NDB; ++db) {
#pragma unroll
            for (int sb = 0; sb < 2; ++sb) {
#pragma unroll
                for (int u = 0; u < 2; ++u) {
                    const vec8 a = *(const vec8*)(vl + (32 * db + lr) * VP + 32 * sb + 16 * hh + 8 * u);
                    o[db] = Tr::mfma(a, pf[sb][u], o[db]);
                }
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

    // ---- normalise and store: lane holds O[row][32*db + 8*a + 4*hh + c] in o[db][4*a + c]
    if (!row_valid) return;
    const float l = l_run + __shfl_xor(l_run, 32);
    const float inv = l > 0.0f ? 1.0f / l : 0.0f;
    scalar* orow = (scalar*)p.out + (int64_t)b * p.o_stride_b + (int64_t)h * p.o_stride_h + row * p.o_stride_i;
#pragma unroll
    for (int db = 0; db < NDB; ++db) {
#pragma unroll
        for (int a = 0; a < 4; ++a) {
            const int d = 32 * db + 8 * a + 4 * hh;
            if (d >= D) continue;
            f32x4 val;
#pragma unroll
            for (int c = 0; c < 4; ++c) val[c] = o[db][4 * a + c] * inv;
            const vec4 cv = __builtin_convertvector(val, vec4);
            if (p.vec_out) {
                *(vec4*)(orow + d) = cv;
            } else {
#pragma unroll
                for (int c = 0; c < 4; ++c)
                    if (d + c < D) orow[d + c] = cv[c];
            }
        }
    }
}

// Launch one instantiation; returns the HIP status of the launch.
template <typename Tr, int DP, int MASKK, bool SOFTCAP>
hipError_t launch_fwd16_one(const FwdParams& p, int grid, hipStream_t stream) {
    hipLaunchKernelGGL((fwd16_kernel<Tr, DP, MASKK, SOFTCAP>), dim3(grid), dim3(kThreads), 0, stream, p);
    return hipGetLastError();
}

template <typename Tr, int DP>
hipError_t launch_fwd16_dp(const FwdParams& p, int grid, int maskk, bool softcap, hipStream_t s) {
    if (softcap) {
        if (maskk == kMaskF32) return launch_fwd16_one<Tr, DP, kMaskF32, true>(p, grid, s);
        if (maskk == kMaskT) return launch_fwd16_one<Tr, DP, kMaskT, true>(p, grid, s);
        return launch_fwd16_one<Tr, DP, kMaskNone, true>(p, grid, s);
    }
    if (maskk == kMaskF32) return launch_fwd16_one<Tr, DP, kMaskF32, false>(p, grid, s);
    if (maskk == kMaskT) return launch_fwd16_one<Tr, DP, kMaskT, false>(p, grid, s);
    return launch_fwd16_one<Tr, DP, kMaskNone, false>(p, grid, s);
}

template <typename Tr>
hipError_t launch_fwd16(const FwdParams& p, int dp, int grid, int maskk, bool softcap, hipStream_t s) {
    switch (dp) {
        case 32: return launch_fwd16_dp<Tr, 32>(p, grid, maskk, softcap, s);
        case 64: return launch_fwd16_dp<Tr, 64>(p, grid, maskk, softcap, s);
        case 96: return launch_fwd16_dp<Tr, 96>(p, grid, maskk, softcap, s);
        default: return launch_fwd16_dp<Tr, 128>(p, grid, maskk, softcap, s);
    }
}

}  // namespace fa
