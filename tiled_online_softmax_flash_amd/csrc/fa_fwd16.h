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
//   * K/V tiles of 64 keys move HBM -> registers -> LDS through raw buffer loads whose range
//     ends at the last valid key (hardware zero-fill past it), two LDS slots each.  K is stored
//     row-major (rows permuted, see lds_row_of_key); V is stored transposed (V^T[d][key]) so
//     that every MFMA operand is one 16-byte LDS read.
//   * S^T = K Q^T and O^T += V^T P^T run on v_mfma_f32_32x32x16_{bf16,f16} with fp32
//     accumulators.  Computing the transposed products makes every accumulator value of a
//     lane belong to the lane's own query row (m = lane % 32): the running maximum, the
//     denominator and the rescale of O are per-lane scalars, and P leaves the S accumulator
//     already in the B-operand layout of the P.V product; no LDS round trip, no shuffles.
//   * Software pipeline inside each wave: while the matrix cores compute S for key tile t+1,
//     the vector ALUs run the softmax of tile t (instruction groups interleaved with
//     sched_group_barrier), then P.V of tile t runs.  V is consumed one tile after K, which
//     keeps two LDS slots per operand and one barrier per tile.
//   * The two lanes sharing a row (lane, lane ^ 32) combine row maxima with v_permlane32_swap;
//     the denominators are combined once at the end.
//   * Softmax arithmetic is base 2: p = 2^(x*k - m*k) with log2(e) folded into k.  The maximum
//     is moved lazily (only when a tile raises it by more than 2^8), so O is rarely rescaled.
//   * Only the key tiles that intersect the workgroup's attended range are visited; tiles
//     entirely inside every row's range of a wave skip the per-element structural mask.
//   * The epilogue writes O / l rounded to nearest even, or 0 for rows with no attended key
//     (the `denominator > 0` rule of the pages' final store).
#pragma once

#include <type_traits>

#include "fa_device.h"

namespace fa {

struct TraitsBF16 {
    typedef __bf16 vec8 __attribute__((ext_vector_type(8)));
    typedef __bf16 vec4 __attribute__((ext_vector_type(4)));
    typedef __bf16 vec2 __attribute__((ext_vector_type(2)));
    typedef __bf16 scalar;
    __device__ __forceinline__ static f32x16 mfma(vec8 a, vec8 b, f32x16 c) {
        return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
    }
    // c + a.x + a.y, exact products, fp32 accumulation
    __device__ __forceinline__ static float sum2(vec2 a, float c) {
        const vec2 one = {(__bf16)1.0f, (__bf16)1.0f};
        return __builtin_amdgcn_fdot2_f32_bf16(a, one, c, false);
    }
};

struct TraitsF16 {
    typedef _Float16 vec8 __attribute__((ext_vector_type(8)));
    typedef _Float16 vec4 __attribute__((ext_vector_type(4)));
    typedef _Float16 vec2 __attribute__((ext_vector_type(2)));
    typedef _Float16 scalar;
    __device__ __forceinline__ static f32x16 mfma(vec8 a, vec8 b, f32x16 c) {
        return __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0);
    }
    __device__ __forceinline__ static float sum2(vec2 a, float c) {
        const vec2 one = {(_Float16)1.0f, (_Float16)1.0f};
        return __builtin_amdgcn_fdot2(a, one, c, false);
    }
};

// Mask element kinds: none, fp32, or the input's own 16-bit type.
enum MaskKind { kMaskNone = 0, kMaskF32 = 1, kMaskT = 2 };

template <bool B>
using bool_c = std::integral_constant<bool, B>;

#ifndef WAVES_PER_EU
#define WAVES_PER_EU 2
#endif

// RAW: no mask, no softcap and scale > 0: the tracked score is the raw dot product and the scale
// is folded into the base-2 exponent factor.
template <typename Tr, int DP, int MASKK, bool SOFTCAP, bool RAW>
__global__ void __attribute__((amdgpu_flat_work_group_size(256, 256), amdgpu_waves_per_eu(WAVES_PER_EU, WAVES_PER_EU)))
fwd16_kernel(const FwdParams p) {
    using vec8 = typename Tr::vec8;
    using vec4 = typename Tr::vec4;
    using vec2 = typename Tr::vec2;
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
    constexpr bool MASKED = MASKK != kMaskNone;
    // masked scores may sit near -FLT_MAX, where (x - m) must be formed before scaling
    constexpr bool SUB_FIRST = MASKED;
    static_assert(DP % 32 == 0 && DP <= 128, "padded head dim");

    // K slots 0, 1 then V^T slots 0, 1
    __shared__ __attribute__((aligned(16))) uint16_t lds[2 * KSZ + 2 * VSZ];
    uint16_t* const lds_k = lds;
    uint16_t* const lds_v = lds + 2 * KSZ;

    const WorkItem w = decode_work(p, blockIdx.x);
    if (!w.valid) return;
    const int b = w.b, h = w.h;
    const int kvh = h / p.group;
    const int tid = threadIdx.x;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform: keep in SGPRs
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
    // 32-bit copies for the per-element test on partial tiles: keys are < sk <= INT32_MAX, so a
    // lower bound above INT32_MAX or an upper bound below -1 leaves the row just as empty.
    const int my_lo32 = (int)(my_lo < 0x7fffffffLL ? my_lo : 0x7fffffffLL);
    const int my_hi32 = (int)(my_hi > -1 ? my_hi : -1);
    const int64_t w_lo_min = rule.lo(wr0), w_lo_max = rule.lo(wr1);
    const int64_t w_hi_min = rule.hi(wr0), w_hi_max = rule.hi(wr1);

    // workgroup key-tile range
    const int64_t lo_wg = rule.lo(q0), hi_wg = rule.hi(q_last);
    const int kt_begin = hi_wg >= lo_wg ? (int)(lo_wg / BN) : 0;
    const int n_tiles = hi_wg >= lo_wg ? (int)(hi_wg / BN) - kt_begin + 1 : 0;

    const scalar* __restrict__ qg = (const scalar*)p.q;
    const uint16_t* kg = (const uint16_t*)p.k + ((int64_t)b * p.kv_heads + kvh) * p.kv_capacity * D;
    const uint16_t* vg = (const uint16_t*)p.v + ((int64_t)b * p.kv_heads + kvh) * p.kv_capacity * D;

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

    // ---- mask rows of this workgroup: one descriptor from row q0, per-lane row offsets
    constexpr uint32_t MESZ = MASKK == kMaskF32 ? 4u : 2u;
    __amdgpu_buffer_rsrc_t rmask;
    uint32_t mask_row_off = 0;
    if constexpr (MASKED) {
        const int64_t rows_here = q_last - q0 + 1;
        const char* mbase = (const char*)p.mask + ((mask_plane(p, b, h) * p.sq + q0) * (int64_t)p.sk) * MESZ;
        rmask = make_rsrc(mbase, (int)(rows_here * p.sk * MESZ));
        mask_row_off = (uint32_t)((row - q0) * (int64_t)p.sk) * MESZ;
    }

    // ---- running state
    f32x16 o[NDB];
#pragma unroll
    for (int i = 0; i < NDB; ++i) o[i] = f32x16(0.0f);
    float m_run = neg_inf();
    float l_run = 0.0f;
    const float kfac = p.kfac;
    const float th_x = kRescaleLog2 / kfac;

    // ---- per-thread byte offsets inside a K/V tile, computed once.  Each tile is read through a
    // buffer descriptor whose range ends at key L (or the tile end), so chunks of keys >= L come
    // back as zeros and rows past the cache length are never read.
    uint32_t k_off[NKC];
    bool k_dok[NKC];
    int k_lds[NKC];
#pragma unroll
    for (int n = 0; n < NKC; ++n) {
        const int c = tid + 256 * n;
        const int krow = c / CPR;
        const int kcol = (c % CPR) * 8;
        k_off[n] = (uint32_t)(krow * D + kcol) * 2u;
        k_dok[n] = kcol < D;
        k_lds[n] = ((krow & ~31) + lds_row_of_key(krow & 31)) * KP + kcol;
    }
    uint32_t v_off[NVB];
    bool v_ok[NVB];
    int v_lds[NVB];
#pragma unroll
    for (int n = 0; n < NVB; ++n) {
        const int blk = tid + 256 * n;
        const int kq = (blk / 8 / (DP / 4)) * 8 + (blk & 7);
        const int dq = (blk / 8) % (DP / 4);
        v_off[n] = (uint32_t)(4 * kq * D + 4 * dq) * 2u;
        v_ok[n] = (NVBLK % 256 == 0 || blk < NVBLK) && 4 * dq < D;
        v_lds[n] = 4 * dq * VP + 4 * kq;
    }
    const uint32_t row_bytes = (uint32_t)D * 2u;
    const bool fast_rows = p.vec_kv && D == DP && (NVBLK % 256 == 0);

    u32x4 kreg[NKC];
    u32x2 vreg[NVB][4];

    auto tile_rsrc = [&](const uint16_t* base, int kt) __attribute__((always_inline)) {
        const int64_t k0 = (int64_t)kt * BN;
        const int64_t keys = rule.L - k0 < BN ? rule.L - k0 : BN;   // >= 1 for visited tiles
        return make_rsrc(base + k0 * D, (int)(keys * D * 2));
    };

    auto load_k = [&](int kt) __attribute__((always_inline)) {
        const __amdgpu_buffer_rsrc_t rk = tile_rsrc(kg, kt);
        if (fast_rows) {
#pragma unroll
            for (int n = 0; n < NKC; ++n) kreg[n] = __builtin_amdgcn_raw_buffer_load_b128(rk, k_off[n], 0, 0);
        } else if (p.vec_kv) {
#pragma unroll
            for (int n = 0; n < NKC; ++n)
                kreg[n] = k_dok[n] ? __builtin_amdgcn_raw_buffer_load_b128(rk, k_off[n], 0, 0) : u32x4(0u);
        } else {
            // head dims that do not split into 16-byte rows: element loads, dims >= D zeroed
#pragma unroll
            for (int n = 0; n < NKC; ++n) {
                const int kcol = ((tid + 256 * n) % CPR) * 8;
                uint32_t t[4] = {0u, 0u, 0u, 0u};
#pragma unroll
                for (int e = 0; e < 8; ++e)
                    if (kcol + e < D)
                        t[e >> 1] |= (uint32_t)__builtin_amdgcn_raw_buffer_load_b16(rk, k_off[n] + 2 * e, 0, 0) << (16 * (e & 1));
                kreg[n] = u32x4{t[0], t[1], t[2], t[3]};
            }
        }
    };

    auto load_v = [&](int kt) __attribute__((always_inline)) {
        const __amdgpu_buffer_rsrc_t rv = tile_rsrc(vg, kt);
        if (fast_rows) {
#pragma unroll
            for (int n = 0; n < NVB; ++n)
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    vreg[n][e] = __builtin_amdgcn_raw_buffer_load_b64(rv, v_off[n] + e * row_bytes, 0, 0);
        } else if (p.vec_kv) {
#pragma unroll
            for (int n = 0; n < NVB; ++n)
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    vreg[n][e] = v_ok[n] ? __builtin_amdgcn_raw_buffer_load_b64(rv, v_off[n] + e * row_bytes, 0, 0)
                                         : u32x2(0u);
        } else {
#pragma unroll
            for (int n = 0; n < NVB; ++n) {
                const int blk = tid + 256 * n;
                const int dq = (blk / 8) % (DP / 4);
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    uint32_t t[2] = {0u, 0u};
                    if (NVBLK % 256 == 0 || blk < NVBLK) {
#pragma unroll
                        for (int x = 0; x < 4; ++x)
                            if (4 * dq + x < D)
                                t[x >> 1] |= (uint32_t)__builtin_amdgcn_raw_buffer_load_b16(rv, v_off[n] + e * row_bytes + 2 * x, 0, 0) << (16 * (x & 1));
                    }
                    vreg[n][e] = u32x2{t[0], t[1]};
                }
            }
        }
    };

    auto store_k = [&](int slot) __attribute__((always_inline)) {
        uint16_t* kl = lds_k + slot * KSZ;
#pragma unroll
        for (int n = 0; n < NKC; ++n) *(u32x4*)(kl + k_lds[n]) = kreg[n];
    };

    auto store_v = [&](int slot) __attribute__((always_inline)) {
        uint16_t* vl = lds_v + slot * VSZ;
#pragma unroll
        for (int n = 0; n < NVB; ++n) {
            if (NVBLK % 256 == 0 || tid + 256 * n < NVBLK) {
                // 4x4 transpose of 16-bit elements: vreg[n][e] holds key e, dims 0..3
#pragma unroll
                for (int c = 0; c < 4; ++c) {
                    const int word = c >> 1;
                    const int sh = 16 * (c & 1);
                    const uint32_t k0v = (vreg[n][0][word] >> sh) & 0xffffu;
                    const uint32_t k1v = (vreg[n][1][word] >> sh) & 0xffffu;
                    const uint32_t k2v = (vreg[n][2][word] >> sh) & 0xffffu;
                    const uint32_t k3v = (vreg[n][3][word] >> sh) & 0xffffu;
                    *(u32x2*)(vl + v_lds[n] + c * VP) = u32x2{k0v | (k1v << 16), k2v | (k3v << 16)};
                }
            }
        }
    };

    // additive mask values for this lane's 32 keys of tile kt: k0 + 32*sb + 16*hh + v.  The
    // descriptor spans this workgroup's mask rows, so rows >= sq read as 0 (never stored).
    auto load_mask = [&](int kt, float (&mv)[2][16]) __attribute__((always_inline)) {
        if constexpr (MASKED) {
            const int64_t k0 = (int64_t)kt * BN;
            const bool tile_inside = k0 + BN <= p.sk && p.vec_mask;
#pragma unroll
            for (int sb = 0; sb < 2; ++sb) {
#pragma unroll
                for (int c = 0; c < 4; ++c) {
                    const int jl = (int)k0 + 32 * sb + 16 * hh + 4 * c;   // key of element 0
                    const uint32_t off = mask_row_off + (uint32_t)jl * MESZ;
                    float val[4];
                    if (tile_inside) {
                        if constexpr (MASKK == kMaskF32) {
                            const f32x4 t = __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(rmask, off, 0, 0));
#pragma unroll
                            for (int e = 0; e < 4; ++e) val[e] = t[e];
                        } else {
                            const vec4 t = __builtin_bit_cast(vec4, __builtin_amdgcn_raw_buffer_load_b64(rmask, off, 0, 0));
#pragma unroll
                            for (int e = 0; e < 4; ++e) val[e] = (float)t[e];
                        }
                    } else {
#pragma unroll
                        for (int e = 0; e < 4; ++e) {
                            val[e] = 0.0f;
                            if (jl + e < p.sk) {
                                if constexpr (MASKK == kMaskF32)
                                    val[e] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rmask, off + 4u * e, 0, 0));
                                else
                                    val[e] = (float)__builtin_bit_cast(scalar, __builtin_amdgcn_raw_buffer_load_b16(rmask, off + 2u * e, 0, 0));
                            }
                        }
                    }
#pragma unroll
                    for (int e = 0; e < 4; ++e) mv[sb][4 * c + e] = val[e];
                }
            }
        }
    };

    // Work is pipelined in half-tiles of 32 keys: half-tile u covers keys
    // (kt_begin + u/2) * 64 + 32 * (u % 2) + [0, 32).
    constexpr int HB = BN / 2;
    const int n_half = 2 * n_tiles;
    auto half_active = [&](int u) __attribute__((always_inline)) {
        const int64_t k0 = (int64_t)(kt_begin + (u >> 1)) * BN + HB * (u & 1);
        return wave_has_rows && k0 <= w_hi_max && k0 + HB - 1 >= w_lo_min && w_lo_min <= w_hi_max;
    };
    auto half_full = [&](int u) __attribute__((always_inline)) {
        const int64_t k0 = (int64_t)(kt_begin + (u >> 1)) * BN + HB * (u & 1);
        return k0 >= w_lo_max && k0 + HB - 1 <= w_hi_min;
    };

    // S^T = K Q^T for half-tile u: LDS row 32*(u%2) + lr of K slot (u/2)%2 holds key kk(lr).
    auto qk = [&](int u, f32x16& acc) __attribute__((always_inline)) {
        const uint16_t* kl = lds_k + ((u >> 1) & 1) * KSZ + (HB * (u & 1) + lr) * KP + 8 * hh;
        acc = f32x16(0.0f);
#pragma unroll
        for (int ks = 0; ks < NKS; ++ks) {
            const vec8 a = *(const vec8*)(kl + 16 * ks);
            acc = Tr::mfma(a, qf[ks], acc);
        }
    };

    // Softmax of half-tile u (scores sc, keys base + 16*hh + v) into 16-bit P; moves the running
    // maximum lazily and returns the factor the caller applies to O (1 when unmoved).
    auto softmax = [&](auto full_c, int u, f32x16& sc, const float (&mv)[16], vec8 (&pf)[2],
                       bool& moved) __attribute__((always_inline)) -> float {
        constexpr bool FULL = decltype(full_c)::value;
        float mt = neg_inf();
        const int base = (kt_begin + (u >> 1)) * BN + HB * (u & 1) + 16 * hh;
        const int lo_rel = my_lo32 - base;
        const int hi_rel = my_hi32 - base;
#pragma unroll
        for (int v = 0; v < 16; ++v) {
            float x = sc[v];
            if constexpr (SOFTCAP) {
                const float th = tanh_fast(x * p.cap_y);
                x = MASKED ? __builtin_fmaf(p.softcap, th, mv[v]) : th;
            } else if constexpr (MASKED) {
                x = __builtin_fmaf(x, p.scale, mv[v]);
            } else if constexpr (!RAW) {
                x = x * p.scale;
            }
            if constexpr (!FULL) x = (v >= lo_rel && v <= hi_rel) ? x : neg_inf();
            sc[v] = x;
            mt = __builtin_fmaxf(mt, x);
        }
        mt = half_swap_max(mt);
        // lazy move of the running maximum
        const bool need = mt > m_run + th_x;
        const float m_new = need ? mt : m_run;
        const float alpha = need ? exp2_hw((m_run - m_new) * kfac) : 1.0f;
        moved = need;
        m_run = m_new;
        const float m_safe = (m_run == neg_inf()) ? 0.0f : m_run;
        const float nmk = -m_safe * kfac;
        float lsum = l_run * alpha;
        f32x8 lo8, hi8;
#pragma unroll
        for (int v = 0; v < 8; ++v) {
            if constexpr (SUB_FIRST) {
                lo8[v] = exp2_hw((sc[v] - m_safe) * kfac);
                hi8[v] = exp2_hw((sc[v + 8] - m_safe) * kfac);
            } else {
                lo8[v] = exp2_hw(__builtin_fmaf(sc[v], kfac, nmk));
                hi8[v] = exp2_hw(__builtin_fmaf(sc[v + 8], kfac, nmk));
            }
        }
        pf[0] = __builtin_convertvector(lo8, vec8);
        pf[1] = __builtin_convertvector(hi8, vec8);
#pragma unroll
        for (int q = 0; q < 8; ++q)
            lsum = Tr::sum2(vec2{pf[q >> 2][2 * (q & 3)], pf[q >> 2][2 * (q & 3) + 1]}, lsum);
        l_run = lsum;
        return alpha;
    };

    // Instruction-group order for one pipelined block: the S-MFMAs of the next half-tile, one LDS
    // read ahead each, with the softmax VALU work of the current half-tile spread between them.
    auto interleave_hint = [&]() __attribute__((always_inline)) {
        __builtin_amdgcn_sched_group_barrier(kSchedDsRead, 2, 0);
#pragma unroll
        for (int i = 0; i < NKS; ++i) {
            __builtin_amdgcn_sched_group_barrier(kSchedMfma, 1, 0);
            __builtin_amdgcn_sched_group_barrier(kSchedDsRead, 1, 0);
            __builtin_amdgcn_sched_group_barrier(kSchedValu, 128 / NKS, 0);
        }
    };

    // O^T += V^T P^T for half-tile u: k-slot 8*hh + i of step j is key 16*hh + 8*j + i of the half.
    auto pv = [&](int u, const vec8 (&pf)[2]) __attribute__((always_inline)) {
        const uint16_t* vl = lds_v + ((u >> 1) & 1) * VSZ + lr * VP + HB * (u & 1) + 16 * hh;
#pragma unroll
        for (int db = 0; db < NDB; ++db) {
#pragma unroll
            for (int j = 0; j < 2; ++j) {
                const vec8 a = *(const vec8*)(vl + 32 * db * VP + 8 * j);
                o[db] = Tr::mfma(a, pf[j], o[db]);
            }
        }
    };

    // One pipeline step: softmax(u) with S(u) in sc and S(u+1) into sn, then P.V(u).
    auto substep = [&](int u, f32x16& sc, f32x16& sn, const float (&mc)[16]) __attribute__((always_inline)) {
        const bool has_next = u + 1 < n_half;
        const bool act_cur = half_active(u);
        const bool act_nxt = has_next && half_active(u + 1);
        vec8 pf[2];
        bool moved = false;
        float alpha = 1.0f;
        if (act_cur) {
            const bool full = half_full(u);
            if (act_nxt) {
                if (full) {
                    alpha = softmax(bool_c<true>{}, u, sc, mc, pf, moved);
                    qk(u + 1, sn);
                    interleave_hint();
                } else {
                    alpha = softmax(bool_c<false>{}, u, sc, mc, pf, moved);
                    qk(u + 1, sn);
                    interleave_hint();
                }
            } else {
                if (full) alpha = softmax(bool_c<true>{}, u, sc, mc, pf, moved);
                else alpha = softmax(bool_c<false>{}, u, sc, mc, pf, moved);
            }
            if (wave_any(moved)) {
#pragma unroll
                for (int i = 0; i < NDB; ++i) o[i] *= alpha;
            }
            pv(u, pf);
        } else if (act_nxt) {
            qk(u + 1, sn);
        }
    };

    // Per 64-key tile t: half-step 2t reads K(t) rows 32..63 and V(t) keys 0..31; then a barrier
    // frees K(t)'s slot for K(t+2); half-step 2t+1 reads K(t+1) rows 0..31 and V(t) keys 32..63;
    // V(t+1) goes into the slot V(t-1) used; a closing barrier publishes both.
    if (n_tiles > 0) {
        f32x16 sa, sb2;
        float ma[2][16], mb[2][16];
        load_k(kt_begin);
        load_v(kt_begin);
        load_mask(kt_begin, ma);
        store_k(0);
        store_v(0);
        if (n_tiles > 1) {
            load_k(kt_begin + 1);
            store_k(1);
        }
        __syncthreads();
        if (half_active(0)) qk(0, sa);
        auto tile_step = [&](int t, float (&mc)[2][16], float (&mn)[2][16]) __attribute__((always_inline)) {
            const int kt = kt_begin + t;
            if (t + 2 < n_tiles) load_k(kt + 2);
            if (t + 1 < n_tiles) {
                load_v(kt + 1);
                load_mask(kt + 1, mn);
            }
            substep(2 * t, sa, sb2, mc[0]);
            __syncthreads();
            if (t + 2 < n_tiles) store_k(t & 1);
            substep(2 * t + 1, sb2, sa, mc[1]);
            if (t + 1 < n_tiles) store_v((t + 1) & 1);
            __syncthreads();
        };
        for (int t = 0; t < n_tiles; t += 2) {
            tile_step(t, ma, mb);
            if (t + 1 < n_tiles) tile_step(t + 1, mb, ma);
        }
    }

    // ---- normalise and store: lane holds O[row][32*db + 8*a + 4*hh + c] in o[db][4*a + c]
    const float l = half_swap_sum(l_run);
    if (!row_valid) return;
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
template <typename Tr, int DP, int MASKK, bool SOFTCAP, bool RAW>
hipError_t launch_fwd16_one(const FwdParams& p, int grid, hipStream_t stream) {
    hipLaunchKernelGGL((fwd16_kernel<Tr, DP, MASKK, SOFTCAP, RAW>), dim3(grid), dim3(kThreads), 0, stream, p);
    return hipGetLastError();
}

template <typename Tr, int DP>
hipError_t launch_fwd16_dp(const FwdParams& p, int grid, int maskk, bool softcap, hipStream_t s) {
    if (softcap) {
        if (maskk == kMaskF32) return launch_fwd16_one<Tr, DP, kMaskF32, true, false>(p, grid, s);
        if (maskk == kMaskT) return launch_fwd16_one<Tr, DP, kMaskT, true, false>(p, grid, s);
        return launch_fwd16_one<Tr, DP, kMaskNone, true, false>(p, grid, s);
    }
    if (maskk == kMaskF32) return launch_fwd16_one<Tr, DP, kMaskF32, false, false>(p, grid, s);
    if (maskk == kMaskT) return launch_fwd16_one<Tr, DP, kMaskT, false, false>(p, grid, s);
    if (p.raw_scores) return launch_fwd16_one<Tr, DP, kMaskNone, false, true>(p, grid, s);
    return launch_fwd16_one<Tr, DP, kMaskNone, false, false>(p, grid, s);
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
