// Tiled online-softmax attention forward, 16-bit inputs, head dim 64 or 128 (gfx950 fast path).
//
// Same method as fa_fwd16.h (tile-granular online softmax with a running maximum, denominator
// and rescaled numerator, per the onnx-runtime-ep-cuda page `src/kernels/flash_attention.rs`,
// `flash_attention_body`), laid out for a whole CDNA4 compute unit per workgroup:
//
//   * 8 waves x 32 query rows = 256 rows per workgroup, one workgroup per CU, 2 waves per SIMD.
//     Every K/V tile staged in LDS now serves 256 rows (half the L2->LDS traffic per flop of a
//     128-row tile).
//   * K/V tiles of 64 keys stream through a 4-slot LDS ring with 16-byte buffer-to-LDS loads
//     (no staging registers), issued three tiles ahead; one barrier per tile.  Each tile's
//     buffer descriptor ends at the last valid key, so rows past the cache length arrive as 0.
//   * LDS layouts are chosen lane by lane through the DMA source addresses:
//       K: row r of a 32-row half holds key kk(r) (see lds_row_of_key) and its 16-byte chunk c
//          sits at position c ^ k_swz(r), so the 16 rows one 16-byte read cycle touches hit 16
//          different bank slots;
//       V: row-major V[key][d], chunk c of key j at c ^ v_swz(j).  V^T operands come from
//          ds_read_b64_tr_b16, which transposes 4 keys x 4 dims per 16-lane group, so V is never
//          transposed in registers.
//   * Compute per half-tile of 32 keys as in fa_fwd16.h: S^T = K Q^T on 32x32x16 MFMA,
//     softmax on the VALU overlapped with the next half-tile's MFMAs, then O^T += V^T P^T.
#pragma once

#include <type_traits>

#include "fa_device.h"
#include "fa_fwd16.h"
#include "fa_fwd16_ring_consts.h"

namespace fa {


template <typename Tr, int DP, int MASKK, bool SOFTCAP, bool RAW>
__global__ void __attribute__((amdgpu_flat_work_group_size(512, 512), amdgpu_waves_per_eu(2, 2)))
fwd16_ring_kernel(const FwdParams p) {
    using vec8 = typename Tr::vec8;
    using vec4 = typename Tr::vec4;
    using vec2 = typename Tr::vec2;
    using scalar = typename Tr::scalar;
    typedef short s16x4 __attribute__((ext_vector_type(4)));
    typedef __attribute__((address_space(3))) s16x4 lds_s16x4;
    constexpr int WAVES = 8;
    constexpr int BN = 64, HB = 32, STAGES = 4;
    constexpr int ROWB = DP * 2;                 // bytes per K/V row
    constexpr int CPR = DP / 8;                  // 16-byte chunks per row
    constexpr int TILE_BYTES = BN * ROWB;
    constexpr int STAGE_BYTES = 2 * TILE_BYTES;  // K tile then V tile
    constexpr int LDW = TILE_BYTES / 1024 / WAVES;  // 1 KiB DMA ops per wave per operand per tile
    constexpr int NKS = DP / 16;
    constexpr int NDB = DP / 32;
    constexpr bool MASKED = MASKK != kMaskNone;
    constexpr bool SUB_FIRST = MASKED;
    static_assert(DP == 64 || DP == 128, "ring kernel covers head dims 64 and 128");
    static_assert(LDW >= 1, "tile must cover every wave");

    __shared__ __attribute__((aligned(1024))) char lds[STAGES * STAGE_BYTES];
    const uint32_t lds_base = lds_addr(lds);

    const WorkItem w = decode_work(p, blockIdx.x);
    if (!w.valid) return;
    const int b = w.b, h = w.h;
    const int kvh = h / p.group;
    const int tid = threadIdx.x;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int lane = tid & 63;
    const int lr = lane & 31;
    const int hh = lane >> 5;
    const int D = DP;

    const KeyRule rule = make_rule(p, b);
    const int64_t q0 = (int64_t)w.qt * kRingBlockRows;
    const int64_t q_last = (q0 + kRingBlockRows < p.sq ? q0 + kRingBlockRows : p.sq) - 1;
    const int64_t wr0 = q0 + wave * kWaveRows;
    const bool wave_has_rows = wr0 < p.sq;
    const int64_t wr1 = (wr0 + kWaveRows - 1 < p.sq ? wr0 + kWaveRows - 1 : p.sq - 1);
    const int64_t row = wr0 + lr;
    const bool row_valid = row < p.sq;
    const int64_t my_lo = row_valid ? rule.lo(row) : 1;
    const int64_t my_hi = row_valid ? rule.hi(row) : 0;
    const int my_lo32 = (int)(my_lo < 0x7fffffffLL ? my_lo : 0x7fffffffLL);
    const int my_hi32 = (int)(my_hi > -1 ? my_hi : -1);
    const int64_t w_lo_min = rule.lo(wr0), w_lo_max = rule.lo(wr1);
    const int64_t w_hi_min = rule.hi(wr0), w_hi_max = rule.hi(wr1);

    const int64_t lo_wg = rule.lo(q0), hi_wg = rule.hi(q_last);
    const int kt_begin = hi_wg >= lo_wg ? (int)(lo_wg / BN) : 0;
    const int n_tiles = hi_wg >= lo_wg ? (int)(hi_wg / BN) - kt_begin + 1 : 0;

    const scalar* __restrict__ qg = (const scalar*)p.q;
    const char* kg = (const char*)p.k + ((int64_t)b * p.kv_heads + kvh) * p.kv_capacity * ROWB;
    const char* vg = (const char*)p.v + ((int64_t)b * p.kv_heads + kvh) * p.kv_capacity * ROWB;

    // ---- Q fragments: lane (m, hh) holds Q[row][16*ks + 8*hh .. +7]
    vec8 qf[NKS];
    {
        const scalar* qrow = qg + (((int64_t)b * p.heads + h) * p.sq + (row_valid ? row : 0)) * D;
#pragma unroll
        for (int ks = 0; ks < NKS; ++ks)
            qf[ks] = row_valid ? *(const vec8*)(qrow + 16 * ks + 8 * hh) : vec8((scalar)0.0f);
        // Retire the Q loads here and hand the fragments on through an empty asm: the tile loop
        // then holds no register the compiler sees as loaded from memory, so its wait-count
        // pass never drains the K/V ring inside the loop.
        dma_wait<0>();
#pragma unroll
        for (int ks = 0; ks < NKS; ++ks) {
            u32x4 t = __builtin_bit_cast(u32x4, qf[ks]);
            asm volatile("" : "+v"(t));
            qf[ks] = __builtin_bit_cast(vec8, t);
        }
    }

    // ---- mask rows of this workgroup
    constexpr uint32_t MESZ = MASKK == kMaskF32 ? 4u : 2u;
    __amdgpu_buffer_rsrc_t rmask;
    uint32_t mask_row_off = 0;
    if constexpr (MASKED) {
        const int64_t rows_here = q_last - q0 + 1;
        const char* mbase = (const char*)p.mask + ((mask_plane(p, b, h) * p.sq + q0) * (int64_t)p.sk) * MESZ;
        rmask = make_rsrc(mbase, (int)(rows_here * p.sk * MESZ));
        mask_row_off = (uint32_t)((row - q0) * (int64_t)p.sk) * MESZ;
    }

    f32x16 o[NDB];
#pragma unroll
    for (int i = 0; i < NDB; ++i) o[i] = f32x16(0.0f);
    float m_run = neg_inf();
    float l_run = 0.0f;
    const float kfac = p.kfac;
    const float th_x = kRescaleLog2 / kfac;

    // ---- LDS swizzles (the LDS serves 256 bytes per cycle: 16 lanes of a 16-byte read, 32 lanes
    // of an 8-byte read).  K: the 16 rows one read cycle touches sit in 16 distinct 16-byte bank
    // slots.  V: the 4 keys x 2 halves of dims one transpose-read cycle touches likewise.
    auto k_swz = [](int r) -> int { return DP == 128 ? (r & 15) : ((r >> 1) & 7); };
    auto v_swz = [](int key) -> int { return DP == 128 ? 4 * (key & 3) : 4 * ((key >> 1) & 1); };

    // ---- DMA source offsets: DMA op i of a tile writes physical chunks [64 i, 64 i + 64)
    uint32_t k_src[LDW], v_src[LDW];
#pragma unroll
    for (int j = 0; j < LDW; ++j) {
        const int pc = 64 * (wave * LDW + j) + lane;   // physical chunk index in the tile
        const int prow = pc / CPR;
        const int pch = pc % CPR;
        const int kkey = (prow & ~31) + [](int r) {   // key held by LDS row r (inverse of lds_row_of_key)
            return 16 * ((r >> 2) & 1) + 4 * (r >> 3) + (r & 3);
        }(prow & 31);
        k_src[j] = (uint32_t)(kkey * ROWB + ((pch ^ k_swz(prow)) * 16));
        v_src[j] = (uint32_t)(prow * ROWB + ((pch ^ v_swz(prow)) * 16));
    }

    auto issue_tile = [&](int t) __attribute__((always_inline)) {
        // tiles past the end are loaded through an empty descriptor: they write zeros
        const int64_t k0 = (int64_t)(kt_begin + t) * BN;
        int64_t keys = rule.L - k0;
        keys = keys < 0 ? 0 : (keys > BN ? BN : keys);
        if (t >= n_tiles) keys = 0;
        const int bytes = (int)(keys * ROWB);
        const int64_t base_off = keys > 0 ? k0 * ROWB : 0;
        const u32x4 rk = make_rsrc_words(kg + base_off, bytes);
        const u32x4 rv = make_rsrc_words(vg + base_off, bytes);
        const uint32_t sk = lds_base + (uint32_t)((t & (STAGES - 1)) * STAGE_BYTES);
        const uint32_t sv = sk + TILE_BYTES;
#pragma unroll
        for (int j = 0; j < LDW; ++j) {
            const uint32_t op = (uint32_t)__builtin_amdgcn_readfirstlane(wave * LDW + j);
            dma_lds16(rk, sk + 1024u * op, k_src[j]);
            dma_lds16(rv, sv + 1024u * op, v_src[j]);
        }
    };

    auto load_mask = [&](int t, float (&mv)[2][16]) __attribute__((always_inline)) {
        if constexpr (MASKED) {
            const int64_t k0 = (int64_t)(kt_begin + t) * BN;
            const bool tile_inside = k0 + BN <= p.sk && p.vec_mask;
#pragma unroll
            for (int sb = 0; sb < 2; ++sb) {
#pragma unroll
                for (int c = 0; c < 4; ++c) {
                    const int jl = (int)k0 + 32 * sb + 16 * hh + 4 * c;
                    const uint32_t off = mask_row_off + (uint32_t)jl * MESZ;
                    float val[4];
                    if (tile_inside) {
                        if constexpr (MASKK == kMaskF32) {
                            const f32x4 t4 = __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(rmask, off, 0, 0));
#pragma unroll
                            for (int e = 0; e < 4; ++e) val[e] = t4[e];
                        } else {
                            const vec4 t4 = __builtin_bit_cast(vec4, __builtin_amdgcn_raw_buffer_load_b64(rmask, off, 0, 0));
#pragma unroll
                            for (int e = 0; e < 4; ++e) val[e] = (float)t4[e];
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

    const int n_half = 2 * n_tiles;
    // wave-uniform key bounds as 32-bit scalars (keys are < sk <= INT32_MAX)
    auto clamp32 = [](int64_t v) -> int { return (int)(v < -1 ? -1 : (v > 0x7fffffffLL ? 0x7fffffffLL : v)); };
    const int wlo_min = __builtin_amdgcn_readfirstlane(clamp32(w_lo_min));
    const int wlo_max = __builtin_amdgcn_readfirstlane(clamp32(w_lo_max));
    const int whi_min = __builtin_amdgcn_readfirstlane(clamp32(w_hi_min));
    const int whi_max = __builtin_amdgcn_readfirstlane(clamp32(w_hi_max));
    const bool wave_live = wave_has_rows && w_lo_min <= w_hi_max;
    auto half_k0 = [&](int u) __attribute__((always_inline)) { return (kt_begin + (u >> 1)) * BN + HB * (u & 1); };
    auto half_active = [&](int u) __attribute__((always_inline)) {
        const int k0 = half_k0(u);
        return wave_live && k0 <= whi_max && k0 + HB - 1 >= wlo_min;
    };
    auto half_full = [&](int u) __attribute__((always_inline)) {
        const int k0 = half_k0(u);
        return k0 >= wlo_max && k0 + HB - 1 <= whi_min;
    };

    // K operand reads: row 32*(u%2) + lr, chunk (2 ks + hh) ^ k_swz(lr) of ring slot (u/2) % 4
    const uint32_t k_lane = (uint32_t)(lr * ROWB) ^ (uint32_t)(k_swz(lr) << 4);
    auto qk = [&](int u, f32x16& acc) __attribute__((always_inline)) {
        const char* kl = lds + ((u >> 1) & (STAGES - 1)) * STAGE_BYTES + HB * (u & 1) * ROWB;
        acc = f32x16(0.0f);
#pragma unroll
        for (int ks = 0; ks < NKS; ++ks) {
            const uint32_t off = k_lane ^ (uint32_t)((2 * ks + hh) << 4);
            const vec8 a = *(const vec8*)(kl + off);
            acc = Tr::mfma(a, qf[ks], acc);
        }
    };

    // V operand reads through ds_read_b64_tr_b16.  Source lane l = 16 g + 4 k + c points at key
    // 16*hh + 8*j + 4*r + k and dims 32*db + 16*(g%2) + 4*c .. +3 of the half-tile; the transpose
    // hands lane l dims d = l % 32 of those four keys.
    const int gq = (lane >> 4) & 1;
    const int kq = (lane >> 2) & 3;
    const int cq = lane & 3;
    const uint32_t v_row = (uint32_t)((16 * hh + kq) * ROWB);
    uint32_t v_col[NDB];
#pragma unroll
    for (int db = 0; db < NDB; ++db) {
        const int lc = 4 * db + 2 * gq + (cq >> 1);
        v_col[db] = v_row + (uint32_t)(((lc ^ v_swz(kq)) << 4) + 8 * (cq & 1));
    }
    auto pv = [&](int u, const vec8 (&pf)[2]) __attribute__((always_inline)) {
        const char* vl = lds + ((u >> 1) & (STAGES - 1)) * STAGE_BYTES + TILE_BYTES + HB * (u & 1) * ROWB;
        // all V^T fragments of the half-tile are requested before the first MFMA
        vec8 vf[NDB][2];
#pragma unroll
        for (int db = 0; db < NDB; ++db) {
#pragma unroll
            for (int j = 0; j < 2; ++j) {
                const s16x4 lo4 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(vl + v_col[db] + (8 * j) * ROWB));
                const s16x4 hi4 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(vl + v_col[db] + (8 * j + 4) * ROWB));
                vf[db][j] = __builtin_bit_cast(vec8, __builtin_shufflevector(lo4, hi4, 0, 1, 2, 3, 4, 5, 6, 7));
            }
        }
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
            for (int db = 0; db < NDB; ++db) o[db] = Tr::mfma(vf[db][j], pf[j], o[db]);
    };

    // score epilogue of one element: tracked units x (see RAW / SOFTCAP / MASKED)
    auto epi = [&](float sv, float mvv) __attribute__((always_inline)) -> float {
        if constexpr (SOFTCAP) {
            const float th = tanh_fast(sv * p.cap_y);
            return MASKED ? __builtin_fmaf(p.softcap, th, mvv) : th;
        } else if constexpr (MASKED) {
            return __builtin_fmaf(sv, p.scale, mvv);
        } else if constexpr (!RAW) {
            return sv * p.scale;
        } else {
            return sv;
        }
    };

    // Softmax of half-tile u split in 8 phases so that it can be spread between MFMAs:
    //   0, 1: epilogue and maximum of elements 0..7 / 8..15; 2: row maximum across the two
    //   lanes of the row, lazy move of the running maximum; 3..6: exponentials of four elements
    //   each; 7: 16-bit packing and the denominator.  FULL: the half-tile needs no structural mask.
    struct SoftmaxState {
        float mt, alpha, m_safe, nmk, lsum;
        bool moved;
        f32x8 lo8, hi8;
    };
    auto softmax_phase = [&](auto full_c, int ph, int u, f32x16& sc, const float (&mv)[16], vec8 (&pf)[2],
                             SoftmaxState& st) __attribute__((always_inline)) {
        constexpr bool FULL = decltype(full_c)::value;
        if (ph == 0 || ph == 1) {
            const int base = half_k0(u) + 16 * hh;
            const int lo_rel = my_lo32 - base;
            const int hi_rel = my_hi32 - base;
            if (ph == 0) st.mt = neg_inf();
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const int v = 8 * ph + e;
                float x = epi(sc[v], MASKED ? mv[v] : 0.0f);
                if constexpr (!FULL) x = (v >= lo_rel && v <= hi_rel) ? x : neg_inf();
                sc[v] = x;
                st.mt = __builtin_fmaxf(st.mt, x);
            }
        } else if (ph == 2) {
            const float mt = half_swap_max(st.mt);
            const bool need = mt > m_run + th_x;
            const float m_new = need ? mt : m_run;
            st.alpha = need ? exp2_hw((m_run - m_new) * kfac) : 1.0f;
            st.moved = need;
            m_run = m_new;
            st.m_safe = (m_run == neg_inf()) ? 0.0f : m_run;
            st.nmk = -st.m_safe * kfac;
            st.lsum = l_run * st.alpha;
        } else if (ph <= 6) {
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int v = 4 * (ph - 3) + e;
                float pv_;
                if constexpr (SUB_FIRST) pv_ = exp2_hw((sc[v] - st.m_safe) * kfac);
                else pv_ = exp2_hw(__builtin_fmaf(sc[v], kfac, st.nmk));
                if (v < 8) st.lo8[v] = pv_;
                else st.hi8[v - 8] = pv_;
            }
        } else {
            pf[0] = __builtin_convertvector(st.lo8, vec8);
            pf[1] = __builtin_convertvector(st.hi8, vec8);
            float lsum = st.lsum;
#pragma unroll
            for (int q = 0; q < 8; ++q)
                lsum = Tr::sum2(vec2{pf[q >> 2][2 * (q & 3)], pf[q >> 2][2 * (q & 3) + 1]}, lsum);
            l_run = lsum;
        }
    };

    // Whole softmax of one half-tile (no MFMAs to overlap with).
    auto softmax = [&](auto full_c, int u, f32x16& sc, const float (&mv)[16], vec8 (&pf)[2],
                       bool& moved) __attribute__((always_inline)) -> float {
        SoftmaxState st;
#pragma unroll
        for (int ph = 0; ph < 8; ++ph) softmax_phase(full_c, ph, u, sc, mv, pf, st);
        moved = st.moved;
        return st.alpha;
    };

    // S^T of half-tile u+1 on the matrix cores, with the softmax phases of half-tile u placed
    // between its MFMAs (8 phases over NKS MFMAs).
    auto fused = [&](int u, f32x16& sc, f32x16& sn, const float (&mv)[16], vec8 (&pf)[2],
                     bool& moved) __attribute__((always_inline)) -> float {
        const char* kl = lds + (((u + 1) >> 1) & (STAGES - 1)) * STAGE_BYTES + HB * ((u + 1) & 1) * ROWB;
        SoftmaxState st;
        // all K fragments of the half-tile are requested before the first MFMA
        vec8 kf[NKS];
#pragma unroll
        for (int ks = 0; ks < NKS; ++ks) kf[ks] = *(const vec8*)(kl + (k_lane ^ (uint32_t)((2 * ks + hh) << 4)));
        sn = f32x16(0.0f);
#pragma unroll
        for (int ks = 0; ks < NKS; ++ks) {
            sn = Tr::mfma(kf[ks], qf[ks], sn);
#pragma unroll
            for (int ph = ks * 8 / NKS; ph < (ks + 1) * 8 / NKS; ++ph)
                softmax_phase(bool_c<true>{}, ph, u, sc, mv, pf, st);
        }
        moved = st.moved;
        return st.alpha;
    };

    auto substep = [&](int u, f32x16& sc, f32x16& sn, const float (&mc)[16]) __attribute__((always_inline)) {
        const bool has_next = u + 1 < n_half;
        const bool act_cur = half_active(u);
        const bool act_nxt = has_next && half_active(u + 1);
        vec8 pf[2];
        bool moved = false;
        float alpha = 1.0f;
        if (act_cur && act_nxt && half_full(u)) {
            alpha = fused(u, sc, sn, mc, pf, moved);
        } else {
            if (act_cur) {
                if (half_full(u)) alpha = softmax(bool_c<true>{}, u, sc, mc, pf, moved);
                else alpha = softmax(bool_c<false>{}, u, sc, mc, pf, moved);
            }
            if (act_nxt) qk(u + 1, sn);
        }
        if (act_cur) {
            if (wave_any(moved)) {
#pragma unroll
                for (int i = 0; i < NDB; ++i) o[i] *= alpha;
            }
            pv(u, pf);
        }
    };

    // Ring schedule: slot t % 4 holds tile t.  Step t consumes tiles t (K rows 32..63, all of V)
    // and t+1 (K rows 0..31) and starts the loads of tile t+3 into the slot tile t-1 used.
    if (n_tiles > 0) {
        f32x16 sa, sb2;
        float ma[2][16], mb[2][16];
        load_mask(0, ma);
        issue_tile(0);
        issue_tile(1);
        issue_tile(2);
        dma_wait<2 * LDW>();   // tiles 0 and 1 landed; tile 2 may be in flight
        __syncthreads();
        if (half_active(0)) qk(0, sa);
        auto tile_step = [&](int t, float (&mc)[2][16], float (&mn)[2][16]) __attribute__((always_inline)) {
            if (t + 1 < n_tiles) load_mask(t + 1, mn);
            issue_tile(t + 3);
            substep(2 * t, sa, sb2, mc[0]);
            substep(2 * t + 1, sb2, sa, mc[1]);
            dma_wait<2 * LDW>();   // everything but tile t+3 landed
            __syncthreads();
        };
        for (int t = 0; t < n_tiles; t += 2) {
            tile_step(t, ma, mb);
            if (t + 1 < n_tiles) tile_step(t + 1, mb, ma);
        }
    }

    const float l = half_swap_sum(l_run);
    if (!row_valid) return;
    const float inv = l > 0.0f ? 1.0f / l : 0.0f;
    scalar* orow = (scalar*)p.out + (int64_t)b * p.o_stride_b + (int64_t)h * p.o_stride_h + row * p.o_stride_i;
#pragma unroll
    for (int db = 0; db < NDB; ++db) {
#pragma unroll
        for (int a = 0; a < 4; ++a) {
            const int d = 32 * db + 8 * a + 4 * hh;
            f32x4 val;
#pragma unroll
            for (int c = 0; c < 4; ++c) val[c] = o[db][4 * a + c] * inv;
            *(vec4*)(orow + d) = __builtin_convertvector(val, vec4);
        }
    }
}

template <typename Tr, int DP, int MASKK, bool SOFTCAP, bool RAW>
hipError_t launch_ring_one(const FwdParams& p, int grid, hipStream_t stream) {
    hipLaunchKernelGGL((fwd16_ring_kernel<Tr, DP, MASKK, SOFTCAP, RAW>), dim3(grid), dim3(kRingThreads), 0, stream, p);
    return hipGetLastError();
}

template <typename Tr, int DP>
hipError_t launch_ring_dp(const FwdParams& p, int grid, int maskk, bool softcap, hipStream_t s) {
    if (softcap) {
        if (maskk == kMaskF32) return launch_ring_one<Tr, DP, kMaskF32, true, false>(p, grid, s);
        if (maskk == kMaskT) return launch_ring_one<Tr, DP, kMaskT, true, false>(p, grid, s);
        return launch_ring_one<Tr, DP, kMaskNone, true, false>(p, grid, s);
    }
    if (maskk == kMaskF32) return launch_ring_one<Tr, DP, kMaskF32, false, false>(p, grid, s);
    if (maskk == kMaskT) return launch_ring_one<Tr, DP, kMaskT, false, false>(p, grid, s);
    if (p.raw_scores) return launch_ring_one<Tr, DP, kMaskNone, false, true>(p, grid, s);
    return launch_ring_one<Tr, DP, kMaskNone, false, false>(p, grid, s);
}

template <typename Tr>
hipError_t launch_ring(const FwdParams& p, int dp, int grid, int maskk, bool softcap, hipStream_t s) {
    return dp == 64 ? launch_ring_dp<Tr, 64>(p, grid, maskk, softcap, s)
                    : launch_ring_dp<Tr, 128>(p, grid, maskk, softcap, s);
}

}  // namespace fa
