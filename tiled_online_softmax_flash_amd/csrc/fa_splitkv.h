// Split-key attention forward for few query rows per KV head (decode), 16-bit inputs, head dim
// 64 or 128, on gfx950.
//
// The onnx-runtime-ep-cuda page names a separate decode kernel beside its prefill kernel (its
// support gate sends one-query calls elsewhere); its source is not on the pages.  Same method as
// the prefill kernels: tile-granular online softmax with a running maximum, denominator and
// rescaled numerator, whose partial states merge exactly (the same rule the kernels apply between
// tiles, as in the online-softmax derivation of `flash_attention_body`):
//   * One (batch, KV head) group's query rows, all `group` query heads times sq rows (at most
//     32), form the 32-row MFMA block, so every K/V byte read serves all heads sharing it.
//   * The key range is cut into num_splits spans of `span` keys.  Each wave runs one span on its
//     own: it streams the span's 32-key K/V tiles through registers (two tiles in flight) into
//     two LDS slots of its own, and keeps the span's running maximum, denominator and
//     unnormalised output in registers, which it writes to the workspace.  The kernel is bound
//     by HBM bandwidth; its registers allow one wave per SIMD, so the grid is best at one
//     workgroup per compute unit (fa_splitkv_suggested_splits).
//   * An additive mask (one plane, one per batch or one per head) is read per lane, 16 keys of
//     a tile at a time, and added after the optional softcap.
//   * A second kernel merges the spans of every output row: with M the largest span maximum,
//     O = sum_s 2^((m_s - M) k) O_s / sum_s 2^((m_s - M) k) l_s (0 when no span has a key).
// LDS layouts, fragments and the softmax are those of the 256-row ring kernel (fa_fwd16_ring.h)
// for one 32-key half-tile.
#pragma once

#include "fa_device.h"
#include "fa_fwd16.h"

namespace fa {

constexpr int kSplitThreads = 256;

// MT: additive mask 0 none, 1 float32, 2 of the input type.
template <typename Tr, int DP, bool SOFTCAP, bool RAW, int MT>
__global__ void __attribute__((amdgpu_flat_work_group_size(kSplitThreads, kSplitThreads)))
splitkv_kernel(const FwdParams p, const SplitParams sp) {
    using vec8 = typename Tr::vec8;
    using vec2 = typename Tr::vec2;
    using scalar = typename Tr::scalar;
    typedef short s16x4 __attribute__((ext_vector_type(4)));
    typedef __attribute__((address_space(3))) s16x4 lds_s16x4;
    constexpr int ROWB = DP * 2;             // bytes per K/V row
    constexpr int HALF = 32 * ROWB;          // one 32-key tile of K (or V)
    constexpr int SLOT = 2 * HALF;           // K then V
    constexpr int WAVE_LDS = 2 * SLOT;       // two slots per wave
    constexpr int NKS = DP / 16;             // Q.K MFMAs per tile
    constexpr int NDB = DP / 32;             // 32-dim output blocks
    constexpr int NOPS = HALF / 1024;        // 1 KiB DMA ops per operand per tile
    static_assert(DP == 64 || DP == 128, "head dims 64 and 128");

    __shared__ __attribute__((aligned(1024))) char lds[4 * WAVE_LDS];

    const int tid = threadIdx.x;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int lane = tid & 63;
    const int lr = lane & 31;
    const int hh = lane >> 5;
    const int nsw = sp.num_splits >> 2;
    const int grp = (int)blockIdx.x / nsw;                   // b * kv_heads + kvh
    const int split = ((int)blockIdx.x - grp * nsw) * 4 + wave;
    const int b = grp / p.kv_heads, kvh = grp - b * p.kv_heads;
    const KeyRule rule = make_rule(p, b);

    // row lr of the block: query row i = lr / group of head kvh * group + lr % group
    const bool row_valid = lr < sp.rows;
    const int qi = row_valid ? lr / p.group : 0;
    const int hq = kvh * p.group + (row_valid ? lr - qi * p.group : 0);
    const int64_t lo = row_valid ? rule.lo(qi) : 1;
    const int64_t hi = row_valid ? rule.hi(qi) : 0;
    const int my_lo32 = (int)(lo < 0x7fffffffLL ? lo : 0x7fffffffLL);
    const int my_hi32 = (int)(hi > -1 ? hi : -1);
    // additive mask row of this query row (plane 0, b, or b * heads + h); read at clamped
    // in-range key indices, keys past the row's range being removed by the key rule anyway
    const char* mrow = nullptr;
    if constexpr (MT != 0) {
        const int64_t plane = mask_plane(p, b, hq);
        const int64_t esz = MT == 1 ? 4 : 2;
        mrow = (const char*)p.mask + ((plane * p.sq + qi) * (int64_t)p.sk) * esz;
    }
    // keys any row of the block attends (lo and hi grow with the query row)
    const int64_t last_i = (sp.rows - 1) / p.group;
    const int64_t u_lo = rule.lo(0), u_hi = rule.hi(last_i);
    const int64_t s_lo = (int64_t)split * sp.span, s_hi = s_lo + sp.span - 1;
    const int64_t k_lo = s_lo > u_lo ? s_lo : u_lo;
    const int64_t k_hi = s_hi < u_hi ? s_hi : u_hi;
    const int t_begin = k_hi >= k_lo ? (int)(k_lo / 32) : 0;
    const int n_tiles = k_hi >= k_lo ? (int)(k_hi / 32) - t_begin + 1 : 0;

    // Q fragments: lane (lr, hh) holds Q[hq][qi][16 ks + 8 hh .. +7] (zero for padding rows)
    vec8 qf[NKS];
    {
        const scalar* qrow = (const scalar*)p.q + (((int64_t)b * p.heads + hq) * p.sq + qi) * DP;
#pragma unroll
        for (int ks = 0; ks < NKS; ++ks)
            qf[ks] = row_valid ? *(const vec8*)(qrow + 16 * ks + 8 * hh) : vec8((scalar)0.0f);
    }

    // K/V of the group through buffer descriptors that end at the cache length: keys past it
    // arrive as zeros and are never read from memory
    const char* kg = (const char*)p.k + (int64_t)grp * p.kv_capacity * ROWB;
    const char* vg = (const char*)p.v + (int64_t)grp * p.kv_capacity * ROWB;
    const __amdgpu_buffer_rsrc_t rkb = make_rsrc(kg, (int)(rule.L * ROWB));
    const __amdgpu_buffer_rsrc_t rvb = make_rsrc(vg, (int)(rule.L * ROWB));
    // source offsets within a tile (the ring kernel's half-tile layouts): load j of this lane
    // fills 16-byte chunk 64 j + lane of the K (V) tile in LDS
    uint32_t k_src[NOPS], v_src[NOPS];
#pragma unroll
    for (int j = 0; j < NOPS; ++j) {
        const int q = 64 * j + lane;
        {
            const int ks = q / 64, r = (q >> 1) & 31, c = q & 1;
            const int key = 16 * ((r >> 2) & 1) + 4 * (r >> 3) + (r & 3);
            k_src[j] = (uint32_t)(key * ROWB + (2 * ks + (c ^ ((r >> 3) & 1))) * 16);
        }
        {
            const int db = q / 128, key = (q >> 2) & 31, c = q & 3;
            v_src[j] = (uint32_t)(key * ROWB + (4 * db + c) * 16);
        }
    }
    // two tiles in flight in registers; a landed tile is stored to one of the wave's two LDS
    // slots (plain loads and stores: at one wave per SIMD the registers hold more bytes in
    // flight than buffer-to-LDS DMA into a third slot would)
    u32x4 ra_k[NOPS], ra_v[NOPS], rb_k[NOPS], rb_v[NOPS];
    auto load = [&](int t, u32x4 (&kk)[NOPS], u32x4 (&vv)[NOPS]) {
        const uint32_t off = (uint32_t)(t_begin + t) * (uint32_t)HALF;
#pragma unroll
        for (int j = 0; j < NOPS; ++j) {
            kk[j] = __builtin_amdgcn_raw_buffer_load_b128(rkb, k_src[j] + off, 0, 0);
            vv[j] = __builtin_amdgcn_raw_buffer_load_b128(rvb, v_src[j] + off, 0, 0);
        }
    };
    auto store = [&](int slot, const u32x4 (&kk)[NOPS], const u32x4 (&vv)[NOPS]) {
        char* base = lds + wave * WAVE_LDS + slot * SLOT + lane * 16;
#pragma unroll
        for (int j = 0; j < NOPS; ++j) {
            *(u32x4*)(base + 1024 * j) = kk[j];
            *(u32x4*)(base + HALF + 1024 * j) = vv[j];
        }
    };
    const uint32_t k_base = (uint32_t)(lr * 32 + ((hh ^ ((lr >> 3) & 1)) << 4));
    const uint32_t v_base = (uint32_t)((16 * hh + ((lane >> 2) & 3)) * 64 + ((lane >> 4) & 1) * 32 + (lane & 3) * 8);

    f32x16 o[NDB];
#pragma unroll
    for (int i = 0; i < NDB; ++i) o[i] = f32x16(0.0f);
    float m_run = neg_inf(), l_run = 0.0f;
    const float kfac = p.kfac;
    const float th_x = kRescaleLog2 / kfac;

    auto compute = [&](int t, int slot) {
        const char* kt = lds + wave * WAVE_LDS + slot * SLOT;
        const char* vt = kt + HALF;
        // mask values of this lane's 16 keys, requested before the tile's products
        float mv[16];
        if constexpr (MT != 0) {
            const int kb = (t_begin + t) * 32 + 16 * hh;
#pragma unroll
            for (int v = 0; v < 16; ++v) {
                const int k = kb + v < p.sk ? kb + v : p.sk - 1;
                if constexpr (MT == 1) mv[v] = row_valid ? ((const float*)mrow)[k] : 0.0f;
                else mv[v] = row_valid ? (float)((const scalar*)mrow)[k] : 0.0f;
            }
        }
        f32x16 s = f32x16(0.0f);
#pragma unroll
        for (int ks = 0; ks < NKS; ++ks) {
            const u32x4 a = *(const u32x4*)(kt + k_base + ks * 1024);
            s = Tr::mfma(__builtin_bit_cast(vec8, a), qf[ks], s);
        }
        const int base = (t_begin + t) * 32 + 16 * hh;
        const int lo_rel = my_lo32 - base, hi_rel = my_hi32 - base;
        float mt = neg_inf();
#pragma unroll
        for (int v = 0; v < 16; ++v) {
            float x;
            if constexpr (MT != 0) {
                // natural units (kfac = log2 e): softcap first, then the mask
                x = SOFTCAP ? __builtin_fmaf(p.softcap, tanh_fast(s[v] * p.cap_y), mv[v])
                            : __builtin_fmaf(s[v], p.scale, mv[v]);
            } else if constexpr (SOFTCAP) {
                x = tanh_fast(s[v] * p.cap_y);
            } else {
                x = RAW ? s[v] : s[v] * p.scale;
            }
            x = (v >= lo_rel && v <= hi_rel) ? x : neg_inf();
            s[v] = x;
            mt = __builtin_fmaxf(mt, x);
        }
        mt = half_swap_max(mt);
        const bool need = mt > m_run + th_x;
        if (wave_any(need)) {
            const float m_new = need ? mt : m_run;
            const float alpha = need ? exp2_hw((m_run - m_new) * kfac) : 1.0f;
#pragma unroll
            for (int i = 0; i < NDB; ++i) o[i] *= alpha;
            l_run *= alpha;
            m_run = m_new;
        }
        const float m_safe = m_run == neg_inf() ? 0.0f : m_run;
#pragma unroll
        for (int v = 0; v < 16; ++v) s[v] = exp2_hw((s[v] - m_safe) * kfac);
        vec8 pf[2];
        pf[0] = __builtin_convertvector(__builtin_shufflevector(s, s, 0, 1, 2, 3, 4, 5, 6, 7), vec8);
        pf[1] = __builtin_convertvector(__builtin_shufflevector(s, s, 8, 9, 10, 11, 12, 13, 14, 15), vec8);
#pragma unroll
        for (int q = 0; q < 8; ++q)
            l_run = Tr::sum2(vec2{pf[q >> 2][2 * (q & 3)], pf[q >> 2][2 * (q & 3) + 1]}, l_run);
#pragma unroll
        for (int f = 0; f < 2 * NDB; ++f) {
            const int j = f / NDB, db = f % NDB;
            const u32x2 lo2 = __builtin_bit_cast(u32x2, __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                (lds_s16x4*)(vt + v_base + db * 2048 + (8 * j) * 64)));
            const u32x2 hi2 = __builtin_bit_cast(u32x2, __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                (lds_s16x4*)(vt + v_base + db * 2048 + (8 * j + 4) * 64)));
            o[db] = Tr::mfma(__builtin_bit_cast(vec8, u32x4{lo2[0], lo2[1], hi2[0], hi2[1]}), pf[j], o[db]);
        }
    };

    if (n_tiles > 0) load(0, ra_k, ra_v);
    if (n_tiles > 1) load(1, rb_k, rb_v);
    if (n_tiles > 0) store(0, ra_k, ra_v);
    for (int t = 0; t < n_tiles; t += 2) {
        compute(t, 0);
        if (t + 2 < n_tiles) load(t + 2, ra_k, ra_v);
        if (t + 1 < n_tiles) {
            store(1, rb_k, rb_v);
            compute(t + 1, 1);
            if (t + 3 < n_tiles) load(t + 3, rb_k, rb_v);
        }
        if (t + 2 < n_tiles) store(0, ra_k, ra_v);
    }

    // this span's state of row lr: lane (lr, hh) holds dims 32 db + 8 a + 4 hh .. +3; padding
    // rows are not written (the merge reads rows below sp.rows only)
    const float l_row = half_swap_sum(l_run);
    if (!row_valid) return;
    const int64_t srow = ((int64_t)split * (p.batch * p.kv_heads) + grp) * 32 + lr;
    float* const orow = sp.ws_o + srow * DP;
#pragma unroll
    for (int db = 0; db < NDB; ++db) {
#pragma unroll
        for (int a = 0; a < 4; ++a)
            *(f32x4*)(orow + 32 * db + 8 * a + 4 * hh) =
                f32x4{o[db][4 * a], o[db][4 * a + 1], o[db][4 * a + 2], o[db][4 * a + 3]};
    }
    if (hh == 0) {
        sp.ws_m[srow] = m_run;
        sp.ws_l[srow] = l_row;
    }
}

// Merge of the spans: thread (output row, 4 dims).
template <typename Tr, int DP>
__global__ void __attribute__((amdgpu_flat_work_group_size(256, 256)))
splitkv_merge_kernel(const FwdParams p, const SplitParams sp) {
    using scalar = typename Tr::scalar;
    typedef scalar vec4s __attribute__((ext_vector_type(4)));
    constexpr int C4 = DP / 4;
    const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
    const int64_t n_rows = (int64_t)p.batch * p.heads * p.sq;
    if (idx >= n_rows * C4) return;
    const int64_t orow_i = idx / C4;
    const int d = (int)(idx - orow_i * C4) * 4;
    // output row (b, h, i)
    const int64_t bh = orow_i / p.sq;
    const int i = (int)(orow_i - bh * p.sq);
    const int b = (int)(bh / p.heads), h = (int)(bh - (int64_t)b * p.heads);
    const int kvh = h / p.group;
    const int grp = b * p.kv_heads + kvh;
    const int r = i * p.group + (h - kvh * p.group);
    const int64_t groups = (int64_t)p.batch * p.kv_heads;
    // the loops carry no load-dependent branch, so the loads of several spans are in flight
    // together (a span without keys has m = -inf, l = 0, O = 0 and gets weight 0)
    const int64_t step = groups * 32;
    const int64_t r0 = (int64_t)grp * 32 + r;
    float big = neg_inf();
#pragma unroll 8
    for (int s = 0; s < sp.num_splits; ++s) big = __builtin_fmaxf(big, sp.ws_m[r0 + s * step]);
    f32x4 acc = f32x4(0.0f);
    float den = 0.0f;
    if (big != neg_inf()) {
#pragma unroll 8
        for (int s = 0; s < sp.num_splits; ++s) {
            const int64_t srow = r0 + s * step;
            const float wgt = exp2_hw((sp.ws_m[srow] - big) * p.kfac);
            den += wgt * sp.ws_l[srow];
            acc += wgt * *(const f32x4*)(sp.ws_o + srow * DP + d);
        }
    }
    const float inv = den > 0.0f ? 1.0f / den : 0.0f;
    scalar* dst = (scalar*)p.out + (int64_t)b * p.o_stride_b + (int64_t)h * p.o_stride_h + (int64_t)i * p.o_stride_i + d;
    *(vec4s*)dst = __builtin_convertvector(acc * inv, vec4s);
}

template <typename Tr, int DP, bool SOFTCAP, bool RAW, int MT>
hipError_t launch_splitkv_one(const FwdParams& p, const SplitParams& sp, hipStream_t s) {
    const int groups = p.batch * p.kv_heads;
    hipLaunchKernelGGL((splitkv_kernel<Tr, DP, SOFTCAP, RAW, MT>), dim3(groups * (sp.num_splits / 4)),
                       dim3(kSplitThreads), 0, s, p, sp);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    const int64_t threads = (int64_t)p.batch * p.heads * p.sq * (DP / 4);
    hipLaunchKernelGGL((splitkv_merge_kernel<Tr, DP>), dim3((unsigned)((threads + 255) / 256)), dim3(256), 0, s, p, sp);
    return hipGetLastError();
}

template <typename Tr, int DP>
hipError_t launch_splitkv_dp(const FwdParams& p, const SplitParams& sp, int maskk, hipStream_t s) {
    const bool cap = p.softcap > 0.0f;
    if (maskk == 1) return cap ? launch_splitkv_one<Tr, DP, true, false, 1>(p, sp, s)
                               : launch_splitkv_one<Tr, DP, false, false, 1>(p, sp, s);
    if (maskk == 2) return cap ? launch_splitkv_one<Tr, DP, true, false, 2>(p, sp, s)
                               : launch_splitkv_one<Tr, DP, false, false, 2>(p, sp, s);
    if (cap) return launch_splitkv_one<Tr, DP, true, false, 0>(p, sp, s);
    return p.raw_scores ? launch_splitkv_one<Tr, DP, false, true, 0>(p, sp, s)
                        : launch_splitkv_one<Tr, DP, false, false, 0>(p, sp, s);
}

// maskk: 0 none, 1 float32 mask, 2 mask of the input type
template <typename Tr>
hipError_t launch_splitkv(const FwdParams& p, const SplitParams& sp, int dp, int maskk, hipStream_t s) {
    return dp == 64 ? launch_splitkv_dp<Tr, 64>(p, sp, maskk, s) : launch_splitkv_dp<Tr, 128>(p, sp, maskk, s);
}

}  // namespace fa
