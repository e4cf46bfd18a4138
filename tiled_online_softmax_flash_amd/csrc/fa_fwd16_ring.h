// Tiled online-softmax attention forward, 16-bit inputs, head dim 64 or 128 (gfx950 fast path).
//
// Same method as fa_fwd16.h (tile-granular online softmax with a running maximum, denominator
// and rescaled numerator, per the onnx-runtime-ep-cuda page `src/kernels/flash_attention.rs`,
// `flash_attention_body`), laid out for a whole CDNA4 compute unit per workgroup:
//
//   * 8 waves x 32 query rows = 256 rows per workgroup, one workgroup per CU, 2 waves per SIMD.
//     Every K/V tile staged in LDS serves 256 rows.
//   * K/V tiles of 64 keys stream through a 4-slot LDS ring with 16-byte buffer-to-LDS loads
//     (no staging registers), issued three tiles ahead; one barrier per tile.  Each tile's
//     buffer descriptor ends at the last valid key, so rows past the cache length arrive as 0.
//     K slots fill the lower part of the LDS and V slots the upper part, and the tile loop is
//     unrolled by the ring depth, so every LDS operand read is a per-lane base register plus
//     an immediate offset.
//   * LDS layouts are chosen lane by lane through the DMA source addresses.  Each 32-key half of
//     a tile is stored operand-block-major, so that one per-lane base address serves every MFMA
//     operand of a block and the bank pattern holds without per-read swizzle arithmetic:
//       K: [16-dim slice ks][row r][32 bytes]; row r holds key kk(r) (see lds_row_of_key) and
//          its two 16-byte chunks trade places when bit 3 of r is set, so the 16 rows one
//          16-byte read cycle touches hit 16 different bank slots;
//       V: [32-dim block db][key][64 bytes].  V^T operands come from ds_read_b64_tr_b16, which
//          transposes 4 keys x 4 dims per 16-lane group; the 4 consecutive keys one read cycle
//          touches fill all 64 banks.  V is never transposed in registers.
//   * Work per half-tile of 32 keys: S^T = K Q^T and O^T += V^T P^T on 32x32x16 MFMA.  The
//     schedule is software-pipelined by one half-tile: block u issues the P.V products of
//     half-tile u-1 and the Q.K products of half-tile u+1 back to back on the matrix cores and
//     spreads the softmax of half-tile u (VALU) between them, so that both units stay busy in
//     every wave.
#pragma once

#include <type_traits>

#include "fa_device.h"
#include "fa_fwd16.h"
#include "fa_fwd16_ring_consts.h"

namespace fa {

template <int N>
using int_c = std::integral_constant<int, N>;

// f(int_c<I>{}) for I in [B, E), unrolled at compile time.
template <int B, int E, typename F>
__device__ __forceinline__ void static_for(F&& f) {
    if constexpr (B < E) {
        f(int_c<B>{});
        static_for<B + 1, E>(f);
    }
}

// Mask values of one half-tile for one lane (16 keys), exactly as loaded: fp32 words, or
// 16-bit values packed two per word.
template <int MASKK> struct MaskHalf {};
template <> struct MaskHalf<kMaskF32> { u32x4 w[4]; };
template <> struct MaskHalf<kMaskT> { u32x2 w[4]; };

// Vector loads issued through inline asm, like the K/V ring's DMA: the kernel places their
// waits itself (they retire before the dma_wait that ends the ring step after their issue),
// where the compiler's wait-count pass would drain the whole K/V ring in flight.  Their result
// registers must not be read before that wait; launder() hands them on after it.
__device__ __forceinline__ u32x4 vload_b128(u32x4 rsrc, uint32_t voff) {
    u32x4 r;
    asm volatile("buffer_load_dwordx4 %0, %1, %2, 0 offen" : "=v"(r) : "v"(voff), "s"(rsrc));
    return r;
}
__device__ __forceinline__ u32x2 vload_b64(u32x4 rsrc, uint32_t voff) {
    u32x2 r;
    asm volatile("buffer_load_dwordx2 %0, %1, %2, 0 offen" : "=v"(r) : "v"(voff), "s"(rsrc));
    return r;
}
template <int MASKK>
__device__ __forceinline__ void launder(MaskHalf<MASKK>& m) {
    if constexpr (MASKK != kMaskNone) {
#pragma unroll
        for (int c = 0; c < 4; ++c) asm volatile("" : "+v"(m.w[c]));
    }
}

// parts of a pipelined block (see the block body)
constexpr int kBlkPV = 1, kBlkQK = 2, kBlkSM = 4, kBlkEnd = 8, kBlkExact = 16;

// SOFTCAP: 0 none, 1 tanh_fast, 2 tanh_identity (softcap <= kTanhIdentityMaxCap).
template <typename Tr, int DP, int MASKK, int SOFTCAP, bool RAW, int RB>
__global__ void __attribute__((amdgpu_flat_work_group_size(ring_threads(RB), ring_threads(RB)),
                               amdgpu_waves_per_eu(RB == 1 ? 2 : 1, RB == 1 ? 2 : 1)))
fwd16_ring_kernel(const FwdParams p) {
    using vec8 = typename Tr::vec8;
    using vec4 = typename Tr::vec4;
    using vec2 = typename Tr::vec2;
    using scalar = typename Tr::scalar;
    typedef short s16x4 __attribute__((ext_vector_type(4)));
    typedef __attribute__((address_space(3))) s16x4 lds_s16x4;
    constexpr int WAVES = ring_threads(RB) / 64;
    constexpr int WROWS = kWaveRows * RB;        // query rows per wave: RB blocks of 32
    constexpr int BN = 64, HB = 32, STAGES = 4;
    constexpr int ROWB = DP * 2;                 // bytes per K/V row
    constexpr int CPR = DP / 8;                  // 16-byte chunks per row
    constexpr int TILE_BYTES = BN * ROWB;
    constexpr int V_REGION = STAGES * TILE_BYTES;   // K slots [0, V_REGION), V slots after
    // Every wave issues an equal share of the K/V ring loads, one load at a time between the
    // MFMAs of a step's first block: a burst of loads at the start of a step would hold up the
    // issuing wave's MFMA stream (and the whole workgroup at the step's barrier) while the
    // loads are accepted.
    constexpr int DMA_WAVES = WAVES;
    constexpr int LDW = TILE_BYTES / 1024 / DMA_WAVES;  // 1 KiB DMA ops per loading wave per operand per tile
    constexpr int NKS = DP / 16;                 // Q.K MFMAs per half-tile
    constexpr int NDB = DP / 32;                 // 32-dim output blocks
    constexpr bool MASKED = MASKK != kMaskNone;
    constexpr bool SUB_FIRST = MASKED;
    // head dim 64, masked: a step's mask values are loaded one step ahead.  With an fp32 mask
    // they come through a per-wave LDS buffer filled by whole-line DMA: loading them straight
    // into the lanes that use them makes every load touch 32 rows' cache lines, and those line
    // lookups, not the bytes, bounded the kernel.
    constexpr bool MASK_AHEAD = MASKED && DP == 64;
    constexpr bool MASK_LDS = MASK_AHEAD && MASKK == kMaskF32 && RB == 1;
    // RAW with a mask: the scale is a power of two that Q takes exactly (multiplied in once per
    // item), and each half-tile's Q.K products start from its mask values instead of zero, so
    // the accumulators hold scale * (Q.K) + mask and the scores need no per-element
    // multiply-add.  The second block of a step then reads the mask of the next step's first
    // half-tile: only the LDS-staged fp32 mask has it in registers by then (read out at the end
    // of the step before); the 16-bit masks' loads of that step are still in flight.
    constexpr bool MASK_ACC = MASKED && RAW;
    static_assert(!MASK_ACC || (MASK_LDS && SOFTCAP == 0), "mask accumulation needs the LDS-staged mask");
    constexpr int MSK_WAVE = 2 * 32 * 128;   // one step's fp32 mask of a wave: 2 half-tiles x 32 rows x 128 B
    // LDS operand reads kept in flight ahead of their MFMA; the masked head-dim-128 variants hold
    // a step's mask values as well, and the head-dim-128 variants with a softcap or a scale
    // multiply, and the fp32-masked head-dim-64 ones with a softcap, keep fewer too, so that no
    // register spills (a spill copy of a register that an asm load has
    // not filled yet would save stale data)
    constexpr int AHEAD = MASKK != kMaskNone && DP == 128 ? 6
                        : (SOFTCAP != 0 || !RAW) && DP == 128 ? 10
                        : MASK_LDS && SOFTCAP != 0 ? 10 : 12;
    constexpr int NPRE = 4 * NDB < AHEAD ? 4 * NDB : AHEAD;   // V reads a block issues for the next one
    using MaskH = MaskHalf<MASKK>;
    static_assert(DP == 64 || DP == 128, "ring kernel covers head dims 64 and 128");
    static_assert(LDW >= 1 && LDW * DMA_WAVES * 1024 == TILE_BYTES, "tile must split evenly over the loading waves");
    static_assert((STAGES - 1) * TILE_BYTES + HB * ROWB + 12 * ROWB + 8 < 65536,
                  "LDS operand offsets must fit the 16-bit immediate");

    // LDS: the K/V ring, then each wave's item table (TBL_ROUNDS rounds of 32 bytes), then each
    // wave's output staging buffer (8 chunks of 32 lanes x 8 bytes, each padded by 32 bytes so
    // that the 4 rows x 8 chunks one read-back half-wave touches fill all 64 banks)
    constexpr int TBL_ROUNDS = 32;
    constexpr int TBL_OFF = 2 * STAGES * TILE_BYTES;
    constexpr int STG_CHUNK = 32 * 8 + 32;
    constexpr int STG_OFF = TBL_OFF + WAVES * TBL_ROUNDS * 32;
    constexpr int MSK_OFF = STG_OFF + WAVES * 8 * STG_CHUNK;   // per-wave mask buffers (MASK_LDS)
    static_assert(MSK_OFF % 128 == 0, "mask buffer rows must start on 128-byte boundaries");
    __shared__ __attribute__((aligned(1024))) char lds[MSK_OFF + (MASK_LDS ? WAVES * MSK_WAVE : 0)];
    static_assert(sizeof(lds) <= 160 * 1024, "LDS budget of one workgroup");
    const uint32_t lds_base = lds_addr(lds);

    const int tid = threadIdx.x;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int lane = tid & 63;
    const int lr = lane & 31;
    const int hh = lane >> 5;
    const int D = DP;
    const float kfac = p.kfac;
    const float th_x = kRescaleLog2 / kfac;
    const float cap_z = p.cap_y * kTanhZ;   // dot product -> argument of tanh_*_z
    // Identity-form softcap without a mask: the speculative softmax (full and partial half-tiles)
    // takes the base-2 exponent k tanh(c s) straight from the dot product s as the odd polynomial
    // s (b1 + s^2 (b3 + b5 s^2)) (the series of tanh, valid while |s| < s_lim); a lane with a
    // larger |s| sends its row through fix_up, which forms the scores exactly.
    constexpr bool POLY = SOFTCAP == 2 && !MASKED;
    const scalar* __restrict__ qg = (const scalar*)p.q;

    // ---- DMA source offsets: DMA op i of a tile writes physical 16-byte chunks [64 i, 64 i + 64)
    // (K and V alike); a half-tile holds HB * CPR chunks.  With q the chunk index inside half H:
    //   K chunk pc of half H: slice ks = q / 64, row r = (q / 2) % 32, position c = q % 2
    //     (q = pc within the half) <- key 32 H + kk(r), dim chunk 2 ks + (c ^ bit 3 of r);
    //   V chunk pc of half H: block db = q / 128, key j = (q / 4) % 32, chunk c = q % 4
    //     <- key 32 H + j, dim chunk 4 db + c.
    constexpr int HALF_CHUNKS = HB * CPR;
    uint32_t k_src[LDW], v_src[LDW];
#pragma unroll
    for (int j = 0; j < LDW; ++j) {
        const int pc = 64 * (wave * LDW + j) + lane;   // chunk index in the tile
        const int hf = pc / HALF_CHUNKS;
        const int q = pc % HALF_CHUNKS;
        {
            const int ks = q / 64, r = (q >> 1) & 31, c = q & 1;
            const int key = 32 * hf + 16 * ((r >> 2) & 1) + 4 * (r >> 3) + (r & 3);   // kk(r)
            k_src[j] = (uint32_t)(key * ROWB + (2 * ks + (c ^ ((r >> 3) & 1))) * 16);
        }
        {
            const int db = q / 128, key = 32 * hf + ((q >> 2) & 31), c = q & 3;
            v_src[j] = (uint32_t)(key * ROWB + (4 * db + c) * 16);
        }
    }

    // ---- mask buffer (MASK_LDS).  Half h of a wave's buffer holds 32 rows x 32 keys; row r is
    // 128 bytes, its logical 16-byte chunk c (keys 4c .. 4c+3) stored at chunk c ^ (r % 8), so
    // that the eight lanes of a 16-byte read cycle (rows r .. r+7, one chunk each) hit different
    // banks.  DMA op j (0..7) fills half j / 4, rows 8 (j % 4) .. +7: lane l takes row
    // 8 (j % 4) + l / 8, physical chunk l % 8.  msk_src: the lane's byte offset in the item's
    // mask rows for ops with j % 4 = 0 (rows 8 further on for each step of j % 4; add the
    // half-tile's key offset); msk_rd: LDS offset of lane (lr, hh)'s logical chunk 4 hh (chunk
    // 4 hh + c is at msk_rd ^ 16 c).
    uint32_t msk_src = 0, msk_rd = 0;
    const uint32_t msk_row8 = (uint32_t)(8 * p.sk * 4);   // 8 mask rows in bytes
    if constexpr (MASK_LDS) {
        const int pr = lane >> 3, pc = lane & 7;
        msk_src = (uint32_t)((int64_t)(wave * WROWS + pr) * p.sk * 4) + (uint32_t)(16 * (pc ^ pr));
        msk_rd = (uint32_t)(MSK_OFF + wave * MSK_WAVE + lr * 128 + 16 * ((4 * hh) ^ (lr & 7)));
    }

    // ---- LDS operand addresses: one per-lane base per operand; ring slot, half-tile, K slice and
    // V block are immediates.
    // K (A operand of S^T = K Q^T): lane (lr, hh) reads row lr, dims 16 ks + 8 hh .. +7.
    const uint32_t k_base = (uint32_t)(lr * 32 + ((hh ^ ((lr >> 3) & 1)) << 4));
    // V^T (A operand of O^T += V^T P^T) through ds_read_b64_tr_b16.  Source lane
    // l = 16 g + 4 k + c points at key 16 hh + 8 j + 4 r + k and dims 32 db + 16 g + 4 c .. +3 of
    // the half-tile (g = bit 4 of l, hh = bit 5); the transpose hands lane l dims d = l % 32 of
    // those four keys.
    const uint32_t v_base = (uint32_t)V_REGION + (uint32_t)((16 * hh + ((lane >> 2) & 3)) * 64 +
                                                            ((lane >> 4) & 1) * 32 + (lane & 3) * 8);

    // ---- Work items (batch, query head, 256-row query tile).  The workgroup is persistent: the
    // workgroup with id j runs on XCD j % 8 and takes, in round r, XCD-local slot
    // r * ncu + (c or ncu - 1 - c) (c = j / 8, ncu = workgroups per XCD; the order within a
    // round alternates so that the heavy-first slot order of decode_work pairs heavy items
    // with light ones on each CU).  While an item runs its last three ring steps, the ring
    // positions past its last tile receive the next item's first three K/V tiles, and its last
    // step loads the next item's Q, so the next item starts with tiles 0 and 1 in LDS and its
    // first step needs no wait or barrier (unmasked variants; masked ones keep their mask buffers
    // busy to the end and start each item afresh).
    const int xcd = blockIdx.x & 7;
    const int cu = blockIdx.x >> 3;
    const int ncu = (int)(gridDim.x >> 3);
    auto slot_of_round = [&](int r) -> int { return r * ncu + ((r & 1) ? ncu - 1 - cu : cu); };
    struct ItemGeo {
        WorkItem w;
        KeyRule rule;
        int64_t q0, q_last;
        int kt_begin, n_tiles;
        const char* kg;
        const char* vg;
    };
    // Item table: lane i of a wave works out round r0 + i's work item, key rule and key-tile
    // range (one vector pass for TBL_ROUNDS rounds instead of a scalar pass per round) into the
    // wave's own table; a round reads its entry back.  Entry: b, h, qt, valid | kt_begin,
    // n_tiles, L, base (the key rule's cache length and causal base).
    char* const tbl = lds + TBL_OFF + wave * (TBL_ROUNDS * 32);
    auto fill_table = [&](int r0) __attribute__((always_inline)) {
        const int slot = slot_of_round(r0 + lane);
        WorkItem w = decode_work(p, slot * 8 + xcd);
        w.valid = w.valid && slot < p.items_per_xcd;
        if (!w.valid) w.b = w.h = w.qt = 0;   // never index past the inputs
        const KeyRule rule = make_rule(p, w.b);
        const int64_t q0 = (int64_t)w.qt * kRingBlockRows;
        const int64_t q_last = (q0 + kRingBlockRows < p.sq ? q0 + kRingBlockRows : p.sq) - 1;
        const int64_t lo_wg = rule.lo(q0), hi_wg = rule.hi(q_last);
        const int kt_begin = hi_wg >= lo_wg ? (int)(lo_wg / BN) : 0;
        const int n_tiles = hi_wg >= lo_wg ? (int)(hi_wg / BN) - kt_begin + 1 : 0;
        if (lane < TBL_ROUNDS) {
            *(u32x4*)(tbl + 32 * lane) = u32x4{(uint32_t)w.b, (uint32_t)w.h, (uint32_t)w.qt, w.valid ? 1u : 0u};
            *(u32x4*)(tbl + 32 * lane + 16) =
                u32x4{(uint32_t)kt_begin, (uint32_t)n_tiles, (uint32_t)rule.L, (uint32_t)(int32_t)rule.base};
        }
    };
    auto item_geo = [&](int r) __attribute__((always_inline)) -> ItemGeo {
        const u32x4 e0 = *(const u32x4*)(tbl + 32 * (r & (TBL_ROUNDS - 1)));
        const u32x4 e1 = *(const u32x4*)(tbl + 32 * (r & (TBL_ROUNDS - 1)) + 16);
        ItemGeo g;
        g.w.b = __builtin_amdgcn_readfirstlane((int)e0[0]);
        g.w.h = __builtin_amdgcn_readfirstlane((int)e0[1]);
        g.w.qt = __builtin_amdgcn_readfirstlane((int)e0[2]);
        g.w.valid = __builtin_amdgcn_readfirstlane((int)e0[3]) != 0;
        g.kt_begin = __builtin_amdgcn_readfirstlane((int)e1[0]);
        g.n_tiles = __builtin_amdgcn_readfirstlane((int)e1[1]);
        g.rule.L = __builtin_amdgcn_readfirstlane((int)e1[2]);
        g.rule.base = __builtin_amdgcn_readfirstlane((int)e1[3]);
        g.rule.window = p.window;
        g.rule.causal = p.causal;
        g.q0 = (int64_t)g.w.qt * kRingBlockRows;
        g.q_last = (g.q0 + kRingBlockRows < p.sq ? g.q0 + kRingBlockRows : p.sq) - 1;
        const int kvh = g.w.h / p.group;
        g.kg = (const char*)p.k + ((int64_t)g.w.b * p.kv_heads + kvh) * p.kv_capacity * ROWB;
        g.vg = (const char*)p.v + ((int64_t)g.w.b * p.kv_heads + kvh) * p.kv_capacity * ROWB;
        return g;
    };
    // Q fragment loads of one item into q: lane (m, hh) of row block rb holds
    // Q[row][16*ks + 8*hh .. +7].  Through inline asm like the K/V ring, so that a ring wait
    // retires them together with ring tiles and the tile loop holds no register the compiler
    // sees as loaded from memory (its wait-count pass would otherwise drain the ring).
    auto load_q = [&](const ItemGeo& g, vec8 (&q)[RB][NKS]) __attribute__((always_inline)) {
#pragma unroll
        for (int rb = 0; rb < RB; ++rb) {
            const int64_t r = g.q0 + wave * WROWS + 32 * rb + lr;
            const scalar* qrow = qg + (((int64_t)g.w.b * p.heads + g.w.h) * p.sq + (r < p.sq ? r : 0)) * D;
#pragma unroll
            for (int ks = 0; ks < NKS; ++ks) {
                u32x4 t;
                asm volatile("global_load_dwordx4 %0, %1, off" : "=v"(t) : "v"(qrow + 16 * ks + 8 * hh));
                q[rb][ks] = __builtin_bit_cast(vec8, t);
            }
        }
    };
    // K/V loads of an item go through two buffer descriptors over its (batch, KV head) rows
    // that end with the item's last tile (or the cache length, if shorter): loads of positions
    // past that end, and every load of an invalid item, read zeros.  A tile is then a byte
    // offset into them.  A plan for one tile is worked out on the scalar unit; its NDMA loads
    // per wave are issued one by one.
    struct ItemDma {
        u32x4 rk, rv;
        int tile0;   // the item's first key tile
    };
    auto item_dma = [&](const ItemGeo& g) __attribute__((always_inline)) -> ItemDma {
        int64_t keys_end = (int64_t)(g.kt_begin + g.n_tiles) * BN;
        if (keys_end > g.rule.L) keys_end = g.rule.L;
        if (!g.w.valid || g.n_tiles <= 0) keys_end = 0;
        const int bytes = (int)(keys_end * ROWB);
        ItemDma d;
        d.rk = make_rsrc_words(g.kg, bytes);
        d.rv = make_rsrc_words(g.vg, bytes);
        d.tile0 = g.kt_begin;
        return d;
    };
    struct DmaPlan {
        u32x4 rk, rv;
        uint32_t off;      // byte offset of the tile in the K and V rows
        uint32_t sk, sv;   // LDS addresses of the ring slot's K and V halves
    };
    constexpr int NDMA = 2 * LDW;   // ring loads per wave per tile: K and V alternately
    // load i of this wave's share of a planned tile (1 KiB of K for even i, of V for odd i)
    auto dma_issue = [&](const DmaPlan& d, auto i_c) __attribute__((always_inline)) {
        constexpr int i = decltype(i_c)::value, j = i / 2;
        const uint32_t op = (uint32_t)__builtin_amdgcn_readfirstlane(wave * LDW + j);
        if constexpr (i % 2 == 0) dma_lds16(d.rk, d.sk + 1024u * op, k_src[j] + d.off);
        else dma_lds16(d.rv, d.sv + 1024u * op, v_src[j] + d.off);
    };
    auto dma_issue_all = [&](const DmaPlan& d) __attribute__((always_inline)) {
        static_for<0, NDMA>([&](auto i_c) __attribute__((always_inline)) { dma_issue(d, i_c); });
    };
    // Wait until every ring load of this wave but the last tile's has landed (loads issued
    // before that tile included).
    auto ring_wait = [&]() __attribute__((always_inline)) { dma_wait<NDMA>(); };

    int ring_base = 0;     // ring position of the current item's tile 0 (slot = position % 4)
    bool pre = false;      // the current item's Q and first two tiles are already in flight
    // Q fragments of the current item.  With pre, the previous item's last ring step loaded them
    // in place: that step's own Q.K products only score half-tiles past its item, which no later
    // block reads, so they may read these registers while the loads are in flight.
    vec8 qf[RB][NKS];
    fill_table(0);
    ItemGeo cur = item_geo(0);
    for (int round = 0; cur.w.valid; ++round) {
    if (((round + 1) & (TBL_ROUNDS - 1)) == 0) fill_table(round + 1);   // (this round's entry is read)
    const ItemGeo nxt = item_geo(round + 1);
    const WorkItem w = cur.w;
    const int b = w.b, h = w.h;
    const KeyRule rule = cur.rule;
    const int64_t q0 = cur.q0;
    const int64_t q_last = cur.q_last;
    const int64_t wr0 = q0 + wave * WROWS;
    const bool wave_has_rows = wr0 < p.sq;
    const int64_t wr1 = (wr0 + WROWS - 1 < p.sq ? wr0 + WROWS - 1 : p.sq - 1);
    // row block rb of the wave: rows wr0 + 32 rb + (0..31); lane (lr, hh) owns row wr0 + 32 rb + lr
    int64_t row[RB];
    bool row_valid[RB];
    int my_lo32[RB], my_hi32[RB];
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
        row[rb] = wr0 + 32 * rb + lr;
        row_valid[rb] = row[rb] < p.sq;
        const int64_t lo = row_valid[rb] ? rule.lo(row[rb]) : 1;
        const int64_t hi = row_valid[rb] ? rule.hi(row[rb]) : 0;
        my_lo32[rb] = (int)(lo < 0x7fffffffLL ? lo : 0x7fffffffLL);
        my_hi32[rb] = (int)(hi > -1 ? hi : -1);
    }

    const int kt_begin = cur.kt_begin;
    const int n_tiles = cur.n_tiles;

    if (!pre) load_q(cur, qf);
    auto launder_q = [&]() __attribute__((always_inline)) {
#pragma unroll
        for (int rb = 0; rb < RB; ++rb) {
#pragma unroll
            for (int ks = 0; ks < NKS; ++ks) {
                u32x4 t = __builtin_bit_cast(u32x4, qf[rb][ks]);
                asm volatile("" : "+v"(t));
                qf[rb][ks] = row_valid[rb] ? __builtin_bit_cast(vec8, t) : vec8((scalar)0.0f);
                if constexpr (MASK_ACC) {
                    // exact: a power-of-two scale only moves the exponent
                    typedef float f32x8 __attribute__((ext_vector_type(8)));
                    qf[rb][ks] = __builtin_convertvector(__builtin_convertvector(qf[rb][ks], f32x8) * p.scale, vec8);
                }
            }
        }
    };

    // ---- mask rows of this workgroup (rows are 16-byte aligned: the dispatcher checks it)
    constexpr uint32_t MESZ = MASKK == kMaskF32 ? 4u : 2u;
    u32x4 rmask = u32x4{0u, 0u, 0u, 0u};
    const char* mbase = nullptr;   // the item's first mask row
    int64_t mask_bytes = 0;        // bytes of the item's mask rows
    uint32_t mask_row_off[RB];
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) mask_row_off[rb] = 0;
    if constexpr (MASKED) {
        const int64_t rows_here = q_last - q0 + 1;
        mbase = (const char*)p.mask + ((mask_plane(p, b, h) * p.sq + q0) * (int64_t)p.sk) * MESZ;
        mask_bytes = rows_here * p.sk * MESZ;
        rmask = make_rsrc_words(mbase, (int)mask_bytes);
#pragma unroll
        for (int rb = 0; rb < RB; ++rb) mask_row_off[rb] = (uint32_t)((row[rb] - q0) * (int64_t)p.sk) * MESZ;
    }

    f32x16 o[RB][NDB];
    // running maximum m (-inf: no key yet), denominator, and the exponent offset the weights
    // are taken against: m_safe = m (0 while m is -inf) and nmk = -m_safe * k
    float m_run[RB], l_run[RB], m_safe_run[RB], nmk_run[RB];
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
#pragma unroll
        for (int i = 0; i < NDB; ++i) o[rb][i] = f32x16(0.0f);
        m_run[rb] = neg_inf();
        l_run[rb] = 0.0f;
        m_safe_run[rb] = 0.0f;
        nmk_run[rb] = 0.0f;
    }

    // The item's tile t sits at ring position ring_base + t.  A step issues ring position
    // t + 3: the item's own tile while there is one, then (pre_next) the next item's tiles 0, 1
    // and 2 at positions t_last + 1 .. t_last + 3 (issued by steps t_last - 2 .. t_last; the
    // last step's Q.K products, which score past the item, read position t_last + 1), else an
    // empty tile.
    // steps 0 .. n_steps - 1 follow step -1; masked variants run steps in pairs (their mask
    // buffers alternate), so their step count is even
    const int n_steps = MASKED ? 2 * ((n_tiles + 1) / 2) : n_tiles;
    const int t_last = n_steps - 1;   // last ring step of the item (steps -1 .. t_last)
    // (one row block per wave; at least three tiles, so that positions t_last + 1 .. t_last + 3
    // are issued by the item's own steps)
    const bool pre_next = RB == 1 && !MASKED && nxt.w.valid && nxt.n_tiles > 0 && n_tiles >= 3;
    const ItemDma cdma = item_dma(cur);
    const ItemDma ndma = item_dma(nxt);
    auto plan_tile = [&](int t) __attribute__((always_inline)) -> DmaPlan {
        const bool to_next = pre_next && t > t_last;
        DmaPlan d;
        d.rk = to_next ? ndma.rk : cdma.rk;
        d.rv = to_next ? ndma.rv : cdma.rv;
        d.off = (uint32_t)(to_next ? ndma.tile0 + (t - t_last - 1) : cdma.tile0 + t) * (uint32_t)TILE_BYTES;
        const uint32_t so = (uint32_t)((ring_base + t) & (STAGES - 1)) * TILE_BYTES;
        d.sk = lds_base + so;
        d.sv = lds_base + V_REGION + so;
        return d;
    };

    const int key_base = kt_begin * BN;
    auto half_k0 = [&](int u) __attribute__((always_inline)) { return key_base + HB * u; };

    // mask values of half-tile u for this lane: keys half_k0(u) + 16 hh + 0..15.  Keys past sk
    // read the next row (or zeros past the buffer): they are structurally masked anyway.
    auto load_mask_half = [&](int u, MaskH (&mh)[RB]) __attribute__((always_inline)) {
        if constexpr (MASKED) {
#pragma unroll
            for (int rb = 0; rb < RB; ++rb) {
                const uint32_t off = mask_row_off[rb] + (uint32_t)(half_k0(u) + 16 * hh) * MESZ;
#pragma unroll
                for (int c = 0; c < 4; ++c) {
                    if constexpr (MASKK == kMaskF32) mh[rb].w[c] = vload_b128(rmask, off + 16u * c);
                    else mh[rb].w[c] = vload_b64(rmask, off + 8u * c);
                }
            }
        }
    };
    auto launder_mask = [&](MaskH (&mh)[RB]) __attribute__((always_inline)) {
#pragma unroll
        for (int rb = 0; rb < RB; ++rb) launder(mh[rb]);
    };
    // MASK_LDS: DMA of ring step s's mask (half-tiles 2s+1, 2s+2) into the wave's buffer, and
    // the buffer's two halves into the lanes' mask registers
    auto mask_dma_op = [&](int s, auto j_c) __attribute__((always_inline)) {
        if constexpr (MASK_LDS) {
            constexpr int j = decltype(j_c)::value;
            const uint32_t dst = lds_base + (uint32_t)(MSK_OFF + wave * MSK_WAVE);
            // The descriptor starts at the half-tile's first key of the item's first row (and ends
            // where the item's mask rows end), so that the lane offsets stay fixed: the same
            // bounds check as an offset from the rows' start, with no per-load vector addition.
            const int64_t koff = (int64_t)half_k0(2 * s + 1 + j / 4) * 4;
            const int64_t left = mask_bytes - koff;
            const u32x4 rm = make_rsrc_words(mbase + koff, left > 0 ? (int)left : 0);
            dma_lds16(rm, dst + 1024u * j, msk_src + (uint32_t)(j % 4) * msk_row8);
        }
    };
    auto mask_dma = [&](int s) __attribute__((always_inline)) {
        static_for<0, 8>([&](auto j_c) __attribute__((always_inline)) { mask_dma_op(s, j_c); });
    };
    auto mask_from_lds = [&](MaskH (&mh)[2][RB]) __attribute__((always_inline)) {
        if constexpr (MASK_LDS) {
#pragma unroll
            for (int hf = 0; hf < 2; ++hf)
#pragma unroll
                for (int c = 0; c < 4; ++c) mh[hf][0].w[c] = *(const u32x4*)(lds + (msk_rd ^ (16u * c)) + hf * (32 * 128));
        }
    };
    auto mask_val = [&](const MaskH& mh, int v) __attribute__((always_inline)) -> float {
        if constexpr (MASKK == kMaskF32) {
            return __uint_as_float(mh.w[v >> 2][v & 3]);
        } else if constexpr (MASKK == kMaskT) {
            const uint32_t word = mh.w[v >> 2][(v >> 1) & 1];
            const uint16_t bits = (uint16_t)((v & 1) ? (word >> 16) : (word & 0xffffu));
            return (float)__builtin_bit_cast(scalar, bits);
        } else {
            return 0.0f;
        }
    };

    // ---- wave-uniform half-tile ranges.  Half-tile u covers keys [half_k0(u), half_k0(u) + 31].
    // active [ua, ub]: some row of the wave attends some key of it; full [fa, fb]: every row of
    // the wave attends every key of it.  Both ranges are contiguous because lo and hi grow with
    // the row.
    const int n_half = 2 * n_tiles;
    auto clamp32 = [](int64_t v) -> int { return (int)(v < -1 ? -1 : (v > 0x7fffffffLL ? 0x7fffffffLL : v)); };
    // lo and hi of the wave's first and last rows, evaluated on lanes 0 and 1: as both grow
    // with the row, they bound those of every row of the wave
    int wlo_min, wlo_max, whi_min, whi_max;
    {
        const int64_t ext_row = (lane & 1) ? wr1 : wr0;
        const int e_lo = clamp32(rule.lo(ext_row)), e_hi = clamp32(rule.hi(ext_row));
        wlo_min = __builtin_amdgcn_readlane(e_lo, 0);
        wlo_max = __builtin_amdgcn_readlane(e_lo, 1);
        whi_min = __builtin_amdgcn_readlane(e_hi, 0);
        whi_max = __builtin_amdgcn_readlane(e_hi, 1);
    }
    const bool wave_live = wave_has_rows && wlo_min <= whi_max;
    int ua, ub, fa, fb;
    {
        // (bounds lie in [-1, 2^31 - 1] and key_base in [0, 2^30): no step overflows 32 bits)
        auto fdiv = [](int x) -> int { return x >> 5; };      // floor(x / HB)
        auto cdiv = [](int x) -> int { return -((-x) >> 5); };  // ceil(x / HB)
        auto clip = [&](int x) -> int { return x < -1 ? -1 : (x > n_half ? n_half : x); };
        static_assert(HB == 32, "fdiv/cdiv divide by 32");
        int a = cdiv(wlo_min - key_base - (HB - 1));
        int z = fdiv(whi_max - key_base);
        a = a < 0 ? 0 : a;
        z = z > n_half - 1 ? n_half - 1 : z;
        if (!wave_live) { a = 0; z = -1; }
        ua = clip(a);
        ub = clip(z);
        fa = clip(cdiv(wlo_max - key_base));
        fb = clip(fdiv(whi_min - key_base - (HB - 1)));
    }
    // full(u) implies that the wave attends half-tile u: [fa, fb] lies inside [ua, ub]
    auto full = [&](int u) __attribute__((always_inline)) { return u >= fa && u <= fb; };

    // score epilogue of one element: tracked units x (see RAW / SOFTCAP / MASKED)
    auto epi = [&](float sv, float mvv) __attribute__((always_inline)) -> float {
        if constexpr (SOFTCAP) {
            const float th = tanh_fast(sv * p.cap_y);
            return MASKED ? __builtin_fmaf(p.softcap, th, mvv) : th;
        } else if constexpr (MASK_ACC) {
            return sv;   // scale * (Q.K) + mask, formed by the products
        } else if constexpr (MASKED) {
            return __builtin_fmaf(sv, p.scale, mvv);
        } else if constexpr (!RAW) {
            return sv * p.scale;
        } else {
            return sv;
        }
    };

    // Softmax of half-tile u split in 8 phases so that it can be spread between MFMAs.
    // FULL: the half-tile needs no structural mask.  Two forms:
    //   EXACT (an item's first half-tile): 0, 1: epilogue and maximum of elements 0..7 / 8..15;
    //   2: row maximum across the two lanes of the row, lazy move of the running maximum (only
    //   when the half-tile raises it by more than 2^kRescaleLog2 in weight); 3..6: exponentials
    //   of four elements each; 7: 16-bit packing and the denominator.
    //   Speculative (every later half-tile): no maximum is formed.  The weights are taken
    //   against the running maximum as it stands, p = 2^(x k - m k), which stays valid as long
    //   as no weight grows past kSpecBound
    //   (relative rounding of the 16-bit weights does not depend on their size).  Phases 3..6
    //   leave the scores in sc and pack the weights of each phase one phase later; phase 7 sums
    //   the lane's 16 packed weights.  A lane sum above kSpecBound (which any weight above it
    //   implies), a non-finite sum, or a row with no running maximum yet sends the wave through
    //   fix_up after the block, which redoes the half-tile exactly for the rows concerned.
    // The weights of a half-tile live as 8 words of two 16-bit values (elements 2j, 2j + 1 in word
    // j % 4 of pf[j / 4]); the P.V products take pf[i] whole as their B operand.  A word is
    // copied into a scalar before it is reinterpreted: __builtin_bit_cast applied directly to a
    // vector element reads the vector's first element whatever the index.
    // weights v, v + 1 (v even), rounded to the input type, into their word
    auto set_pair = [](u32x4 (&pf)[2], int v, float p0, float p1) __attribute__((always_inline)) {
        pf[v >> 3][(v & 7) >> 1] = __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2){p0, p1}, vec2));
    };
    // sum of the 16 packed weights (exact products, fp32 accumulation)
    auto sum_packed = [](const u32x4 (&pf)[2], float lsum) __attribute__((always_inline)) -> float {
#pragma unroll
        for (int q = 0; q < 8; ++q) {
            const uint32_t w = pf[q >> 2][q & 3];
            lsum = Tr::sum2(__builtin_bit_cast(vec2, w), lsum);
        }
        return lsum;
    };
    struct SoftmaxState {
        float mt, alpha, m_safe, nmk, lsum, l_prev;
        float pt[4];   // speculative: weights of the last four exponentials, not yet packed
        uint32_t keep;
        bool moved;   // EXACT: the running maximum moved
        bool redo;    // speculative: the row needs fix_up
        bool big;     // speculative, masked: the row's exponent offset is too large to fold in
        float smax;   // speculative, POLY: largest |s| of the lane's scores
        bool fb;      // exact, POLY: some score of the wave is out of the series' range
    };
    auto softmax_phase = [&](auto full_c, auto rb_c, int ph, int u, f32x16& sc, const MaskH& mh, u32x4 (&pf)[2],
                             SoftmaxState& st, auto exact_c) __attribute__((always_inline)) {
        constexpr bool FULL = decltype(full_c)::value;
        constexpr bool EXACT = decltype(exact_c)::value;
        constexpr int rb = decltype(rb_c)::value;
        constexpr bool SPEC_POLY = POLY && !EXACT;
        // exact softmax with POLY: the scores become base-2 exponents k x (the polynomial, or the
        // exact forms times k when some score of the wave is out of the series' range), and the
        // running maximum is taken over them
        constexpr bool EXACT_POLY = POLY && EXACT;
        // bit v of keep: element v (key base + v) lies in the row's key range
        auto set_keep = [&]() __attribute__((always_inline)) {
            const int base = half_k0(u) + 16 * hh;
            const int lo_rel = my_lo32[rb] - base;
            const int hi_rel = my_hi32[rb] - base;
            const uint32_t below_hi = hi_rel < 0 ? 0u : (hi_rel >= 15 ? 0xffffu : (2u << hi_rel) - 1u);
            const uint32_t below_lo = lo_rel <= 0 ? 0u : (lo_rel >= 16 ? 0xffffu : (1u << lo_rel) - 1u);
            st.keep = below_hi & ~below_lo;
        };
        if (SPEC_POLY && (ph == 0 || ph == 1)) {
            // the scores stay raw dot products; only their range is checked (masked elements
            // included: a large one costs a redo, not a wrong result)
            if (ph == 0) {
                st.smax = 0.0f;
                if constexpr (!FULL) set_keep();
            }
#pragma unroll
            for (int e = 0; e < 8; e += 2)
                st.smax = __builtin_fmaxf(__builtin_fmaxf(st.smax, __builtin_fabsf(sc[8 * ph + e])),
                                          __builtin_fabsf(sc[8 * ph + e + 1]));
        } else if (EXACT_POLY && (ph == 0 || ph == 1)) {
            if (ph == 0) {
                st.mt = neg_inf();
                if constexpr (!FULL) set_keep();
                float am = 0.0f;
#pragma unroll
                for (int e = 0; e < 16; e += 2)
                    am = __builtin_fmaxf(__builtin_fmaxf(am, __builtin_fabsf(sc[e])), __builtin_fabsf(sc[e + 1]));
                st.fb = wave_any(!(am < p.tc_slim));
            }
            float ex[8];
            if (!st.fb) {
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    const float sv = sc[8 * ph + e], s2 = sv * sv;
                    ex[e] = sv * __builtin_fmaf(s2, __builtin_fmaf(s2, p.tc_b5, p.tc_b3), p.tc_b1);
                }
            } else {
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    const float z = sc[8 * ph + e] * cap_z;
                    ex[e] = (__builtin_fabsf(z) < kTanhSeriesMaxZ ? tanh_series_z(z) : tanh_identity_z(z)) * kfac;
                }
            }
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const int v = 8 * ph + e;
                float x = ex[e];
                if constexpr (!FULL) {
                    const uint32_t sel = (uint32_t)((int32_t)(st.keep << (31 - v)) >> 31);
                    x = __uint_as_float((sel & __float_as_uint(x)) | (~sel & 0xff800000u));
                }
                sc[v] = x;
                st.mt = __builtin_fmaxf(st.mt, x);
            }
        } else if (ph == 0 || ph == 1) {
            if (ph == 0) {
                st.mt = neg_inf();
                if constexpr (!FULL) set_keep();
            }
            // identity-form softcap: the eight tanh arguments of the phase take the series when
            // all of the wave's are below 1/8 (no transcendental), else the identity
            float th[8];
            if constexpr (SOFTCAP == 2) {
                float z[8];
                float zmax = 0.0f;
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    z[e] = sc[8 * ph + e] * cap_z;
                    zmax = __builtin_fmaxf(zmax, __builtin_fabsf(z[e]));
                }
                if (!wave_any(!(zmax < kTanhSeriesMaxZ))) {
#pragma unroll
                    for (int e = 0; e < 8; ++e) th[e] = tanh_series_z(z[e]);
                } else {
#pragma unroll
                    for (int e = 0; e < 8; ++e) th[e] = tanh_identity_z(z[e]);
                }
            }
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const int v = 8 * ph + e;
                float x;
                if constexpr (SOFTCAP == 2) x = MASKED ? __builtin_fmaf(p.softcap, th[e], mask_val(mh, v)) : th[e];
                else x = epi(sc[v], mask_val(mh, v));
                if constexpr (!FULL) {
                    // all ones where element v is kept, else zero; masked elements become -inf
                    const uint32_t sel = (uint32_t)((int32_t)(st.keep << (31 - v)) >> 31);
                    x = __uint_as_float((sel & __float_as_uint(x)) | (~sel & 0xff800000u));
                }
                sc[v] = x;
                if constexpr (EXACT) st.mt = __builtin_fmaxf(st.mt, x);
            }
        } else if (ph == 2 && !EXACT) {
            st.m_safe = m_safe_run[rb];
            st.nmk = nmk_run[rb];
            // One multiply-add forms x k - m k with nmk = -m k rounded once: an error of at most
            // |m k| 2^-24 in every exponent of the row, a common factor that cancels.  With an
            // additive mask the running maximum can be huge (masks near the float range's end)
            // and that error far above 1: such rows (|m k| > kSpecOffsetMax) always go through
            // fix_up, which forms the difference before scaling.  Without a mask the scores, and
            // so m k, stay moderate.
            if constexpr (MASKED) st.big = !(__builtin_fabsf(st.nmk) <= kSpecOffsetMax);
        } else if (ph <= 6 && !EXACT) {
            // weights of the previous phase's four elements are packed here, a phase (one MFMA)
            // after their exponentials were issued, so the packing never waits for them
            if (ph > 3) {
                const int v0 = 4 * (ph - 4);
                set_pair(pf, v0, st.pt[0], st.pt[1]);
                set_pair(pf, v0 + 2, st.pt[2], st.pt[3]);
            }
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int v = 4 * (ph - 3) + e;
                // (the scores stay in sc for fix_up)
                if constexpr (SPEC_POLY) {
                    const float sv = sc[v], s2 = sv * sv;
                    float ex = __builtin_fmaf(sv, __builtin_fmaf(s2, __builtin_fmaf(s2, p.tc_b5, p.tc_b3), p.tc_b1), st.nmk);
                    if constexpr (!FULL) {
                        // masked elements get the exponent -inf, weight 0
                        const uint32_t sel = (uint32_t)((int32_t)(st.keep << (31 - v)) >> 31);
                        ex = __uint_as_float((sel & __float_as_uint(ex)) | (~sel & 0xff800000u));
                    }
                    st.pt[e] = exp2_hw(ex);
                } else {
                    st.pt[e] = exp2_hw(__builtin_fmaf(sc[v], kfac, st.nmk));
                }
            }
        } else if (ph == 7 && !EXACT) {
            set_pair(pf, 12, st.pt[0], st.pt[1]);
            set_pair(pf, 14, st.pt[2], st.pt[3]);
            const float lsum = sum_packed(pf, 0.0f);
            st.l_prev = l_run[rb];
            l_run[rb] += lsum;
            st.redo = !(lsum <= kSpecBound) || m_run[rb] == neg_inf();
            if constexpr (MASKED) st.redo = st.redo || st.big;
            if constexpr (SPEC_POLY) st.redo = st.redo || !(st.smax < p.tc_slim);
        } else if (ph == 2) {
            // (EXACT_POLY: the maximum of exponents k x, back in units of x; th_x / kRescaleLog2 is
            // 1 / k rounded once, kRescaleLog2 being a power of two)
            static_assert(kRescaleLog2 == 8.0f, "th_x / kRescaleLog2 must be exact");
            const float mt = EXACT_POLY ? half_swap_max(st.mt) * (th_x * (1.0f / kRescaleLog2)) : half_swap_max(st.mt);
            const bool need = mt > m_run[rb] + th_x;
            const float m_new = need ? mt : m_run[rb];
            st.alpha = need ? exp2_hw((m_run[rb] - m_new) * kfac) : 1.0f;
            st.moved = need;
            m_run[rb] = m_new;
            st.m_safe = (m_new == neg_inf()) ? 0.0f : m_new;
            st.nmk = -st.m_safe * kfac;
            m_safe_run[rb] = st.m_safe;
            nmk_run[rb] = st.nmk;
            st.lsum = l_run[rb] * st.alpha;
        } else if (ph <= 6) {
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int v = 4 * (ph - 3) + e;
                float pv_;
                if constexpr (SUB_FIRST) pv_ = exp2_hw((sc[v] - st.m_safe) * kfac);
                else if constexpr (EXACT_POLY) pv_ = exp2_hw(sc[v] + st.nmk);   // (sc holds k x)
                else pv_ = exp2_hw(__builtin_fmaf(sc[v], kfac, st.nmk));
                sc[v] = pv_;   // probabilities overwrite the scores
            }
        } else {
            pf[0] = __builtin_bit_cast(u32x4, __builtin_convertvector(__builtin_shufflevector(sc, sc, 0, 1, 2, 3, 4, 5, 6, 7), vec8));
            pf[1] = __builtin_bit_cast(u32x4, __builtin_convertvector(__builtin_shufflevector(sc, sc, 8, 9, 10, 11, 12, 13, 14, 15), vec8));
            l_run[rb] = sum_packed(pf, st.lsum);
        }
    };

    // Speculative softmax of half-tile u in row block rb went wrong for some row of the wave (see
    // SoftmaxState): for each flagged row (either of its lanes flagged) that has or gets a key,
    // take the row maximum of the half-tile's scores (still in sc), move the running maximum to
    // it if it is larger, and recompute the row's weights as 2^((x - m) k) with the difference
    // formed before scaling (safe for scores near the float range's end, as in the exact form);
    // O and the denominator are scaled by 2^((m_old - m) k), or by 0 for a row that had no key.
    auto fix_up = [&](auto full_c, auto rb_c, f32x16& sc, u32x4 (&pf)[2], SoftmaxState& st) __attribute__((always_inline)) {
        constexpr int rb = decltype(rb_c)::value;
        if constexpr (POLY) {
            // the speculative pass left raw dot products: form the capped scores exactly (and
            // -inf for masked elements of a partial half-tile)
#pragma unroll
            for (int v = 0; v < 16; ++v) {
                const float z = sc[v] * cap_z;
                float x = __builtin_fabsf(z) < kTanhSeriesMaxZ ? tanh_series_z(z) : tanh_identity_z(z);
                if constexpr (!decltype(full_c)::value) {
                    if (!((st.keep >> v) & 1u)) x = neg_inf();
                }
                sc[v] = x;
            }
        }
        float am = neg_inf();
#pragma unroll
        for (int v = 0; v < 16; ++v) am = __builtin_fmaxf(am, sc[v]);
        const float ax = half_swap_max(am);
        const uint32_t flag = st.redo ? 1u : 0u;
        const auto fl = __builtin_amdgcn_permlane32_swap(flag, flag, false, false);
        const bool empty = m_run[rb] == neg_inf();
        // (rows that stay without a key, such as fully masked ones, change nothing)
        const bool doit = (fl[0] | fl[1]) != 0u && (ax != neg_inf() || !empty);
        if (!wave_any(doit)) return;
        const float m_new = doit ? (empty ? ax : __builtin_fmaxf(m_run[rb], ax)) : 0.0f;
        const float alpha = doit ? (empty ? 0.0f : exp2_hw((m_run[rb] - m_new) * kfac)) : 1.0f;
        if (doit) {
            m_run[rb] = m_new;
            m_safe_run[rb] = m_new;
            nmk_run[rb] = -m_new * kfac;
        }
        u32x4 np[2];
#pragma unroll
        for (int v = 0; v < 16; v += 2)
            set_pair(np, v, exp2_hw((sc[v] - m_new) * kfac), exp2_hw((sc[v + 1] - m_new) * kfac));
        const float lsum = sum_packed(np, 0.0f);
        if (doit) {
            pf[0] = np[0];
            pf[1] = np[1];
            l_run[rb] = st.l_prev * alpha + lsum;
        }
        // (rows without a running maximum have O = 0: only moved ones need the scaling)
        if (wave_any(doit && !empty)) {
#pragma unroll
            for (int i = 0; i < NDB; ++i) o[rb][i] *= alpha;
        }
    };

    // Read r of the V^T operand reads of a block whose V half-tile starts OFFH bytes into the
    // V tile in ring slot `slot`: half r % 2 of V^T fragment r / 2 (fragment f covers dims
    // 32 (f % NDB) .. +31 and keys 16 (f / NDB) .. +15 of the half-tile).
    auto read_vt = [&](auto offh_c, auto r_c, uint32_t slot) __attribute__((always_inline)) -> u32x2 {
        constexpr int r = decltype(r_c)::value;
        constexpr int f = r / 2, hv = r % 2, j = f / NDB, db = f % NDB;
        return __builtin_bit_cast(u32x2, __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (lds_s16x4*)(lds + slot + v_base + (decltype(offh_c)::value + db * 2048 + (8 * j + 4 * hv) * 64))));
    };

    // ---- Pipelined block u: O^T += V^T P^T for half-tile u-1, the softmax of half-tile u
    // (scores s_cur, probabilities into p_cur) and S^T = K Q^T for half-tile u+1 (into s_nxt),
    // for each of the wave's RB row blocks; every K/V operand fragment read from LDS feeds the RB
    // row blocks' MFMAs back to back.  v_slot / k_slot: ring slots (byte offsets) of the tiles
    // holding half-tile u-1's V and half-tile u+1's K; par_c = (u-1) % 2 = (u+1) % 2.  The rescale
    // of O by the softmax's alpha follows the P.V products of half-tile u-1 and precedes those of
    // half-tile u in the next block.
    //
    // Both products always run, so that every block has one MFMA sequence: P of a half-tile a row
    // block does not attend is 0 (the masked softmax masks every element), which adds exactly 0
    // because every V row in the ring is finite (rows past the cache length arrive as zeros), and
    // scores of such a half-tile are masked away.  FULL: the softmax needs no structural mask.
    // MODE (bits kBlkPV, kBlkQK, kBlkSM) drops the parts of a block that have nothing to work
    // on: the first block of an item has no V tile for half-tile u-1 and only masked scores for
    // half-tile -1; in an item's last step the Q.K products (and the second block's softmax)
    // would score half-tiles past the item.  kBlkEnd: no block follows in this item.
    auto xbody = [&](auto full_c, auto mode_c, auto par_c, uint32_t v_slot, uint32_t k_slot, int u,
                     f32x16 (&s_cur)[RB], f32x16 (&s_nxt)[RB], u32x4 (&p_prev)[RB][2], u32x4 (&p_cur)[RB][2],
                     const MaskH (&mh)[RB], const MaskH (&mq)[RB], u32x2 (&rpre)[NPRE], auto&& unit_hook)
                     __attribute__((always_inline)) {
        constexpr int MODE = decltype(mode_c)::value;
        constexpr bool WITH_PV = (MODE & kBlkPV) != 0;
        constexpr bool WITH_QK = (MODE & kBlkQK) != 0;
        constexpr bool WITH_SM = (MODE & kBlkSM) != 0;
        // the exact softmax for an item's first half-tile (no P.V part) and where asked for
        constexpr bool EXACT_SM = (MODE & kBlkExact) != 0 || !WITH_PV;
        constexpr int PAR = decltype(par_c)::value;
        constexpr int NPV = WITH_PV ? 2 * NDB : 0;   // V^T fragments (one per P.V MFMA per row block)
        constexpr int NQK = WITH_QK ? NKS : 0;       // K fragments
        constexpr int NF = NPV + NQK;                // operand fragments of the block
        constexpr int NM = RB * NF;                  // MFMAs of the block
        // LDS operand reads, in the order the MFMAs consume them: read r < 2*NPV is half r % 2
        // of V^T fragment r / 2 (4 keys x 4 dims per transpose read), read 2*NPV + ks is K
        // fragment ks.  Reads run AHEAD operands in front of the first MFMA that needs them
        // (the compiler's waits then let each MFMA wait for its own reads only).  The first
        // NPRE reads of a block with P.V products come from the block before it (rpre): they
        // read V, which is resident one block earlier, so a block starts without an LDS round
        // trip.  Reads NR .. NR + NPRE - 1 of this block are those of the next block: V of the
        // same tile's other half (PAR 0), or the first half of the next step's V tile, which
        // sits in this step's K slot (PAR 1).  A first block without P.V (PAR 0) is followed by
        // another one and issues none.
        constexpr int NR = 2 * NPV + NQK;
        constexpr int OFFH = PAR * HB * ROWB;
        constexpr int PRE_IN = WITH_PV ? NPRE : 0;
        constexpr int PRE_OUT = ((WITH_PV || PAR == 1) && (MODE & kBlkEnd) == 0) ? NPRE : 0;
        constexpr int NT = NR + PRE_OUT;
        u32x2 rv[NPV > 0 ? 2 * NPV : 1];
        u32x4 rk[NQK > 0 ? NQK : 1];
        auto issue = [&](auto r_c) __attribute__((always_inline)) {
            constexpr int r = decltype(r_c)::value;
            if constexpr (r < PRE_IN) {
                // issued by the block before
            } else if constexpr (r < 2 * NPV) {
                rv[r] = read_vt(int_c<OFFH>{}, r_c, v_slot);
            } else if constexpr (r < NR) {
                constexpr int ks = r - 2 * NPV;
                rk[ks] = *(const u32x4*)(lds + k_slot + k_base + (OFFH + ks * 1024));
            } else {
                constexpr int rn = r - NR;
                if constexpr (PAR == 0) rpre[rn] = read_vt(int_c<HB * ROWB>{}, int_c<rn>{}, v_slot);
                else rpre[rn] = read_vt(int_c<0>{}, int_c<rn>{}, k_slot);
            }
        };
        static_for<0, (NR < AHEAD ? NR : AHEAD)>(issue);
        SoftmaxState st[RB];
        u32x4 frag = u32x4{0u, 0u, 0u, 0u};
        static_for<0, NM>([&](auto m_c) __attribute__((always_inline)) {
            constexpr int m = decltype(m_c)::value;
            constexpr int f = m / RB, rb = m % RB;
            if constexpr (rb == 0) {
                // reads issued by the end of unit g: AHEAD past the last one fragment g needs,
                // and a next-block read reuses an rpre entry only once units 0 .. g consumed it
                constexpr auto upto_of = [](int g) constexpr -> int {
                    const int last = g < NPV ? 2 * g + 1 : NPV + g;   // last read fragment g needs
                    int x = last + 1 + AHEAD < NT ? last + 1 + AHEAD : NT;
                    if (PRE_IN > 0) {
                        const int used = g < NPV ? (2 * g + 2 < PRE_IN ? 2 * g + 2 : PRE_IN) : PRE_IN;
                        x = x < NR + used ? x : NR + used;
                    }
                    return x;
                };
                constexpr int top = NR < AHEAD ? NR : AHEAD;
                constexpr int from = f == 0 ? top : upto_of(f - 1);
                constexpr int upto = upto_of(f) > from ? upto_of(f) : from;
                // the fragment is taken before this unit's reads are issued: with head dim 64 they
                // already include the next block's leading reads, which reuse the rpre entries
                // this unit consumes
                if constexpr (f < NPV) {
                    auto vt = [&](auto i_c) __attribute__((always_inline)) -> u32x2 {
                        constexpr int i = decltype(i_c)::value;
                        if constexpr (i < PRE_IN) return rpre[i];
                        else return rv[i];
                    };
                    const u32x2 lo = vt(int_c<2 * f>{}), hi = vt(int_c<2 * f + 1>{});
                    frag = u32x4{lo[0], lo[1], hi[0], hi[1]};
                } else {
                    frag = rk[f - NPV];
                }
                static_for<(from < upto ? from : upto), upto>(issue);
            }
            if constexpr (f < NPV) {
                constexpr int j = f / NDB, db = f % NDB;
                o[rb][db] = Tr::mfma(__builtin_bit_cast(vec8, frag), __builtin_bit_cast(vec8, p_prev[rb][j]), o[rb][db]);
            } else {
                constexpr int ks = f - NPV;
                f32x16 c0 = f32x16(0.0f);
                if constexpr (MASK_ACC) {
                    // the mask of half-tile u+1, element v at accumulator element v
#pragma unroll
                    for (int v = 0; v < 16; ++v) c0[v] = mask_val(mq[rb], v);
                }
                s_nxt[rb] = Tr::mfma(__builtin_bit_cast(vec8, frag), qf[rb][ks], ks == 0 ? c0 : s_nxt[rb]);
            }
            // softmax phases of the RB row blocks, interleaved (slot q: phase q / RB of row block q % RB)
            if constexpr (WITH_SM) {
                static_for<m * 8 * RB / NM, (m + 1) * 8 * RB / NM>([&](auto q_c) __attribute__((always_inline)) {
                    constexpr int q = decltype(q_c)::value;
                    constexpr int srb = q % RB;
                    softmax_phase(full_c, int_c<srb>{}, q / RB, u, s_cur[srb], mh[srb], p_cur[srb], st[srb],
                                  bool_c<EXACT_SM>{});
                });
            }
            unit_hook(m_c);
            // units (reads, wait, MFMA, softmax phases) stay in this order: a later unit's wait
            // must not run ahead of this unit's MFMA
            __builtin_amdgcn_sched_barrier(0);
        });
        if constexpr (WITH_SM) {
#pragma unroll
            for (int rb = 0; rb < RB; ++rb) {
                // Keep the probabilities and the row sum inside this block: otherwise they are
                // sunk past the rescale branch below, next to the next block's P.V products that
                // consume them, and no longer overlap this block's MFMAs.
                asm volatile("" : "+v"(p_cur[rb][0]), "+v"(p_cur[rb][1]), "+v"(l_run[rb]));
            }
            if constexpr (EXACT_SM) {
#pragma unroll
                for (int rb = 0; rb < RB; ++rb) {
                    if (wave_any(st[rb].moved)) {
#pragma unroll
                        for (int i = 0; i < NDB; ++i) o[rb][i] *= st[rb].alpha;
                    }
                }
            } else {
                static_for<0, RB>([&](auto rb_c) __attribute__((always_inline)) {
                    constexpr int rb = decltype(rb_c)::value;
                    if (wave_any(st[rb].redo)) fix_up(full_c, rb_c, s_cur[rb], p_cur[rb], st[rb]);
                });
            }
        }
    };

    // ---- Ring schedule.  Slot t % 4 holds tile t.  Step t runs blocks 2t+1 and 2t+2: they read
    // V of tile t and K of tile t+1, both landed before the step's barrier, and the step first
    // starts the loads of tile t+3 into the slot tile t-1 used (free since the last barrier).
    // Mask values: with head dim 64 those of the next step's two half-tiles are requested
    // before that DMA, so the step's closing wait (everything but tile t+3) covers them; with
    // head dim 128 (fewer free registers) the step requests its own before the DMA and waits
    // for them (and tile t+2) right after it.
    //
    // Kinds of step: 0 skip (no half-tile of the step's blocks is attended by the wave: no
    // compute, P = 0), 1 masked, 2 full (both blocks need no structural mask), 3 masked with the
    // exact softmax: the leading masked steps of a wave, where rows that have attended nothing
    // yet take their first keys (with the speculative softmax every such row would need the
    // fix-up; the exact form sets their maximum directly).  Steps go in
    // pairs (2p, 2p+1) so that the mask buffers alternate statically; along p a wave's pairs
    // run skip, masked, full, masked, skip, each kind in a loop of its own (no branch on the
    // kind inside a loop, so the compiler keeps one register assignment per loop).
    f32x16 s_even[RB], s_odd[RB];
    u32x4 p_even[RB][2], p_odd[RB][2];
    u32x2 rpre[NPRE];   // leading V operand reads of the next block, issued by the block before
#pragma unroll
    for (int i = 0; i < NPRE; ++i) rpre[i] = u32x2{0u, 0u};
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
        s_even[rb] = s_odd[rb] = f32x16(0.0f);
        p_even[rb][0] = p_even[rb][1] = p_odd[rb][0] = p_odd[rb][1] = u32x4{0u, 0u, 0u, 0u};
    }
    MaskH mask_a[2][RB], mask_b[2][RB];   // [half parity][row block]: odd half-tile first
    // PHASE 0: step -1 (Q.K of half-tiles 0 and 1, softmax of half-tile 0); 1: any other step.
    auto step = [&](auto kind_c, auto phase_c, int t, MaskH (&mcur)[2][RB], MaskH (&mnext)[2][RB]) __attribute__((always_inline)) {
        constexpr int KIND = decltype(kind_c)::value;
        constexpr int PHASE = decltype(phase_c)::value;
        constexpr int EX = KIND == 3 ? kBlkExact : 0;
        constexpr int MODE_A = PHASE == 0 ? kBlkQK : kBlkPV | kBlkQK | kBlkSM | EX;
        constexpr int MODE_B = PHASE == 0 ? kBlkQK | kBlkSM : kBlkPV | kBlkQK | kBlkSM | EX;
        // unmasked step -1: tiles 0 .. 2 are issued and tiles 0 and 1 landed and visible before
        // it, so it issues no loads and runs into step 0 without a wait or a barrier
        constexpr bool EARLY = PHASE == 0 && !MASKED;
        if constexpr (MASK_LDS) {
            // the buffer holds this step's successor's mask (DMA of two steps back): read it out,
            // then refill the buffer with the mask of the step after that
            // (its refill is spread over the first block below, or issued here in a skip step)
            // (steps after the first read it out at the end of the step before, ahead of that
            // step's barrier, so that the read's latency overlaps the barrier's wait; the wait
            // here keeps the refill from overwriting the buffer before the reads are done)
            if constexpr (PHASE == 0) mask_from_lds(mnext);
            asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
            if constexpr (KIND == 0) mask_dma(t + 2);
        } else if constexpr (MASK_AHEAD) {
            load_mask_half(2 * t + 3, mnext[0]);
            load_mask_half(2 * t + 4, mnext[1]);
        } else if constexpr (MASKED) {
            if constexpr (KIND != 0) {
                load_mask_half(2 * t + 1, mcur[0]);
                load_mask_half(2 * t + 2, mcur[1]);
            }
        }
        if (pre_next && t == t_last) load_q(nxt, qf);
        const DmaPlan dp = plan_tile(t + 3);
        if constexpr (KIND == 0) {
            dma_issue_all(dp);
#pragma unroll
            for (int rb = 0; rb < RB; ++rb)
                p_odd[rb][0] = p_odd[rb][1] = p_even[rb][0] = p_even[rb][1] = u32x4{0u, 0u, 0u, 0u};
            // the next step's first block expects its leading V reads in flight
            const uint32_t vn_slot = (uint32_t)((ring_base + t + 1) & (STAGES - 1)) * TILE_BYTES;
            static_for<0, NPRE>([&](auto r_c) __attribute__((always_inline)) {
                rpre[decltype(r_c)::value] = read_vt(int_c<0>{}, r_c, vn_slot);
            });
        } else {
            if constexpr (MASKED && !MASK_AHEAD) {
                dma_wait<0>();   // this step's mask values (and tile t+2) landed
                launder_mask(mcur[0]);
                launder_mask(mcur[1]);
            }
            const uint32_t v_slot = (uint32_t)((ring_base + t) & (STAGES - 1)) * TILE_BYTES;
            const uint32_t k_slot = (uint32_t)((ring_base + t + 1) & (STAGES - 1)) * TILE_BYTES;
            using F = bool_c<KIND == 2>;
            // tile t+3's loads, spread evenly over the MFMAs of one block (MODE): the first block,
            // or with MASK_LDS the second, the first then carrying the mask refill (the ring
            // loads stay the step's most recent loads, which its closing wait leaves in flight)
            auto spread_in = [&](auto mode_c, auto m_c) __attribute__((always_inline)) {
                if constexpr (EARLY) return;
                constexpr int MODE = decltype(mode_c)::value;
                constexpr int m = decltype(m_c)::value;
                constexpr int NMB = RB * (((MODE & kBlkPV) ? 2 * NDB : 0) + ((MODE & kBlkQK) ? NKS : 0));
                static_assert(NMB >= NDMA, "one load per MFMA at most");
                static_for<0, NDMA>([&](auto i_c) __attribute__((always_inline)) {
                    constexpr int i = decltype(i_c)::value;
                    if constexpr ((2 * i + 1) * NMB / (2 * NDMA) == m) dma_issue(dp, i_c);   // load i after MFMA m
                });
            };
            auto hook_a = [&](auto m_c) __attribute__((always_inline)) {
                if constexpr (MASK_LDS) {
                    constexpr int m = decltype(m_c)::value;
                    constexpr int NMB = RB * (((MODE_A & kBlkPV) ? 2 * NDB : 0) + ((MODE_A & kBlkQK) ? NKS : 0));
                    static_for<0, 8>([&](auto j_c) __attribute__((always_inline)) {
                        constexpr int j = decltype(j_c)::value;
                        if constexpr (j * NMB / 8 == m) mask_dma_op(t + 2, j_c);   // mask op j after MFMA m
                    });
                } else {
                    spread_in(int_c<MODE_A>{}, m_c);
                }
            };
            auto hook_b = [&](auto m_c) __attribute__((always_inline)) {
                if constexpr (MASK_LDS) spread_in(int_c<MODE_B>{}, m_c);
            };
            // The two waves of a SIMD run the same work; at equal priority the older one (waves
            // below WAVES / 2) wins the issue slots, runs ahead, and the younger one finishes
            // every step alone.  Raising the younger wave's priority for the first block lets
            // the pair finish a step together more closely.
            if (wave >= WAVES / 2) __builtin_amdgcn_s_setprio(1);
            // (block 2t+1 scores half-tile 2t+2, whose mask is mcur[1]; block 2t+2 scores half-tile
            // 2t+3, whose mask mnext[0] was read out at the start of this step)
            xbody(F{}, int_c<MODE_A>{}, int_c<0>{}, v_slot, k_slot, 2 * t + 1, s_odd, s_even, p_even, p_odd, mcur[0],
                  mcur[1], rpre, hook_a);
            if (wave >= WAVES / 2) __builtin_amdgcn_s_setprio(0);
            xbody(F{}, int_c<MODE_B>{}, int_c<1>{}, v_slot, k_slot, 2 * t + 2, s_even, s_odd, p_odd, p_even, mcur[1],
                  mnext[0], rpre, hook_b);
        }
        if constexpr (!EARLY) {
            ring_wait();   // everything but tile t+3 landed
            if constexpr (MASK_AHEAD) {
                launder_mask(mnext[0]);
                launder_mask(mnext[1]);
            }
            // MASK_LDS: the buffer now holds the mask of step t+2 (this step's refill landed),
            // which the next step holds as its mnext, this step's mcur (no longer read)
            if constexpr (MASK_LDS) mask_from_lds(mcur);
            __syncthreads();
        }
    };
    auto run_pairs = [&](auto kind_c, int p0, int p1) __attribute__((always_inline)) {
        for (int pp = p0; pp < p1; ++pp) {
            step(kind_c, int_c<1>{}, 2 * pp, mask_a, mask_b);
            step(kind_c, int_c<1>{}, 2 * pp + 1, mask_b, mask_a);
        }
    };

    auto run_steps = [&](auto kind_c, int t0, int t1) __attribute__((always_inline)) {
        for (int t = t0; t < t1; ++t) step(kind_c, int_c<1>{}, t, mask_a, mask_b);
    };

    if (n_tiles > 0) {
        // pair p holds blocks 4p+1 .. 4p+4, which touch half-tiles 4p .. 4p+5
        const int n_pairs = n_steps / 2;
        int a0, a1, f0, f1;
        if constexpr (!MASKED) {
            // step t runs blocks 2t+1 and 2t+2, which touch half-tiles 2t .. 2t+3; without mask
            // buffers the kinds change from step to step
            auto fdiv2 = [](int x) -> int { return x >> 1; };
            auto cdiv2 = [](int x) -> int { return -((-x) >> 1); };
            auto clip = [&](int x, int lo, int hi) -> int { return x < lo ? lo : (x > hi ? hi : x); };
            // not skip: 2t+3 >= ua and 2t <= ub; full: 2t+1 >= fa and 2t+2 <= fb
            a0 = clip(cdiv2(ua - 3), 0, n_steps);
            a1 = clip(fdiv2(ub) + 1, a0, n_steps);
            f0 = clip(cdiv2(fa - 1), a0, a1);
            f1 = clip(fdiv2(fb - 2) + 1, f0, a1);
            a0 = __builtin_amdgcn_readfirstlane(a0);
            a1 = __builtin_amdgcn_readfirstlane(a1);
            f0 = __builtin_amdgcn_readfirstlane(f0);
            f1 = __builtin_amdgcn_readfirstlane(f1);
        } else {
            auto fdiv4 = [](int x) -> int { return x >> 2; };
            auto cdiv4 = [](int x) -> int { return -((-x) >> 2); };
            auto clip = [&](int x, int lo, int hi) -> int { return x < lo ? lo : (x > hi ? hi : x); };
            // not skip: 4p+5 >= ua and 4p <= ub
            a0 = clip(cdiv4(ua - 5), 0, n_pairs);
            a1 = clip(fdiv4(ub) + 1, a0, n_pairs);
            // full: 4p+1 >= fa and 4p+4 <= fb
            f0 = clip(cdiv4(fa - 1), a0, a1);
            f1 = clip(fdiv4(fb - 4) + 1, f0, a1);
            a0 = __builtin_amdgcn_readfirstlane(a0);
            a1 = __builtin_amdgcn_readfirstlane(a1);
            f0 = __builtin_amdgcn_readfirstlane(f0);
            f1 = __builtin_amdgcn_readfirstlane(f1);
        }
        if constexpr (MASK_AHEAD) load_mask_half(0, mask_b[1]);
        mask_dma(0);   // (MASK_LDS) step 0's mask, read out by step -1
        if (!pre) {
            dma_issue_all(plan_tile(0));
            dma_issue_all(plan_tile(1));
            if constexpr (!MASKED) dma_issue_all(plan_tile(2));
            ring_wait();   // Q, tile 0 (unmasked: and tile 1) and the mask loads before them landed
        }
        // (prefetched: the previous item's closing wait and barrier retired Q and tiles 0 and 1)
        launder_q();
        if constexpr (MASK_AHEAD) launder_mask(mask_b[1]);
        if (!pre) __syncthreads();
        // step -1: S of half-tiles 0 and 1, softmax of half-tile 0
        step(int_c<1>{}, int_c<0>{}, -1, mask_b, mask_a);
        if constexpr (!MASKED) {
            run_steps(int_c<0>{}, 0, a0);
            run_steps(int_c<3>{}, a0, f0);
            run_steps(int_c<2>{}, f0, f1);
            run_steps(int_c<1>{}, f1, a1);
            run_steps(int_c<0>{}, a1, n_steps);
        } else {
            run_pairs(int_c<0>{}, 0, a0);
            run_pairs(int_c<3>{}, a0, f0);
            run_pairs(int_c<2>{}, f0, f1);
            run_pairs(int_c<1>{}, f1, a1);
            run_pairs(int_c<0>{}, a1, n_pairs);
        }
    }
    if (!pre_next) dma_wait<0>();   // nothing of this item's ring stays in flight

    // Output: O / l, rounded to 16 bits, in whole 128-byte row pieces (64 dims) through the
    // wave's staging buffer, 16 rows at a time.  Lane (m, hh) holds dims 32 db + 8a + 4hh .. +3
    // (a = 0..3) of its row m.  For rows 16 H .. 16 H + 15 and dims 64 P .. 64 P + 63, the lanes of
    // those rows write chunk c = 4 (db - 2P) + a (8 bytes) to position 16 hh + m % 16 of staging
    // chunk c; lane 8 r' + q of store s then reads back the two halves of dims 64 P + 8q .. +7 of
    // row 16 H + 8 s + r'.  Each store instruction writes 8 whole 128-byte row pieces (written
    // directly from the accumulator layout, every instruction would cover 16 bytes of each of 32
    // rows, which holds up the memory pipeline and, with non-temporal stores, splits lines).  The
    // stores are non-temporal: nothing reads the output again here.  A wave without a valid row
    // stores nothing; rows past sq are skipped lane by lane.
    if (wave_has_rows) {
        constexpr int NP = DP / 64;   // 64-dim pieces per row
        char* const stg = lds + STG_OFF + wave * (8 * STG_CHUNK);
        const int rr = lane >> 3, q = lane & 7;
#pragma unroll
        for (int rb = 0; rb < RB; ++rb) {
            const float l = half_swap_sum(l_run[rb]);
            const float inv = l > 0.0f ? 1.0f / l : 0.0f;
#pragma unroll
            for (int P = 0; P < NP; ++P) {
#pragma unroll
                for (int H = 0; H < 2; ++H) {
                    if ((lr >> 4) == H) {
#pragma unroll
                        for (int dd = 0; dd < 2; ++dd) {
#pragma unroll
                            for (int a = 0; a < 4; ++a) {
                                f32x4 val;
#pragma unroll
                                for (int c = 0; c < 4; ++c) val[c] = o[rb][2 * P + dd][4 * a + c] * inv;
                                *(u32x2*)(stg + (4 * dd + a) * STG_CHUNK + (16 * hh + (lr & 15)) * 8) =
                                    __builtin_bit_cast(u32x2, __builtin_convertvector(val, vec4));
                            }
                        }
                    }
#pragma unroll
                    for (int sh = 0; sh < 2; ++sh) {
                        const int r = 8 * sh + rr;
                        const u32x2 lo = *(const u32x2*)(stg + q * STG_CHUNK + r * 8);
                        const u32x2 hi = *(const u32x2*)(stg + q * STG_CHUNK + 128 + r * 8);
                        const int64_t orow_i = wr0 + 32 * rb + 16 * H + r;
                        scalar* const dst = (scalar*)p.out + (int64_t)b * p.o_stride_b + (int64_t)h * p.o_stride_h +
                                            orow_i * p.o_stride_i + 64 * P + 8 * q;
                        if (orow_i < p.sq) __builtin_nontemporal_store(u32x4{lo[0], lo[1], hi[0], hi[1]}, (u32x4*)dst);
                    }
                }
            }
        }
    }
    ring_base = pre_next ? ring_base + t_last + 1 : 0;
    pre = pre_next;
    cur = nxt;
    }   // items
    dma_wait<0>();   // no ring load stays in flight past the workgroup's end
}


template <typename Tr, int DP, int MASKK, int SOFTCAP, bool RAW>
hipError_t launch_ring_one(const FwdParams& p, int grid, hipStream_t stream) {
    constexpr int RB = kRingRowBlocks;
    hipLaunchKernelGGL((fwd16_ring_kernel<Tr, DP, MASKK, SOFTCAP, RAW, RB>), dim3(grid), dim3(ring_threads(RB)), 0,
                       stream, p);
    return hipGetLastError();
}

template <typename Tr, int DP>
hipError_t launch_ring_dp(const FwdParams& p, int grid, int maskk, bool softcap, hipStream_t s) {
    if (softcap) {
        const bool identity = p.softcap <= kTanhIdentityMaxCap;
        if (maskk == kMaskF32)
            return identity ? launch_ring_one<Tr, DP, kMaskF32, 2, false>(p, grid, s)
                            : launch_ring_one<Tr, DP, kMaskF32, 1, false>(p, grid, s);
        if (maskk == kMaskT)
            return identity ? launch_ring_one<Tr, DP, kMaskT, 2, false>(p, grid, s)
                            : launch_ring_one<Tr, DP, kMaskT, 1, false>(p, grid, s);
        return identity ? launch_ring_one<Tr, DP, kMaskNone, 2, false>(p, grid, s)
                        : launch_ring_one<Tr, DP, kMaskNone, 1, false>(p, grid, s);
    }
    // (mask accumulation: bf16 only, whose exponent range lets Q take the scale exactly, with
    // the LDS-staged fp32 mask)
    if constexpr (DP == 64 && std::is_same<Tr, TraitsBF16>::value) {
        if (p.mask_in_acc && maskk == kMaskF32) return launch_ring_one<Tr, DP, kMaskF32, 0, true>(p, grid, s);
    }
    if (maskk == kMaskF32) return launch_ring_one<Tr, DP, kMaskF32, 0, false>(p, grid, s);
    if (maskk == kMaskT) return launch_ring_one<Tr, DP, kMaskT, 0, false>(p, grid, s);
    if (p.raw_scores) return launch_ring_one<Tr, DP, kMaskNone, 0, true>(p, grid, s);
    return launch_ring_one<Tr, DP, kMaskNone, 0, false>(p, grid, s);
}

template <typename Tr>
hipError_t launch_ring(const FwdParams& p, int dp, int grid, int maskk, bool softcap, hipStream_t s) {
    return dp == 64 ? launch_ring_dp<Tr, 64>(p, grid, maskk, softcap, s)
                    : launch_ring_dp<Tr, 128>(p, grid, maskk, softcap, s);
}

}  // namespace fa
