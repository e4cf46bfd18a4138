// Device helpers shared by the attention kernels: work decoding, the per-row key rule,
// tile classification and a few arithmetic primitives.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "fa_params.h"

namespace fa {

typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr float kLog2e = 1.4426950408889634f;

__device__ __forceinline__ float neg_inf() { return -__builtin_huge_valf(); }

// 2^x on the hardware exponential unit (v_exp_f32); -inf -> 0.
__device__ __forceinline__ float exp2_hw(float x) { return __builtin_amdgcn_exp2f(x); }

// tanh(y).  For |y| >= 1/8 it uses the identity tanh y = 1 - 2 / (e^{2y} + 1) on the hardware
// exponential and reciprocal (absolute error a few fp32 ulps of 1, relative error below 1e-6
// there); it saturates cleanly to +-1.  For |y| < 1/8 the identity would cancel, so the odd
// Taylor series y - y^3/3 + 2y^5/15 - 17y^7/315 is used instead (truncation below 2e-9
// relative).  Relative accuracy near 0 matters when a huge softcap multiplies the result.
__device__ __forceinline__ float tanh_fast(float y) {
    const float e = exp2_hw(y * (2.0f * kLog2e));
    const float big = 1.0f - 2.0f * __builtin_amdgcn_rcpf(e + 1.0f);
    const float y2 = y * y;
    const float poly = __builtin_fmaf(y2, __builtin_fmaf(y2, __builtin_fmaf(y2, -17.0f / 315.0f, 2.0f / 15.0f), -1.0f / 3.0f), 1.0f);
    const float small = y * poly;
    return __builtin_fabsf(y) < 0.125f ? small : big;
}

// The identity tanh y = 1 - 2 / (e^{2y} + 1) alone (tanh_identity_z below) has an absolute
// error of a few fp32 ulps of 1 everywhere (it saturates cleanly to +-1), but no relative
// accuracy near 0.  Scaled by a softcap c <= kTanhIdentityMaxCap the capped score is off by at
// most about c * 2^-21 < 5e-4, which leaves the softmax weights within 1e-3 relative; larger caps
// use tanh_fast.
constexpr float kTanhIdentityMaxCap = 1024.0f;

// tanh in terms of z = 2 log2(e) y (the argument of the identity's exponential).
//   tanh_identity_z: 1 - 2 / (2^z + 1), one exponential and one reciprocal (accuracy above).
//   tanh_series_z, for |y| < 1/8 (|z| < kTanhSeriesMaxZ): the odd series y - y^3/3 + 2 y^5/15
//   written in z, no transcendental instruction.  Its truncation error is below
//   (17/315) y^7 <= 2.1e-7 |y| there, under the identity's absolute error of a few ulps of 1.
constexpr float kTanhZ = 2.0f * kLog2e;
constexpr float kTanhSeriesMaxZ = kTanhZ / 8.0f;
__device__ __forceinline__ float tanh_identity_z(float z) {
    return 1.0f - 2.0f * __builtin_amdgcn_rcpf(exp2_hw(z) + 1.0f);
}
__device__ __forceinline__ float tanh_series_z(float z) {
    constexpr double k = 2.0 * 1.4426950408889634;
    constexpr float a1 = (float)(1.0 / k);
    constexpr float a3 = (float)(-1.0 / (3.0 * k * k * k));
    constexpr float a5 = (float)(2.0 / (15.0 * k * k * k * k * k));
    const float z2 = z * z;
    return z * __builtin_fmaf(z2, __builtin_fmaf(z2, a5, a3), a1);
}

// One workgroup's share of the problem: batch b, query head h, query tile qt.
struct WorkItem {
    int b, h, qt;
    bool valid;
};

// Workgroups are dealt to the 8 XCDs round-robin by block id; each XCD has its own L2.  Two
// orders are used:
//   * group-major (p.xcd_groups != 0, requires batch * kv_heads to be a multiple of 8): every
//     workgroup of one (batch, KV head) group -- all its query heads and query tiles -- runs on
//     one XCD, so the group's K/V rows are fetched into that L2 once and then shared.  Groups
//     are dealt to XCDs round-robin; inside a group, query tiles go in descending order (causal
//     tiles late in the sequence carry the most keys, so they start first).
//   * pair-major: all query heads of one (batch, query tile) pair run on one XCD, so heads that
//     share a mask plane read it through the same L2; pairs are dealt round-robin in descending
//     query-tile order.  The grid holds ceil(pairs / 8) * 8 * heads blocks; blocks of the
//     padding pairs exit at once.
__device__ __forceinline__ WorkItem decode_work(const FwdParams& p, int bid) {
    WorkItem w;
    const int xcd = bid & 7;
    const int slot = bid >> 3;
    if (p.xcd_groups) {
        const int per_group = p.group * p.q_tiles;
        const int gl = slot / per_group;
        const int r = slot - gl * per_group;
        const int grp = gl * 8 + xcd;                 // b * kv_heads + kvh
        const int qr = r / p.group;
        const int hg = r - qr * p.group;
        w.b = grp / p.kv_heads;
        w.h = (grp - w.b * p.kv_heads) * p.group + hg;
        w.qt = p.q_tiles - 1 - qr;
        w.valid = w.b < p.batch;
        return w;
    }
    const int pair_local = slot / p.heads;
    w.h = slot - pair_local * p.heads;
    const int pair = pair_local * 8 + xcd;
    w.valid = pair < p.pairs;
    w.qt = p.q_tiles - 1 - pair / p.batch;
    w.b = pair - (pair / p.batch) * p.batch;
    return w;
}

// The key rule of one batch entry (see fa.h): key j is attended by query row i iff
// lo(i) <= j <= hi(i).  Both bounds are non-decreasing in i.
struct KeyRule {
    int64_t L;      // min(total, sk), at least 0
    int64_t base;   // cmax(i) = base + i
    int64_t window;
    int causal;

    __device__ __forceinline__ int64_t lo(int64_t i) const {
        if (window <= 0) return 0;
        const int64_t v = base + i + 1 - window;
        return v > 0 ? v : 0;
    }
    __device__ __forceinline__ int64_t hi(int64_t i) const {
        const int64_t cm = base + i;
        return (causal && cm < L - 1) ? cm : L - 1;
    }
};

__device__ __forceinline__ KeyRule make_rule(const FwdParams& p, int b) {
    KeyRule r;
    int64_t L = p.sk;
    if (p.total_lengths != nullptr) {
        const int64_t t = p.total_lengths[b];
        if (t < L) L = t;
    }
    if (L < 0) L = 0;
    r.L = L;
    r.base = p.past_lengths != nullptr ? (int64_t)p.past_lengths[b] : L - p.sq;
    r.window = p.window;
    r.causal = p.causal;
    return r;
}

// Mask plane of (b, h): 0, b, or b*heads + h (tested in that order).
__device__ __forceinline__ int64_t mask_plane(const FwdParams& p, int b, int h) {
    if (p.mask_planes == p.batch) return b;
    if (p.mask_planes == p.batch * p.heads) return (int64_t)b * p.heads + h;
    return 0;
}

// Row of the key tile held in LDS row r (0..31) of a 32-key block.  A 32x32 MFMA accumulator
// gives lane (m, half) the values of rows 8*(v/4) + 4*half + v%4; storing key kk(r) in row r
// makes those rows hold keys 16*half + v, i.e. each lane owns 16 consecutive keys.
__device__ __forceinline__ int lds_row_of_key(int key_in_block) {
    const int half = key_in_block >> 4;
    const int v = key_in_block & 15;
    return 8 * (v >> 2) + 4 * half + (v & 3);
}

// Raw buffer descriptor (gfx9 family: stride 0, byte-addressed, dword 3 = 0x00020000) over
// `bytes` bytes at `base`.  Buffer loads at offsets past `bytes` return 0 without touching
// memory, which is how tiles ending past the last valid key are zero-filled.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, int bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, bytes, 0x00020000);
}

// max(x[lane % 32], x[32 + lane % 32]) in every lane: the row maximum of the two lanes that
// share a query row, via v_permlane32_swap (a VALU op, no LDS crossbar).
__device__ __forceinline__ float half_swap_max(float x) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __builtin_fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}

// x[lane % 32] + x[32 + lane % 32] in every lane.
__device__ __forceinline__ float half_swap_sum(float x) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// Scheduling-group masks of __builtin_amdgcn_sched_group_barrier.
constexpr int kSchedValu = 0x002;
constexpr int kSchedMfma = 0x008;
constexpr int kSchedDsRead = 0x100;
constexpr int kSchedDsWrite = 0x200;
constexpr int kSchedVmemRead = 0x020;

// Wait until at most N vector-memory operations of this wave are outstanding (gfx9 s_waitcnt
// encoding: vmcnt in bits [3:0] and [15:14]; expcnt and lgkmcnt left at their maxima).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
    static_assert(N >= 0 && N < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

// 16-byte buffer load straight into LDS: lane l's 16 bytes (from `voffset` within the buffer
// described by `rsrc`) land at LDS byte address `lds_addr + 16 * l`.  Issued through inline asm
// so that the compiler's wait-count pass leaves these loads to the kernel's own waits
// (dma_wait) instead of draining all vector-memory loads before every LDS read.
__device__ __forceinline__ void dma_lds16(u32x4 rsrc, uint32_t lds_addr, uint32_t voffset) {
    asm volatile("s_mov_b32 m0, %0\n\tbuffer_load_dwordx4 %1, %2, 0 offen lds"
                 :
                 : "s"(lds_addr), "v"(voffset), "s"(rsrc)
                 : "m0");
}

// 4-byte buffer load straight into LDS: lane l's dword (from byte voffset + soffset of the
// buffer described by `rsrc`) lands at LDS byte address `lds_addr + 4 * l`.  A lane whose
// voffset lies past the buffer's size writes 0.
__device__ __forceinline__ void dma_lds4(u32x4 rsrc, uint32_t lds_addr, uint32_t voffset, uint32_t soffset) {
    asm volatile("s_mov_b32 m0, %0\n\tbuffer_load_dword %1, %2, %3 offen lds"
                 :
                 : "s"(lds_addr), "v"(voffset), "s"(rsrc), "s"(soffset)
                 : "m0");
}

// Wait until at most N vector-memory operations of this wave are in flight (loads retire in
// order; stores count too).
template <int N>
__device__ __forceinline__ void dma_wait() {
    static_assert(N >= 0 && N <= 63, "vmcnt range");
    asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

// Raw buffer descriptor as four wave-uniform dwords (gfx9 family, stride 0, byte-addressed).
__device__ __forceinline__ u32x4 make_rsrc_words(const void* base, int bytes) {
    const uint64_t a = (uint64_t)base;
    return u32x4{(uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)a),
                 (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)((a >> 32) & 0xffffu)),
                 (uint32_t)__builtin_amdgcn_readfirstlane(bytes), 0x00020000u};
}

// LDS byte address of a pointer into __shared__ memory.
__device__ __forceinline__ uint32_t lds_addr(const void* p) {
    return (uint32_t)(uintptr_t)((const __attribute__((address_space(3))) char*)p);
}

// Wave-level any() of a per-lane predicate.
__device__ __forceinline__ bool wave_any(bool pred) { return __ballot(pred) != 0ull; }

}  // namespace fa
