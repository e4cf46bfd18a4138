// Per-dtype launch entry points, one translation unit each.
#pragma once

#include <hip/hip_runtime.h>

#include "fa_params.h"

namespace fa {
// maskk: 0 none, 1 fp32 mask, 2 mask of the input type.  dp: head dim padded to 32/64/96/128.
hipError_t launch_bf16(const FwdParams& p, int dp, int grid, int maskk, bool softcap, hipStream_t s);
hipError_t launch_f16(const FwdParams& p, int dp, int grid, int maskk, bool softcap, hipStream_t s);
// split: 32-row workgroups, each key range in two halves (grid and p.q_tiles in 32-row tiles)
hipError_t launch_f32(const FwdParams& p, int dp, int grid, bool masked, bool softcap, bool split, hipStream_t s);
// fp32, head dims 129..384
hipError_t launch_f32_wide(const FwdParams& p, int grid, bool masked, bool softcap, hipStream_t s);
// split-key kernels (few query rows per KV head), head dims 64 and 128; maskk as above
hipError_t launch_bf16_splitkv(const FwdParams& p, const SplitParams& sp, int dp, int maskk, hipStream_t s);
hipError_t launch_f16_splitkv(const FwdParams& p, const SplitParams& sp, int dp, int maskk, hipStream_t s);
// 256-row, 512-thread kernels for head dims 64 and 128 with 16-byte aligned rows.
hipError_t launch_bf16_ring(const FwdParams& p, int dp, int grid, int maskk, bool softcap, hipStream_t s);
hipError_t launch_f16_ring(const FwdParams& p, int dp, int grid, int maskk, bool softcap, hipStream_t s);
}  // namespace fa
