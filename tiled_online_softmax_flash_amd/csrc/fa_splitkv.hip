// bf16 and f16 instantiations of the split-key (decode) attention kernels.
#include "fa_splitkv.h"
#include "fa_launch.h"

namespace fa {
hipError_t launch_bf16_splitkv(const FwdParams& p, const SplitParams& sp, int dp, int maskk, hipStream_t s) {
    return launch_splitkv<TraitsBF16>(p, sp, dp, maskk, s);
}
hipError_t launch_f16_splitkv(const FwdParams& p, const SplitParams& sp, int dp, int maskk, hipStream_t s) {
    return launch_splitkv<TraitsF16>(p, sp, dp, maskk, s);
}
}  // namespace fa
