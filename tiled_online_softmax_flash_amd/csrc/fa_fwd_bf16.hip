// bf16 instantiations of the 16-bit attention kernel.
#include "fa_fwd16.h"
#include "fa_launch.h"

namespace fa {
hipError_t launch_bf16(const FwdParams& p, int dp, int grid, int maskk, bool softcap, hipStream_t s) {
    return launch_fwd16<TraitsBF16>(p, dp, grid, maskk, softcap, s);
}
}  // namespace fa
