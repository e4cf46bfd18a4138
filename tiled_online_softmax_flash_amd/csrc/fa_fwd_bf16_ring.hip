// bf16 instantiations of the 256-row LDS-ring attention kernel.
#include "fa_fwd16_ring.h"
#include "fa_launch.h"

namespace fa {
hipError_t launch_bf16_ring(const FwdParams& p, int dp, int grid, int maskk, bool softcap, hipStream_t s) {
    return launch_ring<TraitsBF16>(p, dp, grid, maskk, softcap, s);
}
}  // namespace fa
