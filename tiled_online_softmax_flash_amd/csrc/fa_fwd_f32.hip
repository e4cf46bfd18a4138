// fp32 instantiations of the attention kernel.
#include "fa_fwd32.h"
#include "fa_fwd32w.h"
#include "fa_launch.h"

namespace fa {
hipError_t launch_f32(const FwdParams& p, int dp, int grid, bool masked, bool softcap, bool split, hipStream_t s) {
    return launch_fwd32(p, dp, grid, masked, softcap, split, s);
}
hipError_t launch_f32_wide(const FwdParams& p, int grid, bool masked, bool softcap, hipStream_t s) {
    return launch_fwd32w(p, grid, masked, softcap, s);
}
}  // namespace fa
