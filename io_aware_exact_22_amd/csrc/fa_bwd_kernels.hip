// fa_bwd_kernels.hip -- the launch of the backward pass (fa_bwd_device.h) at
// head dimensions 64 and 128; the other multiples of 16 up to 128 go to
// fa_bwd_padded.hip.
#include <hip/hip_runtime.h>

#include "fa_bwd_device.h"
#include "fa_launch.h"

namespace fa {

hipError_t launch_bwd(const BwdArgs& a) {
    if (a.D != 64 && a.D != 128) return launch_bwd_padded(a);
    if (a.dtype == kDtypeBf16)
        return a.D == 64 ? launch_bwd_t<__bf16, 64, false>(a) : launch_bwd_t<__bf16, 128, false>(a);
    return a.D == 64 ? launch_bwd_t<_Float16, 64, false>(a) : launch_bwd_t<_Float16, 128, false>(a);
}

}  // namespace fa
