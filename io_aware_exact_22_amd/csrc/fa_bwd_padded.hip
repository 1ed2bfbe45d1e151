// fa_bwd_padded.hip -- the backward pass at head dimensions other than 64 and
// 128 (a multiple of 16 up to 128): the kernels of the next of 64 and 128 with
// PAD = true, which read the columns past the tensors' head dimension as
// zeros and never write them (fa_bwd_device.h).  A translation unit of its
// own so that these instantiations compile beside the others.
#include <hip/hip_runtime.h>

#include "fa_bwd_device.h"
#include "fa_launch.h"

namespace fa {

hipError_t launch_bwd_padded(const BwdArgs& a) {
    if (a.dtype == kDtypeBf16)
        return a.D < 64 ? launch_bwd_t<__bf16, 64, true>(a) : launch_bwd_t<__bf16, 128, true>(a);
    return a.D < 64 ? launch_bwd_t<_Float16, 64, true>(a) : launch_bwd_t<_Float16, 128, true>(a);
}

}  // namespace fa
