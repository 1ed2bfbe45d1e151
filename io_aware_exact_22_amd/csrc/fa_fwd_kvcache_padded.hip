// fa_fwd_kvcache_padded.hip -- the KV-cache forward at head dimensions other
// than 64 and 128 (a multiple of 16 up to 128): the MFMA kernel (KVC = true)
// of the next of 64 and 128 with PAD = true, which reads the columns past the
// tensors' head dimension as zeros and never writes them, for any number of
// queries per sequence.  A translation unit of its own so that these
// instantiations compile beside the others.
#include <hip/hip_runtime.h>

#include "fa_fwd_launch_cfg.h"
#include "fa_launch.h"

namespace fa {

hipError_t launch_kvcache_padded(const LaunchArgs& a) {
    if (a.dtype == kDtypeBf16)
        return a.D < 64 ? launch_kvc_mfma_cfg<__bf16, 64, true>(a)
                        : launch_kvc_mfma_cfg<__bf16, 128, true>(a);
    return a.D < 64 ? launch_kvc_mfma_cfg<_Float16, 64, true>(a)
                    : launch_kvc_mfma_cfg<_Float16, 128, true>(a);
}

}  // namespace fa
