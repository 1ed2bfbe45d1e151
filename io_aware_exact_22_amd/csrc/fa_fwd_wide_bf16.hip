// fa_fwd_wide_bf16.hip -- the bf16 forward at head dimensions above 128 (a
// multiple of 16 up to 256): the D = 256 kernel with 32-key K/V tiles (a
// 64-key tile of 512-byte rows would not fit the LDS stages' 16-bit offsets),
// with PAD = true below 256.  One translation unit per dtype so that the
// instantiations compile in parallel.
#include <hip/hip_runtime.h>

#include "fa_fwd_launch_cfg.h"
#include "fa_launch.h"

namespace fa {

hipError_t launch_fwd_wide_bf16(const LaunchArgs& a) {
    return a.D == 256 ? launch_mfma_cfg<__bf16, 256, kMfmaWaves, kWideKeys, false>(a)
                      : launch_mfma_cfg<__bf16, 256, kMfmaWaves, kWideKeys, true>(a);
}

}  // namespace fa
