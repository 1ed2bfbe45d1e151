// fa_fwd_padded.hip -- the forward at head dimensions other than 64 and 128
// (bf16 / fp16: any multiple of 16 up to 256; fp32: up to 128): below 128, the kernel for the
// next of 64 and 128 with PAD = true, which reads the columns at or past the
// tensors' own head dimension as zeros and never writes them; above 128, the
// D = 256 kernels of fa_fwd_wide_bf16.hip / fa_fwd_wide_fp16.hip.  (The
// KV-cache forward at such a D: fa_fwd_kvcache_padded.hip.)  The pages ask Tensor
// Core shapes in multiples of 8 (section 4.2 of "FlashAttention技术解析：加速
// GPT训练的核心优化"); 16 is the k step of the gfx950 MFMA.  A translation
// unit of its own so that these instantiations compile beside the others.
#include <hip/hip_runtime.h>

#include "fa_fwd_launch_cfg.h"
#include "fa_launch.h"

namespace fa {

hipError_t launch_fwd_padded(const LaunchArgs& a) {
    if (a.dtype == kDtypeFp32) return a.D < 64 ? launch_fp32<64, true>(a) : launch_fp32<128, true>(a);
    if (a.D > 128) return a.dtype == kDtypeBf16 ? launch_fwd_wide_bf16(a) : launch_fwd_wide_fp16(a);
    if (a.dtype == kDtypeBf16)
        return a.D < 64 ? launch_mfma_cfg<__bf16, 64, kMfmaWaves, kMfmaKeys, true>(a)
                        : launch_mfma_cfg<__bf16, 128, kMfmaWaves, kMfmaKeys, true>(a);
    return a.D < 64 ? launch_mfma_cfg<_Float16, 64, kMfmaWaves, kMfmaKeys, true>(a)
                    : launch_mfma_cfg<_Float16, 128, kMfmaWaves, kMfmaKeys, true>(a);
}

}  // namespace fa
