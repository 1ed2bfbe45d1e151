// fa_fwd_kernels.hip -- launchers of the fused exact-attention forward
// (fa_fwd, the split-KV, block-sparse and paged variants) and the part-merge
// launch the KV-cache launcher shares.  The kernels are in fa_fwd_device.h.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "fa_fwd_device.h"
#include "fa_fwd_launch_cfg.h"
#include "fa_launch.h"
#include "fa_schedule.h"

namespace fa {

// ---------------------------------------------------------------- launchers
template <typename T, int D>
static hipError_t launch_merge_cfg(const LaunchArgs& a) {
    constexpr int RPB = kMergeThreads / (D / 4);
    const int64_t rows = a.B * a.H * a.S;
    hipLaunchKernelGGL((fa_merge_parts_kernel<T, D>), dim3((unsigned)((rows + RPB - 1) / RPB)),
                       dim3(kMergeThreads), 0, a.stream, (const float*)a.part_o,
                       (const float*)a.part_lse, (T*)a.out, a.lse, (int)a.B, (int)a.H, (int)a.S,
                       a.n_splits, (int)a.D);
    return hipGetLastError();
}

hipError_t launch_merge_parts(const LaunchArgs& a) {
    if (a.dtype == kDtypeBf16)
        return a.D <= 64    ? launch_merge_cfg<__bf16, 64>(a)
               : a.D <= 128 ? launch_merge_cfg<__bf16, 128>(a)
                            : launch_merge_cfg<__bf16, 256>(a);
    return a.D <= 64    ? launch_merge_cfg<_Float16, 64>(a)
           : a.D <= 128 ? launch_merge_cfg<_Float16, 128>(a)
                        : launch_merge_cfg<_Float16, 256>(a);
}

template <typename T, int D>
static hipError_t launch_mfma(const LaunchArgs& a) {
    if (a.D != D) return launch_fwd_padded(a);  // fa_fwd_padded.hip
    return launch_mfma_cfg<T, D, kMfmaWaves, kMfmaKeys, false>(a);
}


hipError_t launch_fwd(const LaunchArgs& a) {
    if (a.kv_lens) return launch_kvcache(a);
    switch (a.dtype) {
    // bf16 / fp16: a head dimension other than 64 and 128 runs the kernel of
    // the next of 64, 128 and 256 up, its extra columns zeros (launch_mfma
    // hands it to fa_fwd_padded.hip)
    case kDtypeBf16:
        return a.D <= 64 ? launch_mfma<__bf16, 64>(a)
                         : a.D <= 128 ? launch_mfma<__bf16, 128>(a) : launch_fwd_padded(a);
    case kDtypeFp16:
        return a.D <= 64 ? launch_mfma<_Float16, 64>(a)
                         : a.D <= 128 ? launch_mfma<_Float16, 128>(a) : launch_fwd_padded(a);
    default:  // fp32: other head dimensions (multiples of 16 up to 128) in fa_fwd_padded.hip
        if (a.D != 64 && a.D != 128) return launch_fwd_padded(a);
        return a.D == 64 ? launch_fp32<64, false>(a) : launch_fp32<128, false>(a);
    }
}

// K/V parts per Q tile for the split launch.  Splitting pays only when the
// unsplit grid leaves compute units short of work: the fp32 partials and the
// merge pass cost about as much as a 2-workgroups-per-CU grid gains from
// shorter chains (measured: the 2K causal workload, 512 workgroups on 256
// CUs, is slower split; 16K causal rows of 2 heads, 256 workgroups, are 20%
// faster in 4 parts).  So: 1 when the grid has at least two workgroups per
// compute unit, else enough parts for four per unit, at most kMaxAutoSplits
// and at most the K/V tile count of the longest Q tile; 1 when the device
// cannot be queried.
constexpr int kMaxAutoSplits = 8;

template <typename T, int D>
static int auto_splits_cfg(const LaunchArgs& a) {
    constexpr int BN = D > 128 ? kWideKeys : kMfmaKeys;
    constexpr int BM = Tile<D, kMfmaWaves, BN>::BM;
    int dev = 0, cus = 0;
    if (hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) {
        (void)hipGetLastError();
        return 1;
    }
    const int64_t n_qt = (a.S + BM - 1) / BM, tiles = a.B * a.H * n_qt;
    const MaskSpec m{a.S, a.causal, a.wl, a.wr};
    int64_t longest = 1;
    for (int64_t t = 0; t < n_qt; ++t) {
        int64_t t0, t1;
        q_tile_kv_range(m, t, BM, BN, &t0, &t1);
        if (t1 - t0 > longest) longest = t1 - t0;
    }
    if (tiles >= 2 * (int64_t)cus) return 1;
    int64_t ns = (4 * (int64_t)cus + tiles - 1) / tiles;
    if (ns > kMaxAutoSplits) ns = kMaxAutoSplits;
    if (ns > longest) ns = longest;
    return ns < 1 ? 1 : (int)ns;
}

int auto_splits(const LaunchArgs& a) {
    switch (a.dtype) {
    case kDtypeBf16:
        return a.D <= 64    ? auto_splits_cfg<__bf16, 64>(a)
               : a.D <= 128 ? auto_splits_cfg<__bf16, 128>(a)
                            : auto_splits_cfg<__bf16, 256>(a);
    case kDtypeFp16:
        return a.D <= 64    ? auto_splits_cfg<_Float16, 64>(a)
               : a.D <= 128 ? auto_splits_cfg<_Float16, 128>(a)
                            : auto_splits_cfg<_Float16, 256>(a);
    default: return 1;  // fp32 inputs run in one part
    }
}

int64_t blocksparse_lut_bytes(int dtype, int64_t D, int64_t S, int64_t n_mask) {
    if (dtype == kDtypeFp32) return 0;  // the fp32 kernel reads the mask itself
    constexpr int BM = kMfmaWaves * kWaveRows;
    const int64_t bn = kv_tile_keys(dtype, D, S, -1, -1);
    const int64_t n_qt = (S + BM - 1) / BM, n_kt = (S + bn - 1) / bn;
    return n_mask * n_qt * sparse_lut_stride(n_kt) * 4;
}

int64_t q_tile_rows(int dtype, int64_t, int64_t, int64_t, int64_t) {
    return dtype == kDtypeFp32 ? kBM32 : kMfmaWaves * kWaveRows;
}
int64_t kv_tile_keys(int dtype, int64_t D, int64_t, int64_t, int64_t) {
    return dtype == kDtypeFp32 ? Lds32<64>::BN : D > 128 ? kWideKeys : kMfmaKeys;
}

}  // namespace fa
