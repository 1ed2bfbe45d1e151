// fa_fwd_launch_cfg.h -- the launches of fa_fwd_mfma_kernel for a dense,
// split, block-sparse or paged forward and for the KV-cache forward, shared by
// fa_fwd_kernels.hip and fa_fwd_kvcache.hip (head dimensions 64 and 128),
// fa_fwd_padded.hip (PAD = true: the kernel for the next of 64 and 128 with
// zero columns) and fa_fwd_wide_*.hip (D above 128), so that the sets of
// instantiations compile in parallel.  Not part of the public ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "fa_fwd_device.h"
#include "fa_launch.h"

namespace fa {

// The first dynamic list position of a dense or paged launch
// (dyn_first_position), for a device holding per_cu workgroups per compute
// unit; -1 (the static order) when the device cannot be queried.
template <int D, int BM, int BN>
int dynamic_first(const LaunchArgs& a, int per_cu) {
    if (!a.causal) return -1;
    int dev = 0, cus = 0;
    if (hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) {
        (void)hipGetLastError();
        return -1;
    }
    const MaskSpec m{a.S, a.causal, a.wl, a.wr};
    return (int)dyn_first_position(m, a.B * a.H, BM, BN, per_cu * (int64_t)cus);
}

// Zeroes the dynamic order's counter (the LSE word of row 0 of head 0) ahead
// of a launch that takes the dynamic tail (dyn >= 0).
inline hipError_t zero_dynamic_counter(const LaunchArgs& a, int dyn) {
    if (dyn < 0) return hipSuccess;
    hipLaunchKernelGGL((fa_zero_word_kernel<>), dim3(1), dim3(64), 0, a.stream,
                       reinterpret_cast<unsigned*>(a.lse));
    return hipGetLastError();
}

template <typename T, int D, int NW, int BN, bool PAD>
hipError_t launch_mfma_cfg(const LaunchArgs& a) {
    constexpr int BM = Tile<D, NW, BN>::BM;
    const int n_qt = (int)((a.S + BM - 1) / BM);
    const int64_t n_wg = a.B * a.H * n_qt;
    if (a.bmask) {  // block-sparse: compact the kept tiles, then walk them
        const int n_kt = (int)((a.S + BN - 1) / BN);
        const int stride = (int)sparse_lut_stride(n_kt);
        hipLaunchKernelGGL((sparse_lut_kernel<BM, BN>), dim3((unsigned)(a.n_mask * n_qt)), dim3(64),
                           0, a.stream, a.bmask, (int)a.S, a.causal, (int)a.wl, (int)a.wr, n_qt,
                           (int)((a.S + a.block_n - 1) / a.block_n),
                           (int)((a.S + a.block_m - 1) / a.block_m), (int)a.block_m,
                           (int)a.block_n, stride, a.lut);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
        hipLaunchKernelGGL((fa_fwd_mfma_kernel<T, D, NW, BN, false, true, false, false, PAD>),
                           dim3((unsigned)n_wg), dim3(NW * 64), 0, a.stream, (const T*)a.q,
                           (const T*)a.k, (const T*)a.v, (T*)a.out, a.lse, (int)a.B, (int)a.H,
                           (int)a.S, a.c, a.causal, (int)a.wl, (int)a.wr, n_qt, 1, nullptr, nullptr,
                           (const int*)a.lut, (int)a.n_mask, stride, nullptr, 0, 1, 0, nullptr, 0, (int)a.D, -1);
        return hipGetLastError();
    }
    const bool paged = a.pg_table != nullptr;
    const int pg_stride = (int)a.pg_stride, pg_rows = paged ? (int)a.pg_rows : 1,
              pg_count = (int)a.pg_count;
    if (a.n_splits <= 1) {
        if (paged) {
            // (the paged kernel holds two workgroups per compute unit at D = 64)
            const int dyn = dynamic_first<D, BM, BN>(a, D <= 64 ? 2 : resident_wgs_per_cu(D));
            const hipError_t e = zero_dynamic_counter(a, dyn);
            if (e != hipSuccess) return e;
            hipLaunchKernelGGL((fa_fwd_mfma_kernel<T, D, NW, BN, false, false, true, false, PAD>),
                               dim3((unsigned)n_wg), dim3(NW * 64), 0, a.stream, (const T*)a.q,
                               (const T*)a.k, (const T*)a.v, (T*)a.out, a.lse, (int)a.B, (int)a.H,
                               (int)a.S, a.c, a.causal, (int)a.wl, (int)a.wr, n_qt, 1, nullptr,
                               nullptr, nullptr, 0, 0, a.pg_table, pg_stride, pg_rows, pg_count,
                               nullptr, 0, (int)a.D, dyn);
        } else {
            const int dyn = dynamic_first<D, BM, BN>(a, resident_wgs_per_cu(D));
            const hipError_t e = zero_dynamic_counter(a, dyn);
            if (e != hipSuccess) return e;
            hipLaunchKernelGGL((fa_fwd_mfma_kernel<T, D, NW, BN, false, false, false, false, PAD>),
                               dim3((unsigned)n_wg), dim3(NW * 64), 0, a.stream, (const T*)a.q,
                               (const T*)a.k, (const T*)a.v, (T*)a.out, a.lse, (int)a.B, (int)a.H,
                               (int)a.S, a.c, a.causal, (int)a.wl, (int)a.wr, n_qt, 1, nullptr,
                               nullptr, nullptr, 0, 0, nullptr, 0, 1, 0, nullptr, 0, (int)a.D, dyn);
        }
        return hipGetLastError();
    }
    if (paged)
        hipLaunchKernelGGL((fa_fwd_mfma_kernel<T, D, NW, BN, true, false, true, false, PAD>),
                           dim3((unsigned)(n_wg * a.n_splits)), dim3(NW * 64), 0, a.stream,
                           (const T*)a.q, (const T*)a.k, (const T*)a.v, (T*)a.out, a.lse, (int)a.B,
                           (int)a.H, (int)a.S, a.c, a.causal, (int)a.wl, (int)a.wr, n_qt,
                           a.n_splits, a.part_o, a.part_lse, nullptr, 0, 0, a.pg_table, pg_stride,
                           pg_rows, pg_count, nullptr, 0, (int)a.D, -1);
    else
        hipLaunchKernelGGL((fa_fwd_mfma_kernel<T, D, NW, BN, true, false, false, false, PAD>),
                           dim3((unsigned)(n_wg * a.n_splits)), dim3(NW * 64), 0, a.stream,
                           (const T*)a.q, (const T*)a.k, (const T*)a.v, (T*)a.out, a.lse, (int)a.B,
                           (int)a.H, (int)a.S, a.c, a.causal, (int)a.wl, (int)a.wr, n_qt,
                           a.n_splits, a.part_o, a.part_lse, nullptr, 0, 0, nullptr, 0, 1, 0,
                           nullptr, 0, (int)a.D, -1);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    return launch_merge_parts(a);
}

// The KV-cache forward on the MFMA kernel (KVC = true), split or not, paged
// or not (fa_fwd_kvcache.hip; with PAD, fa_fwd_kvcache_padded.hip).
template <typename T, int D, bool PAD>
hipError_t launch_kvc_mfma_cfg(const LaunchArgs& a) {
    constexpr int NW = kMfmaWaves, BN = kMfmaKeys;
    constexpr int BM = Tile<D, NW, BN>::BM;
    const int n_qt = (int)((a.S + BM - 1) / BM);
    const int64_t n_wg = a.B * a.H * n_qt;
    const bool paged = a.pg_table != nullptr;
    const int pg_stride = (int)a.pg_stride, pg_rows = paged ? (int)a.pg_rows : 1,
              pg_count = (int)a.pg_count;
    const int cap = (int)a.kv_cap;
    if (a.n_splits <= 1) {
        if (paged)
            hipLaunchKernelGGL((fa_fwd_mfma_kernel<T, D, NW, BN, false, false, true, true, PAD>),
                               dim3((unsigned)n_wg), dim3(NW * 64), 0, a.stream, (const T*)a.q,
                               (const T*)a.k, (const T*)a.v, (T*)a.out, a.lse, (int)a.B, (int)a.H,
                               (int)a.S, a.c, a.causal, (int)a.wl, (int)a.wr, n_qt, 1, nullptr,
                               nullptr, nullptr, 0, 0, a.pg_table, pg_stride, pg_rows, pg_count,
                               a.kv_lens, cap, (int)a.D, -1);
        else
            hipLaunchKernelGGL((fa_fwd_mfma_kernel<T, D, NW, BN, false, false, false, true, PAD>),
                               dim3((unsigned)n_wg), dim3(NW * 64), 0, a.stream, (const T*)a.q,
                               (const T*)a.k, (const T*)a.v, (T*)a.out, a.lse, (int)a.B, (int)a.H,
                               (int)a.S, a.c, a.causal, (int)a.wl, (int)a.wr, n_qt, 1, nullptr,
                               nullptr, nullptr, 0, 0, nullptr, 0, 1, 0, a.kv_lens, cap, (int)a.D, -1);
        return hipGetLastError();
    }
    if (paged)
        hipLaunchKernelGGL((fa_fwd_mfma_kernel<T, D, NW, BN, true, false, true, true, PAD>),
                           dim3((unsigned)(n_wg * a.n_splits)), dim3(NW * 64), 0, a.stream,
                           (const T*)a.q, (const T*)a.k, (const T*)a.v, (T*)a.out, a.lse, (int)a.B,
                           (int)a.H, (int)a.S, a.c, a.causal, (int)a.wl, (int)a.wr, n_qt,
                           a.n_splits, a.part_o, a.part_lse, nullptr, 0, 0, a.pg_table, pg_stride,
                           pg_rows, pg_count, a.kv_lens, cap, (int)a.D, -1);
    else
        hipLaunchKernelGGL((fa_fwd_mfma_kernel<T, D, NW, BN, true, false, false, true, PAD>),
                           dim3((unsigned)(n_wg * a.n_splits)), dim3(NW * 64), 0, a.stream,
                           (const T*)a.q, (const T*)a.k, (const T*)a.v, (T*)a.out, a.lse, (int)a.B,
                           (int)a.H, (int)a.S, a.c, a.causal, (int)a.wl, (int)a.wr, n_qt,
                           a.n_splits, a.part_o, a.part_lse, nullptr, 0, 0, nullptr, 0, 1, 0,
                           a.kv_lens, cap, (int)a.D, -1);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    return launch_merge_parts(a);
}

// fp32 inputs always run in one part (n_splits is ignored): the fp32 kernel
// has no split path.
template <int D, bool PAD>
hipError_t launch_fp32(const LaunchArgs& a) {
    const int n_qt = (int)((a.S + kBM32 - 1) / kBM32);
    const int64_t n_wg = a.B * a.H * n_qt;
    if (a.bmask) {
        hipLaunchKernelGGL((fa_fwd_fp32_kernel<D, true, false, PAD>), dim3((unsigned)n_wg),
                           dim3(kThreads32), 0, a.stream, (const float*)a.q, (const float*)a.k,
                           (const float*)a.v, (float*)a.out, a.lse, (int)a.B, (int)a.H, (int)a.S,
                           a.c, a.causal, (int)a.wl, (int)a.wr, n_qt, a.bmask, (int)a.n_mask,
                           (int)((a.S + a.block_m - 1) / a.block_m),
                           (int)((a.S + a.block_n - 1) / a.block_n), (int)a.block_m, (int)a.block_n,
                           nullptr, 0, 1, 0, (int)a.D);
        return hipGetLastError();
    }
    if (a.pg_table) {
        hipLaunchKernelGGL((fa_fwd_fp32_kernel<D, false, true, PAD>), dim3((unsigned)n_wg),
                           dim3(kThreads32), 0, a.stream, (const float*)a.q, (const float*)a.k,
                           (const float*)a.v, (float*)a.out, a.lse, (int)a.B, (int)a.H, (int)a.S,
                           a.c, a.causal, (int)a.wl, (int)a.wr, n_qt, nullptr, 0, 0, 0, 1, 1,
                           a.pg_table, (int)a.pg_stride, (int)a.pg_rows, (int)a.pg_count, (int)a.D);
        return hipGetLastError();
    }
    hipLaunchKernelGGL((fa_fwd_fp32_kernel<D, false, false, PAD>), dim3((unsigned)n_wg),
                       dim3(kThreads32), 0, a.stream, (const float*)a.q, (const float*)a.k,
                       (const float*)a.v, (float*)a.out, a.lse, (int)a.B, (int)a.H, (int)a.S, a.c,
                       a.causal, (int)a.wl, (int)a.wr, n_qt, nullptr, 0, 0, 0, 1, 1, nullptr, 0, 1,
                       0, (int)a.D);
    return hipGetLastError();
}

}  // namespace fa
