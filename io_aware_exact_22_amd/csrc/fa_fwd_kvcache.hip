// fa_fwd_kvcache.hip -- launcher of the forward against a key/value cache
// (decoding: a few new queries per sequence against its cached keys and
// values, per-sequence cache lengths, contiguous or paged caches, optionally
// split over K/V parts with the log-domain merge).  FlashDecoding, the variant
// of the method that serves the KV cache of inference, is named in section 5
// of "FlashAttention技术解析：加速GPT训练的核心优化"; the call
// flash_attn_with_kvcache and the block table of a paged cache in sections
// 总结与最佳实践 and Paged KV Cache支持 of "突破大模型训练瓶颈：Flash-Attention
// 编译优化与内存占用解决方案".  The kernel is fa_fwd_mfma_kernel with KVC = true
// (fa_fwd_device.h).
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "fa_fwd_device.h"
#include "fa_launch.h"
#include "fa_schedule.h"

namespace fa {

template <typename T, int D>
static hipError_t launch_kvcache_cfg(const LaunchArgs& a) {
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
            hipLaunchKernelGGL((fa_fwd_mfma_kernel<T, D, NW, BN, false, false, true, true>),
                               dim3((unsigned)n_wg), dim3(NW * 64), 0, a.stream, (const T*)a.q,
                               (const T*)a.k, (const T*)a.v, (T*)a.out, a.lse, (int)a.B, (int)a.H,
                               (int)a.S, a.c, a.causal, (int)a.wl, (int)a.wr, n_qt, 1, nullptr,
                               nullptr, nullptr, 0, 0, a.pg_table, pg_stride, pg_rows, pg_count,
                               a.kv_lens, cap);
        else
            hipLaunchKernelGGL((fa_fwd_mfma_kernel<T, D, NW, BN, false, false, false, true>),
                               dim3((unsigned)n_wg), dim3(NW * 64), 0, a.stream, (const T*)a.q,
                               (const T*)a.k, (const T*)a.v, (T*)a.out, a.lse, (int)a.B, (int)a.H,
                               (int)a.S, a.c, a.causal, (int)a.wl, (int)a.wr, n_qt, 1, nullptr,
                               nullptr, nullptr, 0, 0, nullptr, 0, 1, 0, a.kv_lens, cap);
        return hipGetLastError();
    }
    if (paged)
        hipLaunchKernelGGL((fa_fwd_mfma_kernel<T, D, NW, BN, true, false, true, true>),
                           dim3((unsigned)(n_wg * a.n_splits)), dim3(NW * 64), 0, a.stream,
                           (const T*)a.q, (const T*)a.k, (const T*)a.v, (T*)a.out, a.lse, (int)a.B,
                           (int)a.H, (int)a.S, a.c, a.causal, (int)a.wl, (int)a.wr, n_qt,
                           a.n_splits, a.part_o, a.part_lse, nullptr, 0, 0, a.pg_table, pg_stride,
                           pg_rows, pg_count, a.kv_lens, cap);
    else
        hipLaunchKernelGGL((fa_fwd_mfma_kernel<T, D, NW, BN, true, false, false, true>),
                           dim3((unsigned)(n_wg * a.n_splits)), dim3(NW * 64), 0, a.stream,
                           (const T*)a.q, (const T*)a.k, (const T*)a.v, (T*)a.out, a.lse, (int)a.B,
                           (int)a.H, (int)a.S, a.c, a.causal, (int)a.wl, (int)a.wr, n_qt,
                           a.n_splits, a.part_o, a.part_lse, nullptr, 0, 0, nullptr, 0, 1, 0,
                           a.kv_lens, cap);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    return launch_merge_parts(a);
}

hipError_t launch_kvcache(const LaunchArgs& a) {
    if (a.dtype == kDtypeBf16)
        return a.D == 64 ? launch_kvcache_cfg<__bf16, 64>(a) : launch_kvcache_cfg<__bf16, 128>(a);
    return a.D == 64 ? launch_kvcache_cfg<_Float16, 64>(a) : launch_kvcache_cfg<_Float16, 128>(a);
}

// Parts per Q tile for a KV-cache launch.  Decoding reads each sequence's
// cache once: the time is the HBM stream, which needs several workgroups per
// compute unit in flight.  So: enough parts for four workgroups per unit, at
// most kMaxKvSplits and at most one part per 4 K/V tiles of a full cache (a
// part's partials and the merge cost about one tile step); 1 when the grid
// already has two workgroups per unit or the device cannot be queried.
int kvcache_auto_splits(int64_t B, int64_t H, int64_t S_q, int64_t S_k, int dtype) {
    (void)dtype;
    int dev = 0, cus = 0;
    if (hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) {
        (void)hipGetLastError();
        return 1;
    }
    constexpr int BM = kMfmaWaves * kWaveRows;
    const int64_t tiles = B * H * ((S_q + BM - 1) / BM);
    if (tiles >= 2 * (int64_t)cus) return 1;
    int64_t ns = (4 * (int64_t)cus + tiles - 1) / tiles;
    const int64_t kv_tiles = (S_k + kMfmaKeys - 1) / kMfmaKeys;
    if (ns > kv_tiles / 4) ns = kv_tiles / 4;
    if (ns > kMaxKvSplits) ns = kMaxKvSplits;
    return ns < 1 ? 1 : (int)ns;
}

}  // namespace fa
