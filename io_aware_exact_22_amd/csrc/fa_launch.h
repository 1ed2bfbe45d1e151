// fa_launch.h -- internal interface between the C ABI (fa_api.hip) and the
// kernel launchers (fa_fwd_kernels.hip).  Not part of the public ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fa {

constexpr int kDtypeFp32 = 0;
constexpr int kDtypeFp16 = 1;
constexpr int kDtypeBf16 = 2;

// bf16 / fp16 kernels: 4 waves, 128-row Q tiles, 64-key K/V tiles (32-key
// tiles above D = 128, whose rows are twice as long)
constexpr int kMfmaWaves = 4, kMfmaKeys = 64, kWideKeys = 32;
// the most K/V parts per Q tile a KV-cache launch takes (FA_MAX_KV_SPLITS)
constexpr int kMaxKvSplits = 64;
// workgroups of the bf16 / fp16 forward kernel one compute unit holds at once
// (register and LDS limits): three at D = 64, two up to 128, one above
constexpr int resident_wgs_per_cu(int64_t D) { return D <= 64 ? 3 : D <= 128 ? 2 : 1; }
// the head dimension a kernel runs at for tensors of head dimension D (other
// multiples of 16 run padded with zero columns)
constexpr int64_t kernel_head_dim(int64_t D) { return D <= 64 ? 64 : D <= 128 ? 128 : 256; }

struct LaunchArgs {
    const void* q;
    const void* k;
    const void* v;
    void* out;
    float* lse;
    int64_t B, H, S, D;
    float c;  // max(scale * log2(e), FLT_MIN): scores enter exp2 directly
    int causal;
    int64_t wl, wr;  // already clamped to [-1, S]
    int dtype;
    hipStream_t stream;
    // split launch (bf16 / fp16 only): > 1 = K/V parts per Q tile, partial
    // results in part_o [n_splits, B, H, S, D] and part_lse [n_splits, B, H, S]
    // (fp32), merged into out / lse by a second kernel
    int n_splits = 1;
    float* part_o = nullptr;
    float* part_lse = nullptr;
    // block-sparse launch: one byte per (query block, key block) in bmask
    // [n_mask, ceil(S / block_m), ceil(S / block_n)], nonzero = the block is
    // kept.  bf16 / fp16 first compact every Q tile's kept K/V tiles into
    // `lut` (blocksparse_lut_bytes); fp32 reads bmask directly.
    const uint8_t* bmask = nullptr;
    int64_t n_mask = 0, block_m = 0, block_n = 0;
    int* lut = nullptr;
    // paged K/V: k and v are pools [pg_count, pg_rows, H, D]; key j of batch b
    // is row j % pg_rows of page pg_table[b * pg_stride + j / pg_rows]
    const int* pg_table = nullptr;
    int64_t pg_stride = 0, pg_rows = 0, pg_count = 0;
    // KV-cache launch (decoding): S is the number of queries per sequence; k
    // and v are caches of kv_cap rows per sequence ([B, kv_cap, H, D], or page
    // pools as above), of which sequence b's first kv_lens[b] (device int32
    // [B], clamped to [0, kv_cap]) are its keys; query row r sits at position
    // r + kv_lens[b] - S.
    const int* kv_lens = nullptr;
    int64_t kv_cap = 0;
};

// The backward pass: gradients for an output gradient dout (bf16 / fp16).
struct BwdArgs {
    const void* q;
    const void* k;
    const void* v;
    const void* out;
    const float* lse;
    const void* dout;
    void* dq;
    void* dk;
    void* dv;
    float* di;  // workspace: D_i = dO_i . O_i, fp32 [B, H, S]
    // workspace, after di: the dynamic-order counters of the dQ and the
    // dK / dV pass (zeroed by the D_i pass)
    unsigned* counters;
    int64_t B, H, S, D;
    float c;      // as in LaunchArgs
    float scale;  // softmax scale
    int causal;
    int64_t wl, wr;
    int dtype;
    hipStream_t stream;
};
// workspace bytes after D_i: the two counters, padded
constexpr int64_t kBwdCounterBytes = 64;
// Enqueues the three backward kernels for validated arguments; D other than
// 64 and 128 (a multiple of 16 up to 128) through launch_bwd_padded.
hipError_t launch_bwd(const BwdArgs& a);
hipError_t launch_bwd_padded(const BwdArgs& a);

// Enqueues the forward kernel (and, for a split launch, the merge kernel) for
// validated arguments.
hipError_t launch_fwd(const LaunchArgs& a);
// The bf16 / fp16 forward at a head dimension other than 64 and 128 (a
// multiple of 16 up to 256), dense, split, block-sparse or paged; above 128,
// launch_fwd_wide_bf16 / _fp16 (one translation unit each).
hipError_t launch_fwd_padded(const LaunchArgs& a);
hipError_t launch_fwd_wide_bf16(const LaunchArgs& a);
hipError_t launch_fwd_wide_fp16(const LaunchArgs& a);
// The KV-cache forward (a.kv_lens set; bf16 / fp16), split or not; at a head
// dimension other than 64 and 128, launch_kvcache_padded.
hipError_t launch_kvcache(const LaunchArgs& a);
hipError_t launch_kvcache_padded(const LaunchArgs& a);
// The merge of a split launch's partial (O, LSE) into out / lse (bf16 / fp16).
hipError_t launch_merge_parts(const LaunchArgs& a);
// K/V parts per Q tile for a KV-cache launch on the current device.
int kvcache_auto_splits(int64_t B, int64_t H, int64_t S_q, int64_t S_k, int64_t D, int dtype);
// Bytes of the compacted tile lists a block-sparse launch needs (0 for fp32).
int64_t blocksparse_lut_bytes(int dtype, int64_t D, int64_t S, int64_t n_mask);

// K/V parts per Q tile that fill the current device for this problem (1 for
// fp32 inputs, or when the device cannot be queried).
int auto_splits(const LaunchArgs& a);
// Tile shape the kernels use: Q rows per workgroup (it depends on the
// configuration the launcher picks for S and the window; wl, wr already
// clamped to [-1, S)), keys per K/V tile.
int64_t q_tile_rows(int dtype, int64_t D, int64_t S, int64_t wl, int64_t wr);
int64_t kv_tile_keys(int dtype, int64_t D, int64_t S, int64_t wl, int64_t wr);

}  // namespace fa
