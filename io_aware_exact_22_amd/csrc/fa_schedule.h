// fa_schedule.h -- integer tile schedule of the fused attention forward,
// shared by the host side (argument checks, fa_fwd_tile_schedule) and the
// gfx950 kernels.
//
// The method cuts Q, K and V into tiles ("分块加载" in step 1 of section 二.1
// of "大模型加速新突破：Flash Attention V2核心网络算子解析"; block-wise
// processing in section 3 of "FlashAttention 剖析").  A workgroup owns one Q
// tile and walks the K/V tiles that hold at least one allowed key for one of
// its rows; tiles wholly outside the causal / sliding-window mask are never
// loaded (the window bounds the work to O(n w), section 滑动窗口注意力 of
// "突破大模型训练瓶颈：Flash-Attention编译优化与内存占用解决方案").  Tiles
// where every key is allowed for every row skip the mask.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fa {

// allowed(i, j) with inclusive window bounds; wl/wr < 0 = unbounded.
struct MaskSpec {
    int64_t S;
    int causal;
    int64_t wl, wr;
};

// Keys [lo, hi] hold every allowed key of rows [r0, r1] (r1 <= S-1); every
// key in the range is allowed for at least one of those rows.
__host__ __device__ inline void key_range(const MaskSpec& m, int64_t r0, int64_t r1, int64_t* lo,
                                          int64_t* hi) {
    int64_t a = (m.wl < 0) ? 0 : (r0 - m.wl > 0 ? r0 - m.wl : 0);
    int64_t b = m.S - 1;
    if (m.causal && r1 < b) b = r1;
    if (m.wr >= 0 && r1 + m.wr < b) b = r1 + m.wr;
    *lo = a;
    *hi = b;
}

// K/V tile [k0, k0+bn) against rows [r0, r1] (r1 may exceed S-1: those rows
// are padding and never stored).  True when some (row, key) pair of the block
// is not allowed or the tile runs past S, so the mask must be applied.
__host__ __device__ inline bool tile_needs_mask(const MaskSpec& m, int64_t r0, int64_t r1,
                                                int64_t k0, int64_t bn) {
    const int64_t k1 = k0 + bn - 1;
    if (k1 >= m.S) return true;
    if (m.causal && k1 > r0) return true;
    if (m.wl >= 0 && r1 - k0 > m.wl) return true;
    if (m.wr >= 0 && k1 - r0 > m.wr) return true;
    return false;
}

// True when no (row, key) pair of the block is allowed: the rows skip the
// tile's arithmetic entirely.
__host__ __device__ inline bool tile_fully_masked(const MaskSpec& m, int64_t r0, int64_t r1,
                                                  int64_t k0, int64_t bn) {
    const int64_t k1 = k0 + bn - 1;
    if (r0 >= m.S || k0 >= m.S) return true;
    if (m.causal && k0 > r1) return true;
    if (m.wl >= 0 && r0 - k1 > m.wl) return true;
    if (m.wr >= 0 && k0 - r1 > m.wr) return true;
    return false;
}

// K/V tile range [*kt0, *kt1) visited by Q tile qt of height bm.
__host__ __device__ inline void q_tile_kv_range(const MaskSpec& m, int64_t qt, int64_t bm,
                                                int64_t bn, int64_t* kt0, int64_t* kt1) {
    const int64_t r0 = qt * bm;
    int64_t r1 = r0 + bm - 1;
    if (r1 > m.S - 1) r1 = m.S - 1;
    int64_t lo, hi;
    key_range(m, r0, r1, &lo, &hi);
    if (lo > hi) {
        *kt0 = *kt1 = 0;
        return;
    }
    *kt0 = lo / bn;
    *kt1 = hi / bn + 1;
}

// K/V tiles [*ki0, *ki1) inside [kt0, kt1) where every key is allowed for
// every row of [r0, r0 + bm - 1] and lies below S: the kernel runs them
// without the mask.  The set is contiguous: a tile qualifies when its first
// key is >= F (left window edge of the last row) and its last key is <= L
// (causal / right window edge of the first row, and S - 1).  Tiles of
// [kt0, ki0) and [ki1, kt1) need the mask.
__host__ __device__ inline void q_tile_interior_range(const MaskSpec& m, int64_t r0, int64_t bm,
                                                      int64_t bn, int64_t kt0, int64_t kt1,
                                                      int64_t* ki0, int64_t* ki1) {
    int64_t F = 0;
    if (m.wl >= 0) F = r0 + bm - 1 - m.wl > 0 ? r0 + bm - 1 - m.wl : 0;
    int64_t L = m.S - 1;
    if (m.causal && r0 < L) L = r0;
    if (m.wr >= 0 && r0 + m.wr < L) L = r0 + m.wr;
    int64_t a = (F + bn - 1) / bn;  // first tile with t * bn >= F
    int64_t b = (L + 1) / bn;       // tiles with t * bn + bn - 1 <= L
    if (a < kt0) a = kt0;
    if (a > kt1) a = kt1;
    if (b > kt1) b = kt1;
    if (b < a) b = a;
    *ki0 = a;
    *ki1 = b;
}

// Workgroup id -> logical tile id.  Consecutive workgroup ids are dispatched
// round-robin over the 8 XCDs of the MI355X; this gives each XCD a contiguous
// block of logical ids, so the Q tiles of one (batch, head) -- which stream
// the same K/V -- share that XCD's L2.
__host__ __device__ inline int64_t xcd_remap(int64_t w, int64_t n) {
    constexpr int64_t kXcds = 8;
    const int64_t xcd = w % kXcds, idx = w / kXcds;
    const int64_t per = n / kXcds, rem = n % kXcds;
    return xcd * per + (xcd < rem ? xcd : rem) + idx;
}

}  // namespace fa
