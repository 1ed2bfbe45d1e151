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

// K/V tile range [*kt0, *kt1) holding every allowed key of the query
// positions [p0, p1] (p1 <= m.S - 1; positions may be negative, see below);
// empty (0, 0) when they allow no key.
__host__ __device__ inline void positions_kv_range(const MaskSpec& m, int64_t p0, int64_t p1,
                                                   int64_t bn, int64_t* kt0, int64_t* kt1) {
    int64_t lo, hi;
    key_range(m, p0, p1, &lo, &hi);
    if (lo > hi) {
        *kt0 = *kt1 = 0;
        return;
    }
    *kt0 = lo / bn;
    *kt1 = hi / bn + 1;
}

// K/V tile range [*kt0, *kt1) visited by Q tile qt of height bm.
__host__ __device__ inline void q_tile_kv_range(const MaskSpec& m, int64_t qt, int64_t bm,
                                                int64_t bn, int64_t* kt0, int64_t* kt1) {
    const int64_t r0 = qt * bm;
    int64_t r1 = r0 + bm - 1;
    if (r1 > m.S - 1) r1 = m.S - 1;
    positions_kv_range(m, r0, r1, bn, kt0, kt1);
}

// Decoding against a key/value cache: a sequence's S_q queries are the last
// S_q positions of its L keys, so query row r sits at position r + L - S_q
// (negative when the cache is shorter than the query block).  With
// MaskSpec{L, ...} every function above then applies to positions: keys are
// [0, L), and the last query's position is L - 1 = m.S - 1.

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

// Workgroup id -> (b * H + h, Q tile).  Consecutive workgroup ids are
// dispatched round-robin over the 8 XCDs of the MI355X, so workgroup w runs on
// XCD w % 8 and is that XCD's (w / 8)-th workgroup.  Each XCD gets a
// contiguous block of the (head-major, Q-tile-minor) list of all tiles: the Q
// tiles of one (batch, head), which stream the same K/V, share that XCD's L2.
//
// by_weight (causal launches, where Q tile t visits about t + 1 K/V tiles):
// rank r of a head's tiles is Q tile n_qt - 1 - r (rank 0 = heaviest).  The
// XCD first runs the heavy ranks [0, R) head by head, heaviest first (one
// head's K/V in its L2 at a time), then the light ranks [R, n_qt) of all its
// heads rank by rank, so that the launch ends on the lightest tiles of every
// head and the workgroups still running at the end have little work left.
// Otherwise the block is walked in list order.  Either way the map is a
// bijection of [0, n_bh * n_qt).  All counts are 32-bit (the host bounds the
// grid well below 2^32 workgroups), which keeps the index arithmetic short.
#ifndef FA_LIGHT_DIV
#define FA_LIGHT_DIV 4  // the lightest 1/FA_LIGHT_DIV of each head's Q tiles close the launch
#endif
//
// snake (by_weight only): the tiles of all heads are sorted heaviest first and
// dealt in snake order instead (snake_item below): every XCD gets one tile of
// each group of eight consecutive weights and runs them heaviest first.  With
// fewer (batch, head) pairs than XCDs this is the only balanced choice (whole
// heads cannot go to XCDs, and contiguous blocks of one head's list would give
// one XCD its heaviest Q tiles and another its lightest); it is also the
// closer fit to longest-first scheduling whenever every head's K/V can stay in
// the MALL while all XCDs work on all heads (snake_launch).
constexpr uint32_t kXcds = 8;
// compute units per XCD of the MI355X (256 / 8)
constexpr uint32_t kCusPerXcd = 32;
// K/V bytes of all heads up to which a causal launch is dealt in snake order:
// half of the MI355X's 256 MB MALL
constexpr int64_t kSnakeKvBytes = int64_t(128) << 20;
__host__ __device__ inline bool snake_launch(int64_t n_bh, int64_t S, int64_t D, int64_t esz) {
    return n_bh < (int64_t)kXcds || 2 * n_bh * S * D * esz <= kSnakeKvBytes;
}

// Item of a weight-sorted list (position 0 = heaviest) that workgroup w runs:
// workgroup w is XCD w % 8's (w / 8)-th workgroup, and the 8 items of group k
// go to the XCDs in the order 0..7 for even k and 7..0 for odd k, so that the
// XCDs' summed weights differ by at most about the heaviest item.  A last,
// partial group goes in order.  A bijection of [0, n).
__host__ __device__ inline uint32_t snake_item(uint32_t w, uint32_t n) {
    const uint32_t x = w % kXcds, k = w / kXcds;
    const bool whole = kXcds * k + kXcds <= n;
    return kXcds * k + ((whole && (k & 1)) ? kXcds - 1 - x : x);
}

__host__ __device__ inline void workgroup_tile(uint32_t w, uint32_t n_bh, uint32_t n_qt,
                                               bool by_weight, bool snake, uint32_t* bh,
                                               uint32_t* qt) {
    const uint32_t n = n_bh * n_qt;
    if (by_weight && snake) {  // list: rank-major, heads next to each other
        // An XCD places its first kCusPerXcd workgroups one per compute unit,
        // then the next kCusPerXcd on the same units again, and so on; every
        // odd such group takes its positions in reverse, so that a unit that
        // got one of the heaviest tiles shares with one of the lighter ones
        // (whole groups of 8 * kCusPerXcd workgroups only: a bijection).
        const uint32_t x = w % kXcds, k = w / kXcds, g = k / kCusPerXcd;
        uint32_t ww = w;
        if ((g & 1) && kXcds * kCusPerXcd * (g + 1) <= n)
            ww = x + kXcds * (g * kCusPerXcd + (kCusPerXcd - 1 - k % kCusPerXcd));
        const uint32_t p = snake_item(ww, n);
        *bh = p % n_bh;
        *qt = n_qt - 1 - p / n_bh;
        return;
    }
    const uint32_t xcd = w % kXcds, idx = w / kXcds;
    const uint32_t per = n / kXcds, rem = n % kXcds;
    const uint32_t s = xcd * per + (xcd < rem ? xcd : rem);  // block start in the list
    if (!by_weight) {
        *bh = (s + idx) / n_qt;
        *qt = (s + idx) % n_qt;
        return;
    }
    // list position p = row * n_qt + rank; the block [s, e] covers row r0 from
    // rank a0 on, rows r0+1 .. r1-1 whole (`full` of them), and row r1 up to
    // rank b1 (r0 == r1: ranks a0 .. b1 of one row)
    const uint32_t e = s + per + (xcd < rem ? 1 : 0) - 1;
    const uint32_t r0 = s / n_qt, a0 = s - r0 * n_qt, r1 = e / n_qt, b1 = e - r1 * n_qt;
    const uint32_t full = r1 > r0 ? r1 - r0 - 1 : 0;
    uint32_t row, rank;
    if (r0 == r1) {  // one row: rank order is heaviest first already
        *bh = r0;
        *qt = n_qt - 1 - (a0 + idx);
        return;
    }
    // block entries with rank < c
    auto before = [&](uint32_t c) {
        return c * full + (c > a0 ? c - a0 : 0) + (c < b1 + 1 ? c : b1 + 1);
    };
    const uint32_t R = n_qt - n_qt / FA_LIGHT_DIV;  // heavy ranks [0, R)
    const uint32_t n_heavy = before(R);
    if (idx < n_heavy) {  // heavy part, row by row
        const uint32_t c0 = R > a0 ? R - a0 : 0;  // heavy entries of row r0
        if (idx < c0) {
            row = r0;
            rank = a0 + idx;
        } else if (idx - c0 < full * R) {
            row = r0 + 1 + (idx - c0) / R;
            rank = (idx - c0) % R;
        } else {
            row = r1;
            rank = idx - c0 - full * R;
        }
    } else {  // light part, rank by rank
        uint32_t lo = R, hi = n_qt - 1;  // the largest c >= R with before(c) <= idx
        while (lo < hi) {
            const uint32_t mid = (lo + hi + 1) / 2;
            if (before(mid) <= idx)
                lo = mid;
            else
                hi = mid - 1;
        }
        rank = lo;
        uint32_t k = idx - before(lo);  // position inside column `rank`
        bool done = false;
        if (rank >= a0) {
            if (k == 0) {
                row = r0;
                done = true;
            } else {
                --k;
            }
        }
        if (!done) row = k < full ? r0 + 1 + k : r1;
    }
    *bh = row;
    *qt = n_qt - 1 - rank;
}

// Workgroup w of a split launch (n_parts K/V parts per Q tile) -> (b * H + h,
// Q tile, part).  by_weight: the parts of all tiles form one list, heaviest
// tile first (rank-major, then head, then part: a part's weight is its tile's
// over n_parts), dealt to the XCDs in snake order.  Otherwise the parts of a
// tile are consecutive workgroups and the tiles follow workgroup_tile.  A
// bijection of [0, n_bh * n_qt * n_parts).
__host__ __device__ inline void workgroup_tile_part(uint32_t w, uint32_t n_bh, uint32_t n_qt,
                                                    uint32_t n_parts, bool by_weight,
                                                    uint32_t* bh, uint32_t* qt, uint32_t* part) {
    if (!by_weight) {
        *part = w % n_parts;
        workgroup_tile(w / n_parts, n_bh, n_qt, false, false, bh, qt);
        return;
    }
    const uint32_t p = snake_item(w, n_bh * n_qt * n_parts);
    const uint32_t t = p / n_parts;
    *part = p % n_parts;
    *bh = t % n_bh;
    *qt = n_qt - 1 - t / n_bh;
}

// ---- Dynamic tail of a causal launch.  A causal launch with more
// workgroups than the device holds at once takes its lightest tiles, about
// kDynSharePct of its K/V steps, in a dynamic order: the Q tiles of all heads
// form one list by rank (rank r: Q tile n_qt - 1 - r, heaviest first), heads
// next to each other.  The ranks below r0 keep the static order by workgroup
// id (snake order, or blocks of whole heads as workgroup_tile deals them);
// each workgroup from id first = r0 * n_bh on takes the next free position
// of the list from a device counter when it starts.  The light tiles then go
// wherever a slot frees up, so a faster XCD takes more of them: XCDs differ
// in speed by a few percent, and with a fixed share each the fast ones idle
// at the end of the launch (measured: 92% of the slot time busy at the 16K
// causal workload, with XCDs ending up to 8% apart).
constexpr int kDynSharePct = 10;

// List position pos -> (b * H + h, Q tile).  The heads rotate by one, so that
// the last position, n_bh * n_qt - 1, is (0, Q tile 0): the tile holding row
// 0 of (b, h) = (0, 0), whose LSE word serves as the counter.
__host__ __device__ inline void dyn_list_tile(uint32_t pos, uint32_t n_bh, uint32_t n_qt,
                                              uint32_t* bh, uint32_t* qt) {
    *bh = (pos + 1) % n_bh;
    *qt = n_qt - 1 - pos / n_bh;
}

// Workgroup w < first -> its list position (a bijection onto [0, first)).
__host__ __device__ inline uint32_t dyn_static_position(uint32_t w, uint32_t n_bh, uint32_t first,
                                                        bool snake) {
    if (snake) return snake_item(w, first);
    const uint32_t r0 = first / n_bh;
    uint32_t bh, q;
    workgroup_tile(w, n_bh, r0, true, false, &bh, &q);  // Q tile q of ranks [0, r0): rank r0-1-q
    return (r0 - 1 - q) * n_bh + (bh + n_bh - 1) % n_bh;
}

// Workgroup w's (b * H + h, tile) in a launch with a dynamic tail from
// position first: by id below it, else the next position from *counter (zero
// before the launch), taken by thread 0 and shared through LDS.  Every thread
// of the workgroup calls it (it holds a barrier).  tile = n_tiles - 1 - rank.
__device__ inline void dynamic_tile(uint32_t w, uint32_t n_bh, uint32_t n_tiles, int first,
                                    bool snake, unsigned* counter, uint32_t* bh,
                                    uint32_t* tile) {
    __shared__ uint32_t s_pos;
    uint32_t pos;
    if ((int)w < first) {
        pos = dyn_static_position(w, n_bh, (uint32_t)first, snake);
    } else {
        if (threadIdx.x == 0) s_pos = (uint32_t)first + atomicAdd(counter, 1u);
        __syncthreads();
        pos = s_pos;
    }
    dyn_list_tile(pos, n_bh, n_tiles, bh, tile);
}

// The first dynamic position of a list of n_tiles ranks over n_bh (batch,
// head) pairs on a device that holds `slots` workgroups at once, where rank r
// weighs weight(r) steps: r0 * n_bh, r0 the first rank whose tail (ranks r0 ..
// n_tiles - 1 of all heads) holds at most kDynSharePct of the steps, or -1
// for the static order (no more workgroups than slots, or an empty tail).
template <typename Weight>
inline int64_t dyn_first_from_weights(int64_t n_bh, int64_t n_tiles, int64_t slots,
                                      Weight weight) {
    if (n_bh * n_tiles <= slots) return -1;
    int64_t total = 0;
    for (int64_t r = 0; r < n_tiles; ++r) total += weight(r);
    int64_t tail = 0, r0 = n_tiles;
    for (int64_t r = n_tiles - 1; r >= 0; --r) {
        if (100 * (tail + weight(r)) > kDynSharePct * total) break;
        tail += weight(r);
        r0 = r;
    }
    return r0 < n_tiles ? r0 * n_bh : -1;
}

// The forward (and the dQ pass): Q tiles bm x K/V tiles bn, rank r = Q tile
// n_qt - 1 - r weighing its K/V tiles; -1 unless causal.
inline int64_t dyn_first_position(const MaskSpec& m, int64_t n_bh, int64_t bm, int64_t bn,
                                  int64_t slots) {
    if (!m.causal) return -1;
    const int64_t n_qt = (m.S + bm - 1) / bm;
    return dyn_first_from_weights(n_bh, n_qt, slots, [&](int64_t r) {
        int64_t t0, t1;
        q_tile_kv_range(m, n_qt - 1 - r, bm, bn, &t0, &t1);
        return t1 - t0;
    });
}

// Query rows [*r0, *r1] that hold an allowed key of key block [j0, j0 + bk)
// (empty when *r0 > *r1).
__host__ __device__ inline void key_block_rows(const MaskSpec& m, int64_t j0, int64_t bk,
                                               int64_t* r0, int64_t* r1) {
    const int64_t j1 = j0 + bk - 1 < m.S - 1 ? j0 + bk - 1 : m.S - 1;
    int64_t lo = m.causal ? j0 : 0, hi = m.S - 1;
    if (m.wr >= 0 && j0 - m.wr > lo) lo = j0 - m.wr;
    if (m.wl >= 0 && j1 + m.wl < hi) hi = j1 + m.wl;
    *r0 = lo;
    *r1 = hi;
}

// The dK / dV pass: key blocks of bk keys, rank r = key block r (with the
// causal mask the lowest blocks hold the most rows) weighing its rows; -1
// unless causal.
inline int64_t dyn_first_key_blocks(const MaskSpec& m, int64_t n_bh, int64_t bk, int64_t slots) {
    if (!m.causal) return -1;
    const int64_t n_kt = (m.S + bk - 1) / bk;
    return dyn_first_from_weights(n_bh, n_kt, slots, [&](int64_t r) {
        int64_t r0, r1;
        key_block_rows(m, r * bk, bk, &r0, &r1);
        return r1 >= r0 ? r1 - r0 + 1 : 0;
    });
}

}  // namespace fa
