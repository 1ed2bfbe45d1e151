// fa_fwd_device.h -- gfx950 (CDNA4) kernels of the fused exact-attention
// forward: O = softmax(scale * Q K^T + mask) V and the row log-sum-exp, with
// the S x S scores kept in registers and never written to HBM.  Included by
// the launcher sources (fa_fwd_kernels.hip: dense, split, block-sparse and
// paged launches; fa_fwd_kvcache.hip: decoding against a KV cache), each of
// which instantiates only the kernels it launches.  Not part of the public ABI.
//
// Pages cited by title:
//   [V2] "大模型加速新突破：Flash Attention V2核心网络算子解析"
//   [FA] "FlashAttention技术解析：加速GPT训练的核心优化"
//   [CG] "突破大模型训练瓶颈：Flash-Attention编译优化与内存占用解决方案"
//   [AN] "FlashAttention 剖析"
//
// Method (as the pages state it): tile Q, K and V ([V2] section 二.1 step 1;
// [AN] section 3), compute each block's scores, keep a running row max and row
// sum and renormalise online ([FA] section 1 item 3; [V2] section 二.1 step 2),
// accumulate the weighted V blocks ([AN] section 3), keep intermediates in
// registers / on-chip memory ([CG] 项目核心价值; [AN] section 2), fuse the
// steps into one kernel ([CG] 项目核心价值), overlap loads with compute ([FA]
// section 1 item 2; [V2] section 二.2), and use exp2 with log2(e) folded into
// the scale ([CG] 内存优化编译选项, CK_TILE_FMHA_FWD_FAST_EXP2).
//
// gfx950 design (what differs from the pages' CUDA/Tensor Core design):
//  * A workgroup is NW wave64s and owns a 32*NW-row Q tile; each wave owns 32
//    query rows.  K/V tiles of 64 keys stream through LDS: K double-buffered
//    two tiles ahead, V double-buffered one tile ahead, one barrier per tile.
//  * The scores are computed transposed, S^T = K Q^T, on the 32x32x16
//    bf16/f16 MFMA: in the MFMA result layout every lane holds one query row
//    (lane % 32) and 16 of the tile's keys per 32-key block, so the row max /
//    row sum are in-lane reductions plus one exchange between the two wave
//    halves (v_permlane32_swap) instead of a 32-lane shuffle tree.
//  * The output is accumulated transposed too, O^T += V^T P^T: P^T is the
//    B operand straight from the score registers (the K rows of the score MFMA
//    are permuted so each lane's keys come out as 8 consecutive keys per
//    16-key chunk), and V^T is read from the row-major V tile in LDS with the
//    gfx950 transposing LDS read ds_read_b64_tr_b16.  The per-row rescale
//    factor then multiplies whole lanes -- no cross-lane traffic at all.
//  * Software pipeline within each wave: the score MFMAs of tile j+1 run
//    while the VALU computes exp / pack / row sum of tile j, and the P V MFMAs
//    of tile j run while the VALU takes the row max of tile j+1.  The
//    interleave is fixed with scheduling-group barriers so the matrix cores
//    and the vector ALU work at the same time.  bf16 skips the row max on the
//    mask-free tiles after the first and checks each tile's weight sum
//    instead (check_sum): the reference only has to bound the weights.
//  * Whole K/V tiles outside the causal / window mask are not visited; the
//    tiles inside it for every row of the workgroup run a loop body that has
//    no mask code at all; the few boundary tiles apply the mask.
//  * Workgroup ids are remapped so each XCD holds whole (batch, head) groups
//    (L2 reuse of K/V); for causal masks each XCD runs the heaviest Q tiles of
//    all its heads first, so the light tiles fill the end of the launch.  When
//    every head's K/V fits in half the MALL, or there are fewer heads than
//    XCDs, and for causal split launches, the tiles (parts) of all heads are
//    instead dealt to the XCDs in snake order of weight (fa_schedule.h).  A
//    causal launch larger than the device runs its lightest tenth of the
//    work in a dynamic order, each late workgroup taking the next tile from a
//    counter (dynamic_tile), so faster XCDs take more of it.
//  * Probabilities are rounded to the input dtype (RNE, v_cvt_pk_*) for the
//    P V MFMA.  The row sum adds the fp32 weights for bf16 and the fp16-rounded
//    weights two at a time (v_dot2c with ones) for fp16.  Max, exp and the
//    accumulators stay fp32.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "fa_kernel_common.h"
#include "fa_launch.h"
#include "fa_schedule.h"

namespace fa {

// ---------------------------------------------------------------- exact rows
// The P V MFMA multiplies every key of a visited K/V tile by its weight, and a
// key outside a row's mask has weight exactly 0.  For finite values that adds
// exactly 0, but a NaN or an infinity in such a key's value row turns 0 * v
// into NaN for rows that do not allow the key, while the definition sums over
// allowed keys only.  Any non-finite value in a visited tile leaves a
// non-finite O in every row of the wave, so after its last tile a wave tests
// its O accumulator (one FMA with 0 per element) and, only if it finds a NaN
// or an infinity, recomputes its rows with the vector ALU from the final row
// statistics, summing the allowed keys alone.  Finite inputs never take this
// path.  (It also bounds every weight by 1, so huge finite values that
// overflowed the un-normalised fp32 accumulator come out finite.)

// Eight consecutive elements of a row as fp32 (16-byte aligned for 2-byte types).
template <typename T> __device__ inline void load8(const T* p, float (&x)[8]);
template <> __device__ inline void load8<__bf16>(const __bf16* p, float (&x)[8]) {
    const u32x4 w = *reinterpret_cast<const u32x4*>(p);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        x[2 * i] = __uint_as_float(w[i] << 16);
        x[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
    }
}
template <> __device__ inline void load8<_Float16>(const _Float16* p, float (&x)[8]) {
    const f16x8 w = *reinterpret_cast<const f16x8*>(p);
#pragma unroll
    for (int i = 0; i < 8; ++i) x[i] = (float)w[i];
}
template <> __device__ inline void load8<float>(const float* p, float (&x)[8]) {
    const f32x4 a = *reinterpret_cast<const f32x4*>(p), b = *reinterpret_cast<const f32x4*>(p + 4);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        x[i] = a[i];
        x[4 + i] = b[i];
    }
}

// The normalised O columns [hh * D/2, hh * D/2 + D/2) of this lane's query row
// over the keys of K/V positions [w0, w1) that allowed(key) admits, from the
// definition in two passes: the row max m of x_j = c * s_j (a NaN score makes
// it NaN), then l = sum of p_j = exp2(x_j - m) and sum of p_j * v_j, divided
// by l.  m and l come back in m_row and l_row (l = 0: no allowed key, or
// every allowed score -inf; O = 0).  The two lanes of a row (wave halves)
// split the dot product s_j = q . k_j by the same column halves and add the
// halves in the same order.  q_half points at the row's columns of
// this half (nullptr for a padding row past S).  tile_of(pos, k0, row0, valid)
// gives position pos's first key, the row of that key in the K/V tensors (or
// pools) counted from k_head / v_head, and whether the tile lies inside them
// (a tile outside reads as zeros, as the tile loads make it).  Every loop
// bound is wave-uniform, so the half exchange sees all 64 lanes.  PAD: D is
// the padded head dimension of the kernel, dv < D the tensors' own: columns
// at or past dv read as zeros and their acc entries stay 0 (otherwise dv = D).
template <typename T, int D, int BN, bool PAD, typename TileOf, typename Allowed>
__device__ inline __attribute__((always_inline)) void exact_row(
    const T* __restrict__ q_half, const T* __restrict__ k_head, const T* __restrict__ v_head,
    int64_t row_stride, int hh, int dv, int S, int w0, int w1, TileOf tile_of, Allowed allowed,
    float c, float& m_row, float& l_row, float (&acc)[D / 2]) {
    constexpr int DH = D / 2;
    // x_j of the key at element offset off (every lane of the wave calls it)
    auto scaled_score = [&](int64_t off, bool valid) __attribute__((always_inline)) {
        float part = 0.f;
        // a rolled loop: unrolled, the compiler would hoist every chunk's
        // loads at once and raise the kernel's register count
#pragma unroll 1
        for (int c8 = 0; c8 < DH / 8; ++c8) {
            float x[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
            float y[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
            const bool col = !PAD || hh * DH + 8 * c8 < dv;
            if (valid && col) load8<T>(k_head + off + 8 * c8, x);
            if (q_half && col) load8<T>(q_half + 8 * c8, y);
#pragma unroll
            for (int i = 0; i < 8; ++i) part = __builtin_fmaf(y[i], x[i], part);
        }
        return halves_sum(part) * c;
    };
    float m = kNegInf;
    for (int pos = w0; pos < w1; ++pos) {
        int k0;
        int64_t row0;
        bool valid;
        tile_of(pos, k0, row0, valid);
        for (int jj = 0; jj < BN && k0 + jj < S; ++jj) {
            const float x = scaled_score((row0 + jj) * row_stride + (int64_t)hh * DH, valid);
            if (q_half && allowed(k0 + jj) && m == m && (x > m || x != x)) m = x;
        }
    }
#pragma unroll
    for (int d = 0; d < DH; ++d) acc[d] = 0.f;
    float l = 0.f;
    for (int pos = w0; pos < w1; ++pos) {
        int k0;
        int64_t row0;
        bool valid;
        tile_of(pos, k0, row0, valid);
        for (int jj = 0; jj < BN && k0 + jj < S; ++jj) {
            const int64_t off = (row0 + jj) * row_stride + (int64_t)hh * DH;
            const float x = scaled_score(off, valid);
            if (q_half && m != kNegInf && allowed(k0 + jj)) {
                const float p = __builtin_amdgcn_exp2f(x - m);
                l += p;
#pragma unroll
                for (int c8 = 0; c8 < DH / 8; ++c8) {
                    float y[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
                    if (valid && (!PAD || hh * DH + 8 * c8 < dv))
                        load8<T>(v_head + off + 8 * c8, y);
#pragma unroll
                    for (int i = 0; i < 8; ++i) acc[8 * c8 + i] = __builtin_fmaf(p, y[i], acc[8 * c8 + i]);
                }
            }
        }
    }
    const float inv = l == 0.f ? 0.f : 1.f / l;
#pragma unroll
    for (int d = 0; d < DH; ++d) acc[d] *= inv;
    m_row = m;
    l_row = l;
}

// True in every lane when some lane's accumulator holds a NaN or an infinity.
template <int DB> __device__ inline bool any_nonfinite(const f32x16 (&o)[DB]) {
    float z0 = 0.f, z1 = 0.f;
#pragma unroll
    for (int d = 0; d < DB; ++d)
#pragma unroll
        for (int i = 0; i < 16; i += 2) {
            z0 = __builtin_fmaf(o[d][i], 0.f, z0);
            z1 = __builtin_fmaf(o[d][i + 1], 0.f, z1);
        }
    return __any((z0 + z1) != (z0 + z1));
}

// Zeroes the word the dynamic order counts in (lane 0 of one workgroup).
template <int kUnused = 0> __global__ void fa_zero_word_kernel(unsigned* p) {
    if (threadIdx.x == 0) *p = 0u;
}

// SPLIT: the K/V tiles of each Q tile are cut into n_splits contiguous parts,
// one workgroup per (Q tile, part); each writes the partial (O, LSE) of its
// part, in fp32, to part_o [n_splits, B, H, S, D] and part_lse
// [n_splits, B, H, S], for the merge kernel below (the log-domain merge of the
// online softmax, applied once across parts).
// SPARSE and PAGED: see the look-ahead table below.
// Occupancy: D = 64 fits three workgroups per CU in 168 VGPRs; the paged
// variant's page look-ahead needs a few more, and at that cap it spills (bf16:
// 10 dwords a lane), which cost more than the third workgroup gains, so it
// takes two.
// KVC: decoding against a key/value cache.  S is the number of queries per
// sequence; k and v are caches of kv_cap rows per sequence (or page pools),
// of which sequence b's first kv_lens[b] (clamped to [0, kv_cap]) hold its
// keys; query row r sits at position r + kv_lens[b] - S and the masks apply
// to positions.  Cache rows past a sequence's length read as zeros.  A wave
// whose rows are all padding, or allow no key, only takes part in the
// workgroup's loads and barriers.
template <typename T, int D, int NW, int BN_, bool SPLIT, bool SPARSE, bool PAGED, bool KVC,
          bool PAD = false>
__global__ __launch_bounds__(NW * 64, D == 64 ? (PAGED ? 2 : 3) : 1) void fa_fwd_mfma_kernel(
    const T* __restrict__ q, const T* __restrict__ k, const T* __restrict__ v, T* __restrict__ out,
    float* __restrict__ lse, int B, int H, int S, float c, int causal, int wl, int wr, int n_qt,
    int n_splits, float* __restrict__ part_o, float* __restrict__ part_lse,
    const int* __restrict__ sp_lut, int sp_heads, int sp_stride, const int* __restrict__ pg_table,
    int pg_stride, int pg_rows, int pg_count, const int* __restrict__ kv_lens, int kv_cap,
    int dv_in, int dyn_first) {
    static_assert(!(SPLIT && SPARSE), "a block-sparse launch runs in one part");
    static_assert(!(SPARSE && PAGED), "block-sparse and paged K/V do not combine");
    static_assert(!(SPARSE && KVC), "a block mask does not apply to a KV cache");
    typedef Tile<D, NW, BN_> L;
    constexpr int BN = L::BN;
    constexpr int BM = L::BM;
    constexpr int KB = L::KB;
    constexpr int NCH = L::NCH;
    constexpr int RB = L::RB;
    constexpr int KSTEPS = D / 16;  // 16-wide d chunks of the score MFMA
    constexpr int DB = D / 32;      // 32-wide d blocks of the output
    // LDS operand reads run this many MFMAs ahead of their score / P V MFMA;
    // at D = 128 longer leads hide more LDS latency (measured), at D = 64 the
    // extra registers cost more than they hide
    constexpr int kLeadK = D >= 128 ? FA_LEAD_K_D128 : FA_LEAD_K;
    constexpr int kLeadV = D >= 128 ? FA_LEAD_V_D128 : FA_LEAD_V;
    // one object per K / V stage: the compiler then sees that the direct-to-LDS
    // load of one stage never aliases the operand reads of the other, and does
    // not wait for the load before them
    __shared__ __attribute__((aligned(1024))) unsigned char lds_k0[L::MAT];
    __shared__ __attribute__((aligned(1024))) unsigned char lds_k1[L::MAT];
    __shared__ __attribute__((aligned(1024))) unsigned char lds_v0[L::MAT];
    __shared__ __attribute__((aligned(1024))) unsigned char lds_v1[L::MAT];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform per wave
    const int hh = lane >> 5;   // wave half
    const int ql = lane & 31;   // query row of this lane within the wave

    // ---- workgroup -> (b, h, q tile[, part]); causal: heaviest Q tiles first per XCD
    uint32_t bh, qt32, sp32 = 0;
    // (KVC: the tiles' weights depend on cache lengths in device memory; the
    // tiles run in list order)
    if (SPLIT) {  // K/V part sp of the tile
        workgroup_tile_part(blockIdx.x, (uint32_t)B * (uint32_t)H, (uint32_t)n_qt,
                            (uint32_t)n_splits, !KVC && causal != 0, &bh, &qt32, &sp32);
    } else if (!SPARSE && !KVC && dyn_first >= 0) {
        // The dynamic tail of a causal launch (dyn_first_position): workgroups
        // from dyn_first on take the next list position from a counter in the
        // word of lse row 0 of (b, h) = (0, 0), which the host zeroes before
        // the launch.  That row belongs to the last position, so its
        // workgroup writes the word only after every position has been taken.
        dynamic_tile(blockIdx.x, (uint32_t)B * (uint32_t)H, (uint32_t)n_qt, dyn_first,
                     snake_launch((int64_t)B * H, S, D, sizeof(T)),
                     reinterpret_cast<unsigned*>(lse), &bh, &qt32);
    } else {
        workgroup_tile(blockIdx.x, (uint32_t)B * (uint32_t)H, (uint32_t)n_qt, !KVC && causal != 0,
                       snake_launch((int64_t)B * H, S, D, sizeof(T)), &bh, &qt32);
    }
    const int sp = (int)sp32;
    const int qt = (int)qt32;
    const int bb = (int)(bh / (uint32_t)H), h = (int)(bh % (uint32_t)H);

    // ---- keys of this sequence: [0, Sk); query row r sits at position r + off
    // (both S and 0 unless KVC)
    int Sk = S;
    if (KVC) {
        const int len = __builtin_amdgcn_readfirstlane(kv_lens[bb]);
        Sk = len < 0 ? 0 : len > kv_cap ? kv_cap : len;
    }
    const int off = KVC ? Sk - S : 0;

    // ---- K/V tiles of this Q tile: [kt0, kt1); mask-free ones: [ki0, ki1)
    const MaskSpec ms{Sk, causal, wl, wr};
    int kt0, kt1, ki0, ki1;
    {
        int64_t a0, a1, b0, b1;
        if (KVC) {
            const int64_t r1 = (int64_t)qt * BM + BM - 1 < S - 1 ? (int64_t)qt * BM + BM - 1 : S - 1;
            positions_kv_range(ms, (int64_t)qt * BM + off, r1 + off, BN, &a0, &a1);
        } else {
            q_tile_kv_range(ms, qt, BM, BN, &a0, &a1);
        }
        if (SPLIT) {  // part sp of [a0, a1): near-equal tile counts, possibly empty
            const int64_t len = a1 - a0;
            const int64_t p0 = a0 + len * sp / n_splits, p1 = a0 + len * (sp + 1) / n_splits;
            a0 = p0;
            a1 = p1;
        }
        q_tile_interior_range(ms, (int64_t)qt * BM + off, BM, BN, a0, a1, &b0, &b1);
        kt0 = (int)a0;
        kt1 = (int)a1;
        ki0 = (int)b0;
        ki1 = (int)b1;
    }
    // SPARSE: the workgroup walks only the kept K/V tiles of its Q tile, in
    // ascending order: its row of sp_lut holds {kept count, kept tiles below
    // ki0, kept tiles below ki1, 0, tile 0, tile 1, ...} (sparse_lut_kernel).
    // From here on kt0, kt1, ki0 and ki1 count positions in that list; the
    // pipeline steps over positions and maps each to its tile.
    const int* sp_row = nullptr;
    if (SPARSE) {
        const int64_t hm = sp_heads == 1 ? 0 : (sp_heads == H ? (int64_t)h : (int64_t)bh);
        sp_row = sp_lut + (hm * n_qt + qt) * (int64_t)sp_stride;
        kt0 = 0;
        kt1 = __builtin_amdgcn_readfirstlane(sp_row[0]);
        ki0 = __builtin_amdgcn_readfirstlane(sp_row[1]);
        ki1 = __builtin_amdgcn_readfirstlane(sp_row[2]);
    }

    // PAD: the tensors' head dimension is dv_in (a multiple of 16 below D);
    // the kernel works on D columns, the ones at or past dv being zeros that
    // are read as such and never stored.  Otherwise dv = D and every column
    // test below folds away.
    const int dv = PAD ? dv_in : D;
    const int64_t row_stride = (int64_t)H * dv;                     // elements between rows
    const int64_t head_base = ((int64_t)bb * S * H + h) * dv;       // element (b, 0, h, 0)
    // element (b, 0, h, 0) of the K/V tensors (KVC: of the caches)
    const int64_t kv_head_base = KVC ? ((int64_t)bb * kv_cap * H + h) * dv : head_base;
    const int q0 = qt * BM;
    const int qw0 = q0 + wave * kWaveRows;  // first row of this wave
    const int qrow = qw0 + ql;              // this lane's query row
    // SPLIT: this part's partial output rows
    const int64_t part_row = ((int64_t)sp * B * H + bh) * S + qrow;
    if (SPLIT && kt0 == kt1) {  // an empty part (fewer tiles than parts): no keys
        if (qrow < S) {
            if (hh == 0) part_lse[part_row] = kNegInf;
#pragma unroll
            for (int d = 0; d < D / 32; ++d)
#pragma unroll
                for (int g = 0; g < 4; ++g)
                    if (32 * d + 8 * g < dv)
                        *reinterpret_cast<f32x4*>(part_o + part_row * dv + 32 * d + 8 * g + 4 * hh) =
                            f32x4{0.f, 0.f, 0.f, 0.f};
        }
        return;
    }

    // allowed keys of this lane's row: [key_lo, key_lo + key_w] (rows past S
    // are padding: any finite range will do, their results are not stored)
    int key_lo = 0, key_w = S - 1;
    if (qrow < S) {
        const int64_t pos = (int64_t)qrow + off;
        int64_t lo = 0, hi = Sk - 1;
        if (wl >= 0) lo = pos - wl > 0 ? pos - wl : 0;
        if (causal && pos < hi) hi = pos;
        if (wr >= 0 && pos + wr < hi) hi = pos + wr;
        key_lo = (int)lo;
        key_w = (int)(hi - lo);
        if (KVC && hi < lo) {  // no allowed key: a range no key reaches
            key_lo = -(1 << 30);
            key_w = 0;
        }
    }

    // ---- buffer resources over rows [r0, S) of this head: a row past S lies
    // past num_records, so the hardware returns zeros for it
    auto rows_rsrc = [&](const T* base, int64_t r0) __attribute__((always_inline)) {
        const T* p = base + head_base + r0 * row_stride;
        const int64_t bytes = ((S - r0 - 1) * row_stride + dv) * (int64_t)sizeof(T);
        const int64_t nrec = bytes > 0xFFFFFFFFll ? 0xFFFFFFFFll : bytes;
        return __builtin_amdgcn_make_buffer_rsrc((void*)p, (short)0, (int)(uint32_t)nrec,
                                                 kBufferFlags);
    };

    // ---- Q fragment (B operand of S^T = K Q^T): row qrow, d = 16*ks + 8*hh .. +8
    u32x4 qf[KSTEPS];
    {
        const __amdgpu_buffer_rsrc_t rq = rows_rsrc(q, qw0 < S ? qw0 : S - 1);
        const int voff = (ql * (int)row_stride + 8 * hh) * (int)sizeof(T);
#pragma unroll
        for (int ks = 0; ks < KSTEPS; ++ks) {  // columns past dv are zeros
            const bool col = !PAD || 16 * ks + 8 * hh < dv;
            qf[ks] = __builtin_bit_cast(
                u32x4, __builtin_amdgcn_raw_buffer_load_b128(rq, col ? voff + 32 * ks : voff, 0, 0));
            if (!col) qf[ks] = u32x4{0, 0, 0, 0};
        }
        if (qw0 >= S) {
#pragma unroll
            for (int ks = 0; ks < KSTEPS; ++ks) qf[ks] = u32x4{0, 0, 0, 0};
        }
    }

    // ---- K/V tile loader: wave `wave` fills the contiguous LDS bytes
    // [wave * DMA_PER_WAVE KiB, +DMA_PER_WAVE KiB) of the tile; load j writes
    // [(wave * DMA_PER_WAVE + j) * 1024 + 16*lane, +16) with the logical chunk
    // stored there.  dma_voff[j] leaves out the j KiB the load's immediate
    // offset adds.  That is >= 0 when the tensors' rows (H * dv elements) are
    // at least as long as the LDS rows (D elements); PAD, where they can be
    // shorter, starts the tile's buffer resource kBias = kDmaBias bytes
    // before the tile (with kBias more records) instead.  A chunk of columns
    // at or past dv gets an offset past every record count (records are
    // below 2^31 + kDmaBias: one tile, checked on the host), so the load
    // writes zeros.
    constexpr int kBias = PAD ? kDmaBias : 0;
    int dma_voff[L::DMA_PER_WAVE];
#pragma unroll
    for (int j = 0; j < L::DMA_PER_WAVE; ++j) {
        const int byte = (wave * L::DMA_PER_WAVE + j) * 1024 + 16 * lane;
        const int r = byte / RB, pc = (byte % RB) / 16;
        const int lc = pc ^ L::swz(r);  // the logical chunk (8 columns) stored there
        dma_voff[j] = (!PAD || 8 * lc < dv)
                          ? r * (int)row_stride * (int)sizeof(T) + 16 * lc + kBias - 1024 * j
                          : kDmaPastRecords;
    }
    // Buffer resource of K/V tile kt, built with a few scalar ops per tile:
    // base = head start + kt * tile bytes, records = the head's bytes from
    // there on, clamped to 32 bits.  tile_bytes < 2^31 (64 rows, checked on
    // the host), so kt * tile_bytes is one 32 x 32 -> 64-bit product.
    const uint32_t tile_bytes = (uint32_t)(BN * row_stride * (int64_t)sizeof(T));
    const uint64_t head_bytes =
        Sk > 0 ? (uint64_t)(((int64_t)Sk - 1) * row_stride + dv) * sizeof(T) : 0;
    // K/V tiles of the head and the bytes of its last one (<= tile_bytes)
    const int n_kt_head = (Sk + BN - 1) / BN;
    const uint32_t last_bytes =
        (uint32_t)(head_bytes - (uint64_t)(uint32_t)(n_kt_head - 1) * tile_bytes);
    // PAGED: k and v are pools [pg_count, pg_rows, H, D]; key j of batch bb is
    // row j % pg_rows of page pg_table[bb * pg_stride + j / pg_rows].  pg_rows is
    // a multiple of BN, so a tile lies in one page.
    const int64_t kv_base = PAGED ? (int64_t)h * dv : kv_head_base;
    const unsigned char* const k_head = (const unsigned char*)(k + kv_base);
    const unsigned char* const v_head = (const unsigned char*)(v + kv_base);
    // the bases the tile loads use (kBias bytes before the heads)
    const unsigned char* const k_dma = k_head - kBias;
    const unsigned char* const v_dma = v_head - kBias;
    // PAGED: tiles per page, and the bytes of one page of one pool
    const int pg_tiles = PAGED ? pg_rows / BN : 1;
    const uint64_t page_bytes = PAGED ? (uint64_t)pg_rows * (uint64_t)row_stride * sizeof(T) : 0;
    // K/V tile kt (head: k_dma or v_dma, kBias bytes before the head's first
    // row); PAGED: it is tile `in_page` of page `page`
    auto tile_rsrc = [&](const unsigned char* head, int kt, int page, int in_page) __attribute__((always_inline)) {
        if (PAGED) {
            // records stop at row S, and a page index outside the pool reads
            // as zeros instead of reaching past it
            const int k0 = kt * BN;
            const int rows = Sk - k0 < BN ? Sk - k0 : BN;
            const bool ok = (unsigned)page < (unsigned)pg_count && rows > 0;
            const uint64_t off = (uint64_t)(uint32_t)page * page_bytes +
                                 (uint64_t)(uint32_t)in_page * tile_bytes;
            const uint32_t nrec =
                ok ? (uint32_t)(((int64_t)(rows - 1) * row_stride + dv) * (int64_t)sizeof(T)) : 0u;
            return __builtin_amdgcn_make_buffer_rsrc((void*)(head + (ok ? off : 0)), (short)0,
                                                     (int)(nrec + kBias), kBufferFlags);
        }
        const uint64_t off = (uint64_t)(uint32_t)kt * tile_bytes;
        // records cover the tile up to the end of the head's last row: every
        // tile below the last one lies inside the head (its rows are < S - 1),
        // the last one ends at the head's end, and a tile that starts at or
        // past S gets none, so the hardware range check turns every read past
        // the tensor into a zero.  32-bit scalar compares only.
        const uint32_t nrec = kt < n_kt_head - 1 ? tile_bytes + kBias
                              : kt == n_kt_head - 1 ? last_bytes + kBias
                                                    : (uint32_t)kBias;
        return __builtin_amdgcn_make_buffer_rsrc((void*)(head + off), (short)0, (int)nrec,
                                                 kBufferFlags);
    };
    auto load_k = [&](int kt, int page, int rem, unsigned char* buf) __attribute__((always_inline)) {
        dma_matrix<L::DMA_PER_WAVE>(tile_rsrc(k_dma, kt, page, rem),
                                    buf + wave * L::DMA_PER_WAVE * 1024, dma_voff);
    };
    auto load_v = [&](int kt, int page, int rem, unsigned char* buf) __attribute__((always_inline)) {
        dma_matrix<L::DMA_PER_WAVE>(tile_rsrc(v_dma, kt, page, rem),
                                    buf + wave * L::DMA_PER_WAVE * 1024, dma_voff);
    };
    // Look-ahead table (SPARSE: the kept-tile list, indexed by position;
    // PAGED: the batch's block table, indexed by page).  Entries are read by a
    // vector load one step ahead: it lands with the step's K/V loads and is
    // waited for with them (a scalar load would make every LDS wait of the
    // step wait for it too).  Entries past the table read 0.
    const int* const la_base = SPARSE ? sp_row + 4 : PAGED ? pg_table + (int64_t)bb * pg_stride : sp_lut;
    const int la_count = SPARSE ? kt1 : PAGED ? (Sk + pg_rows - 1) / pg_rows : 0;
    const __amdgpu_buffer_rsrc_t la_rsrc = __builtin_amdgcn_make_buffer_rsrc(
        (void*)la_base, (short)0, la_count * 4, kBufferFlags);
    auto la_entry = [&](int idx) __attribute__((always_inline)) {
        return (int)__builtin_amdgcn_raw_buffer_load_b32(la_rsrc, 4 * idx, 0, 0);
    };

    // ---- per-lane LDS operand addresses (bytes within a tile)
    // K: MFMA row m of the score block is key k_row_for_mfma_row(m); lane reads
    // logical chunk 2*kk + hh of it: byte = kaddr[kk] (+ 32*RB per 32-key block)
    int kaddr[KSTEPS];
    {
        const int krow = k_row_for_mfma_row(ql);
        const int kbase = krow * RB + 16 * (hh ^ L::swz(krow));
#pragma unroll
        for (int kk = 0; kk < KSTEPS; ++kk) kaddr[kk] = kbase ^ (32 * kk);
    }
    // V (transposing reads): row 16*cch + 8*hh + 4*rd + jv, element column
    // 32*d + tcol; byte = 16*cch*RB + vaddr[rd][d]
    int vaddr[2][DB];
    {
        const int jv = (lane & 15) >> 2;
        const int tcol = 16 * ((lane >> 4) & 1) + 4 * (lane & 3);
#pragma unroll
        for (int rd = 0; rd < 2; ++rd) {
            const int r = 8 * hh + 4 * rd + jv;
            const int vb = r * RB + 16 * ((tcol / 8) ^ L::swz(r)) + 2 * (tcol % 8);
#pragma unroll
            for (int d = 0; d < DB; ++d) vaddr[rd][d] = vb ^ (64 * d);
        }
    }

    // ---- running statistics (log2 domain: m is a max of c * s).  c >= FLT_MIN
    // (the host clamps it), so a masked score -inf stays -inf after scaling
    // and its weight exp2(-inf) is exactly 0.
    float m_run = kNegInf;  // running reference max
    float m_use = 0.f;      // reference the current tile's weights use
    float m_prev = kNegInf; // running max before the current tile
    bool moved = false;     // some row's reference moved for the current tile (wave-uniform)
    float l_run = 0.f;      // running sum over this half's keys
    float t_sum = 0.f;      // the current tile's weights of this lane (steps that check them)
    // bf16: once every row of the wave has a reference, the steps skip the row
    // max of the next tile and check the weights afterwards (check_sum).  The
    // reference is then no longer a max of the scores, only a bound that
    // keeps the weights finite, which is all O, l and LSE need: they are
    // exact for any reference.  fp16 keeps the max on every tile, since an
    // fp16 weight overflows past 2^16.
    constexpr bool kRefBySum = __is_same(T, __bf16);
    f32x16 o[DB];
#pragma unroll
    for (int d = 0; d < DB; ++d) o[d] = f32x16{0};

    // S^T of one tile for this wave's 32 rows (two 32-key blocks)
    auto qk = [&](f32x16(&s)[KB], const unsigned char* kst) __attribute__((always_inline)) {
#pragma unroll
        for (int kk = 0; kk < KSTEPS; ++kk)
#pragma unroll
            for (int kb = 0; kb < KB; ++kb) {
                const u32x4 a =
                    *reinterpret_cast<const u32x4*>(kst + 32 * kb * RB + kaddr[kk]);
                s[kb] = Mfma<T>::mma(a, qf[kk], kk == 0 ? f32x16{0} : s[kb]);
            }
    };
    // keys outside this lane's allowed range -> -inf
    auto apply_mask = [&](f32x16(&s)[KB], int k0) __attribute__((always_inline)) {
        const int a = k0 + 8 * hh - key_lo;
#pragma unroll
        for (int kb = 0; kb < KB; ++kb)
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                const bool ok = (unsigned)(a + 32 * kb + score_key_base(i)) <= (unsigned)key_w;
                s[kb][i] = ok ? s[kb][i] : kNegInf;
            }
    };
    // row max of a tile -> next reference.  The reference only moves when the
    // tile's max exceeds it by more than kRescaleSlack: weights stay below
    // 2^kRescaleSlack and the O / l rescale is rare.  O, l and LSE all use the
    // same reference, so the result is unchanged up to rounding.
    auto update_max = [&](const f32x16(&s)[KB], bool valid = true) __attribute__((always_inline)) {
        float mx = kNegInf;
#pragma unroll
        for (int kb = 0; kb < KB; ++kb)
#pragma unroll
            for (int i = 0; i < 16; ++i) mx = fmaxf(mx, s[kb][i]);
        const float mt = halves_max(mx) * c;
        const float m_new = (valid && mt > m_run + kRescaleSlack) ? mt : m_run;
        m_use = (m_new == kNegInf) ? 0.f : m_new;  // row fully masked so far
        moved = __any(m_new != m_run);
        m_prev = m_run;
        m_run = m_new;
    };
    // weights of a tile, rounded and packed as the B operand of O^T += V^T P^T;
    // the row sum adds the weights.  The source is skewed (fma of weight i,
    // exp of weight i - 4, pack and sum of weights i - 9 and i - 8) so that the
    // interleave with the MFMAs hands each MFMA slot a mix of independent
    // instructions rather than an exp and the pack that waits for it.
    // SEP: the tile's sum is kept apart in t_sum, then added to l_run.
    auto softmax = [&](const f32x16(&s)[KB], u32x4(&p)[NCH], auto sep_tag) __attribute__((always_inline)) {
        constexpr bool SEP = decltype(sep_tag)::value;
        constexpr int kExpLag = 4, kPackLag = 8;
        constexpr int NE = 16 * KB;  // weights per lane
        float e[NE];
        // partial row sums: the first one starts from the running sum, the
        // others from their first weight (no zero-initialised accumulators,
        // no additions of 0)
        float ls[4];
#pragma unroll
        for (int st = 0; st < NE + kPackLag; ++st) {
            if (st < NE) e[st] = __builtin_fmaf(s[st >> 4][st & 15], c, -m_use);
            const int ie = st - kExpLag;
            if (ie >= 0 && ie < NE) e[ie] = __builtin_amdgcn_exp2f(e[ie]);
            const int ip = st - kPackLag;
            if (ip >= 1 && ip < NE && (ip & 1)) {
                const int q = ip >> 1;  // weight pair
                p[ip >> 3][(ip & 7) >> 1] = Mfma<T>::pack2(e[ip - 1], e[ip]);
                if (Mfma<T>::kSumRounded) {  // two partial sums of packed pairs
                    const unsigned pk = p[ip >> 3][(ip & 7) >> 1];
                    if (q == 0) ls[0] = Mfma<T>::sum2(pk, l_run);
                    else if (q == 1) ls[1] = Mfma<T>::sum2(pk, 0.f);
                    else ls[q & 1] = Mfma<T>::sum2(pk, ls[q & 1]);
                } else {  // four partial sums of single weights
                    if (q == 0) {
                        ls[0] = SEP ? e[ip - 1] : l_run + e[ip - 1];
                        ls[2] = e[ip];
                    } else if (q == 1) {
                        ls[1] = e[ip - 1];
                        ls[3] = e[ip];
                    } else {
                        ls[q & 3] += e[ip - 1];
                        ls[(q + 2) & 3] += e[ip];
                    }
                }
            }
        }
        if (Mfma<T>::kSumRounded) {
            l_run = ls[0] + ls[1];
        } else if (SEP) {
            t_sum = (ls[0] + ls[1]) + (ls[2] + ls[3]);
            l_run += t_sum;
        } else {
            l_run = (ls[0] + ls[1]) + (ls[2] + ls[3]);
        }
    };
    // O^T += V^T P^T with V^T from transposing LDS reads of the row-major tile
    auto pv = [&](const u32x4(&p)[NCH], const unsigned char* vst) __attribute__((always_inline)) {
#pragma unroll
        for (int cch = 0; cch < NCH; ++cch)
#pragma unroll
            for (int d = 0; d < DB; ++d) {
                const unsigned char* vp = vst + 16 * cch * RB;
                const i16x4 lo =
                    __builtin_amdgcn_ds_read_tr16_b64_v4i16((FA_LDS i16x4*)(vp + vaddr[0][d]));
                const i16x4 hi =
                    __builtin_amdgcn_ds_read_tr16_b64_v4i16((FA_LDS i16x4*)(vp + vaddr[1][d]));
                const u32x2 l2 = __builtin_bit_cast(u32x2, lo), h2 = __builtin_bit_cast(u32x2, hi);
                const u32x4 a = {l2[0], l2[1], h2[0], h2[1]};
                o[d] = Mfma<T>::mma(a, p[cch], o[d]);
            }
    };
    // After a tile whose weights were made without its row max: when some
    // lane's share of them exceeds kSumLimit (rare), each such row's reference
    // moves up by n = ceil(log2) of the row's tile sum, and its O and l are
    // scaled by 2^-n, exactly.  Its tile weights are then at most 1.  A sum
    // that is not finite leaves O or l non-finite, and the epilogue's exact
    // recomputation takes the wave.
    auto check_sum = [&]() __attribute__((always_inline)) {
        if (__any(t_sum > kSumLimit)) {
            const float rt = halves_sum(t_sum);
            const int n = rt > kSumLimit ? (int)__builtin_ceilf(__log2f(fminf(rt, 0x1p126f))) : 0;
            m_run += (float)n;
            m_use = (m_run == kNegInf) ? 0.f : m_run;
            l_run = __builtin_amdgcn_ldexpf(l_run, -n);
#pragma unroll
            for (int d = 0; d < DB; ++d)
#pragma unroll
                for (int i = 0; i < 16; ++i) o[d][i] = __builtin_amdgcn_ldexpf(o[d][i], -n);
        }
    };
    auto rescale_if_moved = [&]() __attribute__((always_inline)) {
        if (moved) {  // only when some row's reference moved
            // factor O and l take: old reference over new (0 for a row whose
            // first allowed keys are in this tile: O and l are still 0)
            const float alpha = __builtin_amdgcn_exp2f(m_prev - m_use);
            l_run *= alpha;
#pragma unroll
            for (int d = 0; d < DB; ++d) o[d] *= alpha;
        }
    };

    // K/V positions this wave computed: [ex_w0, ex_w1) (for the exact
    // recomputation in the epilogue)
    int ex_w0 = kt0, ex_w1 = kt0;
    // A block-sparse Q tile may keep no tile at all: its rows have no allowed
    // key, and the epilogue writes O = 0, LSE = -inf.
    if ((!SPARSE && !KVC) || kt1 > kt0) {
    // ---- prologue: K of the first two tiles, V of the first, scores of the first
    f32x16 sc[KB];  // scores of the current tile (masked)
    int tile_a = kt0, tile_b = kt0 + 1;  // tiles of positions kt0, kt0 + 1
    int page_a = 0, page_b = 0;          // PAGED: their pages
    int rem_a = 0, rem_b = 0;            // PAGED: their tile numbers within their pages
    // look-ahead state at step j: the entry of position j + 1 (la_t1) and the
    // entry of position j + 2 (la_nx, in flight since step j - 1); PAGED also
    // carries the in-page tile numbers of positions j + 1, j + 2 (rm1, rm2)
    // and the table index and in-page number of position j + 3 (nx_idx,
    // nx_rem), advanced by counting instead of dividing
    int la_t1 = 0, la_nx = 0, rm1 = 0, rm2 = 0, nx_idx = 0, nx_rem = 0;
    auto next_tile = [&](int& idx, int& rem) __attribute__((always_inline)) {
        if (++rem == pg_tiles) {
            rem = 0;
            ++idx;
        }
    };
    if (SPARSE) {
        tile_a = __builtin_amdgcn_readfirstlane(sp_row[4]);
        tile_b = kt1 > 1 ? __builtin_amdgcn_readfirstlane(sp_row[5]) : 0;
    }
    int idx_b = 0;
    if (PAGED) {
        const int idx_a = kt0 / pg_tiles;
        rem_a = kt0 - idx_a * pg_tiles;
        idx_b = idx_a;
        rem_b = rem_a;
        next_tile(idx_b, rem_b);
        page_a = __builtin_amdgcn_readfirstlane(la_base[idx_a]);
        page_b = kt0 + 1 < kt1 ? __builtin_amdgcn_readfirstlane(la_base[idx_b]) : 0;
    }
    load_k(tile_a, page_a, rem_a, lds_k0);
    if (kt0 + 1 < kt1) load_k(tile_b, page_b, rem_b, lds_k1);
    load_v(tile_a, page_a, rem_a, lds_v0);
    if (SPARSE) {
        la_t1 = tile_b;
        la_nx = la_entry(kt0 + 2);
    }
    if (PAGED) {
        la_t1 = page_b;
        rm1 = rem_b;
        nx_idx = idx_b;
        nx_rem = rem_b;
        next_tile(nx_idx, nx_rem);  // position kt0 + 2
        la_nx = la_entry(nx_idx);
        rm2 = nx_rem;
        next_tile(nx_idx, nx_rem);  // position kt0 + 3
    }
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
    // K/V tiles this wave computes: [kw0, kw1), the tiles of [kt0, kt1) that
    // hold an allowed key for one of its own 32 rows (a window or the causal
    // diagonal leaves some tiles of the workgroup empty for some of its
    // waves).  The loads and barriers still run over the workgroup's
    // [kt0, kt1), so every wave passes the same barriers.  Padding rows past
    // S take the workgroup's range.
    // (SPARSE: every wave walks every kept tile; a tile without an allowed key
    // for some of a wave's rows gives those rows weight 0.)
    int kw0 = kt0, kw1 = kt1;
    bool wave_idle = KVC && qw0 >= S;  // KVC: no query row in this wave
    if (!SPARSE && qw0 < S) {
        int64_t lo, hi;
        key_range(ms, (int64_t)qw0 + off,
                  (int64_t)(qw0 + kWaveRows - 1 < S - 1 ? qw0 + kWaveRows - 1 : S - 1) + off, &lo,
                  &hi);
        kw0 = (int)(lo / BN) > kt0 ? (int)(lo / BN) : kt0;
        kw1 = (int)(hi / BN) + 1 < kt1 ? (int)(hi / BN) + 1 : kt1;
        if (KVC && (lo > hi || kw0 >= kw1)) wave_idle = true;  // its rows allow no key
    }
    if (SPLIT && kw0 >= kw1) {  // no allowed key of these rows in this part:
        kw0 = kt0;              // run it all, fully masked (l = 0, O = 0)
        kw1 = kt1;
    }
    kw0 = __builtin_amdgcn_readfirstlane(kw0);
    kw1 = __builtin_amdgcn_readfirstlane(kw1);
    ex_w0 = kw0;
    ex_w1 = kw1;
    // the tiles this wave runs without the mask: every key allowed for each of
    // its own 32 rows (a superset of the workgroup's [ki0, ki1): near a window
    // edge or the causal diagonal a wave needs the mask on fewer tiles than the
    // workgroup as a whole).  SPARSE positions keep the workgroup's range.
    if (!SPARSE && qw0 < S) {
        int64_t b0, b1;
        q_tile_interior_range(ms, (int64_t)qw0 + off, kWaveRows, BN, kt0, kt1, &b0, &b1);
        ki0 = __builtin_amdgcn_readfirstlane((int)b0);
        ki1 = __builtin_amdgcn_readfirstlane((int)b1);
    }
    // tiles (and pages) of positions j + 1 and j + 2 at the step of position
    // j; advances the look-ahead by one position (every wave runs it once per
    // position, in its compute steps and its idle steps alike)
    auto look_ahead = [&](int j, int& tn1, int& tn2, int& pn1, int& pn2, int& r1, int& r2)
                          __attribute__((always_inline)) {
        tn1 = j + 1;
        tn2 = j + 2;
        pn1 = pn2 = r1 = r2 = 0;
        if (SPARSE) {
            tn1 = la_t1;
            tn2 = __builtin_amdgcn_readfirstlane(la_nx);
            la_t1 = tn2;
            la_nx = la_entry(j + 3);
        }
        if (PAGED) {
            pn1 = la_t1;
            pn2 = __builtin_amdgcn_readfirstlane(la_nx);
            r1 = rm1;
            r2 = rm2;
            la_t1 = pn2;
            rm1 = rm2;
            la_nx = la_entry(nx_idx);  // position j + 3
            rm2 = nx_rem;
            next_tile(nx_idx, nx_rem);
        }
    };
    // scores of the tile at position pos (tile number `tile`)
    auto first_scores = [&](int pos, int tile, unsigned char* kst) __attribute__((always_inline)) {
        qk(sc, kst);
        if (pos < ki0 || pos >= ki1) apply_mask(sc, tile * BN);
        update_max(sc);
        moved = false;  // O and l are still zero
    };
    if (!wave_idle && kw0 == kt0) first_scores(kt0, tile_a, lds_k0);

    // ---- one pipelined step for tile j: S_{j+1} = K_{j+1} Q^T and the weights
    // of tile j, then O += P_j V_j and the row max of tile j+1.  STAGE = (j -
    // kt0) & 1: K_j sat in K stage STAGE (its slot is free now), K_{j+1} is in
    // K stage STAGE^1, V_j in V stage STAGE.  MASK_NEXT: tile j+1 needs the
    // mask.  LAST: j is the final tile.  MODE 0: the row max of tile j+1 sets
    // its reference; 1: no row max, tile j's weights are checked after the
    // step (check_sum); 2: tile j's weights are checked, then the row max of
    // tile j+1 (the step after a run of mode 1).
    auto step = [&](int j, auto stage_tag, auto mask_next_tag, auto last_tag, auto mode_tag)
                    __attribute__((always_inline)) {
        constexpr int ST = decltype(stage_tag)::value;
        constexpr bool MASK_NEXT = decltype(mask_next_tag)::value;
        constexpr bool LAST = decltype(last_tag)::value;
        constexpr int MODE = decltype(mode_tag)::value;
        unsigned char* const k_this = ST ? lds_k1 : lds_k0;  // K_j (free), later K_{j+2}
        unsigned char* const k_next = ST ? lds_k0 : lds_k1;  // K_{j+1}
        unsigned char* const v_this = ST ? lds_v1 : lds_v0;  // V_j
        unsigned char* const v_next = ST ? lds_v0 : lds_v1;  // V_{j+1}
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");  // K_{j+1}, V_j have landed
        __syncthreads();  // ... for every wave; every wave is done with tile j-1
        int tn1, tn2, pn1, pn2, r1, r2;  // tiles of positions j + 1, j + 2; their pages
        look_ahead(j, tn1, tn2, pn1, pn2, r1, r2);
        if (!LAST) {
            if (j + 2 < kt1) load_k(tn2, pn2, r2, k_this);
            load_v(tn1, pn1, r1, v_next);
        } else {  // this wave's last tile; the workgroup may go on
            if (j + 2 < kt1) load_k(tn2, pn2, r2, k_this);
            if (j + 1 < kt1) load_v(tn1, pn1, r1, v_next);
        }
        rescale_if_moved();
        u32x4 p[NCH];
        if (!LAST) {
            f32x16 sn[KB];
            qk(sn, k_next);
            softmax(sc, p, BoolTag<(MODE != 0)>{});
            pv(p, v_this);
            // interleave: every MFMA of the step (score MFMAs first, then P V)
            // carries the same share of the VALU work -- the weights of tile
            // j, then (mode 0) the row max of tile j+1 -- so neither phase is
            // VALU-bound while the other leaves the vector ALU idle.
            // Operand reads from LDS run ahead of their MFMA: kLeadK score
            // MFMAs, kLeadV P V MFMAs (LDS latency under load is several
            // MFMAs).  Mode 2 branches between its P V MFMAs and the row max,
            // so its interleave covers the weights only.
            auto interleave = [&]() __attribute__((always_inline)) {
                constexpr int NQK = KB * KSTEPS, NPV = NCH * DB;
                // fma + exp per weight, one cvt per pair, the row sum, the max
                constexpr int NVALU =
                    KB * (32 + 8 + (MODE == 0 ? 8 : 0) + (Mfma<T>::kSumRounded ? 8 : 16)) +
                    (MODE == 0 ? 16 : 4);
                constexpr int VALU_PER = (NVALU + NQK + NPV - 1) / (NQK + NPV);
                __builtin_amdgcn_sched_group_barrier(kSgDsRead, kLeadK, 0);
#pragma unroll
                for (int i = 0; i < NQK; ++i) {
                    __builtin_amdgcn_sched_group_barrier(kSgMfma, 1, 0);
                    __builtin_amdgcn_sched_group_barrier(kSgValu, VALU_PER, 0);
                    if (i + kLeadK < NQK) __builtin_amdgcn_sched_group_barrier(kSgDsRead, 1, 0);
                    // the first V reads start under the last score MFMAs
                    if (i + kLeadV >= NQK) __builtin_amdgcn_sched_group_barrier(kSgDsRead, 2, 0);
                }
#pragma unroll
                for (int i = 0; i < NPV; ++i) {
                    __builtin_amdgcn_sched_group_barrier(kSgMfma, 1, 0);
                    __builtin_amdgcn_sched_group_barrier(kSgValu, VALU_PER, 0);
                    if (i + kLeadV < NPV) __builtin_amdgcn_sched_group_barrier(kSgDsRead, 2, 0);
                }
            };
            if (MODE == 2) {
                asm volatile("" : "+v"(l_run));
                interleave();
                check_sum();
            }
            if (MASK_NEXT) apply_mask(sn, tn1 * BN);
            if (MODE == 1)
                moved = false;
            else
                update_max(sn);
#pragma unroll
            for (int kb = 0; kb < KB; ++kb) sc[kb] = sn[kb];
            // The row sum of this tile's weights is finished inside this step,
            // among its MFMAs.  Without this the compiler sinks the adds of
            // every other step into the next one, ahead of its first MFMA,
            // where no MFMA hides them (and ten P V MFMAs go without VALU work).
            asm volatile("" : "+v"(l_run));
            if (MODE != 2) interleave();
            if (MODE == 1) check_sum();
        } else {
            softmax(sc, p, BoolTag<kRefBySum>{});
            pv(p, v_this);
            if (kRefBySum) check_sum();
        }
    };
    // iterations [j0, j1), none of them the last; the stage alternates
    auto run = [&](int j0, int j1, auto mask_next_tag, auto mode_tag) __attribute__((always_inline)) {
        int j = j0;
        if (j < j1 && ((j - kt0) & 1)) {
            step(j, IntTag<1>{}, mask_next_tag, BoolTag<false>{}, mode_tag);
            ++j;
        }
        for (; j + 1 < j1; j += 2) {
            step(j, IntTag<0>{}, mask_next_tag, BoolTag<false>{}, mode_tag);
            step(j + 1, IntTag<1>{}, mask_next_tag, BoolTag<false>{}, mode_tag);
        }
        if (j < j1) step(j, IntTag<0>{}, mask_next_tag, BoolTag<false>{}, mode_tag);
    };

    // a step of the workgroup's loads and barrier only (outside [kw0, kw1))
    auto idle_step = [&](int j) __attribute__((always_inline)) {
        const bool st = ((j - kt0) & 1) != 0;
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        __syncthreads();
        int tn1, tn2, pn1, pn2, r1, r2;
        look_ahead(j, tn1, tn2, pn1, pn2, r1, r2);
        if (j + 2 < kt1) load_k(tn2, pn2, r2, st ? lds_k1 : lds_k0);
        if (j + 1 < kt1) load_v(tn1, pn1, r1, st ? lds_v0 : lds_v1);
    };
    if (wave_idle) {  // KVC: loads and barriers only; O = 0, l = 0 (LSE = -inf)
        for (int j = kt0; j < kt1; ++j) idle_step(j);
    } else {
    if (!SPARSE) {
        for (int j = kt0; j + 1 < kw0; ++j) idle_step(j);
        if (kw0 > kt0) {  // the step before the wave's first tile: its scores
            const int j = kw0 - 1;
            idle_step(j);
            first_scores(kw0, kw0, ((j - kt0) & 1) ? lds_k0 : lds_k1);
        }
    }
    // iteration j has a mask-free next tile iff ki0 <= j + 1 < ki1
    const int jl = kw1 - 1;
    int ja = ki0 - 1 > kw0 ? ki0 - 1 : kw0;
    if (ja > jl) ja = jl;
    int jb = ki1 - 1 < jl ? ki1 - 1 : jl;
    if (jb < ja) jb = ja;
    if constexpr (kRefBySum) {
        // The row max of the first mask-free tile gives every row of the wave
        // a reference (all its keys are allowed for every row): the head
        // steps take it too (its mask changes nothing).  The mask-free steps
        // after it skip the row max; the steps after them check their tile
        // before the row max of the next (mode 2), and so does the last.
        const int jh = ja < jb ? ja + 1 : ja;
        run(kw0, jh, BoolTag<true>{}, IntTag<0>{});
        run(jh, jb, BoolTag<false>{}, IntTag<1>{});
        run(jb, jl, BoolTag<true>{}, IntTag<2>{});
    } else {
        run(kw0, ja, BoolTag<true>{}, IntTag<0>{});
        run(ja, jb, BoolTag<false>{}, IntTag<0>{});
        run(jb, jl, BoolTag<true>{}, IntTag<0>{});
    }
    if ((jl - kt0) & 1)
        step(jl, IntTag<1>{}, BoolTag<false>{}, BoolTag<true>{}, IntTag<0>{});
    else
        step(jl, IntTag<0>{}, BoolTag<false>{}, BoolTag<true>{}, IntTag<0>{});
    if (!SPARSE)
        for (int j = kw1; j < kt1; ++j) idle_step(j);
    }  // the wave computes
    }  // kt1 > kt0

    // ---- epilogue: O = O_acc / l, LSE = ln2 * (m + log2 l)
    // l == 0 only for a row with no allowed key; a NaN l (NaN scores) propagates
    const float l_tot = halves_sum(l_run);
    const float inv = (l_tot == 0.f) ? 0.f : 1.f / l_tot;
    const float m_fin = (m_run == kNegInf) ? 0.f : m_run;
    const float lse_v = (l_tot == 0.f) ? kNegInf : 0.69314718055994531f * (m_fin + __log2f(l_tot));
    // a NaN or an infinity in O, or a row sum that is not finite: this wave
    // recomputes its rows over their allowed keys only (exact_row), stores
    // them and their LSE, and is done
    if (any_nonfinite<DB>(o) || __any(!(l_tot < __builtin_inff()))) {
        constexpr int DH = D / 2;
        float acc[DH];
        auto tile_of = [&](int pos, int& k0, int64_t& row0, bool& valid) __attribute__((always_inline)) {
            const int tile = SPARSE ? sp_row[4 + pos] : pos;
            k0 = tile * BN;
            row0 = k0;
            valid = true;
            if (PAGED) {
                const int page = pg_table[(int64_t)bb * pg_stride + tile / pg_tiles];
                valid = (unsigned)page < (unsigned)pg_count;
                row0 = (int64_t)(valid ? page : 0) * pg_rows + (int64_t)(tile % pg_tiles) * BN;
            }
        };
        auto allowed = [&](int key) __attribute__((always_inline)) {
            return (unsigned)(key - key_lo) <= (unsigned)key_w;
        };
        const T* q_half = qrow < S ? q + head_base + (int64_t)qrow * row_stride + hh * DH : nullptr;
        float m_x, l_x;
        exact_row<T, D, BN, PAD>(q_half, (const T*)k_head, (const T*)v_head, row_stride, hh, dv, Sk, ex_w0,
                            ex_w1, tile_of, allowed, c, m_x, l_x, acc);
        const float lse_x = (l_x == 0.f) ? kNegInf : 0.69314718055994531f * (m_x + __log2f(l_x));
        if (qrow < S) {
            if (SPLIT) {
                if (hh == 0) part_lse[part_row] = lse_x;
#pragma unroll
                for (int c4 = 0; c4 < DH / 4; ++c4)
                    if (!PAD || hh * DH + 4 * c4 < dv)
                        *reinterpret_cast<f32x4*>(part_o + part_row * dv + hh * DH + 4 * c4) =
                            f32x4{acc[4 * c4], acc[4 * c4 + 1], acc[4 * c4 + 2], acc[4 * c4 + 3]};
            } else {
                if (hh == 0) lse[((int64_t)bb * H + h) * S + qrow] = lse_x;
                T* const orow = out + head_base + (int64_t)qrow * row_stride + hh * DH;
#pragma unroll
                for (int c8 = 0; c8 < DH / 8; ++c8)
                    if (!PAD || hh * DH + 8 * c8 < dv)
                        *reinterpret_cast<u32x4*>(orow + 8 * c8) = u32x4{
                            Mfma<T>::pack2(acc[8 * c8], acc[8 * c8 + 1]),
                            Mfma<T>::pack2(acc[8 * c8 + 2], acc[8 * c8 + 3]),
                            Mfma<T>::pack2(acc[8 * c8 + 4], acc[8 * c8 + 5]),
                            Mfma<T>::pack2(acc[8 * c8 + 6], acc[8 * c8 + 7])};
            }
        }
        return;
    }
    if (SPLIT) {  // the part's normalised O and its LSE, in fp32
        if (qrow < S) {
            if (hh == 0) part_lse[part_row] = lse_v;
#pragma unroll
            for (int d = 0; d < DB; ++d)
#pragma unroll
                for (int g = 0; g < 4; ++g)
                    if (32 * d + 8 * g < dv)
                        *reinterpret_cast<f32x4*>(part_o + part_row * dv + 32 * d + 8 * g + 4 * hh) =
                            f32x4{o[d][4 * g] * inv, o[d][4 * g + 1] * inv, o[d][4 * g + 2] * inv,
                                  o[d][4 * g + 3] * inv};
        }
        return;
    }
    if (qrow < S && hh == 0) lse[((int64_t)bb * H + h) * S + qrow] = lse_v;
    if constexpr (D > 128) {
        // The K stages hold half of the output tile: each lane stores its own
        // 8-byte pieces (columns 32d + 8g + 4*hh .. +3 of its row) directly.
        if (qrow < S) {
            T* const orow = out + head_base + (int64_t)qrow * row_stride + 4 * hh;
#pragma unroll
            for (int d = 0; d < DB; ++d)
#pragma unroll
                for (int g = 0; g < 4; ++g)
                    if (!PAD || 32 * d + 8 * g < dv)
                        *reinterpret_cast<u32x2*>(orow + 32 * d + 8 * g) =
                            u32x2{Mfma<T>::pack2(o[d][4 * g] * inv, o[d][4 * g + 1] * inv),
                                  Mfma<T>::pack2(o[d][4 * g + 2] * inv, o[d][4 * g + 3] * inv)};
        }
        return;
    } else {
    // O leaves through LDS so that the global stores run along whole rows: a
    // lane holds one row's columns 32d + 8g + 4*hh .. +3, so it writes them
    // into the wave's 32 x D staging tile (16-byte chunk c of row r stored at
    // chunk c ^ (r % NC): the column-wise writes spread over the banks), and
    // then each lane reads and stores 16 contiguous bytes of a row.  The K
    // stages are free here: no wave reads K in the last step.
    constexpr int NC = RB / 16;                 // 16-byte chunks per row
    constexpr int WAVE_BYTES = kWaveRows * RB;  // one wave's staging tile
    constexpr int ROWS_PER_READ = 1024 / RB;    // rows one 16-byte-per-lane read covers
    static_assert(2 * L::MAT >= NW * WAVE_BYTES, "the K stages hold the output tile");
    unsigned char* const stg = wave * WAVE_BYTES < L::MAT
                                   ? lds_k0 + wave * WAVE_BYTES
                                   : lds_k1 + (wave * WAVE_BYTES - L::MAT);
#pragma unroll
    for (int d = 0; d < DB; ++d)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
            const u32x2 w = {Mfma<T>::pack2(o[d][4 * g] * inv, o[d][4 * g + 1] * inv),
                             Mfma<T>::pack2(o[d][4 * g + 2] * inv, o[d][4 * g + 3] * inv)};
            const int chunk = (4 * d + g) ^ (ql & (NC - 1));
            *reinterpret_cast<u32x2*>(stg + ql * RB + 16 * chunk + 8 * hh) = w;
        }
    {
        const int rl = lane / NC, cl = lane % NC;
        T* const orow = out + head_base + 8 * cl;
#pragma unroll
        for (int i = 0; i < kWaveRows / ROWS_PER_READ; ++i) {
            const int r = i * ROWS_PER_READ + rl;
            const u32x4 x =
                *reinterpret_cast<const u32x4*>(stg + r * RB + 16 * (cl ^ (r & (NC - 1))));
            if (qw0 + r < S && (!PAD || 8 * cl < dv))
                *reinterpret_cast<u32x4*>(orow + (int64_t)(qw0 + r) * row_stride) = x;
        }
    }
    }  // D <= 128
}

// ================================================================ block-sparse
// Block-sparse attention keeps key j for query i only where the mask byte of
// (query block i / block_m, key block j / block_n) is nonzero, on top of the
// causal / window mask ("FlashAttention技术解析：加速GPT训练的核心优化" section
// 5 lists the block-sparse variant for very long contexts).  block_m is a
// multiple of the Q tile and block_n of the K/V tile, so a kept block is a
// set of whole tiles for every row of a Q tile: skipping a dropped tile needs
// no per-element mask, and a kept one is masked exactly as in the dense case.
//
// sparse_lut_kernel compacts, for every (mask head, Q tile), the kept K/V
// tiles of the tile range the dense kernel would walk into an ascending list:
// row r = hm * n_qt + qt of lut, sp_stride ints, holds {count, kept tiles
// below the mask-free range, kept tiles below its end, 0, tiles...}.  One
// wave per row; lanes take 64 consecutive tiles at a time and place the kept
// ones by the ballot's prefix count.
__host__ __device__ constexpr int64_t sparse_lut_stride(int64_t n_kt) {
    return 4 + (n_kt + 3) / 4 * 4;
}

template <int BM, int BN>
__global__ __launch_bounds__(64) void sparse_lut_kernel(
    const uint8_t* __restrict__ mask, int S, int causal, int wl, int wr, int n_qt, int n_kb,
    int n_qb, int block_m, int block_n, int sp_stride, int* __restrict__ lut) {
    const int lane = threadIdx.x;
    const int64_t row = blockIdx.x;
    const int64_t hm = row / n_qt;
    const int qt = (int)(row - hm * n_qt);
    const MaskSpec ms{S, causal, wl, wr};
    int64_t a0, a1, b0, b1;
    q_tile_kv_range(ms, qt, BM, BN, &a0, &a1);
    q_tile_interior_range(ms, (int64_t)qt * BM, BM, BN, a0, a1, &b0, &b1);
    const uint8_t* const mrow = mask + (hm * n_qb + (int64_t)qt * BM / block_m) * n_kb;
    int* const out = lut + row * sp_stride;
    int n = 0, r0 = 0, r1 = 0;
    for (int64_t t0 = a0; t0 < a1; t0 += 64) {
        const int64_t t = t0 + lane;
        const bool kept = t < a1 && mrow[t * BN / block_n] != 0;
        const uint64_t m = __ballot(kept);
        const int below = __builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32),
                                                    __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0));
        if (kept) out[4 + n + below] = (int)t;
        n += __popcll(m);
        r0 += __popcll(m & __ballot(t < b0));
        r1 += __popcll(m & __ballot(t < b1));
    }
    if (lane == 0) *reinterpret_cast<int4*>(out) = int4{n, r0, r1, 0};
}

// ---------------------------------------------------------------- part merge
// A row's O and LSE from the partial (O_p, LSE_p) of its K/V parts: with
// M = max_p LSE_p and w_p = exp(LSE_p - M), LSE = M + ln(sum_p w_p) and
// O = sum_p w_p O_p / sum_p w_p -- the online softmax's rescale-and-add
// ([FA] section 1 item 3; [V2] section 二.1 step 2), applied once across the
// parts.  A part with no allowed key has LSE_p = -inf and weight 0.  A NaN LSE
// in any part makes the row NaN, as it would be without the split.
template <typename T> __device__ inline void store4(T* p, f32x4 x);
template <> __device__ inline void store4<float>(float* p, f32x4 x) {
    *reinterpret_cast<f32x4*>(p) = x;
}
template <> __device__ inline void store4<__bf16>(__bf16* p, f32x4 x) {
    *reinterpret_cast<u32x2*>(p) = u32x2{Mfma<__bf16>::pack2(x[0], x[1]), Mfma<__bf16>::pack2(x[2], x[3])};
}
template <> __device__ inline void store4<_Float16>(_Float16* p, f32x4 x) {
    *reinterpret_cast<u32x2*>(p) =
        u32x2{Mfma<_Float16>::pack2(x[0], x[1]), Mfma<_Float16>::pack2(x[2], x[3])};
}

constexpr int kMergeThreads = 256;

template <typename T, int D>
__global__ __launch_bounds__(kMergeThreads) void fa_merge_parts_kernel(
    const float* __restrict__ part_o, const float* __restrict__ part_lse, T* __restrict__ out,
    float* __restrict__ lse, int B, int H, int S, int n_splits, int dv) {
    // D: the padded head dimension (threads per row); dv <= D: the tensors'
    // own, the column count of the partial rows and of O
    constexpr int TPR = D / 4;                  // threads per row, 4 columns each
    constexpr int RPB = kMergeThreads / TPR;    // rows per workgroup
    const int64_t R = (int64_t)B * H * S;       // rows, ordered (b * H + h) * S + s
    const int64_t row = (int64_t)blockIdx.x * RPB + threadIdx.x / TPR;
    const int c4 = threadIdx.x % TPR;
    if (row >= R || 4 * c4 >= dv) return;
    float m = kNegInf;
    bool nan = false;
    for (int p = 0; p < n_splits; ++p) {
        const float l = part_lse[p * R + row];
        nan |= l != l;
        m = fmaxf(m, l);
    }
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
    float wsum = 0.f;
    if (m != kNegInf) {
        for (int p = 0; p < n_splits; ++p) {
            const float l = part_lse[p * R + row];
            const float w = (l == kNegInf) ? 0.f : expf(l - m);
            const f32x4 x = *reinterpret_cast<const f32x4*>(part_o + (p * R + row) * dv + 4 * c4);
            acc += w * x;
            wsum += w;
        }
    }
    const float inv = wsum > 0.f ? 1.f / wsum : 0.f;
    f32x4 o = acc * inv;
    float lv = (m == kNegInf) ? kNegInf : m + logf(wsum);
    if (nan) {
        o = f32x4{__builtin_nanf(""), __builtin_nanf(""), __builtin_nanf(""), __builtin_nanf("")};
        lv = __builtin_nanf("");
    }
    const int64_t bh = row / S, srow = row - bh * S;
    const int64_t b = bh / H, h = bh - b * H;
    store4<T>(out + ((b * S + srow) * H + h) * dv + 4 * c4, o);
    if (c4 == 0) lse[row] = lv;
}

// ---------------------------------------------------------------- fp32
// fp32 inputs run the same transposed-score structure on the fp32 MFMA
// (v_mfma_f32_32x32x2_f32), so every product is an fp32 product; one key
// (or one d) per lane per MFMA means V needs no transposition.
constexpr int kThreads32 = 256;  // 4 waves
constexpr int kBM32 = 4 * kWaveRows;
template <int D> struct Lds32 {
    static constexpr int BN = 32;
    static constexpr int KS = D + 1;
    static constexpr int VS = D + 4;
};

// SPARSE: K/V tiles whose mask byte is 0 are skipped (bmask [sp_heads, n_qb,
// n_kb]; block_m a multiple of the Q tile, block_n of the K/V tile).
// PAGED: k and v are pools [pg_count, pg_rows, H, D] read through the block
// table (pg_rows a multiple of the K/V tile; a page index outside the pool
// reads as zeros).
// PAD: the tensors' head dimension is dv_in < D (a multiple of 16); the
// columns past it are read as zeros and never stored.
template <int D, bool SPARSE, bool PAGED, bool PAD = false>
__global__ __launch_bounds__(kThreads32, 2) void fa_fwd_fp32_kernel(
    const float* __restrict__ q, const float* __restrict__ k, const float* __restrict__ v,
    float* __restrict__ out, float* __restrict__ lse, int B, int H, int S, float c, int causal,
    int wl, int wr, int n_qt, const uint8_t* __restrict__ bmask, int sp_heads, int n_qb, int n_kb,
    int block_m, int block_n, const int* __restrict__ pg_table, int pg_stride, int pg_rows,
    int pg_count, int dv_in) {
    typedef Lds32<D> L;
    const int dv = PAD ? dv_in : D;
    constexpr int BN = L::BN;
    constexpr int DB = D / 32;
    __shared__ float ks[BN * L::KS];
    __shared__ float vs[BN * L::VS];

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int hh = lane >> 5, ql = lane & 31;
    uint32_t bh, qt32;
    workgroup_tile(blockIdx.x, (uint32_t)B * (uint32_t)H, (uint32_t)n_qt, causal != 0,
                   snake_launch((int64_t)B * H, S, D, sizeof(float)), &bh, &qt32);
    const int qt = (int)qt32;
    const int bb = (int)(bh / (uint32_t)H), h = (int)(bh % (uint32_t)H);
    const MaskSpec ms{S, causal, wl, wr};
    int64_t kt0, kt1;
    q_tile_kv_range(ms, qt, kBM32, BN, &kt0, &kt1);
    const int64_t row_stride = (int64_t)H * dv;
    const int64_t head_base = ((int64_t)bb * S * H + h) * dv;
    const int qw0 = qt * kBM32 + wave * kWaveRows;
    const int qrow = qw0 + ql;
    const uint8_t* mrow = nullptr;  // SPARSE: the Q tile's row of the block mask
    if (SPARSE) {
        const int64_t hm = sp_heads == 1 ? 0 : (sp_heads == H ? (int64_t)h : (int64_t)bh);
        mrow = bmask + (hm * n_qb + (int64_t)qt * kBM32 / block_m) * n_kb;
    }

    // Q fragment: lane supplies d = 2*kk + hh of its row
    float qf[D / 2];
    {
        const bool ok = qrow < S;
        const float* qp = q + head_base + (int64_t)(ok ? qrow : 0) * row_stride;
#pragma unroll
        for (int kk = 0; kk < D / 2; ++kk)
            qf[kk] = ok && (!PAD || 2 * kk + hh < dv) ? qp[2 * kk + hh] : 0.f;
    }
    float m_run = kNegInf, l_run = 0.f;
    f32x16 o[DB];
#pragma unroll
    for (int d = 0; d < DB; ++d) o[d] = f32x16{0};

    // K/V tiles go global -> registers -> LDS; the loads of tile kt + 1 are
    // issued right after tile kt is stored, so their latency runs under tile
    // kt's MFMAs.  NLD f32x4 per thread and matrix; the tile's element (r, cc)
    // of load i is id = tid + i * kThreads32.  At D = 128 the registers hold
    // the next K tile only (both would spill): V is loaded when it is stored.
    constexpr int NLD = BN * (D / 4) / kThreads32;
    constexpr bool kAheadV = D <= 64;
    static_assert(NLD * kThreads32 == BN * (D / 4), "the threads split a tile evenly");
    f32x4 xk[NLD], xv[kAheadV ? NLD : 1];
    int64_t fetched_row0 = 0;  // PAGED: pool row of the fetched tile's first key (-1: outside)
    auto tile_ok = [&](int64_t k0, int64_t row0, int i, int& r, int& cc) __attribute__((always_inline)) {
        const int id = tid + i * kThreads32;
        r = id / (D / 4);
        cc = id % (D / 4);
        return k0 + r < S && row0 >= 0 && (!PAD || 4 * cc < dv);
    };
    // element offset of load i of the tile at k0 (a key past S, a page
    // outside the pool or (PAD) a column past dv reads, and discards, element
    // 0 of a valid row)
    auto tile_off = [&](int64_t k0, int64_t row0, int i, bool& ok) __attribute__((always_inline)) {
        int r, cc;
        ok = tile_ok(k0, row0, i, r, cc);
        const int col = !ok ? 0 : cc * 4;
        return PAGED ? ((ok ? row0 + r : 0) * H + h) * dv + col
                     : head_base + (ok ? k0 + r : 0) * row_stride + col;
    };
    auto fetch = [&](int64_t kt) __attribute__((always_inline)) {
        const int64_t k0 = kt * BN;
        int64_t row0 = 0;
        if (PAGED) {
            const int page = pg_table[(int64_t)bb * pg_stride + k0 / pg_rows];
            row0 = (unsigned)page < (unsigned)pg_count ? (int64_t)page * pg_rows + k0 % pg_rows : -1;
        }
        fetched_row0 = row0;
#pragma unroll
        for (int i = 0; i < NLD; ++i) {
            bool ok;
            const int64_t off = tile_off(k0, row0, i, ok);
            xk[i] = *reinterpret_cast<const f32x4*>(k + off);
            if (kAheadV) xv[kAheadV ? i : 0] = *reinterpret_cast<const f32x4*>(v + off);
        }
    };
    if (kt0 < kt1) fetch(kt0);
    for (int64_t kt = kt0; kt < kt1; ++kt) {
        const int64_t k0 = kt * BN;
        // SPARSE: a dropped tile (the same for the whole workgroup) is neither
        // stored nor computed, but the next one is still fetched
        const bool keep = !SPARSE || mrow[k0 / block_n] != 0;
        __syncthreads();  // every wave is done with the previous tile
        if (keep) {
#pragma unroll
            for (int i = 0; i < NLD; ++i) {
                int r, cc;
                const bool ok = tile_ok(k0, fetched_row0, i, r, cc);
                f32x4 x = xv[kAheadV ? i : 0];
                if (!kAheadV) {
                    bool ok2;
                    x = *reinterpret_cast<const f32x4*>(v + tile_off(k0, fetched_row0, i, ok2));
                }
#pragma unroll
                for (int t = 0; t < 4; ++t) {
                    ks[r * L::KS + cc * 4 + t] = ok ? xk[i][t] : 0.f;
                    vs[r * L::VS + cc * 4 + t] = ok ? x[t] : 0.f;
                }
            }
        }
        if (kt + 1 < kt1) fetch(kt + 1);
        __syncthreads();
        if (!keep) continue;
        if (tile_fully_masked(ms, qw0, qw0 + kWaveRows - 1, k0, BN)) continue;
        // S^T (32 keys x 32 queries): A = K row (lane % 32), d = 2*kk + hh
        f32x16 s = f32x16{0};
#pragma unroll
        for (int kk = 0; kk < D / 2; ++kk)
            s = __builtin_amdgcn_mfma_f32_32x32x2f32(ks[ql * L::KS + 2 * kk + hh], qf[kk], s, 0, 0, 0);
        // scaled scores t = c * s (log2 domain); masked keys -> -inf.  Scaling
        // before the max makes the max element's weight exp2(0) = 1 exactly.
        // Register i holds key 8*(i/4) + 4*hh + (i%4).
#pragma unroll
        for (int i = 0; i < 16; ++i) s[i] *= c;
        if (tile_needs_mask(ms, qw0, qw0 + kWaveRows - 1, k0, BN)) {
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                const int key = (int)k0 + 8 * (i >> 2) + 4 * hh + (i & 3);
                bool ok = key < S;
                if (causal) ok = ok && key <= qrow;
                if (wl >= 0) ok = ok && qrow - key <= wl;
                if (wr >= 0) ok = ok && key - qrow <= wr;
                s[i] = ok ? s[i] : kNegInf;
            }
        }
        float mx = kNegInf;
#pragma unroll
        for (int i = 0; i < 16; ++i) mx = fmaxf(mx, s[i]);
        const float m_new = fmaxf(m_run, halves_max(mx));
        const float m_use = (m_new == kNegInf) ? 0.f : m_new;
        const float alpha = __builtin_amdgcn_exp2f(m_run - m_use);
        m_run = m_new;
        float p[16], rs = 0.f;
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            p[i] = __builtin_amdgcn_exp2f(s[i] - m_use);
            rs += p[i];
        }
        l_run = alpha * l_run + rs;
#pragma unroll
        for (int d = 0; d < DB; ++d) o[d] *= alpha;
        // O^T += V^T P^T, one key per wave half per MFMA: register i of half hh
#pragma unroll
        for (int d = 0; d < DB; ++d)
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                const int key = 8 * (i >> 2) + 4 * hh + (i & 3);
                o[d] = __builtin_amdgcn_mfma_f32_32x32x2f32(vs[key * L::VS + 32 * d + ql], p[i], o[d],
                                                            0, 0, 0);
            }
    }
    // l == 0 only for a row with no allowed key; a NaN l (NaN scores) propagates
    const float l_tot = halves_sum(l_run);
    const float inv = (l_tot == 0.f) ? 0.f : 1.f / l_tot;
    const float m_fin = (m_run == kNegInf) ? 0.f : m_run;
    const float lse_v = (l_tot == 0.f) ? kNegInf : 0.69314718055994531f * (m_fin + __log2f(l_tot));
    // a NaN or an infinity in O: this wave recomputes its rows over their
    // allowed keys only (exact_row), stores them and its LSE, and is done
    if (any_nonfinite<DB>(o)) {
        constexpr int DH = D / 2;
        float acc[DH];
        const int64_t kv_base = PAGED ? (int64_t)h * dv : head_base;
        auto tile_of = [&](int pos, int& k0, int64_t& row0, bool& valid) __attribute__((always_inline)) {
            k0 = pos * BN;
            row0 = k0;
            valid = !SPARSE || mrow[k0 / block_n] != 0;  // a dropped tile adds nothing
            if (PAGED) {
                const int page = pg_table[(int64_t)bb * pg_stride + k0 / pg_rows];
                valid = (unsigned)page < (unsigned)pg_count;
                row0 = (int64_t)(valid ? page : 0) * pg_rows + k0 % pg_rows;
            }
        };
        auto allowed = [&](int key) __attribute__((always_inline)) {
            bool ok = key < S;
            if (causal) ok = ok && key <= qrow;
            if (wl >= 0) ok = ok && qrow - key <= wl;
            if (wr >= 0) ok = ok && key - qrow <= wr;
            return ok && (!SPARSE || mrow[key / block_n] != 0);
        };
        const float* q_half = qrow < S ? q + head_base + (int64_t)qrow * row_stride + hh * DH : nullptr;
        float m_x, l_x;
        exact_row<float, D, BN, PAD>(q_half, k + kv_base, v + kv_base, row_stride, hh, dv, S, (int)kt0,
                                (int)kt1, tile_of, allowed, c, m_x, l_x, acc);
        const float lse_x = (l_x == 0.f) ? kNegInf : 0.69314718055994531f * (m_x + __log2f(l_x));
        if (qrow < S) {
            float* eo = out + head_base + (int64_t)qrow * row_stride + hh * DH;
#pragma unroll
            for (int c4 = 0; c4 < DH / 4; ++c4)
                if (!PAD || hh * DH + 4 * c4 < dv)
                    *reinterpret_cast<f32x4*>(eo + 4 * c4) =
                        f32x4{acc[4 * c4], acc[4 * c4 + 1], acc[4 * c4 + 2], acc[4 * c4 + 3]};
            if (hh == 0) lse[((int64_t)bb * H + h) * S + qrow] = lse_x;
        }
        return;
    }
    if (qrow < S) {
        float* op = out + head_base + (int64_t)qrow * row_stride + 4 * hh;
#pragma unroll
        for (int d = 0; d < DB; ++d)
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                f32x4 w = {o[d][4 * g] * inv, o[d][4 * g + 1] * inv, o[d][4 * g + 2] * inv,
                           o[d][4 * g + 3] * inv};
                if (!PAD || 32 * d + 8 * g < dv) *reinterpret_cast<f32x4*>(op + 32 * d + 8 * g) = w;
            }
        if (hh == 0) lse[((int64_t)bb * H + h) * S + qrow] = lse_v;
    }
}

}  // namespace fa
