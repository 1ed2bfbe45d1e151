// fa_fwd_kvcache.hip -- launcher of the forward against a key/value cache
// (decoding: a few new queries per sequence against its cached keys and
// values, per-sequence cache lengths, contiguous or paged caches, optionally
// split over K/V parts with the log-domain merge).  FlashDecoding, the variant
// of the method that serves the KV cache of inference, is named in section 5
// of "FlashAttention技术解析：加速GPT训练的核心优化"; the call
// flash_attn_with_kvcache and the block table of a paged cache in sections
// 总结与最佳实践 and Paged KV Cache支持 of "突破大模型训练瓶颈：Flash-Attention
// 编译优化与内存占用解决方案".  Several queries per sequence run
// fa_fwd_mfma_kernel with KVC = true (fa_fwd_device.h); one query per
// sequence runs fa_decode_kernel below, on the vector ALU.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "fa_fwd_device.h"
#include "fa_fwd_launch_cfg.h"
#include "fa_launch.h"
#include "fa_schedule.h"

namespace fa {

// ---------------------------------------------------------------- one query
// Decoding one token per sequence (S_q = 1) is a matrix-vector product: 2
// flops per cached byte, far below the MFMA's ridge, so the time is the HBM
// stream of K and V.  This kernel runs it on the vector ALU and keeps many
// waves in flight instead: no LDS, a wave per (sequence, head, K/V part).
//  * loads: each 16-byte load instruction covers whole rows -- lane l reads
//    columns 8 * (l % LPK) .. +8 of key KPI * i + l / LPK of the 64-key chunk
//    (LPK = D / 8 lanes per row) -- and K and V use the same offsets, so both
//    tiles of a chunk are in flight together;
//  * scores: each lane takes the dot product of its 8 columns with q (v_dot2,
//    fp32 accumulation) and the LPK lanes of a row add theirs with DPP, so
//    every lane of the row holds the key's score;
//  * online softmax over chunks with a wave-uniform running max; the weight of
//    a key is in the lanes that hold its value columns, so P V is a
//    multiply-add per column, and the lanes holding the same columns are
//    summed once at the end.
// The query sits at position L - 1 (L = the sequence's cache length), so the
// allowed keys are [lo, L), lo = max(0, L - 1 - wl) with a left window, else
// 0: causal or not, no key past the query exists.  Keys outside [lo, L) are
// read through out-of-range buffer offsets, which return zeros, and get no
// weight; no cached value outside them reaches a sum.
template <typename T> struct Dot2;
template <> struct Dot2<__bf16> {
    __device__ static inline float dot(unsigned a, unsigned b, float c) {
        return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, a),
                                               __builtin_bit_cast(bf16x2, b), c, false);
    }
    __device__ static inline void unpack(unsigned w, float& lo, float& hi) {
        lo = __uint_as_float(w << 16);
        hi = __uint_as_float(w & 0xffff0000u);
    }
};
template <> struct Dot2<_Float16> {
    __device__ static inline float dot(unsigned a, unsigned b, float c) {
        return __builtin_amdgcn_fdot2(__builtin_bit_cast(f16x2, a), __builtin_bit_cast(f16x2, b), c,
                                      false);
    }
    __device__ static inline void unpack(unsigned w, float& lo, float& hi) {
        const f16x2 x = __builtin_bit_cast(f16x2, w);
        lo = (float)x[0];
        hi = (float)x[1];
    }
};

// Sum over the N (8 or 16) consecutive lanes of a DPP row group, in every one
// of them: pairs, quads (quad_perm), then half rows and rows (mirrors).
template <int CTRL> __device__ inline float dpp_read(float v) {
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xF, 0xF, false));
}
template <int N> __device__ inline float row_sum(float x) {
    x += dpp_read<0xB1>(x);   // quad_perm [1, 0, 3, 2]: lane ^ 1
    x += dpp_read<0x4E>(x);   // quad_perm [2, 3, 0, 1]: lane ^ 2
    x += dpp_read<0x141>(x);  // row_half_mirror: 7 - lane within 8
    if (N == 16) x += dpp_read<0x140>(x);  // row_mirror: 15 - lane within 16
    return x;
}


template <typename T, int D, int CK, bool PAGED, bool SPLIT>
__global__ __launch_bounds__(64) void fa_decode_kernel(
    const T* __restrict__ q, const T* __restrict__ k, const T* __restrict__ v, T* __restrict__ out,
    float* __restrict__ lse, int B, int H, float c, int wl, const int* __restrict__ kv_lens,
    int kv_cap, int n_splits, float* __restrict__ part_o, float* __restrict__ part_lse,
    const int* __restrict__ pg_table, int pg_stride, int pg_rows, int pg_count) {
    constexpr int LPK = D / 8;    // lanes per row (16 bytes each)
    constexpr int KPI = 64 / LPK; // keys per load instruction
    constexpr int NI = CK / KPI;  // load instructions per chunk of CK keys (each of K and V)
    static_assert(NI * KPI == CK && 64 % CK == 0, "a chunk is whole load rows within 64 keys");
    const int lane = threadIdx.x;
    const int r = lane / LPK, cc = lane % LPK;  // key row within an instruction, column chunk
    // Workgroup w runs on XCD w % 8.  Renumber so that each XCD takes a
    // contiguous range, and within it heads fastest: the heads of one
    // (sequence, part) read neighbouring slices of the same cache rows, on one
    // XCD and through its address translation caches.
    const unsigned n_wg = gridDim.x, w = blockIdx.x;
    const unsigned lw = (n_wg % 8u == 0u) ? (w % 8u) * (n_wg / 8u) + w / 8u : w;
    const int h = (int)(lw % (unsigned)H);
    const int rest = (int)(lw / (unsigned)H);
    const int part = rest % n_splits, bb = rest / n_splits;
    const int bh = bb * H + h;
    int L = __builtin_amdgcn_readfirstlane(kv_lens[bb]);
    L = L < 0 ? 0 : L > kv_cap ? kv_cap : L;
    const int lo = (wl >= 0 && L - 1 - wl > 0) ? L - 1 - wl : 0;
    const int c0 = lo / CK, c1 = (L + CK - 1) / CK;
    const int nch = L > 0 ? c1 - c0 : 0;
    const int p0 = c0 + (int)((int64_t)nch * part / n_splits);
    const int p1 = c0 + (int)((int64_t)nch * (part + 1) / n_splits);
    const int64_t row_stride = (int64_t)H * D;
    const int row_bytes = (int)(row_stride * (int64_t)sizeof(T));

    // this lane's 8 columns of q
    const u32x4 qv = *reinterpret_cast<const u32x4*>(q + ((int64_t)bb * H + h) * D + 8 * cc);

    // A chunk's K and V loads are all issued before any of it is used.  (Two
    // register stages, the next chunk's loads in flight while one is summed,
    // measured slower at the launch sizes below: the HBM stream, not the wait
    // per chunk, is the limit once about two waves per compute unit run.)  A
    // chunk near the end of the sequence has records up to key L - 1 only, an
    // unusable page none.
    const int64_t kv_base = PAGED ? (int64_t)h * D : ((int64_t)bb * kv_cap * H + h) * D;
    struct Stage {
        u32x4 k[NI], v[NI];
    };
    auto issue = [&](Stage& s, int ci) __attribute__((always_inline)) {
        const int k0 = ci * CK;
        int64_t row0 = k0;
        bool ok = true;
        if (PAGED) {
            const int page =
                __builtin_amdgcn_readfirstlane(pg_table[(int64_t)bb * pg_stride + k0 / pg_rows]);
            ok = (unsigned)page < (unsigned)pg_count;
            row0 = (int64_t)(ok ? page : 0) * pg_rows + k0 % pg_rows;
        }
        const int rows = L - k0 < CK ? L - k0 : CK;
        const int nrec = ok ? (int)(((int64_t)(rows - 1) * row_stride + D) * (int64_t)sizeof(T)) : 0;
        const __amdgpu_buffer_rsrc_t rk = __builtin_amdgcn_make_buffer_rsrc(
            (void*)(k + kv_base + row0 * row_stride), (short)0, nrec, kBufferFlags);
        const __amdgpu_buffer_rsrc_t rv = __builtin_amdgcn_make_buffer_rsrc(
            (void*)(v + kv_base + row0 * row_stride), (short)0, nrec, kBufferFlags);
#pragma unroll
        for (int i = 0; i < NI; ++i) {
            const int key = k0 + KPI * i + r;
            // a key outside [lo, L): an offset past every record count (a chunk's
            // records are below 2^31 bytes), so the load returns zeros
            const int off = (key >= lo && key < L) ? (KPI * i + r) * row_bytes + 16 * cc : kDmaPastRecords;
            s.k[i] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rk, off, 0, 0));
            s.v[i] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rv, off, 0, 0));
        }
    };

    float m = kNegInf;   // running max (log2 domain), uniform
    float l_row = 0.f;   // the row sum over this lane's keys (those of row r)
    float acc[8];        // columns 8 * cc .. +8 over this lane's keys
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[e] = 0.f;
    auto consume = [&](const Stage& s, int ci) __attribute__((always_inline)) {
        const int k0 = ci * CK;
        float t[NI];
        float cmax = kNegInf;
#pragma unroll
        for (int i = 0; i < NI; ++i) {
            const int key = k0 + KPI * i + r;
            float d = 0.f;
#pragma unroll
            for (int e = 0; e < 4; ++e) d = Dot2<T>::dot(qv[e], s.k[i][e], d);
            d = row_sum<LPK>(d);
            t[i] = (key >= lo && key < L) ? d * c : kNegInf;
            cmax = fmaxf(cmax, t[i]);
        }
        // max over the wave's rows (each row's lanes hold the same values)
#pragma unroll
        for (int sh = LPK; sh < 64; sh *= 2) cmax = fmaxf(cmax, __shfl_xor(cmax, sh));
        const float mn = fmaxf(m, cmax);
        if (mn > m) {  // wave-uniform: rescale what is accumulated so far
            const float alpha = (m == kNegInf) ? 0.f : __builtin_amdgcn_exp2f(m - mn);
            l_row *= alpha;
#pragma unroll
            for (int e = 0; e < 8; ++e) acc[e] *= alpha;
            m = mn;
        }
#pragma unroll
        for (int i = 0; i < NI; ++i) {
            const float p = __builtin_amdgcn_exp2f(t[i] - m);
            l_row += p;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                float x0, x1;
                Dot2<T>::unpack(s.v[i][e], x0, x1);
                acc[2 * e] = __builtin_fmaf(p, x0, acc[2 * e]);
                acc[2 * e + 1] = __builtin_fmaf(p, x1, acc[2 * e + 1]);
            }
        }
    };
    for (int ci = p0; ci < p1; ++ci) {
        Stage s;
        issue(s, ci);
        consume(s, ci);
    }
    // sum over the rows: the lanes holding the same columns (lane % LPK equal)
    float l = l_row;
#pragma unroll
    for (int sh = LPK; sh < 64; sh *= 2) {
        l += __shfl_xor(l, sh);
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[e] += __shfl_xor(acc[e], sh);
    }
    const float inv = (l == 0.f) ? 0.f : 1.f / l;
    const float lse_v = (l == 0.f) ? kNegInf : 0.69314718055994531f * (m + __log2f(l));
    if (lane < LPK) {
        if (SPLIT) {
            const int64_t prow = (int64_t)part * B * H + bh;
            float* po = part_o + prow * D + 8 * lane;
            *reinterpret_cast<f32x4*>(po) = f32x4{acc[0] * inv, acc[1] * inv, acc[2] * inv, acc[3] * inv};
            *reinterpret_cast<f32x4*>(po + 4) =
                f32x4{acc[4] * inv, acc[5] * inv, acc[6] * inv, acc[7] * inv};
            if (lane == 0) part_lse[prow] = lse_v;
        } else {
            T* o = out + (int64_t)bh * D + 8 * lane;
            *reinterpret_cast<u32x4*>(o) =
                u32x4{Mfma<T>::pack2(acc[0] * inv, acc[1] * inv), Mfma<T>::pack2(acc[2] * inv, acc[3] * inv),
                      Mfma<T>::pack2(acc[4] * inv, acc[5] * inv), Mfma<T>::pack2(acc[6] * inv, acc[7] * inv)};
            if (lane == 0) lse[bh] = lse_v;
        }
    }
}

template <typename T, int D>
static hipError_t launch_decode_cfg(const LaunchArgs& a) {
    const int64_t n_wg = a.B * a.H * a.n_splits;
    const bool paged = a.pg_table != nullptr;
    const int pg_stride = (int)a.pg_stride, pg_rows = paged ? (int)a.pg_rows : 64,
              pg_count = (int)a.pg_count;
#define FA_DECODE_LAUNCH(PG, SP)                                                                   \
    hipLaunchKernelGGL((fa_decode_kernel<T, D, 64, PG, SP>), dim3((unsigned)n_wg), dim3(64), 0,        \
                       a.stream, (const T*)a.q, (const T*)a.k, (const T*)a.v, (T*)a.out, a.lse,     \
                       (int)a.B, (int)a.H, a.c, (int)a.wl, a.kv_lens, (int)a.kv_cap, a.n_splits,   \
                       a.part_o, a.part_lse, a.pg_table, pg_stride, pg_rows, pg_count)
    if (a.n_splits <= 1) {
        if (paged)
            FA_DECODE_LAUNCH(true, false);
        else
            FA_DECODE_LAUNCH(false, false);
        return hipGetLastError();
    }
    if (paged)
        FA_DECODE_LAUNCH(true, true);
    else
        FA_DECODE_LAUNCH(false, true);
#undef FA_DECODE_LAUNCH
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    return launch_merge_parts(a);
}

template <typename T, int D>
static hipError_t launch_kvcache_cfg(const LaunchArgs& a) {
    if (a.S == 1) return launch_decode_cfg<T, D>(a);  // one query per sequence
    return launch_kvc_mfma_cfg<T, D, false>(a);
}

hipError_t launch_kvcache(const LaunchArgs& a) {
    // a head dimension other than 64 and 128 (a multiple of 16 up to 128):
    // the MFMA kernel of the next of them with PAD (fa_fwd_kvcache_padded.hip), also
    // for one query per sequence
    if (a.D != 64 && a.D != 128) return launch_kvcache_padded(a);
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
int kvcache_auto_splits(int64_t B, int64_t H, int64_t S_q, int64_t S_k, int64_t D, int dtype) {
    (void)dtype;
    int dev = 0, cus = 0;
    if (hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) {
        (void)hipGetLastError();
        return 1;
    }
    const int64_t kv_tiles = (S_k + kMfmaKeys - 1) / kMfmaKeys;
    if (S_q == 1 && (D == 64 || D == 128)) {
        // the one-query kernel: a wave per (sequence, head, part).  Its HBM
        // stream peaks at about two waves per compute unit (more waves, each
        // on a shorter range, measured slower), each with at least 4 chunks
        // of 64 keys of a full cache
        const int64_t rows = B * H;
        int64_t ns = (2 * (int64_t)cus + rows - 1) / rows;
        if (ns > kv_tiles / 4) ns = kv_tiles / 4;
        if (ns > kMaxKvSplits) ns = kMaxKvSplits;
        return ns < 1 ? 1 : (int)ns;
    }
    constexpr int BM = kMfmaWaves * kWaveRows;
    const int64_t tiles = B * H * ((S_q + BM - 1) / BM);
    if (tiles >= 2 * (int64_t)cus) return 1;
    int64_t ns = (4 * (int64_t)cus + tiles - 1) / tiles;
    if (ns > kv_tiles / 4) ns = kv_tiles / 4;
    if (ns > kMaxKvSplits) ns = kMaxKvSplits;
    return ns < 1 ? 1 : (int)ns;
}

}  // namespace fa
