// fa_bwd_device.h -- gfx950 (CDNA4) kernels of the exact-attention backward
// pass: dQ, dK and dV for an output gradient dO, recomputed tile by tile from
// the forward's saved log-sum-exp, and their launch.  The building blocks (LDS
// tile geometry and swizzle, direct-to-LDS loads, the MFMA traits and the
// score key map) are the forward's, from fa_kernel_common.h.  Included by
// fa_bwd_kernels.hip (head dimensions 64 and 128) and fa_bwd_padded.hip (the
// other multiples of 16 up to 128: PAD = true, the next kernel up with zero
// columns, as in the forward).  Not part of the public ABI.
//
// Pages cited by title:
//   [V2] "大模型加速新突破：Flash Attention V2核心网络算子解析"
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "fa_kernel_common.h"
#include "fa_launch.h"
#include "fa_schedule.h"

namespace fa {

// ================================================================ backward
// Gradients of the exact forward for an output gradient dO, recomputed from
// the saved LSE instead of a stored S x S matrix ("大模型加速新突破：Flash
// Attention V2核心网络算子解析" section 二.1 step 3: the backward pass reuses
// what the forward saved):
//   P = exp(scale * S - LSE)    dP = dO V^T    D_i = sum_d dO_id O_id
//   dS = P * (dP - D)           dQ = scale * dS K
//   dK = scale * dS^T Q         dV = P^T dO
// Three launches: the row dots D; dQ with each workgroup owning a Q tile (the
// forward's layout, lane = query row); dK and dV with each workgroup owning
// 128 keys (lane = key), streaming Q, dO and the row statistics through LDS.
// P and dS are rounded to the input dtype for the MFMA, as P is in the
// forward; every accumulation is fp32.
constexpr float kLog2e = 1.4426950408889634f;

template <typename T> __device__ inline void unpack2(unsigned x, float& a, float& b);
template <> __device__ inline void unpack2<__bf16>(unsigned x, float& a, float& b) {
    a = __uint_as_float(x << 16);
    b = __uint_as_float(x & 0xffff0000u);
}
template <> __device__ inline void unpack2<_Float16>(unsigned x, float& a, float& b) {
    const f16x2 h = __builtin_bit_cast(f16x2, x);
    a = (float)h[0];
    b = (float)h[1];
}

// D_i = dO_i . O_i in fp32, [B, H, S]; one thread per row.  PAD: the
// tensors' head dimension is dv_in < D (a multiple of 16); otherwise D.  Also
// zeroes the two dynamic-order counters of the passes that follow.
template <typename T, int D, bool PAD>
__global__ __launch_bounds__(256) void fa_bwd_rowdot_kernel(const T* __restrict__ out,
                                                            const T* __restrict__ dout,
                                                            float* __restrict__ di, int B, int H,
                                                            int S, int dv_in,
                                                            unsigned* __restrict__ counters) {
    if (blockIdx.x == 0 && threadIdx.x < 2) counters[threadIdx.x] = 0u;
    const int dv = PAD ? dv_in : D;
    const int64_t R = (int64_t)B * H * S;
    const int64_t row = (int64_t)blockIdx.x * 256 + threadIdx.x;  // (b * H + h) * S + s
    if (row >= R) return;
    const int64_t bh = row / S, s = row - bh * S, b = bh / H, h = bh - b * H;
    const int64_t base = ((b * S + s) * H + h) * dv;
    float acc = 0.f;
#pragma unroll
    for (int d = 0; d < D; d += 8) {
        if (PAD && d >= dv) break;
        const u32x4 o = *reinterpret_cast<const u32x4*>(out + base + d);
        const u32x4 g = *reinterpret_cast<const u32x4*>(dout + base + d);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            float o0, o1, g0, g1;
            unpack2<T>(o[e], o0, o1);
            unpack2<T>(g[e], g0, g1);
            acc = __builtin_fmaf(o0, g0, acc);
            acc = __builtin_fmaf(o1, g1, acc);
        }
    }
    di[row] = acc;
}

// lse * log2(e) of a row (+inf for a row with no allowed key, so that every
// weight exp2(c s - L) of it is 0)
__device__ inline float log2_lse(float l) { return l == kNegInf ? __builtin_inff() : l * kLog2e; }

// ---- dQ: workgroup = 128 query rows (4 waves x 32), K/V tiles of 64 keys.
// Per tile: S^T = K Q^T and dP^T = V dO^T on the score MFMA (lane = query
// row, as in the forward), dS = P (dP - D) in registers, dQ^T += K^T dS^T on
// the P V MFMA with K read through the transposing LDS read.  PAD: the
// tensors' head dimension is dv_in < D; the columns past it are read as zeros
// (fragments zeroed, tile chunks loaded from past the records, with the
// forward's kDmaBias) and never stored.
template <typename T, int D, bool PAD>
__global__ __launch_bounds__(256, 1) void fa_bwd_dq_kernel(
    const T* __restrict__ q, const T* __restrict__ k, const T* __restrict__ v,
    const T* __restrict__ dout, const float* __restrict__ lse, const float* __restrict__ di,
    T* __restrict__ dq, int B, int H, int S, float c, float scale, int causal, int wl, int wr,
    int n_qt, int dv_in, unsigned* __restrict__ counter, int dyn_first) {
    const int dv = PAD ? dv_in : D;
    constexpr int kBias = PAD ? kDmaBias : 0;
    typedef Tile<D, 4, 64> L;
    constexpr int BN = L::BN, BM = L::BM, KB = L::KB, NCH = L::NCH, RB = L::RB;
    constexpr int KSTEPS = D / 16, DB = D / 32;
    __shared__ __attribute__((aligned(1024))) unsigned char lds_k0[L::MAT];
    __shared__ __attribute__((aligned(1024))) unsigned char lds_k1[L::MAT];
    __shared__ __attribute__((aligned(1024))) unsigned char lds_v0[L::MAT];
    __shared__ __attribute__((aligned(1024))) unsigned char lds_v1[L::MAT];
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int hh = lane >> 5, ql = lane & 31;

    uint32_t bh, qt32;
    if (dyn_first >= 0)  // the forward's dynamic tail (dyn_first_position)
        dynamic_tile(blockIdx.x, (uint32_t)B * (uint32_t)H, (uint32_t)n_qt, dyn_first,
                     snake_launch((int64_t)B * H, S, D, sizeof(T)), counter, &bh, &qt32);
    else
        workgroup_tile(blockIdx.x, (uint32_t)B * (uint32_t)H, (uint32_t)n_qt, causal != 0,
                       snake_launch((int64_t)B * H, S, D, sizeof(T)), &bh, &qt32);
    const int qt = (int)qt32;
    const int bb = (int)(bh / (uint32_t)H), h = (int)(bh % (uint32_t)H);
    const MaskSpec ms{S, causal, wl, wr};
    int kt0, kt1, ki0, ki1;
    {
        int64_t a0, a1, b0, b1;
        q_tile_kv_range(ms, qt, BM, BN, &a0, &a1);
        q_tile_interior_range(ms, (int64_t)qt * BM, BM, BN, a0, a1, &b0, &b1);
        kt0 = (int)a0;
        kt1 = (int)a1;
        ki0 = (int)b0;
        ki1 = (int)b1;
    }
    const int64_t row_stride = (int64_t)H * dv;
    const int64_t head_base = ((int64_t)bb * S * H + h) * dv;
    const int qw0 = qt * BM + wave * kWaveRows, qrow = qw0 + ql;
    int key_lo = 0, key_w = S - 1;
    if (qrow < S) {
        int64_t lo = 0, hi = S - 1;
        if (wl >= 0) lo = (int64_t)qrow - wl > 0 ? (int64_t)qrow - wl : 0;
        if (causal && qrow < hi) hi = qrow;
        if (wr >= 0 && (int64_t)qrow + wr < hi) hi = (int64_t)qrow + wr;
        key_lo = (int)lo;
        key_w = (int)(hi - lo);
    }
    auto rows_rsrc = [&](const T* base, int64_t r0) __attribute__((always_inline)) {
        const T* p = base + head_base + r0 * row_stride;
        const int64_t bytes = ((S - r0 - 1) * row_stride + dv) * (int64_t)sizeof(T);
        const int64_t nrec = bytes > 0xFFFFFFFFll ? 0xFFFFFFFFll : bytes;
        return __builtin_amdgcn_make_buffer_rsrc((void*)p, (short)0, (int)(uint32_t)nrec,
                                                 kBufferFlags);
    };
    // Q and dO fragments of this lane's row (B operands)
    u32x4 qf[KSTEPS], gf[KSTEPS];
    {
        const __amdgpu_buffer_rsrc_t rq = rows_rsrc(q, qw0 < S ? qw0 : S - 1);
        const __amdgpu_buffer_rsrc_t rg = rows_rsrc(dout, qw0 < S ? qw0 : S - 1);
        const int voff = (ql * (int)row_stride + 8 * hh) * (int)sizeof(T);
#pragma unroll
        for (int ks = 0; ks < KSTEPS; ++ks) {
            const bool col = !PAD || 16 * ks + 8 * hh < dv;  // columns past dv: zeros
            const int o = col ? voff + 32 * ks : voff;
            qf[ks] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rq, o, 0, 0));
            gf[ks] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rg, o, 0, 0));
            if (!col) qf[ks] = gf[ks] = u32x4{0, 0, 0, 0};
        }
        if (qw0 >= S) {
#pragma unroll
            for (int ks = 0; ks < KSTEPS; ++ks) qf[ks] = gf[ks] = u32x4{0, 0, 0, 0};
        }
    }
    float Lr = __builtin_inff(), Dr = 0.f;  // padding rows: weights 0
    if (qrow < S) {
        Lr = log2_lse(lse[(int64_t)bh * S + qrow]);
        Dr = di[(int64_t)bh * S + qrow];
    }
    int dma_voff[L::DMA_PER_WAVE];
#pragma unroll
    for (int j = 0; j < L::DMA_PER_WAVE; ++j) {
        const int byte = (wave * L::DMA_PER_WAVE + j) * 1024 + 16 * lane;
        const int r = byte / RB, pc = (byte % RB) / 16;
        const int lc = pc ^ L::swz(r);  // the logical chunk stored there
        dma_voff[j] = (!PAD || 8 * lc < dv)
                          ? r * (int)row_stride * (int)sizeof(T) + 16 * lc + kBias - 1024 * j
                          : kDmaPastRecords;
    }
    const uint32_t tile_bytes = (uint32_t)(BN * row_stride * (int64_t)sizeof(T));
    const uint64_t head_bytes = (uint64_t)(((int64_t)S - 1) * row_stride + dv) * sizeof(T);
    // records cover the tile up to the head's end (32-bit scalar compares):
    // tiles below the last lie inside the head, the last ends at its end, and
    // a tile at or past S gets none (its reads return zeros)
    const int n_t = (S + BN - 1) / BN;
    const uint32_t last_bytes = (uint32_t)(head_bytes - (uint64_t)(uint32_t)(n_t - 1) * tile_bytes);
    auto tile_rsrc = [&](const T* base, int kt) __attribute__((always_inline)) {
        const unsigned char* head = (const unsigned char*)(base + head_base) - kBias;
        const uint64_t off = (uint64_t)(uint32_t)kt * tile_bytes;
        const uint32_t nrec = kt < n_t - 1    ? tile_bytes + kBias
                              : kt == n_t - 1 ? last_bytes + kBias
                                              : (uint32_t)kBias;
        return __builtin_amdgcn_make_buffer_rsrc((void*)(head + off), (short)0, (int)nrec,
                                                 kBufferFlags);
    };
    auto load = [&](const T* base, int kt, unsigned char* buf) __attribute__((always_inline)) {
        dma_matrix<L::DMA_PER_WAVE>(tile_rsrc(base, kt), buf + wave * L::DMA_PER_WAVE * 1024, dma_voff);
    };
    int kaddr[KSTEPS];
    {
        const int krow = k_row_for_mfma_row(ql);
        const int kbase = krow * RB + 16 * (hh ^ L::swz(krow));
#pragma unroll
        for (int kk = 0; kk < KSTEPS; ++kk) kaddr[kk] = kbase ^ (32 * kk);
    }
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
    // S^T (or dP^T) of one tile: rows of `tile` against the fragment f
    // (block by block: the weights of block 0 can start while block 1 is
    // still on the matrix core)
    auto scores = [&](f32x16(&s)[KB], const unsigned char* tile, const u32x4(&f)[KSTEPS]) __attribute__((always_inline)) {
#pragma unroll
        for (int kb = 0; kb < KB; ++kb)
#pragma unroll
            for (int kk = 0; kk < KSTEPS; ++kk) {
                const u32x4 a = *reinterpret_cast<const u32x4*>(tile + 32 * kb * RB + kaddr[kk]);
                s[kb] = Mfma<T>::mma(a, f[kk], kk == 0 ? f32x16{0} : s[kb]);
            }
    };
    // acc^T += tile^T x^T, the tile read transposed (x: 16 keys per chunk)
    auto tmul = [&](f32x16(&acc)[DB], const u32x4(&x)[NCH], const unsigned char* tile) __attribute__((always_inline)) {
#pragma unroll
        for (int cch = 0; cch < NCH; ++cch)
#pragma unroll
            for (int d = 0; d < DB; ++d) {
                const unsigned char* tp = tile + 16 * cch * RB;
                const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((FA_LDS i16x4*)(tp + vaddr[0][d]));
                const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((FA_LDS i16x4*)(tp + vaddr[1][d]));
                const u32x2 l2 = __builtin_bit_cast(u32x2, lo), h2 = __builtin_bit_cast(u32x2, hi);
                acc[d] = Mfma<T>::mma(u32x4{l2[0], l2[1], h2[0], h2[1]}, x[cch], acc[d]);
            }
    };
    f32x16 acc[DB];
#pragma unroll
    for (int d = 0; d < DB; ++d) acc[d] = f32x16{0};

    load(k, kt0, lds_k0);
    load(v, kt0, lds_v0);
    // one tile; MASK: it lies outside the mask-free run [ki0, ki1) and takes the mask
    auto step = [&](int j, auto mask_tag) __attribute__((always_inline)) {
        constexpr bool MASK = decltype(mask_tag)::value;
        const bool st = ((j - kt0) & 1) != 0;
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        __syncthreads();  // tile j has landed; every wave is done with tile j-1
        if (j + 1 < kt1) {
            load(k, j + 1, st ? lds_k0 : lds_k1);
            load(v, j + 1, st ? lds_v0 : lds_v1);
        }
        const unsigned char* kst = st ? lds_k1 : lds_k0;
        const unsigned char* vst = st ? lds_v1 : lds_v0;
        f32x16 s[KB], dp[KB];
        scores(s, kst, qf);
        scores(dp, vst, gf);
        if (MASK) {
            const int a = j * BN + 8 * hh - key_lo;
#pragma unroll
            for (int kb = 0; kb < KB; ++kb)
#pragma unroll
                for (int i = 0; i < 16; ++i) {
                    const bool ok = (unsigned)(a + 32 * kb + score_key_base(i)) <= (unsigned)key_w;
                    s[kb][i] = ok ? s[kb][i] : kNegInf;
                }
        }
        u32x4 ds[NCH];
#pragma unroll
        for (int e = 0; e < 16 * KB; e += 2) {
            const int kb = e >> 4, i = e & 15;
            const float p0 = __builtin_amdgcn_exp2f(__builtin_fmaf(s[kb][i], c, -Lr));
            const float p1 = __builtin_amdgcn_exp2f(__builtin_fmaf(s[kb][i + 1], c, -Lr));
            ds[e >> 3][(e & 7) >> 1] = Mfma<T>::pack2(p0 * (dp[kb][i] - Dr), p1 * (dp[kb][i + 1] - Dr));
        }
        tmul(acc, ds, kst);
    };
    // the masked tiles before and after the mask-free run get a loop of their
    // own, so no branch splits the mask-free step's MFMA / VALU schedule
    {
        int j = kt0;
        for (; j < ki0; ++j) step(j, BoolTag<true>{});
        for (; j < ki1; ++j) step(j, BoolTag<false>{});
        for (; j < kt1; ++j) step(j, BoolTag<true>{});
    }
    if (qrow < S) {
        T* op = dq + head_base + (int64_t)qrow * row_stride + 4 * hh;
#pragma unroll
        for (int d = 0; d < DB; ++d)
#pragma unroll
            for (int g = 0; g < 4; ++g)
                if (!PAD || 32 * d + 8 * g < dv)
                    *reinterpret_cast<u32x2*>(op + 32 * d + 8 * g) =
                        u32x2{Mfma<T>::pack2(acc[d][4 * g] * scale, acc[d][4 * g + 1] * scale),
                              Mfma<T>::pack2(acc[d][4 * g + 2] * scale, acc[d][4 * g + 3] * scale)};
    }
}

// ---- dK, dV: workgroup = 128 keys (4 waves x 32, lane = key), Q tiles of
// bwd_rows(D) rows streamed with dO and their LSE / D values.  Per 32-row half
// of a Q tile: S = Q K^T and
// dP = dO V^T on the score MFMA with the K and V fragments of the lane's key
// as B operands (the rows of the Q / dO tile are fed in the permuted order
// that leaves each lane 8 consecutive rows per 16-row chunk), P = exp2(c S -
// L) and dS = P (dP - D) in registers, then dV^T += dO^T P and dK^T += Q^T dS
// on the P V MFMA with the tiles read through the transposing LDS read.
// Two workgroups share a CU, so one wave's exp / dS work runs beside the
// other's MFMAs.  D = 64 fits that with both fragments in registers and
// 64-row tiles.  D = 128 does not fit 256 registers with both fragments, both
// accumulators and the rows' L and D, so there the V fragment is parked in
// LDS (each lane reads back its own 16 bytes per d chunk, conflict-free), L
// and D are read from LDS when used, and the Q / dO tiles are 32 rows, which
// leaves room for two workgroups' LDS in a CU (measured: the kernel 20%
// faster than at one workgroup per CU with everything in registers; the
// same changes at D = 64 cost 3%).
constexpr int kBwdKeys = 128;  // keys per dK / dV workgroup
__host__ __device__ constexpr int bwd_rows(int d) { return d == 128 ? 32 : 64; }
__host__ __device__ constexpr bool bwd_vf_in_lds(int d) { return d == 128; }
__host__ __device__ constexpr bool bwd_stats_when_used(int d) { return d == 128; }

template <typename T, int D, bool PAD>
__global__ __launch_bounds__(256, D == 128 ? 2 : 1) void fa_bwd_dkdv_kernel(
    const T* __restrict__ q, const T* __restrict__ k, const T* __restrict__ v,
    const T* __restrict__ dout, const float* __restrict__ lse, const float* __restrict__ di,
    T* __restrict__ dk, T* __restrict__ dv, int B, int H, int S, float c, float scale, int causal,
    int wl, int wr, int n_kt, int dv_in, unsigned* __restrict__ counter, int dyn_first) {
    // PAD: the tensors' head dimension is ncol = dv_in < D, as in the dQ kernel
    const int ncol = PAD ? dv_in : D;
    constexpr int kBias = PAD ? kDmaBias : 0;
    typedef Tile<D, 4, bwd_rows(D)> L;  // here: Q / dO tiles of bwd_rows(D) rows
    constexpr int BQ = L::BN, RB = L::RB, NCH = L::NCH;
    constexpr int KSTEPS = D / 16, DB = D / 32;
    constexpr bool VF_LDS = bwd_vf_in_lds(D);
    __shared__ __attribute__((aligned(1024))) unsigned char lds_q0[L::MAT];
    __shared__ __attribute__((aligned(1024))) unsigned char lds_q1[L::MAT];
    __shared__ __attribute__((aligned(1024))) unsigned char lds_g0[L::MAT];
    __shared__ __attribute__((aligned(1024))) unsigned char lds_g1[L::MAT];
    __shared__ __attribute__((aligned(16))) float lds_l[2][BQ];  // log2-domain LSE per row
    __shared__ __attribute__((aligned(16))) float lds_d[2][BQ];  // D per row
    // VF_LDS: V fragments [wave][d chunk][lane]
    __shared__ __attribute__((aligned(16))) u32x4 lds_vf[4][VF_LDS ? KSTEPS : 1][64];
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int hh = lane >> 5, ql = lane & 31;

    // key blocks: with the causal mask block 0 sees every row, so the lowest
    // blocks (the heaviest) run first
    // (the dynamic tail, dyn_first_key_blocks: rank r = key block r)
    uint32_t bh, t32;
    if (dyn_first >= 0)
        dynamic_tile(blockIdx.x, (uint32_t)B * (uint32_t)H, (uint32_t)n_kt, dyn_first,
                     snake_launch((int64_t)B * H, S, D, sizeof(T)), counter, &bh, &t32);
    else
        workgroup_tile(blockIdx.x, (uint32_t)B * (uint32_t)H, (uint32_t)n_kt, causal != 0,
                       snake_launch((int64_t)B * H, S, D, sizeof(T)), &bh, &t32);
    const int kblk = causal ? n_kt - 1 - (int)t32 : (int)t32;
    const int bb = (int)(bh / (uint32_t)H), h = (int)(bh % (uint32_t)H);
    const int64_t row_stride = (int64_t)H * ncol;
    const int64_t head_base = ((int64_t)bb * S * H + h) * ncol;
    const int j0 = kblk * kBwdKeys;
    const int j1 = j0 + kBwdKeys - 1 < S - 1 ? j0 + kBwdKeys - 1 : S - 1;
    const int kw0 = j0 + wave * kWaveRows;  // first key of this wave
    const int key = kw0 + ql;               // this lane's key
    // rows with an allowed key in [j0, j1]: [qlo, qhi]
    int64_t qlo = causal ? j0 : 0, qhi = S - 1;
    if (wr >= 0 && (int64_t)j0 - wr > qlo) qlo = (int64_t)j0 - wr;
    if (wl >= 0 && (int64_t)j1 + wl < qhi) qhi = (int64_t)j1 + wl;
    const int t0 = (int)(qlo / BQ), t1 = (int)(qhi / BQ) + 1;
    const MaskSpec ms{S, causal, wl, wr};

    auto rows_rsrc = [&](const T* base, int64_t r0) __attribute__((always_inline)) {
        const T* p = base + head_base + r0 * row_stride;
        const int64_t bytes = ((S - r0 - 1) * row_stride + ncol) * (int64_t)sizeof(T);
        const int64_t nrec = bytes > 0xFFFFFFFFll ? 0xFFFFFFFFll : bytes;
        return __builtin_amdgcn_make_buffer_rsrc((void*)p, (short)0, (int)(uint32_t)nrec,
                                                 kBufferFlags);
    };
    // K and V fragments of this lane's key (B operands; VF_LDS: the V fragment
    // parked in LDS for this lane alone); keys past S read 0
    u32x4 kf[KSTEPS], vf[VF_LDS ? 1 : KSTEPS];
    u32x4(&vfl)[VF_LDS ? KSTEPS : 1][64] = lds_vf[wave];
    {
        const __amdgpu_buffer_rsrc_t rk = rows_rsrc(k, kw0 < S ? kw0 : S - 1);
        const __amdgpu_buffer_rsrc_t rv = rows_rsrc(v, kw0 < S ? kw0 : S - 1);
        const int voff = (ql * (int)row_stride + 8 * hh) * (int)sizeof(T);
#pragma unroll
        for (int ks = 0; ks < KSTEPS; ++ks) {
            const bool col = !PAD || 16 * ks + 8 * hh < ncol;  // columns past ncol: zeros
            const int o = col ? voff + 32 * ks : voff;
            kf[ks] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rk, o, 0, 0));
            u32x4 vx = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rv, o, 0, 0));
            if (!col) kf[ks] = u32x4{0, 0, 0, 0};
            if (kw0 >= S || !col) vx = u32x4{0, 0, 0, 0};
            if (VF_LDS)
                vfl[VF_LDS ? ks : 0][lane] = vx;
            else
                vf[VF_LDS ? 0 : ks] = vx;
        }
        if (kw0 >= S) {
#pragma unroll
            for (int ks = 0; ks < KSTEPS; ++ks) kf[ks] = u32x4{0, 0, 0, 0};
        }
    }
    int dma_voff[L::DMA_PER_WAVE];
#pragma unroll
    for (int j = 0; j < L::DMA_PER_WAVE; ++j) {
        const int byte = (wave * L::DMA_PER_WAVE + j) * 1024 + 16 * lane;
        const int r = byte / RB, pc = (byte % RB) / 16;
        const int lc = pc ^ L::swz(r);  // the logical chunk stored there
        dma_voff[j] = (!PAD || 8 * lc < ncol)
                          ? r * (int)row_stride * (int)sizeof(T) + 16 * lc + kBias - 1024 * j
                          : kDmaPastRecords;
    }
    const uint32_t tile_bytes = (uint32_t)(BQ * row_stride * (int64_t)sizeof(T));
    const uint64_t head_bytes = (uint64_t)(((int64_t)S - 1) * row_stride + ncol) * sizeof(T);
    // records cover the tile up to the head's end, as in the dQ kernel
    const int n_t = (S + BQ - 1) / BQ;
    const uint32_t last_bytes = (uint32_t)(head_bytes - (uint64_t)(uint32_t)(n_t - 1) * tile_bytes);
    auto load = [&](const T* base, int t, unsigned char* buf) __attribute__((always_inline)) {
        const unsigned char* head = (const unsigned char*)(base + head_base) - kBias;
        const uint64_t off = (uint64_t)(uint32_t)t * tile_bytes;
        const uint32_t nrec = t < n_t - 1    ? tile_bytes + kBias
                              : t == n_t - 1 ? last_bytes + kBias
                                             : (uint32_t)kBias;
        dma_matrix<L::DMA_PER_WAVE>(
            __builtin_amdgcn_make_buffer_rsrc((void*)(head + off), (short)0, (int)nrec, kBufferFlags),
            buf + wave * L::DMA_PER_WAVE * 1024, dma_voff);
    };
    // row statistics of Q tile t: threads 0..BQ-1 fetch L, BQ..2BQ-1 fetch D
    const float* lse_h = lse + (int64_t)bh * S;
    const float* di_h = di + (int64_t)bh * S;
    auto fetch_stats = [&](int t) __attribute__((always_inline)) {
        const int r = t * BQ + (tid % BQ);
        float x = tid < BQ ? __builtin_inff() : 0.f;  // rows past S: weights 0
        if (tid < 2 * BQ && r < S) x = tid < BQ ? log2_lse(lse_h[r]) : di_h[r];
        return x;
    };
    auto store_stats = [&](int stage, float x) __attribute__((always_inline)) {
        if (tid < BQ) lds_l[stage][tid] = x;
        else if (tid < 2 * BQ) lds_d[stage][tid - BQ] = x;
    };
    int kaddr[KSTEPS];
    {
        const int krow = k_row_for_mfma_row(ql);
        const int kbase = krow * RB + 16 * (hh ^ L::swz(krow));
#pragma unroll
        for (int kk = 0; kk < KSTEPS; ++kk) kaddr[kk] = kbase ^ (32 * kk);
    }
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
    // the 32 rows of half kb of `tile` against the K fragment (lane = key), or,
    // FROM_LDS, against the V fragment (parked in LDS when VF_LDS)
    auto scores = [&](f32x16& s, const unsigned char* tile, int kb, auto from_lds_tag) __attribute__((always_inline)) {
        constexpr bool FROM_LDS = decltype(from_lds_tag)::value;
#pragma unroll
        for (int kk = 0; kk < KSTEPS; ++kk) {
            const u32x4 a = *reinterpret_cast<const u32x4*>(tile + 32 * kb * RB + kaddr[kk]);
            const u32x4 b = !FROM_LDS ? kf[kk] : VF_LDS ? vfl[VF_LDS ? kk : 0][lane] : vf[VF_LDS ? 0 : kk];
            s = Mfma<T>::mma(a, b, kk == 0 ? f32x16{0} : s);
        }
    };
    // acc^T += tile^T x over the two 16-row chunks of half kb
    auto tmul = [&](f32x16(&acc)[DB], const u32x4(&x)[2], const unsigned char* tile, int kb) __attribute__((always_inline)) {
#pragma unroll
        for (int c2 = 0; c2 < 2; ++c2)
#pragma unroll
            for (int d = 0; d < DB; ++d) {
                const unsigned char* tp = tile + 16 * (2 * kb + c2) * RB;
                const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((FA_LDS i16x4*)(tp + vaddr[0][d]));
                const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((FA_LDS i16x4*)(tp + vaddr[1][d]));
                const u32x2 l2 = __builtin_bit_cast(u32x2, lo), h2 = __builtin_bit_cast(u32x2, hi);
                acc[d] = Mfma<T>::mma(u32x4{l2[0], l2[1], h2[0], h2[1]}, x[c2], acc[d]);
            }
    };
    f32x16 acc_k[DB], acc_v[DB];
#pragma unroll
    for (int d = 0; d < DB; ++d) acc_k[d] = acc_v[d] = f32x16{0};
    static_assert(NCH == 2 * (BQ / 32), "32-row halves of two 16-row chunks");

    load(q, t0, lds_q0);
    load(dout, t0, lds_g0);
    store_stats(0, fetch_stats(t0));
    for (int t = t0; t < t1; ++t) {
        const int st = (t - t0) & 1;
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        __syncthreads();  // tile t and its statistics are in; tile t-1 is done
        float nx = 0.f;
        if (t + 1 < t1) {
            load(q, t + 1, st ? lds_q0 : lds_q1);
            load(dout, t + 1, st ? lds_g0 : lds_g1);
            nx = fetch_stats(t + 1);
        }
        const unsigned char* qst = st ? lds_q1 : lds_q0;
        const unsigned char* gst = st ? lds_g1 : lds_g0;
        const int r0 = t * BQ;
        const bool masked = r0 + BQ - 1 >= S ||
                            tile_needs_mask(ms, r0, r0 + BQ - 1, j0, kBwdKeys);
#pragma unroll
        for (int kb = 0; kb < BQ / 32; ++kb) {
            f32x16 s, dp;
            scores(s, qst, kb, BoolTag<false>{});
            scores(dp, gst, kb, BoolTag<true>{});
            if (masked) {
#pragma unroll
                for (int i = 0; i < 16; ++i) {
                    const int row = r0 + 32 * kb + score_key_base(i) + 8 * hh;
                    bool ok = row < S && key < S;
                    if (causal && key > row) ok = false;
                    if (wl >= 0 && row - key > wl) ok = false;
                    if (wr >= 0 && key - row > wr) ok = false;
                    s[i] = ok ? s[i] : kNegInf;
                }
            }
            // L and D of the rows in registers 4g .. 4g+3: rows 32 kb + 16 (g/2)
            // + 8 hh + 4 (g%2) + 0..3 (read all up front, or each group when used)
            auto stats = [&](int g, f32x4& l4, f32x4& d4) __attribute__((always_inline)) {
                const int r = 32 * kb + 16 * (g >> 1) + 8 * hh + 4 * (g & 1);
                l4 = *reinterpret_cast<const f32x4*>(&lds_l[st][r]);
                d4 = *reinterpret_cast<const f32x4*>(&lds_d[st][r]);
            };
            f32x4 lpre[4], dpre[4];
            if (!bwd_stats_when_used(D)) {
#pragma unroll
                for (int g = 0; g < 4; ++g) stats(g, lpre[g], dpre[g]);
            }
            u32x4 pp[2], ds[2];
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                f32x4 l4, d4;
                if (bwd_stats_when_used(D)) {
                    stats(g, l4, d4);
                } else {
                    l4 = lpre[g];
                    d4 = dpre[g];
                }
#pragma unroll
                for (int e = 0; e < 4; e += 2) {
                    const int i = 4 * g + e;
                    const float p0 = __builtin_amdgcn_exp2f(__builtin_fmaf(s[i], c, -l4[e]));
                    const float p1 = __builtin_amdgcn_exp2f(__builtin_fmaf(s[i + 1], c, -l4[e + 1]));
                    pp[i >> 3][(i & 7) >> 1] = Mfma<T>::pack2(p0, p1);
                    ds[i >> 3][(i & 7) >> 1] =
                        Mfma<T>::pack2(p0 * (dp[i] - d4[e]), p1 * (dp[i + 1] - d4[e + 1]));
                }
            }
            tmul(acc_v, pp, gst, kb);
            tmul(acc_k, ds, qst, kb);
        }
        if (t + 1 < t1) store_stats(st ^ 1, nx);
    }
    if (key < S) {
        T* kp = dk + head_base + (int64_t)key * row_stride + 4 * hh;
        T* vp = dv + head_base + (int64_t)key * row_stride + 4 * hh;
#pragma unroll
        for (int d = 0; d < DB; ++d)
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                if (PAD && 32 * d + 8 * g >= ncol) continue;
                *reinterpret_cast<u32x2*>(kp + 32 * d + 8 * g) =
                    u32x2{Mfma<T>::pack2(acc_k[d][4 * g] * scale, acc_k[d][4 * g + 1] * scale),
                          Mfma<T>::pack2(acc_k[d][4 * g + 2] * scale, acc_k[d][4 * g + 3] * scale)};
                *reinterpret_cast<u32x2*>(vp + 32 * d + 8 * g) =
                    u32x2{Mfma<T>::pack2(acc_v[d][4 * g], acc_v[d][4 * g + 1]),
                          Mfma<T>::pack2(acc_v[d][4 * g + 2], acc_v[d][4 * g + 3])};
            }
    }
}

template <typename T, int D, bool PAD>
hipError_t launch_bwd_t(const BwdArgs& a) {
    const int64_t rows = a.B * a.H * a.S;
    hipLaunchKernelGGL((fa_bwd_rowdot_kernel<T, D, PAD>), dim3((unsigned)((rows + 255) / 256)),
                       dim3(256), 0, a.stream, (const T*)a.out, (const T*)a.dout, a.di, (int)a.B,
                       (int)a.H, (int)a.S, (int)a.D, a.counters);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    // the dynamic tails of causal passes (dyn_first_position, dyn_first_key_blocks):
    // three dQ workgroups per compute unit at D = 64, two at 128; two dK / dV
    int dev = 0, cus = 0;
    if (hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) {
        (void)hipGetLastError();
        cus = 0;  // the static order
    }
    const MaskSpec ms{a.S, a.causal, a.wl, a.wr};
    const int n_qt = (int)((a.S + 127) / 128);
    const int dyn_q = cus > 0 ? (int)dyn_first_position(ms, a.B * a.H, 128, 64,
                                                        resident_wgs_per_cu(D) * (int64_t)cus)
                              : -1;
    hipLaunchKernelGGL((fa_bwd_dq_kernel<T, D, PAD>), dim3((unsigned)(a.B * a.H * n_qt)), dim3(256),
                       0, a.stream, (const T*)a.q, (const T*)a.k, (const T*)a.v, (const T*)a.dout,
                       a.lse, (const float*)a.di, (T*)a.dq, (int)a.B, (int)a.H, (int)a.S, a.c,
                       a.scale, a.causal, (int)a.wl, (int)a.wr, n_qt, (int)a.D, a.counters,
                       dyn_q);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    const int n_kt = (int)((a.S + kBwdKeys - 1) / kBwdKeys);
    const int dyn_k = cus > 0 ? (int)dyn_first_key_blocks(ms, a.B * a.H, kBwdKeys, 2 * (int64_t)cus)
                              : -1;
    hipLaunchKernelGGL((fa_bwd_dkdv_kernel<T, D, PAD>), dim3((unsigned)(a.B * a.H * n_kt)),
                       dim3(256), 0, a.stream, (const T*)a.q, (const T*)a.k, (const T*)a.v,
                       (const T*)a.dout, a.lse, (const float*)a.di, (T*)a.dk, (T*)a.dv, (int)a.B,
                       (int)a.H, (int)a.S, a.c, a.scale, a.causal, (int)a.wl, (int)a.wr, n_kt,
                       (int)a.D, a.counters + 1, dyn_k);
    return hipGetLastError();
}

}  // namespace fa
