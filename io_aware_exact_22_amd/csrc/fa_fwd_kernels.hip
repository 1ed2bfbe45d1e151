// fa_fwd_kernels.hip -- gfx950 (CDNA4) kernels of the fused exact-attention
// forward: O = softmax(scale * Q K^T + mask) V and the row log-sum-exp, with
// the S x S scores kept in registers and never written to HBM.
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
//  * A workgroup is 4 wave64s and owns a 128-row Q tile; each wave owns 32
//    query rows.  K/V tiles of 64 keys stream through double-buffered LDS.
//  * The scores are computed transposed, S^T = K Q^T, on the 32x32x16
//    bf16/f16 MFMA: in the MFMA result layout every lane then holds one query
//    row (lane % 32) and 16 of the tile's keys per 32-key block, so the row
//    max / row sum are in-lane reductions plus one exchange between the two
//    wave halves (v_permlane32_swap) instead of a 32-lane shuffle tree.
//  * The output is accumulated transposed too, O^T += V^T P^T: P^T is the
//    B operand straight from the score registers (the K rows of the score MFMA
//    are permuted so each lane's keys come out as 8 consecutive keys per
//    16-key chunk), and V^T is read from the row-major V tile in LDS with the
//    gfx950 transposing LDS read ds_read_b64_tr_b16.  The per-row rescale
//    factor then multiplies whole lanes -- no cross-lane traffic at all.
//  * Whole K/V tiles outside the causal / window mask are not visited; tiles
//    inside it for every row skip the mask; a wave skips the arithmetic of a
//    tile that is fully masked for its 32 rows.
//  * Workgroup ids are remapped so each XCD holds whole (batch, head) groups
//    (L2 reuse of K/V), and causal Q tiles run heaviest first.
//  * Probabilities are rounded to the input dtype (RNE, v_cvt_pk_*) for the
//    P V MFMA; max, sum, exp and the accumulators stay fp32.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "fa_launch.h"
#include "fa_schedule.h"

namespace fa {

typedef __bf16 bf16x8 __attribute__((__vector_size__(16)));
typedef _Float16 f16x8 __attribute__((__vector_size__(16)));
typedef short i16x4 __attribute__((__vector_size__(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned u32x2 __attribute__((ext_vector_type(2)));

#define FA_LDS __attribute__((address_space(3)))

constexpr int kWaves = 4;
constexpr int kThreads = kWaves * 64;
constexpr int kWaveRows = 32;             // query rows per wave
constexpr int kBM = kWaves * kWaveRows;   // query rows per workgroup
constexpr float kNegInf = -__builtin_inff();

// ---------------------------------------------------------------- dtype traits
template <typename T> struct Mfma;
template <> struct Mfma<__bf16> {
    typedef bf16x8 vec8;
    __device__ static inline f32x16 mma(u32x4 a, u32x4 b, f32x16 c) {
        return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a),
                                                       __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
    }
    // two fp32 -> two RNE-rounded bf16 packed in one dword (v_cvt_pk_bf16_f32)
    __device__ static inline unsigned pack2(float x, float y) {
        typedef __bf16 bf16x2 __attribute__((__vector_size__(4)));
        bf16x2 r;
        r[0] = (__bf16)x;
        r[1] = (__bf16)y;
        return __builtin_bit_cast(unsigned, r);
    }
};
template <> struct Mfma<_Float16> {
    typedef f16x8 vec8;
    __device__ static inline f32x16 mma(u32x4 a, u32x4 b, f32x16 c) {
        return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8, a),
                                                      __builtin_bit_cast(f16x8, b), c, 0, 0, 0);
    }
    __device__ static inline unsigned pack2(float x, float y) {
        typedef _Float16 f16x2 __attribute__((__vector_size__(4)));
        f16x2 r;
        r[0] = (_Float16)x;
        r[1] = (_Float16)y;
        return __builtin_bit_cast(unsigned, r);
    }
};

// max over both wave halves: permlane32_swap(x, x) returns x of the lower
// half in element 0 and x of the upper half in element 1, in every lane.
__device__ inline float halves_max(float x) {
    auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ inline float halves_sum(float x) {
    auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// Key offset (within a 32-key block) of score register i in wave half hh:
// the K row fed to MFMA row m = 8*(m/8) + 4*hh' + (m%4) is chosen so that
// register i of half hh holds key 16*(i/8) + 8*hh + (i%8).
__device__ inline int score_key(int i, int hh) { return 16 * (i >> 3) + 8 * hh + (i & 7); }
// K row fed to MFMA row m (the inverse view of score_key).
__device__ inline int k_row_for_mfma_row(int m) {
    const int g = m >> 3, hh = (m >> 2) & 1, r = m & 3;
    return 16 * (g >> 1) + 8 * hh + 4 * (g & 1) + r;
}

// ---------------------------------------------------------------- bf16 / fp16
// LDS row strides (elements), padded for conflict-free MFMA operand reads.
template <int D> struct Lds {
    static constexpr int BN = 64;
    static constexpr int KS = D + 8;   // K rows: 16-byte reads of 32 different rows
    static constexpr int VS = D + 32;  // V rows: transposing 8-byte reads of 8 rows
    static constexpr int K_ELEMS = BN * KS;
    static constexpr int V_ELEMS = BN * VS;
    static constexpr int STAGE = K_ELEMS + V_ELEMS;
    static constexpr int CHUNKS = BN * D / 8;             // 16-byte chunks per K (or V) tile
    static constexpr int PER_THREAD = CHUNKS / kThreads;  // per thread, per matrix
};

template <typename T, int D>
__global__ __launch_bounds__(kThreads, 2) void fa_fwd_mfma_kernel(
    const T* __restrict__ q, const T* __restrict__ k, const T* __restrict__ v, T* __restrict__ out,
    float* __restrict__ lse, int B, int H, int S, float c, int causal, int wl, int wr, int n_qt) {
    typedef Lds<D> L;
    constexpr int BN = L::BN;
    constexpr int KSTEPS = D / 16;  // 16-wide d chunks of the score MFMA
    constexpr int DB = D / 32;      // 32-wide d blocks of the output
    static_assert(L::CHUNKS % kThreads == 0, "tile chunks must split evenly");
    __shared__ __attribute__((aligned(16))) T lds[2 * L::STAGE];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int hh = lane >> 5;   // wave half
    const int ql = lane & 31;   // query row of this lane within the wave

    // ---- workgroup -> (b, h, q tile)
    const int64_t n_wg = (int64_t)B * H * n_qt;
    const int64_t logical = xcd_remap(blockIdx.x, n_wg);
    const int64_t bh = logical / n_qt;
    int qt = (int)(logical % n_qt);
    if (causal) qt = n_qt - 1 - qt;  // heaviest Q tiles first
    const int bb = (int)(bh / H), h = (int)(bh % H);

    const MaskSpec ms{S, causal, wl, wr};
    int64_t kt0, kt1;
    q_tile_kv_range(ms, qt, kBM, BN, &kt0, &kt1);

    const int64_t row_stride = (int64_t)H * D;                      // elements between rows
    const int64_t head_base = ((int64_t)bb * S * H + h) * D;        // element (b, 0, h, 0)
    const int q0 = qt * kBM;
    const int qw0 = q0 + wave * kWaveRows;  // first row of this wave
    const int qrow = qw0 + ql;              // this lane's query row

    // ---- Q fragment (B operand of S^T = K Q^T): row qrow, d = 16*ks + 8*hh .. +8
    u32x4 qf[KSTEPS];
    {
        const bool ok = qrow < S;
        const T* qp = q + head_base + (int64_t)(ok ? qrow : 0) * row_stride + 8 * hh;
#pragma unroll
        for (int ks = 0; ks < KSTEPS; ++ks) {
            u32x4 x = *reinterpret_cast<const u32x4*>(qp + 16 * ks);
            qf[ks] = ok ? x : u32x4{0, 0, 0, 0};
        }
    }

    // ---- K/V tile loader: 16-byte chunks, rows past S read as zero
    auto load_tile = [&](int64_t kt, u32x4* kr, u32x4* vr) {
        const int64_t k0 = kt * BN;
#pragma unroll
        for (int u = 0; u < L::PER_THREAD; ++u) {
            const int id = u * kThreads + tid;
            const int r = id / (D / 8), cc = id % (D / 8);
            const int64_t key = k0 + r;
            const bool ok = key < S;
            const int64_t off = head_base + (ok ? key : 0) * row_stride + cc * 8;
            u32x4 xk = *reinterpret_cast<const u32x4*>(k + off);
            u32x4 xv = *reinterpret_cast<const u32x4*>(v + off);
            kr[u] = ok ? xk : u32x4{0, 0, 0, 0};
            vr[u] = ok ? xv : u32x4{0, 0, 0, 0};
        }
    };
    auto store_tile = [&](int stage, const u32x4* kr, const u32x4* vr) {
        T* ks = lds + stage * L::STAGE;
        T* vs = ks + L::K_ELEMS;
#pragma unroll
        for (int u = 0; u < L::PER_THREAD; ++u) {
            const int id = u * kThreads + tid;
            const int r = id / (D / 8), cc = id % (D / 8);
            *reinterpret_cast<u32x4*>(ks + r * L::KS + cc * 8) = kr[u];
            *reinterpret_cast<u32x4*>(vs + r * L::VS + cc * 8) = vr[u];
        }
    };

    // ---- running statistics (log2 domain: m is a max of c * s)
    float m_run = kNegInf;  // running max
    float l_run = 0.f;      // running sum over this half's keys
    f32x16 o[DB];
#pragma unroll
    for (int d = 0; d < DB; ++d) o[d] = f32x16{0};

    u32x4 kr[L::PER_THREAD], vr[L::PER_THREAD];
    if (kt0 < kt1) {
        load_tile(kt0, kr, vr);
        store_tile(0, kr, vr);
    }
    __syncthreads();

    const int krow0 = k_row_for_mfma_row(ql);  // K row this lane feeds to the score MFMA
    for (int64_t kt = kt0; kt < kt1; ++kt) {
        const int stage = (int)((kt - kt0) & 1);
        const bool has_next = kt + 1 < kt1;
        if (has_next) load_tile(kt + 1, kr, vr);  // in flight during this tile's math

        const int64_t k0 = kt * BN;
        const bool skip = tile_fully_masked(ms, qw0, qw0 + kWaveRows - 1, k0, BN);
        if (!skip) {
            const T* ks = lds + stage * L::STAGE;
            const T* vs = ks + L::K_ELEMS;
            // S^T for two 32-key blocks
            f32x16 s[2];
#pragma unroll
            for (int kb = 0; kb < 2; ++kb) {
                s[kb] = f32x16{0};
                const T* kp = ks + (32 * kb + krow0) * L::KS + 8 * hh;
#pragma unroll
                for (int kk = 0; kk < KSTEPS; ++kk) {
                    u32x4 a = *reinterpret_cast<const u32x4*>(kp + 16 * kk);
                    s[kb] = Mfma<T>::mma(a, qf[kk], s[kb]);
                }
            }
            // mask (boundary tiles only)
            const bool need_mask = tile_needs_mask(ms, qw0, qw0 + kWaveRows - 1, k0, BN);
            if (need_mask) {
#pragma unroll
                for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                    for (int i = 0; i < 16; ++i) {
                        const int key = (int)k0 + 32 * kb + score_key(i, hh);
                        bool ok = key < S;
                        if (causal) ok = ok && key <= qrow;
                        if (wl >= 0) ok = ok && qrow - key <= wl;
                        if (wr >= 0) ok = ok && key - qrow <= wr;
                        s[kb][i] = ok ? s[kb][i] : kNegInf;
                    }
            }
            // row max over the tile (in-lane, then across halves)
            float mx = kNegInf;
#pragma unroll
            for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                for (int i = 0; i < 16; ++i) mx = fmaxf(mx, s[kb][i]);
            mx = halves_max(mx);
            const float mt = (mx == kNegInf) ? kNegInf : mx * c;  // scaled; c may be 0
            const float m_new = fmaxf(m_run, mt);
            const float m_use = (m_new == kNegInf) ? 0.f : m_new;  // row fully masked so far
            const float alpha = __builtin_amdgcn_exp2f(m_run - m_use);
            m_run = m_new;
            // probabilities, row sum, pack to the input dtype for P V
            u32x4 p[4];
            float rs = 0.f;
#pragma unroll
            for (int kb = 0; kb < 2; ++kb) {
                float e[16];
#pragma unroll
                for (int i = 0; i < 16; ++i) {
                    float x = __builtin_amdgcn_exp2f(__builtin_fmaf(s[kb][i], c, -m_use));
                    if (need_mask) x = (s[kb][i] == kNegInf) ? 0.f : x;
                    e[i] = x;
                    rs += x;
                }
#pragma unroll
                for (int half = 0; half < 2; ++half) {
                    u32x4 pk;
#pragma unroll
                    for (int t = 0; t < 4; ++t)
                        pk[t] = Mfma<T>::pack2(e[8 * half + 2 * t], e[8 * half + 2 * t + 1]);
                    p[2 * kb + half] = pk;
                }
            }
            l_run = alpha * l_run + rs;
            if (__any(alpha != 1.f)) {  // skip the rescale when no row max moved
#pragma unroll
                for (int d = 0; d < DB; ++d) o[d] *= alpha;
            }
            // O^T += V^T P^T: V^T via transposing LDS reads of the row-major V tile
            const int tr_row = 8 * hh + ((lane & 15) >> 2);
            const int tr_col = 16 * ((lane >> 4) & 1) + 4 * (lane & 3);
#pragma unroll
            for (int d = 0; d < DB; ++d) {
#pragma unroll
                for (int cch = 0; cch < 4; ++cch) {
                    const T* vp = vs + (16 * cch + tr_row) * L::VS + 32 * d + tr_col;
                    i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((FA_LDS i16x4*)(vp));
                    i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((FA_LDS i16x4*)(vp + 4 * L::VS));
                    u32x2 l2 = __builtin_bit_cast(u32x2, lo), h2 = __builtin_bit_cast(u32x2, hi);
                    u32x4 a = {l2[0], l2[1], h2[0], h2[1]};
                    o[d] = Mfma<T>::mma(a, p[cch], o[d]);
                }
            }
        }
        if (has_next) store_tile(stage ^ 1, kr, vr);
        __syncthreads();
    }

    // ---- epilogue: O = O_acc / l, LSE = ln2 * (m + log2 l)
    const float l_tot = halves_sum(l_run);
    const float inv = (l_tot > 0.f) ? 1.f / l_tot : 0.f;
    if (qrow < S) {
        T* op = out + head_base + (int64_t)qrow * row_stride + 4 * hh;
#pragma unroll
        for (int d = 0; d < DB; ++d)
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                u32x2 w = {Mfma<T>::pack2(o[d][4 * g] * inv, o[d][4 * g + 1] * inv),
                           Mfma<T>::pack2(o[d][4 * g + 2] * inv, o[d][4 * g + 3] * inv)};
                *reinterpret_cast<u32x2*>(op + 32 * d + 8 * g) = w;
            }
        if (hh == 0) {
            const float m_fin = (m_run == kNegInf) ? 0.f : m_run;
            const float lse_v = (l_tot > 0.f) ? 0.69314718055994531f * (m_fin + __log2f(l_tot)) : kNegInf;
            lse[((int64_t)bb * H + h) * S + qrow] = lse_v;
        }
    }
}

// ---------------------------------------------------------------- fp32
// fp32 inputs run the same transposed-score structure on the fp32 MFMA
// (v_mfma_f32_32x32x2_f32), so every product is an fp32 product; one key
// (or one d) per lane per MFMA means V needs no transposition.
template <int D> struct Lds32 {
    static constexpr int BN = 32;
    static constexpr int KS = D + 1;
    static constexpr int VS = D + 4;
};

template <int D>
__global__ __launch_bounds__(kThreads, 2) void fa_fwd_fp32_kernel(
    const float* __restrict__ q, const float* __restrict__ k, const float* __restrict__ v,
    float* __restrict__ out, float* __restrict__ lse, int B, int H, int S, float c, int causal,
    int wl, int wr, int n_qt) {
    typedef Lds32<D> L;
    constexpr int BN = L::BN;
    constexpr int DB = D / 32;
    __shared__ float ks[BN * L::KS];
    __shared__ float vs[BN * L::VS];

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int hh = lane >> 5, ql = lane & 31;
    const int64_t n_wg = (int64_t)B * H * n_qt;
    const int64_t logical = xcd_remap(blockIdx.x, n_wg);
    const int64_t bh = logical / n_qt;
    int qt = (int)(logical % n_qt);
    if (causal) qt = n_qt - 1 - qt;
    const int bb = (int)(bh / H), h = (int)(bh % H);
    const MaskSpec ms{S, causal, wl, wr};
    int64_t kt0, kt1;
    q_tile_kv_range(ms, qt, kBM, BN, &kt0, &kt1);
    const int64_t row_stride = (int64_t)H * D;
    const int64_t head_base = ((int64_t)bb * S * H + h) * D;
    const int qw0 = qt * kBM + wave * kWaveRows;
    const int qrow = qw0 + ql;

    // Q fragment: lane supplies d = 2*kk + hh of its row
    float qf[D / 2];
    {
        const bool ok = qrow < S;
        const float* qp = q + head_base + (int64_t)(ok ? qrow : 0) * row_stride;
#pragma unroll
        for (int kk = 0; kk < D / 2; ++kk) qf[kk] = ok ? qp[2 * kk + hh] : 0.f;
    }
    float m_run = kNegInf, l_run = 0.f;
    f32x16 o[DB];
#pragma unroll
    for (int d = 0; d < DB; ++d) o[d] = f32x16{0};

    for (int64_t kt = kt0; kt < kt1; ++kt) {
        const int64_t k0 = kt * BN;
        __syncthreads();
        for (int id = tid; id < BN * (D / 4); id += kThreads) {
            const int r = id / (D / 4), cc = id % (D / 4);
            const int64_t key = k0 + r;
            const bool ok = key < S;
            const int64_t off = head_base + (ok ? key : 0) * row_stride + cc * 4;
            f32x4 xk = *reinterpret_cast<const f32x4*>(k + off);
            f32x4 xv = *reinterpret_cast<const f32x4*>(v + off);
#pragma unroll
            for (int t = 0; t < 4; ++t) {
                ks[r * L::KS + cc * 4 + t] = ok ? xk[t] : 0.f;
                vs[r * L::VS + cc * 4 + t] = ok ? xv[t] : 0.f;
            }
        }
        __syncthreads();
        if (tile_fully_masked(ms, qw0, qw0 + kWaveRows - 1, k0, BN)) continue;
        // S^T (32 keys x 32 queries): A = K row (lane % 32), d = 2*kk + hh
        f32x16 s = f32x16{0};
#pragma unroll
        for (int kk = 0; kk < D / 2; ++kk)
            s = __builtin_amdgcn_mfma_f32_32x32x2f32(ks[ql * L::KS + 2 * kk + hh], qf[kk], s, 0, 0, 0);
        // register i holds key 8*(i/4) + 4*hh + (i%4)
        const bool need_mask = tile_needs_mask(ms, qw0, qw0 + kWaveRows - 1, k0, BN);
        if (need_mask) {
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
        mx = halves_max(mx);
        const float mt = (mx == kNegInf) ? kNegInf : mx * c;
        const float m_new = fmaxf(m_run, mt);
        const float m_use = (m_new == kNegInf) ? 0.f : m_new;
        const float alpha = __builtin_amdgcn_exp2f(m_run - m_use);
        m_run = m_new;
        float p[16], rs = 0.f;
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            float x = __builtin_amdgcn_exp2f(__builtin_fmaf(s[i], c, -m_use));
            if (need_mask) x = (s[i] == kNegInf) ? 0.f : x;
            p[i] = x;
            rs += x;
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
    const float l_tot = halves_sum(l_run);
    const float inv = (l_tot > 0.f) ? 1.f / l_tot : 0.f;
    if (qrow < S) {
        float* op = out + head_base + (int64_t)qrow * row_stride + 4 * hh;
#pragma unroll
        for (int d = 0; d < DB; ++d)
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                f32x4 w = {o[d][4 * g] * inv, o[d][4 * g + 1] * inv, o[d][4 * g + 2] * inv,
                           o[d][4 * g + 3] * inv};
                *reinterpret_cast<f32x4*>(op + 32 * d + 8 * g) = w;
            }
        if (hh == 0) {
            const float m_fin = (m_run == kNegInf) ? 0.f : m_run;
            const float lse_v = (l_tot > 0.f) ? 0.69314718055994531f * (m_fin + __log2f(l_tot)) : kNegInf;
            lse[((int64_t)bb * H + h) * S + qrow] = lse_v;
        }
    }
}

// ---------------------------------------------------------------- launchers
template <typename T, int D>
static hipError_t launch_mfma(const LaunchArgs& a) {
    const int n_qt = (int)((a.S + kBM - 1) / kBM);
    const int64_t n_wg = a.B * a.H * n_qt;
    hipLaunchKernelGGL((fa_fwd_mfma_kernel<T, D>), dim3((unsigned)n_wg), dim3(kThreads), 0, a.stream,
                       (const T*)a.q, (const T*)a.k, (const T*)a.v, (T*)a.out, a.lse, (int)a.B,
                       (int)a.H, (int)a.S, a.c, a.causal, (int)a.wl, (int)a.wr, n_qt);
    return hipGetLastError();
}

template <int D>
static hipError_t launch_fp32(const LaunchArgs& a) {
    const int n_qt = (int)((a.S + kBM - 1) / kBM);
    const int64_t n_wg = a.B * a.H * n_qt;
    hipLaunchKernelGGL((fa_fwd_fp32_kernel<D>), dim3((unsigned)n_wg), dim3(kThreads), 0, a.stream,
                       (const float*)a.q, (const float*)a.k, (const float*)a.v, (float*)a.out, a.lse,
                       (int)a.B, (int)a.H, (int)a.S, a.c, a.causal, (int)a.wl, (int)a.wr, n_qt);
    return hipGetLastError();
}

hipError_t launch_fwd(const LaunchArgs& a) {
    switch (a.dtype) {
    case kDtypeBf16: return a.D == 64 ? launch_mfma<__bf16, 64>(a) : launch_mfma<__bf16, 128>(a);
    case kDtypeFp16: return a.D == 64 ? launch_mfma<_Float16, 64>(a) : launch_mfma<_Float16, 128>(a);
    default: return a.D == 64 ? launch_fp32<64>(a) : launch_fp32<128>(a);
    }
}

int64_t q_tile_rows() { return kBM; }
int64_t kv_tile_keys(int dtype) { return dtype == kDtypeFp32 ? Lds32<64>::BN : Lds<64>::BN; }

}  // namespace fa
