/*
 * fa_oracle.c -- the CPU oracle for exact attention (forward, and the backward
 * gradients at the end of the file).
 *
 * TEST INFRASTRUCTURE, NOT PRODUCT CODE.  Only the tests, the smoke check and
 * the CPU-baseline leg of the benchmark may load this library.  It shares no
 * code, header, table or constant with the GPU library, and the GPU library
 * never calls it.
 *
 * What it computes is the plain definition of exact attention, written out in
 * fp64 with the full score matrix materialised, one (batch, head) at a time:
 *
 *   allowed(i,j) = (!causal || j <= i) && (wl < 0 || i - j <= wl)
 *                                       && (wr < 0 || j - i <= wr)
 *   s_ij  = scale * sum_d q[b,i,h,d] * k[b,j,h,d]     (allowed j only)
 *   p_ij  = exp(s_ij - m_i) / sum_j' exp(s_ij' - m_i),  m_i = max_j s_ij
 *   O[b,i,h,:]  = sum_j p_ij * v[b,j,h,:]
 *   LSE[b,h,i]  = m_i + ln(sum_j exp(s_ij - m_i))   (= ln sum_j exp(s_ij))
 *
 * Sources (pages are named by their titles):
 *  - the formula Softmax(QK^T / sqrt(d_k)) V: "大模型加速新突破：Flash Attention
 *    V2核心网络算子解析", section 二.1 (算法核心创新), the core formula;
 *  - the arguments softmax_scale (default 1/sqrt(head_dim)), causal and
 *    window_size=(left,right) with (-1,-1) meaning full attention:
 *    "FlashAttention技术解析：加速GPT训练的核心优化", section 2.2, the
 *    configuration example and its parameter notes; the window example
 *    window_size=(128,128) in "突破大模型训练瓶颈：Flash-Attention编译优化与
 *    内存占用解决方案", section 滑动窗口注意力;
 *  - the input layout (batch, seq_len, head, dim): the V2 page, section 三.1
 *    (代码实现要点), the comment on the input shape;
 *  - the result is exact, not approximated: the project tagline quoted on the
 *    compile-guide page ("exact attention");
 *  - the log-domain statistic (log of the sum of exponentials) that LSE is:
 *    the V2 page, section 二.1, step 2 (增量软最大值).
 *
 * Readings where the pages are silent:
 *  - window bounds are inclusive and "left" means earlier positions;
 *  - causal together with a window is the intersection of the two masks;
 *  - a row with no allowed key (unreachable with windows >= -1, since j = i is
 *    always allowed) gets O = 0 and LSE = -inf;
 *  - NaN propagates as in IEEE arithmetic: the max of a set holding a NaN is
 *    NaN, so a NaN score makes the whole row NaN;
 *  - bf16/fp16/fp32 inputs are decoded exactly to fp64 (subnormals kept).
 *
 * Block-sparse attention ("FlashAttention技术解析：加速GPT训练的核心优化",
 * section 5, lists a block-sparse variant of the method that reaches very long
 * contexts through a sparse pattern) is the same definition with one more
 * factor in allowed(i, j): the block mask bit of the (query block, key block)
 * pair,
 *
 *   allowed_bs(i,j) = allowed(i,j) && mask[i / block_m][j / block_n] != 0,
 *
 * with mask a row-major [ceil(S/block_m), ceil(S/block_n)] byte matrix per
 * (b, h) -- shared by every head (n_mask = 1), by every batch (n_mask = H) or
 * one per (b, h) (n_mask = B*H).  Reading: the pages name the variant and its
 * purpose only; the plainest reading, a block-granular mask intersected with
 * the causal and window masks, is the one taken.  A row whose blocks are all
 * off has no allowed key: O = 0, LSE = -inf, as above.
 *
 * Paged K/V ("突破大模型训练瓶颈：Flash-Attention编译优化与内存占用解决方案",
 * section Paged KV Cache支持: the K/V cache is kept in non-contiguous blocks, like
 * memory pages of an operating system, found through a block table) changes
 * where keys and values are read, not what is computed: key j of batch b is
 * row j % page_size of page block_table[b][j / page_size] of the pools
 * k_pages / v_pages [num_pages, page_size, H, D].  fa_oracle_fwd_paged gathers
 * those rows into contiguous [B, S, H, D] tensors and runs the definition
 * above on them.  Reading: the pages give the block table and nothing else;
 * one S for queries and keys, as above.
 *
 * Build: gcc -O2 -fopenmp -shared -fPIC fa_oracle.c -o libfa_oracle.so -lm
 * No -ffast-math: the oracle depends on IEEE inf/NaN semantics.
 */
#include <math.h>
#include <omp.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define ORC_FP32 0
#define ORC_FP16 1
#define ORC_BF16 2

/* IEEE-754 binary32: reinterpret the 32 bits. */
static double orc_decode_fp32(uint32_t bits) {
    float f;
    memcpy(&f, &bits, sizeof f);
    return (double)f;
}

/* IEEE-754 binary16: 1 sign bit, 5 exponent bits (bias 15), 10 fraction
 * bits.  Written from the format's definition, subnormals included. */
static double orc_decode_fp16(uint16_t h) {
    int sign = (h >> 15) & 1;
    int e = (h >> 10) & 0x1f;
    int f = h & 0x3ff;
    double mag;
    if (e == 0)
        mag = ldexp((double)f, -24); /* 0.f * 2^-14 */
    else if (e == 31)
        mag = (f == 0) ? INFINITY : NAN;
    else
        mag = ldexp(1024.0 + (double)f, e - 25); /* 1.f * 2^(e-15) */
    return sign ? -mag : mag;
}

/* bfloat16: 1 sign bit, 8 exponent bits (bias 127), 7 fraction bits -- the
 * upper half of a binary32.  Written from the field definition. */
static double orc_decode_bf16(uint16_t b) {
    int sign = (b >> 15) & 1;
    int e = (b >> 7) & 0xff;
    int f = b & 0x7f;
    double mag;
    if (e == 0)
        mag = ldexp((double)f, -133); /* 0.f * 2^-126 */
    else if (e == 255)
        mag = (f == 0) ? INFINITY : NAN;
    else
        mag = ldexp(128.0 + (double)f, e - 134); /* 1.f * 2^(e-127) */
    return sign ? -mag : mag;
}

static double orc_load(const void* base, int dtype, int64_t idx) {
    switch (dtype) {
    case ORC_FP32: return orc_decode_fp32(((const uint32_t*)base)[idx]);
    case ORC_FP16: return orc_decode_fp16(((const uint16_t*)base)[idx]);
    default: return orc_decode_bf16(((const uint16_t*)base)[idx]);
    }
}

static int orc_allowed(int64_t i, int64_t j, int causal, int64_t wl, int64_t wr) {
    if (causal && j > i) return 0;
    if (wl >= 0 && i - j > wl) return 0;
    if (wr >= 0 && j - i > wr) return 0;
    return 1;
}

/* The block mask factor of allowed_bs: mask is one (b, h)'s row-major
 * [n_qb, n_kb] byte matrix, or NULL for no block mask. */
static int orc_block_on(const uint8_t* mask, int64_t i, int64_t j, int64_t block_m,
                        int64_t block_n, int64_t n_kb) {
    if (!mask) return 1;
    return mask[(i / block_m) * n_kb + j / block_n] != 0;
}

/* Decodes n elements of raw input bits to fp64, so the tests can check the
 * decoders against other implementations of the formats. */
int fa_oracle_decode(const void* base, int dtype, int64_t n, double* out) {
    if (dtype != ORC_FP32 && dtype != ORC_FP16 && dtype != ORC_BF16) return -1;
    for (int64_t i = 0; i < n; ++i) out[i] = orc_load(base, dtype, i);
    return 0;
}

/* Number of (i, j) pairs with allowed(i, j), over 0 <= i, j < S. */
int64_t fa_oracle_allowed_pairs(int64_t S, int causal, int64_t wl, int64_t wr) {
    int64_t n = 0;
    for (int64_t i = 0; i < S; ++i)
        for (int64_t j = 0; j < S; ++j) n += orc_allowed(i, j, causal, wl, wr);
    return n;
}

static int orc_check(int dtype, int64_t B, int64_t H, int64_t S, int64_t D,
                     int64_t wl, int64_t wr) {
    if (dtype != ORC_FP32 && dtype != ORC_FP16 && dtype != ORC_BF16) return -1;
    if (B < 1 || H < 1 || S < 1 || D < 1) return -1;
    if (wl < -1 || wr < -1) return -1;
    return 0;
}

/*
 * Query rows [i0, i1) of one (b, h), with an optional block mask (bmask: this
 * (b, h)'s [ceil(S/block_m), ceil(S/block_n)] bytes, or NULL).  out_rows is
 * [(i1 - i0), D] fp64, lse_rows is [(i1 - i0)] fp64.  The (i1 - i0) x S score
 * matrix of this head is materialised in full; rows run in parallel over
 * nthreads OpenMP threads (0 = the OpenMP default).
 */
static int orc_fwd_rows(const void* q, const void* k, const void* v, int dtype, int64_t B,
                        int64_t H, int64_t S, int64_t D, double scale, int causal, int64_t wl,
                        int64_t wr, const uint8_t* bmask, int64_t block_m, int64_t block_n,
                        int64_t b, int64_t h, int64_t i0, int64_t i1, double* out_rows,
                        double* lse_rows, int nthreads) {
    if (orc_check(dtype, B, H, S, D, wl, wr)) return -1;
    if (b < 0 || b >= B || h < 0 || h >= H || i0 < 0 || i1 > S || i0 > i1) return -1;
    if (bmask && (block_m < 1 || block_n < 1)) return -1;
    const int64_t n_kb = bmask ? (S + block_n - 1) / block_n : 0;
    const int64_t R = i1 - i0;
    if (R == 0) return 0;
    /* element (b, s, h, d) of a [B, S, H, D] tensor */
#define ORC_IDX(s_, d_) ((((b) * S + (s_)) * H + (h)) * D + (d_))
    double* Q = (double*)malloc(sizeof(double) * (size_t)(R * D));
    double* K = (double*)malloc(sizeof(double) * (size_t)(S * D));
    double* V = (double*)malloc(sizeof(double) * (size_t)(S * D));
    double* P = (double*)malloc(sizeof(double) * (size_t)(R * S)); /* scores, then probabilities */
    if (!Q || !K || !V || !P) {
        free(Q); free(K); free(V); free(P);
        return -2;
    }
    for (int64_t r = 0; r < R; ++r)
        for (int64_t d = 0; d < D; ++d) Q[r * D + d] = orc_load(q, dtype, ORC_IDX(i0 + r, d));
    for (int64_t j = 0; j < S; ++j)
        for (int64_t d = 0; d < D; ++d) {
            K[j * D + d] = orc_load(k, dtype, ORC_IDX(j, d));
            V[j * D + d] = orc_load(v, dtype, ORC_IDX(j, d));
        }
#undef ORC_IDX
    if (nthreads <= 0) nthreads = omp_get_max_threads();
#pragma omp parallel for schedule(dynamic, 4) num_threads(nthreads)
    for (int64_t r = 0; r < R; ++r) {
        const int64_t i = i0 + r;
        double* prow = P + r * S;
        /* 1. scores of the allowed keys; -inf elsewhere */
        for (int64_t j = 0; j < S; ++j) {
            if (!orc_allowed(i, j, causal, wl, wr) ||
                !orc_block_on(bmask, i, j, block_m, block_n, n_kb)) {
                prow[j] = -INFINITY;
                continue;
            }
            double dot = 0.0;
            for (int64_t d = 0; d < D; ++d) dot += Q[r * D + d] * K[j * D + d];
            prow[j] = scale * dot;
        }
        /* 2. row max (a NaN anywhere makes it NaN) */
        double m = -INFINITY;
        for (int64_t j = 0; j < S; ++j) {
            if (isnan(prow[j])) {
                m = prow[j];
                break;
            }
            if (prow[j] > m) m = prow[j];
        }
        double* orow = out_rows + r * D;
        if (m == -INFINITY) { /* no allowed key */
            for (int64_t d = 0; d < D; ++d) orow[d] = 0.0;
            lse_rows[r] = -INFINITY;
            continue;
        }
        /* 3. softmax: exp(s - m), sum, divide */
        double l = 0.0;
        for (int64_t j = 0; j < S; ++j) {
            prow[j] = exp(prow[j] - m);
            l += prow[j];
        }
        for (int64_t j = 0; j < S; ++j) prow[j] /= l;
        /* 4. O = P V */
        for (int64_t d = 0; d < D; ++d) orow[d] = 0.0;
        for (int64_t j = 0; j < S; ++j) {
            if (!orc_allowed(i, j, causal, wl, wr) ||
                !orc_block_on(bmask, i, j, block_m, block_n, n_kb))
                continue; /* p = 0 exactly */
            const double p = prow[j];
            for (int64_t d = 0; d < D; ++d) orow[d] += p * V[j * D + d];
        }
        lse_rows[r] = m + log(l);
    }
    free(Q); free(K); free(V); free(P);
    return 0;
}

/* Query rows [i0, i1) of one (b, h), no block mask. */
int fa_oracle_fwd_rows(const void* q, const void* k, const void* v, int dtype,
                       int64_t B, int64_t H, int64_t S, int64_t D, double scale,
                       int causal, int64_t wl, int64_t wr, int64_t b, int64_t h,
                       int64_t i0, int64_t i1, double* out_rows, double* lse_rows,
                       int nthreads) {
    return orc_fwd_rows(q, k, v, dtype, B, H, S, D, scale, causal, wl, wr, NULL, 0, 0, b, h,
                        i0, i1, out_rows, lse_rows, nthreads);
}

/* The (b, h) block mask of a [n_mask, n_qb, n_kb] mask: one shared matrix
 * (n_mask = 1), one per head (n_mask = H) or one per (b, h) (n_mask = B*H);
 * NULL for any other n_mask.  Where H = 1 or B = 1 two readings coincide. */
static const uint8_t* orc_head_mask(const uint8_t* mask, int64_t n_mask, int64_t B, int64_t H,
                                    int64_t S, int64_t block_m, int64_t block_n, int64_t b,
                                    int64_t h) {
    const int64_t per = ((S + block_m - 1) / block_m) * ((S + block_n - 1) / block_n);
    int64_t hm;
    if (n_mask == 1)
        hm = 0;
    else if (n_mask == H)
        hm = h;
    else if (n_mask == B * H)
        hm = b * H + h;
    else
        return NULL;
    return mask + hm * per;
}

/* Block-sparse rows [i0, i1) of one (b, h): mask is [n_mask, n_qb, n_kb]. */
int fa_oracle_fwd_rows_blocksparse(const void* q, const void* k, const void* v, int dtype,
                                   int64_t B, int64_t H, int64_t S, int64_t D, double scale,
                                   int causal, int64_t wl, int64_t wr, const uint8_t* mask,
                                   int64_t n_mask, int64_t block_m, int64_t block_n, int64_t b,
                                   int64_t h, int64_t i0, int64_t i1, double* out_rows,
                                   double* lse_rows, int nthreads) {
    if (!mask || block_m < 1 || block_n < 1 || b < 0 || b >= B || h < 0 || h >= H) return -1;
    const uint8_t* hmask = orc_head_mask(mask, n_mask, B, H, S, block_m, block_n, b, h);
    if (!hmask) return -1;
    return orc_fwd_rows(q, k, v, dtype, B, H, S, D, scale, causal, wl, wr, hmask, block_m,
                        block_n, b, h, i0, i1, out_rows, lse_rows, nthreads);
}

/*
 * Every (b, h), all rows.  out is [B, S, H, D] fp64 and lse is [B, H, S] fp64.
 */
int fa_oracle_fwd(const void* q, const void* k, const void* v, int dtype, int64_t B,
                  int64_t H, int64_t S, int64_t D, double scale, int causal, int64_t wl,
                  int64_t wr, double* out, double* lse, int nthreads) {
    if (orc_check(dtype, B, H, S, D, wl, wr)) return -1;
    double* rows = (double*)malloc(sizeof(double) * (size_t)(S * D));
    if (!rows) return -2;
    for (int64_t b = 0; b < B; ++b)
        for (int64_t h = 0; h < H; ++h) {
            int rc = fa_oracle_fwd_rows(q, k, v, dtype, B, H, S, D, scale, causal, wl, wr, b,
                                        h, 0, S, rows, lse + (b * H + h) * S, nthreads);
            if (rc) {
                free(rows);
                return rc;
            }
            for (int64_t i = 0; i < S; ++i)
                memcpy(out + ((b * S + i) * H + h) * D, rows + i * D, sizeof(double) * (size_t)D);
        }
    free(rows);
    return 0;
}

/*
 * Block-sparse attention over every (b, h), all rows: fa_oracle_fwd with the
 * block mask factor (mask [n_mask, ceil(S/block_m), ceil(S/block_n)] bytes).
 */
int fa_oracle_fwd_blocksparse(const void* q, const void* k, const void* v, int dtype,
                              int64_t B, int64_t H, int64_t S, int64_t D, double scale,
                              int causal, int64_t wl, int64_t wr, const uint8_t* mask,
                              int64_t n_mask, int64_t block_m, int64_t block_n, double* out,
                              double* lse, int nthreads) {
    if (orc_check(dtype, B, H, S, D, wl, wr)) return -1;
    if (!mask || block_m < 1 || block_n < 1) return -1;
    double* rows = (double*)malloc(sizeof(double) * (size_t)(S * D));
    if (!rows) return -2;
    for (int64_t b = 0; b < B; ++b)
        for (int64_t h = 0; h < H; ++h) {
            int rc = fa_oracle_fwd_rows_blocksparse(q, k, v, dtype, B, H, S, D, scale, causal,
                                                    wl, wr, mask, n_mask, block_m, block_n, b,
                                                    h, 0, S, rows, lse + (b * H + h) * S,
                                                    nthreads);
            if (rc) {
                free(rows);
                return rc;
            }
            for (int64_t i = 0; i < S; ++i)
                memcpy(out + ((b * S + i) * H + h) * D, rows + i * D, sizeof(double) * (size_t)D);
        }
    free(rows);
    return 0;
}

/*
 * Gathers one paged pool [num_pages, page_size, H, D] (element size esize
 * bytes) into a contiguous [B, S, H, D] tensor by the block table
 * [B, table_stride]: row j of batch b comes from page block_table[b *
 * table_stride + j / page_size], row j % page_size.  Returns -1 when a page
 * index the sequence uses lies outside [0, num_pages).
 */
int fa_oracle_gather_pages(const void* pages, int64_t esize, int64_t num_pages,
                           int64_t page_size, const int32_t* block_table, int64_t table_stride,
                           int64_t B, int64_t S, int64_t H, int64_t D, void* dense) {
    if (!pages || !block_table || !dense || esize < 1 || page_size < 1 || num_pages < 1) return -1;
    if (table_stride < (S + page_size - 1) / page_size) return -1;
    const int64_t row_bytes = H * D * esize;
    for (int64_t b = 0; b < B; ++b)
        for (int64_t j = 0; j < S; ++j) {
            const int64_t page = block_table[b * table_stride + j / page_size];
            if (page < 0 || page >= num_pages) return -1;
            const int64_t src_row = page * page_size + j % page_size;
            memcpy((char*)dense + (b * S + j) * row_bytes, (const char*)pages + src_row * row_bytes,
                   (size_t)row_bytes);
        }
    return 0;
}

/*
 * fa_oracle_bwd -- gradients of exact attention with respect to q, k and v for
 * an output gradient dout, in fp64, with the full probability and score-
 * gradient matrices of each (b, h) materialised.  It is the chain rule through
 * the forward definition above, written out (the V2 page, section 二.1, step 3
 * names the backward pass that reuses what the forward saved):
 *
 *   p_ij  = exp(s_ij - m_i) / sum_j' exp(s_ij' - m_i)    (0 where j is not allowed)
 *   dV_j  = sum_i p_ij dO_i
 *   dP_ij = dO_i . v_j
 *   D_i   = sum_j p_ij dP_ij
 *   dS_ij = p_ij (dP_ij - D_i)
 *   dQ_i  = scale * sum_j dS_ij k_j
 *   dK_j  = scale * sum_i dS_ij q_i
 *
 * dout has the inputs' dtype and layout.  dq, dk, dv are [B, S, H, D] fp64.  A
 * row with no allowed key contributes nothing.  NaN propagates.
 */
int fa_oracle_bwd(const void* q, const void* k, const void* v, const void* dout, int dtype,
                  int64_t B, int64_t H, int64_t S, int64_t D, double scale, int causal,
                  int64_t wl, int64_t wr, double* dq, double* dk, double* dv, int nthreads) {
    if (orc_check(dtype, B, H, S, D, wl, wr)) return -1;
    if (nthreads <= 0) nthreads = omp_get_max_threads();
    const size_t sd = (size_t)(S * D), ss = (size_t)(S * S);
    double* Q = (double*)malloc(sizeof(double) * sd);
    double* K = (double*)malloc(sizeof(double) * sd);
    double* V = (double*)malloc(sizeof(double) * sd);
    double* dO = (double*)malloc(sizeof(double) * sd);
    double* P = (double*)malloc(sizeof(double) * ss);  /* probabilities */
    double* dS = (double*)malloc(sizeof(double) * ss); /* dP, then dS */
    if (!Q || !K || !V || !dO || !P || !dS) {
        free(Q); free(K); free(V); free(dO); free(P); free(dS);
        return -2;
    }
    for (int64_t b = 0; b < B; ++b)
        for (int64_t h = 0; h < H; ++h) {
#define ORC_BIDX(s_, d_) (((b * S + (s_)) * H + h) * D + (d_))
            for (int64_t s = 0; s < S; ++s)
                for (int64_t d = 0; d < D; ++d) {
                    Q[s * D + d] = orc_load(q, dtype, ORC_BIDX(s, d));
                    K[s * D + d] = orc_load(k, dtype, ORC_BIDX(s, d));
                    V[s * D + d] = orc_load(v, dtype, ORC_BIDX(s, d));
                    dO[s * D + d] = orc_load(dout, dtype, ORC_BIDX(s, d));
                }
            /* rows: probabilities, dP, D_i, dS, dQ */
#pragma omp parallel for schedule(dynamic, 4) num_threads(nthreads)
            for (int64_t i = 0; i < S; ++i) {
                double* prow = P + i * S;
                double* grow = dS + i * S;
                double m = -INFINITY;
                for (int64_t j = 0; j < S; ++j) {
                    if (!orc_allowed(i, j, causal, wl, wr)) {
                        prow[j] = -INFINITY;
                        continue;
                    }
                    double dot = 0.0;
                    for (int64_t d = 0; d < D; ++d) dot += Q[i * D + d] * K[j * D + d];
                    prow[j] = dot * scale;
                    if (isnan(prow[j]) || isnan(m)) m = NAN;
                    else if (prow[j] > m) m = prow[j];
                }
                double* dqrow = dq + ORC_BIDX(i, 0);
                if (m == -INFINITY) { /* no allowed key */
                    for (int64_t j = 0; j < S; ++j) prow[j] = grow[j] = 0.0;
                    for (int64_t d = 0; d < D; ++d) dqrow[d] = 0.0;
                    continue;
                }
                double l = 0.0;
                for (int64_t j = 0; j < S; ++j) {
                    prow[j] = exp(prow[j] - m) /* 0 for a masked key */;
                    l += prow[j];
                }
                for (int64_t j = 0; j < S; ++j) prow[j] = prow[j] / l;
                double Di = 0.0;
                for (int64_t j = 0; j < S; ++j) {
                    grow[j] = 0.0;
                    if (!orc_allowed(i, j, causal, wl, wr)) continue;
                    double dot = 0.0;
                    for (int64_t d = 0; d < D; ++d) dot += dO[i * D + d] * V[j * D + d];
                    grow[j] = dot; /* dP_ij */
                    Di += prow[j] * dot;
                }
                for (int64_t j = 0; j < S; ++j)
                    if (orc_allowed(i, j, causal, wl, wr)) grow[j] = prow[j] * (grow[j] - Di);
                for (int64_t d = 0; d < D; ++d) {
                    double acc = 0.0;
                    for (int64_t j = 0; j < S; ++j)
                        if (orc_allowed(i, j, causal, wl, wr)) acc += grow[j] * K[j * D + d];
                    dqrow[d] = scale * acc;
                }
            }
            /* columns: dK, dV */
#pragma omp parallel for schedule(dynamic, 4) num_threads(nthreads)
            for (int64_t j = 0; j < S; ++j) {
                double* dkrow = dk + ORC_BIDX(j, 0);
                double* dvrow = dv + ORC_BIDX(j, 0);
                for (int64_t d = 0; d < D; ++d) {
                    double ak = 0.0, av = 0.0;
                    for (int64_t i = 0; i < S; ++i) {
                        if (!orc_allowed(i, j, causal, wl, wr)) continue;
                        ak += dS[i * S + j] * Q[i * D + d];
                        av += P[i * S + j] * dO[i * D + d];
                    }
                    dkrow[d] = scale * ak;
                    dvrow[d] = av;
                }
            }
#undef ORC_BIDX
        }
    free(Q); free(K); free(V); free(dO); free(P); free(dS);
    return 0;
}

/*
 * fa_oracle_bwd_sampled -- the gradients of fa_oracle_bwd for chosen query rows
 * (dq) and chosen keys (dk, dv) of one (b, h), without the S x S matrices:
 * every row's max m_i, sum l_i and D_i = sum_j p_ij dP_ij are computed first,
 * then p_ij = exp(s_ij - m_i) / l_i and dS_ij = p_ij (dP_ij - D_i) are formed
 * again wherever a sampled row or key needs them:
 *   dQ_i = scale * sum_j dS_ij k_j,  dK_j = scale * sum_i dS_ij q_i,
 *   dV_j = sum_i p_ij dO_i.
 * Equal to fa_oracle_bwd's entries up to fp64 rounding (summation order).
 * rows[n_rows], keys[n_keys] in [0, S); dq_rows is [n_rows, D], dk_keys and
 * dv_keys [n_keys, D], fp64.  A row with no allowed key contributes nothing.
 */
int fa_oracle_bwd_sampled(const void* q, const void* k, const void* v, const void* dout,
                          int dtype, int64_t B, int64_t H, int64_t S, int64_t D, double scale,
                          int causal, int64_t wl, int64_t wr, int64_t b, int64_t h,
                          const int64_t* rows, int64_t n_rows, const int64_t* keys,
                          int64_t n_keys, double* dq_rows, double* dk_keys, double* dv_keys,
                          int nthreads) {
    if (orc_check(dtype, B, H, S, D, wl, wr)) return -1;
    if (b < 0 || b >= B || h < 0 || h >= H || n_rows < 0 || n_keys < 0) return -1;
    for (int64_t r = 0; r < n_rows; ++r)
        if (rows[r] < 0 || rows[r] >= S) return -1;
    for (int64_t c = 0; c < n_keys; ++c)
        if (keys[c] < 0 || keys[c] >= S) return -1;
    if (nthreads <= 0) nthreads = omp_get_max_threads();
    const size_t sd = (size_t)(S * D);
    double* Qh = (double*)malloc(sizeof(double) * sd);
    double* Kh = (double*)malloc(sizeof(double) * sd);
    double* Vh = (double*)malloc(sizeof(double) * sd);
    double* Gh = (double*)malloc(sizeof(double) * sd); /* dO */
    double* rmax = (double*)malloc(sizeof(double) * (size_t)S);
    double* rsum = (double*)malloc(sizeof(double) * (size_t)S);
    double* rdot = (double*)malloc(sizeof(double) * (size_t)S); /* D_i */
    if (!Qh || !Kh || !Vh || !Gh || !rmax || !rsum || !rdot) {
        free(Qh); free(Kh); free(Vh); free(Gh); free(rmax); free(rsum); free(rdot);
        return -2;
    }
#define ORC_SIDX(s_, d_) (((b * S + (s_)) * H + h) * D + (d_))
    for (int64_t t = 0; t < S; ++t)
        for (int64_t d = 0; d < D; ++d) {
            Qh[t * D + d] = orc_load(q, dtype, ORC_SIDX(t, d));
            Kh[t * D + d] = orc_load(k, dtype, ORC_SIDX(t, d));
            Vh[t * D + d] = orc_load(v, dtype, ORC_SIDX(t, d));
            Gh[t * D + d] = orc_load(dout, dtype, ORC_SIDX(t, d));
        }
#undef ORC_SIDX
    /* per-row statistics: every row when keys are sampled, else the sampled rows */
    const int64_t n_stat = n_keys > 0 ? S : n_rows;
#pragma omp parallel for schedule(dynamic, 16) num_threads(nthreads)
    for (int64_t x = 0; x < n_stat; ++x) {
        const int64_t i = n_keys > 0 ? x : rows[x];
        double m = -INFINITY;
        for (int64_t j = 0; j < S; ++j) {
            if (!orc_allowed(i, j, causal, wl, wr)) continue;
            double acc = 0.0;
            for (int64_t d = 0; d < D; ++d) acc += Qh[i * D + d] * Kh[j * D + d];
            const double sij = scale * acc;
            if (isnan(sij) || isnan(m)) m = NAN;
            else if (sij > m) m = sij;
        }
        double l = 0.0, di = 0.0;
        if (m != -INFINITY) {
            for (int64_t j = 0; j < S; ++j) {
                if (!orc_allowed(i, j, causal, wl, wr)) continue;
                double acc = 0.0, g = 0.0;
                for (int64_t d = 0; d < D; ++d) {
                    acc += Qh[i * D + d] * Kh[j * D + d];
                    g += Gh[i * D + d] * Vh[j * D + d];
                }
                const double e = exp(scale * acc - m);
                l += e;
                di += e * g; /* divided by l below: sum_j p_ij dP_ij */
            }
            di /= l;
        }
        rmax[i] = m;
        rsum[i] = l;
        rdot[i] = di;
    }
    /* p_ij and dS_ij of an allowed pair, from the row statistics */
#define ORC_P_DS(i_, j_, p_, ds_)                                                    \
    do {                                                                             \
        double a_ = 0.0, g_ = 0.0;                                                   \
        for (int64_t d_ = 0; d_ < D; ++d_) {                                         \
            a_ += Qh[(i_) * D + d_] * Kh[(j_) * D + d_];                             \
            g_ += Gh[(i_) * D + d_] * Vh[(j_) * D + d_];                             \
        }                                                                            \
        (p_) = exp(scale * a_ - rmax[i_]) / rsum[i_];                                \
        (ds_) = (p_) * (g_ - rdot[i_]);                                              \
    } while (0)
#pragma omp parallel for schedule(dynamic, 1) num_threads(nthreads)
    for (int64_t r = 0; r < n_rows; ++r) {
        const int64_t i = rows[r];
        double* out = dq_rows + r * D;
        for (int64_t d = 0; d < D; ++d) out[d] = 0.0;
        if (rmax[i] == -INFINITY) continue;
        for (int64_t j = 0; j < S; ++j) {
            if (!orc_allowed(i, j, causal, wl, wr)) continue;
            double p, ds;
            ORC_P_DS(i, j, p, ds);
            for (int64_t d = 0; d < D; ++d) out[d] += ds * Kh[j * D + d];
        }
        for (int64_t d = 0; d < D; ++d) out[d] *= scale;
    }
#pragma omp parallel for schedule(dynamic, 1) num_threads(nthreads)
    for (int64_t c = 0; c < n_keys; ++c) {
        const int64_t j = keys[c];
        double* ok = dk_keys + c * D;
        double* ov = dv_keys + c * D;
        for (int64_t d = 0; d < D; ++d) ok[d] = ov[d] = 0.0;
        for (int64_t i = 0; i < S; ++i) {
            if (!orc_allowed(i, j, causal, wl, wr) || rmax[i] == -INFINITY) continue;
            double p, ds;
            ORC_P_DS(i, j, p, ds);
            for (int64_t d = 0; d < D; ++d) {
                ok[d] += ds * Qh[i * D + d];
                ov[d] += p * Gh[i * D + d];
            }
        }
        for (int64_t d = 0; d < D; ++d) ok[d] *= scale;
    }
#undef ORC_P_DS
    free(Qh); free(Kh); free(Vh); free(Gh); free(rmax); free(rsum); free(rdot);
    return 0;
}

/*
 * fa_oracle_fwd_kvcache -- attention of S_q new queries against a key/value
 * cache, as at inference ("FlashAttention技术解析：加速GPT训练的核心优化",
 * section 5, names FlashDecoding, the variant of the method for the KV cache of
 * inference; "突破大模型训练瓶颈：Flash-Attention编译优化与内存占用解决方案",
 * section 总结与最佳实践, names the call flash_attn_with_kvcache).  The pages
 * give no more, and the plainest reading is taken:
 *  - sequence b's keys and values are the first L_b = seqlens[b] rows of the
 *    cache, the new tokens' own keys and values included (rows past L_b are
 *    never read);
 *  - its S_q queries are the last S_q positions of that sequence, so query i
 *    sits at position  p = L_b - S_q + i;
 *  - key j (0 <= j < L_b) is allowed for it when allowed(p, j), the causal and
 *    window rules of the dense definition applied to positions.
 * Then, as before, s_pj = scale * q_i . k_j over the allowed keys,
 * O_i = softmax(s) V and LSE_i = ln sum_j exp(s_pj).  A row with no allowed
 * key (p < 0 under the causal mask, or L_b = 0) gets O = 0 and LSE = -inf.
 * With S_q = L_b = S_k every row sits at its own index and this is
 * fa_oracle_fwd.
 *
 * q, out: [B, S_q, H, D]; k, v: [B, S_k, H, D], S_k the cache's capacity
 * (0 <= L_b <= S_k); lse: [B, H, S_q].  Outputs fp64.  Each (b, h) scores
 * matrix (S_q x L_b) is materialised; rows run over nthreads threads.
 */
int fa_oracle_fwd_kvcache(const void* q, const void* k, const void* v, int dtype, int64_t B,
                          int64_t H, int64_t S_q, int64_t S_k, int64_t D, double scale,
                          int causal, int64_t wl, int64_t wr, const int64_t* seqlens,
                          double* out, double* lse, int nthreads) {
    if (orc_check(dtype, B, H, S_q, D, wl, wr) || S_k < 1 || !seqlens) return -1;
    for (int64_t b = 0; b < B; ++b)
        if (seqlens[b] < 0 || seqlens[b] > S_k) return -1;
    if (nthreads <= 0) nthreads = omp_get_max_threads();
    for (int64_t b = 0; b < B; ++b) {
        const int64_t L = seqlens[b];
        for (int64_t h = 0; h < H; ++h) {
            double* Qc = (double*)malloc(sizeof(double) * (size_t)(S_q * D));
            double* Kc = (double*)malloc(sizeof(double) * (size_t)((L > 0 ? L : 1) * D));
            double* Vc = (double*)malloc(sizeof(double) * (size_t)((L > 0 ? L : 1) * D));
            double* Pc = (double*)malloc(sizeof(double) * (size_t)(S_q * (L > 0 ? L : 1)));
            if (!Qc || !Kc || !Vc || !Pc) {
                free(Qc); free(Kc); free(Vc); free(Pc);
                return -2;
            }
            for (int64_t r = 0; r < S_q; ++r)
                for (int64_t d = 0; d < D; ++d)
                    Qc[r * D + d] = orc_load(q, dtype, ((b * S_q + r) * H + h) * D + d);
            for (int64_t j = 0; j < L; ++j)
                for (int64_t d = 0; d < D; ++d) {
                    Kc[j * D + d] = orc_load(k, dtype, ((b * S_k + j) * H + h) * D + d);
                    Vc[j * D + d] = orc_load(v, dtype, ((b * S_k + j) * H + h) * D + d);
                }
#pragma omp parallel for schedule(dynamic, 4) num_threads(nthreads)
            for (int64_t r = 0; r < S_q; ++r) {
                const int64_t p = L - S_q + r; /* the query's position in its sequence */
                double* srow = Pc + r * (L > 0 ? L : 1);
                double* orow = out + ((b * S_q + r) * H + h) * D;
                double* lrow = lse + (b * H + h) * S_q + r;
                /* 1. scores of the allowed keys; -inf elsewhere */
                for (int64_t j = 0; j < L; ++j) {
                    if (!orc_allowed(p, j, causal, wl, wr)) {
                        srow[j] = -INFINITY;
                        continue;
                    }
                    double dot = 0.0;
                    for (int64_t d = 0; d < D; ++d) dot += Qc[r * D + d] * Kc[j * D + d];
                    srow[j] = scale * dot;
                }
                /* 2. row max (a NaN anywhere makes it NaN) */
                double m = -INFINITY;
                for (int64_t j = 0; j < L; ++j) {
                    if (isnan(srow[j])) {
                        m = srow[j];
                        break;
                    }
                    if (srow[j] > m) m = srow[j];
                }
                if (m == -INFINITY) { /* no allowed key */
                    for (int64_t d = 0; d < D; ++d) orow[d] = 0.0;
                    *lrow = -INFINITY;
                    continue;
                }
                /* 3. softmax */
                double l = 0.0;
                for (int64_t j = 0; j < L; ++j) {
                    srow[j] = exp(srow[j] - m);
                    l += srow[j];
                }
                for (int64_t j = 0; j < L; ++j) srow[j] /= l;
                /* 4. O = P V over the allowed keys */
                for (int64_t d = 0; d < D; ++d) orow[d] = 0.0;
                for (int64_t j = 0; j < L; ++j) {
                    if (!orc_allowed(p, j, causal, wl, wr)) continue; /* p = 0 exactly */
                    for (int64_t d = 0; d < D; ++d) orow[d] += srow[j] * Vc[j * D + d];
                }
                *lrow = m + log(l);
            }
            free(Qc); free(Kc); free(Vc); free(Pc);
        }
    }
    return 0;
}
