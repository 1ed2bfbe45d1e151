// fa_api.hip -- the C ABI of libfa_mi355x (declared in include/fa_mi355x.h):
// argument validation, status strings, the host view of the tile schedule and
// the dispatch to the gfx950 kernels.  No allocation, no global state.
#include <hip/hip_runtime.h>

#include <cfloat>
#include <cmath>
#include <cstdint>
#include <mutex>

#include "fa_launch.h"
#include "fa_mi355x.h"
#include "fa_schedule.h"

#define FA_API extern "C" __attribute__((visibility("default")))

namespace {

bool mul_ok(int64_t a, int64_t b, int64_t* r) { return !__builtin_mul_overflow(a, b, r); }

// [p, p + n) and [q, q + m) overlap (byte ranges)
bool overlaps(const void* p, int64_t n, const void* q, int64_t m) {
    const uintptr_t a = (uintptr_t)p, b = (uintptr_t)q;
    return a < b + (uintptr_t)m && b < a + (uintptr_t)n;
}

int64_t elem_size(int dtype) { return dtype == fa::kDtypeFp32 ? 4 : 2; }

// Shape / window / dtype checks shared by the entry points; *tensor_bytes and
// *lse_bytes are set on success.  Head dimensions: any multiple of 16 from 16
// to d_max (other than 64, 128 and 256 the kernels run the next of those up
// with zero columns): 256 for the bf16 / fp16 forward, 128 for fp32 inputs,
// the backward and the KV-cache forward (which reject fp32 by dtype).
constexpr int64_t kFwdMaxD = 256, kBwdMaxD = 128, kKvcMaxD = 128, kFp32MaxD = 128;
int check_problem(int64_t B, int64_t H, int64_t S, int64_t D, int causal, int64_t wl, int64_t wr,
                  int dtype, int64_t* tensor_bytes, int64_t* lse_bytes, int64_t d_max = kFwdMaxD) {
    if (dtype != FA_DTYPE_FP32 && dtype != FA_DTYPE_FP16 && dtype != FA_DTYPE_BF16)
        return FA_ERR_DTYPE;
    if (B < 1 || H < 1 || S < 1) return FA_ERR_SHAPE;
    if (dtype == FA_DTYPE_FP32 && d_max > kFp32MaxD) d_max = kFp32MaxD;
    if (d_max == 0) {
        if (D != 64 && D != 128) return FA_ERR_HEAD_DIM;
    } else if (D < 16 || D > d_max || D % 16 != 0) {
        return FA_ERR_HEAD_DIM;
    }
    if ((causal != 0 && causal != 1) || wl < -1 || wr < -1) return FA_ERR_WINDOW;
    // the kernels index rows with 32-bit S, B, H and launch B*H*ceil(S/128)
    // workgroups of 256 threads (grid limit: 2^32 - 1 work-items)
    if (S > INT32_MAX || B > INT32_MAX || H > INT32_MAX) return FA_ERR_SHAPE;
    // the smallest Q tile of any configuration bounds the grid
    const int64_t bm = 4 * 32;
    const int64_t n_qt = (S + bm - 1) / bm;
    int64_t n_wg, t;
    if (!mul_ok(B, H, &t) || !mul_ok(t, n_qt, &n_wg) || n_wg > (int64_t)(UINT32_MAX / 256))
        return FA_ERR_SHAPE;
    int64_t elems, rows;
    if (!mul_ok(B, S, &rows) || !mul_ok(rows, H, &t) || !mul_ok(t, D, &elems) ||
        !mul_ok(elems, elem_size(dtype), tensor_bytes))
        return FA_ERR_SHAPE;
    if (!mul_ok(rows, H, &t) || !mul_ok(t, 4, lse_bytes)) return FA_ERR_SHAPE;
    // the kernels address the rows of one 64-row K/V tile with 32-bit byte
    // offsets (row stride H * D elements)
    if (H * D * elem_size(dtype) * 64 > (int64_t)INT32_MAX) return FA_ERR_SHAPE;
    return FA_OK;
}

}  // namespace

FA_API const char* fa_status_string(int status) {
    switch (status) {
    case FA_OK: return "ok";
    case FA_ERR_NULL: return "a required pointer is NULL";
    case FA_ERR_SHAPE: return "B, H and S must be >= 1 and the sizes must fit the index ranges";
    case FA_ERR_HEAD_DIM:
        return "unsupported head dimension D (a multiple of 16 from 16 to 256 for the bf16 / fp16 "
               "forward, to 128 for fp32 inputs, fa_bwd and fa_fwd_kvcache)";
    case FA_ERR_WINDOW: return "causal must be 0 or 1 and window bounds must be >= -1";
    case FA_ERR_DTYPE: return "dtype must be FA_DTYPE_FP32, FA_DTYPE_FP16 or FA_DTYPE_BF16";
    case FA_ERR_SCALE: return "scale must be finite and >= 0";
    case FA_ERR_ALIGN: return "q, k, v, out must be 16-byte aligned and lse 4-byte aligned";
    case FA_ERR_ALIAS: return "out and lse must not overlap the inputs or each other";
    case FA_ERR_HIP: return "the HIP kernel launch failed";
    case FA_ERR_WORKSPACE:
        return "the workspace is NULL, too small, not 16-byte aligned or overlaps an input or "
               "output";
    case FA_ERR_SPLITS:
        return "n_splits must be in [1, FA_MAX_SPLITS] (fa_fwd_kvcache: [1, FA_MAX_KV_SPLITS])";
    case FA_ERR_BLOCKMASK:
        return "block_m must be a positive multiple of 128, block_n of 64, and n_mask 1, H or B*H";
    case FA_ERR_PAGES:
        return "page_size must be a positive multiple of 64, num_pages >= 1, the block table as "
               "wide as ceil(S / page_size), and the pools must fit the index ranges";
    case FA_ERR_SCRATCH:
        return "the split partials need more than the library's static scratch buffer "
               "(FA_NOALLOC_SCRATCH_BYTES); use fa_fwd_splitkv with a workspace";
    default: return "unknown status";
    }
}

FA_API int fa_fwd_check_args(const void* q, const void* k, const void* v, const void* out,
                             const float* lse, int64_t B, int64_t H, int64_t S, int64_t D,
                             float scale, int causal, int64_t window_left, int64_t window_right,
                             int dtype) {
    if (!q || !k || !v || !out || !lse) return FA_ERR_NULL;
    int64_t nbytes = 0, lbytes = 0;
    const int rc = check_problem(B, H, S, D, causal, window_left, window_right, dtype, &nbytes,
                                 &lbytes);
    if (rc != FA_OK) return rc;
    if (!std::isfinite(scale) || scale < 0.f) return FA_ERR_SCALE;
    if (((uintptr_t)q | (uintptr_t)k | (uintptr_t)v | (uintptr_t)out) & 15u) return FA_ERR_ALIGN;
    if ((uintptr_t)lse & 3u) return FA_ERR_ALIGN;
    const void* ins[3] = {q, k, v};
    for (const void* in : ins)
        if (overlaps(out, nbytes, in, nbytes) || overlaps(lse, lbytes, in, nbytes))
            return FA_ERR_ALIAS;
    if (overlaps(out, nbytes, lse, lbytes)) return FA_ERR_ALIAS;
    return FA_OK;
}

namespace {

// Launch arguments of a validated problem (pointers may be NULL for queries).
fa::LaunchArgs make_args(const void* q, const void* k, const void* v, void* out, float* lse,
                         int64_t B, int64_t H, int64_t S, int64_t D, float scale, int causal,
                         int64_t window_left, int64_t window_right, int dtype, void* stream) {
    fa::LaunchArgs a;
    a.q = q;
    a.k = k;
    a.v = v;
    a.out = out;
    a.lse = lse;
    a.B = B;
    a.H = H;
    a.S = S;
    a.D = D;
    // exp(scale * s) = exp2(scale * log2(e) * s): one FMA feeds v_exp_f32.
    // c is kept >= FLT_MIN so that a masked score -inf scales to -inf (weight
    // exactly 0) even for scale = 0; a finite score s then scales to at most
    // |s| * 1.2e-38, whose weight exp2(.) rounds to exactly 1 -- the uniform
    // weights scale = 0 asks for.
    const float c = (float)((double)scale * 1.4426950408889634);
    a.c = c < FLT_MIN ? FLT_MIN : c;
    a.causal = causal;
    a.wl = window_left >= S ? -1 : window_left;  // a window reaching past S is unbounded
    a.wr = window_right >= S ? -1 : window_right;
    a.dtype = dtype;
    a.stream = (hipStream_t)stream;
    return a;
}

// Bytes of fp32 partial O and LSE for n_splits parts (0 when nothing is split).
int64_t split_workspace_bytes(int64_t B, int64_t H, int64_t S, int64_t D, int dtype,
                              int64_t n_splits) {
    if (n_splits <= 1 || dtype == FA_DTYPE_FP32) return 0;
    return n_splits * B * H * S * (D + 1) * 4;
}

}  // namespace

FA_API int fa_fwd(const void* q, const void* k, const void* v, void* out, float* lse, int64_t B,
                  int64_t H, int64_t S, int64_t D, float scale, int causal, int64_t window_left,
                  int64_t window_right, int dtype, void* stream) {
    const int rc = fa_fwd_check_args(q, k, v, out, lse, B, H, S, D, scale, causal, window_left,
                                     window_right, dtype);
    if (rc != FA_OK) return rc;
    const fa::LaunchArgs a = make_args(q, k, v, out, lse, B, H, S, D, scale, causal, window_left,
                                       window_right, dtype, stream);
    const hipError_t e = fa::launch_fwd(a);
    return e == hipSuccess ? FA_OK : FA_ERR_HIP;
}

FA_API int fa_fwd_splitkv_workspace_size(int64_t B, int64_t H, int64_t S, int64_t D, int dtype,
                                         int64_t n_splits, int64_t* bytes) {
    if (!bytes) return FA_ERR_NULL;
    int64_t nbytes, lbytes;
    const int rc = check_problem(B, H, S, D, 0, -1, -1, dtype, &nbytes, &lbytes);
    if (rc != FA_OK) return rc;
    if (n_splits < 1 || n_splits > FA_MAX_SPLITS) return FA_ERR_SPLITS;
    // n_splits * (B*H*S) * (D + 1) * 4 fits: B*H*S*D*e is checked to fit int64, and
    // n_splits * 4 * (D + 1) / e <= 16 * 4 * 129 / 2
    int64_t rows, t, r;
    if (!mul_ok(B, H, &t) || !mul_ok(t, S, &rows) || !mul_ok(rows, n_splits * (D + 1) * 4, &r))
        return FA_ERR_SHAPE;
    *bytes = split_workspace_bytes(B, H, S, D, dtype, n_splits);
    return FA_OK;
}

FA_API int fa_fwd_splitkv_auto_splits(int64_t B, int64_t H, int64_t S, int64_t D, int causal,
                                      int64_t window_left, int64_t window_right, int dtype,
                                      int64_t* n_splits) {
    if (!n_splits) return FA_ERR_NULL;
    int64_t nbytes, lbytes;
    const int rc = check_problem(B, H, S, D, causal, window_left, window_right, dtype, &nbytes,
                                 &lbytes);
    if (rc != FA_OK) return rc;
    const fa::LaunchArgs a = make_args(nullptr, nullptr, nullptr, nullptr, nullptr, B, H, S, D, 1.f,
                                       causal, window_left, window_right, dtype, nullptr);
    *n_splits = fa::auto_splits(a);
    return FA_OK;
}

FA_API int fa_fwd_splitkv(const void* q, const void* k, const void* v, void* out, float* lse,
                          int64_t B, int64_t H, int64_t S, int64_t D, float scale, int causal,
                          int64_t window_left, int64_t window_right, int dtype, int64_t n_splits,
                          void* workspace, int64_t workspace_bytes, void* stream) {
    int rc = fa_fwd_check_args(q, k, v, out, lse, B, H, S, D, scale, causal, window_left,
                               window_right, dtype);
    if (rc != FA_OK) return rc;
    int64_t need = 0;
    rc = fa_fwd_splitkv_workspace_size(B, H, S, D, dtype, n_splits, &need);
    if (rc != FA_OK) return rc;
    fa::LaunchArgs a = make_args(q, k, v, out, lse, B, H, S, D, scale, causal, window_left,
                                 window_right, dtype, stream);
    if (need > 0) {
        // the split grid: Q tiles x parts workgroups of 256 threads
        const int64_t bm = fa::q_tile_rows(dtype, D, S, a.wl, a.wr);
        int64_t n_wg;
        if (!mul_ok(B * H, (S + bm - 1) / bm, &n_wg) || !mul_ok(n_wg, n_splits, &n_wg) ||
            n_wg > (int64_t)(UINT32_MAX / 256))
            return FA_ERR_SHAPE;
        if (!workspace || workspace_bytes < need || ((uintptr_t)workspace & 15u))
            return FA_ERR_WORKSPACE;
        int64_t nbytes = 0, lbytes = 0;
        (void)check_problem(B, H, S, D, causal, window_left, window_right, dtype, &nbytes, &lbytes);
        const void* others[5] = {q, k, v, out, lse};
        const int64_t sizes[5] = {nbytes, nbytes, nbytes, nbytes, lbytes};
        for (int i = 0; i < 5; ++i)
            if (overlaps(workspace, need, others[i], sizes[i])) return FA_ERR_WORKSPACE;
        const int64_t rows = B * H * S;
        a.n_splits = (int)n_splits;
        a.part_o = (float*)workspace;
        a.part_lse = (float*)workspace + n_splits * rows * D;
    }
    const hipError_t e = fa::launch_fwd(a);
    return e == hipSuccess ? FA_OK : FA_ERR_HIP;
}

FA_API int fa_fwd_workgroup_tile(int64_t B, int64_t H, int64_t S, int64_t D, int dtype, int causal,
                                 int64_t window_left, int64_t window_right, int64_t wg, int64_t* bh,
                                 int64_t* q_tile) {
    if (!bh || !q_tile) return FA_ERR_NULL;
    int64_t nbytes, lbytes;
    const int rc = check_problem(B, H, S, D, causal, window_left, window_right, dtype, &nbytes,
                                 &lbytes);
    if (rc != FA_OK) return rc;
    const int64_t wlc = window_left >= S ? -1 : window_left;
    const int64_t wrc = window_right >= S ? -1 : window_right;
    const int64_t BM = fa::q_tile_rows(dtype, D, S, wlc, wrc);
    const int64_t nq = (S + BM - 1) / BM;
    if (wg < 0 || wg >= B * H * nq) return FA_ERR_SHAPE;
    uint32_t r_bh, r_qt;
    const int64_t esz = dtype == FA_DTYPE_FP32 ? 4 : 2;
    fa::workgroup_tile((uint32_t)wg, (uint32_t)(B * H), (uint32_t)nq, causal != 0,
                       fa::snake_launch(B * H, S, fa::kernel_head_dim(D), esz), &r_bh, &r_qt);
    *bh = r_bh;
    *q_tile = r_qt;
    return FA_OK;
}

FA_API int fa_fwd_launch_order(int64_t B, int64_t H, int64_t S, int64_t D, int dtype, int causal,
                               int64_t window_left, int64_t window_right, int64_t n_cus,
                               int64_t wg, int64_t* bh, int64_t* q_tile,
                               int64_t* first_dynamic) {
    if (!bh || !q_tile || !first_dynamic) return FA_ERR_NULL;
    if (n_cus < 1) return FA_ERR_SHAPE;
    int64_t nbytes, lbytes;
    const int rc = check_problem(B, H, S, D, causal, window_left, window_right, dtype, &nbytes,
                                 &lbytes);
    if (rc != FA_OK) return rc;
    const int64_t wlc = window_left >= S ? -1 : window_left;
    const int64_t wrc = window_right >= S ? -1 : window_right;
    const int64_t BM = fa::q_tile_rows(dtype, D, S, wlc, wrc);
    const int64_t nq = (S + BM - 1) / BM, n_bh = B * H;
    if (wg < 0 || wg >= n_bh * nq) return FA_ERR_SHAPE;
    int64_t first = -1;
    if (dtype != FA_DTYPE_FP32)  // the fp32 kernel keeps the static order
        first = fa::dyn_first_position(fa::MaskSpec{S, causal, wlc, wrc}, n_bh, BM,
                                       fa::kv_tile_keys(dtype, D, S, wlc, wrc),
                                       fa::resident_wgs_per_cu(D) * n_cus);
    *first_dynamic = first;
    if (first < 0)
        return fa_fwd_workgroup_tile(B, H, S, D, dtype, causal, window_left, window_right, wg, bh,
                                     q_tile);
    const uint32_t pos =
        wg < first ? fa::dyn_static_position((uint32_t)wg, (uint32_t)n_bh, (uint32_t)first,
                                             fa::snake_launch(n_bh, S, fa::kernel_head_dim(D), 2))
                   : (uint32_t)wg;
    uint32_t r_bh, r_qt;
    fa::dyn_list_tile(pos, (uint32_t)n_bh, (uint32_t)nq, &r_bh, &r_qt);
    *bh = r_bh;
    *q_tile = r_qt;
    return FA_OK;
}

FA_API int fa_fwd_splitkv_workgroup_tile(int64_t B, int64_t H, int64_t S, int64_t D, int dtype,
                                         int causal, int64_t window_left, int64_t window_right,
                                         int64_t n_splits, int64_t wg, int64_t* bh,
                                         int64_t* q_tile, int64_t* part) {
    if (!part) return FA_ERR_NULL;
    if (n_splits < 1 || n_splits > FA_MAX_SPLITS) return FA_ERR_SPLITS;
    if (n_splits == 1 || dtype == FA_DTYPE_FP32) {  // the unsplit launch
        *part = 0;
        return fa_fwd_workgroup_tile(B, H, S, D, dtype, causal, window_left, window_right, wg, bh,
                                     q_tile);
    }
    if (!bh || !q_tile) return FA_ERR_NULL;
    int64_t nbytes, lbytes;
    const int rc = check_problem(B, H, S, D, causal, window_left, window_right, dtype, &nbytes,
                                 &lbytes);
    if (rc != FA_OK) return rc;
    const int64_t wlc = window_left >= S ? -1 : window_left;
    const int64_t wrc = window_right >= S ? -1 : window_right;
    const int64_t BM = fa::q_tile_rows(dtype, D, S, wlc, wrc);
    const int64_t nq = (S + BM - 1) / BM;
    if (wg < 0 || wg >= B * H * nq * n_splits) return FA_ERR_SHAPE;
    uint32_t r_bh, r_qt, r_part;
    fa::workgroup_tile_part((uint32_t)wg, (uint32_t)(B * H), (uint32_t)nq, (uint32_t)n_splits,
                            causal != 0, &r_bh, &r_qt, &r_part);
    *bh = r_bh;
    *q_tile = r_qt;
    *part = r_part;
    return FA_OK;
}

FA_API int fa_fwd_tile_schedule(int64_t S, int64_t D, int dtype, int causal, int64_t window_left,
                                int64_t window_right, int64_t q_tile, int64_t* bm, int64_t* bn,
                                int64_t* n_q_tiles, int64_t* kt_begin, int64_t* kt_end,
                                uint8_t* needs_mask, int64_t max_tiles) {
    if (!bm || !bn || !n_q_tiles || !kt_begin || !kt_end) return FA_ERR_NULL;
    int64_t nbytes, lbytes;
    const int rc = check_problem(1, 1, S, D, causal, window_left, window_right, dtype, &nbytes,
                                 &lbytes);
    if (rc != FA_OK) return rc;
    const int64_t wlc = window_left >= S ? -1 : window_left;
    const int64_t wrc = window_right >= S ? -1 : window_right;
    const int64_t BM = fa::q_tile_rows(dtype, D, S, wlc, wrc), BN = fa::kv_tile_keys(dtype, D, S, wlc, wrc);
    const int64_t nq = (S + BM - 1) / BM;
    if (q_tile < 0 || q_tile >= nq) return FA_ERR_SHAPE;
    const fa::MaskSpec m{S, causal, wlc, wrc};
    int64_t t0, t1;
    fa::q_tile_kv_range(m, q_tile, BM, BN, &t0, &t1);
    *bm = BM;
    *bn = BN;
    *n_q_tiles = nq;
    *kt_begin = t0;
    *kt_end = t1;
    if (needs_mask) {
        if (max_tiles < t1 - t0) return FA_ERR_SHAPE;
        const int64_t r0 = q_tile * BM;
        if (dtype == FA_DTYPE_FP32) {  // the fp32 kernel decides per tile
            for (int64_t t = t0; t < t1; ++t)
                needs_mask[t - t0] = fa::tile_needs_mask(m, r0, r0 + BM - 1, t * BN, BN) ? 1 : 0;
        } else {  // the bf16/fp16 kernel runs [ki0, ki1) without the mask
            int64_t i0, i1;
            fa::q_tile_interior_range(m, r0, BM, BN, t0, t1, &i0, &i1);
            for (int64_t t = t0; t < t1; ++t) needs_mask[t - t0] = (t < i0 || t >= i1) ? 1 : 0;
        }
    }
    return FA_OK;
}

FA_API int fa_bwd_workspace_size(int64_t B, int64_t H, int64_t S, int64_t D, int dtype,
                                 int64_t* bytes) {
    if (!bytes) return FA_ERR_NULL;
    int64_t nbytes, lbytes;
    const int rc = check_problem(B, H, S, D, 0, -1, -1, dtype, &nbytes, &lbytes, kBwdMaxD);
    if (rc != FA_OK) return rc;
    if (dtype == FA_DTYPE_FP32) return FA_ERR_DTYPE;
    *bytes = lbytes + fa::kBwdCounterBytes;  // fp32 [B, H, S] (the size of lse), two counters
    return FA_OK;
}

FA_API int fa_bwd(const void* q, const void* k, const void* v, const void* out, const float* lse,
                  const void* dout, void* dq, void* dk, void* dv, int64_t B, int64_t H, int64_t S,
                  int64_t D, float scale, int causal, int64_t window_left, int64_t window_right,
                  int dtype, void* workspace, int64_t workspace_bytes, void* stream) {
    if (!q || !k || !v || !out || !lse || !dout || !dq || !dk || !dv) return FA_ERR_NULL;
    int64_t nbytes = 0, lbytes = 0;
    int rc = check_problem(B, H, S, D, causal, window_left, window_right, dtype, &nbytes, &lbytes,
                           kBwdMaxD);
    if (rc != FA_OK) return rc;
    if (dtype == FA_DTYPE_FP32) return FA_ERR_DTYPE;
    if (!std::isfinite(scale) || scale < 0.f) return FA_ERR_SCALE;
    const void* tens[8] = {q, k, v, out, dout, dq, dk, dv};
    for (const void* t : tens)
        if ((uintptr_t)t & 15u) return FA_ERR_ALIGN;
    if ((uintptr_t)lse & 3u) return FA_ERR_ALIGN;
    const void* ins[6] = {q, k, v, out, dout, lse};
    const int64_t in_bytes[6] = {nbytes, nbytes, nbytes, nbytes, nbytes, lbytes};
    void* outs[3] = {dq, dk, dv};
    for (int o = 0; o < 3; ++o) {
        for (int i = 0; i < 6; ++i)
            if (overlaps(outs[o], nbytes, ins[i], in_bytes[i])) return FA_ERR_ALIAS;
        for (int p = o + 1; p < 3; ++p)
            if (overlaps(outs[o], nbytes, outs[p], nbytes)) return FA_ERR_ALIAS;
    }
    const int64_t wbytes = lbytes + fa::kBwdCounterBytes;
    if (!workspace || workspace_bytes < wbytes || ((uintptr_t)workspace & 15u))
        return FA_ERR_WORKSPACE;
    for (int i = 0; i < 6; ++i)
        if (overlaps(workspace, wbytes, ins[i], in_bytes[i])) return FA_ERR_WORKSPACE;
    for (int o = 0; o < 3; ++o)
        if (overlaps(workspace, wbytes, outs[o], nbytes)) return FA_ERR_WORKSPACE;
    const fa::LaunchArgs f = make_args(q, k, v, nullptr, nullptr, B, H, S, D, scale, causal,
                                       window_left, window_right, dtype, stream);
    fa::BwdArgs a;
    a.q = q;
    a.k = k;
    a.v = v;
    a.out = out;
    a.lse = lse;
    a.dout = dout;
    a.dq = dq;
    a.dk = dk;
    a.dv = dv;
    a.di = (float*)workspace;
    a.counters = (unsigned*)((char*)workspace + lbytes);
    a.B = B;
    a.H = H;
    a.S = S;
    a.D = D;
    a.c = f.c;
    a.scale = scale;
    a.causal = causal;
    a.wl = f.wl;
    a.wr = f.wr;
    a.dtype = dtype;
    a.stream = (hipStream_t)stream;
    const hipError_t e = fa::launch_bwd(a);
    return e == hipSuccess ? FA_OK : FA_ERR_HIP;
}

namespace {

// Bytes of a [n_mask, ceil(S / block_m), ceil(S / block_n)] block mask, or -1
// for block sizes / head counts fa_fwd_blocksparse does not take.
int64_t block_mask_bytes(int64_t B, int64_t H, int64_t S, int64_t n_mask, int64_t block_m,
                         int64_t block_n) {
    if (block_m < 128 || block_m % 128 != 0 || block_n < 64 || block_n % 64 != 0) return -1;
    if (n_mask != 1 && n_mask != H && n_mask != B * H) return -1;
    int64_t t, r;
    if (!mul_ok(n_mask, (S + block_m - 1) / block_m, &t) ||
        !mul_ok(t, (S + block_n - 1) / block_n, &r))
        return -1;
    return r;
}

}  // namespace

FA_API int fa_fwd_blocksparse_workspace_size(int64_t B, int64_t H, int64_t S, int64_t D, int dtype,
                                             int64_t n_mask, int64_t* bytes) {
    if (!bytes) return FA_ERR_NULL;
    int64_t nbytes, lbytes;
    const int rc = check_problem(B, H, S, D, 0, -1, -1, dtype, &nbytes, &lbytes);
    if (rc != FA_OK) return rc;
    if (n_mask != 1 && n_mask != H && n_mask != B * H) return FA_ERR_BLOCKMASK;
    // n_mask * ceil(S/128) rows of 4 + ceil(S/64) ints: below 2 * B*H*S*4 + small
    *bytes = fa::blocksparse_lut_bytes(dtype, D, S, n_mask);
    return FA_OK;
}

FA_API int fa_fwd_blocksparse(const void* q, const void* k, const void* v, void* out, float* lse,
                              int64_t B, int64_t H, int64_t S, int64_t D, float scale, int causal,
                              int64_t window_left, int64_t window_right, int dtype,
                              const uint8_t* block_mask, int64_t n_mask, int64_t block_m,
                              int64_t block_n, void* workspace, int64_t workspace_bytes,
                              void* stream) {
    int rc = fa_fwd_check_args(q, k, v, out, lse, B, H, S, D, scale, causal, window_left,
                               window_right, dtype);
    if (rc != FA_OK) return rc;
    if (!block_mask) return FA_ERR_NULL;
    const int64_t mbytes = block_mask_bytes(B, H, S, n_mask, block_m, block_n);
    if (mbytes < 0) return FA_ERR_BLOCKMASK;
    int64_t need = 0;
    rc = fa_fwd_blocksparse_workspace_size(B, H, S, D, dtype, n_mask, &need);
    if (rc != FA_OK) return rc;
    int64_t nbytes = 0, lbytes = 0;
    (void)check_problem(B, H, S, D, causal, window_left, window_right, dtype, &nbytes, &lbytes);
    if (overlaps(out, nbytes, block_mask, mbytes) || overlaps(lse, lbytes, block_mask, mbytes))
        return FA_ERR_ALIAS;
    if (need > 0) {
        if (!workspace || workspace_bytes < need || ((uintptr_t)workspace & 15u))
            return FA_ERR_WORKSPACE;
        const void* others[6] = {q, k, v, out, lse, block_mask};
        const int64_t sizes[6] = {nbytes, nbytes, nbytes, nbytes, lbytes, mbytes};
        for (int i = 0; i < 6; ++i)
            if (overlaps(workspace, need, others[i], sizes[i])) return FA_ERR_WORKSPACE;
    }
    fa::LaunchArgs a = make_args(q, k, v, out, lse, B, H, S, D, scale, causal, window_left,
                                 window_right, dtype, stream);
    a.bmask = block_mask;
    a.n_mask = n_mask;
    a.block_m = block_m;
    a.block_n = block_n;
    a.lut = (int*)workspace;
    const hipError_t e = fa::launch_fwd(a);
    return e == hipSuccess ? FA_OK : FA_ERR_HIP;
}

FA_API int fa_fwd_paged(const void* q, const void* k_pages, const void* v_pages,
                        const int32_t* block_table, void* out, float* lse, int64_t B, int64_t H,
                        int64_t S, int64_t D, float scale, int causal, int64_t window_left,
                        int64_t window_right, int dtype, int64_t num_pages, int64_t page_size,
                        int64_t table_stride, int64_t n_splits, void* workspace,
                        int64_t workspace_bytes, void* stream) {
    if (!q || !k_pages || !v_pages || !block_table || !out || !lse) return FA_ERR_NULL;
    int64_t nbytes = 0, lbytes = 0;
    int rc = check_problem(B, H, S, D, causal, window_left, window_right, dtype, &nbytes, &lbytes);
    if (rc != FA_OK) return rc;
    if (!std::isfinite(scale) || scale < 0.f) return FA_ERR_SCALE;
    // page geometry: a page holds whole 64-key tiles; the kernels index pages
    // and rows with 32-bit values and pool rows with 64-bit offsets
    if (page_size < 64 || page_size % 64 != 0 || page_size > INT32_MAX || num_pages < 1 ||
        num_pages > INT32_MAX || table_stride < (S + page_size - 1) / page_size ||
        table_stride > INT32_MAX)
        return FA_ERR_PAGES;
    int64_t t, pool_bytes, table_bytes;
    if (!mul_ok(num_pages, page_size, &t) || !mul_ok(t, H * D * elem_size(dtype), &pool_bytes) ||
        !mul_ok(B, table_stride, &t) || !mul_ok(t, 4, &table_bytes))
        return FA_ERR_PAGES;
    if (((uintptr_t)q | (uintptr_t)k_pages | (uintptr_t)v_pages | (uintptr_t)out) & 15u)
        return FA_ERR_ALIGN;
    if (((uintptr_t)lse | (uintptr_t)block_table) & 3u) return FA_ERR_ALIGN;
    const void* ins[4] = {q, k_pages, v_pages, block_table};
    const int64_t in_bytes[4] = {nbytes, pool_bytes, pool_bytes, table_bytes};
    for (int i = 0; i < 4; ++i)
        if (overlaps(out, nbytes, ins[i], in_bytes[i]) || overlaps(lse, lbytes, ins[i], in_bytes[i]))
            return FA_ERR_ALIAS;
    if (overlaps(out, nbytes, lse, lbytes)) return FA_ERR_ALIAS;
    int64_t need = 0;
    rc = fa_fwd_splitkv_workspace_size(B, H, S, D, dtype, n_splits, &need);
    if (rc != FA_OK) return rc;
    fa::LaunchArgs a = make_args(q, k_pages, v_pages, out, lse, B, H, S, D, scale, causal,
                                 window_left, window_right, dtype, stream);
    a.pg_table = block_table;
    a.pg_stride = table_stride;
    a.pg_rows = page_size;
    a.pg_count = num_pages;
    if (need > 0) {
        const int64_t bm = fa::q_tile_rows(dtype, D, S, a.wl, a.wr);
        int64_t n_wg;
        if (!mul_ok(B * H, (S + bm - 1) / bm, &n_wg) || !mul_ok(n_wg, n_splits, &n_wg) ||
            n_wg > (int64_t)(UINT32_MAX / 256))
            return FA_ERR_SHAPE;
        if (!workspace || workspace_bytes < need || ((uintptr_t)workspace & 15u))
            return FA_ERR_WORKSPACE;
        for (int i = 0; i < 4; ++i)
            if (overlaps(workspace, need, ins[i], in_bytes[i])) return FA_ERR_WORKSPACE;
        if (overlaps(workspace, need, out, nbytes) || overlaps(workspace, need, lse, lbytes))
            return FA_ERR_WORKSPACE;
        const int64_t rows = B * H * S;
        a.n_splits = (int)n_splits;
        a.part_o = (float*)workspace;
        a.part_lse = (float*)workspace + n_splits * rows * D;
    }
    const hipError_t e = fa::launch_fwd(a);
    return e == hipSuccess ? FA_OK : FA_ERR_HIP;
}

// ---------------------------------------------------------------- KV cache
namespace {

// Bytes of the fp32 partials of a KV-cache launch in n_splits parts (0 for one
// part), or -1 when the size overflows.
int64_t kvcache_workspace_bytes(int64_t B, int64_t H, int64_t S_q, int64_t D, int64_t n_splits) {
    if (n_splits <= 1) return 0;
    int64_t t, r;
    if (!mul_ok(B, H, &t) || !mul_ok(t, S_q, &t) || !mul_ok(t, n_splits * (D + 1) * 4, &r))
        return -1;
    return r;
}

// Checks shared by the KV-cache entry points: the query side as fa_fwd, the
// cache capacity, and the dtypes the KV-cache kernels take (bf16, fp16).
int check_kvcache_problem(int64_t B, int64_t H, int64_t S_q, int64_t S_k, int64_t D, int causal,
                          int64_t wl, int64_t wr, int dtype, int64_t* q_bytes, int64_t* lse_bytes) {
    const int rc = check_problem(B, H, S_q, D, causal, wl, wr, dtype, q_bytes, lse_bytes, kKvcMaxD);
    if (rc != FA_OK) return rc;
    if (dtype == FA_DTYPE_FP32) return FA_ERR_DTYPE;
    if (S_k < 1 || S_k > INT32_MAX) return FA_ERR_SHAPE;
    return FA_OK;
}

}  // namespace

FA_API int fa_fwd_kvcache_workspace_size(int64_t B, int64_t H, int64_t S_q, int64_t D, int dtype,
                                         int64_t n_splits, int64_t* bytes) {
    if (!bytes) return FA_ERR_NULL;
    int64_t qb, lb;
    const int rc = check_kvcache_problem(B, H, S_q, 1, D, 0, -1, -1, dtype, &qb, &lb);
    if (rc != FA_OK) return rc;
    if (n_splits < 1 || n_splits > FA_MAX_KV_SPLITS) return FA_ERR_SPLITS;
    const int64_t need = kvcache_workspace_bytes(B, H, S_q, D, n_splits);
    if (need < 0) return FA_ERR_SHAPE;
    *bytes = need;
    return FA_OK;
}

FA_API int fa_fwd_kvcache_auto_splits(int64_t B, int64_t H, int64_t S_q, int64_t S_k, int64_t D,
                                      int dtype, int64_t* n_splits) {
    if (!n_splits) return FA_ERR_NULL;
    int64_t qb, lb;
    const int rc = check_kvcache_problem(B, H, S_q, S_k, D, 0, -1, -1, dtype, &qb, &lb);
    if (rc != FA_OK) return rc;
    *n_splits = fa::kvcache_auto_splits(B, H, S_q, S_k, D, dtype);
    return FA_OK;
}

FA_API int fa_fwd_kvcache(const void* q, const void* k_cache, const void* v_cache,
                          const int32_t* cache_seqlens, const int32_t* block_table, void* out,
                          float* lse, int64_t B, int64_t H, int64_t S_q, int64_t S_k, int64_t D,
                          float scale, int causal, int64_t window_left, int64_t window_right,
                          int dtype, int64_t num_pages, int64_t page_size, int64_t table_stride,
                          int64_t n_splits, void* workspace, int64_t workspace_bytes,
                          void* stream) {
    if (!q || !k_cache || !v_cache || !cache_seqlens || !out || !lse) return FA_ERR_NULL;
    int64_t q_bytes = 0, lse_bytes = 0;
    int rc = check_kvcache_problem(B, H, S_q, S_k, D, causal, window_left, window_right, dtype,
                                   &q_bytes, &lse_bytes);
    if (rc != FA_OK) return rc;
    if (!std::isfinite(scale) || scale < 0.f) return FA_ERR_SCALE;
    // the caches: contiguous [B, S_k, H, D], or page pools [num_pages, page_size, H, D]
    const int64_t row_bytes = H * D * elem_size(dtype);
    int64_t t, cache_bytes, table_bytes = 0;
    if (block_table) {
        if (page_size < 64 || page_size % 64 != 0 || page_size > INT32_MAX || num_pages < 1 ||
            num_pages > INT32_MAX || table_stride < (S_k + page_size - 1) / page_size ||
            table_stride > INT32_MAX)
            return FA_ERR_PAGES;
        if (!mul_ok(num_pages, page_size, &t) || !mul_ok(t, row_bytes, &cache_bytes) ||
            !mul_ok(B, table_stride, &t) || !mul_ok(t, 4, &table_bytes))
            return FA_ERR_PAGES;
    } else {
        if (!mul_ok(B, S_k, &t) || !mul_ok(t, row_bytes, &cache_bytes)) return FA_ERR_SHAPE;
    }
    if (((uintptr_t)q | (uintptr_t)k_cache | (uintptr_t)v_cache | (uintptr_t)out) & 15u)
        return FA_ERR_ALIGN;
    if (((uintptr_t)lse | (uintptr_t)cache_seqlens | (uintptr_t)block_table) & 3u)
        return FA_ERR_ALIGN;
    const void* ins[5] = {q, k_cache, v_cache, cache_seqlens, block_table};
    const int64_t in_bytes[5] = {q_bytes, cache_bytes, cache_bytes, B * 4, table_bytes};
    for (int i = 0; i < 5; ++i)
        if (ins[i] && (overlaps(out, q_bytes, ins[i], in_bytes[i]) ||
                       overlaps(lse, lse_bytes, ins[i], in_bytes[i])))
            return FA_ERR_ALIAS;
    if (overlaps(out, q_bytes, lse, lse_bytes)) return FA_ERR_ALIAS;
    if (n_splits < 1 || n_splits > FA_MAX_KV_SPLITS) return FA_ERR_SPLITS;
    const int64_t need = kvcache_workspace_bytes(B, H, S_q, D, n_splits);
    if (need < 0) return FA_ERR_SHAPE;
    {  // the grid: B * H * ceil(S_q / 128) * n_splits workgroups of 256 threads
        int64_t n_wg;
        if (!mul_ok(B * H, (S_q + 127) / 128, &n_wg) || !mul_ok(n_wg, n_splits, &n_wg) ||
            n_wg > (int64_t)(UINT32_MAX / 256))
            return FA_ERR_SHAPE;
    }
    fa::LaunchArgs a = make_args(q, k_cache, v_cache, out, lse, B, H, S_q, D, scale, causal,
                                 window_left, window_right, dtype, stream);
    // a window wider than any position difference is unbounded: a query sees
    // keys at most S_k - 1 positions before it and S_q - 1 after it
    a.wl = window_left >= S_k ? -1 : window_left;
    a.wr = window_right >= S_q ? -1 : window_right;
    a.kv_lens = cache_seqlens;
    a.kv_cap = S_k;
    if (block_table) {
        a.pg_table = block_table;
        a.pg_stride = table_stride;
        a.pg_rows = page_size;
        a.pg_count = num_pages;
    }
    if (need > 0) {
        if (!workspace || workspace_bytes < need || ((uintptr_t)workspace & 15u))
            return FA_ERR_WORKSPACE;
        for (int i = 0; i < 5; ++i)
            if (ins[i] && overlaps(workspace, need, ins[i], in_bytes[i])) return FA_ERR_WORKSPACE;
        if (overlaps(workspace, need, out, q_bytes) || overlaps(workspace, need, lse, lse_bytes))
            return FA_ERR_WORKSPACE;
        const int64_t rows = B * H * S_q;
        a.n_splits = (int)n_splits;
        a.part_o = (float*)workspace;
        a.part_lse = (float*)workspace + n_splits * rows * D;
    }
    const hipError_t e = fa::launch_fwd(a);
    return e == hipSuccess ? FA_OK : FA_ERR_HIP;
}

// ---------------------------------------------------------------- no allocation
// fa_fwd_splitkv_noalloc keeps the split partials in this file-scope device
// array instead of a caller's workspace.  In host code `scratch` names a
// host-side stand-in, not device memory: its device address is taken once per
// device with hipGetSymbolAddress and only that address is used afterwards.
// Every call on a device shares that device's copy; the split kernel writes
// every partial the merge reads (empty parts included), so nothing needs
// clearing between calls, and calls that overlap on one device race.
static __device__ __align__(256) unsigned char scratch[FA_NOALLOC_SCRATCH_BYTES];

namespace {

constexpr int kMaxScratchDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxScratchDevices] = {};

// The device address of `scratch` on device `dev`, looked up (with that device
// current) the first time and kept.  FA_OK or FA_ERR_HIP.
int scratch_address(int dev, void** ptr) {
    if (dev < 0 || dev >= kMaxScratchDevices) return FA_ERR_HIP;
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        int cur = -1;
        if (hipGetDevice(&cur) != hipSuccess) {
            (void)hipGetLastError();
            return FA_ERR_HIP;
        }
        if (cur != dev && hipSetDevice(dev) != hipSuccess) {
            (void)hipGetLastError();
            return FA_ERR_HIP;
        }
        void* p = nullptr;
        const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (cur != dev) (void)hipSetDevice(cur);
        if (e != hipSuccess || !p) {
            (void)hipGetLastError();
            return FA_ERR_HIP;
        }
        g_scratch_ptr[dev] = p;
    }
    *ptr = g_scratch_ptr[dev];
    return FA_OK;
}

}  // namespace

FA_API int fa_fwd_splitkv_noalloc(const void* q, const void* k, const void* v, void* out,
                                  float* lse, int64_t B, int64_t H, int64_t S, int64_t D,
                                  float scale, int causal, int64_t window_left,
                                  int64_t window_right, int dtype, int64_t n_splits,
                                  void* stream) {
    int rc = fa_fwd_check_args(q, k, v, out, lse, B, H, S, D, scale, causal, window_left,
                               window_right, dtype);
    if (rc != FA_OK) return rc;
    int64_t need = 0;
    rc = fa_fwd_splitkv_workspace_size(B, H, S, D, dtype, n_splits, &need);
    if (rc != FA_OK) return rc;
    if (need > (int64_t)FA_NOALLOC_SCRATCH_BYTES) return FA_ERR_SCRATCH;
    fa::LaunchArgs a = make_args(q, k, v, out, lse, B, H, S, D, scale, causal, window_left,
                                 window_right, dtype, stream);
    if (need > 0) {
        const int64_t bm = fa::q_tile_rows(dtype, D, S, a.wl, a.wr);
        int64_t n_wg;
        if (!mul_ok(B * H, (S + bm - 1) / bm, &n_wg) || !mul_ok(n_wg, n_splits, &n_wg) ||
            n_wg > (int64_t)(UINT32_MAX / 256))
            return FA_ERR_SHAPE;
        // the device the launch runs on: the stream's, or the current one
        int dev = -1;
        if (stream) {
            if (hipStreamGetDevice((hipStream_t)stream, &dev) != hipSuccess) {
                (void)hipGetLastError();
                return FA_ERR_HIP;
            }
        } else if (hipGetDevice(&dev) != hipSuccess) {
            (void)hipGetLastError();
            return FA_ERR_HIP;
        }
        void* base = nullptr;
        rc = scratch_address(dev, &base);
        if (rc != FA_OK) return rc;
        const int64_t rows = B * H * S;
        a.n_splits = (int)n_splits;
        a.part_o = (float*)base;
        a.part_lse = (float*)base + n_splits * rows * D;
    }
    const hipError_t e = fa::launch_fwd(a);
    return e == hipSuccess ? FA_OK : FA_ERR_HIP;
}
