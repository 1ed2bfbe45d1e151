/*
 * fa_mi355x.h -- C ABI of libfa_mi355x: exact attention forward on MI355X
 * (gfx950), fused so the S x S score matrix never reaches HBM.
 *
 * Pages are cited by their titles:
 *   [V2]  "大模型加速新突破：Flash Attention V2核心网络算子解析"
 *   [FA]  "FlashAttention技术解析：加速GPT训练的核心优化"
 *   [CG]  "突破大模型训练瓶颈：Flash-Attention编译优化与内存占用解决方案"
 *   [AN]  "FlashAttention 剖析"
 *
 * What fa_fwd computes, for every batch b, head h and query row i:
 *   allowed(i,j) = (!causal || j <= i) && (wl < 0 || i - j <= wl)
 *                                       && (wr < 0 || j - i <= wr)
 *   O[b,i,h,:]   = sum_j softmax_j(scale * q_i . k_j over allowed j) * v[b,j,h,:]
 *   LSE[b,h,i]   = ln sum_{allowed j} exp(scale * q_i . k_j)
 * The formula is [V2] section 二.1; softmax_scale, causal and
 * window_size = (left, right) with -1 = unbounded are [FA] section 2.2 and
 * [CG] section 滑动窗口注意力 (bounds inclusive, "left" = earlier keys, causal
 * with a window = both masks); the (batch, seq_len, head, dim) layout is [V2]
 * section 三.1.  The method -- tiles of Q, K, V, a running row max and row sum
 * ("online renormalisation", [FA] section 1; [AN] section 3), intermediates
 * kept on chip ([CG] 项目核心价值; [AN] section 2) -- reaches this exact result
 * up to floating-point rounding.
 *
 * The library allocates no memory.  Its one piece of state is the static
 * device buffer of fa_fwd_splitkv_noalloc (with that buffer's address per
 * GPU, looked up once); every other function is stateless, thread-safe and
 * re-entrant.
 */
#ifndef FA_MI355X_H
#define FA_MI355X_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    FA_DTYPE_FP32 = 0, /* IEEE binary32 inputs and output; fp32 MFMA arithmetic */
    FA_DTYPE_FP16 = 1, /* IEEE binary16 inputs and output; fp32 accumulation */
    FA_DTYPE_BF16 = 2  /* bfloat16 inputs and output; fp32 accumulation */
} fa_dtype_t;

typedef enum {
    FA_OK = 0,
    FA_ERR_NULL = -1,     /* a required pointer is NULL */
    FA_ERR_SHAPE = -2,    /* B, H or S < 1, a size overflows int64 / the index range, or
                             64 rows of one tensor (64*H*D elements) exceed 2^31 - 1 bytes */
    FA_ERR_HEAD_DIM = -3, /* D not supported (a multiple of 16 in [16, 256] for the
                             bf16 / fp16 forward, [16, 128] for fp32 inputs, fa_bwd
                             and fa_fwd_kvcache) */
    FA_ERR_WINDOW = -4,   /* window_left or window_right < -1, or causal not 0/1 */
    FA_ERR_DTYPE = -5,    /* dtype not one of fa_dtype_t */
    FA_ERR_SCALE = -6,    /* scale NaN, infinite or negative */
    FA_ERR_ALIGN = -7,    /* q, k, v or out not 16-byte aligned, or lse not 4-byte aligned */
    FA_ERR_ALIAS = -8,    /* out or lse overlaps an input, or out overlaps lse */
    FA_ERR_HIP = -9,      /* the kernel launch failed (hipGetLastError) */
    FA_ERR_WORKSPACE = -10, /* a workspace argument is NULL, too small, not 16-byte
                               aligned, or overlapping an input or output */
    FA_ERR_SPLITS = -11,  /* fa_fwd_splitkv: n_splits outside [1, FA_MAX_SPLITS];
                             fa_fwd_kvcache: outside [1, FA_MAX_KV_SPLITS] */
    FA_ERR_BLOCKMASK = -12, /* fa_fwd_blocksparse: block_m not a positive multiple of 128,
                               block_n not a positive multiple of 64, or n_mask not 1, H
                               or B*H */
    FA_ERR_PAGES = -13,   /* fa_fwd_paged: page_size not a positive multiple of 64,
                             num_pages < 1, table_stride < ceil(S / page_size), or a
                             pool / table size outside the index ranges */
    FA_ERR_SCRATCH = -14  /* fa_fwd_splitkv_noalloc: the partials need more than
                             FA_NOALLOC_SCRATCH_BYTES */
} fa_status_t;

/* The most K/V parts per Q tile fa_fwd_splitkv takes. */
#define FA_MAX_SPLITS 16
/* The most K/V parts per query block fa_fwd_kvcache takes. */
#define FA_MAX_KV_SPLITS 64

/*
 * fa_fwd -- one fused attention forward over all (b, h).
 *
 * q, k, v  device pointers, contiguous [B, S, H, D] of `dtype` (row stride
 *          H*D elements).  Read only.
 * out      device pointer, contiguous [B, S, H, D] of `dtype`; fully written.
 *          O is rounded to nearest-even from fp32.
 * lse      device pointer, contiguous [B, H, S] fp32; fully written with the
 *          natural-log log-sum-exp of the scaled, masked scores of each row.
 *          A causal bf16 / fp16 launch larger than the device also counts its
 *          dynamic tile order in the word of row 0 of (b, h) = (0, 0) while it
 *          runs (fa_fwd_launch_order); the word holds its LSE on return.
 * B, H, S  batch, heads, sequence length (one S for queries and keys), >= 1.
 * D        head dimension.  bf16 / fp16: any multiple of 16 from 16 to 256
 *          (the pages ask Tensor Core shapes to be multiples of 8: section 4.2
 *          of "FlashAttention技术解析：加速GPT训练的核心优化"; 16 is the k
 *          step of the gfx950 MFMA); a D other than 64, 128 and 256 runs the
 *          kernel for the next of them with the extra columns read as zeros
 *          and never written, and D above 128 uses 32-key K/V tiles.  fp32: a
 *          multiple of 16 up to 128.  The same holds for fa_fwd_splitkv, fa_fwd_splitkv_noalloc,
 *          fa_fwd_blocksparse and fa_fwd_paged; fa_bwd and fa_fwd_kvcache take
 *          multiples of 16 up to 128.
 * scale    softmax scale applied to q.k in fp32 (finite, >= 0); callers that
 *          want the pages' default pass 1/sqrt(D).
 * causal   0 or 1.
 * window_left, window_right   >= -1; -1 = unbounded on that side; a value
 *          >= S behaves as unbounded.
 * stream   hipStream_t to enqueue on; NULL = the default stream.
 *
 * Ownership: the caller owns all five buffers; the library allocates nothing.
 * The call validates its arguments first (no HIP call, no write on error),
 * then enqueues one kernel (after a one-thread kernel that zeroes that LSE
 * word, when the dynamic order is taken) and returns without synchronising.
 * Results are valid once `stream` has been synchronised; faults during execution surface
 * there.  Repeated calls on the same inputs give bitwise identical results.
 * Returns FA_OK or a negative fa_status_t.
 */
int fa_fwd(const void* q, const void* k, const void* v, void* out, float* lse, int64_t B,
           int64_t H, int64_t S, int64_t D, float scale, int causal, int64_t window_left,
           int64_t window_right, int dtype, void* stream);

/*
 * fa_fwd_check_args -- the validation fa_fwd performs, as a pure function: no
 * HIP call, no memory access through the pointers (they are compared only).
 * Returns FA_OK or the status fa_fwd would return before launching.
 */
int fa_fwd_check_args(const void* q, const void* k, const void* v, const void* out,
                      const float* lse, int64_t B, int64_t H, int64_t S, int64_t D, float scale,
                      int causal, int64_t window_left, int64_t window_right, int dtype);

/* fa_status_string -- a static, human-readable message for a status code. */
const char* fa_status_string(int status);

/*
 * fa_fwd_tile_schedule -- host-side description of the tile schedule fa_fwd
 * uses for one Q tile (tiles of Q and of K/V: [V2] section 二.1 step 1; [AN]
 * section 3).  Pure function, no HIP call.
 *
 * For Q tile `q_tile` (rows [q_tile*BM, min(S, (q_tile+1)*BM))), writes the
 * tile shape (*bm, *bn), the number of Q tiles (*n_q_tiles) and the
 * half-open range [*kt_begin, *kt_end) of K/V tiles the kernel visits; K/V
 * tiles outside it hold no allowed key for any row of the Q tile and are
 * skipped.  If needs_mask is non-NULL and has room for (*kt_end - *kt_begin)
 * entries (max_tiles), needs_mask[t - *kt_begin] is 1 when tile t holds at
 * least one key that is not allowed for some row of the Q tile (or lies past
 * S), else 0 (the kernel skips the mask there).
 * Returns FA_OK, or FA_ERR_* for bad arguments / q_tile out of range /
 * max_tiles too small.
 */
int fa_fwd_tile_schedule(int64_t S, int64_t D, int dtype, int causal, int64_t window_left,
                         int64_t window_right, int64_t q_tile, int64_t* bm, int64_t* bn,
                         int64_t* n_q_tiles, int64_t* kt_begin, int64_t* kt_end,
                         uint8_t* needs_mask, int64_t max_tiles);

/*
 * fa_fwd_workgroup_tile -- host-side view of the launch order fa_fwd uses:
 * the (b * H + h, Q tile) that workgroup `wg` of the grid processes.  Pure
 * function, no HIP call.  The grid has B * H * n_q_tiles workgroups (n_q_tiles
 * as fa_fwd_tile_schedule reports), and the map is a bijection onto the
 * (batch-head, Q tile) pairs.  Workgroup ids are dispatched round-robin over
 * the 8 XCDs, and each XCD gets a contiguous block of the head-major list of
 * tiles (its heads' K/V stay in its L2); with causal = 1 each XCD visits its
 * block's Q tiles heaviest first across heads (more K/V tiles to walk =
 * earlier), so that light tiles end the launch (thread-block load balance,
 * the note closing [FA] section 1).  With causal = 1 and either fewer than 8
 * (batch, head) pairs (whole heads cannot go to XCDs) or K and V of all heads
 * within 128 MiB (half the MALL, so every XCD can work on every head), the
 * tiles of all heads are instead ordered heaviest first and dealt to the XCDs
 * in snake order (0..7, 7..0, ...): every XCD gets the same share of the work
 * and runs it heaviest first, in groups of 32 workgroups (one per compute
 * unit of the XCD), every odd whole group lightest first, so that the units
 * that got the heaviest tiles also get lighter ones.
 * Returns FA_OK, or FA_ERR_* for bad arguments or wg outside the grid.
 */
int fa_fwd_workgroup_tile(int64_t B, int64_t H, int64_t S, int64_t D, int dtype, int causal,
                          int64_t window_left, int64_t window_right, int64_t wg, int64_t* bh,
                          int64_t* q_tile);

/*
 * fa_fwd_launch_order -- host-side view of the order fa_fwd runs its tiles in
 * on a device with n_cus compute units.  Pure function, no HIP call.  A
 * causal bf16 / fp16 launch with more workgroups than the device holds at
 * once (3 per compute unit at D <= 64, 2 at D <= 128, 1 above) runs its
 * lightest Q tiles, about 10% of its K/V tile steps, in a dynamic order, so
 * that faster XCDs take more of them (thread-block load balance, the note
 * closing [FA] section 1).  All heads' Q tiles then form one list, heaviest
 * first (rank r = Q tile n_q_tiles - 1 - r, heads next to each other, the
 * heads of a rank rotated by one: position p is (b * H + h, Q tile) =
 * ((p + 1) mod (B * H), n_q_tiles - 1 - p / (B * H))).  Workgroups below
 * *first_dynamic take the heavy positions [0, *first_dynamic) in the static
 * order's fashion (snake order, or blocks of whole heads per XCD, as
 * fa_fwd_workgroup_tile describes); each later workgroup takes the next
 * position when it starts, and wg >= *first_dynamic reports position wg,
 * the tile of the (wg - *first_dynamic)-th of them to start.  During the
 * call the word of LSE row 0 of (b, h) = (0, 0) counts the positions taken
 * (that row is the last position, whose workgroup writes it afterwards).
 * Otherwise *first_dynamic = -1 and the order is fa_fwd_workgroup_tile's.
 * Returns FA_OK, or FA_ERR_* for bad arguments (n_cus < 1 or wg outside the
 * grid: FA_ERR_SHAPE).
 */
int fa_fwd_launch_order(int64_t B, int64_t H, int64_t S, int64_t D, int dtype, int causal,
                        int64_t window_left, int64_t window_right, int64_t n_cus, int64_t wg,
                        int64_t* bh, int64_t* q_tile, int64_t* first_dynamic);

/*
 * fa_fwd_splitkv -- fa_fwd with the K/V tiles of every Q tile cut into
 * n_splits contiguous parts that separate workgroups process at the same
 * time.  Each workgroup writes the partial (O, LSE) of its part, in fp32, to
 * `workspace`; a second kernel then merges a row's parts with the log-domain
 * rule of the online softmax ([FA] section 1 item 3; [V2] section 二.1 step 2):
 * LSE = log-sum-exp of the parts' LSEs, O = the parts' O weighted by
 * exp(LSE_p - LSE).  The result equals fa_fwd's up to rounding.  It pays off
 * when fa_fwd's grid cannot fill the device or one Q tile's long row of K/V
 * tiles sets the time (short sequences, few heads, causal masks): the longest
 * chain of K/V tiles one workgroup walks shrinks by n_splits.
 *
 * Arguments and results as fa_fwd, plus:
 * n_splits         parts per Q tile, 1 .. FA_MAX_SPLITS.  1 runs fa_fwd itself.
 *                  A Q tile with fewer K/V tiles than parts leaves some parts
 *                  empty (they add nothing).  fp32 inputs always run in one
 *                  part.
 * workspace        device buffer of at least fa_fwd_splitkv_workspace_size
 *                  bytes, 16-byte aligned, not overlapping q, k, v, out or lse;
 *                  owned by the caller, its contents on return unspecified.
 *                  May be NULL when that size is 0.
 * workspace_bytes  its size in bytes.
 * Validation happens before any HIP call, as for fa_fwd.  Enqueues two
 * kernels on `stream` (one when no split is used) and returns without
 * synchronising.  Returns FA_OK or a negative fa_status_t.
 */
int fa_fwd_splitkv(const void* q, const void* k, const void* v, void* out, float* lse, int64_t B,
                   int64_t H, int64_t S, int64_t D, float scale, int causal, int64_t window_left,
                   int64_t window_right, int dtype, int64_t n_splits, void* workspace,
                   int64_t workspace_bytes, void* stream);

/*
 * fa_fwd_splitkv_workspace_size -- the workspace fa_fwd_splitkv needs, in
 * *bytes: n_splits * B * H * S * (D + 1) * 4 (the fp32 partial O and LSE of
 * every part), or 0 when n_splits is 1 or dtype is FA_DTYPE_FP32.  Pure
 * function, no HIP call.  Returns FA_OK, FA_ERR_NULL, FA_ERR_SPLITS, or the
 * status fa_fwd_check_args gives for the shape, head dimension and dtype.
 */
int fa_fwd_splitkv_workspace_size(int64_t B, int64_t H, int64_t S, int64_t D, int dtype,
                                  int64_t n_splits, int64_t* bytes);

/*
 * fa_fwd_splitkv_auto_splits -- a part count for this problem on the current
 * device: 1 when fa_fwd's own grid has at least two workgroups per compute
 * unit (then the fp32 partials and the merge cost about what the split saves),
 * else enough parts for four workgroups per unit, at most 8 and at most the
 * K/V tile count of the longest Q tile; 1 for fp32 inputs or when the device
 * cannot be queried.
 * Queries the device (HIP calls) but launches nothing.  Returns FA_OK or the
 * status fa_fwd_check_args gives for the problem arguments (pointers are not
 * needed).
 */
int fa_fwd_splitkv_auto_splits(int64_t B, int64_t H, int64_t S, int64_t D, int causal,
                               int64_t window_left, int64_t window_right, int dtype,
                               int64_t* n_splits);

/*
 * fa_fwd_splitkv_workgroup_tile -- host-side view of the launch order of
 * fa_fwd_splitkv (and of fa_fwd_paged with n_splits parts): the (b * H + h,
 * Q tile, part) that workgroup `wg` of its attention kernel processes.  Pure
 * function, no HIP call.  With n_splits = 1, or fp32 inputs (which run in one
 * part), it is fa_fwd_workgroup_tile with part 0.  Otherwise the grid has
 * B * H * n_q_tiles * n_splits workgroups and the map is a bijection onto the
 * (batch-head, Q tile, part) triples.  With causal = 1 the parts of all tiles
 * are ordered heaviest tile first and dealt to the 8 XCDs in snake order, so
 * that every XCD gets the same share of the work (thread-block load balance,
 * the note closing [FA] section 1); without the causal mask a tile's parts
 * are consecutive workgroups, and the tiles follow fa_fwd_workgroup_tile.
 * Returns FA_OK, or FA_ERR_* for bad arguments (FA_ERR_SPLITS for n_splits
 * outside [1, FA_MAX_SPLITS]) or wg outside the grid.
 */
int fa_fwd_splitkv_workgroup_tile(int64_t B, int64_t H, int64_t S, int64_t D, int dtype,
                                  int causal, int64_t window_left, int64_t window_right,
                                  int64_t n_splits, int64_t wg, int64_t* bh, int64_t* q_tile,
                                  int64_t* part);

/*
 * fa_bwd -- gradients of fa_fwd's output with respect to q, k and v for an
 * output gradient dout, recomputed tile by tile from the saved LSE instead of
 * a stored S x S matrix ([V2] section 二.1, step 3: the backward pass reuses
 * what the forward saved).  With P = exp(scale q.k - LSE) over the allowed
 * keys, D_i = dout_i . out_i and dS = P (dout v^T - D):
 *   dq = scale dS k,   dk = scale dS^T q,   dv = P^T dout.
 *
 * q, k, v, out, lse  the forward's inputs and results (out and lse exactly as
 *          fa_fwd wrote them for these q, k, v and arguments).
 * dout     the output gradient, [B, S, H, D] of `dtype`.
 * dq, dk, dv  outputs, [B, S, H, D] of `dtype` (fp32 accumulation, RNE).
 * workspace  device buffer of at least fa_bwd_workspace_size bytes (fp32
 *          D_i), 16-byte aligned; owned by the caller, contents on return
 *          unspecified.
 * dtype    FA_DTYPE_BF16 or FA_DTYPE_FP16 (fp32 is not supported here:
 *          FA_ERR_DTYPE).
 * D        a multiple of 16 from 16 to 128 (not 64 or 128: the kernels for the
 *          next of them, the extra columns read as zeros and never written).
 *          Other arguments as fa_fwd.
 * Pointers as in fa_fwd: 16-byte aligned tensors, lse 4-byte aligned; the
 * outputs and the workspace must not overlap the inputs or each other
 * (FA_ERR_ALIAS, FA_ERR_WORKSPACE).  Validation happens before any HIP call.
 * Enqueues three kernels on `stream` and returns without synchronising.
 * Returns FA_OK or a negative fa_status_t.
 */
int fa_bwd(const void* q, const void* k, const void* v, const void* out, const float* lse,
           const void* dout, void* dq, void* dk, void* dv, int64_t B, int64_t H, int64_t S,
           int64_t D, float scale, int causal, int64_t window_left, int64_t window_right,
           int dtype, void* workspace, int64_t workspace_bytes, void* stream);

/* fa_bwd_workspace_size -- the workspace fa_bwd needs in *bytes: B * H * S * 4
 * (fp32 D_i per row) plus 64 (the counters of the passes' dynamic order).
 * Pure function.  Returns FA_OK, FA_ERR_NULL or the shape / head-dimension /
 * dtype status of fa_fwd_check_args (fp32: FA_ERR_DTYPE). */
int fa_bwd_workspace_size(int64_t B, int64_t H, int64_t S, int64_t D, int dtype, int64_t* bytes);

/*
 * fa_fwd_blocksparse -- fa_fwd restricted to the blocks a block mask keeps
 * (block-sparse attention: [FA] section 5 lists it as the variant of the
 * method that reaches very long contexts through a sparse pattern).  Key j is
 * allowed for query i of head (b, h) when fa_fwd allows it and
 *   block_mask[hm][i / block_m][j / block_n] != 0,
 * hm = 0 (n_mask = 1: one mask for every head), h (n_mask = H) or b * H + h
 * (n_mask = B * H).  Dropped blocks are never read: the work and the K/V
 * traffic scale with the kept blocks.  A row with no allowed key gets O = 0
 * and LSE = -inf.
 *
 * Arguments and results as fa_fwd, plus:
 * block_mask  device pointer, contiguous uint8 [n_mask, ceil(S / block_m),
 *             ceil(S / block_n)], nonzero = kept; read only, any alignment.
 * n_mask      1, H or B * H.
 * block_m     query rows per mask block: a positive multiple of 128.
 * block_n     keys per mask block: a positive multiple of 64.
 * workspace   device buffer of at least fa_fwd_blocksparse_workspace_size
 *             bytes, 16-byte aligned, not overlapping q, k, v, out, lse or the
 *             mask; owned by the caller, contents on return unspecified (the
 *             compacted list of kept tiles).  May be NULL when that size is 0.
 * workspace_bytes  its size in bytes.
 * Validation happens before any HIP call (FA_ERR_BLOCKMASK for bad block
 * sizes or n_mask, FA_ERR_ALIAS when out or lse overlaps the mask).  Enqueues
 * two kernels on `stream` (one for fp32, which reads the mask directly) and
 * returns without synchronising.  Returns FA_OK or a negative fa_status_t.
 */
int fa_fwd_blocksparse(const void* q, const void* k, const void* v, void* out, float* lse,
                       int64_t B, int64_t H, int64_t S, int64_t D, float scale, int causal,
                       int64_t window_left, int64_t window_right, int dtype,
                       const uint8_t* block_mask, int64_t n_mask, int64_t block_m,
                       int64_t block_n, void* workspace, int64_t workspace_bytes, void* stream);

/*
 * fa_fwd_blocksparse_workspace_size -- the workspace fa_fwd_blocksparse needs,
 * in *bytes: n_mask * ceil(S / 128) * (4 + 4 * ceil(ceil(S / BN) / 4)) * 4 for
 * bf16 / fp16 (one list of kept K/V tiles per mask head and Q tile; BN = 64,
 * or 32 above D = 128), 0 for fp32.  Pure function, no HIP call.  Returns FA_OK, FA_ERR_NULL,
 * FA_ERR_BLOCKMASK (n_mask not 1, H or B * H) or the status fa_fwd_check_args
 * gives for the shape, head dimension and dtype.
 */
int fa_fwd_blocksparse_workspace_size(int64_t B, int64_t H, int64_t S, int64_t D, int dtype,
                                      int64_t n_mask, int64_t* bytes);

/*
 * fa_fwd_paged -- fa_fwd with keys and values kept in a paged cache: fixed-size
 * pages in two pools, found through a block table, like the pages of an
 * operating system's memory ([CG] section Paged KV Cache支持: non-contiguous
 * blocks managed by a block table).  Key j of batch b is row j % page_size of
 * page block_table[b * table_stride + j / page_size] of k_pages and v_pages.
 * What is computed is fa_fwd's result on the gathered keys and values; pages
 * may be shared between sequences and placed anywhere in the pools.
 *
 * q, out, lse  as fa_fwd.
 * k_pages, v_pages  device pointers, contiguous [num_pages, page_size, H, D]
 *             of `dtype`, 16-byte aligned; read only.  Rows of a page past S
 *             are never read.
 * block_table device pointer, int32 [B, table_stride], 4-byte aligned; read
 *             only.  Entries 0 .. ceil(S / page_size) - 1 of each row are used;
 *             each must lie in [0, num_pages) -- a page index outside the pool
 *             is not an error the call can see (the table is device memory):
 *             its keys and values read as zeros.
 * num_pages   pages in each pool, >= 1.
 * page_size   rows per page: a positive multiple of 64 (a K/V tile never
 *             straddles pages).
 * table_stride  int32 entries per table row, >= ceil(S / page_size).
 * n_splits, workspace, workspace_bytes  as fa_fwd_splitkv (1 = one part; the
 *             workspace is fa_fwd_splitkv_workspace_size bytes and may be
 *             NULL when that is 0).  fp32 inputs run in one part.
 * Other arguments as fa_fwd.  out and lse must not overlap q, the pools, the
 * table or each other (FA_ERR_ALIAS); bad page geometry is FA_ERR_PAGES.
 * Validation happens before any HIP call.  Enqueues one kernel on `stream`
 * (two with a split) and returns without synchronising.  A causal bf16 / fp16
 * call in one part with more workgroups than the device holds (two per
 * compute unit at D <= 64, as at D <= 128) takes fa_fwd's dynamic order, with
 * the same counter in the LSE word of row 0 of (b, h) = (0, 0) and the same
 * one-thread kernel that zeroes it first.  Returns FA_OK or a negative
 * fa_status_t.
 */
int fa_fwd_paged(const void* q, const void* k_pages, const void* v_pages,
                 const int32_t* block_table, void* out, float* lse, int64_t B, int64_t H,
                 int64_t S, int64_t D, float scale, int causal, int64_t window_left,
                 int64_t window_right, int dtype, int64_t num_pages, int64_t page_size,
                 int64_t table_stride, int64_t n_splits, void* workspace,
                 int64_t workspace_bytes, void* stream);

/*
 * fa_fwd_kvcache -- attention of S_q new queries per sequence against a
 * key/value cache, as in decoding (FlashDecoding, the variant of the method
 * for the KV cache of inference: [FA] section 5; the call
 * flash_attn_with_kvcache and a paged cache found through a block table:
 * [CG] sections 总结与最佳实践 and Paged KV Cache支持).  For sequence b the
 * cache's first L_b = cache_seqlens[b] rows are its keys and values (the new
 * tokens' own included); its queries are the sequence's last S_q positions,
 * query i at position p = L_b - S_q + i, and
 *   allowed(i, j) = j < L_b && (!causal || j <= p) && (wl < 0 || p - j <= wl)
 *                                                 && (wr < 0 || j - p <= wr)
 *   O[b,i,h,:]   = sum_j softmax_j(scale * q_i . k_j over allowed j) * v[b,j,h,:]
 *   LSE[b,h,i]   = ln sum_{allowed j} exp(scale * q_i . k_j)
 * A row with no allowed key (p < 0 under the causal mask, or L_b = 0) gets
 * O = 0 and LSE = -inf.  With S_q = L_b = S_k this is fa_fwd.  Cache rows past
 * L_b are never read.  The K/V tiles of each query block may be cut into
 * n_splits parts processed at the same time and merged in the log domain as
 * in fa_fwd_splitkv -- the usual case for decoding, where B * H query blocks
 * of one row each cannot fill the device.
 *
 * q, out      device, contiguous [B, S_q, H, D] of `dtype` (bf16 or fp16); D a
 *             multiple of 16 from 16 to 128 (one query per sequence runs a
 *             vector-ALU kernel at D = 64 and 128, the MFMA kernel otherwise).
 * lse         device, contiguous fp32 [B, H, S_q].
 * k_cache, v_cache  device, read only: contiguous [B, S_k, H, D] caches when
 *             block_table is NULL, else page pools [num_pages, page_size, H, D]
 *             (key j of sequence b: row j % page_size of page
 *             block_table[b * table_stride + j / page_size]; a page index
 *             outside [0, num_pages) reads as zeros).
 * cache_seqlens  device int32 [B]: L_b, clamped to [0, S_k] by the kernel (the
 *             host cannot read it without a synchronisation).
 * block_table device int32 [B, table_stride] or NULL (contiguous caches).
 * S_q, S_k    queries per sequence (>= 1), cache capacity in rows (>= 1).
 * num_pages, page_size, table_stride  as fa_fwd_paged (ignored without a table).
 * n_splits    parts per query block, 1 .. FA_MAX_KV_SPLITS.
 * workspace, workspace_bytes  as fa_fwd_splitkv: at least
 *             fa_fwd_kvcache_workspace_size bytes, 16-byte aligned, caller-owned;
 *             may be NULL when that size is 0.
 * Other arguments as fa_fwd; window_left >= S_k and window_right >= S_q are
 * unbounded.  fp32 is FA_ERR_DTYPE.  Validation happens before any HIP call
 * (pointer alignment: tensors 16 bytes, lse / seqlens / table 4 bytes;
 * out and lse must not overlap any input or each other).  Enqueues one kernel
 * on `stream` (two with a split) and returns without synchronising.  Returns
 * FA_OK or a negative fa_status_t.
 */
int fa_fwd_kvcache(const void* q, const void* k_cache, const void* v_cache,
                   const int32_t* cache_seqlens, const int32_t* block_table, void* out, float* lse,
                   int64_t B, int64_t H, int64_t S_q, int64_t S_k, int64_t D, float scale,
                   int causal, int64_t window_left, int64_t window_right, int dtype,
                   int64_t num_pages, int64_t page_size, int64_t table_stride, int64_t n_splits,
                   void* workspace, int64_t workspace_bytes, void* stream);

/* fa_fwd_kvcache_workspace_size -- the workspace fa_fwd_kvcache needs, in
 * *bytes: n_splits * B * H * S_q * (D + 1) * 4, or 0 for one part.  Pure
 * function.  Returns FA_OK, FA_ERR_NULL, FA_ERR_SPLITS, FA_ERR_DTYPE (fp32) or
 * the shape / head-dimension status of fa_fwd_check_args. */
int fa_fwd_kvcache_workspace_size(int64_t B, int64_t H, int64_t S_q, int64_t D, int dtype,
                                  int64_t n_splits, int64_t* bytes);

/* fa_fwd_kvcache_auto_splits -- a part count for fa_fwd_kvcache on the current
 * device: 1 when B * H * ceil(S_q / 128) query blocks give two workgroups per
 * compute unit, else enough parts for four per unit, at most
 * FA_MAX_KV_SPLITS and at most one part per 4 K/V tiles (64 keys each) of a
 * full cache.  Queries the device, launches nothing.  Returns FA_OK or the
 * status fa_fwd_kvcache_workspace_size gives. */
int fa_fwd_kvcache_auto_splits(int64_t B, int64_t H, int64_t S_q, int64_t S_k, int64_t D,
                               int dtype, int64_t* n_splits);

/* Bytes of the static device buffer fa_fwd_splitkv_noalloc keeps its split
 * partials in (one copy per GPU, held until the process ends). */
#define FA_NOALLOC_SCRATCH_BYTES (128LL << 20)

/*
 * fa_fwd_splitkv_noalloc -- fa_fwd_splitkv for callers that cannot allocate
 * device memory: code under HIP graph capture, tight serving loops, and
 * harnesses that forbid allocation.  It computes exactly what fa_fwd_splitkv
 * computes, with the same kernels, but keeps the fp32 partial O and LSE in a
 * static device buffer of the library (FA_NOALLOC_SCRATCH_BYTES, one per GPU)
 * instead of a workspace argument.  It calls no allocator.  The first call on
 * a GPU looks the buffer's address up (hipGetSymbolAddress) and keeps it.
 *
 * Arguments and results as fa_fwd_splitkv without workspace and
 * workspace_bytes; the launch runs on `stream`'s device (the current device
 * for NULL).  Returns FA_ERR_SCRATCH, before any launch, when the partials
 * (fa_fwd_splitkv_workspace_size bytes) exceed FA_NOALLOC_SCRATCH_BYTES.
 * Every call on one GPU uses the same buffer: calls that overlap in time on
 * one GPU (other streams, other host threads) race and must be serialised
 * by the caller.  Nothing in the buffer needs to start at zero -- every
 * partial the merge reads is written by the same call.
 */
int fa_fwd_splitkv_noalloc(const void* q, const void* k, const void* v, void* out, float* lse,
                           int64_t B, int64_t H, int64_t S, int64_t D, float scale, int causal,
                           int64_t window_left, int64_t window_right, int dtype,
                           int64_t n_splits, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* FA_MI355X_H */
