"""ctypes binding of libfa_mi355x (declared in include/fa_mi355x.h).

Same names as the C ABI: ``fa_fwd``, ``fa_fwd_check_args``,
``fa_status_string``, ``fa_fwd_tile_schedule``, ``fa_fwd_workgroup_tile``, ``fa_fwd_launch_order``,
``fa_fwd_splitkv_workgroup_tile``, ``fa_fwd_splitkv``,
``fa_fwd_splitkv_workspace_size``, ``fa_fwd_splitkv_auto_splits``, ``fa_bwd``,
``fa_bwd_workspace_size``, ``fa_fwd_blocksparse``, ``fa_fwd_blocksparse_workspace_size``,
``fa_fwd_paged``; plus ``flash_attn_fwd`` (and ``flash_attn_fwd_splitkv``, ``flash_attn_bwd``,
``flash_attn_fwd_blocksparse``, ``flash_attn_fwd_paged``), the
tensor-level call that mirrors the pages' ``flash_attention(q, k, v,
softmax_scale=None, causal=..., window_size=(-1, -1))`` argument list
("FlashAttention技术解析：加速GPT训练的核心优化", section 2.2).  This module only
marshals arguments; it computes nothing of the method itself.
"""
from __future__ import annotations

import ctypes
import math
import os
import threading

FA_DTYPE_FP32 = 0
FA_DTYPE_FP16 = 1
FA_DTYPE_BF16 = 2
FA_MAX_SPLITS = 16
FA_MAX_KV_SPLITS = 64
FA_NOALLOC_SCRATCH_BYTES = 128 << 20
FA_ERR_SCRATCH = -14

_PKG = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_PKG, "libfa_mi355x.so")
_lock = threading.Lock()
_lib = None


class FaError(RuntimeError):
    """A non-zero fa_status_t from the library."""

    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: {fa_status_string(status)} (status {status})")


def library_path() -> str:
    return _LIB_PATH


def _load():
    global _lib
    with _lock:
        if _lib is not None:
            return _lib
        if not os.path.exists(_LIB_PATH):
            raise RuntimeError(
                f"{_LIB_PATH} is not built; build it with io_aware_exact_22_amd.build.build() "
                "(or __graft_entry__.build()).  There is no fallback implementation.")
        # torch first: its HIP runtime (same soname) must be the one the library binds to, so
        # that torch's streams and allocations are valid in the library
        import torch  # noqa: F401

        lib = ctypes.CDLL(_LIB_PATH)
        i64, vp, cint = ctypes.c_int64, ctypes.c_void_p, ctypes.c_int
        lib.fa_fwd.argtypes = [vp, vp, vp, vp, vp, i64, i64, i64, i64, ctypes.c_float, cint, i64,
                               i64, cint, vp]
        lib.fa_fwd.restype = cint
        lib.fa_fwd_check_args.argtypes = [vp, vp, vp, vp, vp, i64, i64, i64, i64, ctypes.c_float,
                                          cint, i64, i64, cint]
        lib.fa_fwd_check_args.restype = cint
        lib.fa_status_string.argtypes = [cint]
        lib.fa_status_string.restype = ctypes.c_char_p
        p64 = ctypes.POINTER(ctypes.c_int64)
        lib.fa_fwd_tile_schedule.argtypes = [i64, i64, cint, cint, i64, i64, i64, p64, p64, p64,
                                             p64, p64, vp, i64]
        lib.fa_fwd_tile_schedule.restype = cint
        lib.fa_fwd_workgroup_tile.argtypes = [i64, i64, i64, i64, cint, cint, i64, i64, i64, p64,
                                              p64]
        lib.fa_fwd_workgroup_tile.restype = cint
        lib.fa_fwd_launch_order.argtypes = [i64, i64, i64, i64, cint, cint, i64, i64, i64, i64,
                                            p64, p64, p64]
        lib.fa_fwd_launch_order.restype = cint
        lib.fa_fwd_splitkv_workgroup_tile.argtypes = [i64, i64, i64, i64, cint, cint, i64, i64,
                                                      i64, i64, p64, p64, p64]
        lib.fa_fwd_splitkv_workgroup_tile.restype = cint
        lib.fa_fwd_splitkv.argtypes = [vp, vp, vp, vp, vp, i64, i64, i64, i64, ctypes.c_float, cint,
                                       i64, i64, cint, i64, vp, i64, vp]
        lib.fa_fwd_splitkv.restype = cint
        lib.fa_fwd_splitkv_workspace_size.argtypes = [i64, i64, i64, i64, cint, i64, p64]
        lib.fa_fwd_splitkv_workspace_size.restype = cint
        lib.fa_fwd_splitkv_auto_splits.argtypes = [i64, i64, i64, i64, cint, i64, i64, cint, p64]
        lib.fa_fwd_splitkv_auto_splits.restype = cint
        lib.fa_bwd.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, i64, i64, i64, i64,
                               ctypes.c_float, cint, i64, i64, cint, vp, i64, vp]
        lib.fa_bwd.restype = cint
        lib.fa_fwd_blocksparse.argtypes = [vp, vp, vp, vp, vp, i64, i64, i64, i64, ctypes.c_float,
                                           cint, i64, i64, cint, vp, i64, i64, i64, vp, i64, vp]
        lib.fa_fwd_blocksparse.restype = cint
        lib.fa_fwd_blocksparse_workspace_size.argtypes = [i64, i64, i64, i64, cint, i64, p64]
        lib.fa_fwd_blocksparse_workspace_size.restype = cint
        lib.fa_fwd_paged.argtypes = [vp, vp, vp, vp, vp, vp, i64, i64, i64, i64, ctypes.c_float,
                                     cint, i64, i64, cint, i64, i64, i64, i64, vp, i64, vp]
        lib.fa_fwd_paged.restype = cint
        lib.fa_bwd_workspace_size.argtypes = [i64, i64, i64, i64, cint, p64]
        lib.fa_bwd_workspace_size.restype = cint
        lib.fa_fwd_kvcache.argtypes = [vp, vp, vp, vp, vp, vp, vp, i64, i64, i64, i64, i64,
                                       ctypes.c_float, cint, i64, i64, cint, i64, i64, i64, i64,
                                       vp, i64, vp]
        lib.fa_fwd_kvcache.restype = cint
        lib.fa_fwd_kvcache_workspace_size.argtypes = [i64, i64, i64, i64, cint, i64, p64]
        lib.fa_fwd_kvcache_workspace_size.restype = cint
        lib.fa_fwd_kvcache_auto_splits.argtypes = [i64, i64, i64, i64, i64, cint, p64]
        lib.fa_fwd_kvcache_auto_splits.restype = cint
        lib.fa_fwd_splitkv_noalloc.argtypes = [vp, vp, vp, vp, vp, i64, i64, i64, i64,
                                               ctypes.c_float, cint, i64, i64, cint, i64, vp]
        lib.fa_fwd_splitkv_noalloc.restype = cint
        _lib = lib
        return lib


# ------------------------------------------------------------------ raw C ABI
def fa_fwd(q: int, k: int, v: int, out: int, lse: int, B: int, H: int, S: int, D: int,
           scale: float, causal: int, window_left: int, window_right: int, dtype: int,
           stream: int | None) -> int:
    """The C entry point with raw device pointers (ints); returns the status."""
    return _load().fa_fwd(q, k, v, out, lse, B, H, S, D, scale, causal, window_left, window_right,
                          dtype, stream)


def fa_fwd_check_args(q: int, k: int, v: int, out: int, lse: int, B: int, H: int, S: int, D: int,
                      scale: float, causal: int, window_left: int, window_right: int,
                      dtype: int) -> int:
    return _load().fa_fwd_check_args(q, k, v, out, lse, B, H, S, D, scale, causal, window_left,
                                     window_right, dtype)


def fa_status_string(status: int) -> str:
    return _load().fa_status_string(int(status)).decode()


def fa_fwd_tile_schedule(S: int, D: int, dtype: int, causal: int, window_left: int,
                         window_right: int, q_tile: int) -> dict:
    """Host view of the K/V tiles the kernel visits for one Q tile."""
    lib = _load()
    vals = [ctypes.c_int64() for _ in range(5)]
    rc = lib.fa_fwd_tile_schedule(S, D, dtype, causal, window_left, window_right, q_tile,
                                  *[ctypes.byref(x) for x in vals], None, 0)
    if rc != 0:
        raise FaError(rc, "fa_fwd_tile_schedule")
    bm, bn, nq, t0, t1 = (x.value for x in vals)
    mask = (ctypes.c_uint8 * max(1, t1 - t0))()
    rc = lib.fa_fwd_tile_schedule(S, D, dtype, causal, window_left, window_right, q_tile,
                                  *[ctypes.byref(x) for x in vals], mask, t1 - t0)
    if rc != 0:
        raise FaError(rc, "fa_fwd_tile_schedule")
    return {"bm": bm, "bn": bn, "n_q_tiles": nq, "kt_begin": t0, "kt_end": t1,
            "needs_mask": [int(mask[i]) for i in range(t1 - t0)]}


def fa_fwd_workgroup_tile(B: int, H: int, S: int, D: int, dtype: int, causal: int,
                          window_left: int, window_right: int, wg: int) -> tuple[int, int]:
    """Host view of the launch order: (b * H + h, Q tile) of workgroup ``wg``."""
    bh, qt = ctypes.c_int64(), ctypes.c_int64()
    rc = _load().fa_fwd_workgroup_tile(B, H, S, D, dtype, causal, window_left, window_right, wg,
                                       ctypes.byref(bh), ctypes.byref(qt))
    if rc != 0:
        raise FaError(rc, "fa_fwd_workgroup_tile")
    return bh.value, qt.value


def fa_fwd_launch_order(B: int, H: int, S: int, D: int, dtype: int, causal: int,
                        window_left: int, window_right: int, n_cus: int,
                        wg: int) -> tuple[int, int, int]:
    """Host view of the launch order on a device of ``n_cus`` compute units:
    (b * H + h, Q tile, first dynamic workgroup or -1) of workgroup ``wg``."""
    bh, qt, first = ctypes.c_int64(), ctypes.c_int64(), ctypes.c_int64()
    rc = _load().fa_fwd_launch_order(B, H, S, D, dtype, causal, window_left, window_right, n_cus,
                                     wg, ctypes.byref(bh), ctypes.byref(qt), ctypes.byref(first))
    if rc != 0:
        raise FaError(rc, "fa_fwd_launch_order")
    return bh.value, qt.value, first.value


def fa_fwd_splitkv_workgroup_tile(B: int, H: int, S: int, D: int, dtype: int, causal: int,
                                  window_left: int, window_right: int, n_splits: int,
                                  wg: int) -> tuple[int, int, int]:
    """Host view of the split launch order: (b * H + h, Q tile, part) of workgroup ``wg``."""
    bh, qt, part = ctypes.c_int64(), ctypes.c_int64(), ctypes.c_int64()
    rc = _load().fa_fwd_splitkv_workgroup_tile(B, H, S, D, dtype, causal, window_left,
                                               window_right, n_splits, wg, ctypes.byref(bh),
                                               ctypes.byref(qt), ctypes.byref(part))
    if rc != 0:
        raise FaError(rc, "fa_fwd_splitkv_workgroup_tile")
    return bh.value, qt.value, part.value


def fa_fwd_splitkv(q: int, k: int, v: int, out: int, lse: int, B: int, H: int, S: int, D: int,
                   scale: float, causal: int, window_left: int, window_right: int, dtype: int,
                   n_splits: int, workspace: int, workspace_bytes: int, stream: int | None) -> int:
    """The split-KV C entry point with raw device pointers (ints); returns the status."""
    return _load().fa_fwd_splitkv(q, k, v, out, lse, B, H, S, D, scale, causal, window_left,
                                  window_right, dtype, n_splits, workspace, workspace_bytes,
                                  stream)


def fa_fwd_splitkv_workspace_size(B: int, H: int, S: int, D: int, dtype: int,
                                  n_splits: int) -> int:
    n = ctypes.c_int64()
    rc = _load().fa_fwd_splitkv_workspace_size(B, H, S, D, dtype, n_splits, ctypes.byref(n))
    if rc != 0:
        raise FaError(rc, "fa_fwd_splitkv_workspace_size")
    return n.value


def fa_fwd_splitkv_auto_splits(B: int, H: int, S: int, D: int, causal: int, window_left: int,
                               window_right: int, dtype: int) -> int:
    n = ctypes.c_int64()
    rc = _load().fa_fwd_splitkv_auto_splits(B, H, S, D, causal, window_left, window_right, dtype,
                                            ctypes.byref(n))
    if rc != 0:
        raise FaError(rc, "fa_fwd_splitkv_auto_splits")
    return n.value


def fa_bwd(q: int, k: int, v: int, out: int, lse: int, dout: int, dq: int, dk: int, dv: int,
           B: int, H: int, S: int, D: int, scale: float, causal: int, window_left: int,
           window_right: int, dtype: int, workspace: int, workspace_bytes: int,
           stream: int | None) -> int:
    """The backward C entry point with raw device pointers (ints); returns the status."""
    return _load().fa_bwd(q, k, v, out, lse, dout, dq, dk, dv, B, H, S, D, scale, causal,
                          window_left, window_right, dtype, workspace, workspace_bytes, stream)


def fa_bwd_workspace_size(B: int, H: int, S: int, D: int, dtype: int) -> int:
    n = ctypes.c_int64()
    rc = _load().fa_bwd_workspace_size(B, H, S, D, dtype, ctypes.byref(n))
    if rc != 0:
        raise FaError(rc, "fa_bwd_workspace_size")
    return n.value


def fa_fwd_blocksparse(q: int, k: int, v: int, out: int, lse: int, B: int, H: int, S: int, D: int,
                       scale: float, causal: int, window_left: int, window_right: int, dtype: int,
                       block_mask: int, n_mask: int, block_m: int, block_n: int, workspace: int,
                       workspace_bytes: int, stream: int | None) -> int:
    """The block-sparse C entry point with raw device pointers (ints); returns the status."""
    return _load().fa_fwd_blocksparse(q, k, v, out, lse, B, H, S, D, scale, causal, window_left,
                                      window_right, dtype, block_mask, n_mask, block_m, block_n,
                                      workspace, workspace_bytes, stream)


def fa_fwd_blocksparse_workspace_size(B: int, H: int, S: int, D: int, dtype: int,
                                      n_mask: int) -> int:
    n = ctypes.c_int64()
    rc = _load().fa_fwd_blocksparse_workspace_size(B, H, S, D, dtype, n_mask, ctypes.byref(n))
    if rc != 0:
        raise FaError(rc, "fa_fwd_blocksparse_workspace_size")
    return n.value


def fa_fwd_paged(q: int, k_pages: int, v_pages: int, block_table: int, out: int, lse: int, B: int,
                 H: int, S: int, D: int, scale: float, causal: int, window_left: int,
                 window_right: int, dtype: int, num_pages: int, page_size: int,
                 table_stride: int, n_splits: int, workspace: int, workspace_bytes: int,
                 stream: int | None) -> int:
    """The paged-K/V C entry point with raw device pointers (ints); returns the status."""
    return _load().fa_fwd_paged(q, k_pages, v_pages, block_table, out, lse, B, H, S, D, scale,
                                causal, window_left, window_right, dtype, num_pages, page_size,
                                table_stride, n_splits, workspace, workspace_bytes, stream)


def fa_fwd_kvcache(q: int, k_cache: int, v_cache: int, cache_seqlens: int, block_table: int | None,
                   out: int, lse: int, B: int, H: int, S_q: int, S_k: int, D: int, scale: float,
                   causal: int, window_left: int, window_right: int, dtype: int, num_pages: int,
                   page_size: int, table_stride: int, n_splits: int, workspace: int | None,
                   workspace_bytes: int, stream: int | None) -> int:
    """The KV-cache C entry point with raw device pointers (ints); returns the status."""
    return _load().fa_fwd_kvcache(q, k_cache, v_cache, cache_seqlens, block_table, out, lse, B, H,
                                  S_q, S_k, D, scale, causal, window_left, window_right, dtype,
                                  num_pages, page_size, table_stride, n_splits, workspace,
                                  workspace_bytes, stream)


def fa_fwd_kvcache_workspace_size(B: int, H: int, S_q: int, D: int, dtype: int,
                                  n_splits: int) -> int:
    n = ctypes.c_int64()
    rc = _load().fa_fwd_kvcache_workspace_size(B, H, S_q, D, dtype, n_splits, ctypes.byref(n))
    if rc != 0:
        raise FaError(rc, "fa_fwd_kvcache_workspace_size")
    return n.value


def fa_fwd_kvcache_auto_splits(B: int, H: int, S_q: int, S_k: int, D: int, dtype: int) -> int:
    n = ctypes.c_int64()
    rc = _load().fa_fwd_kvcache_auto_splits(B, H, S_q, S_k, D, dtype, ctypes.byref(n))
    if rc != 0:
        raise FaError(rc, "fa_fwd_kvcache_auto_splits")
    return n.value


def fa_fwd_splitkv_noalloc(q: int, k: int, v: int, out: int, lse: int, B: int, H: int, S: int,
                           D: int, scale: float, causal: int, window_left: int, window_right: int,
                           dtype: int, n_splits: int, stream: int | None) -> int:
    """The split-KV C entry point that keeps its partials in the library's static
    device buffer (no workspace, no allocation); raw device pointers; returns
    the status."""
    return _load().fa_fwd_splitkv_noalloc(q, k, v, out, lse, B, H, S, D, scale, causal,
                                          window_left, window_right, dtype, n_splits, stream)


# ------------------------------------------------------------------ tensor call
# Every tensor whose data pointer reaches the C ABI is checked here first:
# type, device (q's device -- a host tensor or one on another GPU would hand
# the kernels an address they cannot reach), dtype, shape and contiguity.
# Nothing is launched before these checks pass.
def _dtype_code(t) -> int:
    import torch

    codes = {torch.float32: FA_DTYPE_FP32, torch.float16: FA_DTYPE_FP16,
             torch.bfloat16: FA_DTYPE_BF16}
    if t.dtype not in codes:
        raise TypeError(f"unsupported dtype {t.dtype} (fp32, fp16, bf16)")
    return codes[t.dtype]


def _check_q(q):
    import torch

    if not isinstance(q, torch.Tensor) or q.device.type != "cuda":
        raise TypeError("q must be a GPU tensor")
    if q.dim() != 4:
        raise ValueError("q must be [B, S, H, D]")
    if not q.is_contiguous():
        raise ValueError("q must be contiguous [B, S, H, D]")


def _check_like(name, t, q, shape=None, dtype=None):
    """``t`` is a contiguous tensor on q's device, of ``dtype`` (q's by default)
    and ``shape`` (q's by default)."""
    import torch

    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch tensor")
    if t.device != q.device:
        raise ValueError(f"{name} is on {t.device}; it must be on q's device {q.device}")
    want_shape = tuple(q.shape) if shape is None else tuple(shape)
    want_dtype = q.dtype if dtype is None else dtype
    if tuple(t.shape) != want_shape or t.dtype != want_dtype:
        raise ValueError(f"{name} must be {want_dtype} {list(want_shape)}, got {t.dtype} "
                         f"{list(t.shape)}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def _check_qkv(q, k, v):
    _check_q(q)
    _check_like("k", k, q)
    _check_like("v", v, q)


def _outputs(q, out, lse, rows=None):
    """out (like q) and lse (fp32 [B, H, rows]), allocated when None, checked
    otherwise."""
    import torch

    B, S, H, _ = q.shape
    rows = S if rows is None else rows
    out = torch.empty_like(q) if out is None else out
    lse = torch.empty((B, H, rows), dtype=torch.float32, device=q.device) if lse is None else lse
    _check_like("out", out, q)
    _check_like("lse", lse, q, shape=(B, H, rows), dtype=torch.float32)
    return out, lse


def _workspace(workspace, need: int, q, dtype, stream=None):
    """(pointer or None, bytes, tensor) of a caller's workspace (a contiguous
    tensor on q's device; the library checks its size), or of one allocated
    here when None and ``need`` > 0.  An allocated workspace is marked as used
    by ``stream``, so torch does not hand its memory out again before the
    launch on that stream has run."""
    import torch

    if workspace is None:
        if need <= 0:
            return None, 0, None
        workspace = torch.empty((need + 3) // 4, dtype=dtype, device=q.device)
        if stream is not None:
            workspace.record_stream(stream)
    if not isinstance(workspace, torch.Tensor):
        raise TypeError("workspace must be a torch tensor")
    if workspace.device != q.device:
        raise ValueError(f"workspace is on {workspace.device}; it must be on q's device {q.device}")
    if not workspace.is_contiguous():
        raise ValueError("workspace must be contiguous")
    nbytes = workspace.numel() * workspace.element_size()
    return (workspace.data_ptr() or None), nbytes, workspace


def _stream(stream, q):
    import torch

    return (stream if stream is not None else torch.cuda.current_stream(q.device)).cuda_stream


def flash_attn_fwd(q, k, v, softmax_scale: float | None = None, causal: bool = False,
                   window_size=(-1, -1), out=None, lse=None, dropout_p: float = 0.0,
                   alibi_slopes=None, stream=None):
    """Exact attention forward on the GPU.

    q, k, v: CUDA (HIP) tensors [B, S, H, D], contiguous, one dtype (fp32,
    fp16 or bf16); D a multiple of 16 from 16 to 256 for fp16 / bf16, up to
    128 for fp32.  softmax_scale None means 1/sqrt(D).
    Returns (out [B, S, H, D] in the input dtype, lse [B, H, S] fp32).  Runs
    on ``stream`` (a torch stream) or torch's current stream, asynchronously.
    """
    if dropout_p != 0.0:
        raise NotImplementedError("dropout is not part of the exact forward pass")
    if alibi_slopes is not None:
        raise NotImplementedError("ALiBi slopes are not supported")
    import torch

    _check_qkv(q, k, v)
    B, S, H, D = q.shape
    dtype = _dtype_code(q)
    scale = 1.0 / math.sqrt(D) if softmax_scale is None else float(softmax_scale)
    out, lse = _outputs(q, out, lse)
    wl, wr = (int(x) for x in window_size)
    with torch.cuda.device(q.device):
        rc = fa_fwd(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(), lse.data_ptr(), B, H,
                    S, D, scale, int(bool(causal)), wl, wr, dtype, _stream(stream, q))
    if rc != 0:
        raise FaError(rc, "fa_fwd")
    return out, lse


def flash_attn_fwd_splitkv(q, k, v, softmax_scale: float | None = None, causal: bool = False,
                           window_size=(-1, -1), n_splits: int = 0, out=None, lse=None,
                           workspace=None, stream=None):
    """flash_attn_fwd with the K/V tiles of each Q tile split into ``n_splits``
    parts (0 = the library's choice for the current device) and merged.  The
    fp32 workspace is a torch tensor on q's device of at least the size
    fa_fwd_splitkv_workspace_size reports (allocated here when None).
    Returns (out, lse) like flash_attn_fwd."""
    import torch

    _check_qkv(q, k, v)
    B, S, H, D = q.shape
    dtype = _dtype_code(q)
    scale = 1.0 / math.sqrt(D) if softmax_scale is None else float(softmax_scale)
    wl, wr = (int(x) for x in window_size)
    with torch.cuda.device(q.device):
        if n_splits == 0:
            n_splits = fa_fwd_splitkv_auto_splits(B, H, S, D, int(bool(causal)), wl, wr, dtype)
        need = fa_fwd_splitkv_workspace_size(B, H, S, D, dtype, n_splits)
    out, lse = _outputs(q, out, lse)
    ws_ptr, ws_bytes, _ws = _workspace(workspace, need, q, torch.float32, stream)
    with torch.cuda.device(q.device):
        rc = fa_fwd_splitkv(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(),
                            lse.data_ptr(), B, H, S, D, scale, int(bool(causal)), wl, wr, dtype,
                            n_splits, ws_ptr, ws_bytes, _stream(stream, q))
    if rc != 0:
        raise FaError(rc, "fa_fwd_splitkv")
    return out, lse


def flash_attn_fwd_blocksparse(q, k, v, block_mask, block_m: int, block_n: int,
                               softmax_scale: float | None = None, causal: bool = False,
                               window_size=(-1, -1), out=None, lse=None, workspace=None,
                               stream=None):
    """flash_attn_fwd restricted to the blocks ``block_mask`` keeps: key j is
    allowed for query i of head (b, h) only where
    block_mask[hm, i // block_m, j // block_n] != 0 (hm = 0, h or b * H + h
    for a mask of 1, H or B * H matrices).  block_mask: a contiguous uint8 or
    bool GPU tensor [n_mask, ceil(S / block_m), ceil(S / block_n)] (2-D means
    n_mask = 1); block_m a multiple of 128, block_n of 64.  The workspace (the
    list of kept tiles) is a GPU tensor of at least
    fa_fwd_blocksparse_workspace_size bytes, allocated here when None.
    Returns (out, lse) like flash_attn_fwd."""
    import torch

    _check_qkv(q, k, v)
    if not isinstance(block_mask, torch.Tensor) or block_mask.device != q.device:
        raise ValueError("block_mask must be a tensor on q's device")
    if block_mask.dtype not in (torch.uint8, torch.bool) or not block_mask.is_contiguous():
        raise ValueError("block_mask must be a contiguous uint8 or bool tensor")
    mask = block_mask.view(torch.uint8) if block_mask.dtype == torch.bool else block_mask
    if mask.dim() == 2:
        mask = mask.unsqueeze(0)
    B, S, H, D = q.shape
    n_qb, n_kb = -(-S // int(block_m)), -(-S // int(block_n))
    if mask.dim() != 3 or tuple(mask.shape[1:]) != (n_qb, n_kb):
        raise ValueError(f"block_mask must be [n_mask, {n_qb}, {n_kb}] for S={S}, "
                         f"block_m={block_m}, block_n={block_n}")
    n_mask = mask.shape[0]
    dtype = _dtype_code(q)
    scale = 1.0 / math.sqrt(D) if softmax_scale is None else float(softmax_scale)
    wl, wr = (int(x) for x in window_size)
    need = fa_fwd_blocksparse_workspace_size(B, H, S, D, dtype, n_mask)
    out, lse = _outputs(q, out, lse)
    ws_ptr, ws_bytes, _ws = _workspace(workspace, need, q, torch.int32, stream)
    with torch.cuda.device(q.device):
        rc = fa_fwd_blocksparse(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(),
                                lse.data_ptr(), B, H, S, D, scale, int(bool(causal)), wl, wr,
                                dtype, mask.data_ptr(), n_mask, int(block_m), int(block_n),
                                ws_ptr, ws_bytes, _stream(stream, q))
    if rc != 0:
        raise FaError(rc, "fa_fwd_blocksparse")
    return out, lse


def _check_pools(q, k_pages, v_pages):
    import torch

    _, _, H, D = q.shape
    for name, t in (("k_pages", k_pages), ("v_pages", v_pages)):
        if not isinstance(t, torch.Tensor):
            raise TypeError(f"{name} must be a torch tensor")
        if t.device != q.device:
            raise ValueError(f"{name} is on {t.device}; it must be on q's device {q.device}")
        if t.dtype != q.dtype:
            raise ValueError(f"{name} must have q's dtype {q.dtype}")
        if t.dim() != 4 or t.shape != k_pages.shape or tuple(t.shape[2:]) != (H, D):
            raise ValueError(f"{name} must be [num_pages, page_size, H, D] like the other pool")
        if not t.is_contiguous():
            raise ValueError(f"{name} must be contiguous")


def _check_table(name, t, q, rows: int):
    import torch

    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch tensor")
    if t.device != q.device:
        raise ValueError(f"{name} is on {t.device}; it must be on q's device {q.device}")
    if t.dtype != torch.int32 or t.dim() != 2 or t.shape[0] != rows or not t.is_contiguous():
        raise ValueError(f"{name} must be a contiguous int32 tensor [{rows}, n]")


def flash_attn_fwd_paged(q, k_pages, v_pages, block_table, softmax_scale: float | None = None,
                         causal: bool = False, window_size=(-1, -1), n_splits: int = 1, out=None,
                         lse=None, workspace=None, stream=None):
    """flash_attn_fwd with keys and values in a paged cache: k_pages and
    v_pages are contiguous GPU tensors [num_pages, page_size, H, D] (page_size
    a multiple of 64) and block_table an int32 GPU tensor [B, n] with
    n >= ceil(S / page_size): key j of batch b is row j % page_size of page
    block_table[b, j // page_size].  ``n_splits`` > 1 runs the split-KV path
    (0 = the library's choice); its fp32 workspace is allocated here when
    None.  Returns (out, lse) like flash_attn_fwd."""
    import torch

    _check_q(q)
    B, S, H, D = q.shape
    _check_pools(q, k_pages, v_pages)
    _check_table("block_table", block_table, q, B)
    num_pages, page_size = k_pages.shape[0], k_pages.shape[1]
    dtype = _dtype_code(q)
    scale = 1.0 / math.sqrt(D) if softmax_scale is None else float(softmax_scale)
    wl, wr = (int(x) for x in window_size)
    with torch.cuda.device(q.device):
        if n_splits == 0:
            n_splits = fa_fwd_splitkv_auto_splits(B, H, S, D, int(bool(causal)), wl, wr, dtype)
        need = fa_fwd_splitkv_workspace_size(B, H, S, D, dtype, n_splits)
    out, lse = _outputs(q, out, lse)
    ws_ptr, ws_bytes, _ws = _workspace(workspace, need, q, torch.float32, stream)
    with torch.cuda.device(q.device):
        rc = fa_fwd_paged(q.data_ptr(), k_pages.data_ptr(), v_pages.data_ptr(),
                          block_table.data_ptr(), out.data_ptr(), lse.data_ptr(), B, H, S, D,
                          scale, int(bool(causal)), wl, wr, dtype, num_pages, page_size,
                          block_table.shape[1], n_splits, ws_ptr, ws_bytes, _stream(stream, q))
    if rc != 0:
        raise FaError(rc, "fa_fwd_paged")
    return out, lse


def flash_attn_fwd_kvcache(q, k_cache, v_cache, cache_seqlens, block_table=None,
                           softmax_scale: float | None = None, causal: bool = False,
                           window_size=(-1, -1), n_splits: int = 0, out=None, lse=None,
                           workspace=None, stream=None):
    """Attention of new queries against a key/value cache (decoding).

    q: GPU tensor [B, S_q, H, D] (bf16 or fp16).  Without ``block_table``,
    k_cache and v_cache are contiguous [B, S_k, H, D] caches; with it (an
    int32 [B, n] GPU tensor), they are page pools [num_pages, page_size, H, D]
    and key j of sequence b is row j % page_size of page block_table[b, j //
    page_size].  cache_seqlens: int32 GPU tensor [B], the rows of each
    sequence's cache that hold its keys (the new tokens' own included); query
    i of sequence b sits at position cache_seqlens[b] - S_q + i.  ``n_splits``
    parts per query block (0 = the library's choice for the device); the fp32
    workspace is allocated here when None.  Returns (out [B, S_q, H, D],
    lse [B, H, S_q] fp32)."""
    import torch

    _check_q(q)
    B, S_q, H, D = q.shape
    paged = block_table is not None
    if paged:
        _check_pools(q, k_cache, v_cache)
        _check_table("block_table", block_table, q, B)
        num_pages, page_size = k_cache.shape[0], k_cache.shape[1]
        table_stride = block_table.shape[1]
        S_k = table_stride * page_size
    else:
        if not isinstance(k_cache, torch.Tensor) or k_cache.dim() != 4 or k_cache.shape[0] != B:
            raise ValueError("k_cache must be a [B, S_k, H, D] tensor")
        S_k = k_cache.shape[1]
        _check_like("k_cache", k_cache, q, shape=(B, S_k, H, D))
        _check_like("v_cache", v_cache, q, shape=(B, S_k, H, D))
        num_pages = page_size = table_stride = 0
    _check_like("cache_seqlens", cache_seqlens, q, shape=(B,), dtype=torch.int32)
    dtype = _dtype_code(q)
    scale = 1.0 / math.sqrt(D) if softmax_scale is None else float(softmax_scale)
    wl, wr = (int(x) for x in window_size)
    with torch.cuda.device(q.device):
        if n_splits == 0:
            n_splits = fa_fwd_kvcache_auto_splits(B, H, S_q, S_k, D, dtype)
        need = fa_fwd_kvcache_workspace_size(B, H, S_q, D, dtype, n_splits)
    out, lse = _outputs(q, out, lse)
    ws_ptr, ws_bytes, _ws = _workspace(workspace, need, q, torch.float32, stream)
    with torch.cuda.device(q.device):
        rc = fa_fwd_kvcache(q.data_ptr(), k_cache.data_ptr(), v_cache.data_ptr(),
                            cache_seqlens.data_ptr(), block_table.data_ptr() if paged else None,
                            out.data_ptr(), lse.data_ptr(), B, H, S_q, S_k, D, scale,
                            int(bool(causal)), wl, wr, dtype, num_pages, page_size, table_stride,
                            n_splits, ws_ptr, ws_bytes, _stream(stream, q))
    if rc != 0:
        raise FaError(rc, "fa_fwd_kvcache")
    return out, lse


def flash_attn_bwd(dout, q, k, v, out, lse, softmax_scale: float | None = None,
                   causal: bool = False, window_size=(-1, -1), workspace=None, dq=None, dk=None,
                   dv=None, stream=None):
    """Gradients (dq, dk, dv) of flash_attn_fwd's output for the output
    gradient ``dout``, given the forward's q, k, v and its out and lse.
    bf16 / fp16 tensors [B, S, H, D]; the workspace (fa_bwd_workspace_size
    bytes) and the gradients are allocated here when None."""
    import torch

    _check_qkv(q, k, v)
    _check_like("dout", dout, q)
    _check_like("out", out, q)
    B, S, H, D = q.shape
    _check_like("lse", lse, q, shape=(B, H, S), dtype=torch.float32)
    dtype = _dtype_code(q)
    scale = 1.0 / math.sqrt(D) if softmax_scale is None else float(softmax_scale)
    wl, wr = (int(x) for x in window_size)
    dq = torch.empty_like(q) if dq is None else dq
    dk = torch.empty_like(k) if dk is None else dk
    dv = torch.empty_like(v) if dv is None else dv
    for name, t in (("dq", dq), ("dk", dk), ("dv", dv)):
        _check_like(name, t, q)
    need = fa_bwd_workspace_size(B, H, S, D, dtype)
    ws_ptr, ws_bytes, _ws = _workspace(workspace, need, q, torch.float32, stream)
    with torch.cuda.device(q.device):
        rc = fa_bwd(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(), lse.data_ptr(),
                    dout.data_ptr(), dq.data_ptr(), dk.data_ptr(), dv.data_ptr(), B, H, S, D,
                    scale, int(bool(causal)), wl, wr, dtype, ws_ptr, ws_bytes,
                    _stream(stream, q))
    if rc != 0:
        raise FaError(rc, "fa_bwd")
    return dq, dk, dv
