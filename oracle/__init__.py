"""CPU oracle for exact attention (forward and backward): plain, slow, fp64.

TEST INFRASTRUCTURE, NOT PRODUCT CODE.  Only ``tests/``, ``__graft_entry__.smoke()``
and the ``cpu_baseline`` leg of ``bench.py`` may import this package.  It shares
no code with the GPU library (``io_aware_exact_22_amd``) and imports nothing
from it; the two meet only in the seeded input generator, which holds none of
the method's arithmetic.

The arithmetic lives in ``fa_oracle.c`` (the definition of exact attention,
materialising the score matrix in fp64, one head at a time).  This module only
builds and loads that file and marshals arguments to it.

Pages are cited by title: the formula is in "大模型加速新突破：Flash Attention V2
核心网络算子解析" section 二.1; the causal/window/scale arguments are in
"FlashAttention技术解析：加速GPT训练的核心优化" section 2.2.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
import threading

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "fa_oracle.c")
_LIB_PATH = os.path.join(_HERE, "libfa_oracle.so")
_lock = threading.Lock()
_lib = None

DTYPE_CODES = {"fp32": 0, "fp16": 1, "bf16": 2}


def build(force: bool = True) -> str:
    """Compile fa_oracle.c with gcc (CPU only) into libfa_oracle.so."""
    if not force and os.path.exists(_LIB_PATH) and os.path.getmtime(_LIB_PATH) >= os.path.getmtime(_SRC):
        return _LIB_PATH
    tmp = _LIB_PATH + ".tmp%d" % os.getpid()
    cmd = ["gcc", "-O2", "-std=c11", "-fopenmp", "-shared", "-fPIC", "-Wall", "-Wextra",
           _SRC, "-o", tmp, "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def _load():
    global _lib
    with _lock:
        if _lib is not None:
            return _lib
        override = os.environ.get("FA_ORACLE_LIB")  # a prebuilt variant, for the mutation tests
        if override:
            lib = ctypes.CDLL(override)
        else:
            build(force=False)
            lib = ctypes.CDLL(_LIB_PATH)
        i64, vp, dp = ctypes.c_int64, ctypes.c_void_p, ctypes.c_double
        lib.fa_oracle_fwd.argtypes = [vp, vp, vp, ctypes.c_int, i64, i64, i64, i64, dp,
                                      ctypes.c_int, i64, i64, vp, vp, ctypes.c_int]
        lib.fa_oracle_fwd.restype = ctypes.c_int
        lib.fa_oracle_fwd_rows.argtypes = [vp, vp, vp, ctypes.c_int, i64, i64, i64, i64, dp,
                                           ctypes.c_int, i64, i64, i64, i64, i64, i64, vp, vp,
                                           ctypes.c_int]
        lib.fa_oracle_fwd_rows.restype = ctypes.c_int
        lib.fa_oracle_allowed_pairs.argtypes = [i64, ctypes.c_int, i64, i64]
        lib.fa_oracle_allowed_pairs.restype = i64
        lib.fa_oracle_decode.argtypes = [vp, ctypes.c_int, i64, vp]
        lib.fa_oracle_decode.restype = ctypes.c_int
        lib.fa_oracle_bwd.argtypes = [vp, vp, vp, vp, ctypes.c_int, i64, i64, i64, i64, dp,
                                      ctypes.c_int, i64, i64, vp, vp, vp, ctypes.c_int]
        lib.fa_oracle_bwd.restype = ctypes.c_int
        lib.fa_oracle_fwd_blocksparse.argtypes = [vp, vp, vp, ctypes.c_int, i64, i64, i64, i64,
                                                  dp, ctypes.c_int, i64, i64, vp, i64, i64, i64,
                                                  vp, vp, ctypes.c_int]
        lib.fa_oracle_fwd_blocksparse.restype = ctypes.c_int
        lib.fa_oracle_fwd_rows_blocksparse.argtypes = [vp, vp, vp, ctypes.c_int, i64, i64, i64,
                                                       i64, dp, ctypes.c_int, i64, i64, vp, i64,
                                                       i64, i64, i64, i64, i64, i64, vp, vp,
                                                       ctypes.c_int]
        lib.fa_oracle_fwd_rows_blocksparse.restype = ctypes.c_int
        lib.fa_oracle_gather_pages.argtypes = [vp, i64, i64, i64, vp, i64, i64, i64, i64, i64, vp]
        lib.fa_oracle_gather_pages.restype = ctypes.c_int
        lib.fa_oracle_bwd_sampled.argtypes = [vp, vp, vp, vp, ctypes.c_int, i64, i64, i64, i64, dp,
                                              ctypes.c_int, i64, i64, i64, i64, vp, i64, vp, i64,
                                              vp, vp, vp, ctypes.c_int]
        lib.fa_oracle_bwd_sampled.restype = ctypes.c_int
        lib.fa_oracle_fwd_kvcache.argtypes = [vp, vp, vp, ctypes.c_int, i64, i64, i64, i64, i64,
                                              dp, ctypes.c_int, i64, i64, vp, vp, vp,
                                              ctypes.c_int]
        lib.fa_oracle_fwd_kvcache.restype = ctypes.c_int
        _lib = lib
        return lib


def _dtype_code(t) -> int:
    import torch

    codes = {torch.float32: 0, torch.float16: 1, torch.bfloat16: 2}
    if t.dtype not in codes:
        raise TypeError(f"oracle: unsupported dtype {t.dtype}")
    return codes[t.dtype]


def _check_inputs(q, k, v):
    import torch

    for name, t in (("q", q), ("k", k), ("v", v)):
        if not isinstance(t, torch.Tensor) or t.device.type != "cpu":
            raise TypeError(f"oracle: {name} must be a CPU torch tensor")
        if not t.is_contiguous():
            raise ValueError(f"oracle: {name} must be contiguous [B, S, H, D]")
        if t.dim() != 4 or t.shape != q.shape or t.dtype != q.dtype:
            raise ValueError("oracle: q, k, v must share shape [B, S, H, D] and dtype")


def _window(window_size):
    wl, wr = window_size
    return int(wl), int(wr)


def fwd(q, k, v, scale: float, causal: bool = False, window_size=(-1, -1), nthreads: int = 0):
    """Exact attention over all rows.  q, k, v: CPU tensors [B, S, H, D] in fp32,
    fp16 or bf16 (their bits are decoded exactly).  Returns (out [B,S,H,D] fp64,
    lse [B,H,S] fp64) as numpy arrays."""
    _check_inputs(q, k, v)
    lib = _load()
    B, S, H, D = q.shape
    wl, wr = _window(window_size)
    out = np.empty((B, S, H, D), dtype=np.float64)
    lse = np.empty((B, H, S), dtype=np.float64)
    rc = lib.fa_oracle_fwd(q.data_ptr(), k.data_ptr(), v.data_ptr(), _dtype_code(q), B, H, S, D,
                           float(scale), int(bool(causal)), wl, wr, out.ctypes.data,
                           lse.ctypes.data, int(nthreads))
    if rc != 0:
        raise ValueError(f"oracle: fa_oracle_fwd failed ({rc})")
    return out, lse


def fwd_rows(q, k, v, scale: float, causal: bool, window_size, b: int, h: int, i0: int, i1: int,
             nthreads: int = 0):
    """Exact attention for query rows [i0, i1) of head (b, h).  Returns
    (out [(i1-i0), D] fp64, lse [(i1-i0)] fp64)."""
    _check_inputs(q, k, v)
    lib = _load()
    B, S, H, D = q.shape
    wl, wr = _window(window_size)
    R = i1 - i0
    out = np.empty((max(R, 0), D), dtype=np.float64)
    lse = np.empty((max(R, 0),), dtype=np.float64)
    rc = lib.fa_oracle_fwd_rows(q.data_ptr(), k.data_ptr(), v.data_ptr(), _dtype_code(q), B, H, S,
                                D, float(scale), int(bool(causal)), wl, wr, b, h, i0, i1,
                                out.ctypes.data, lse.ctypes.data, int(nthreads))
    if rc != 0:
        raise ValueError(f"oracle: fa_oracle_fwd_rows failed ({rc})")
    return out, lse


def _check_mask(mask, B, H, S, block_m, block_n):
    """The block mask as a contiguous uint8 numpy array [n_mask, n_qb, n_kb]."""
    m = np.ascontiguousarray(np.asarray(mask), dtype=np.uint8)
    n_qb, n_kb = -(-S // block_m), -(-S // block_n)
    if m.ndim == 2:
        m = m[None]
    if m.ndim != 3 or m.shape[1:] != (n_qb, n_kb) or m.shape[0] not in (1, H, B * H):
        raise ValueError(f"oracle: block mask must be [1|H|B*H, {n_qb}, {n_kb}], got {m.shape}")
    return np.ascontiguousarray(m)


def fwd_blocksparse(q, k, v, scale: float, mask, block_m: int, block_n: int,
                    causal: bool = False, window_size=(-1, -1), nthreads: int = 0):
    """Block-sparse exact attention: ``fwd`` with key j allowed for query i only
    where mask[hm, i // block_m, j // block_n] != 0 ("FlashAttention技术解析：
    加速GPT训练的核心优化" section 5 lists the block-sparse variant).  mask:
    uint8/bool array [n_mask, ceil(S/block_m), ceil(S/block_n)] with n_mask in
    {1, H, B*H} (a 2-D mask is taken as n_mask = 1).  Returns (out, lse) as fwd."""
    _check_inputs(q, k, v)
    lib = _load()
    B, S, H, D = q.shape
    m = _check_mask(mask, B, H, S, block_m, block_n)
    wl, wr = _window(window_size)
    out = np.empty((B, S, H, D), dtype=np.float64)
    lse = np.empty((B, H, S), dtype=np.float64)
    rc = lib.fa_oracle_fwd_blocksparse(q.data_ptr(), k.data_ptr(), v.data_ptr(), _dtype_code(q),
                                       B, H, S, D, float(scale), int(bool(causal)), wl, wr,
                                       m.ctypes.data, m.shape[0], int(block_m), int(block_n),
                                       out.ctypes.data, lse.ctypes.data, int(nthreads))
    if rc != 0:
        raise ValueError(f"oracle: fa_oracle_fwd_blocksparse failed ({rc})")
    return out, lse


def fwd_rows_blocksparse(q, k, v, scale: float, mask, block_m: int, block_n: int, causal: bool,
                         window_size, b: int, h: int, i0: int, i1: int, nthreads: int = 0):
    """Block-sparse attention for query rows [i0, i1) of head (b, h); as fwd_rows."""
    _check_inputs(q, k, v)
    lib = _load()
    B, S, H, D = q.shape
    m = _check_mask(mask, B, H, S, block_m, block_n)
    wl, wr = _window(window_size)
    R = i1 - i0
    out = np.empty((max(R, 0), D), dtype=np.float64)
    lse = np.empty((max(R, 0),), dtype=np.float64)
    rc = lib.fa_oracle_fwd_rows_blocksparse(q.data_ptr(), k.data_ptr(), v.data_ptr(),
                                            _dtype_code(q), B, H, S, D, float(scale),
                                            int(bool(causal)), wl, wr, m.ctypes.data, m.shape[0],
                                            int(block_m), int(block_n), b, h, i0, i1,
                                            out.ctypes.data, lse.ctypes.data, int(nthreads))
    if rc != 0:
        raise ValueError(f"oracle: fa_oracle_fwd_rows_blocksparse failed ({rc})")
    return out, lse


def gather_pages(pages, block_table, S: int):
    """Contiguous [B, S, H, D] keys (or values) from a paged pool ``pages``
    [num_pages, page_size, H, D] (CPU tensor) and ``block_table`` [B, n] int32:
    row j of batch b is row j % page_size of page block_table[b, j // page_size]
    ("突破大模型训练瓶颈：Flash-Attention编译优化与内存占用解决方案", section Paged KV
    Cache支持, names the block table)."""
    import torch

    if not isinstance(pages, torch.Tensor) or pages.device.type != "cpu" or not pages.is_contiguous():
        raise TypeError("oracle: pages must be a contiguous CPU tensor")
    bt = np.ascontiguousarray(np.asarray(block_table), dtype=np.int32)
    if pages.dim() != 4 or bt.ndim != 2:
        raise ValueError("oracle: pages [num_pages, page_size, H, D], block_table [B, n]")
    num_pages, page_size, H, D = pages.shape
    B = bt.shape[0]
    dense = torch.empty((B, S, H, D), dtype=pages.dtype)
    rc = _load().fa_oracle_gather_pages(pages.data_ptr(), pages.element_size(), num_pages,
                                        page_size, bt.ctypes.data, bt.shape[1], B, S, H, D,
                                        dense.data_ptr())
    if rc != 0:
        raise ValueError("oracle: bad block table or page geometry")
    return dense


def fwd_paged(q, k_pages, v_pages, block_table, scale: float, causal: bool = False,
              window_size=(-1, -1), nthreads: int = 0):
    """Exact attention with keys and values in paged pools: the pools are
    gathered by the block table (gather_pages), then ``fwd`` runs on them.
    q: [B, S, H, D]; k_pages, v_pages: [num_pages, page_size, H, D]."""
    S = q.shape[1]
    k = gather_pages(k_pages, block_table, S)
    v = gather_pages(v_pages, block_table, S)
    return fwd(q, k, v, scale, causal, window_size, nthreads)


def fwd_kvcache(q, k_cache, v_cache, seqlens, scale: float, causal: bool = False,
                window_size=(-1, -1), nthreads: int = 0):
    """Attention of S_q new queries against a key/value cache (decoding):
    q [B, S_q, H, D]; k_cache, v_cache [B, S_k, H, D] of q's dtype; seqlens
    [B] ints, the valid rows L_b <= S_k of each sequence's cache.  Query i of
    sequence b sits at position L_b - S_q + i, and the causal / window masks
    apply to positions ("FlashAttention技术解析：加速GPT训练的核心优化" section 5
    names FlashDecoding for the KV cache of inference).  Returns (out
    [B, S_q, H, D] fp64, lse [B, H, S_q] fp64)."""
    _check_inputs(q, q, q)
    _check_inputs(k_cache, k_cache, v_cache)
    if k_cache.dtype != q.dtype or k_cache.shape[0] != q.shape[0] or \
            tuple(k_cache.shape[2:]) != tuple(q.shape[2:]):
        raise ValueError("oracle: the caches must be [B, S_k, H, D] of q's dtype")
    lib = _load()
    B, S_q, H, D = q.shape
    S_k = k_cache.shape[1]
    lens = np.ascontiguousarray(np.asarray(seqlens, dtype=np.int64))
    if lens.shape != (B,):
        raise ValueError("oracle: seqlens must hold one length per sequence")
    wl, wr = _window(window_size)
    out = np.empty((B, S_q, H, D), dtype=np.float64)
    lse = np.empty((B, H, S_q), dtype=np.float64)
    rc = lib.fa_oracle_fwd_kvcache(q.data_ptr(), k_cache.data_ptr(), v_cache.data_ptr(),
                                   _dtype_code(q), B, H, S_q, S_k, D, float(scale),
                                   int(bool(causal)), wl, wr, lens.ctypes.data, out.ctypes.data,
                                   lse.ctypes.data, int(nthreads))
    if rc != 0:
        raise ValueError(f"oracle: fa_oracle_fwd_kvcache failed ({rc})")
    return out, lse


def fwd_kvcache_paged(q, k_pages, v_pages, block_table, seqlens, S_k: int, scale: float,
                      causal: bool = False, window_size=(-1, -1), nthreads: int = 0):
    """fwd_kvcache with the caches in paged pools [num_pages, page_size, H, D]
    found through block_table [B, n]: sequence b's first L_b rows are gathered
    (gather_pages) into a contiguous cache of capacity S_k, the rest of which
    stays zero and is never read."""
    import torch

    bt = np.ascontiguousarray(np.asarray(block_table), dtype=np.int32)
    B = q.shape[0]
    _, _, H, D = k_pages.shape
    caches = []
    for pool in (k_pages, v_pages):
        dense = torch.zeros((B, S_k, H, D), dtype=pool.dtype)
        for b in range(B):
            L = int(seqlens[b])
            if L > 0:
                dense[b, :L] = gather_pages(pool, bt[b:b + 1], L)[0]
        caches.append(dense)
    return fwd_kvcache(q, caches[0], caches[1], seqlens, scale, causal, window_size, nthreads)


def bwd(q, k, v, dout, scale: float, causal: bool = False, window_size=(-1, -1),
        nthreads: int = 0):
    """Gradients of exact attention for the output gradient ``dout``: the chain
    rule through the forward definition, fp64 ("大模型加速新突破：Flash Attention
    V2核心网络算子解析" section 二.1 step 3 names this backward pass).  q, k, v,
    dout: CPU tensors [B, S, H, D] of one dtype.  Returns (dq, dk, dv), each
    [B, S, H, D] fp64 numpy."""
    _check_inputs(q, k, v)
    _check_inputs(q, dout, dout)
    lib = _load()
    B, S, H, D = q.shape
    wl, wr = _window(window_size)
    dq, dk, dv = (np.empty((B, S, H, D), dtype=np.float64) for _ in range(3))
    rc = lib.fa_oracle_bwd(q.data_ptr(), k.data_ptr(), v.data_ptr(), dout.data_ptr(),
                           _dtype_code(q), B, H, S, D, float(scale), int(bool(causal)), wl, wr,
                           dq.ctypes.data, dk.ctypes.data, dv.ctypes.data, int(nthreads))
    if rc != 0:
        raise ValueError(f"oracle: fa_oracle_bwd failed ({rc})")
    return dq, dk, dv


def bwd_sampled(q, k, v, dout, scale: float, causal: bool, window_size, b: int, h: int, rows,
                keys, nthreads: int = 0):
    """The gradients of ``bwd`` for the query ``rows`` (dq) and the ``keys`` (dk,
    dv) of head (b, h), without materialising the S x S matrices.  Returns
    (dq [len(rows), D], dk [len(keys), D], dv [len(keys), D]) fp64 numpy."""
    _check_inputs(q, k, v)
    _check_inputs(q, dout, dout)
    lib = _load()
    B, S, H, D = q.shape
    wl, wr = _window(window_size)
    r = np.ascontiguousarray(np.asarray(rows, dtype=np.int64))
    c = np.ascontiguousarray(np.asarray(keys, dtype=np.int64))
    dq = np.empty((len(r), D)); dk = np.empty((len(c), D)); dv = np.empty((len(c), D))
    rc = lib.fa_oracle_bwd_sampled(q.data_ptr(), k.data_ptr(), v.data_ptr(), dout.data_ptr(),
                                   _dtype_code(q), B, H, S, D, float(scale), int(bool(causal)), wl,
                                   wr, b, h, r.ctypes.data, len(r), c.ctypes.data, len(c),
                                   dq.ctypes.data, dk.ctypes.data, dv.ctypes.data, int(nthreads))
    if rc != 0:
        raise ValueError(f"oracle: fa_oracle_bwd_sampled failed ({rc})")
    return dq, dk, dv


def allowed_pairs(S: int, causal: bool, window_size=(-1, -1)) -> int:
    """Brute-force count of allowed (query, key) pairs, i.e. S * S_eff."""
    wl, wr = _window(window_size)
    return int(_load().fa_oracle_allowed_pairs(S, int(bool(causal)), wl, wr))


def decode(t) -> np.ndarray:
    """The oracle's own decoding of every element of a contiguous CPU tensor
    (fp32, fp16 or bf16) to fp64, flattened."""
    if not t.is_contiguous():
        raise ValueError("oracle: decode needs a contiguous tensor")
    out = np.empty((t.numel(),), dtype=np.float64)
    rc = _load().fa_oracle_decode(t.data_ptr(), _dtype_code(t), t.numel(), out.ctypes.data)
    if rc != 0:
        raise ValueError("oracle: decode failed")
    return out
