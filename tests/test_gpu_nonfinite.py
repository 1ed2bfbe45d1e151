"""Non-finite values at keys a row does not allow.

The definition sums each row over its allowed keys only, so a NaN or an
infinity in k_j or v_j reaches exactly the rows that allow key j (IEEE
propagation; "FlashAttention技术解析：加速GPT训练的核心优化" section 4.1 troubleshoots
NaN outputs).  The oracle skips the keys a row does not allow.  These tests
put NaN, +inf and -inf into v (and +-inf into k) on keys next to the causal
diagonal and at window edges -- keys that share a K/V tile with rows that do
not allow them -- and compare every element with the oracle: NaN where it is
NaN, the same infinity where it is infinite, and within the tolerances
elsewhere.  Every path is covered: fa_fwd (bf16, fp16, fp32), split-KV, paged
K/V and block-sparse.
"""
import math

import numpy as np
import pytest
import torch

import oracle
from fa_inputs import make_qkv, random_block_mask

pytestmark = pytest.mark.gpu

TOL_O = {torch.float32: 1e-4, torch.float16: 4e-3, torch.bfloat16: 2e-2}


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")


def poison(q, k, v):
    """NaN / +-inf planted at keys beside the causal diagonal and the edges of
    the windows used below, in both heads."""
    S = v.shape[1]
    v[0, 100, 0, 3] = float("nan")       # rows 96..99 share its tile but not the key (causal)
    v[0, 130, 0, 5] = float("inf")
    v[0, 37, 1, 9] = float("inf")        # +inf and -inf in one column: NaN where both allowed
    v[0, 38, 1, 9] = float("-inf")
    v[0, 200, 1, 0] = float("nan")
    k[0, 250, 0, 1] = float("inf")       # an infinite score: NaN or a zero weight
    k[0, 251, 1, 2] = float("-inf")
    v[0, S - 1, 0, 11] = float("-inf")   # the last key (ragged tail tile)
    return q, k, v


def compare(out, lse, ref_o, ref_l, dtype, what):
    o = out.double().cpu().numpy()
    ls = lse.double().cpu().numpy()
    for name, g, r, tol in (("O", o, ref_o, TOL_O[dtype]), ("LSE", ls, ref_l, 1e-3)):
        assert np.array_equal(np.isnan(g), np.isnan(r)), \
            f"{what}: {name} NaN pattern differs ({int(np.isnan(g).sum())} vs {int(np.isnan(r).sum())})"
        inf = np.isinf(r)
        assert np.array_equal(np.isinf(g), inf), f"{what}: {name} infinity pattern differs"
        assert np.array_equal(g[inf], r[inf]), f"{what}: {name} infinity signs differ"
        fin = np.isfinite(r)
        err = float(np.max(np.abs(g[fin] - r[fin]))) if fin.any() else 0.0
        assert err <= tol, f"{what}: {name} error {err} > {tol}"
    n_nan = int(np.isnan(ref_o).sum())
    print(f"{what}: NaN O elements {n_nan}, inf {int(np.isinf(ref_o).sum())}; pattern and values "
          f"match", flush=True)
    assert n_nan > 0  # the planted values did reach some rows


MASKS = [(True, (-1, -1)), (False, (16, 16)), (True, (50, -1)), (False, (-1, -1))]


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float16, torch.float32])
@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("causal,window", MASKS)
def test_nonfinite_fa_fwd(dtype, D, causal, window):
    import io_aware_exact_22_amd as fa

    q, k, v = poison(*make_qkv(1, 300, 2, D, dtype, 31))
    scale = 1.0 / math.sqrt(D)
    out, lse = fa.flash_attn_fwd(q.cuda(), k.cuda(), v.cuda(), softmax_scale=scale, causal=causal,
                                 window_size=window)
    torch.cuda.synchronize()
    ref_o, ref_l = oracle.fwd(q, k, v, scale, causal, window)
    compare(out, lse, ref_o, ref_l, dtype, f"fa_fwd {dtype} D{D} causal={causal} {window}")


@pytest.mark.parametrize("dtype,D,causal,window,n_splits", [
    (torch.bfloat16, 128, True, (-1, -1), 3), (torch.float16, 64, False, (16, 16), 2),
    (torch.bfloat16, 64, True, (50, -1), 4)])
def test_nonfinite_splitkv(dtype, D, causal, window, n_splits):
    import io_aware_exact_22_amd as fa

    q, k, v = poison(*make_qkv(1, 300, 2, D, dtype, 32))
    scale = 1.0 / math.sqrt(D)
    out, lse = fa.flash_attn_fwd_splitkv(q.cuda(), k.cuda(), v.cuda(), softmax_scale=scale,
                                         causal=causal, window_size=window, n_splits=n_splits)
    torch.cuda.synchronize()
    ref_o, ref_l = oracle.fwd(q, k, v, scale, causal, window)
    compare(out, lse, ref_o, ref_l, dtype, f"splitkv x{n_splits} {dtype} D{D} causal={causal}")


@pytest.mark.parametrize("dtype,n_splits", [(torch.bfloat16, 1), (torch.bfloat16, 2),
                                            (torch.float32, 1)])
def test_nonfinite_paged(dtype, n_splits):
    import io_aware_exact_22_amd as fa

    B, S, H, D, ps = 1, 300, 2, 128, 64
    q, k, v = poison(*make_qkv(B, S, H, D, dtype, 33))
    n_pg = -(-S // ps)
    perm = torch.randperm(n_pg + 2, generator=torch.Generator().manual_seed(5))[:n_pg]
    pools = []
    for t in (k, v):
        pool = torch.zeros((n_pg + 2, ps, H, D), dtype=dtype)
        pad = torch.zeros((n_pg * ps, H, D), dtype=dtype)
        pad[:S] = t[0]
        pool[perm] = pad.view(n_pg, ps, H, D)
        pools.append(pool.cuda())
    table = perm.view(1, n_pg).to(torch.int32).cuda()
    scale = 1.0 / math.sqrt(D)
    out, lse = fa.flash_attn_fwd_paged(q.cuda(), pools[0], pools[1], table, softmax_scale=scale,
                                       causal=True, n_splits=n_splits)
    torch.cuda.synchronize()
    ref_o, ref_l = oracle.fwd(q, k, v, scale, True, (-1, -1))
    compare(out, lse, ref_o, ref_l, dtype, f"paged x{n_splits} {dtype}")


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
def test_nonfinite_blocksparse(dtype):
    import io_aware_exact_22_amd as fa

    B, S, H, D = 1, 300, 2, 128
    q, k, v = poison(*make_qkv(B, S, H, D, dtype, 34))
    mask = random_block_mask(1, 3, 5, 0.7, 9)
    mask[0, :, 0] = 1
    scale = 1.0 / math.sqrt(D)
    out, lse = fa.flash_attn_fwd_blocksparse(q.cuda(), k.cuda(), v.cuda(), mask.cuda(), 128, 64,
                                             softmax_scale=scale, causal=True)
    torch.cuda.synchronize()
    ref_o, ref_l = oracle.fwd_blocksparse(q, k, v, scale, mask.numpy(), 128, 64, True)
    compare(out, lse, ref_o, ref_l, dtype, f"blocksparse {dtype}")
