"""fa_fwd_splitkv_noalloc (the split-KV forward that keeps its partials in the
library's static device buffer) through the C ABI, against fa_fwd_splitkv with
a caller's workspace: the same kernels, so bit for bit the same outputs -- on
two calls in a row, the second smaller than the first (the buffer keeps the
first call's partials), and within tolerance of the oracle."""
import math

import numpy as np
import pytest
import torch

import oracle
from fa_inputs import make_qkv

pytestmark = pytest.mark.gpu

TOL_O = {torch.float16: 4e-3, torch.bfloat16: 2e-2}
DT = {torch.float16: 1, torch.bfloat16: 2}


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")


def _noalloc(q, k, v, scale, causal, window, n_splits, stream):
    import io_aware_exact_22_amd as fa

    B, S, H, D = q.shape
    out = torch.full_like(q, float("nan"))
    lse = torch.full((B, H, S), float("nan"), dtype=torch.float32, device=q.device)
    rc = fa.fa_fwd_splitkv_noalloc(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(),
                                   lse.data_ptr(), B, H, S, D, scale, int(causal), window[0],
                                   window[1], DT[q.dtype], n_splits, stream.cuda_stream)
    assert rc == 0, fa.fa_status_string(rc)
    return out, lse


def _with_workspace(q, k, v, scale, causal, window, n_splits, stream):
    import io_aware_exact_22_amd as fa

    B, S, H, D = q.shape
    need = fa.fa_fwd_splitkv_workspace_size(B, H, S, D, DT[q.dtype], n_splits)
    ws = torch.full(((need + 3) // 4,), float("nan"), dtype=torch.float32, device=q.device)
    return fa.flash_attn_fwd_splitkv(q, k, v, softmax_scale=scale, causal=causal,
                                     window_size=window, n_splits=n_splits, workspace=ws,
                                     stream=stream)


# (B, S, H, D, dtype, causal, window, n_splits): the first call is the larger one
CALLS = [
    [(2, 3000, 6, 128, torch.bfloat16, True, (-1, -1), 4),
     (1, 700, 2, 64, torch.float16, False, (100, 30), 3)],
    [(1, 4097, 8, 64, torch.float16, False, (-1, -1), 5),
     (2, 389, 3, 128, torch.bfloat16, True, (64, -1), 2)],
    # head dimensions other than 64 and 128 (D = 256 and a padded 48)
    [(1, 2000, 4, 256, torch.bfloat16, True, (-1, -1), 3),
     (2, 500, 3, 48, torch.float16, False, (100, 30), 2)],
]


@pytest.mark.parametrize("calls", CALLS)
def test_noalloc_matches_workspace_entry_point(calls):
    dev = torch.device("cuda:0")
    stream = torch.cuda.current_stream(dev)
    for i, (B, S, H, D, dtype, causal, window, ns) in enumerate(calls):
        print(f"call {i}: B{B} S{S} H{H} D{D} {dtype} causal={causal} window={window} "
              f"n_splits={ns}", flush=True)
        q, k, v = make_qkv(B, S, H, D, dtype, 900 + i)
        qd, kd, vd = (t.to(dev) for t in (q, k, v))
        scale = 1.0 / math.sqrt(D)
        out, lse = _noalloc(qd, kd, vd, scale, causal, window, ns, stream)
        ref_out, ref_lse = _with_workspace(qd, kd, vd, scale, causal, window, ns, stream)
        torch.cuda.synchronize()
        assert torch.equal(out.view(torch.int16), ref_out.view(torch.int16)), "O differs"
        assert torch.equal(lse.view(torch.int32), ref_lse.view(torch.int32)), "LSE differs"
        oo, ol = oracle.fwd(q, k, v, scale, causal, window)
        eo = float(np.max(np.abs(out.cpu().double().numpy() - oo)))
        el = float(np.max(np.abs(lse.cpu().double().numpy() - ol)))
        print(f"  bitwise equal to fa_fwd_splitkv; max|dO|={eo:.3e} max|dLSE|={el:.3e}",
              flush=True)
        assert eo <= TOL_O[dtype] and el <= 1e-3


def test_noalloc_refuses_partials_beyond_the_buffer():
    """The partials of 16 parts over B1 H16 S16384 D128 need 2.16 GB, more than
    the buffer holds: FA_ERR_SCRATCH before any launch, outputs untouched."""
    import io_aware_exact_22_amd as fa

    dev = torch.device("cuda:0")
    B, S, H, D = 1, 16384, 16, 128
    q = torch.zeros((B, S, H, D), dtype=torch.bfloat16, device=dev)
    out = torch.full_like(q, 3.0)
    lse = torch.full((B, H, S), 5.0, dtype=torch.float32, device=dev)
    need = fa.fa_fwd_splitkv_workspace_size(B, H, S, D, fa.FA_DTYPE_BF16, 16)
    assert need > fa.FA_NOALLOC_SCRATCH_BYTES
    rc = fa.fa_fwd_splitkv_noalloc(q.data_ptr(), q.data_ptr(), q.data_ptr(), out.data_ptr(),
                                   lse.data_ptr(), B, H, S, D, 0.1, 1, -1, -1,
                                   fa.FA_DTYPE_BF16, 16, None)
    assert rc == fa.FA_ERR_SCRATCH
    torch.cuda.synchronize()
    assert bool((out == 3.0).all()) and bool((lse == 5.0).all())
