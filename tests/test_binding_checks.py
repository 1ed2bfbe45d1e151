"""The Python binding refuses, before any launch, tensors whose pointers the
kernels could not use: on another device than q (a host tensor, or another
GPU), of the wrong dtype or shape, or not contiguous."""
import pytest
import torch

import io_aware_exact_22_amd as fa
from io_aware_exact_22_amd import fa as fa_mod


def test_check_like_rejects_other_device_dtype_shape():
    q = torch.zeros(1, 8, 2, 64)
    fa_mod._check_like("k", torch.zeros(1, 8, 2, 64), q)
    with pytest.raises(ValueError, match="device"):
        fa_mod._check_like("k", torch.zeros(1, 8, 2, 64, device="meta"), q)
    with pytest.raises(ValueError, match="float16"):
        fa_mod._check_like("k", torch.zeros(1, 8, 2, 64, dtype=torch.float16), q)
    with pytest.raises(ValueError):
        fa_mod._check_like("k", torch.zeros(1, 9, 2, 64), q)
    with pytest.raises(ValueError, match="contiguous"):
        fa_mod._check_like("k", torch.zeros(1, 2, 8, 64).transpose(1, 2), q)
    with pytest.raises(ValueError, match="device"):
        fa_mod._workspace(torch.zeros(4, device="meta"), 16, q, torch.float32)


@pytest.mark.gpu
def test_host_tensors_are_refused_before_launch():
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")
    dev = torch.device("cuda:0")
    B, S, H, D = 1, 256, 2, 64
    q, k, v = (torch.randn(B, S, H, D, dtype=torch.bfloat16, device=dev) for _ in range(3))
    cpu_out = torch.empty(B, S, H, D, dtype=torch.bfloat16)
    cpu_lse = torch.empty(B, H, S, dtype=torch.float32)
    with pytest.raises(ValueError, match="device"):
        fa.flash_attn_fwd(q, k.cpu(), v)
    with pytest.raises(ValueError, match="device"):
        fa.flash_attn_fwd(q, k, v, out=cpu_out)
    with pytest.raises(ValueError, match="device"):
        fa.flash_attn_fwd(q, k, v, lse=cpu_lse)
    with pytest.raises(ValueError, match="device"):
        fa.flash_attn_fwd_splitkv(q, k, v, n_splits=2, workspace=torch.empty(1 << 20))
    with pytest.raises(ValueError, match="device"):
        fa.flash_attn_fwd_splitkv(q, k, v, n_splits=2, lse=cpu_lse)
    mask = torch.ones(1, 2, 4, dtype=torch.uint8, device=dev)
    with pytest.raises(ValueError, match="device"):
        fa.flash_attn_fwd_blocksparse(q, k, v, mask.cpu(), 128, 64)
    with pytest.raises(ValueError, match="device"):
        fa.flash_attn_fwd_blocksparse(q, k, v, mask, 128, 64, workspace=torch.empty(64,
                                                                                   dtype=torch.int32))
    pool = torch.zeros(4, 64, H, D, dtype=torch.bfloat16, device=dev)
    table = torch.arange(4, dtype=torch.int32, device=dev).view(1, 4)
    with pytest.raises(ValueError, match="device"):
        fa.flash_attn_fwd_paged(q, pool.cpu(), pool, table)
    with pytest.raises(ValueError, match="device"):
        fa.flash_attn_fwd_paged(q, pool, pool, table.cpu())
    out, lse = fa.flash_attn_fwd(q, k, v)
    with pytest.raises(ValueError, match="device"):
        fa.flash_attn_bwd(q.cpu(), q, k, v, out, lse)
    with pytest.raises(ValueError, match="device"):
        fa.flash_attn_bwd(q, q, k, v, out, lse.cpu())
    with pytest.raises(ValueError, match="device"):
        fa.flash_attn_bwd(q, q, k, v, out, lse, dq=torch.empty_like(q, device="cpu"))
    with pytest.raises(ValueError, match="device"):
        fa.flash_attn_bwd(q, q, k, v, out, lse, workspace=torch.empty(B * H * S))
    torch.cuda.synchronize()
