"""Pins for the oracle's paged K/V: gathering keys and values through a block
table ("突破大模型训练瓶颈：Flash-Attention编译优化与内存占用解决方案", section
Paged KV Cache支持) must give back exactly the contiguous tensors the pages were
cut from, however the pages are placed in the pool.  The attention on the
gathered tensors is the dense oracle, pinned in test_oracle_pins.py.
"""
import numpy as np
import pytest
import torch

import oracle
from fa_inputs import make_qkv


def paginate(x, page_size, slots, num_pages, table_stride, fill=float("nan")):
    """Cut contiguous x [B, S, H, D] into pages of page_size rows and place
    logical page p of batch b at pool slot slots[b][p]; unused pool rows hold
    ``fill``.  Returns (pool [num_pages, page_size, H, D], table [B, stride])."""
    B, S, H, D = x.shape
    n = -(-S // page_size)
    pool = torch.full((num_pages, page_size, H, D), fill, dtype=x.dtype)
    table = np.full((B, table_stride), -7, dtype=np.int32)
    for b in range(B):
        for p in range(n):
            rows = x[b, p * page_size: (p + 1) * page_size]
            pool[slots[b][p], : rows.shape[0]] = rows
            table[b, p] = slots[b][p]
    return pool.contiguous(), table


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16, torch.float16])
@pytest.mark.parametrize("S,page_size", [(16, 4), (19, 4), (7, 8), (30, 1)])
def test_gather_inverts_a_scattered_placement(dtype, S, page_size):
    """Pages scattered to a random permutation of pool slots (a table wider
    than needed, unused rows NaN) gather back to the original tensor, bit for
    bit (catches / and % swapped, a wrong in-page row, a wrong table stride)."""
    B, H, D = 3, 2, 4
    x = make_qkv(B, S, H, D, dtype, S + page_size)[0]
    n = -(-S // page_size)
    num_pages = B * n + 5
    perm = np.random.default_rng(S).permutation(num_pages)
    slots = [[int(perm[b * n + p]) for p in range(n)] for b in range(B)]
    pool, table = paginate(x, page_size, slots, num_pages, n + 3)
    got = oracle.gather_pages(pool, table, S)
    assert torch.equal(got.view(torch.uint8), x.view(torch.uint8))


def test_paged_forward_is_the_dense_forward_on_the_original_tensors():
    """Attention over paged K/V equals, bit for bit, the dense oracle on the
    tensors the pages were cut from, for every mask mode."""
    B, S, H, D, ps = 2, 37, 2, 8, 8
    q, k, v = make_qkv(B, S, H, D, torch.float32, 5)
    n = -(-S // ps)
    slots = [[(7 * (b * n + p) + 3) % (B * n + 1) for p in range(n)] for b in range(B)]
    kp, table = paginate(k, ps, slots, B * n + 1, n)
    vp, _ = paginate(v, ps, slots, B * n + 1, n)
    for causal, window in [(False, (-1, -1)), (True, (-1, -1)), (False, (5, 3)), (True, (9, -1))]:
        o1, l1 = oracle.fwd_paged(q, kp, vp, table, 0.3, causal, window)
        o2, l2 = oracle.fwd(q, k, v, 0.3, causal, window)
        assert np.array_equal(o1, o2) and np.array_equal(l1, l2)


def test_shared_prefix_pages():
    """Two sequences whose tables share their first pages see the same keys
    there: with equal queries, their causal rows over the shared prefix are
    equal, and they differ after it."""
    S, H, D, ps = 24, 1, 8, 8
    q1, k1, v1 = make_qkv(1, S, H, D, torch.float32, 6)
    _, k2, v2 = make_qkv(1, ps, H, D, torch.float32, 7)  # the second sequence's own last page
    pool_k = torch.cat([k1[0].reshape(3, ps, H, D), k2[0].reshape(1, ps, H, D)]).contiguous()
    pool_v = torch.cat([v1[0].reshape(3, ps, H, D), v2[0].reshape(1, ps, H, D)]).contiguous()
    table = np.array([[0, 1, 2], [0, 1, 3]], dtype=np.int32)
    q = torch.cat([q1, q1]).contiguous()
    o, l = oracle.fwd_paged(q, pool_k, pool_v, table, 0.5, True)
    assert np.array_equal(o[0, :16], o[1, :16]) and np.array_equal(l[0, :, :16], l[1, :, :16])
    assert not np.array_equal(o[0, 16:], o[1, 16:])


def test_bad_tables_are_refused():
    pool = torch.zeros((4, 8, 1, 4))
    with pytest.raises(ValueError):
        oracle.gather_pages(pool, np.array([[0, 4]], dtype=np.int32), 16)  # page 4 of 4
    with pytest.raises(ValueError):
        oracle.gather_pages(pool, np.array([[0, -1]], dtype=np.int32), 16)
    with pytest.raises(ValueError):
        oracle.gather_pages(pool, np.array([[0]], dtype=np.int32), 16)  # table too narrow
