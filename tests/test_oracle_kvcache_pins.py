"""Pins of the oracle's KV-cache forward (oracle.fwd_kvcache, decoding against a
cache: "FlashAttention技术解析：加速GPT训练的核心优化" section 5 names FlashDecoding;
"突破大模型训练瓶颈：Flash-Attention编译优化与内存占用解决方案" section 总结与最佳实践
names flash_attn_with_kvcache).  Reading: sequence b's keys are the first L_b
rows of its cache, and its S_q queries are the sequence's last S_q positions,
query i at L_b - S_q + i.  Each pin reduces a case to the dense oracle (pinned
in test_oracle_pins.py) by a route that does not use the position formula:
the queries are placed into a full-length sequence of their own and the dense
oracle's rows are read back."""
import math

import numpy as np
import pytest
import torch

import oracle
from fa_inputs import make_qkv

MASKS = [(False, (-1, -1)), (True, (-1, -1)), (False, (7, 3)), (True, (12, -1)),
         (False, (0, 0)), (True, (5, 5))]


def cache_case(B, S_q, S_k, H, D, dtype, seed):
    q, _, _ = make_qkv(B, S_q, H, D, dtype, seed)
    _, k, v = make_qkv(B, S_k, H, D, dtype, seed + 1)
    return q, k, v


def dense_rows_of(q_b, k_b, v_b, L, scale, causal, window):
    """The rows [L - S_q, L) of the dense oracle on a length-L sequence whose
    last S_q queries are q_b (the earlier queries are arbitrary: rows are
    independent) and whose keys / values are the first L rows of k_b, v_b."""
    S_q, H, D = q_b.shape
    qf = torch.randn((1, L, H, D), generator=torch.Generator().manual_seed(L)).to(q_b.dtype)
    qf[0, L - S_q:] = q_b
    kf = k_b[:L].unsqueeze(0).contiguous()
    vf = v_b[:L].unsqueeze(0).contiguous()
    outs, lses = [], []
    for h in range(H):
        o, l = oracle.fwd_rows(qf.contiguous(), kf, vf, scale, causal, window, 0, h, L - S_q, L)
        outs.append(o)
        lses.append(l)
    return np.stack(outs, axis=1), np.stack(lses, axis=0)  # [S_q, H, D], [H, S_q]


@pytest.mark.parametrize("causal,window", MASKS)
def test_full_cache_is_the_dense_forward(causal, window):
    """S_q = L_b = S_k: every query sits at its own index; the dense oracle."""
    B, S, H, D = 2, 37, 2, 16
    q, k, v = make_qkv(B, S, H, D, torch.float32, 3)
    o, l = oracle.fwd_kvcache(q, k, v, [S, S], 0.3, causal, window)
    ro, rl = oracle.fwd(q, k, v, 0.3, causal, window)
    assert np.allclose(o, ro, atol=1e-13, rtol=0) and np.allclose(l, rl, atol=1e-13, rtol=0)


@pytest.mark.parametrize("causal,window", MASKS)
@pytest.mark.parametrize("S_q", [1, 4])
def test_queries_are_the_last_positions(causal, window, S_q):
    """Decoding (S_q = 1) and a short query block against caches of different
    lengths per sequence: rows equal the dense oracle's last S_q rows of each
    sequence.  A top-left alignment (query i at position i) fails this."""
    B, S_k, H, D = 3, 40, 2, 16
    lens = [S_q + 9, 40, S_q + 23]
    q, k, v = cache_case(B, S_q, S_k, H, D, torch.bfloat16, 11)
    scale = 1.0 / math.sqrt(D)
    o, l = oracle.fwd_kvcache(q, k, v, lens, scale, causal, window)
    for b, L in enumerate(lens):
        ro, rl = dense_rows_of(q[b], k[b], v[b], L, scale, causal, window)
        assert np.allclose(o[b], ro, atol=1e-12, rtol=0), (b, L)
        assert np.allclose(l[b], rl, atol=1e-12, rtol=0), (b, L)


def test_rows_past_the_length_are_never_read():
    B, S_q, S_k, H, D = 2, 3, 50, 2, 16
    q, k, v = cache_case(B, S_q, S_k, H, D, torch.float16, 21)
    lens = [10, 33]
    o1, l1 = oracle.fwd_kvcache(q, k, v, lens, 0.25, True, (-1, -1))
    k2, v2 = k.clone(), v.clone()
    for b, L in enumerate(lens):
        k2[b, L:] = float("nan")
        v2[b, L:] = float("inf")
    o2, l2 = oracle.fwd_kvcache(q, k2, v2, lens, 0.25, True, (-1, -1))
    assert np.isfinite(o2).all() and np.array_equal(o1, o2) and np.array_equal(l1, l2)


def test_sequences_are_independent():
    B, S_q, S_k, H, D = 3, 2, 30, 2, 16
    q, k, v = cache_case(B, S_q, S_k, H, D, torch.bfloat16, 31)
    lens = [5, 30, 17]
    o, l = oracle.fwd_kvcache(q, k, v, lens, 0.2, False, (4, 1))
    for b, L in enumerate(lens):
        ob, lb = oracle.fwd_kvcache(q[b:b + 1].contiguous(), k[b:b + 1].contiguous(),
                                    v[b:b + 1].contiguous(), [L], 0.2, False, (4, 1))
        assert np.array_equal(o[b], ob[0]) and np.array_equal(l[b], lb[0])


def test_rows_without_keys():
    """A cache shorter than the query block leaves its first queries at
    negative positions: under the causal mask they allow no key (O = 0,
    LSE = -inf); an empty cache gives that for every row; without the causal
    mask a negative position still sees the whole cache."""
    B, S_q, S_k, H, D = 2, 6, 8, 1, 16
    q, k, v = cache_case(B, S_q, S_k, H, D, torch.float32, 41)
    o, l = oracle.fwd_kvcache(q, k, v, [4, 0], 0.5, True, (-1, -1))
    assert np.all(o[0, :2] == 0) and np.all(np.isneginf(l[0, :, :2]))
    assert np.all(np.isfinite(l[0, :, 2:]))
    assert np.all(o[1] == 0) and np.all(np.isneginf(l[1]))
    o, l = oracle.fwd_kvcache(q, k, v, [4, 0], 0.5, False, (-1, -1))
    ref = oracle.fwd_kvcache(q[:1, :1].contiguous(), k[:1], v[:1], [4], 0.5, False, (-1, -1))[0]
    assert np.allclose(o[0, 0], ref[0, 0], atol=1e-13, rtol=0)
    # row 0 (position -2) allows all four keys: the closed-form softmax over them
    qq = q[0, 0, 0].double()
    kk = k[0, :4, 0].double()
    s = 0.5 * (kk @ qq)
    p = torch.softmax(s, 0)
    assert np.allclose(o[0, 0, 0], (p @ v[0, :4, 0].double()).numpy(), atol=1e-12, rtol=0)
    assert abs(l[0, 0, 0] - float(torch.logsumexp(s, 0))) < 1e-12


def test_merge_of_cache_halves():
    """Without the causal mask or a window, positions do not matter: the keys
    [0, t) and [t, L) form two caches, and the log-domain merge of their
    results ([V2] section 二.1 step 2) is the whole cache's result."""
    B, S_q, S_k, H, D = 1, 3, 48, 2, 16
    q, k, v = cache_case(B, S_q, S_k, H, D, torch.float32, 51)
    L, t = 45, 19
    o, l = oracle.fwd_kvcache(q, k, v, [L], 0.3)
    oa, la = oracle.fwd_kvcache(q, k, v, [t], 0.3)
    kb, vb = k[:, t:].contiguous(), v[:, t:].contiguous()
    ob, lb = oracle.fwd_kvcache(q, kb, vb, [L - t], 0.3)
    lm = np.logaddexp(la, lb)
    wa = np.exp(la - lm).transpose(0, 2, 1)[..., None]
    wb = np.exp(lb - lm).transpose(0, 2, 1)[..., None]
    assert np.allclose(lm, l, atol=1e-12, rtol=0)
    assert np.allclose(wa * oa + wb * ob, o, atol=1e-12, rtol=0)


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
def test_paged_cache_is_the_gathered_cache(dtype):
    """Pools with pages at a random permutation of slots, NaN in every row no
    sequence uses: the paged call equals the contiguous cache's."""
    B, S_q, S_k, H, D, ps = 2, 2, 48, 2, 16, 8
    q, k, v = cache_case(B, S_q, S_k, H, D, dtype, 61)
    lens = [21, 48]
    n_pg = S_k // ps
    perm = torch.randperm(B * n_pg + 3, generator=torch.Generator().manual_seed(7))[:B * n_pg]
    table = perm.view(B, n_pg).to(torch.int32)
    pools = []
    for t in (k, v):
        pool = torch.full((B * n_pg + 3, ps, H, D), float("nan"), dtype=dtype)
        for b in range(B):
            for j in range(lens[b]):
                pool[table[b, j // ps], j % ps] = t[b, j]
        pools.append(pool)
    o, l = oracle.fwd_kvcache_paged(q, pools[0], pools[1], table.numpy(), lens, S_k, 0.25, True)
    ro, rl = oracle.fwd_kvcache(q, k, v, lens, 0.25, True)
    assert np.isfinite(o).all() and np.array_equal(o, ro) and np.array_equal(l, rl)
