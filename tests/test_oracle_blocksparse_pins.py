"""Pins for the oracle's block-sparse forward: checks against the dense
forward (pinned in test_oracle_pins.py) through reductions that do not run
the oracle's block-mask factor, never against that factor retyped.

The reading pinned here: key j is allowed for query i when the dense forward
allows it and the mask byte of (query block i // block_m, key block
j // block_n) is nonzero ("FlashAttention技术解析：加速GPT训练的核心优化",
section 5, names block-sparse attention as a variant of the method).  Each
test names the mistakes it catches (mask ignored, blocks transposed, a wrong
block divisor or row stride, a wrong mask head).
"""
import numpy as np
import pytest
import torch

import oracle
from fa_inputs import make_qkv, random_block_mask


def nblocks(S, b):
    return -(-S // b)


def expand(mask2d, S, bm, bn):
    """Element mask [S, S] by repeating each block byte over its rows and
    columns (structural expansion, no index division)."""
    return np.repeat(np.repeat(np.asarray(mask2d, dtype=bool), bm, axis=0), bn, axis=1)[:S, :S]


def dense_over_keys(q, k, v, scale, b, h, i, keys):
    """Dense-oracle attention of query (b, i, h) over exactly the key set
    ``keys``: the keys are gathered in order into a new sequence and the
    query is put at its last row under a causal mask, so that row attends to
    all of them and to nothing else."""
    n = len(keys)
    D = q.shape[-1]
    q2 = torch.zeros((1, n, 1, D), dtype=q.dtype)
    k2 = torch.zeros((1, n, 1, D), dtype=q.dtype)
    v2 = torch.zeros((1, n, 1, D), dtype=q.dtype)
    q2[0, n - 1, 0] = q[b, i, h]
    k2[0, :, 0] = k[b, keys, h]
    v2[0, :, 0] = v[b, keys, h]
    o, l = oracle.fwd_rows(q2.contiguous(), k2.contiguous(), v2.contiguous(), scale, True,
                           (-1, -1), 0, 0, n - 1, n)
    return o[0], l[0]


@pytest.mark.parametrize("causal,window", [(False, (-1, -1)), (True, (-1, -1)), (False, (3, 2)),
                                           (True, (4, -1))])
@pytest.mark.parametrize("bm,bn", [(4, 4), (3, 5), (64, 64), (1, 1)])
def test_all_ones_mask_is_the_dense_forward(causal, window, bm, bn):
    """A mask with every block on reduces to the dense forward, bit for bit
    (catches a factor that drops allowed keys, e.g. an off-by-one block or a
    mask read past its row)."""
    B, S, H, D = 2, 23, 2, 8
    q, k, v = make_qkv(B, S, H, D, torch.float32, 11)
    mask = np.ones((1, nblocks(S, bm), nblocks(S, bn)), dtype=np.uint8)
    o_bs, l_bs = oracle.fwd_blocksparse(q, k, v, 0.4, mask, bm, bn, causal, window)
    o_d, l_d = oracle.fwd(q, k, v, 0.4, causal, window)
    assert np.array_equal(o_bs, o_d)
    assert np.array_equal(l_bs, l_d)


@pytest.mark.parametrize("bm,bn", [(4, 3), (3, 5), (5, 5), (8, 2)])
@pytest.mark.parametrize("causal", [False, True])
def test_rows_match_dense_attention_over_their_key_set(bm, bn, causal):
    """Every query row equals the dense oracle run over exactly the keys its
    expanded block mask (and the causal mask) keeps, gathered into a sequence
    of their own (catches an ignored mask, transposed blocks, a block divisor
    or row stride slip -- bm != bn and a ragged last block make each of these
    change some row's key set)."""
    B, S, H, D = 1, 19, 2, 8
    q, k, v = make_qkv(B, S, H, D, torch.float32, 12)
    mask = random_block_mask(1, nblocks(S, bm), nblocks(S, bn), 0.5, 13)
    el = expand(mask[0], S, bm, bn)
    if causal:
        el &= np.tril(np.ones((S, S), dtype=bool))
    o_bs, l_bs = oracle.fwd_blocksparse(q, k, v, 0.3, mask, bm, bn, causal)
    for h in range(H):
        for i in range(S):
            keys = list(np.nonzero(el[i])[0])
            if not keys:
                assert np.all(o_bs[0, i, h] == 0.0) and l_bs[0, h, i] == -np.inf
                continue
            o_ref, l_ref = dense_over_keys(q, k, v, 0.3, 0, h, i, keys)
            np.testing.assert_allclose(o_bs[0, i, h], o_ref, rtol=0, atol=1e-13)
            assert abs(l_bs[0, h, i] - l_ref) <= 1e-13


@pytest.mark.parametrize("L,S", [(4, 16), (5, 23), (8, 8)])
@pytest.mark.parametrize("causal", [False, True])
def test_block_diagonal_mask_is_independent_segments(L, S, causal):
    """A block-diagonal mask with block_m = block_n = L cuts the sequence into
    segments of L (the last one ragged) that attend only within themselves:
    each equals the dense oracle on that segment as a sequence of its own
    (catches an off-by-one at block boundaries)."""
    B, H, D = 2, 2, 8
    q, k, v = make_qkv(B, S, H, D, torch.float32, 14)
    n = nblocks(S, L)
    mask = np.eye(n, dtype=np.uint8)[None]
    o_bs, l_bs = oracle.fwd_blocksparse(q, k, v, 0.5, mask, L, L, causal)
    for s0 in range(0, S, L):
        s1 = min(S, s0 + L)
        seg = lambda t: t[:, s0:s1].contiguous()
        o_seg, l_seg = oracle.fwd(seg(q), seg(k), seg(v), 0.5, causal)
        np.testing.assert_allclose(o_bs[:, s0:s1], o_seg, rtol=0, atol=1e-13)
        np.testing.assert_allclose(l_bs[:, :, s0:s1], l_seg, rtol=0, atol=1e-13)


def test_lower_block_triangle_with_causal_is_causal():
    """With block_m = block_n, the lower block triangle (query block >= key
    block) holds every causal pair, so with causal = 1 the result is the dense
    causal forward, bit for bit; the strict upper triangle alone leaves no key
    for any row (O = 0, LSE = -inf)."""
    B, S, H, D, L = 1, 20, 2, 8, 4
    q, k, v = make_qkv(B, S, H, D, torch.float32, 15)
    n = nblocks(S, L)
    lower = np.tril(np.ones((n, n), dtype=np.uint8))[None]
    o_bs, l_bs = oracle.fwd_blocksparse(q, k, v, 0.6, lower, L, L, True)
    o_d, l_d = oracle.fwd(q, k, v, 0.6, True)
    assert np.array_equal(o_bs, o_d) and np.array_equal(l_bs, l_d)
    upper = np.triu(np.ones((n, n), dtype=np.uint8), 1)[None]
    o_u, l_u = oracle.fwd_blocksparse(q, k, v, 0.6, upper, L, L, True)
    assert np.all(o_u == 0.0) and np.all(l_u == -np.inf)


def test_empty_rows_and_single_block_rows():
    """A query block with no block on gets O = 0 and LSE = -inf; a query block
    with one key block on is the softmax over that block's keys only, whose LSE
    is ln of the plain sum of exp(scale * q.k) over them (a closed form)."""
    B, S, H, D, bm, bn = 1, 12, 1, 4, 4, 3
    q, k, v = make_qkv(B, S, H, D, torch.float32, 16)
    mask = np.zeros((1, 3, 4), dtype=np.uint8)
    mask[0, 1, 2] = 1  # rows 4..7 see keys 6..8 only
    o, l = oracle.fwd_blocksparse(q, k, v, 0.7, mask, bm, bn)
    for i in list(range(0, 4)) + list(range(8, 12)):
        assert np.all(o[0, i, 0] == 0.0) and l[0, 0, i] == -np.inf
    qd, kd, vd = (t.double().numpy()[0, :, 0] for t in (q, k, v))
    for i in range(4, 8):
        s = 0.7 * kd[6:9] @ qd[i]
        w = np.exp(s)
        np.testing.assert_allclose(o[0, i, 0], (w / w.sum()) @ vd[6:9], rtol=0, atol=1e-14)
        assert abs(l[0, 0, i] - np.log(w.sum())) <= 1e-14


@pytest.mark.parametrize("n_mask", ["H", "BH"])
def test_mask_heads_select_their_own_matrix(n_mask):
    """With one mask per head (n_mask = H) or per (batch, head) (n_mask = B*H),
    head (b, h) equals a shared-mask call with that head's matrix (catches a
    mask head index of b * H + h read as h * B + b, or per-head masks read as
    one)."""
    B, S, H, D, bm, bn = 2, 16, 3, 8, 4, 4
    q, k, v = make_qkv(B, S, H, D, torch.float32, 17)
    nm = H if n_mask == "H" else B * H
    masks = random_block_mask(nm, 4, 4, 0.5, 18)
    o, l = oracle.fwd_blocksparse(q, k, v, 0.4, masks, bm, bn)
    for b in range(B):
        for h in range(H):
            hm = h if n_mask == "H" else b * H + h
            o1, l1 = oracle.fwd_blocksparse(q, k, v, 0.4, masks[hm:hm + 1], bm, bn)
            assert np.array_equal(o[b, :, h], o1[b, :, h])
            assert np.array_equal(l[b, h], l1[b, h])


def test_rows_entry_matches_full_entry():
    """The sampled-rows entry gives the full entry's rows (what the GPU tests
    use at full size)."""
    B, S, H, D, bm, bn = 2, 30, 2, 8, 6, 4
    q, k, v = make_qkv(B, S, H, D, torch.bfloat16, 19)
    mask = random_block_mask(B * H, 5, 8, 0.4, 20)
    o, l = oracle.fwd_blocksparse(q, k, v, 0.35, mask, bm, bn, True, (9, -1))
    o_r, l_r = oracle.fwd_rows_blocksparse(q, k, v, 0.35, mask, bm, bn, True, (9, -1), 1, 1, 7, 25)
    assert np.array_equal(o_r, o[1, 7:25, 1])
    assert np.array_equal(l_r, l[1, 1, 7:25])


def test_bad_masks_are_refused():
    B, S, H, D = 1, 8, 2, 4
    q, k, v = make_qkv(B, S, H, D, torch.float32, 21)
    with pytest.raises(ValueError):
        oracle.fwd_blocksparse(q, k, v, 1.0, np.ones((1, 3, 2), np.uint8), 4, 4)
    with pytest.raises(ValueError):
        oracle.fwd_blocksparse(q, k, v, 1.0, np.ones((3, 2, 2), np.uint8), 4, 4)


def test_keys_of_blocks_that_are_off_never_reach_the_output():
    """O sums over allowed keys only: NaN and inf placed in the keys and values
    of blocks that are off leave every row as it is with those entries zeroed
    (catches a factor applied to the scores but not to the P V sum, where an
    off key's weight 0 times inf would give NaN)."""
    B, S, H, D, bm, bn = 1, 16, 2, 8, 4, 4
    q, k, v = make_qkv(B, S, H, D, torch.float32, 22)
    mask = np.ones((1, 4, 4), dtype=np.uint8)
    mask[0, :, 2] = 0  # keys 8..11 are off for every row
    k_bad, v_bad = k.clone(), v.clone()
    k_bad[:, 8:12] = float("nan")
    v_bad[:, 8:12] = float("inf")
    k0, v0 = k.clone(), v.clone()
    k0[:, 8:12] = 0.0
    v0[:, 8:12] = 0.0
    o_bad, l_bad = oracle.fwd_blocksparse(q, k_bad, v_bad, 0.5, mask, bm, bn)
    o_ok, l_ok = oracle.fwd_blocksparse(q, k0, v0, 0.5, mask, bm, bn)
    assert np.all(np.isfinite(o_bad)) and np.all(np.isfinite(l_bad))
    assert np.array_equal(o_bad, o_ok) and np.array_equal(l_bad, l_ok)
