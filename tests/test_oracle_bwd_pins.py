"""Pins of the CPU oracle's backward pass (oracle.bwd), none of which retype
its formulas:

* finite differences: central differences of the forward oracle's loss
  L = sum(O * dO) on inputs whose perturbed values are exact in fp32;
* a library routine: torch's float64 autograd through softmax(scale QK^T +
  mask) V, an implementation independent of the oracle;
* closed forms and invariants the mathematics fixes: the key-sum of dK is 0
  (each row of dS sums to 0), the key-sum of dV is the row-sum of dO (each row
  of P sums to 1), gradients unchanged when every key is shifted by one vector,
  a single key gives dV = dO and dQ = dK = 0, and causal row 0 has dQ = 0.

The gradient is that of the forward definition ("大模型加速新突破：Flash
Attention V2核心网络算子解析" section 二.1; its step 3 names the backward pass).
"""
import math

import numpy as np
import pytest
import torch

import oracle
from fa_inputs import make_qkv

MASKS = [(False, (-1, -1)), (True, (-1, -1)), (False, (1, 1)), (False, (2, 0)), (True, (1, -1)),
         (False, (0, 3))]


def dyadic(shape, seed, lo=-2.0, hi=2.0, step=2.0 ** -8):
    """fp32 tensor of multiples of `step` in [lo, hi]: values +- 2^-12 stay exact."""
    g = torch.Generator().manual_seed(seed)
    n = int(round((hi - lo) / step))
    return (torch.randint(0, n + 1, shape, generator=g).double() * step + lo).float().contiguous()


def loss(q, k, v, do, scale, causal, window):
    out, _ = oracle.fwd(q, k, v, scale, causal, window)
    return float(np.sum(out * do.double().numpy()))


@pytest.mark.parametrize("causal,window", MASKS)
def test_bwd_finite_differences(causal, window):
    B, S, H, D = 1, 6, 2, 3
    q, k, v, do = (dyadic((B, S, H, D), seed) for seed in (1, 2, 3, 4))
    scale = 0.75
    dq, dk, dv = oracle.bwd(q, k, v, do, scale, causal, window)
    h = 2.0 ** -12
    for name, t, g in (("q", q, dq), ("k", k, dk), ("v", v, dv)):
        flat = t.view(-1)
        num = np.zeros(flat.numel())
        for idx in range(flat.numel()):
            x0 = float(flat[idx])
            flat[idx] = x0 + h
            lp = loss(q, k, v, do, scale, causal, window)
            flat[idx] = x0 - h
            lm = loss(q, k, v, do, scale, causal, window)
            flat[idx] = x0
            num[idx] = (lp - lm) / (2 * h)
        err = np.max(np.abs(num - g.reshape(-1)))
        assert err < 2e-6, f"d{name}: finite differences differ by {err}"


@pytest.mark.parametrize("causal,window", MASKS)
@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
def test_bwd_matches_torch_autograd_fp64(causal, window, dtype):
    B, S, H, D = 2, 17, 2, 8
    q, k, v = make_qkv(B, S, H, D, dtype, 31)
    do = make_qkv(B, S, H, D, dtype, 32)[0]
    scale = 1.0 / math.sqrt(D)
    dq, dk, dv = oracle.bwd(q, k, v, do, scale, causal, window)
    qt, kt, vt = (t.double().permute(0, 2, 1, 3).clone().requires_grad_(True) for t in (q, k, v))
    i = torch.arange(S)[:, None]
    j = torch.arange(S)[None, :]
    ok = torch.ones(S, S, dtype=torch.bool)
    if causal:
        ok &= j <= i
    if window[0] >= 0:
        ok &= i - j <= window[0]
    if window[1] >= 0:
        ok &= j - i <= window[1]
    s = scale * qt @ kt.transpose(-1, -2)
    s = s.masked_fill(~ok, float("-inf"))
    out = torch.softmax(s, dim=-1) @ vt
    out.backward(do.double().permute(0, 2, 1, 3))
    for name, mine, ref in (("q", dq, qt.grad), ("k", dk, kt.grad), ("v", dv, vt.grad)):
        ref = ref.permute(0, 2, 1, 3).numpy()
        assert np.max(np.abs(mine - ref)) < 1e-10, name


@pytest.mark.parametrize("causal,window", [(False, (-1, -1)), (True, (-1, -1)), (False, (30, 5))])
def test_bwd_key_sums(causal, window):
    """sum_j dK_j = 0 and sum_j dV_j = sum_i dO_i, per (b, h)."""
    q, k, v = make_qkv(1, 300, 2, 16, torch.bfloat16, 41)
    do = make_qkv(1, 300, 2, 16, torch.bfloat16, 42)[0]
    dq, dk, dv = oracle.bwd(q, k, v, do, 0.25, causal, window)
    assert np.max(np.abs(dk.sum(axis=1))) < 1e-9
    assert np.max(np.abs(dv.sum(axis=1) - do.double().numpy().sum(axis=1))) < 1e-9


def test_bwd_key_shift_invariance():
    """K -> K + 1 u^T leaves O unchanged for every Q, so every gradient too."""
    B, S, H, D = 1, 40, 2, 8
    q, k, v, do = (dyadic((B, S, H, D), seed, -1.0, 1.0) for seed in (5, 6, 7, 8))
    u = dyadic((1, 1, H, D), 9, -1.0, 1.0)
    k2 = (k + u).contiguous()
    for causal, window in [(False, (-1, -1)), (True, (-1, -1)), (False, (3, 4))]:
        a = oracle.bwd(q, k, v, do, 0.5, causal, window)
        b = oracle.bwd(q, k2, v, do, 0.5, causal, window)
        for x, y in zip(a, b):
            assert np.max(np.abs(x - y)) < 1e-10


def test_bwd_single_key():
    """S = 1: O = v_0 whatever q and k are, so dV = dO and dQ = dK = 0."""
    q, k, v = make_qkv(2, 1, 3, 8, torch.float32, 51)
    do = make_qkv(2, 1, 3, 8, torch.float32, 52)[0]
    dq, dk, dv = oracle.bwd(q, k, v, do, 0.3, False, (-1, -1))
    assert np.array_equal(dv, do.double().numpy())
    assert not dq.any() and not dk.any()


def test_bwd_causal_row0():
    """Causal row 0 sees only key 0: p_00 = 1, dS_00 = 0, so dQ_0 = 0 exactly."""
    q, k, v = make_qkv(1, 50, 2, 16, torch.bfloat16, 61)
    do = make_qkv(1, 50, 2, 16, torch.bfloat16, 62)[0]
    dq, _, _ = oracle.bwd(q, k, v, do, 0.25, True, (-1, -1))
    assert not dq[:, 0].any()


@pytest.mark.parametrize("causal,window", [(False, (-1, -1)), (True, (-1, -1)), (False, (3, 5)),
                                           (True, (6, -1))])
@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
def test_sampled_gradients_equal_the_full_backward(causal, window, dtype):
    """The sampled backward (dq of chosen rows, dk and dv of chosen keys, with
    the S x S matrices formed again entry by entry) gives the full backward's
    entries up to fp64 summation order; it is what the full-size GPU checks
    use."""
    B, S, H, D = 2, 29, 2, 16
    q, k, v = make_qkv(B, S, H, D, dtype, 71)
    do = make_qkv(B, S, H, D, dtype, 72)[0]
    dq, dk, dv = oracle.bwd(q, k, v, do, 0.3, causal, window)
    rows, keys = [0, 1, 7, 28], [0, 13, 27, 28]
    for b, h in ((0, 1), (1, 0)):
        sq, sk, sv = oracle.bwd_sampled(q, k, v, do, 0.3, causal, window, b, h, rows, keys)
        np.testing.assert_allclose(sq, dq[b, rows, h], rtol=1e-12, atol=1e-13)
        np.testing.assert_allclose(sk, dk[b, keys, h], rtol=1e-12, atol=1e-13)
        np.testing.assert_allclose(sv, dv[b, keys, h], rtol=1e-12, atol=1e-13)
    # rows only: no key statistics needed
    sq2, _, _ = oracle.bwd_sampled(q, k, v, do, 0.3, causal, window, 0, 0, [5, 6], [])
    np.testing.assert_allclose(sq2, dq[0, [5, 6], 0], rtol=1e-12, atol=1e-13)
