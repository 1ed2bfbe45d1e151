"""Pins for the CPU oracle: checks against what the pages and the mathematics
fix, never against the oracle's own formula retyped.

Each test names what a plausible mistake in the oracle (a dropped scale, a
wrong mask index, a transposed operand, a missing normalisation, a layout
stride slip, a decoder slip) would break.  Pages are cited by title:
  V2 page      = "大模型加速新突破：Flash Attention V2核心网络算子解析"
  FA page      = "FlashAttention技术解析：加速GPT训练的核心优化"
  compile page = "突破大模型训练瓶颈：Flash-Attention编译优化与内存占用解决方案"
"""
import json
import math
import os
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle
from fa_inputs import make_qkv

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "hand_worked.json")
MASKS = [
    (False, (-1, -1)),
    (True, (-1, -1)),
    (False, (2, 3)),
    (False, (0, 0)),
    (False, (5, 0)),
    (False, (0, 4)),
    (True, (3, -1)),
    (True, (2, 7)),
    (False, (40, 40)),
]


def allowed(i, j, causal, wl, wr):
    # the mask as stated in words on the FA page (causal = no future keys;
    # window = (left, right) with -1 unbounded), inclusive bounds
    return (not causal or j <= i) and (wl < 0 or j >= i - wl) and (wr < 0 or j <= i + wr)


def key_sets(S, causal, window):
    wl, wr = window
    return [[j for j in range(S) if allowed(i, j, causal, wl, wr)] for i in range(S)]


# ---------------------------------------------------------------- decoders
def test_decoders_match_library_formats():
    """Special case that reduces to a library routine: the oracle's bit-level
    fp16/bf16 decoders agree with numpy's float16 and torch's bfloat16 on all
    65536 bit patterns (NaNs compared as NaN), and fp32 round-trips."""
    bits = torch.arange(0, 65536, dtype=torch.int32).to(torch.int16)
    h = bits.view(torch.float16)
    ref16 = np.arange(0, 65536, dtype=np.uint32).astype(np.uint16).view(np.float16).astype(np.float64)
    got16 = oracle.decode(h.contiguous())
    assert np.array_equal(np.isnan(got16), np.isnan(ref16))
    ok = ~np.isnan(ref16)
    assert np.array_equal(got16[ok], ref16[ok])
    bf = bits.view(torch.bfloat16)
    refbf = bf.to(torch.float64).numpy()
    gotbf = oracle.decode(bf.contiguous())
    assert np.array_equal(np.isnan(gotbf), np.isnan(refbf))
    ok = ~np.isnan(refbf)
    assert np.array_equal(gotbf[ok], refbf[ok])
    f = torch.randn(4096, dtype=torch.float32) * 1e3
    f[:4] = torch.tensor([0.0, -0.0, 1e-45, -3.4e38])
    assert np.array_equal(oracle.decode(f), f.double().numpy())


# ---------------------------------------------------------------- golden
def _ratio(s):
    return float(Fraction(s))


@pytest.mark.parametrize("case", json.load(open(GOLDEN))["cases"], ids=lambda c: c["name"])
def test_hand_worked_cases(case):
    """Hand-derived exact rationals (tests/golden/hand_worked.json): pins the
    scale, the sign, the operand roles (q.k, then weights on v), inclusive
    window bounds and the causal/window intersection."""
    q = torch.tensor(case["q"], dtype=torch.float32)[None, :, None, :].contiguous()
    k = torch.tensor(case["k"], dtype=torch.float32)[None, :, None, :].contiguous()
    v = torch.tensor(case["v"], dtype=torch.float32)[None, :, None, :].contiguous()
    assert case["scale"] == "ln2"
    out, lse = oracle.fwd(q, k, v, math.log(2.0), case["causal"], tuple(case["window"]))
    exp_out = np.array([[_ratio(x) for x in row] for row in case["out"]])
    exp_lse = np.array([math.log(_ratio(x)) for x in case["lse_of"]])
    np.testing.assert_allclose(out[0, :, 0, :], exp_out, rtol=0, atol=1e-14)
    np.testing.assert_allclose(lse[0, 0, :], exp_lse, rtol=0, atol=1e-14)


# ---------------------------------------------------------------- P-a
@pytest.mark.parametrize("causal,window", MASKS)
def test_rows_sum_to_one(causal, window):
    """With V = identity (D = S), O's row i is the softmax row itself: it sums
    to 1 and is zero exactly on the masked keys."""
    S = 24
    q, k, _ = make_qkv(1, S, 2, S, torch.float32, 11)
    v = torch.eye(S, dtype=torch.float32)[None, :, None, :].expand(1, S, 2, S).contiguous()
    out, _ = oracle.fwd(q, k, v, 0.3, causal, window)
    keys = key_sets(S, causal, window)
    for h in range(2):
        P = out[0, :, h, :]
        np.testing.assert_allclose(P.sum(axis=1), 1.0, rtol=0, atol=1e-12)
        for i in range(S):
            mask = np.ones(S, dtype=bool)
            mask[keys[i]] = False
            assert np.all(P[i, mask] == 0.0)
            assert np.all(P[i, ~mask] > 0.0)


# ---------------------------------------------------------------- P-b
@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16, torch.float16])
def test_causal_row0_is_v0(dtype):
    """Causal row 0 sees only key 0, so O = V[0] exactly and LSE = scale q0.k0."""
    B, S, H, D = 2, 40, 3, 16
    q, k, v = make_qkv(B, S, H, D, dtype, 21)
    scale = 0.25
    out, lse = oracle.fwd(q, k, v, scale, True, (-1, -1))
    vd, qd, kd = v.double().numpy(), q.double().numpy(), k.double().numpy()
    for b in range(B):
        for h in range(H):
            assert np.array_equal(out[b, 0, h], vd[b, 0, h])
            assert lse[b, h, 0] == pytest.approx(scale * float(qd[b, 0, h] @ kd[b, 0, h]), abs=1e-13)


# ---------------------------------------------------------------- P-c
def test_window_zero_is_identity():
    """Window (0, 0) allows only j = i: O = V exactly, LSE_i = scale q_i.k_i."""
    B, S, H, D = 1, 33, 2, 8
    q, k, v = make_qkv(B, S, H, D, torch.bfloat16, 31)
    out, lse = oracle.fwd(q, k, v, 0.5, False, (0, 0))
    assert np.array_equal(out, v.double().numpy())
    qd, kd = q.double().numpy(), k.double().numpy()
    np.testing.assert_allclose(lse, 0.5 * np.einsum("bshd,bshd->bhs", qd, kd), rtol=0, atol=1e-13)


# ---------------------------------------------------------------- P-d
@pytest.mark.parametrize("causal,window", MASKS)
@pytest.mark.parametrize("how", ["q_zero", "scale_zero"])
def test_uniform_weights_give_window_mean(causal, window, how):
    """Q = 0 or scale = 0 makes all allowed scores equal: O_i is the mean of V
    over the allowed keys (column mean, prefix mean, window mean) and
    LSE_i = ln n_i."""
    B, S, H, D = 2, 37, 2, 8
    q, k, v = make_qkv(B, S, H, D, torch.float32, 41)
    scale = 0.7
    if how == "q_zero":
        q = torch.zeros_like(q)
    else:
        scale = 0.0
    out, lse = oracle.fwd(q, k, v, scale, causal, window)
    keys = key_sets(S, causal, window)
    vd = v.double().numpy()
    for i in range(S):
        n = len(keys[i])
        np.testing.assert_allclose(out[:, i], vd[:, keys[i]].mean(axis=1), rtol=0, atol=1e-14)
        np.testing.assert_allclose(lse[:, :, i], math.log(n), rtol=0, atol=1e-14)


# ---------------------------------------------------------------- P-e
def test_two_keys_logistic():
    """S = 2, causal, row 1: the weight of key 1 is the logistic function of
    s1 - s0, so O_1 = (1 - p) v0 + p v1 and LSE_1 = s0 + ln(1 + e^(s1 - s0))."""
    q, k, v = make_qkv(1, 2, 1, 4, torch.float32, 51)
    scale = 0.9
    out, lse = oracle.fwd(q, k, v, scale, True, (-1, -1))
    qd, kd, vd = (t.double().numpy()[0, :, 0] for t in (q, k, v))
    s0, s1 = scale * qd[1] @ kd[0], scale * qd[1] @ kd[1]
    p = 1.0 / (1.0 + math.exp(-(s1 - s0)))
    np.testing.assert_allclose(out[0, 1, 0], (1 - p) * vd[0] + p * vd[1], rtol=0, atol=1e-14)
    assert lse[0, 0, 1] == pytest.approx(s0 + math.log1p(math.exp(s1 - s0)), abs=1e-14)


# ---------------------------------------------------------------- P-f / P-g
@pytest.mark.parametrize("causal,window", MASKS[:7])
def test_brute_force_long_double(causal, window):
    """Naive long-double evaluation without the max shift (the exponentials of
    moderate scores are summed directly) at S <= 16: O and LSE within 1e-12.
    Pins the LSE identity and the whole row computation."""
    S, D = 13, 5
    q, k, v = make_qkv(1, S, 1, D, torch.float32, 61)
    scale = 0.6
    out, lse = oracle.fwd(q, k, v, scale, causal, window)
    qd = q.numpy()[0, :, 0].astype(np.longdouble)
    kd = k.numpy()[0, :, 0].astype(np.longdouble)
    vd = v.numpy()[0, :, 0].astype(np.longdouble)
    for i, js in enumerate(key_sets(S, causal, window)):
        w = [np.exp(np.longdouble(scale) * np.sum(qd[i] * kd[j])) for j in js]
        Z = sum(w)
        o = sum(wj * vd[j] for wj, j in zip(w, js)) / Z
        np.testing.assert_allclose(out[0, i, 0], o.astype(np.float64), rtol=0, atol=1e-12)
        assert lse[0, 0, i] == pytest.approx(float(np.log(Z)), abs=1e-12)


# ---------------------------------------------------------------- P-h
@pytest.mark.parametrize("causal,window", MASKS)
def test_against_torch_float64(causal, window):
    """External library routine: torch float64 softmax / logsumexp on the CPU
    (B = 2, H = 3 checks the [B, S, H, D] strides)."""
    B, S, H, D = 2, 29, 3, 16
    q, k, v = make_qkv(B, S, H, D, torch.bfloat16, 71)
    scale = 1 / math.sqrt(D)
    out, lse = oracle.fwd(q, k, v, scale, causal, window)
    qd, kd, vd = (t.double().permute(0, 2, 1, 3) for t in (q, k, v))  # [B, H, S, D]
    s = scale * torch.matmul(qd, kd.transpose(-1, -2))
    wl, wr = window
    m = torch.tensor([[allowed(i, j, causal, wl, wr) for j in range(S)] for i in range(S)])
    s = s.masked_fill(~m, float("-inf"))
    ref = torch.matmul(torch.softmax(s, dim=-1), vd).permute(0, 2, 1, 3)
    np.testing.assert_allclose(out, ref.numpy(), rtol=0, atol=1e-12)
    np.testing.assert_allclose(lse, torch.logsumexp(s, dim=-1).numpy(), rtol=0, atol=1e-12)


# ---------------------------------------------------------------- P-i
def test_merge_identity_over_key_halves():
    """The log-domain merge (the V2 page, section 二.1 step 2): split the keys
    into halves A and B.  Attention over [K_A; K_A] gives O_A and LSE_A + ln 2
    (each key counted twice), likewise for B; then LSE = logaddexp(LSE_A,
    LSE_B) and O = e^(LSE_A - LSE) O_A + e^(LSE_B - LSE) O_B."""
    B, S, H, D = 1, 32, 2, 8
    q, k, v = make_qkv(B, S, H, D, torch.float32, 81)
    scale = 0.35
    out, lse = oracle.fwd(q, k, v, scale, False, (-1, -1))
    n = S // 2
    parts = []
    for sl in (slice(0, n), slice(n, S)):
        k2 = torch.cat([k[:, sl], k[:, sl]], dim=1).contiguous()
        v2 = torch.cat([v[:, sl], v[:, sl]], dim=1).contiguous()
        o_p, l_p = oracle.fwd(q, k2, v2, scale, False, (-1, -1))
        parts.append((o_p, l_p - math.log(2.0)))
    (oA, lA), (oB, lB) = parts
    l_m = np.logaddexp(lA, lB)
    np.testing.assert_allclose(lse, l_m, rtol=0, atol=1e-12)
    wA = np.exp(lA - l_m).transpose(0, 2, 1)[..., None]  # [B, S, H, 1]
    wB = np.exp(lB - l_m).transpose(0, 2, 1)[..., None]
    np.testing.assert_allclose(out, wA * oA + wB * oB, rtol=0, atol=1e-12)


def test_incremental_softmax_blockwise_lse():
    """The pages' incremental log-sum update (the V2 page, section 二.1 step 2),
    read as lse' = M + ln(sum_j exp(s_j - M) + exp(lse - M)) with
    M = max(lse, max_j s_j), run over key blocks of 5, reaches the oracle's LSE."""
    S, D = 23, 6
    q, k, v = make_qkv(1, S, 1, D, torch.float32, 82)
    scale = 0.8
    _, lse = oracle.fwd(q, k, v, scale, False, (-1, -1))
    qd, kd = q.double().numpy()[0, :, 0], k.double().numpy()[0, :, 0]
    for i in range(S):
        acc = -math.inf
        for j0 in range(0, S, 5):
            blk = [scale * float(qd[i] @ kd[j]) for j in range(j0, min(S, j0 + 5))]
            M = max(acc, max(blk))
            acc = M + math.log(sum(math.exp(x - M) for x in blk) + math.exp(acc - M))
        assert lse[0, 0, i] == pytest.approx(acc, abs=1e-12)


# ---------------------------------------------------------------- P-j
def test_joint_key_permutation_invariance():
    """Full attention: permuting the rows of K and V jointly changes nothing."""
    q, k, v = make_qkv(1, 31, 2, 8, torch.float32, 91)
    perm = torch.randperm(31, generator=torch.Generator().manual_seed(5))
    out, lse = oracle.fwd(q, k, v, 0.4, False, (-1, -1))
    out2, lse2 = oracle.fwd(q, k[:, perm].contiguous(), v[:, perm].contiguous(), 0.4, False, (-1, -1))
    np.testing.assert_allclose(out2, out, rtol=0, atol=1e-13)
    np.testing.assert_allclose(lse2, lse, rtol=0, atol=1e-13)


# ---------------------------------------------------------------- P-k
@pytest.mark.parametrize("causal,window", MASKS[:4])
def test_key_shift_invariance(causal, window):
    """K -> K + 1 u^T adds scale q_i.u to every allowed score of row i: O is
    unchanged and LSE_i moves by exactly scale q_i.u (catches a dropped or
    misplaced scale, or q and k swapped)."""
    B, S, H, D = 1, 27, 2, 4
    q, k, v = make_qkv(B, S, H, D, torch.float32, 101)
    k = (torch.round(k * 4096) / 4096).contiguous()  # on a 2^-12 grid: k + u is exact in fp32
    u = torch.tensor([0.5, -0.25, 1.0, 0.125], dtype=torch.float32)
    scale = 0.5
    out, lse = oracle.fwd(q, k, v, scale, causal, window)
    k2 = (k + u).contiguous()
    assert torch.equal(k2.double() - k.double(), u.double().expand_as(k2))
    out2, lse2 = oracle.fwd(q, k2, v, scale, causal, window)
    shift = scale * (q.double() @ u.double()).permute(0, 2, 1).numpy()  # [B, H, S]
    np.testing.assert_allclose(out2, out, rtol=0, atol=1e-12)
    np.testing.assert_allclose(lse2 - lse, shift, rtol=0, atol=1e-12)


# ---------------------------------------------------------------- P-l
def test_value_affine_map():
    """O is a convex combination of V rows: V -> aV + b gives O -> aO + b."""
    q, k, v = make_qkv(2, 19, 2, 8, torch.float32, 111)
    v = (torch.round(v * 4096) / 4096).contiguous()  # on a 2^-12 grid: a v + b is exact
    out, _ = oracle.fwd(q, k, v, 0.3, True, (4, -1))
    a, bshift = 2.0, -3.0
    v2 = (a * v + bshift).contiguous()
    assert torch.equal(v2.double(), a * v.double() + bshift)
    out2, _ = oracle.fwd(q, k, v2, 0.3, True, (4, -1))
    np.testing.assert_allclose(out2, a * out + bshift, rtol=0, atol=1e-12)


# ---------------------------------------------------------------- P-m
def test_large_scores_no_overflow():
    """scale = 50 (|s| in the hundreds, exp would overflow without the max
    shift): outputs stay finite and O_i tends to V at the argmax key; the
    stability the pages ask of the block softmax (FA page section 1)."""
    B, S, H, D = 1, 20, 1, 16
    q, k, v = make_qkv(B, S, H, D, torch.float32, 121)
    out, lse = oracle.fwd(q, k, v, 50.0, False, (-1, -1))
    assert np.all(np.isfinite(out)) and np.all(np.isfinite(lse))
    s = 50.0 * (q.double()[0, :, 0] @ k.double()[0, :, 0].T).numpy()
    top = s.argmax(axis=1)
    srt = np.sort(s, axis=1)
    for i in range(S):
        gap = srt[i, -1] - srt[i, -2]
        if gap > 40:  # the runner-up weight is below e^-40
            np.testing.assert_allclose(out[0, i, 0], v.double().numpy()[0, top[i], 0], atol=1e-12)
        assert lse[0, 0, i] >= srt[i, -1] - 1e-9


# ---------------------------------------------------------------- NaN
def test_nan_propagation():
    """NaN in q row i makes row i NaN; NaN in k row j makes every row that
    allows j NaN and no other (IEEE propagation through the scores)."""
    B, S, H, D = 1, 12, 1, 4
    q, k, v = make_qkv(B, S, H, D, torch.float32, 131)
    q2 = q.clone()
    q2[0, 5, 0, 2] = float("nan")
    out, lse = oracle.fwd(q2, k, v, 0.5, True, (-1, -1))
    assert np.all(np.isnan(out[0, 5])) and np.isnan(lse[0, 0, 5])
    others = [i for i in range(S) if i != 5]
    assert np.all(np.isfinite(out[0, others])) and np.all(np.isfinite(lse[0, 0, others]))
    k2 = k.clone()
    k2[0, 7, 0, 0] = float("nan")
    out, lse = oracle.fwd(q, k2, v, 0.5, True, (-1, -1))
    for i in range(S):
        assert np.all(np.isnan(out[0, i])) == (i >= 7)
        assert np.isnan(lse[0, 0, i]) == (i >= 7)


# ---------------------------------------------------------------- rows API
def test_rows_api_matches_full():
    """The per-row entry point (used for sampled checks at full size) returns
    the same rows as the full one."""
    q, k, v = make_qkv(2, 45, 3, 16, torch.bfloat16, 141)
    out, lse = oracle.fwd(q, k, v, 0.25, True, (10, -1))
    o_r, l_r = oracle.fwd_rows(q, k, v, 0.25, True, (10, -1), 1, 2, 7, 30)
    assert np.array_equal(o_r, out[1, 7:30, 2])
    assert np.array_equal(l_r, lse[1, 2, 7:30])


@pytest.mark.parametrize("S,causal,window", [(1, False, (-1, -1)), (17, True, (-1, -1)),
                                             (50, False, (3, 9)), (33, True, (5, 2)),
                                             (8, False, (100, 100))])
def test_allowed_pairs_closed_forms(S, causal, window):
    """The pair count S * S_eff against closed forms: S^2 (full),
    S(S+1)/2 (causal), and the per-row window widths."""
    wl, wr = window
    if not causal and window == (-1, -1):
        expect = S * S
    elif causal and window == (-1, -1):
        expect = S * (S + 1) // 2
    else:
        expect = 0
        for i in range(S):
            lo = 0 if wl < 0 else max(0, i - wl)
            hi = S - 1 if wr < 0 else min(S - 1, i + wr)
            if causal:
                hi = min(hi, i)
            expect += max(0, hi - lo + 1)
    assert oracle.allowed_pairs(S, causal, window) == expect
