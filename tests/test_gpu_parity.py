"""GPU parity: libfa_mi355x's fa_fwd (through the C ABI) against the CPU
oracle on the same seeded, rounded inputs.

Tolerances (max-abs, on every compared element): O <= 1e-4 for fp32,
<= 4e-3 for fp16, <= 2e-2 for bf16; LSE <= 1e-3.  Any NaN or Inf where the
oracle is finite fails.  Sizes here span several Q and K/V tiles plus a ragged
tail, so the oracle checks every element; the named workloads at full size
are checked on every element too, the oracle running head by head.
"""
import math

import numpy as np
import pytest
import torch

import oracle
from fa_inputs import WORKLOADS, make_qkv, workload_qkv

pytestmark = pytest.mark.gpu

TOL_O = {torch.float32: 1e-4, torch.float16: 4e-3, torch.bfloat16: 2e-2}
TOL_LSE = 1e-3


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")
    import io_aware_exact_22_amd  # noqa: F401  (fails loudly if the library is missing)


def gpu_fwd(q, k, v, scale, causal, window):
    import io_aware_exact_22_amd as fa

    qd, kd, vd = (t.cuda() for t in (q, k, v))
    out, lse = fa.flash_attn_fwd(qd, kd, vd, softmax_scale=scale, causal=causal, window_size=window)
    torch.cuda.synchronize()
    return out.cpu(), lse.cpu()


def assert_close(out, lse, ref_out, ref_lse, dtype, what=""):
    o = out.double().numpy()
    ls = lse.double().numpy()
    assert np.all(np.isfinite(ref_out)) and np.all(np.isfinite(ref_lse))
    assert np.all(np.isfinite(o)), f"{what}: non-finite O"
    assert np.all(np.isfinite(ls)), f"{what}: non-finite LSE"
    eo = float(np.max(np.abs(o - ref_out))) if o.size else 0.0
    el = float(np.max(np.abs(ls - ref_lse))) if ls.size else 0.0
    print(f"{what}: max|dO|={eo:.3e} max|dLSE|={el:.3e}", flush=True)
    assert eo <= TOL_O[dtype], f"{what}: O error {eo} > {TOL_O[dtype]}"
    assert el <= TOL_LSE, f"{what}: LSE error {el} > {TOL_LSE}"


def check_full(B, S, H, D, dtype, causal, window, seed, scale=None):
    scale = 1.0 / math.sqrt(D) if scale is None else scale
    q, k, v = make_qkv(B, S, H, D, dtype, seed)
    what = f"B{B} S{S} H{H} D{D} {dtype} causal={causal} window={window} seed={seed}"
    print("run", what, flush=True)
    out, lse = gpu_fwd(q, k, v, scale, causal, window)
    ref_out, ref_lse = oracle.fwd(q, k, v, scale, causal, window)
    assert_close(out, lse, ref_out, ref_lse, dtype, what)


# ---------------------------------------------------------------- small, every element
MASKS = [(False, (-1, -1)), (True, (-1, -1)), (False, (128, 128)), (False, (0, 64)),
         (False, (300, 0)), (True, (100, -1)), (False, (33, 7))]


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float16, torch.float32])
@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("causal,window", MASKS)
def test_parity_ragged(dtype, D, causal, window):
    check_full(2, 389, 3, D, dtype, causal, window, seed=7)


@pytest.mark.parametrize("S", [1, 7, 63, 64, 65, 127, 128, 129, 1000, 4097])
@pytest.mark.parametrize("causal", [False, True])
def test_parity_lengths(S, causal):
    dtype = torch.bfloat16 if causal else torch.float16
    H = 2 if S < 4000 else 1
    check_full(1, S, H, 128 if causal else 64, dtype, causal, (-1, -1), seed=S)


@pytest.mark.parametrize("S", [4096, 4100, 4415])
@pytest.mark.parametrize("dtype,D", [(torch.bfloat16, 128), (torch.float16, 128),
                                     (torch.bfloat16, 64), (torch.float16, 64)])
@pytest.mark.parametrize("causal", [False, True])
def test_parity_long_sequences(S, dtype, D, causal):
    """Sequences of 4096 and more, every element against the oracle, including
    ragged last Q and K/V tiles."""
    check_full(1, S, 2, D, dtype, causal, (-1, -1), seed=S + D)


@pytest.mark.parametrize("window", [(0, 0), (0, 64), (64, 0), (300, 0), (5, 2000), (4096, 4096),
                                    (1, 1), (127, 129)])
@pytest.mark.parametrize("causal", [False, True])
def test_parity_windows(window, causal):
    check_full(1, 700, 2, 128, torch.bfloat16, causal, window, seed=17)


@pytest.mark.parametrize("B,H,S", [(2, 10, 1000), (1, 20, 1024)])
def test_parity_launch_order_blocks(B, H, S):
    """Causal, with B * H not a multiple of 8: the XCD blocks of the launch
    order start and end inside heads and hold whole heads between; every
    element against the oracle."""
    check_full(B, S, H, 128, torch.bfloat16, True, (-1, -1), seed=1000 * B + H)


def test_parity_launch_order_many_workgroups():
    """5 heads of 16384 causal rows: 640 workgroups, more than the device holds
    at once, with XCD blocks that split heads; every element of every head."""
    from types import SimpleNamespace

    w = SimpleNamespace(name="causal_16k_h5", B=1, H=5, S=16384, D=128, dtype=torch.bfloat16,
                        causal=True, window=(-1, -1), scale=1.0 / math.sqrt(128))
    q, k, v = make_qkv(w.B, w.S, w.H, w.D, w.dtype, 55)
    print("run causal 16384 x 5 heads", flush=True)
    out, lse = gpu_fwd(q, k, v, w.scale, w.causal, w.window)
    check_every_row(w, q, k, v, out, lse)


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float16])
@pytest.mark.parametrize("H,D,window", [(32, 64, (-1, -1)), (20, 128, (1024, -1)),
                                        (10, 256, (-1, -1)), (3, 96, (-1, -1))])
def test_parity_dynamic_tail(dtype, H, D, window):
    """Causal launches with more workgroups than the device holds at once run
    their lightest tiles in the dynamic order (workgroups take list positions
    from a counter in the LSE word of row 0 of head 0, zeroed before the
    launch): every element against the oracle, on two calls in a row into
    the same buffers, whose LSE starts as NaN."""
    import io_aware_exact_22_amd as fa

    B = 1
    S = 4096 if H > 3 else 30000
    dcode = fa.FA_DTYPE_BF16 if dtype == torch.bfloat16 else fa.FA_DTYPE_FP16
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    first = fa.fa_fwd_launch_order(B, H, S, D, dcode, 1, window[0], window[1], cus, 0)[2]
    assert first >= 0, "the case must take the dynamic order"
    scale = 1.0 / math.sqrt(D)
    q, k, v = make_qkv(B, S, H, D, dtype, 77 + H)
    what = f"dynamic tail: B{B} S{S} H{H} D{D} {dtype} window={window} first={first}"
    print("run", what, flush=True)
    qd, kd, vd = (x.cuda() for x in (q, k, v))
    out = torch.empty_like(qd)
    lse = torch.full((B, H, S), float("nan"), dtype=torch.float32, device="cuda")
    res = []
    for _ in range(2):
        fa.flash_attn_fwd(qd, kd, vd, softmax_scale=scale, causal=True, window_size=window,
                          out=out, lse=lse)
        torch.cuda.synchronize()
        res.append((out.cpu(), lse.cpu()))
    assert torch.equal(res[0][0], res[1][0]) and torch.equal(res[0][1], res[1][1])
    if S > 4096:  # the 30000-row case: every row through the row-chunked oracle
        from types import SimpleNamespace
        w = SimpleNamespace(name="dyn", B=B, H=H, S=S, D=D, dtype=dtype, causal=True,
                            window=window, scale=scale)
        check_every_row(w, q, k, v, res[0][0], res[0][1], chunk_rows=4096)
        return
    ref_out, ref_lse = oracle.fwd(q, k, v, scale, True, window)
    assert_close(res[0][0], res[0][1], ref_out, ref_lse, dtype, what)


@pytest.mark.parametrize("name", ["tiny_fp32", "gpt_causal_2k", "full_4k_d64"])
@pytest.mark.parametrize("seed", [None, 101, 102])
def test_parity_named_small_workloads(name, seed):
    """The tiny fp32, 2K causal and 4K full workloads at full size, every
    element, three seeds each."""
    w = WORKLOADS[name]
    if name == "full_4k_d64":  # 64 heads: the oracle runs head by head
        q, k, v = workload_qkv(w, seed)
        print("run", w.describe(), "seed", seed, flush=True)
        out, lse = gpu_fwd(q, k, v, w.scale, w.causal, w.window)
        check_every_row(w, q, k, v, out, lse)
        return
    check_full(w.B, w.S, w.H, w.D, w.dtype, w.causal, w.window, w.seed if seed is None else seed)


def check_every_row(w, q, k, v, out, lse, chunk_rows=None):
    """Every element of out and lse against the oracle, head by head in chunks
    of query rows (the oracle materialises a chunk x S score matrix), with the
    largest errors over the whole tensor printed and checked."""
    chunk_rows = w.S if chunk_rows is None else chunk_rows
    assert torch.isfinite(out.float()).all() and torch.isfinite(lse).all()
    eo = el = 0.0
    for b in range(w.B):
        for h in range(w.H):
            for r0 in range(0, w.S, chunk_rows):
                r1 = min(w.S, r0 + chunk_rows)
                ro, rl = oracle.fwd_rows(q, k, v, w.scale, w.causal, w.window, b, h, r0, r1)
                assert np.all(np.isfinite(ro)) and np.all(np.isfinite(rl))
                eo = max(eo, float(np.max(np.abs(out[b, r0:r1, h, :].double().numpy() - ro))))
                el = max(el, float(np.max(np.abs(lse[b, h, r0:r1].double().numpy() - rl))))
    print(f"{w.name} every element: max|dO|={eo:.3e} max|dLSE|={el:.3e}", flush=True)
    assert eo <= TOL_O[w.dtype], f"{w.name}: O error {eo} > {TOL_O[w.dtype]}"
    assert el <= TOL_LSE, f"{w.name}: LSE error {el} > {TOL_LSE}"


@pytest.mark.parametrize("name", ["window_8k", "causal_16k", "causal_32k"])
def test_parity_named_full_size_every_element(name):
    """The full-size named workloads in the launch configuration the benchmark
    times (one fa_fwd over the whole workload): every element of O and LSE
    against the oracle.  The 32K run goes through the oracle in chunks of 8192
    rows (a 32768 x 32768 fp64 matrix per head would be 8 GiB)."""
    w = WORKLOADS[name]
    q, k, v = workload_qkv(w)
    print("run", w.describe(), flush=True)
    out, lse = gpu_fwd(q, k, v, w.scale, w.causal, w.window)
    check_every_row(w, q, k, v, out, lse, chunk_rows=8192)


# ---------------------------------------------------------------- exact cases
@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float16, torch.float32])
def test_causal_row0_is_v0_bitwise(dtype):
    q, k, v = make_qkv(2, 300, 3, 128, dtype, 5)
    out, lse = gpu_fwd(q, k, v, 1 / math.sqrt(128), True, (-1, -1))
    assert torch.equal(out[:, 0], v[:, 0])
    ref = (q[:, 0].double() * k[:, 0].double()).sum(-1) / math.sqrt(128)  # [B, H]
    assert torch.allclose(lse[:, :, 0].double(), ref, atol=1e-4, rtol=0)


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float16, torch.float32])
def test_window_zero_returns_v_bitwise(dtype):
    q, k, v = make_qkv(1, 517, 2, 64, dtype, 6)
    out, _ = gpu_fwd(q, k, v, 0.125, False, (0, 0))
    assert torch.equal(out, v)


@pytest.mark.parametrize("causal,window", [(False, (-1, -1)), (True, (-1, -1)), (False, (50, 20))])
def test_zero_q_gives_window_mean(causal, window):
    q, k, v = make_qkv(1, 333, 2, 128, torch.float32, 8)
    q = torch.zeros_like(q)
    out, lse = gpu_fwd(q, k, v, 0.1, causal, window)
    ref_o, ref_l = oracle.fwd(q, k, v, 0.1, causal, window)
    assert_close(out, lse, ref_o, ref_l, torch.float32, "q=0")
    n = np.exp(ref_l)  # allowed-key counts
    assert np.allclose(lse.double().numpy(), np.log(np.round(n)), atol=1e-5)


def test_scale_zero_uniform():
    q, k, v = make_qkv(1, 200, 2, 64, torch.bfloat16, 9)
    out, lse = gpu_fwd(q, k, v, 0.0, True, (-1, -1))
    ref_o, ref_l = oracle.fwd(q, k, v, 0.0, True, (-1, -1))
    assert_close(out, lse, ref_o, ref_l, torch.bfloat16, "scale=0")


def test_large_scale_stable():
    """scale = 50: |scores| in the hundreds; no overflow, matches the oracle."""
    q, k, v = make_qkv(1, 300, 2, 128, torch.bfloat16, 10)
    out, lse = gpu_fwd(q, k, v, 50.0, False, (-1, -1))
    ref_o, ref_l = oracle.fwd(q, k, v, 50.0, False, (-1, -1))
    assert_close(out, lse, ref_o, ref_l, torch.bfloat16, "scale=50")


@pytest.mark.parametrize("dtype", [torch.float16, torch.bfloat16])
def test_late_large_score_jump(dtype):
    """Every row meets one key late in its K/V range (key 900 of 1000) whose
    scaled score is about 32 above the others' (46 in log2 units): the bf16
    steps, which skip the row max, see the tile's weights far exceed the
    weight-sum check and move the reference up; fp16 takes the row max of
    that tile.  Both match the oracle: O is close to that key's value row."""
    B, S, H, D = 1, 1000, 2, 64
    q, k, v = make_qkv(B, S, H, D, dtype, 12)
    u = q[0, 0, 0].clone()
    q[0, :, 0] = u
    k[0, 900, 0] = 4 * u
    out, lse = gpu_fwd(q, k, v, 0.125, False, (-1, -1))
    ref_o, ref_l = oracle.fwd(q, k, v, 0.125, False, (-1, -1))
    assert float(ref_l[0, 0].min()) > 20, "the jump must dominate every row of head 0"
    assert_close(out, lse, ref_o, ref_l, dtype, f"late jump {dtype}")


# ---------------------------------------------------------------- robustness
def test_nan_rows_propagate_like_the_oracle():
    q, k, v = make_qkv(1, 257, 1, 64, torch.bfloat16, 11)
    q[0, 100, 0, 3] = float("nan")
    k[0, 200, 0, 7] = float("nan")
    out, lse = gpu_fwd(q, k, v, 0.125, True, (-1, -1))
    ref_o, ref_l = oracle.fwd(q, k, v, 0.125, True, (-1, -1))
    nan_rows = np.isnan(ref_l[0, 0])
    assert np.array_equal(torch.isnan(lse[0, 0]).numpy(), nan_rows)
    assert np.array_equal(torch.isnan(out[0, :, 0]).all(-1).numpy(), nan_rows)
    ok = ~nan_rows
    assert_close(out[:, ok], lse[:, :, ok], ref_o[:, ok], ref_l[:, :, ok], torch.bfloat16, "nan")


def test_deterministic_and_guard_bands():
    """Two runs are bitwise identical; memory around out and lse untouched."""
    import io_aware_exact_22_amd as fa

    B, S, H, D = 2, 1000, 4, 128
    q, k, v = (t.cuda() for t in make_qkv(B, S, H, D, torch.bfloat16, 12))
    n, nl = B * S * H * D, B * H * S
    guard = 4096
    obuf = torch.full((n + 2 * guard,), 7.0, dtype=torch.bfloat16, device="cuda")
    lbuf = torch.full((nl + 2 * guard,), -3.0, dtype=torch.float32, device="cuda")
    res = []
    for _ in range(2):
        out = obuf[guard:guard + n].view(B, S, H, D)
        lse = lbuf[guard:guard + nl].view(B, H, S)
        fa.flash_attn_fwd(q, k, v, causal=True, out=out, lse=lse)
        torch.cuda.synchronize()
        res.append((out.clone(), lse.clone()))
    assert torch.equal(res[0][0], res[1][0]) and torch.equal(res[0][1], res[1][1])
    assert (obuf[:guard] == 7.0).all() and (obuf[guard + n:] == 7.0).all()
    assert (lbuf[:guard] == -3.0).all() and (lbuf[guard + nl:] == -3.0).all()


def test_streams():
    """Runs on a non-default stream and on two streams at once."""
    import io_aware_exact_22_amd as fa

    q1, k1, v1 = (t.cuda() for t in make_qkv(1, 640, 2, 64, torch.bfloat16, 13))
    q2, k2, v2 = (t.cuda() for t in make_qkv(1, 900, 2, 128, torch.float16, 14))
    ref1 = fa.flash_attn_fwd(q1, k1, v1, causal=True)
    ref2 = fa.flash_attn_fwd(q2, k2, v2, window_size=(64, 64))
    torch.cuda.synchronize()
    s1, s2 = torch.cuda.Stream(), torch.cuda.Stream()
    torch.cuda.synchronize()
    with torch.cuda.stream(s1):
        o1 = fa.flash_attn_fwd(q1, k1, v1, causal=True)
    with torch.cuda.stream(s2):
        o2 = fa.flash_attn_fwd(q2, k2, v2, window_size=(64, 64))
    torch.cuda.synchronize()
    assert torch.equal(o1[0], ref1[0]) and torch.equal(o1[1], ref1[1])
    assert torch.equal(o2[0], ref2[0]) and torch.equal(o2[1], ref2[1])


def test_raw_c_abi_call():
    """fa_fwd through the raw C signature (pointers and sizes), default stream."""
    import io_aware_exact_22_amd as fa

    q, k, v = make_qkv(1, 130, 2, 64, torch.float32, 15)
    qd, kd, vd = (t.cuda() for t in (q, k, v))
    out = torch.empty_like(qd)
    lse = torch.empty((1, 2, 130), dtype=torch.float32, device="cuda")
    torch.cuda.synchronize()
    rc = fa.fa_fwd(qd.data_ptr(), kd.data_ptr(), vd.data_ptr(), out.data_ptr(), lse.data_ptr(), 1, 2,
                   130, 64, 0.125, 0, -1, -1, fa.FA_DTYPE_FP32, None)
    assert rc == 0
    torch.cuda.synchronize()
    ref_o, ref_l = oracle.fwd(q, k, v, 0.125, False, (-1, -1))
    assert_close(out.cpu(), lse.cpu(), ref_o, ref_l, torch.float32, "raw")
    # invalid arguments: status returned, nothing written
    out.fill_(1.0)
    torch.cuda.synchronize()
    rc = fa.fa_fwd(qd.data_ptr(), kd.data_ptr(), vd.data_ptr(), out.data_ptr(), lse.data_ptr(), 1, 2,
                   130, 64, -1.0, 0, -1, -1, fa.FA_DTYPE_FP32, None)
    assert rc == -6
    torch.cuda.synchronize()
    assert (out == 1.0).all()


# ---------------------------------------------------------------- split-KV
def gpu_fwd_splitkv(q, k, v, scale, causal, window, n_splits):
    import io_aware_exact_22_amd as fa

    qd, kd, vd = (t.cuda() for t in (q, k, v))
    out, lse = fa.flash_attn_fwd_splitkv(qd, kd, vd, softmax_scale=scale, causal=causal,
                                         window_size=window, n_splits=n_splits)
    torch.cuda.synchronize()
    return out.cpu(), lse.cpu()


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float16, torch.float32])
@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("causal,window", [(False, (-1, -1)), (True, (-1, -1)), (False, (128, 128)),
                                           (True, (100, -1)), (False, (33, 7))])
@pytest.mark.parametrize("n_splits", [2, 3])
def test_splitkv_parity(dtype, D, causal, window, n_splits):
    """fa_fwd_splitkv against the oracle, every element: ragged S, several
    heads and batches, each mask mode."""
    q, k, v = make_qkv(2, 389, 3, D, dtype, 29)
    scale = 1.0 / math.sqrt(D)
    what = f"splitkv x{n_splits} D{D} {dtype} causal={causal} window={window}"
    print("run", what, flush=True)
    out, lse = gpu_fwd_splitkv(q, k, v, scale, causal, window, n_splits)
    ref_out, ref_lse = oracle.fwd(q, k, v, scale, causal, window)
    assert_close(out, lse, ref_out, ref_lse, dtype, what)


@pytest.mark.parametrize("S,n_splits", [(100, 4), (130, 16), (1, 2), (4097, 5), (2048, 16)])
@pytest.mark.parametrize("causal", [False, True])
def test_splitkv_more_parts_than_tiles(S, n_splits, causal):
    """More parts than a Q tile has K/V tiles (empty parts), and long rows cut
    into many parts."""
    q, k, v = make_qkv(1, S, 2, 128, torch.bfloat16, S + n_splits)
    print(f"run splitkv S{S} x{n_splits} causal={causal}", flush=True)
    out, lse = gpu_fwd_splitkv(q, k, v, 0.0883883, causal, (-1, -1), n_splits)
    ref_out, ref_lse = oracle.fwd(q, k, v, 0.0883883, causal, (-1, -1))
    assert_close(out, lse, ref_out, ref_lse, torch.bfloat16, f"S{S} x{n_splits}")


@pytest.mark.parametrize("n_splits", [0, 2])
def test_splitkv_gpt_causal_2k(n_splits):
    """The 2K causal workload at full size, every element, in 2 parts and in
    the library's part count (1 here: 512 workgroups fill 256 CUs twice)."""
    import io_aware_exact_22_amd as fa

    w = WORKLOADS["gpt_causal_2k"]
    ns = fa.fa_fwd_splitkv_auto_splits(w.B, w.H, w.S, w.D, 1, -1, -1, fa.FA_DTYPE_BF16)
    print("auto splits", ns, flush=True)
    assert 1 <= ns <= 8
    q, k, v = workload_qkv(w)
    out, lse = gpu_fwd_splitkv(q, k, v, w.scale, w.causal, w.window, n_splits)
    ref_out, ref_lse = oracle.fwd(q, k, v, w.scale, w.causal, w.window)
    assert_close(out, lse, ref_out, ref_lse, w.dtype, f"gpt_causal_2k x{n_splits or ns}")


@pytest.mark.parametrize("n_splits", [0, 4])
def test_splitkv_head_sharded_16k(n_splits):
    """One GPU's share of the 16K causal workload under head sharding (2 of
    16 heads) in the library's part count and in 4 parts: every element of
    both heads."""
    w = WORKLOADS["causal_16k_h2"]
    q, k, v = workload_qkv(w)
    out, lse = gpu_fwd_splitkv(q, k, v, w.scale, w.causal, w.window, n_splits)
    check_every_row(w, q, k, v, out, lse)


def test_splitkv_nan_rows_propagate_like_the_oracle():
    q, k, v = make_qkv(1, 257, 1, 64, torch.bfloat16, 11)
    q[0, 100, 0, 3] = float("nan")
    k[0, 200, 0, 7] = float("nan")
    out, lse = gpu_fwd_splitkv(q, k, v, 0.125, True, (-1, -1), 3)
    ref_o, ref_l = oracle.fwd(q, k, v, 0.125, True, (-1, -1))
    nan_rows = np.isnan(ref_l[0, 0])
    assert np.array_equal(torch.isnan(lse[0, 0]).numpy(), nan_rows)
    assert np.array_equal(torch.isnan(out[0, :, 0]).all(-1).numpy(), nan_rows)
    ok = ~nan_rows
    assert_close(out[:, ok], lse[:, :, ok], ref_o[:, ok], ref_l[:, :, ok], torch.bfloat16, "nan")


def test_splitkv_workspace_guard_bands():
    """The split writes only its workspace, out and lse: memory around a
    caller's workspace is untouched, and a second run is bitwise identical."""
    import io_aware_exact_22_amd as fa

    q, k, v = (t.cuda() for t in make_qkv(2, 300, 3, 64, torch.float16, 5))
    need = fa.fa_fwd_splitkv_workspace_size(2, 3, 300, 64, fa.FA_DTYPE_FP16, 3)
    pad = 4096
    buf = torch.full(((need + 2 * pad) // 4,), 7.0, dtype=torch.float32, device="cuda")
    ws = buf[pad // 4: (pad + need) // 4]
    o1, l1 = fa.flash_attn_fwd_splitkv(q, k, v, causal=True, n_splits=3, workspace=ws)
    o2, l2 = fa.flash_attn_fwd_splitkv(q, k, v, causal=True, n_splits=3, workspace=ws)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)
    assert bool((buf[: pad // 4] == 7.0).all()) and bool((buf[(pad + need) // 4:] == 7.0).all())


# ---------------------------------------------------------------- backward
TOL_GRAD = {torch.float16: 4e-3, torch.bfloat16: 2e-2}


def gpu_bwd(q, k, v, do, scale, causal, window):
    import io_aware_exact_22_amd as fa

    qd, kd, vd, dod = (t.cuda() for t in (q, k, v, do))
    out, lse = fa.flash_attn_fwd(qd, kd, vd, softmax_scale=scale, causal=causal, window_size=window)
    dq, dk, dv = fa.flash_attn_bwd(dod, qd, kd, vd, out, lse, softmax_scale=scale, causal=causal,
                                   window_size=window)
    torch.cuda.synchronize()
    return dq.cpu(), dk.cpu(), dv.cpu()


def check_bwd(B, S, H, D, dtype, causal, window, seed, scale=None):
    """dq, dk, dv against the oracle's fp64 gradients: max-abs error within
    TOL_GRAD[dtype] x max(1, max |reference|), per gradient."""
    scale = 1.0 / math.sqrt(D) if scale is None else scale
    q, k, v = make_qkv(B, S, H, D, dtype, seed)
    do = make_qkv(B, S, H, D, dtype, seed + 1)[0]
    what = f"bwd B{B} S{S} H{H} D{D} {dtype} causal={causal} window={window}"
    print("run", what, flush=True)
    got = gpu_bwd(q, k, v, do, scale, causal, window)
    ref = oracle.bwd(q, k, v, do, scale, causal, window)
    for name, g, r in zip(("dq", "dk", "dv"), got, ref):
        g = g.double().numpy()
        assert np.all(np.isfinite(g)), f"{what}: non-finite {name}"
        bound = TOL_GRAD[dtype] * max(1.0, float(np.max(np.abs(r))))
        err = float(np.max(np.abs(g - r)))
        print(f"{what}: {name} max err {err:.3e} (bound {bound:.3e})", flush=True)
        assert err <= bound, f"{what}: {name} error {err} > {bound}"


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float16])
@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("causal,window", [(False, (-1, -1)), (True, (-1, -1)), (False, (128, 128)),
                                           (True, (100, -1)), (False, (33, 7))])
def test_bwd_parity(dtype, D, causal, window):
    check_bwd(2, 389, 3, D, dtype, causal, window, seed=71)


@pytest.mark.parametrize("S", [1, 63, 64, 65, 128, 129, 1000])
@pytest.mark.parametrize("causal", [False, True])
def test_bwd_lengths(S, causal):
    check_bwd(1, S, 2, 128, torch.bfloat16, causal, (-1, -1), seed=S + 3)


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float16])
@pytest.mark.parametrize("H,D", [(32, 64), (20, 128)])
def test_bwd_dynamic_tail(dtype, H, D):
    """Causal backward passes with more workgroups than the device holds at
    once take their lightest tiles (Q tiles for dQ, key blocks for dK / dV) in
    the dynamic order, with counters in the workspace: every element against
    the oracle."""
    check_bwd(1, 4096, H, D, dtype, True, (-1, -1), seed=90 + H)


def test_bwd_gpt_causal_2k():
    """The 2K causal workload's shape (B2 H16 S2048 D64 bf16), every element."""
    check_bwd(2, 2048, 16, 64, torch.bfloat16, True, (-1, -1), seed=81)


def test_bwd_causal_16k_sampled_and_column_sums():
    """The backward at the benchmark's full size and launch configuration
    (1 x 16 heads x 16384 x 128, bf16, causal): sampled dq rows and dk / dv
    keys of two heads against the oracle's sampled gradients, within
    TOL_GRAD x max(1, max |reference|); and, over every head and d, the column
    sums that hold for any inputs, sum_j dK_j = 0 and sum_j dV_j = sum_i dO_i,
    within 2% of the columns' root-sum-square."""
    B, S, H, D = 1, 16384, 16, 128
    scale = 1.0 / math.sqrt(D)
    q, k, v = make_qkv(B, S, H, D, torch.bfloat16, 5)
    do = make_qkv(B, S, H, D, torch.bfloat16, 6)[0]
    print("run bwd causal 16384 x 16 heads", flush=True)
    dq, dk, dv = gpu_bwd(q, k, v, do, scale, True, (-1, -1))
    for name, g in (("dq", dq), ("dk", dk), ("dv", dv)):
        assert torch.isfinite(g.float()).all(), name
    dkd, dvd, dod = (t.double()[0] for t in (dk, dv, do))  # [S, H, D]
    sum_k = dkd.sum(0)
    assert (sum_k.abs() <= 0.02 * dkd.pow(2).sum(0).sqrt()).all(), "sum_j dK_j != 0"
    sum_v = dvd.sum(0) - dod.sum(0)
    assert (sum_v.abs() <= 0.02 * dod.pow(2).sum(0).sqrt()).all(), "sum_j dV_j != sum_i dO_i"
    rows = [0, 1, 63, 64, 4095, 8192, 16383]
    keys = [0, 1, 127, 128, 8191, 16320, 16383]
    for h in (0, 15):
        rq, rk, rv = oracle.bwd_sampled(q, k, v, do, scale, True, (-1, -1), 0, h, rows, keys)
        for name, g, r in (("dq", dq[0, rows, h], rq), ("dk", dk[0, keys, h], rk),
                           ("dv", dv[0, keys, h], rv)):
            g = g.double().numpy()
            bound = TOL_GRAD[torch.bfloat16] * max(1.0, float(np.max(np.abs(r))))
            err = float(np.max(np.abs(g - r)))
            print(f"bwd 16k head {h}: {name} max err {err:.3e} (bound {bound:.3e})", flush=True)
            assert err <= bound, f"head {h} {name}: {err} > {bound}"
