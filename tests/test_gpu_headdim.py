"""GPU parity at head dimensions other than 64 and 128 (bf16 / fp16): fa_fwd,
fa_fwd_splitkv, fa_fwd_paged and fa_fwd_blocksparse through the C ABI against
the CPU oracle on the same seeded inputs, every element.

The kernels run such a D as the next of 64, 128 and 256 with the extra
columns read as zeros and never written (D = 256 itself runs its own kernel,
with 32-key K/V tiles), so these cases check that the tensors' own row
stride (H * D) is used everywhere, that the padding adds nothing to the
scores or O, and that no byte outside O, LSE or the split partials is
written (guard bands around the outputs).  H = 1 makes the tensors' rows
shorter than the kernel's LDS rows.  fp32 inputs take D up to 128.
Tolerances as for the dense forward (max-abs): O <= 1e-4 fp32, <= 4e-3 fp16,
<= 2e-2 bf16; LSE <= 1e-3.
"""
import math

import numpy as np
import pytest
import torch

import oracle
from fa_inputs import make_qkv, random_block_mask

pytestmark = pytest.mark.gpu

TOL_O = {torch.float32: 1e-4, torch.float16: 4e-3, torch.bfloat16: 2e-2}
TOL_LSE = 1e-3
D_OTHER = [16, 32, 48, 80, 96, 112, 144, 192, 256]
MASKS = [(False, (-1, -1)), (True, (-1, -1)), (False, (200, 100)), (True, (100, -1))]
GUARD = 4096  # elements of guard band on each side of an output


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")
    import io_aware_exact_22_amd  # noqa: F401  (fails loudly if the library is missing)


def guarded(shape, dtype):
    """A tensor of `shape` inside a NaN-filled buffer with GUARD elements on
    each side; returns (view, buffer)."""
    n = int(np.prod(shape))
    buf = torch.full((n + 2 * GUARD,), float("nan"), dtype=dtype, device="cuda")
    return buf[GUARD:GUARD + n].view(shape), buf


def guards_intact(buf):
    g = torch.cat([buf[:GUARD], buf[-GUARD:]]).float()
    return bool(torch.isnan(g).all())


def compare(out, lse, ref_o, ref_l, dtype, what):
    o = out.double().cpu().numpy()
    ls = lse.double().cpu().numpy()
    assert np.all(np.isfinite(ref_o)) and np.all(np.isfinite(ref_l))
    assert np.all(np.isfinite(o)) and np.all(np.isfinite(ls)), f"{what}: non-finite output"
    eo = float(np.max(np.abs(o - ref_o)))
    el = float(np.max(np.abs(ls - ref_l)))
    print(f"{what}: max|dO|={eo:.3e} max|dLSE|={el:.3e}", flush=True)
    assert eo <= TOL_O[dtype], f"{what}: O error {eo} > {TOL_O[dtype]}"
    assert el <= TOL_LSE, f"{what}: LSE error {el} > {TOL_LSE}"


def run_guarded(fn, B, S, H, D, dtype):
    out, obuf = guarded((B, S, H, D), dtype)
    lse, lbuf = guarded((B, H, S), torch.float32)
    fn(out, lse)
    torch.cuda.synchronize()
    assert guards_intact(obuf) and guards_intact(lbuf), "a write landed outside O or LSE"
    return out, lse


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float16, torch.float32])
@pytest.mark.parametrize("D", D_OTHER)
@pytest.mark.parametrize("causal,window", MASKS)
@pytest.mark.parametrize("B,S,H", [(2, 389, 3), (1, 300, 1)])
def test_headdim_fwd(dtype, D, causal, window, B, S, H):
    import io_aware_exact_22_amd as fa

    if dtype == torch.float32 and D > 128:
        pytest.skip("fp32 inputs take head dimensions up to 128")

    q, k, v = make_qkv(B, S, H, D, dtype, 400 + D)
    what = f"fwd B{B} S{S} H{H} D{D} {dtype} causal={causal} window={window}"
    print("run", what, flush=True)
    qd, kd, vd = (t.cuda() for t in (q, k, v))
    out, lse = run_guarded(lambda o, l: fa.flash_attn_fwd(qd, kd, vd, causal=causal,
                                                          window_size=window, out=o, lse=l),
                           B, S, H, D, dtype)
    ref_o, ref_l = oracle.fwd(q, k, v, 1.0 / math.sqrt(D), causal, window)
    compare(out, lse, ref_o, ref_l, dtype, what)


@pytest.mark.parametrize("D", [32, 96, 256])
@pytest.mark.parametrize("causal", [False, True])
def test_headdim_long_sequence(D, causal):
    """4100 rows (ragged last Q and K/V tiles), every element."""
    import io_aware_exact_22_amd as fa

    B, S, H, dtype = 1, 4100, 2, torch.bfloat16
    q, k, v = make_qkv(B, S, H, D, dtype, 500 + D)
    what = f"long S{S} D{D} causal={causal}"
    print("run", what, flush=True)
    qd, kd, vd = (t.cuda() for t in (q, k, v))
    out, lse = fa.flash_attn_fwd(qd, kd, vd, causal=causal)
    torch.cuda.synchronize()
    ref_o, ref_l = oracle.fwd(q, k, v, 1.0 / math.sqrt(D), causal)
    compare(out, lse, ref_o, ref_l, dtype, what)


@pytest.mark.parametrize("D", [16, 48, 80, 112, 160, 256])
@pytest.mark.parametrize("n_splits", [2, 5])
@pytest.mark.parametrize("causal", [False, True])
def test_headdim_splitkv(D, n_splits, causal):
    """Split partials of D columns per row (the workspace holds exactly
    n_splits * B*H*S * (D + 1) fp32 values: guard bands around it stay
    untouched) and the merge."""
    import io_aware_exact_22_amd as fa

    B, S, H, dtype = 2, 700, 2, torch.float16
    q, k, v = make_qkv(B, S, H, D, dtype, 600 + D + n_splits)
    what = f"splitkv D{D} parts={n_splits} causal={causal}"
    print("run", what, flush=True)
    qd, kd, vd = (t.cuda() for t in (q, k, v))
    need = fa.fa_fwd_splitkv_workspace_size(B, H, S, D, fa.FA_DTYPE_FP16, n_splits)
    assert need == n_splits * B * H * S * (D + 1) * 4
    ws, wbuf = guarded((need // 4,), torch.float32)
    out, lse = run_guarded(lambda o, l: fa.flash_attn_fwd_splitkv(
        qd, kd, vd, causal=causal, n_splits=n_splits, out=o, lse=l, workspace=ws),
        B, S, H, D, dtype)
    assert guards_intact(wbuf), "a write landed outside the workspace"
    ref_o, ref_l = oracle.fwd(q, k, v, 1.0 / math.sqrt(D), causal)
    compare(out, lse, ref_o, ref_l, dtype, what)


def paginate(x, page_size, num_pages, seed):
    """Pages of x [B, S, H, D] at a seeded permutation of the pool's slots;
    unused rows and pages hold NaN.  Returns (pool, table [B, n] int32)."""
    B, S, H, D = x.shape
    n = -(-S // page_size)
    g = torch.Generator(device="cpu")
    g.manual_seed(seed)
    slots = torch.randperm(num_pages, generator=g)[: B * n].view(B, n)
    padded = torch.full((B, n * page_size, H, D), float("nan"), dtype=x.dtype, device=x.device)
    padded[:, :S] = x
    pool = torch.full((num_pages, page_size, H, D), float("nan"), dtype=x.dtype, device=x.device)
    pool[slots.reshape(-1).to(x.device)] = padded.view(B * n, page_size, H, D)
    return pool.contiguous(), slots.to(torch.int32).to(x.device).contiguous()


@pytest.mark.parametrize("D,dtype", [(32, torch.bfloat16), (80, torch.bfloat16),
                                     (208, torch.bfloat16), (256, torch.bfloat16),
                                     (48, torch.float32), (112, torch.float32)])
@pytest.mark.parametrize("causal,window", [(False, (-1, -1)), (True, (300, -1))])
def test_headdim_paged(D, dtype, causal, window):
    """Paged K/V equals the contiguous result bit for bit, and the oracle."""
    import io_aware_exact_22_amd as fa

    B, S, H, page = 2, 777, 3, 128
    q, k, v = make_qkv(B, S, H, D, dtype, 700 + D)
    what = f"paged D{D} causal={causal} window={window}"
    print("run", what, flush=True)
    qd, kd, vd = (t.cuda() for t in (q, k, v))
    n = -(-S // page)
    kp, table = paginate(kd, page, B * n + 2, 3)
    vp, _ = paginate(vd, page, B * n + 2, 3)
    o1, l1 = fa.flash_attn_fwd_paged(qd, kp, vp, table, causal=causal, window_size=window)
    o2, l2 = fa.flash_attn_fwd(qd, kd, vd, causal=causal, window_size=window)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2), what
    ref_o, ref_l = oracle.fwd(q, k, v, 1.0 / math.sqrt(D), causal, window)
    compare(o1, l1, ref_o, ref_l, dtype, what)


@pytest.mark.parametrize("D,dtype", [(48, torch.float16), (96, torch.float16),
                                     (224, torch.float16), (256, torch.float16),
                                     (80, torch.float32)])
def test_headdim_blocksparse(D, dtype):
    """A random mask per (batch, head), 40% of the 128 x 64 blocks kept."""
    import io_aware_exact_22_amd as fa

    B, S, H = 2, 777, 3
    q, k, v = make_qkv(B, S, H, D, dtype, 800 + D)
    mask = random_block_mask(B * H, -(-S // 128), -(-S // 64), 0.4, 900 + D)
    what = f"blocksparse D{D}"
    print("run", what, flush=True)
    qd, kd, vd = (t.cuda() for t in (q, k, v))
    out, lse = fa.flash_attn_fwd_blocksparse(qd, kd, vd, mask.cuda(), 128, 64, causal=True)
    torch.cuda.synchronize()
    ref_o, ref_l = oracle.fwd_blocksparse(q, k, v, 1.0 / math.sqrt(D), mask.numpy(), 128, 64,
                                          True)
    o = out.double().cpu().numpy()
    ls = lse.double().cpu().numpy()
    empty = np.isneginf(ref_l)
    assert np.array_equal(np.isneginf(ls), empty), f"{what}: rows without keys differ"
    eo = float(np.max(np.abs(o - ref_o)))
    el = float(np.max(np.abs(ls[~empty] - ref_l[~empty])))
    print(f"{what}: max|dO|={eo:.3e} max|dLSE|={el:.3e}", flush=True)
    assert eo <= TOL_O[dtype] and el <= TOL_LSE, what


@pytest.mark.parametrize("D,H,dtype", [(48, 1, torch.bfloat16), (112, 2, torch.bfloat16),
                                       (176, 1, torch.bfloat16), (256, 2, torch.bfloat16),
                                       (32, 2, torch.float32)])
def test_headdim_nonfinite_values_outside_the_mask(D, H, dtype):
    """NaN and inf in V at keys the causal mask hides from some rows of the
    same tile: the exact recomputation (columns past D read as zeros) gives
    the oracle's NaN pattern, finite rows within tolerance."""
    import io_aware_exact_22_amd as fa

    B, S = 1, 300
    q, k, v = make_qkv(B, S, H, D, dtype, 950 + D)
    v[0, 100, 0, 3] = float("nan")      # rows 96..99 share its K/V tile but not the key
    v[0, 200, H - 1, D - 1] = float("inf")
    qd, kd, vd = (t.cuda() for t in (q, k, v))
    out, lse = fa.flash_attn_fwd(qd, kd, vd, causal=True)
    torch.cuda.synchronize()
    ref_o, ref_l = oracle.fwd(q, k, v, 1.0 / math.sqrt(D), True)
    o = out.double().cpu().numpy()
    assert np.array_equal(np.isnan(o), np.isnan(ref_o)), "NaN pattern differs"
    assert np.array_equal(np.isposinf(o), np.isposinf(ref_o)), "inf pattern differs"
    assert np.isnan(ref_o).any() and np.isfinite(ref_o[0, :100]).all()
    fin = np.isfinite(ref_o)
    eo = float(np.max(np.abs(o[fin] - ref_o[fin])))
    el = float(np.max(np.abs(lse.double().cpu().numpy() - ref_l)))
    print(f"nonfinite D{D} H{H}: max|dO|={eo:.3e} max|dLSE|={el:.3e}", flush=True)
    assert eo <= TOL_O[dtype] and el <= TOL_LSE


# ---------------------------------------------------------------- backward
TOL_GRAD = {torch.float16: 4e-3, torch.bfloat16: 2e-2}


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float16])
@pytest.mark.parametrize("D", [16, 48, 80, 112])
@pytest.mark.parametrize("causal,window", MASKS)
@pytest.mark.parametrize("B,S,H", [(2, 389, 3), (1, 300, 1)])
def test_headdim_bwd(dtype, D, causal, window, B, S, H):
    """dq, dk, dv against the oracle's fp64 gradients (max-abs within
    TOL_GRAD x max(1, max |reference|)), with NaN guard bands around each
    gradient and around the row-dot workspace that must stay untouched."""
    import io_aware_exact_22_amd as fa

    q, k, v = make_qkv(B, S, H, D, dtype, 1000 + D)
    do = make_qkv(B, S, H, D, dtype, 1001 + D)[0]
    scale = 1.0 / math.sqrt(D)
    what = f"bwd B{B} S{S} H{H} D{D} {dtype} causal={causal} window={window}"
    print("run", what, flush=True)
    qd, kd, vd, dod = (t.cuda() for t in (q, k, v, do))
    out, lse = fa.flash_attn_fwd(qd, kd, vd, causal=causal, window_size=window)
    grads = [guarded((B, S, H, D), dtype) for _ in range(3)]
    dcode = fa.FA_DTYPE_BF16 if dtype == torch.bfloat16 else fa.FA_DTYPE_FP16
    ws, wbuf = guarded(((fa.fa_bwd_workspace_size(B, H, S, D, dcode) + 3) // 4,), torch.float32)
    fa.flash_attn_bwd(dod, qd, kd, vd, out, lse, causal=causal, window_size=window, workspace=ws,
                      dq=grads[0][0], dk=grads[1][0], dv=grads[2][0])
    torch.cuda.synchronize()
    assert all(guards_intact(b) for _, b in grads) and guards_intact(wbuf), \
        "a write landed outside a gradient or the workspace"
    ref = oracle.bwd(q, k, v, do, scale, causal, window)
    for name, (g, _), r in zip(("dq", "dk", "dv"), grads, ref):
        g = g.double().cpu().numpy()
        assert np.all(np.isfinite(g)), f"{what}: non-finite {name}"
        bound = TOL_GRAD[dtype] * max(1.0, float(np.max(np.abs(r))))
        err = float(np.max(np.abs(g - r)))
        print(f"{what}: {name} max err {err:.3e} (bound {bound:.3e})", flush=True)
        assert err <= bound, f"{what}: {name} error {err} > {bound}"
