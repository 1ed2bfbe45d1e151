"""GPU parity on seeded random configurations: every entry point of the
forward (fa_fwd, fa_fwd_splitkv, fa_fwd_paged, fa_fwd_blocksparse,
fa_fwd_kvcache) and the backward (fa_bwd) through the C ABI against the CPU
oracle, every element, on
shapes, head dimensions, dtypes and masks drawn from one fixed seed per case
(small sizes: B <= 3, H <= 5, S <= 700), so that combinations no hand-written
case names are still checked.  Tolerances as for the dense forward (max-abs):
O <= 1e-4 fp32, <= 4e-3 fp16, <= 2e-2 bf16; LSE <= 1e-3; rows with no
allowed key exactly O = 0, LSE = -inf."""
import math
import random

import numpy as np
import pytest
import torch

import oracle
from fa_inputs import make_qkv, random_block_mask

pytestmark = pytest.mark.gpu

TOL_O = {torch.float32: 1e-4, torch.float16: 4e-3, torch.bfloat16: 2e-2}
DTYPES = [torch.bfloat16, torch.float16, torch.float32]
N_CASES = 200


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")
    import io_aware_exact_22_amd  # noqa: F401  (fails loudly if the library is missing)


def draw(seed):
    """One random configuration: (entry, B, H, S, D, dtype, causal, window, extra)."""
    r = random.Random(seed)
    entry = r.choice(["fwd", "splitkv", "paged", "blocksparse"])
    dtype = r.choice(DTYPES if entry != "splitkv" else DTYPES[:2])
    dmax = 128 if dtype == torch.float32 else 256
    D = 16 * r.randint(1, dmax // 16)
    B, H = r.randint(1, 3), r.randint(1, 5)
    S = r.choice([r.randint(1, 64), r.randint(65, 300), r.randint(301, 700)])
    causal = r.random() < 0.5
    wl = r.choice([-1, -1, r.randint(0, 300)])
    wr = r.choice([-1, -1, r.randint(0, 300)])
    extra = {"n_splits": r.randint(2, 6), "page": r.choice([64, 128, 192]),
             "density": r.choice([0.2, 0.5, 0.9]), "n_mask": r.choice(["1", "H", "BH"])}
    return entry, B, H, S, D, dtype, causal, (wl, wr), extra


def compare(out, lse, ref_o, ref_l, dtype, what):
    o = out.double().cpu().numpy()
    ls = lse.double().cpu().numpy()
    empty = np.isneginf(ref_l)
    assert np.array_equal(np.isneginf(ls), empty), f"{what}: rows without keys differ"
    assert np.all(np.isfinite(o)), f"{what}: non-finite O"
    live = ~empty
    eo = float(np.max(np.abs(o - ref_o))) if o.size else 0.0
    el = float(np.max(np.abs(ls[live] - ref_l[live]))) if live.any() else 0.0
    print(f"{what}: max|dO|={eo:.3e} max|dLSE|={el:.3e}", flush=True)
    assert eo <= TOL_O[dtype], f"{what}: O error {eo} > {TOL_O[dtype]}"
    assert el <= 1e-3, f"{what}: LSE error {el}"


def paginate(x, page_size, seed):
    """Pages of x [B, S, H, D] at a seeded permutation of a pool with two spare
    pages; unused rows and pages hold NaN.  Returns (pool, table [B, n])."""
    B, S, H, D = x.shape
    n = -(-S // page_size)
    g = torch.Generator(device="cpu")
    g.manual_seed(seed)
    slots = torch.randperm(B * n + 2, generator=g)[: B * n].view(B, n)
    padded = torch.full((B, n * page_size, H, D), float("nan"), dtype=x.dtype, device=x.device)
    padded[:, :S] = x
    pool = torch.full((B * n + 2, page_size, H, D), float("nan"), dtype=x.dtype, device=x.device)
    pool[slots.reshape(-1).to(x.device)] = padded.view(B * n, page_size, H, D)
    return pool.contiguous(), slots.to(torch.int32).to(x.device).contiguous()


@pytest.mark.parametrize("seed", range(N_CASES))
def test_random_forward_configuration(seed):
    import io_aware_exact_22_amd as fa

    entry, B, H, S, D, dtype, causal, window, ex = draw(seed)
    what = f"seed {seed}: {entry} B{B} H{H} S{S} D{D} {dtype} causal={causal} window={window}"
    print("run", what, ex, flush=True)
    q, k, v = make_qkv(B, S, H, D, dtype, 5000 + seed)
    qd, kd, vd = (t.cuda() for t in (q, k, v))
    scale = 1.0 / math.sqrt(D)
    if entry == "blocksparse":
        n_mask = {"1": 1, "H": H, "BH": B * H}[ex["n_mask"]]
        mask = random_block_mask(n_mask, -(-S // 128), -(-S // 64), ex["density"], 6000 + seed)
        out, lse = fa.flash_attn_fwd_blocksparse(qd, kd, vd, mask.cuda(), 128, 64, causal=causal,
                                                 window_size=window)
        torch.cuda.synchronize()
        ref_o, ref_l = oracle.fwd_blocksparse(q, k, v, scale, mask.numpy(), 128, 64, causal,
                                              window)
        compare(out, lse, ref_o, ref_l, dtype, what)
        return
    if entry == "fwd":
        out, lse = fa.flash_attn_fwd(qd, kd, vd, causal=causal, window_size=window)
    elif entry == "splitkv":
        out, lse = fa.flash_attn_fwd_splitkv(qd, kd, vd, causal=causal, window_size=window,
                                             n_splits=ex["n_splits"])
    else:
        kp, table = paginate(kd, ex["page"], 7000 + seed)
        vp, _ = paginate(vd, ex["page"], 7000 + seed)
        out, lse = fa.flash_attn_fwd_paged(qd, kp, vp, table, causal=causal, window_size=window)
    torch.cuda.synchronize()
    ref_o, ref_l = oracle.fwd(q, k, v, scale, causal, window)
    compare(out, lse, ref_o, ref_l, dtype, what)


def draw_kv(seed):
    r = random.Random(10_000 + seed)
    dtype = r.choice(DTYPES[:2])
    D = 16 * r.randint(1, 8)
    B, H = r.randint(1, 4), r.randint(1, 4)
    S_q = r.choice([1, 1, r.randint(2, 40), r.randint(100, 200)])
    S_k = r.randint(64, 600)
    lens = [r.randint(0, S_k) for _ in range(B)]
    causal = r.random() < 0.7
    window = (r.choice([-1, r.randint(0, 200)]), r.choice([-1, r.randint(0, 50)]))
    paged = r.random() < 0.4
    n_splits = r.choice([1, 1, r.randint(2, 8)])
    return B, H, S_q, S_k, D, dtype, lens, causal, window, paged, n_splits


@pytest.mark.parametrize("seed", range(80))
def test_random_kvcache_configuration(seed):
    import io_aware_exact_22_amd as fa

    B, H, S_q, S_k, D, dtype, lens, causal, window, paged, ns = draw_kv(seed)
    what = (f"kv seed {seed}: B{B} H{H} S_q{S_q} S_k{S_k} D{D} {dtype} lens={lens} "
            f"causal={causal} window={window} paged={paged} parts={ns}")
    print("run", what, flush=True)
    q, _, _ = make_qkv(B, S_q, H, D, dtype, 8000 + seed)
    _, k, v = make_qkv(B, S_k, H, D, dtype, 8500 + seed)
    scale = 1.0 / math.sqrt(D)
    sl = torch.tensor(lens, dtype=torch.int32).cuda()
    if paged:
        page = 64
        n_pg = -(-S_k // page)
        kc = torch.zeros((B, n_pg * page, H, D), dtype=dtype)
        vc = torch.zeros((B, n_pg * page, H, D), dtype=dtype)
        kc[:, :S_k], vc[:, :S_k] = k, v
        kp, table = paginate(kc.cuda(), page, 9000 + seed)
        vp, _ = paginate(vc.cuda(), page, 9000 + seed)
        out, lse = fa.flash_attn_fwd_kvcache(q.cuda(), kp, vp, sl, block_table=table,
                                             causal=causal, window_size=window, n_splits=ns)
        ref_o, ref_l = oracle.fwd_kvcache(q, kc, vc, lens, scale, causal, window)
    else:
        out, lse = fa.flash_attn_fwd_kvcache(q.cuda(), k.cuda(), v.cuda(), sl, causal=causal,
                                             window_size=window, n_splits=ns)
        ref_o, ref_l = oracle.fwd_kvcache(q, k, v, lens, scale, causal, window)
    torch.cuda.synchronize()
    compare(out, lse, ref_o, ref_l, dtype, what)


TOL_GRAD = {torch.float16: 4e-3, torch.bfloat16: 2e-2}


def draw_bwd(seed):
    r = random.Random(20_000 + seed)
    dtype = r.choice(DTYPES[:2])
    D = 16 * r.randint(1, 8)
    B, H = r.randint(1, 3), r.randint(1, 4)
    S = r.choice([r.randint(1, 64), r.randint(65, 300), r.randint(301, 600)])
    causal = r.random() < 0.5
    window = (r.choice([-1, -1, r.randint(0, 200)]), r.choice([-1, -1, r.randint(0, 200)]))
    return B, H, S, D, dtype, causal, window


@pytest.mark.parametrize("seed", range(40))
def test_random_backward_configuration(seed):
    """fa_bwd on random shapes, head dimensions and masks: dq, dk, dv within
    TOL_GRAD x max(1, max |reference|) of the oracle's fp64 gradients."""
    import io_aware_exact_22_amd as fa

    B, H, S, D, dtype, causal, window = draw_bwd(seed)
    what = f"bwd seed {seed}: B{B} H{H} S{S} D{D} {dtype} causal={causal} window={window}"
    print("run", what, flush=True)
    q, k, v = make_qkv(B, S, H, D, dtype, 11000 + seed)
    do = make_qkv(B, S, H, D, dtype, 11500 + seed)[0]
    scale = 1.0 / math.sqrt(D)
    qd, kd, vd, dod = (t.cuda() for t in (q, k, v, do))
    out, lse = fa.flash_attn_fwd(qd, kd, vd, causal=causal, window_size=window)
    dq, dk, dv = fa.flash_attn_bwd(dod, qd, kd, vd, out, lse, causal=causal, window_size=window)
    torch.cuda.synchronize()
    ref = oracle.bwd(q, k, v, do, scale, causal, window)
    for name, g, r in zip(("dq", "dk", "dv"), (dq, dk, dv), ref):
        g = g.double().cpu().numpy()
        assert np.all(np.isfinite(g)), f"{what}: non-finite {name}"
        bound = TOL_GRAD[dtype] * max(1.0, float(np.max(np.abs(r))))
        err = float(np.max(np.abs(g - r)))
        print(f"{what}: {name} max err {err:.3e} (bound {bound:.3e})", flush=True)
        assert err <= bound, f"{what}: {name} error {err} > {bound}"
