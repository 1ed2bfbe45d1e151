"""GPU parity of fa_fwd_kvcache (attention of new queries against a key/value
cache: FlashDecoding, "FlashAttention技术解析：加速GPT训练的核心优化" section 5;
flash_attn_with_kvcache and the paged cache's block table,
"突破大模型训练瓶颈：Flash-Attention编译优化与内存占用解决方案" sections
总结与最佳实践 and Paged KV Cache支持) against oracle.fwd_kvcache, every element:
NaN and infinity patterns exactly (rows with no allowed key: O = 0,
LSE = -inf), other values within the tolerances (O <= 4e-3 fp16, <= 2e-2 bf16;
LSE <= 1e-3)."""
import math

import numpy as np
import pytest
import torch

import oracle
from fa_inputs import make_qkv

pytestmark = pytest.mark.gpu

TOL_O = {torch.float16: 4e-3, torch.bfloat16: 2e-2}


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")


def compare(out, lse, ref_o, ref_l, dtype, what):
    o = out.double().cpu().numpy()
    ls = lse.double().cpu().numpy()
    errs = []
    for name, g, r, tol in (("O", o, ref_o, TOL_O[dtype]), ("LSE", ls, ref_l, 1e-3)):
        assert np.array_equal(np.isnan(g), np.isnan(r)), f"{what}: {name} NaN pattern differs"
        inf = np.isinf(r)
        assert np.array_equal(np.isinf(g), inf), f"{what}: {name} infinity pattern differs"
        assert np.array_equal(g[inf], r[inf]), f"{what}: {name} infinity signs differ"
        fin = np.isfinite(r)
        err = float(np.max(np.abs(g[fin] - r[fin]))) if fin.any() else 0.0
        errs.append(err)
        assert err <= tol, f"{what}: {name} error {err} > {tol}"
    print(f"{what}: max|dO|={errs[0]:.3e} max|dLSE|={errs[1]:.3e}", flush=True)


def case(B, S_q, S_k, H, D, dtype, seed):
    q, _, _ = make_qkv(B, S_q, H, D, dtype, seed)
    _, k, v = make_qkv(B, S_k, H, D, dtype, seed + 1)
    return q, k, v


def run(q, k, v, lens, causal, window, n_splits, block_table=None, scale=None):
    import io_aware_exact_22_amd as fa

    D = q.shape[-1]
    scale = 1.0 / math.sqrt(D) if scale is None else scale
    sl = torch.tensor(lens, dtype=torch.int32).cuda()
    out, lse = fa.flash_attn_fwd_kvcache(q.cuda(), k.cuda(), v.cuda(), sl,
                                         block_table=None if block_table is None else
                                         block_table.cuda(), softmax_scale=scale, causal=causal,
                                         window_size=window, n_splits=n_splits)
    torch.cuda.synchronize()
    return out.cpu(), lse.cpu(), scale


MASKS = [(True, (-1, -1)), (False, (-1, -1)), (True, (40, -1)), (False, (16, 16)), (False, (0, 0))]


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float16])
@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("causal,window", MASKS)
@pytest.mark.parametrize("S_q", [1, 5, 130])
@pytest.mark.parametrize("n_splits", [1, 3])
def test_kvcache_parity(dtype, D, causal, window, S_q, n_splits):
    """Three sequences with ragged cache lengths -- one shorter than the query
    block (leading rows without keys under the causal mask), one mid-length,
    one full -- against a 300-row cache (ragged last tile)."""
    B, S_k, H = 3, 300, 2
    q, k, v = case(B, S_q, S_k, H, D, dtype, 100 + S_q)
    lens = [max(0, S_q - 3), 177, S_k]
    out, lse, scale = run(q, k, v, lens, causal, window, n_splits)
    ref_o, ref_l = oracle.fwd_kvcache(q, k, v, lens, scale, causal, window)
    compare(out, lse, ref_o, ref_l, dtype, f"kvcache {dtype} D{D} S_q={S_q} causal={causal} "
                                           f"{window} x{n_splits}")


@pytest.mark.parametrize("dtype,D", [(torch.bfloat16, 128), (torch.float16, 64)])
@pytest.mark.parametrize("causal,window", [(True, (-1, -1)), (False, (30, 2))])
def test_kvcache_full_cache_is_fa_fwd_bitwise(dtype, D, causal, window):
    """S_q = L = S_k: every query sits at its own index, so the result is
    fa_fwd's, bit for bit (same tiles, same arithmetic)."""
    import io_aware_exact_22_amd as fa

    B, S, H = 2, 389, 3
    q, k, v = make_qkv(B, S, H, D, dtype, 7)
    out, lse, scale = run(q, k, v, [S, S], causal, window, 1)
    ro, rl = fa.flash_attn_fwd(q.cuda(), k.cuda(), v.cuda(), softmax_scale=scale, causal=causal,
                               window_size=window)
    torch.cuda.synchronize()
    assert torch.equal(out.view(torch.int16), ro.cpu().view(torch.int16))
    assert torch.equal(lse, rl.cpu())


@pytest.mark.parametrize("S_q", [1, 4])
@pytest.mark.parametrize("n_splits", [1, 4])
@pytest.mark.parametrize("page_size", [64, 128])
def test_kvcache_paged(n_splits, page_size, S_q):
    """Page pools with pages at a seeded permutation of slots and NaN in every
    row no sequence uses: equal to the contiguous cache's result bit for bit,
    and to the oracle (one query per sequence runs the vector-ALU decoding
    kernel, four the MFMA kernel)."""
    B, S_k, H, D, dtype = 3, 640, 2, 128, torch.bfloat16
    q, k, v = case(B, S_q, S_k, H, D, dtype, 300)
    lens = [1, 333, 640]
    n_pg = S_k // page_size
    perm = torch.randperm(B * n_pg + 5, generator=torch.Generator().manual_seed(3))[:B * n_pg]
    table = perm.view(B, n_pg).to(torch.int32)
    pools = []
    for t in (k, v):
        pool = torch.full((B * n_pg + 5, page_size, H, D), float("nan"), dtype=dtype)
        for b in range(B):
            rows = t[b, :lens[b]]
            for p in range(-(-lens[b] // page_size)):
                seg = rows[p * page_size:(p + 1) * page_size]
                pool[table[b, p], :seg.shape[0]] = seg
        pools.append(pool)
    out, lse, scale = run(q, pools[0], pools[1], lens, True, (-1, -1), n_splits, block_table=table)
    kd = k.clone()
    vd = v.clone()
    for b in range(B):
        kd[b, lens[b]:] = float("nan")
        vd[b, lens[b]:] = float("nan")
    out_c, lse_c, _ = run(q, kd, vd, lens, True, (-1, -1), n_splits)
    assert torch.equal(out.view(torch.int16), out_c.view(torch.int16))
    assert torch.equal(lse, lse_c)
    ref_o, ref_l = oracle.fwd_kvcache(q, k, v, lens, scale, True)
    compare(out, lse, ref_o, ref_l, dtype, f"kvcache paged {page_size} x{n_splits}")


def test_kvcache_lengths_are_clamped():
    """A length below 0 reads as 0 (no keys) and one above the capacity as the
    capacity."""
    B, S_q, S_k, H, D, dtype = 2, 2, 200, 2, 64, torch.float16
    q, k, v = case(B, S_q, S_k, H, D, dtype, 400)
    out, lse, scale = run(q, k, v, [-7, S_k + 50], True, (-1, -1), 2)
    ref_o, ref_l = oracle.fwd_kvcache(q, k, v, [0, S_k], scale, True)
    compare(out, lse, ref_o, ref_l, dtype, "kvcache clamped lengths")


@pytest.mark.parametrize("dtype,D", [(torch.bfloat16, 128), (torch.float16, 64)])
@pytest.mark.parametrize("n_splits", [1, 3])
def test_kvcache_decode_nonfinite_outside_the_window(dtype, D, n_splits):
    """One query per sequence: NaN in cached keys and values left of a
    window and in stale rows past the length never reach O; an infinity at an
    allowed key does, as in the oracle."""
    B, S_q, S_k, H = 2, 1, 400, 2
    q, k, v = case(B, S_q, S_k, H, D, dtype, 700)
    lens = [333, 400]
    wl = 100
    for b, L in enumerate(lens):
        k[b, L - 1 - wl - 5, 0, 1] = float("nan")   # left of the window
        v[b, L - 1 - wl - 1, 1, 2] = float("nan")
        if L < S_k:
            k[b, L:, :, 3] = float("nan")           # stale rows past the length
            v[b, L:, :, 4] = float("nan")
    v[1, 399, 0, 7] = float("inf")                   # allowed: the query's own key
    out, lse, scale = run(q, k, v, lens, True, (wl, -1), n_splits)
    ref_o, ref_l = oracle.fwd_kvcache(q, k, v, lens, scale, True, (wl, -1))
    assert np.isinf(ref_o).sum() == 1 and not np.isnan(ref_o).any()
    compare(out, lse, ref_o, ref_l, dtype, f"decode nonfinite {dtype} D{D} x{n_splits}")


def test_kvcache_nonfinite_values_outside_the_mask():
    """NaN / inf in cached values next to the causal edge of a query block
    reach only the rows that allow them (as in the oracle)."""
    B, S_q, S_k, H, D, dtype = 1, 40, 256, 2, 128, torch.bfloat16
    q, k, v = case(B, S_q, S_k, H, D, dtype, 500)
    L = 230
    v[0, L - 10, 0, 4] = float("nan")   # allowed by the last 10 queries only
    v[0, L - 30, 1, 6] = float("inf")
    out, lse, scale = run(q, k, v, [L], True, (-1, -1), 1)
    ref_o, ref_l = oracle.fwd_kvcache(q, k, v, [L], scale, True)
    assert np.isnan(ref_o).any() and np.isfinite(ref_o[0, :S_q - 10, 0]).all()
    compare(out, lse, ref_o, ref_l, dtype, "kvcache nonfinite")


@pytest.mark.parametrize("ragged", [False, True])
def test_kvcache_decode_16k_every_element(ragged):
    """The decoding workload the benchmark times -- 8 sequences x 16 heads,
    one query each against a 16384-row cache, bf16 -- in the library's part
    count, every element against the oracle; with full caches and with
    seeded lengths in [1, 16384]."""
    from fa_inputs import WORKLOADS_KV

    w = WORKLOADS_KV["decode_16k"]
    q, k, v = case(w.B, w.S_q, w.S_k, w.H, w.D, w.dtype, w.seed)
    lens = [w.S_k] * w.B
    if ragged:
        g = torch.Generator().manual_seed(w.seed)
        lens = torch.randint(1, w.S_k + 1, (w.B,), generator=g).tolist()
    out, lse, scale = run(q, k, v, lens, True, (-1, -1), 0)
    ref_o, ref_l = oracle.fwd_kvcache(q, k, v, lens, scale, True)
    compare(out, lse, ref_o, ref_l, w.dtype, f"decode_16k lens={lens}")


def test_kvcache_raw_c_call_on_a_side_stream():
    import io_aware_exact_22_amd as fa

    B, S_q, S_k, H, D = 2, 3, 500, 2, 128
    q, k, v = case(B, S_q, S_k, H, D, torch.bfloat16, 600)
    qd, kd, vd = q.cuda(), k.cuda(), v.cuda()
    sl = torch.tensor([123, 500], dtype=torch.int32, device="cuda")
    out = torch.empty_like(qd)
    lse = torch.empty((B, H, S_q), dtype=torch.float32, device="cuda")
    ns = 2
    ws = torch.empty(fa.fa_fwd_kvcache_workspace_size(B, H, S_q, D, fa.FA_DTYPE_BF16, ns) // 4,
                     dtype=torch.float32, device="cuda")
    s = torch.cuda.Stream()
    torch.cuda.synchronize()
    rc = fa.fa_fwd_kvcache(qd.data_ptr(), kd.data_ptr(), vd.data_ptr(), sl.data_ptr(), None,
                           out.data_ptr(), lse.data_ptr(), B, H, S_q, S_k, D, 1 / math.sqrt(D), 1,
                           -1, -1, fa.FA_DTYPE_BF16, 0, 0, 0, ns, ws.data_ptr(),
                           ws.numel() * 4, s.cuda_stream)
    assert rc == 0
    s.synchronize()
    ref_o, ref_l = oracle.fwd_kvcache(q, k, v, [123, 500], 1 / math.sqrt(D), True)
    compare(out.cpu(), lse.cpu(), ref_o, ref_l, torch.bfloat16, "kvcache raw C side stream")


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float16])
@pytest.mark.parametrize("D", [16, 48, 80, 112])
@pytest.mark.parametrize("causal,window", [(True, (-1, -1)), (True, (40, -1)), (False, (16, 16))])
@pytest.mark.parametrize("S_q", [1, 5])
@pytest.mark.parametrize("n_splits", [1, 3])
def test_kvcache_other_head_dims(dtype, D, causal, window, S_q, n_splits):
    """Head dimensions other than 64 and 128 (the MFMA kernel of the next of
    them, its extra columns zeros; also for one query per sequence), ragged
    cache lengths, against the oracle."""
    B, S_k, H = 3, 300, 2
    q, k, v = case(B, S_q, S_k, H, D, dtype, 1200 + D + S_q)
    lens = [max(0, S_q - 3), 177, S_k]
    out, lse, scale = run(q, k, v, lens, causal, window, n_splits)
    ref_o, ref_l = oracle.fwd_kvcache(q, k, v, lens, scale, causal, window)
    compare(out, lse, ref_o, ref_l, dtype, f"kvcache {dtype} D{D} S_q={S_q} causal={causal} "
                                           f"{window} x{n_splits}")


@pytest.mark.parametrize("D", [32, 96])
@pytest.mark.parametrize("S_q", [1, 4])
def test_kvcache_other_head_dims_paged(D, S_q):
    """Paged pools (NaN in every unused row) at a padded head dimension equal
    the contiguous cache bit for bit, and the oracle."""
    B, S_k, H, dtype, page_size = 2, 256, 3, torch.bfloat16, 64
    q, k, v = case(B, S_q, S_k, H, D, dtype, 1300 + D)
    lens = [100, 256]
    n_pg = S_k // page_size
    perm = torch.randperm(B * n_pg + 3, generator=torch.Generator().manual_seed(5))[:B * n_pg]
    table = perm.view(B, n_pg).to(torch.int32)
    pools = []
    for t in (k, v):
        pool = torch.full((B * n_pg + 3, page_size, H, D), float("nan"), dtype=dtype)
        for b in range(B):
            rows = t[b, :lens[b]]
            for p in range(-(-lens[b] // page_size)):
                seg = rows[p * page_size:(p + 1) * page_size]
                pool[table[b, p], :seg.shape[0]] = seg
        pools.append(pool)
    out, lse, scale = run(q, pools[0], pools[1], lens, True, (-1, -1), 2, block_table=table)
    kd, vd = k.clone(), v.clone()
    for b in range(B):
        kd[b, lens[b]:] = float("nan")
        vd[b, lens[b]:] = float("nan")
    out_c, lse_c, _ = run(q, kd, vd, lens, True, (-1, -1), 2)
    assert torch.equal(out.view(torch.int16), out_c.view(torch.int16))
    assert torch.equal(lse, lse_c)
    ref_o, ref_l = oracle.fwd_kvcache(q, k, v, lens, scale, True)
    compare(out, lse, ref_o, ref_l, dtype, f"kvcache paged D{D} S_q={S_q}")
