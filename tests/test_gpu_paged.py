"""GPU parity of fa_fwd_paged (through the C ABI): keys and values in page
pools read through a block table.

The paged result must equal, bit for bit, fa_fwd (or fa_fwd_splitkv) on the
contiguous tensors the pages were cut from -- the same tiles in the same order
-- and match the oracle's paged forward within the dense tolerances (O <= 1e-4
fp32, <= 4e-3 fp16, <= 2e-2 bf16; LSE <= 1e-3).  Pool rows past S, unused
pages and unused table entries hold NaN or garbage, so any read of them shows.
"""
import math

import numpy as np
import pytest
import torch

import oracle
from fa_inputs import make_qkv

pytestmark = pytest.mark.gpu

TOL_O = {torch.float32: 1e-4, torch.float16: 4e-3, torch.bfloat16: 2e-2}
TOL_LSE = 1e-3


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")
    import io_aware_exact_22_amd  # noqa: F401  (fails loudly if the library is missing)


def paginate(x, page_size, num_pages, seed, extra_cols=2):
    """Pages of x [B, S, H, D] placed at a seeded random permutation of the
    pool's slots.  Rows past S in the last page and every unused page hold NaN;
    table entries past the used ones hold -1.  Returns (pool, table [B, n +
    extra_cols] int32, both on x's device)."""
    B, S, H, D = x.shape
    n = -(-S // page_size)
    assert num_pages >= B * n
    g = torch.Generator(device="cpu")
    g.manual_seed(seed)
    slots = torch.randperm(num_pages, generator=g)[: B * n].view(B, n)
    padded = torch.full((B, n * page_size, H, D), float("nan"), dtype=x.dtype, device=x.device)
    padded[:, :S] = x
    pool = torch.full((num_pages, page_size, H, D), float("nan"), dtype=x.dtype, device=x.device)
    pool[slots.reshape(-1).to(x.device)] = padded.view(B * n, page_size, H, D)
    table = torch.full((B, n + extra_cols), -1, dtype=torch.int32)
    table[:, :n] = slots.to(torch.int32)
    return pool.contiguous(), table.to(x.device).contiguous()


def compare(out, lse, ref_o, ref_l, dtype, what):
    o = out.double().cpu().numpy()
    ls = lse.double().cpu().numpy()
    assert np.all(np.isfinite(o)) and np.all(np.isfinite(ls)), f"{what}: non-finite output"
    eo = float(np.max(np.abs(o - ref_o)))
    el = float(np.max(np.abs(ls - ref_l)))
    print(f"{what}: max|dO|={eo:.3e} max|dLSE|={el:.3e}", flush=True)
    assert eo <= TOL_O[dtype] and el <= TOL_LSE, f"{what}: O {eo}, LSE {el}"


MASKS = [(False, (-1, -1)), (True, (-1, -1)), (False, (200, 100)), (True, (300, -1))]


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float16, torch.float32])
@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("page_size", [64, 192])
@pytest.mark.parametrize("causal,window", MASKS)
def test_paged_equals_contiguous_bitwise_and_oracle(dtype, D, page_size, causal, window):
    """Scattered pages (ragged last page, NaN in unused rows and pages) give
    fa_fwd's result on the contiguous tensors bit for bit, and the oracle's
    within tolerance."""
    import io_aware_exact_22_amd as fa

    B, S, H = 2, 777, 3
    q, k, v = make_qkv(B, S, H, D, dtype, 90 + D + page_size)
    what = f"paged {dtype} D{D} page {page_size} causal={causal} window={window}"
    print("run", what, flush=True)
    qd, kd, vd = (t.cuda() for t in (q, k, v))
    n = -(-S // page_size)
    kp, table = paginate(kd, page_size, B * n + 3, 7)
    vp, _ = paginate(vd, page_size, B * n + 3, 7)
    o1, l1 = fa.flash_attn_fwd_paged(qd, kp, vp, table, causal=causal, window_size=window)
    o2, l2 = fa.flash_attn_fwd(qd, kd, vd, causal=causal, window_size=window)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2), what
    ref = oracle.fwd_paged(q, kp.cpu(), vp.cpu(), table.cpu().numpy(), 1 / math.sqrt(D), causal,
                           window)
    compare(o1, l1, *ref, dtype, what)


@pytest.mark.parametrize("page_size", [64, 128, 256, 320])
@pytest.mark.parametrize("n_splits", [2, 3])
def test_paged_split_equals_contiguous_split_bitwise(page_size, n_splits):
    """The split-KV path over pages equals fa_fwd_splitkv on the contiguous
    tensors, bit for bit."""
    import io_aware_exact_22_amd as fa

    B, S, H, D = 2, 1000, 2, 128
    qd, kd, vd = (t.cuda() for t in make_qkv(B, S, H, D, torch.bfloat16, page_size + n_splits))
    n = -(-S // page_size)
    kp, table = paginate(kd, page_size, B * n + 1, page_size)
    vp, _ = paginate(vd, page_size, B * n + 1, page_size)
    o1, l1 = fa.flash_attn_fwd_paged(qd, kp, vp, table, causal=True, n_splits=n_splits)
    o2, l2 = fa.flash_attn_fwd_splitkv(qd, kd, vd, causal=True, n_splits=n_splits)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)


def test_paged_shared_prefix_pages():
    """Two sequences that share their first two pages (a common prompt) and
    differ after them: rows of the prefix agree between the sequences, causal,
    and each sequence matches fa_fwd on its own contiguous keys."""
    import io_aware_exact_22_amd as fa

    S, H, D, ps = 384, 2, 128, 128
    q1, k1, v1 = (t.cuda() for t in make_qkv(1, S, H, D, torch.float16, 91))
    _, k2, v2 = (t.cuda() for t in make_qkv(1, S, H, D, torch.float16, 92))
    k2[:, :256], v2[:, :256] = k1[:, :256], v1[:, :256]
    pool_k = torch.cat([k1[0].view(3, ps, H, D), k2[0, 256:].view(1, ps, H, D)]).contiguous()
    pool_v = torch.cat([v1[0].view(3, ps, H, D), v2[0, 256:].view(1, ps, H, D)]).contiguous()
    table = torch.tensor([[0, 1, 2], [0, 1, 3]], dtype=torch.int32, device="cuda")
    q = torch.cat([q1, q1]).contiguous()
    o, l = fa.flash_attn_fwd_paged(q, pool_k, pool_v, table, causal=True)
    oa, la = fa.flash_attn_fwd(q1, k1, v1, causal=True)
    ob, lb = fa.flash_attn_fwd(q1, k2, v2, causal=True)
    torch.cuda.synchronize()
    assert torch.equal(o[0], oa[0]) and torch.equal(o[1], ob[0])
    assert torch.equal(l[0], la[0]) and torch.equal(l[1], lb[0])
    assert torch.equal(o[0, :256], o[1, :256])


def test_paged_pages_outside_the_pool_read_as_zeros():
    """A table entry outside [0, num_pages) is not an error the call can see;
    the kernel's bounds make its keys and values read as zeros: the result is
    fa_fwd's with those rows zeroed, bit for bit (bf16 and fp32 kernels)."""
    import io_aware_exact_22_amd as fa

    for dtype in (torch.bfloat16, torch.float32):
        B, S, H, D, ps = 1, 512, 2, 64, 128
        qd, kd, vd = (t.cuda() for t in make_qkv(B, S, H, D, dtype, 93))
        kp, table = paginate(kd, ps, 4, 94)
        vp, _ = paginate(vd, ps, 4, 94)
        table[0, 2] = 4        # one past the pool
        table[0, 3] = -3       # negative
        k0, v0 = kd.clone(), vd.clone()
        k0[:, 256:] = 0
        v0[:, 256:] = 0
        o1, l1 = fa.flash_attn_fwd_paged(qd, kp, vp, table)
        o2, l2 = fa.flash_attn_fwd(qd, k0, v0)
        torch.cuda.synchronize()
        assert torch.equal(o1, o2) and torch.equal(l1, l2), dtype


def test_paged_causal_16k_bitwise_and_sampled():
    """The 16K causal workload (1 x 16 heads x 16384 x 128, bf16) over 256-row
    pages scattered in a pool with spare pages: bit for bit fa_fwd's result,
    and sampled rows against the oracle."""
    import io_aware_exact_22_amd as fa

    B, S, H, D, ps = 1, 16384, 16, 128, 256
    q, k, v = make_qkv(B, S, H, D, torch.bfloat16, 5)
    qd, kd, vd = (t.cuda() for t in (q, k, v))
    kp, table = paginate(kd, ps, S // ps + 16, 95)
    vp, _ = paginate(vd, ps, S // ps + 16, 95)
    print("run paged causal 16384", flush=True)
    o1, l1 = fa.flash_attn_fwd_paged(qd, kp, vp, table, causal=True)
    o2, l2 = fa.flash_attn_fwd(qd, kd, vd, causal=True)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)
    o1c, l1c = o1.cpu(), l1.cpu()
    for h in (0, 9):
        for r in (0, 255, 256, 8191, 16383):
            ro, rl = oracle.fwd_rows(q, k, v, 1 / math.sqrt(D), True, (-1, -1), 0, h, r, r + 1)
            compare(o1c[0, r:r + 1, h], l1c[0, h, r:r + 1], ro, rl, torch.bfloat16,
                    f"16k paged head {h} row {r}")


def test_paged_raw_c_abi_call():
    """fa_fwd_paged with raw device pointers on a side stream, against the oracle."""
    import io_aware_exact_22_amd as fa

    B, S, H, D, ps = 2, 300, 2, 128, 64
    q, k, v = make_qkv(B, S, H, D, torch.float16, 96)
    qd = q.cuda()
    kp, table = paginate(k.cuda(), ps, 12, 97)
    vp, _ = paginate(v.cuda(), ps, 12, 97)
    out = torch.empty_like(qd)
    lse = torch.empty((B, H, S), dtype=torch.float32, device="cuda")
    st = torch.cuda.Stream()
    rc = fa.fa_fwd_paged(qd.data_ptr(), kp.data_ptr(), vp.data_ptr(), table.data_ptr(),
                         out.data_ptr(), lse.data_ptr(), B, H, S, D, 0.1, 1, -1, -1,
                         fa.FA_DTYPE_FP16, 12, ps, table.shape[1], 1, None, 0, st.cuda_stream)
    assert rc == 0
    st.synchronize()
    ref = oracle.fwd_paged(q, kp.cpu(), vp.cpu(), table.cpu().numpy(), 0.1, True)
    compare(out, lse, *ref, torch.float16, "raw C ABI")


@pytest.mark.parametrize("dtype,H,D,window", [(torch.bfloat16, 20, 128, (-1, -1)),
                                              (torch.float16, 32, 64, (-1, -1)),
                                              (torch.bfloat16, 32, 64, (-1, -1)),
                                              (torch.float16, 6, 96, (-1, -1)),
                                              (torch.bfloat16, 20, 128, (1024, -1))])
def test_paged_dynamic_tail_equals_contiguous(dtype, H, D, window):
    """Causal paged launches with more workgroups than the device holds take
    fa_fwd's dynamic order (workgroups take the light tiles' list positions
    from a counter in the LSE word of row 0 of head 0, zeroed first): on two
    calls in a row into buffers whose LSE starts as NaN, the result equals
    fa_fwd's on the contiguous tensors bit for bit, and the oracle's within
    tolerance (D = 96 runs the D = 128 kernel with zero columns)."""
    import io_aware_exact_22_amd as fa

    B = 1
    S = 4096 if H > 6 else 12000
    dcode = fa.FA_DTYPE_BF16 if dtype == torch.bfloat16 else fa.FA_DTYPE_FP16
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    first = fa.fa_fwd_launch_order(B, H, S, D, dcode, 1, window[0], window[1], cus, 0)[2]
    assert first >= 0, "the case must take the dynamic order"
    q, k, v = make_qkv(B, S, H, D, dtype, 300 + H + D)
    what = f"paged dynamic tail: B{B} S{S} H{H} D{D} {dtype} window={window}"
    print("run", what, flush=True)
    qd, kd, vd = (t.cuda() for t in (q, k, v))
    page_size = 256
    n = -(-S // page_size)
    kp, table = paginate(kd, page_size, B * n + 3, 11)
    vp, _ = paginate(vd, page_size, B * n + 3, 11)
    out = torch.empty_like(qd)
    lse = torch.full((B, H, S), float("nan"), dtype=torch.float32, device="cuda")
    res = []
    for _ in range(2):
        fa.flash_attn_fwd_paged(qd, kp, vp, table, causal=True, window_size=window, out=out,
                                lse=lse)
        torch.cuda.synchronize()
        res.append((out.clone(), lse.clone()))
    o2, l2 = fa.flash_attn_fwd(qd, kd, vd, causal=True, window_size=window)
    torch.cuda.synchronize()
    for o1, l1 in res:
        assert torch.equal(o1, o2) and torch.equal(l1, l2), what
    if S <= 4096:
        ref_o, ref_l = oracle.fwd(q, k, v, 1 / math.sqrt(D), True, window)
        compare(res[0][0], res[0][1], ref_o, ref_l, dtype, what)
