"""GPU parity of fa_fwd_blocksparse (through the C ABI) against the oracle's
block-sparse forward on the same seeded inputs and masks.

Tolerances as for the dense forward (max-abs on every compared element): O
<= 1e-4 fp32, <= 4e-3 fp16, <= 2e-2 bf16; LSE <= 1e-3.  Rows with no allowed
key must be exactly O = 0, LSE = -inf.  Small cases compare every element;
the 16K and 64K workloads compare rows the oracle computes one by one.
"""
import math

import numpy as np
import pytest
import torch

import oracle
from fa_inputs import local_global_block_mask, make_qkv, random_block_mask

pytestmark = pytest.mark.gpu

TOL_O = {torch.float32: 1e-4, torch.float16: 4e-3, torch.bfloat16: 2e-2}
TOL_LSE = 1e-3


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")
    import io_aware_exact_22_amd  # noqa: F401  (fails loudly if the library is missing)


def nblocks(S, b):
    return -(-S // b)


def gpu_bs(q, k, v, mask, bm, bn, scale, causal, window, workspace=None):
    import io_aware_exact_22_amd as fa

    qd, kd, vd = (t.cuda() for t in (q, k, v))
    out, lse = fa.flash_attn_fwd_blocksparse(qd, kd, vd, mask.cuda(), bm, bn, softmax_scale=scale,
                                             causal=causal, window_size=window,
                                             workspace=workspace)
    torch.cuda.synchronize()
    return out.cpu(), lse.cpu()


def compare(out, lse, ref_o, ref_l, dtype, what):
    """ref_o [..., D] and ref_l [...] with matching leading shapes (rows as
    out [B, S, H, D] / lse [B, H, S] or already sliced)."""
    o = out.double().numpy()
    ls = lse.double().numpy()
    empty = np.isneginf(ref_l)
    assert np.all(np.isfinite(ref_o))
    assert np.array_equal(np.isneginf(ls), empty), f"{what}: rows without keys differ"
    live = ~empty
    assert np.all(np.isfinite(ls[live])), f"{what}: non-finite LSE"
    assert np.all(np.isfinite(o)), f"{what}: non-finite O"
    el = float(np.max(np.abs(ls[live] - ref_l[live]))) if live.any() else 0.0
    eo = float(np.max(np.abs(o - ref_o))) if o.size else 0.0
    print(f"{what}: max|dO|={eo:.3e} max|dLSE|={el:.3e} empty rows={int(empty.sum())}",
          flush=True)
    assert eo <= TOL_O[dtype], f"{what}: O error {eo} > {TOL_O[dtype]}"
    assert el <= TOL_LSE, f"{what}: LSE error {el} > {TOL_LSE}"


def check_full(B, S, H, D, dtype, causal, window, mask, bm, bn, seed, scale=None):
    scale = 1.0 / math.sqrt(D) if scale is None else scale
    q, k, v = make_qkv(B, S, H, D, dtype, seed)
    what = (f"B{B} S{S} H{H} D{D} {dtype} causal={causal} window={window} mask={tuple(mask.shape)}"
            f" block={bm}x{bn} seed={seed}")
    print("run", what, flush=True)
    out, lse = gpu_bs(q, k, v, mask, bm, bn, scale, causal, window)
    ref_o, ref_l = oracle.fwd_blocksparse(q, k, v, scale, mask.numpy(), bm, bn, causal, window)
    # rows with no key: O exactly 0
    empty_rows = np.isneginf(ref_l).transpose(0, 2, 1)  # [B, S, H]
    assert torch.all(out.float()[torch.from_numpy(empty_rows)] == 0)
    compare(out, lse, ref_o, ref_l, dtype, what)


# ---------------------------------------------------------------- small, every element
MASKS = [(False, (-1, -1)), (True, (-1, -1)), (False, (200, 100)), (True, (300, -1))]


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float16, torch.float32])
@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("causal,window", MASKS)
def test_blocksparse_parity(dtype, D, causal, window):
    """A random mask per (batch, head), 40% of the blocks kept, S = 777 (a
    ragged last Q tile and K/V tile), every element against the oracle."""
    B, S, H = 2, 777, 3
    mask = random_block_mask(B * H, nblocks(S, 128), nblocks(S, 64), 0.4, 100 + D)
    check_full(B, S, H, D, dtype, causal, window, mask, 128, 64, seed=31)


@pytest.mark.parametrize("bm,bn", [(128, 64), (256, 128), (128, 192), (384, 64)])
@pytest.mark.parametrize("n_mask", ["1", "H", "BH"])
def test_blocksparse_block_shapes(bm, bn, n_mask):
    """Mask blocks of several tiles each way, one mask per call, per head or
    per (batch, head)."""
    B, S, H = 2, 1000, 2
    nm = {"1": 1, "H": H, "BH": B * H}[n_mask]
    mask = random_block_mask(nm, nblocks(S, bm), nblocks(S, bn), 0.5, bm + bn + nm)
    causal = bm == 256
    check_full(B, S, H, 128, torch.bfloat16, causal, (-1, -1), mask, bm, bn, seed=bm + bn)


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float16, torch.float32])
@pytest.mark.parametrize("causal,window", MASKS)
def test_blocksparse_all_kept_is_fa_fwd_bitwise(dtype, causal, window):
    """A mask keeping every block gives fa_fwd's result: the same tiles in
    the same order (a wave that holds no allowed key of a tile adds exact
    zeros), bit for bit for fp16 and fp32.  bf16 skips the row max on the
    mask-free tiles after the first, whose range a block-sparse workgroup
    takes as a whole and a dense wave for its own 32 rows, so the two can
    round their weights against different references: equal there within
    the bf16 output tolerance (O 2e-2, LSE 1e-3)."""
    import io_aware_exact_22_amd as fa

    B, S, H, D = 1, 1100, 2, 128
    q, k, v = (t.cuda() for t in make_qkv(B, S, H, D, dtype, 41))
    mask = torch.ones((1, nblocks(S, 128), nblocks(S, 64)), dtype=torch.uint8, device="cuda")
    o1, l1 = fa.flash_attn_fwd_blocksparse(q, k, v, mask, 128, 64, causal=causal,
                                           window_size=window)
    o2, l2 = fa.flash_attn_fwd(q, k, v, causal=causal, window_size=window)
    torch.cuda.synchronize()
    if dtype != torch.bfloat16:
        assert torch.equal(o1, o2) and torch.equal(l1, l2)
        return
    assert torch.equal(torch.isneginf(l1), torch.isneginf(l2))
    live = ~torch.isneginf(l2)
    eo = float((o1.float() - o2.float()).abs().max())
    el = float((l1[live] - l2[live]).abs().max())
    print(f"bf16 all-kept vs dense: max|dO|={eo:.2e} max|dLSE|={el:.2e}", flush=True)
    assert eo <= 2e-2 and el <= 1e-3


def test_blocksparse_rows_without_keys():
    """Q blocks whose kept blocks are none, or all above the causal diagonal,
    get O = 0 and LSE = -inf exactly; an all-zero mask gives that everywhere."""
    B, S, H, D = 1, 640, 2, 64
    q, k, v = make_qkv(B, S, H, D, torch.float16, 43)
    mask = torch.ones((1, 5, 10), dtype=torch.uint8)
    mask[0, 1] = 0          # rows 128..255: nothing kept
    mask[0, 2, :6] = 0      # rows 256..383 keep only keys >= 384: causal leaves none
    out, lse = gpu_bs(q, k, v, mask, 128, 64, 0.125, True, (-1, -1))
    for r0, r1 in ((128, 256), (256, 384)):
        assert torch.all(out[:, r0:r1] == 0)
        assert torch.all(torch.isneginf(lse[:, :, r0:r1]))
    ref_o, ref_l = oracle.fwd_blocksparse(q, k, v, 0.125, mask.numpy(), 128, 64, True)
    compare(out, lse, ref_o, ref_l, torch.float16, "rows without keys")
    zero = torch.zeros_like(mask)
    out0, lse0 = gpu_bs(q, k, v, zero, 128, 64, 0.125, False, (-1, -1))
    assert torch.all(out0 == 0) and torch.all(torch.isneginf(lse0))


def test_blocksparse_dropped_blocks_are_never_read():
    """NaN in the keys and values of blocks no row keeps changes nothing: the
    result equals, bit for bit, the run with those entries zeroed."""
    B, S, H, D = 1, 512, 2, 128
    q, k, v = make_qkv(B, S, H, D, torch.bfloat16, 44)
    mask = torch.ones((1, 4, 8), dtype=torch.uint8)
    mask[0, :, 3] = 0  # keys 192..255
    k_bad, v_bad, k0, v0 = k.clone(), v.clone(), k.clone(), v.clone()
    k_bad[:, 192:256] = float("nan")
    v_bad[:, 192:256] = float("nan")
    k0[:, 192:256] = 0
    v0[:, 192:256] = 0
    o_bad, l_bad = gpu_bs(q, k_bad, v_bad, mask, 128, 64, 0.1, False, (-1, -1))
    o_ok, l_ok = gpu_bs(q, k0, v0, mask, 128, 64, 0.1, False, (-1, -1))
    assert torch.isfinite(o_bad.float()).all() and torch.isfinite(l_bad).all()
    assert torch.equal(o_bad, o_ok) and torch.equal(l_bad, l_ok)


# ---------------------------------------------------------------- full size, sampled rows
def sampled(q, k, v, mask, bm, bn, scale, causal, out, lse, heads, rows, dtype, what):
    for h in heads:
        for r0 in rows:
            r1 = min(q.shape[1], r0 + 1)
            ref_o, ref_l = oracle.fwd_rows_blocksparse(q, k, v, scale, mask.numpy(), bm, bn,
                                                       causal, (-1, -1), 0, h, r0, r1)
            compare(out[0, r0:r1, h], lse[0, h, r0:r1], ref_o, ref_l, dtype,
                    f"{what} head {h} row {r0}")


def test_blocksparse_causal_16k_local_global_sampled():
    """The 16K causal workload (1 x 16 heads x 16384 x 128, bf16) under a
    long-context pattern: each 128-row block keeps the 2048 keys before it and
    the first 64-key block; sampled rows of several heads."""
    B, S, H, D = 1, 16384, 16, 128
    q, k, v = make_qkv(B, S, H, D, torch.bfloat16, 5)
    mask = local_global_block_mask(nblocks(S, 128), nblocks(S, 64), 128, 64, 2048, 1)
    scale = 1.0 / math.sqrt(D)
    print("run causal 16384 local 2048 + global 64 keys", flush=True)
    out, lse = gpu_bs(q, k, v, mask, 128, 64, scale, True, (-1, -1))
    assert torch.isfinite(out.float()).all() and torch.isfinite(lse).all()
    sampled(q, k, v, mask, 128, 64, scale, True, out, lse, [0, 7, 15],
            [0, 1, 127, 128, 2047, 2048, 2049, 8191, 12345, 16383], torch.bfloat16, "16k local")


def test_blocksparse_64k_context_sampled():
    """A 65536-token sequence (2 heads, D 128, bf16, causal) with per-head
    random masks on 256 x 128 blocks plus a kept diagonal: the kernel walks
    lists of up to 512 kept tiles per Q tile; sampled rows."""
    B, S, H, D, bm, bn = 1, 65536, 2, 128, 256, 128
    q, k, v = make_qkv(B, S, H, D, torch.bfloat16, 64)
    mask = random_block_mask(H, nblocks(S, bm), nblocks(S, bn), 0.05, 65)
    for r in range(nblocks(S, bm)):
        mask[:, r, 2 * r: 2 * r + 2] = 1
    scale = 1.0 / math.sqrt(D)
    print("run causal 65536, 5% random blocks + diagonal", flush=True)
    out, lse = gpu_bs(q, k, v, mask, bm, bn, scale, True, (-1, -1))
    assert torch.isfinite(out.float()).all() and torch.isfinite(lse).all()
    sampled(q, k, v, mask, bm, bn, scale, True, out, lse, [0, 1],
            [0, 255, 256, 30000, 65535], torch.bfloat16, "64k random")


# ---------------------------------------------------------------- workspace, C ABI
def test_blocksparse_workspace_guard_bands_and_reuse():
    """The call writes only its workspace, out and lse; a workspace reused
    with another mask gives that mask's result; repeated calls are bitwise
    identical."""
    import io_aware_exact_22_amd as fa

    B, S, H, D = 2, 900, 3, 64
    q, k, v = (t.cuda() for t in make_qkv(B, S, H, D, torch.bfloat16, 45))
    need = fa.fa_fwd_blocksparse_workspace_size(B, H, S, D, fa.FA_DTYPE_BF16, B * H)
    pad = 4096
    buf = torch.full(((need + 2 * pad) // 4,), 12345, dtype=torch.int32, device="cuda")
    ws = buf[pad // 4: (pad + need) // 4]
    m1 = random_block_mask(B * H, 8, 15, 0.3, 46)
    m2 = random_block_mask(B * H, 8, 15, 0.7, 47)
    o1, l1 = fa.flash_attn_fwd_blocksparse(q, k, v, m1.cuda(), 128, 64, causal=True, workspace=ws)
    o1 = o1.clone()
    o2, l2 = fa.flash_attn_fwd_blocksparse(q, k, v, m2.cuda(), 128, 64, causal=True, workspace=ws)
    o3, l3 = fa.flash_attn_fwd_blocksparse(q, k, v, m2.cuda(), 128, 64, causal=True, workspace=ws)
    torch.cuda.synchronize()
    assert torch.equal(o2, o3) and torch.equal(l2, l3)
    assert bool((buf[: pad // 4] == 12345).all()) and bool((buf[(pad + need) // 4:] == 12345).all())
    qc, kc, vc = (t.cpu() for t in (q, k, v))
    r1 = oracle.fwd_blocksparse(qc, kc, vc, 0.125, m1.numpy(), 128, 64, True)
    r2 = oracle.fwd_blocksparse(qc, kc, vc, 0.125, m2.numpy(), 128, 64, True)
    compare(o1.cpu(), l1.cpu(), *r1, torch.bfloat16, "first mask")
    compare(o2.cpu(), l2.cpu(), *r2, torch.bfloat16, "second mask")


def test_blocksparse_raw_c_abi_call():
    """fa_fwd_blocksparse called with raw device pointers on a torch stream."""
    import io_aware_exact_22_amd as fa

    B, S, H, D = 1, 300, 2, 128
    q, k, v = make_qkv(B, S, H, D, torch.float16, 48)
    mask = random_block_mask(1, 3, 5, 0.6, 49)
    qd, kd, vd, md = (t.cuda() for t in (q, k, v, mask))
    out = torch.empty_like(qd)
    lse = torch.empty((B, H, S), dtype=torch.float32, device="cuda")
    need = fa.fa_fwd_blocksparse_workspace_size(B, H, S, D, fa.FA_DTYPE_FP16, 1)
    ws = torch.empty(need // 4, dtype=torch.int32, device="cuda")
    st = torch.cuda.Stream()
    rc = fa.fa_fwd_blocksparse(qd.data_ptr(), kd.data_ptr(), vd.data_ptr(), out.data_ptr(),
                               lse.data_ptr(), B, H, S, D, 0.09, 0, -1, -1, fa.FA_DTYPE_FP16,
                               md.data_ptr(), 1, 128, 64, ws.data_ptr(), need, st.cuda_stream)
    assert rc == 0
    st.synchronize()
    ref = oracle.fwd_blocksparse(q, k, v, 0.09, mask.numpy(), 128, 64)
    compare(out.cpu(), lse.cpu(), *ref, torch.float16, "raw C ABI")
