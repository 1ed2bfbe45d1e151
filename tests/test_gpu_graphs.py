"""fa_fwd and fa_bwd captured in a HIP graph (torch.cuda.CUDAGraph) and
replayed: causal launches larger than the device take the dynamic order,
whose counters are zeroed by kernels (a one-thread kernel before the
forward, the row-dot pass in the backward), so every replay starts them at
zero.  Each replay, with eager library calls and synchronisations between
the replays, must equal the eager result bit for bit (a tile's result does
not depend on the workgroup that computes it)."""
import pytest
import torch

from fa_inputs import make_qkv

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")
    import io_aware_exact_22_amd  # noqa: F401  (fails loudly if the library is missing)


def test_forward_graph_replays_equal_eager():
    import io_aware_exact_22_amd as fa

    B, S, H, D = 1, 4096, 20, 128  # 640 workgroups: more than the device holds
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    assert fa.fa_fwd_launch_order(B, H, S, D, fa.FA_DTYPE_BF16, 1, -1, -1, cus, 0)[2] >= 0
    q, k, v = (t.cuda() for t in make_qkv(B, S, H, D, torch.bfloat16, 31))
    ref_o, ref_l = fa.flash_attn_fwd(q, k, v, causal=True)
    torch.cuda.synchronize()
    out = torch.empty_like(q)
    lse = torch.full((B, H, S), float("nan"), dtype=torch.float32, device="cuda")
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):  # warm-up on the capture stream
        fa.flash_attn_fwd(q, k, v, causal=True, out=out, lse=lse, stream=s)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        fa.flash_attn_fwd(q, k, v, causal=True, out=out, lse=lse, stream=s)
    for rep in range(4):
        out.fill_(float("nan"))
        lse.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        print(f"replay {rep}", flush=True)
        assert torch.equal(out, ref_o) and torch.equal(lse, ref_l), f"replay {rep}"
        # eager library work between the replays
        o2, l2 = fa.flash_attn_fwd(q, k, v, causal=True)
        torch.cuda.synchronize()
        assert torch.equal(o2, ref_o) and torch.equal(l2, ref_l)


def test_backward_graph_replays_equal_eager():
    import io_aware_exact_22_amd as fa

    B, S, H, D = 1, 4096, 20, 128
    q, k, v = (t.cuda() for t in make_qkv(B, S, H, D, torch.bfloat16, 32))
    do = make_qkv(B, S, H, D, torch.bfloat16, 33)[0].cuda()
    out, lse = fa.flash_attn_fwd(q, k, v, causal=True)
    ref = fa.flash_attn_bwd(do, q, k, v, out, lse, causal=True)
    torch.cuda.synchronize()
    need = fa.fa_bwd_workspace_size(B, H, S, D, fa.FA_DTYPE_BF16)
    ws = torch.empty((need + 3) // 4, dtype=torch.float32, device="cuda")
    dq, dk, dv = (torch.empty_like(q) for _ in range(3))
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        fa.flash_attn_bwd(do, q, k, v, out, lse, causal=True, workspace=ws, dq=dq, dk=dk, dv=dv,
                          stream=s)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        fa.flash_attn_bwd(do, q, k, v, out, lse, causal=True, workspace=ws, dq=dq, dk=dk, dv=dv,
                          stream=s)
    for rep in range(4):
        for t in (dq, dk, dv):
            t.fill_(float("nan"))
        ws.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        print(f"replay {rep}", flush=True)
        for name, a, b in zip(("dq", "dk", "dv"), (dq, dk, dv), ref):
            assert torch.equal(a, b), f"replay {rep}: {name}"
        fa.flash_attn_bwd(do, q, k, v, out, lse, causal=True)
        torch.cuda.synchronize()
