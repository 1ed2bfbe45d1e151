"""Host-side tests of libfa_mi355x (no GPU needed): the library loads, exports
every function include/fa_mi355x.h declares, validates arguments as the header
states, and its tile schedule covers exactly the allowed (query, key) pairs."""
import ctypes
import os
import re
import subprocess
import sys

import pytest

import io_aware_exact_22_amd as fa
from io_aware_exact_22_amd import fa as fam

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "fa_mi355x.h")


def declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\s*\*?\s*(fa_\w+)\s*\(", src, flags=re.M)))


def test_library_exports_every_declared_symbol():
    names = declared_functions()
    assert set(names) == {"fa_fwd", "fa_fwd_check_args", "fa_status_string", "fa_fwd_tile_schedule",
                          "fa_fwd_workgroup_tile", "fa_fwd_launch_order",
                          "fa_fwd_splitkv_workgroup_tile",
                          "fa_fwd_splitkv",
                          "fa_fwd_splitkv_workspace_size", "fa_fwd_splitkv_auto_splits",
                          "fa_bwd", "fa_bwd_workspace_size", "fa_fwd_blocksparse",
                          "fa_fwd_blocksparse_workspace_size", "fa_fwd_paged",
                          "fa_fwd_kvcache", "fa_fwd_kvcache_workspace_size",
                          "fa_fwd_kvcache_auto_splits", "fa_fwd_splitkv_noalloc"}
    lib = ctypes.CDLL(fa.library_path())
    for n in names:
        assert hasattr(lib, n), n
    out = subprocess.run(["nm", "-D", "--defined-only", fa.library_path()], capture_output=True,
                         text=True, check=True).stdout
    exported = {ln.split()[-1] for ln in out.splitlines() if " T " in ln}
    assert set(names) <= exported
    # nothing else of ours leaks out (hidden visibility)
    assert not [s for s in exported if s.startswith("_ZN2fa")]


def test_status_strings():
    for st in range(0, -15, -1):
        s = fa.fa_status_string(st)
        assert s and s != "unknown status"
    assert fa.fa_status_string(-99) == "unknown status"


# fake, aligned, disjoint device addresses: fa_fwd_check_args never dereferences
Q, K, V, OUT, LSE = 1 << 32, 2 << 32, 3 << 32, 4 << 32, 5 << 32
GOOD = dict(q=Q, k=K, v=V, out=OUT, lse=LSE, B=2, H=4, S=300, D=128, scale=0.125, causal=1,
            window_left=-1, window_right=-1, dtype=fa.FA_DTYPE_BF16)


def check(**kw):
    a = dict(GOOD, **kw)
    return fa.fa_fwd_check_args(a["q"], a["k"], a["v"], a["out"], a["lse"], a["B"], a["H"], a["S"],
                                a["D"], a["scale"], a["causal"], a["window_left"],
                                a["window_right"], a["dtype"])


@pytest.mark.parametrize("kw,status", [
    ({}, 0),
    ({"q": 0}, -1), ({"k": 0}, -1), ({"v": 0}, -1), ({"out": 0}, -1), ({"lse": 0}, -1),
    ({"B": 0}, -2), ({"H": 0}, -2), ({"S": 0}, -2), ({"S": -5}, -2),
    ({"S": 1 << 40}, -2), ({"B": 1 << 40, "H": 1 << 30}, -2),
    ({"H": 131072, "D": 128, "S": 1}, -2), ({"H": 131071, "D": 128, "S": 1}, 0),
    # bf16 / fp16: any multiple of 16 from 16 to 256; fp32: 64 or 128
    ({"D": 96}, 0), ({"D": 16}, 0), ({"D": 48}, 0), ({"D": 112}, 0), ({"D": 144}, 0),
    ({"D": 256}, 0), ({"D": 0}, -3), ({"D": 8}, -3), ({"D": 24}, -3), ({"D": 100}, -3),
    ({"D": 264}, -3), ({"D": 272}, -3), ({"D": 512}, -3),
    ({"D": 96, "dtype": fa.FA_DTYPE_FP32}, 0), ({"D": 144, "dtype": fa.FA_DTYPE_FP32}, -3),
    ({"D": 256, "dtype": fa.FA_DTYPE_FP32}, -3),
    ({"D": 64, "dtype": fa.FA_DTYPE_FP32}, 0), ({"D": 96, "dtype": fa.FA_DTYPE_FP16}, 0),
    ({"window_left": -2}, -4), ({"window_right": -7}, -4), ({"causal": 2}, -4),
    ({"dtype": 3}, -5), ({"dtype": -1}, -5),
    ({"scale": float("nan")}, -6), ({"scale": float("inf")}, -6), ({"scale": -0.5}, -6),
    ({"scale": 0.0}, 0), ({"window_left": 0, "window_right": 0}, 0), ({"window_left": 10**9}, 0),
    ({"q": Q + 8}, -7), ({"out": OUT + 2}, -7), ({"lse": LSE + 2}, -7), ({"lse": LSE + 4}, 0),
    ({"out": Q}, -8), ({"out": K + 64}, -8), ({"lse": V + 1024}, -8),
    ({"lse": OUT + 2 * 300 * 4 * 128 * 2 - 16}, -8), ({"lse": OUT + 2 * 300 * 4 * 128 * 2}, 0),
    ({"q": K}, 0),  # inputs may alias each other (read only)
])
def test_check_args(kw, status):
    assert check(**kw) == status


def test_fa_fwd_rejects_before_any_hip_call():
    # invalid arguments return the status without touching the GPU (none here)
    rc = fa.fa_fwd(Q, K, V, OUT, LSE, 1, 1, 128, 100, 0.1, 0, -1, -1, fa.FA_DTYPE_BF16, None)
    assert rc == -3
    rc = fa.fa_fwd(0, K, V, OUT, LSE, 1, 1, 128, 64, 0.1, 0, -1, -1, fa.FA_DTYPE_BF16, None)
    assert rc == -1


@pytest.mark.parametrize("B,H,S,D,dtype,ns", [(2, 16, 2048, 64, fa.FA_DTYPE_BF16, 3),
                                                (1, 2, 16384, 128, fa.FA_DTYPE_BF16, 4),
                                                (3, 5, 389, 128, fa.FA_DTYPE_FP16, 16),
                                                (2, 3, 300, 96, fa.FA_DTYPE_BF16, 5),
                                                (1, 1, 77, 16, fa.FA_DTYPE_FP16, 2),
                                                (1, 2, 100, 256, fa.FA_DTYPE_BF16, 3)])
def test_splitkv_workspace_size(B, H, S, D, dtype, ns):
    """fp32 partial O and LSE of every part: ns * B * H * S * (D + 1) * 4 bytes;
    nothing for one part or fp32 inputs."""
    assert fa.fa_fwd_splitkv_workspace_size(B, H, S, D, dtype, ns) == ns * B * H * S * (D + 1) * 4
    assert fa.fa_fwd_splitkv_workspace_size(B, H, S, D, dtype, 1) == 0
    if D in (64, 128):  # fp32 takes these two only
        assert fa.fa_fwd_splitkv_workspace_size(B, H, S, D, fa.FA_DTYPE_FP32, ns) == 0
    for bad in (0, -1, fa.FA_MAX_SPLITS + 1):
        with pytest.raises(fa.FaError) as e:
            fa.fa_fwd_splitkv_workspace_size(B, H, S, D, dtype, bad)
        assert e.value.status == -11
    with pytest.raises(fa.FaError) as e:
        fa.fa_fwd_splitkv_workspace_size(B, H, S, 100, dtype, ns)
    assert e.value.status == -3


WS = 6 << 32  # a fake, aligned workspace address disjoint from the tensors above


@pytest.mark.parametrize("kw,status", [
    ({"ns": 2, "ws": 0}, -10), ({"ns": 2, "wsb": 100}, -10), ({"ns": 2, "ws": WS + 8}, -10),
    ({"ns": 2, "ws": Q}, -10), ({"ns": 2, "ws": LSE - 64}, -10),
    ({"ns": 0}, -11), ({"ns": 17}, -11), ({"ns": -3}, -11),
    ({"ns": 2, "D": 72}, -3), ({"ns": 2, "q": 0}, -1), ({"ns": 2, "out": Q}, -8),
    ({"ns": 2, "dtype": 7}, -5),
])
def test_splitkv_rejects_before_any_hip_call(kw, status):
    """Invalid arguments return their status without touching the GPU."""
    a = dict(GOOD, ns=2, ws=WS, wsb=1 << 40)
    a.update(kw)
    rc = fa.fa_fwd_splitkv(a["q"], a["k"], a["v"], a["out"], a["lse"], a["B"], a["H"], a["S"],
                           a["D"], a["scale"], a["causal"], a["window_left"], a["window_right"],
                           a["dtype"], a["ns"], a["ws"] or None, a["wsb"], None)
    assert rc == status


def test_bwd_workspace_size():
    assert fa.fa_bwd_workspace_size(2, 16, 2048, 64, fa.FA_DTYPE_BF16) == 2 * 16 * 2048 * 4 + 64
    with pytest.raises(fa.FaError) as e:
        fa.fa_bwd_workspace_size(2, 16, 2048, 64, fa.FA_DTYPE_FP32)
    assert e.value.status == -5
    # bf16 / fp16: any multiple of 16 up to 128
    assert fa.fa_bwd_workspace_size(2, 16, 2048, 80, fa.FA_DTYPE_BF16) == 2 * 16 * 2048 * 4 + 64
    for bad in (72, 144, 256):
        with pytest.raises(fa.FaError) as e:
            fa.fa_bwd_workspace_size(2, 16, 2048, bad, fa.FA_DTYPE_BF16)
        assert e.value.status == -3


DO, DQ, DK, DV = 7 << 32, 8 << 32, 9 << 32, 10 << 32


@pytest.mark.parametrize("kw,status", [
    ({"dq": 0}, -1), ({"dout": 0}, -1), ({"dtype": fa.FA_DTYPE_FP32}, -5), ({"D": 100}, -3),
    ({"D": 144}, -3), ({"D": 256}, -3),
    ({"dq": Q}, -8), ({"dk": DV}, -8), ({"dv": LSE}, -8), ({"dq": DQ + 8}, -7), ({"lse": LSE + 2}, -7),
    ({"ws": 0}, -10), ({"wsb": 100}, -10), ({"ws": DQ}, -10), ({"ws": WS + 4}, -10),
    ({"scale": -1.0}, -6), ({"window_left": -3}, -4),
])
def test_bwd_rejects_before_any_hip_call(kw, status):
    a = dict(GOOD, dout=DO, dq=DQ, dk=DK, dv=DV, ws=WS, wsb=1 << 30)
    a.update(kw)
    rc = fa.fa_bwd(a["q"], a["k"], a["v"], a["out"], a["lse"], a["dout"], a["dq"], a["dk"], a["dv"],
                   a["B"], a["H"], a["S"], a["D"], a["scale"], a["causal"], a["window_left"],
                   a["window_right"], a["dtype"], a["ws"] or None, a["wsb"], None)
    assert rc == status


@pytest.mark.parametrize("B,H,S,nm,dtype", [(1, 16, 16384, 1, fa.FA_DTYPE_BF16),
                                             (2, 4, 300, 8, fa.FA_DTYPE_FP16),
                                             (2, 4, 300, 4, fa.FA_DTYPE_BF16),
                                             (2, 4, 300, 1, fa.FA_DTYPE_FP32)])
def test_blocksparse_workspace_size(B, H, S, nm, dtype):
    """One list row per (mask head, 128-row Q tile): a 4-int header and the
    K/V tile count (64-key tiles, 32-key above D = 128) rounded up to 4 ints;
    nothing for fp32."""
    got = fa.fa_fwd_blocksparse_workspace_size(B, H, S, 128, dtype, nm)
    n_qt, n_kt = -(-S // 128), -(-S // 64)
    want = 0 if dtype == fa.FA_DTYPE_FP32 else nm * n_qt * (4 + -(-n_kt // 4) * 4) * 4
    assert got == want
    if dtype != fa.FA_DTYPE_FP32:
        n_kt32 = -(-S // 32)
        assert fa.fa_fwd_blocksparse_workspace_size(B, H, S, 256, dtype, nm) == \
            nm * n_qt * (4 + -(-n_kt32 // 4) * 4) * 4
        assert fa.fa_fwd_blocksparse_workspace_size(B, H, S, 160, dtype, nm) == \
            nm * n_qt * (4 + -(-n_kt32 // 4) * 4) * 4
    with pytest.raises(fa.FaError) as e:
        fa.fa_fwd_blocksparse_workspace_size(B, H, S, 128, dtype, 3)
    assert e.value.status == -12


MASK = 11 << 32  # a fake block-mask address disjoint from everything above


@pytest.mark.parametrize("kw,status", [
    ({"mask": 0}, -1), ({"bm": 64}, -12), ({"bm": 192}, -12), ({"bm": 0}, -12), ({"bn": 32}, -12),
    ({"bn": 96}, -12), ({"nm": 3}, -12), ({"nm": 0}, -12), ({"ws": 0}, -10), ({"wsb": 16}, -10),
    ({"ws": WS + 8}, -10), ({"ws": Q}, -10), ({"ws": MASK}, -10), ({"out": MASK}, -8),
    ({"lse": MASK}, -8), ({"D": 88}, -3), ({"scale": float("nan")}, -6), ({"q": 0}, -1),
])
def test_blocksparse_rejects_before_any_hip_call(kw, status):
    """Invalid arguments return their status without touching the GPU."""
    a = dict(GOOD, mask=MASK, nm=4, bm=128, bn=64, ws=WS, wsb=1 << 30)
    a.update(kw)
    rc = fa.fa_fwd_blocksparse(a["q"], a["k"], a["v"], a["out"], a["lse"], a["B"], a["H"], a["S"],
                               a["D"], a["scale"], a["causal"], a["window_left"],
                               a["window_right"], a["dtype"], a["mask"] or None, a["nm"], a["bm"],
                               a["bn"], a["ws"] or None, a["wsb"], None)
    assert rc == status


KP, VP, BT = 12 << 32, 13 << 32, 14 << 32  # fake page pools and block table


@pytest.mark.parametrize("kw,status", [
    ({"kp": 0}, -1), ({"bt": 0}, -1), ({"ps": 32}, -13), ({"ps": 100}, -13), ({"ps": 0}, -13),
    ({"np": 0}, -13), ({"ts": 2}, -13), ({"kp": KP + 8}, -7), ({"bt": BT + 2}, -7),
    ({"out": KP}, -8), ({"lse": BT}, -8), ({"out": VP + 64}, -8), ({"ns": 17}, -11),
    ({"ns": 2, "ws": 0}, -10), ({"ns": 2, "ws": KP}, -10), ({"ns": 2, "ws": WS + 4}, -10),
    ({"D": 40}, -3), ({"scale": -2.0}, -6), ({"window_right": -5}, -4),
])
def test_paged_rejects_before_any_hip_call(kw, status):
    """Invalid arguments return their status without touching the GPU (S = 300
    needs 3 table entries at page_size 128)."""
    a = dict(GOOD, kp=KP, vp=VP, bt=BT, np=40, ps=128, ts=3, ns=1, ws=WS, wsb=1 << 40)
    a.update(kw)
    rc = fa.fa_fwd_paged(a["q"], a["kp"] or None, a["vp"], a["bt"] or None, a["out"], a["lse"],
                         a["B"], a["H"], a["S"], a["D"], a["scale"], a["causal"],
                         a["window_left"], a["window_right"], a["dtype"], a["np"], a["ps"],
                         a["ts"], a["ns"], a["ws"] or None, a["wsb"], None)
    assert rc == status


def allowed(i, j, causal, wl, wr):
    return (not causal or j <= i) and (wl < 0 or i - j <= wl) and (wr < 0 or j - i <= wr)


SCHEDULES = [
    (1, 0, -1, -1), (7, 1, -1, -1), (63, 0, 3, 0), (129, 1, -1, -1), (200, 0, 20, 40),
    (300, 1, 5, -1), (300, 0, 0, 0), (257, 0, -1, 100), (1000, 1, 64, 64), (520, 0, 128, 128),
    (2048 + 5, 1, -1, -1), (700, 0, 700, 699), (1500, 1, 1499, 3),
    (4096 + 37, 1, -1, -1), (4096, 0, -1, -1), (5000, 1, 5000, -1),
]


@pytest.mark.parametrize("S,causal,wl,wr", SCHEDULES)
@pytest.mark.parametrize("dtype", [fa.FA_DTYPE_BF16, fa.FA_DTYPE_FP32])
def test_tile_schedule_against_brute_force(S, causal, wl, wr, dtype):
    """Every allowed pair lies in a visited tile; every visited tile holds an
    allowed pair of the Q tile; a tile marked mask-free has every pair
    allowed (rows of the Q tile, keys < S)."""
    first = fa.fa_fwd_tile_schedule(S, 128, dtype, causal, wl, wr, 0)
    bm, bn, nq = first["bm"], first["bn"], first["n_q_tiles"]
    assert nq == (S + bm - 1) // bm
    for qt in range(nq):
        sch = fa.fa_fwd_tile_schedule(S, 128, dtype, causal, wl, wr, qt)
        rows = range(qt * bm, min(S, (qt + 1) * bm))
        t0, t1 = sch["kt_begin"], sch["kt_end"]
        for t in range(-(-S // bn)):
            keys = range(t * bn, min(S, (t + 1) * bn))
            any_ok = any(allowed(i, j, causal, wl, wr) for i in rows for j in keys)
            assert any_ok == (t0 <= t < t1), (qt, t)
            if t0 <= t < t1 and not sch["needs_mask"][t - t0]:
                assert (t + 1) * bn <= S
                assert all(allowed(i, j, causal, wl, wr) for i in rows for j in keys)


def test_tile_schedule_counts_causal_16k():
    """S = 16384 causal at 128 x 64 tiles: Q tile t visits 2t + 2 K/V tiles,
    the last two of which (the diagonal) need the mask."""
    s0 = fa.fa_fwd_tile_schedule(16384, 128, fa.FA_DTYPE_BF16, 1, -1, -1, 0)
    assert (s0["bm"], s0["bn"], s0["n_q_tiles"]) == (128, 64, 128)
    tot, masked = 0, 0
    for qt in range(128):
        s = fa.fa_fwd_tile_schedule(16384, 128, fa.FA_DTYPE_BF16, 1, -1, -1, qt)
        assert s["kt_end"] - s["kt_begin"] == 2 * qt + 2
        assert s["needs_mask"] == [0] * (2 * qt) + [1] * 2
        tot += s["kt_end"] - s["kt_begin"]
        masked += sum(s["needs_mask"])
    assert tot == 16512 and masked == 256


def snake_launch(n_bh, S, D, esz):
    """Causal launches dealt in snake order: fewer (batch, head) pairs than XCDs,
    or the K/V of all heads within half of the 256 MB MALL."""
    return n_bh < 8 or 2 * n_bh * S * D * esz <= 128 << 20


@pytest.mark.parametrize("B,H,S", [(1, 16, 16384), (2, 16, 2048), (1, 3, 1000), (1, 5, 16384),
                                   (3, 7, 300), (1, 1, 128), (2, 1, 129), (1, 12, 4096),
                                   (2, 16, 16384), (1, 24, 12288), (3, 5, 30000)])
@pytest.mark.parametrize("causal", [0, 1])
def test_workgroup_order(B, H, S, causal):
    """The launch order is a bijection onto the (batch-head, Q tile) pairs; XCD
    x (workgroups x, x + 8, ...) holds one contiguous block of the head-major
    tile list.  With the causal mask the XCD runs the heavy three quarters of
    each head's Q tiles head by head, heaviest first, and then the lightest
    quarter of all its heads in non-increasing visited K/V tile count, after
    every heavier tile.  With the causal mask and fewer than 8 (batch, head)
    pairs, or K/V of all heads within half the MALL, the tiles are instead
    dealt to the XCDs in snake order of weight: each XCD runs heaviest first
    and the XCDs' summed K/V steps are balanced."""
    dt = fa.FA_DTYPE_BF16
    nq = fa.fa_fwd_tile_schedule(S, 128, dt, causal, -1, -1, 0)["n_q_tiles"]
    n = B * H * nq
    visits = [fa.fa_fwd_tile_schedule(S, 128, dt, causal, -1, -1, t) for t in range(nq)]
    visits = [x["kt_end"] - x["kt_begin"] for x in visits]
    tiles = [fa.fa_fwd_workgroup_tile(B, H, S, 128, dt, causal, -1, -1, w) for w in range(n)]
    assert sorted(tiles) == [(bh, qt) for bh in range(B * H) for qt in range(nq)]
    if causal and snake_launch(B * H, S, 128, 2):
        check_snake_order([visits[qt] for _, qt in tiles], cu_groups=True)
        # the list is rank-major: heads next to each other, heaviest rank first;
        # within an XCD every odd group of 32 workgroups (one per compute unit)
        # takes its positions in reverse
        def unpaired(w):
            x, k = w % 8, w // 8
            g = k // 32
            if g % 2 == 1 and 256 * (g + 1) <= n:
                return x + 8 * (32 * g + 31 - k % 32)
            return w
        order = sorted(range(n), key=lambda w: (unpaired(w) // 8, unpaired(w) % 8
                                                if (unpaired(w) // 8) % 2 == 0 or
                                                (unpaired(w) // 8 + 1) * 8 > n
                                                else 7 - unpaired(w) % 8))
        assert [tiles[w] for w in order] == [(p % (B * H), nq - 1 - p // (B * H))
                                             for p in range(n)]
        return
    for x in range(8):
        seq = tiles[x::8]
        # list position of each tile: head-major, heaviest-first rank when causal
        pos = sorted(bh * nq + (nq - 1 - qt if causal else qt) for bh, qt in seq)
        assert pos == list(range(pos[0], pos[0] + len(pos))) if pos else True
        if causal:
            light = nq // 4  # Q tiles qt < light close the launch
            heavy = [(bh, qt) for bh, qt in seq if qt >= light]
            tail = [(bh, qt) for bh, qt in seq if qt < light]
            assert seq == heavy + tail
            assert heavy == sorted(heavy, key=lambda t: (t[0], -t[1]))
            w = [visits[qt] for _, qt in tail]
            assert all(a >= b for a, b in zip(w, w[1:])), (x, w[:20])
        else:
            assert [bh * nq + qt for bh, qt in seq] == pos
    with pytest.raises(fa.FaError):
        fa.fa_fwd_workgroup_tile(B, H, S, 128, dt, causal, -1, -1, n)


@pytest.mark.parametrize("B,H,S,D,window", [(1, 16, 16384, 128, (-1, -1)),
                                             (1, 16, 32768, 128, (-1, -1)),
                                             (2, 16, 2048, 64, (-1, -1)),
                                             (1, 32, 4096, 64, (-1, -1)),
                                             (1, 20, 4096, 128, (1024, -1)),
                                             (1, 10, 4096, 256, (-1, -1)),
                                             (1, 3, 30000, 96, (-1, -1)),
                                             (4, 16, 4096, 64, (-1, -1))])
@pytest.mark.parametrize("causal", [0, 1])
def test_launch_order_dynamic_tail(B, H, S, D, window, causal):
    """The order on a 256-CU device: a bijection onto the (batch-head, Q tile)
    pairs.  A causal launch with more workgroups than the device holds (3, 2 or
    1 per CU for D <= 64, <= 128, above) has a dynamic tail: it starts at a
    multiple of B * H, its positions are the lightest ranks of all heads
    (heaviest first, heads rotated by one, ending on row 0 of head 0), and it
    holds at most 10% of the K/V steps while the rank before it would push it
    over.  The static part keeps the static order's shape: snake order
    (each XCD heaviest first, summed steps balanced) or blocks of whole heads
    per XCD.  Other launches keep fa_fwd_workgroup_tile's order."""
    dt = fa.FA_DTYPE_BF16
    wl, wr = window
    nq = fa.fa_fwd_tile_schedule(S, D, dt, causal, wl, wr, 0)["n_q_tiles"]
    n_bh = B * H
    n = n_bh * nq
    steps = []
    for t_ in range(nq):
        x = fa.fa_fwd_tile_schedule(S, D, dt, causal, wl, wr, t_)
        steps.append(x["kt_end"] - x["kt_begin"])
    res = [fa.fa_fwd_launch_order(B, H, S, D, dt, causal, wl, wr, 256, w) for w in range(n)]
    tiles = [(bh, qt) for bh, qt, _ in res]
    first = res[0][2]
    assert all(f == first for _, _, f in res)
    assert sorted(tiles) == [(bh, qt) for bh in range(n_bh) for qt in range(nq)]
    slots = 256 * (3 if D <= 64 else 2 if D <= 128 else 1)
    if not causal or n <= slots:
        assert first == -1
        assert tiles == [fa.fa_fwd_workgroup_tile(B, H, S, D, dt, causal, wl, wr, w)
                         for w in range(n)]
        return
    assert first >= 0 and first % n_bh == 0
    r0 = first // n_bh
    # dynamic positions: rank-major, heads rotated by one, last = (0, Q tile 0)
    assert tiles[first:] == [((p + 1) % n_bh, nq - 1 - p // n_bh) for p in range(first, n)]
    assert tiles[-1] == (0, 0)
    total = n_bh * sum(steps)
    tail = n_bh * sum(steps[qt] for qt in range(nq - r0))  # ranks r0 .. nq-1
    assert 100 * tail <= 10 * total
    assert r0 == 0 or 100 * (tail + n_bh * steps[nq - r0]) > 10 * total
    heavy = tiles[:first]
    assert sorted(heavy) == sorted((bh, qt) for bh in range(n_bh) for qt in range(nq - r0, nq))
    if snake_launch(n_bh, S, 64 if D <= 64 else 128 if D <= 128 else 256, 2):
        check_snake_order([steps[qt] for _, qt in heavy])
    else:  # each XCD: a contiguous block of whole heads' heavy ranks
        for x in range(8):
            pos = sorted(bh * r0 + (nq - 1 - qt) for bh, qt in heavy[x::8])
            assert pos == list(range(pos[0], pos[0] + len(pos))) if pos else True
    with pytest.raises(fa.FaError):
        fa.fa_fwd_launch_order(B, H, S, D, dt, causal, wl, wr, 256, n)
    with pytest.raises(fa.FaError):
        fa.fa_fwd_launch_order(B, H, S, D, dt, causal, wl, wr, 0, 0)


def check_snake_order(weights, cu_groups=False):
    """weights[w]: the K/V steps of workgroup w.  Every XCD (workgroups x, x + 8,
    ...) runs its items heaviest first, and the XCDs' summed steps differ by at
    most twice the heaviest item.  cu_groups: the XCD's items come in groups of
    32 (one per compute unit), each group at least as heavy as the next; an odd
    group that is whole runs lightest first, so that the units that got the
    heaviest items get the lighter ones of the next group."""
    sums = []
    for x in range(8):
        seq = weights[x::8]
        if not cu_groups:
            assert all(a >= b for a, b in zip(seq, seq[1:])), (x, seq[:20])
        else:
            groups = [seq[i:i + 32] for i in range(0, len(seq), 32)]
            for g, grp in enumerate(groups):
                whole = 256 * (g + 1) <= len(weights)
                run = grp[::-1] if g % 2 == 1 and whole else grp
                assert all(a >= b for a, b in zip(run, run[1:])), (x, g, grp[:20])
                if g + 1 < len(groups):
                    assert min(grp) >= max(groups[g + 1]), (x, g)
        sums.append(sum(seq))
    assert max(sums) - min(sums) <= 2 * max(weights), sums


@pytest.mark.parametrize("B,H,S,n_splits", [(1, 2, 16384, 4), (1, 2, 16384, 6), (1, 3, 1000, 2),
                                            (2, 16, 2048, 3), (1, 1, 129, 16), (1, 5, 4097, 5)])
@pytest.mark.parametrize("causal", [0, 1])
def test_splitkv_workgroup_order(B, H, S, n_splits, causal):
    """The split launch order is a bijection onto the (batch-head, Q tile, part)
    triples.  With the causal mask the parts are dealt to the XCDs in snake order
    of weight (each XCD heaviest first, summed steps balanced); without it a
    tile's parts are consecutive workgroups and the tiles follow fa_fwd's order.
    One part, or fp32 inputs, is fa_fwd's own order."""
    dt = fa.FA_DTYPE_BF16
    nq = fa.fa_fwd_tile_schedule(S, 128, dt, causal, -1, -1, 0)["n_q_tiles"]
    n = B * H * nq * n_splits
    visits = [fa.fa_fwd_tile_schedule(S, 128, dt, causal, -1, -1, t) for t in range(nq)]
    visits = [x["kt_end"] - x["kt_begin"] for x in visits]
    trip = [fa.fa_fwd_splitkv_workgroup_tile(B, H, S, 128, dt, causal, -1, -1, n_splits, w)
            for w in range(n)]
    assert sorted(trip) == [(bh, qt, p) for bh in range(B * H) for qt in range(nq)
                            for p in range(n_splits)]

    def part_steps(qt, p):  # the kernel's near-equal cut of a tile's K/V range
        L = visits[qt]
        return L * (p + 1) // n_splits - L * p // n_splits

    if causal:
        # heaviest tile first; a tile's parts differ by at most one step
        check_snake_order([visits[qt] for _, qt, _ in trip])
        sums = [sum(part_steps(qt, p) for _, qt, p in trip[x::8]) for x in range(8)]
        assert max(sums) - min(sums) <= 2 * max(visits), sums
    else:
        for w, (bh, qt, p) in enumerate(trip):
            assert p == w % n_splits
            assert (bh, qt) == fa.fa_fwd_workgroup_tile(B, H, S, 128, dt, causal, -1, -1,
                                                         w // n_splits)
    for dtype, ns in ((dt, 1), (fa.FA_DTYPE_FP32, n_splits)):
        nq1 = fa.fa_fwd_tile_schedule(S, 128, dtype, causal, -1, -1, 0)["n_q_tiles"]
        for w in range(0, B * H * nq1, 7):
            assert fa.fa_fwd_splitkv_workgroup_tile(B, H, S, 128, dtype, causal, -1, -1, ns, w) == \
                (*fa.fa_fwd_workgroup_tile(B, H, S, 128, dtype, causal, -1, -1, w), 0)
    with pytest.raises(fa.FaError):
        fa.fa_fwd_splitkv_workgroup_tile(B, H, S, 128, dt, causal, -1, -1, n_splits, n)
    with pytest.raises(fa.FaError):
        fa.fa_fwd_splitkv_workgroup_tile(B, H, S, 128, dt, causal, -1, -1, 17, 0)


def test_missing_library_fails_loudly(monkeypatch, tmp_path):
    monkeypatch.setattr(fam, "_LIB_PATH", str(tmp_path / "absent.so"))
    monkeypatch.setattr(fam, "_lib", None)
    with pytest.raises(RuntimeError, match="not built"):
        fam.fa_status_string(0)


@pytest.mark.parametrize("S,causal,window", [(128, False, (-1, -1)), (2048, True, (-1, -1)),
                                             (1000, False, (128, 128)), (777, True, (30, 5)),
                                             (300, False, (0, 0)), (50, False, (100, 3))])
def test_bench_pair_count_matches_oracle(S, causal, window):
    """bench.py's closed-form S_eff count against the oracle's brute force."""
    import bench
    import oracle

    assert bench.allowed_pairs(S, causal, window) == oracle.allowed_pairs(S, causal, window)


@pytest.mark.parametrize("S,causal,window,bm,bn", [(1000, True, (-1, -1), 128, 64),
                                                   (777, False, (100, 30), 256, 128),
                                                   (640, True, (200, -1), 128, 192)])
def test_bench_blocksparse_pair_count_brute_force(S, causal, window, bm, bn):
    """bench.py's block-sparse pair count against a brute-force count of the
    expanded element mask."""
    import numpy as np

    import bench
    from fa_inputs import local_global_block_mask, random_block_mask

    for mask in (random_block_mask(1, -(-S // bm), -(-S // bn), 0.4, S)[0].numpy(),
                 local_global_block_mask(-(-S // bm), -(-S // bn), bm, bn, 300, 1)[0].numpy()):
        el = np.repeat(np.repeat(mask.astype(bool), bm, 0), bn, 1)[:S, :S]
        i, j = np.meshgrid(np.arange(S), np.arange(S), indexing="ij")
        ok = el & ((not causal) | (j <= i)) & ((window[0] < 0) | (i - j <= window[0])) \
            & ((window[1] < 0) | (j - i <= window[1]))
        assert bench.blocksparse_pairs(S, causal, window, mask, bm, bn) == int(ok.sum())
        assert bench.blocksparse_pairs(S, causal, window, mask, bm, bn, 130, 400) == \
            int(ok[130:400].sum())


def test_bench_refuses_several_gpus():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "8"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2 and "one GPU" in r.stderr


# ---------------------------------------------------------------- KV cache
KC, VC, SL, KT = 10 << 32, 11 << 32, 12 << 32, 13 << 32  # caches, seqlens, table


@pytest.mark.parametrize("B,H,S_q,D,dtype,ns", [(8, 16, 1, 128, fa.FA_DTYPE_BF16, 16),
                                                  (3, 5, 130, 64, fa.FA_DTYPE_FP16, 64)])
def test_kvcache_workspace_size(B, H, S_q, D, dtype, ns):
    """fp32 partial O and LSE of every part: ns * B * H * S_q * (D + 1) * 4
    bytes; nothing for one part; fp32 inputs are not taken."""
    assert fa.fa_fwd_kvcache_workspace_size(B, H, S_q, D, dtype, ns) == ns * B * H * S_q * (D + 1) * 4
    assert fa.fa_fwd_kvcache_workspace_size(B, H, S_q, D, dtype, 1) == 0
    for bad, st in ((0, -11), (fa.FA_MAX_KV_SPLITS + 1, -11)):
        with pytest.raises(fa.FaError) as e:
            fa.fa_fwd_kvcache_workspace_size(B, H, S_q, D, dtype, bad)
        assert e.value.status == st
    with pytest.raises(fa.FaError) as e:
        fa.fa_fwd_kvcache_workspace_size(B, H, S_q, D, fa.FA_DTYPE_FP32, ns)
    assert e.value.status == -5


@pytest.mark.parametrize("kw,status", [
    ({}, None),
    ({"q": 0}, -1), ({"kc": 0}, -1), ({"vc": 0}, -1), ({"sl": 0}, -1), ({"out": 0}, -1),
    ({"D": 100}, -3), ({"D": 144}, -3), ({"dtype": fa.FA_DTYPE_FP32}, -5), ({"Sk": 0}, -2), ({"Sq": 0}, -2),
    ({"scale": float("nan")}, -6), ({"window_left": -3}, -4),
    ({"kc": KC + 8}, -7), ({"sl": SL + 2}, -7), ({"lse": LSE + 2}, -7),
    ({"out": KC}, -8), ({"lse": SL}, -8), ({"out": VC + 4096}, -8),
    ({"ns": 0}, -11), ({"ns": 65}, -11),
    ({"ns": 4, "ws": 0}, -10), ({"ns": 4, "ws": KC}, -10), ({"ns": 4, "wsb": 16}, -10),
    ({"bt": KT, "ps": 100}, -13), ({"bt": KT, "ps": 64, "ts": 3}, -13), ({"bt": KT, "np": 0}, -13),
    ({"bt": KT + 2, "ps": 64, "ts": 8}, -7), ({"bt": KT, "ps": 64, "ts": 8, "lse": KT}, -8),
])
def test_kvcache_rejects_before_any_hip_call(kw, status):
    """Invalid arguments return their status without touching the GPU (B = 2,
    S_q = 3 queries against a 500-row cache; a paged cache of 64-row pages
    needs 8 table entries)."""
    if status is None:  # the valid call itself is a GPU test; here only its checks
        return
    a = dict(GOOD, kc=KC, vc=VC, sl=SL, bt=0, Sq=3, Sk=500, np=40, ps=0, ts=0, ns=1, ws=WS,
             wsb=1 << 40)
    a.update(kw)
    rc = fa.fa_fwd_kvcache(a["q"], a["kc"], a["vc"], a["sl"] or None, a["bt"] or None, a["out"],
                           a["lse"], a["B"], a["H"], a["Sq"], a["Sk"], a["D"], a["scale"],
                           a["causal"], a["window_left"], a["window_right"], a["dtype"], a["np"],
                           a["ps"], a["ts"], a["ns"], a["ws"] or None, a["wsb"], None)
    assert rc == status
