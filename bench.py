"""Benchmark of the exact-attention forward (libfa_mi355x.fa_fwd) on one MI355X.

One step = one fa_fwd over the whole workload (every (batch, head), all rows):
tile schedule, Q/K/V loads, QK^T, mask, online softmax, P V and the epilogue
all run inside that single kernel launch.  Inputs are synthetic (seeded N(0,1),
rounded to the workload dtype) and resident in HBM before timing starts.

Timing: every launch is preceded, outside the HIP events that bracket it on
its stream, by a 512 MiB write that evicts L2 and the 256 MB MALL, then a read
of the same buffer that retires the dirty lines the write left behind (their
write-back would otherwise land inside the timed launch), so each timed launch
starts with cold caches (inputs resident in HBM) and a clean MALL.

Prints ONE JSON line:
  value         TFLOPS = 4 * B * H * S * S_eff * D / t, t = the median cold
                launch (S_eff = allowed (query, key) pairs / S, counted exactly)
  roofline      the kernel's rate over the mean cold launch against the MI355X
                dense bf16/fp16 MFMA peak (or HBM for a bandwidth-bound
                workload); warm back-to-back launches are reported beside it
  cpu_baseline  the fp64 CPU oracle timed on a bounded sample of the same
                workload on this host's cores (rate on the same FLOP count)
"""
from __future__ import annotations

import argparse
import hashlib
import re
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "attention fwd TFLOPS (4·B·H·S·S_eff·D/t) and % of MI355X bf16 MFMA peak"
METRIC_BWD = "attention bwd TFLOPS (10·B·H·S·S_eff·D/t: five products) and % of MI355X bf16 MFMA peak"
METRIC_BS = ("attention fwd TFLOPS over the pairs a block mask keeps (4·B·H·pairs·D/t) and % of "
             "MI355X bf16 MFMA peak")
PEAK_MFMA_TFLOPS = {"bf16": 2516.6, "fp16": 2516.6, "fp32": 157.3}  # MI355X dense, 2.4 GHz
PEAK_HBM_GBS = 8000.0
DEFAULT_WORKLOAD = "causal_16k"
KERNEL_SOURCES = ["io_aware_exact_22_amd/csrc/fa_fwd_device.h",
                  "io_aware_exact_22_amd/csrc/fa_fwd_kernels.hip",
                  "io_aware_exact_22_amd/csrc/fa_fwd_launch_cfg.h",
                  "io_aware_exact_22_amd/csrc/fa_kernel_common.h",
                  "io_aware_exact_22_amd/csrc/fa_launch.h",
                  "io_aware_exact_22_amd/csrc/fa_schedule.h"]


def allowed_pairs(S: int, causal: bool, window) -> int:
    """Sum over rows i of the number of allowed keys: the window [i - wl, i + wr]
    (clipped to [0, S), and to j <= i when causal)."""
    import numpy as np

    wl, wr = window
    i = np.arange(S, dtype=np.int64)
    lo = np.zeros(S, dtype=np.int64) if wl < 0 else np.maximum(0, i - wl)
    hi = np.full(S, S - 1, dtype=np.int64) if wr < 0 else np.minimum(S - 1, i + wr)
    if causal:
        hi = np.minimum(hi, i)
    return int(np.maximum(0, hi - lo + 1).sum())


def rows_pairs(S: int, causal: bool, window, r0: int, r1: int) -> int:
    """Allowed (query, key) pairs of query rows [r0, r1)."""
    import numpy as np

    wl, wr = window
    i = np.arange(r0, r1, dtype=np.int64)
    lo = np.zeros_like(i) if wl < 0 else np.maximum(0, i - wl)
    hi = np.full_like(i, S - 1) if wr < 0 else np.minimum(S - 1, i + wr)
    if causal:
        hi = np.minimum(hi, i)
    return int(np.maximum(0, hi - lo + 1).sum())


def blocksparse_pairs(S: int, causal: bool, window, mask, bm: int, bn: int, r0: int = 0,
                      r1: int | None = None) -> int:
    """Allowed (query, key) pairs of rows [r0, r1) under one head's block mask
    [n_qb, n_kb]: per row, the overlap of each kept key block with the row's
    window interval."""
    import numpy as np

    r1 = S if r1 is None else r1
    wl, wr = window
    mask = np.asarray(mask)
    total = 0
    for qb in range(r0 // bm, (r1 + bm - 1) // bm):
        i = np.arange(max(r0, qb * bm), min(r1, (qb + 1) * bm), dtype=np.int64)
        lo = np.zeros_like(i) if wl < 0 else np.maximum(0, i - wl)
        hi = np.full_like(i, S - 1) if wr < 0 else np.minimum(S - 1, i + wr)
        if causal:
            hi = np.minimum(hi, i)
        c0 = np.nonzero(mask[qb])[0].astype(np.int64) * bn
        c1 = np.minimum(S, c0 + bn)
        cnt = np.minimum(c1[None, :] - 1, hi[:, None]) - np.maximum(c0[None, :], lo[:, None]) + 1
        total += int(np.maximum(cnt, 0).sum())
    return total


def kernel_hash() -> str:
    """Hash of the kernel sources' code: comments and blank space are left
    out, so that editing a comment does not void the counter record."""
    h = hashlib.sha256()
    for p in KERNEL_SOURCES:
        src = open(os.path.join(ROOT, p), encoding="utf-8").read()
        src = re.sub(r"/\*.*?\*/", " ", src, flags=re.S)
        src = re.sub(r"//[^\n]*", " ", src)
        h.update(" ".join(src.split()).encode())
    return h.hexdigest()[:16]


def measured_traffic(workload: str):
    """HBM bytes per launch from the committed rocprofv3 counter summary, if it
    was taken on the current kernel source; else None."""
    p = os.path.join(ROOT, "profiles", f"fa_fwd_{workload}_hbm_traffic.json")
    if not os.path.exists(p):
        return None
    rec = json.load(open(p))
    if rec.get("kernel_hash") != kernel_hash():
        return None
    return rec.get("bytes_per_launch")


def sclk_file(dev_index: int = 0):
    """The sysfs DPM table of the GPU torch calls cuda:dev_index (its current
    shader clock level is the line marked '*'); None if it cannot be told."""
    import glob

    files = sorted(glob.glob("/sys/class/drm/card*/device/pp_dpm_sclk"))
    if len(files) == 1:
        return files[0]
    try:
        import torch

        p = torch.cuda.get_device_properties(dev_index)
        bus = "%02x:%02x" % (p.pci_bus_id, p.pci_device_id)
        for f in files:
            if bus in os.path.realpath(os.path.dirname(f)):
                return f
    except Exception:
        pass
    return None


def sample_sclk(step, stream, launch_ms: float, seconds: float = 0.6):
    """The shader clock while the timed launch runs back to back: about
    `seconds` of launches are queued after the timed steps and the current DPM
    clock is read from sysfs every 20 ms until they have run (the first 0.2 s,
    where the clock may still be ramping, are left out).  None if the clock
    cannot be read."""
    import numpy as np
    import torch

    f = sclk_file()
    if f is None:
        return None

    def read():
        try:
            for ln in open(f):
                if "*" in ln:
                    return float(ln.split(":")[1].strip().rstrip("*").strip().lower()
                                 .replace("mhz", ""))
        except Exception:
            return None
        return None

    n = max(8, int(seconds * 1e3 / max(launch_ms, 1e-3)))
    done = torch.cuda.Event()
    for _ in range(n):
        step()
    done.record(stream)
    t0, mhz = time.perf_counter(), []
    while not done.query():
        x = read()
        if x is not None and time.perf_counter() - t0 > 0.2:
            mhz.append(x)
        time.sleep(0.02)
    torch.cuda.synchronize()
    if not mhz:
        return None
    return {"median_mhz": float(np.median(mhz)), "min_mhz": float(np.min(mhz)),
            "max_mhz": float(np.max(mhz)), "samples": len(mhz),
            "source": f"{f} (current DPM level), read every 20 ms while {n} launches queued "
                      f"after the timed steps ran"}


def cpu_threads() -> int:
    """Threads for the CPU oracle: the host cores this process may use --
    OMP_NUM_THREADS when the host sets it (the CPU share a shared GPU host
    gives one process), else every core in the affinity mask."""
    n = len(os.sched_getaffinity(0))
    env = os.environ.get("OMP_NUM_THREADS", "")
    return max(1, min(n, int(env))) if env.isdigit() and int(env) > 0 else n


def cpu_baseline(w, q, k, v, target_s: float = 15.0):
    """Time the CPU oracle (as it stands) on whole heads of the workload: one
    head first, then as many heads (b, h) in order as fit about target_s
    seconds; report the rate on the metric's FLOP count."""
    import oracle

    threads = cpu_threads()
    per_head_flops = 4.0 * allowed_pairs(w.S, w.causal, w.window) * w.D
    heads = [(b, h) for b in range(w.B) for h in range(w.H)]

    def run(hs):
        t0 = time.perf_counter()
        for b, h in hs:
            oracle.fwd_rows(q, k, v, w.scale, w.causal, w.window, b, h, 0, w.S, nthreads=threads)
        return time.perf_counter() - t0

    dt1 = run(heads[:1])
    n = int(max(1, min(len(heads), target_s / max(dt1, 1e-3))))
    if n > 1:
        dt, used = run(heads[:n]), n
    else:
        dt, used = dt1, 1
    fl = per_head_flops * used
    # per-core figure: one thread on the last rows of head (0, 0), about 1-2 s
    r1 = w.S
    r0 = max(0, r1 - max(1, int(2e9 / (4.0 * w.D * w.S))))
    t0 = time.perf_counter()
    oracle.fwd_rows(q, k, v, w.scale, w.causal, w.window, 0, 0, r0, r1, nthreads=1)
    dt_1 = time.perf_counter() - t0
    fl_1 = 4.0 * rows_pairs(w.S, w.causal, w.window, r0, r1) * w.D
    return {
        "value": fl / dt / 1e12,
        "unit": "TFLOPS",
        "cores": threads,
        "affinity_cores": len(os.sched_getaffinity(0)),
        "kind": "oracle",
        "sample": (f"{w.name}: {used} of {len(heads)} (batch, head) pairs in full, fp64 oracle "
                   f"materialising each head's score matrix; {fl / 1e9:.1f} GFLOP (metric count) "
                   f"in {dt:.1f} s on {threads} threads"),
        "per_core": {"value": fl_1 / dt_1 / 1e12, "unit": "TFLOPS", "threads": 1,
                     "sample": f"rows [{r0}, {r1}) of (batch 0, head 0), {fl_1 / 1e9:.2f} GFLOP "
                               f"in {dt_1:.2f} s on one thread"},
    }


def cpu_baseline_bwd(w, q, k, v, dout, target_s: float = 15.0):
    """Time the CPU oracle's backward on a bounded sample: dq of chunks of 256
    query rows of batch 0, from the middle of head 0 on through the following
    rows and heads, until about target_s seconds (oracle.bwd_sampled: per-row
    statistics, then P and dS formed again for those rows).  Those rows' part
    of the metric is the S, dP and dQ products, 6 flops per allowed pair and d."""
    import numpy as np

    import oracle

    threads = cpu_threads()
    wl, wr = w.window
    CH = 256
    chunks = [(h, r) for h in range(w.H) for r in range(0, w.S, CH)]
    first = (w.S // 2) // CH
    chunks = chunks[first:] + chunks[:first]
    fl, dt, rows = 0.0, 0.0, 0
    for h, r0 in chunks:
        r1 = min(w.S, r0 + CH)
        t0 = time.perf_counter()
        oracle.bwd_sampled(q, k, v, dout, w.scale, w.causal, w.window, 0, h, list(range(r0, r1)),
                           [], nthreads=threads)
        dt += time.perf_counter() - t0
        i = np.arange(r0, r1, dtype=np.int64)
        lo = np.zeros_like(i) if wl < 0 else np.maximum(0, i - wl)
        hi = np.full_like(i, w.S - 1) if wr < 0 else np.minimum(w.S - 1, i + wr)
        if w.causal:
            hi = np.minimum(hi, i)
        fl += 6.0 * float(np.maximum(0, hi - lo + 1).sum()) * w.D
        rows += r1 - r0
        if dt >= target_s:
            break
    return {
        "value": fl / dt / 1e12,
        "unit": "TFLOPS",
        "cores": threads,
        "affinity_cores": len(os.sched_getaffinity(0)),
        "kind": "oracle",
        "sample": (f"{w.name} backward: dq of {rows} rows of batch 0 in chunks of {CH} from row "
                   f"{first * CH} of head 0 on (fp64 oracle, P and dS formed again per row); "
                   f"{fl / 1e9:.1f} GFLOP (S, dP, dQ products of those rows) in {dt:.1f} s on "
                   f"{threads} threads"),
    }


def cpu_baseline_blocksparse(w, q, k, v, mask, bm, bn, target_s: float = 15.0):
    """Time the CPU oracle's block-sparse rows: chunks of 512 rows of batch 0,
    from the middle of head 0 on through the following rows and heads, until
    about target_s seconds have run; report the rate on the metric's FLOP count
    for the rows done."""
    import oracle

    threads = cpu_threads()
    CH = 512
    chunks = [(h, r) for h in range(w.H) for r in range(0, w.S, CH)]
    first = (w.S // 2) // CH
    chunks = chunks[first:] + chunks[:first]
    fl, dt, rows = 0.0, 0.0, 0
    for h, r0 in chunks:
        r1 = min(w.S, r0 + CH)
        t0 = time.perf_counter()
        oracle.fwd_rows_blocksparse(q, k, v, w.scale, mask, bm, bn, w.causal, w.window, 0, h, r0,
                                    r1, nthreads=threads)
        dt += time.perf_counter() - t0
        fl += 4.0 * blocksparse_pairs(w.S, w.causal, w.window, mask[0], bm, bn, r0, r1) * w.D
        rows += r1 - r0
        if dt >= target_s:
            break
    return {
        "value": fl / dt / 1e12,
        "unit": "TFLOPS",
        "cores": threads,
        "affinity_cores": len(os.sched_getaffinity(0)),
        "kind": "oracle",
        "sample": (f"{w.name} under the block mask: {rows} rows of batch 0 in chunks of {CH} from "
                   f"row {first * CH} of head 0 on, fp64 oracle materialising those rows' scores; "
                   f"{fl / 1e9:.2f} GFLOP (metric count) in {dt:.1f} s on {threads} threads"),
    }


METRIC_KV = ("attention decode against a KV cache: HBM GB/s (K and V read once, q/O/LSE) and % "
             "of MI355X 8 TB/s")


def bench_kvcache(args, name: str) -> int:
    """fa_fwd_kvcache on a decoding workload (one new query per sequence
    against a long cache), timed like the forward: the 512 MiB flush (write,
    then read back) before every launch outside its HIP events; the rate is
    algorithmic bytes per launch over the median (value) and mean (roofline)
    cold launch."""
    import numpy as np
    import torch

    import io_aware_exact_22_amd as fa
    from fa_inputs import WORKLOADS_KV, kv_workload_inputs

    w = WORKLOADS_KV[name]
    dev = torch.device("cuda:0")
    q, k, v = kv_workload_inputs(w)
    qd, kd, vd = (t.to(dev) for t in (q, k, v))
    lens = torch.full((w.B,), w.S_k, dtype=torch.int32, device=dev)
    out = torch.empty_like(qd)
    lse = torch.empty((w.B, w.H, w.S_q), dtype=torch.float32, device=dev)
    stream = torch.cuda.current_stream(dev)
    dcode = fa.FA_DTYPE_BF16 if w.dtype == torch.bfloat16 else fa.FA_DTYPE_FP16
    ns = args.splitkv if args.splitkv > 0 else fa.fa_fwd_kvcache_auto_splits(
        w.B, w.H, w.S_q, w.S_k, w.D, dcode)
    need = fa.fa_fwd_kvcache_workspace_size(w.B, w.H, w.S_q, w.D, dcode, ns)
    ws = torch.empty(max(1, need // 4), dtype=torch.float32, device=dev)

    def step():
        fa.flash_attn_fwd_kvcache(qd, kd, vd, lens, softmax_scale=w.scale, causal=True,
                                  n_splits=ns, out=out, lse=lse, workspace=ws, stream=stream)

    flush = torch.empty(args.flush_mib << 18, dtype=torch.float32, device=dev) \
        if args.flush_mib > 0 else None

    def launch(events=None):
        if flush is not None:
            flush.fill_(1.0)
            if args.flush_mode == "write-read":
                flush.sum()
        if events is not None:
            events[0].record(stream)
        step()
        if events is not None:
            events[1].record(stream)

    for _ in range(args.warmup):
        launch()
    torch.cuda.synchronize(dev)
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(args.steps)]
    torch.cuda.synchronize(dev)
    for e in ev:
        launch(e)
    torch.cuda.synchronize(dev)
    ms = [e0.elapsed_time(e1) for e0, e1 in ev]
    del flush
    if not (bool(torch.isfinite(out.float()).all()) and bool(torch.isfinite(lse).all())):
        print("bench.py: non-finite output", file=sys.stderr)
        return 1
    esz = 2
    kv_bytes = 2 * w.B * w.S_k * w.H * w.D * esz
    alg_bytes = kv_bytes + 2 * w.B * w.S_q * w.H * w.D * esz + 4 * w.B * w.H * w.S_q
    flops = 4.0 * w.B * w.H * w.S_q * w.S_k * w.D
    med, mean = float(np.median(ms)), float(np.mean(ms))
    gbs = alg_bytes / (med * 1e-3) / 1e9
    ach = alg_bytes / (mean * 1e-3) / 1e9
    rec = {
        "metric": METRIC_KV, "value": gbs, "unit": "GB/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": med, "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "bf16" if w.dtype == torch.bfloat16 else "fp16",
        "data": "synthetic",
        "config": {"workload": w.name, "B": w.B, "H": w.H, "S_q": w.S_q, "S_k": w.S_k, "D": w.D,
                   "causal": True, "cache_seqlens": "all S_k", "n_splits": ns,
                   "entry": "fa_fwd_kvcache", "parallelism": "single GPU",
                   "flops_per_step": flops},
        "roofline": {"bound": "hbm", "achieved": ach, "peak": PEAK_HBM_GBS, "unit": "GB/s",
                     "frac": ach / PEAK_HBM_GBS, "traffic": None, "kernel_ms": mean,
                     "kernel_ms_median": med, "kernel_ms_min": float(np.min(ms)),
                     "algorithmic_bytes_per_launch": alg_bytes,
                     "timing": f"{args.steps} launches, each preceded outside its HIP events by a "
                               f"{args.flush_mib} MiB {args.flush_mode} flush that evicts L2 and "
                               f"the MALL"},
    }
    if args.no_cpu_baseline:
        rec["cpu_baseline"] = None
    else:
        import oracle

        threads = cpu_threads()
        t0 = time.perf_counter()
        nb = 0
        for b in range(w.B):  # whole sequences until about 10 s
            oracle.fwd_kvcache(q[b:b + 1].contiguous(), k[b:b + 1].contiguous(),
                               v[b:b + 1].contiguous(), [w.S_k], w.scale, True, nthreads=threads)
            nb += 1
            if time.perf_counter() - t0 > 10.0:
                break
        dt = time.perf_counter() - t0
        rec["cpu_baseline"] = {
            "value": alg_bytes * nb / w.B / dt / 1e9, "unit": "GB/s", "cores": threads,
            "affinity_cores": len(os.sched_getaffinity(0)), "kind": "oracle",
            "sample": f"{w.name}: {nb} of {w.B} sequences in full (all heads), fp64 oracle, "
                      f"{dt:.1f} s on {threads} threads; rate on the same byte count"}
    print(json.dumps(rec), flush=True)
    return 0


def main() -> int:
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawTextHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default=DEFAULT_WORKLOAD)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--clock", action="store_true",
                    help="after the timed steps, sample the shader clock while about 0.6 s of "
                         "further launches run back to back (roofline.sclk)")
    ap.add_argument("--no-clock", action="store_true", help=argparse.SUPPRESS)
    ap.add_argument("--backward", action="store_true",
                    help="time fa_bwd (the gradients of the forward) instead of fa_fwd; "
                         "bf16 / fp16 workloads")
    ap.add_argument("--splitkv", type=int, default=-1,
                    help="time fa_fwd_splitkv with this many K/V parts per Q tile (0 = the "
                         "library's choice for the device) instead of fa_fwd")
    ap.add_argument("--blocksparse", default="",
                    help="time fa_fwd_blocksparse under a local + global block mask on 128 x 64 "
                         "blocks: 'local:KEYS[:GLOBAL]' keeps, for each 128-row block, the KEYS "
                         "keys ending at its last row and the first GLOBAL 64-key blocks "
                         "(default 1)")
    ap.add_argument("--paged", type=int, default=0,
                    help="time fa_fwd_paged with K/V cut into pages of this many rows (a multiple "
                         "of 64), placed at a seeded random permutation of a pool with spare "
                         "pages; combines with --splitkv")
    ap.add_argument("--flush-mib", type=int, default=512,
                    help="MiB written before every launch, outside the events, to evict L2 and "
                         "the MALL (0 = no flush: warm back-to-back launches are timed)")
    ap.add_argument("--flush-mode", choices=["write", "write-read"], default="write-read",
                    help="the flush before each launch: a write of the buffer followed by a read "
                         "of it (default: the read retires the dirty lines the write leaves in "
                         "L2 and the MALL, so that writing them back is not part of the timed "
                         "launch), or the write alone")
    ap.add_argument("--warm-steps", type=int, default=0,
                    help="after the timed region, this many warm back-to-back launches, reported "
                         "as roofline.warm (0 = skip)")
    ap.add_argument("--kvcache", default="",
                    help="time fa_fwd_kvcache on this decoding workload (decode_16k, decode_32k) "
                         "instead of fa_fwd; --splitkv N sets the part count (default: the "
                         "library's choice)")
    ap.add_argument("--copy-calibration-mib", type=int, default=0,
                    help="instead of the benchmark, run --steps plain device copies of this many "
                         "MiB (the reference kernel for scaling HBM byte counters)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py: this build runs on one GPU only; --gpus {args.gpus} is not supported "
              "(per-GPU throughput is the single-GPU value)", file=sys.stderr)
        return 2

    import numpy as np
    import torch

    import io_aware_exact_22_amd as fa
    from fa_inputs import WORKLOADS, workload_qkv

    if not torch.cuda.is_available():
        print("bench.py: no GPU visible", file=sys.stderr)
        return 1
    if args.kvcache:
        return bench_kvcache(args, args.kvcache)
    if args.copy_calibration_mib:
        n = args.copy_calibration_mib << 20
        src = torch.ones(n // 4, dtype=torch.float32, device="cuda:0")
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        for _ in range(args.steps):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_calibration_bytes_read": n, "copy_calibration_bytes_written": n,
                          "steps": args.steps}))
        return 0
    w = WORKLOADS[args.workload]
    dt_name = {torch.float32: "fp32", torch.float16: "fp16", torch.bfloat16: "bf16"}[w.dtype]
    q, k, v = workload_qkv(w)
    dev = torch.device("cuda:0")
    qd, kd, vd = (t.to(dev) for t in (q, k, v))
    out = torch.empty_like(qd)
    lse = torch.empty((w.B, w.H, w.S), dtype=torch.float32, device=dev)
    stream = torch.cuda.current_stream(dev)

    n_splits = None
    paged = None  # paged K/V: description of the pools
    bs = None  # block-sparse: (mask [1, n_qb, n_kb] on the CPU, description)
    if args.blocksparse:
        from fa_inputs import local_global_block_mask

        parts = args.blocksparse.split(":")
        if parts[0] != "local" or len(parts) not in (2, 3):
            print("bench.py: --blocksparse takes local:KEYS[:GLOBAL]", file=sys.stderr)
            return 2
        local_keys, glob = int(parts[1]), int(parts[2]) if len(parts) == 3 else 1
        bm, bn = 128, 64
        mask = local_global_block_mask(-(-w.S // bm), -(-w.S // bn), bm, bn, local_keys, glob)
        dcode = {torch.float32: fa.FA_DTYPE_FP32, torch.float16: fa.FA_DTYPE_FP16,
                 torch.bfloat16: fa.FA_DTYPE_BF16}[w.dtype]
        need = fa.fa_fwd_blocksparse_workspace_size(w.B, w.H, w.S, w.D, dcode, 1)
        ws = torch.empty(max(1, need // 4), dtype=torch.int32, device=dev)
        md = mask.to(dev)
        bs = (mask, {"pattern": "local+global", "local_keys": local_keys,
                     "global_key_blocks": glob, "block_m": bm, "block_n": bn,
                     "kept_blocks": int(mask.sum()),
                     "block_density": float(mask.float().mean())})

        def step():
            fa.flash_attn_fwd_blocksparse(qd, kd, vd, md, bm, bn, softmax_scale=w.scale,
                                          causal=w.causal, window_size=w.window, out=out, lse=lse,
                                          workspace=ws, stream=stream)
    elif args.backward:
        out, lse = fa.flash_attn_fwd(qd, kd, vd, softmax_scale=w.scale, causal=w.causal,
                                     window_size=w.window, stream=stream)
        g = torch.Generator(device="cpu")
        g.manual_seed(w.seed + 1000)
        do_cpu = torch.randn(qd.shape, generator=g, dtype=torch.float32).to(w.dtype)
        dod = do_cpu.to(dev)
        need = fa.fa_bwd_workspace_size(
            w.B, w.H, w.S, w.D, fa.FA_DTYPE_BF16 if w.dtype == torch.bfloat16 else fa.FA_DTYPE_FP16)
        ws_b = torch.empty((need + 3) // 4, dtype=torch.float32, device=dev)
        dq, dk, dv = torch.empty_like(qd), torch.empty_like(kd), torch.empty_like(vd)

        def step():
            fa.flash_attn_bwd(dod, qd, kd, vd, out, lse, softmax_scale=w.scale, causal=w.causal,
                              window_size=w.window, workspace=ws_b, dq=dq, dk=dk, dv=dv,
                              stream=stream)
    elif args.paged:
        ps = args.paged
        n_pg = -(-w.S // ps)
        num_pages = w.B * n_pg + max(1, w.B * n_pg // 8)
        g = torch.Generator(device="cpu")
        g.manual_seed(w.seed + 2000)
        slots = torch.randperm(num_pages, generator=g)[: w.B * n_pg]
        pools = []
        for t in (kd, vd):
            pad = torch.zeros((w.B, n_pg * ps, w.H, w.D), dtype=w.dtype, device=dev)
            pad[:, : w.S] = t
            pool = torch.zeros((num_pages, ps, w.H, w.D), dtype=w.dtype, device=dev)
            pool[slots.to(dev)] = pad.view(w.B * n_pg, ps, w.H, w.D)
            pools.append(pool)
            del pad
        kp, vp = pools
        table = slots.view(w.B, n_pg).to(torch.int32).to(dev).contiguous()
        dcode = {torch.float32: fa.FA_DTYPE_FP32, torch.float16: fa.FA_DTYPE_FP16,
                 torch.bfloat16: fa.FA_DTYPE_BF16}[w.dtype]
        ns = max(1, args.splitkv) if args.splitkv >= 0 else 1
        if args.splitkv == 0:
            ns = fa.fa_fwd_splitkv_auto_splits(w.B, w.H, w.S, w.D, int(w.causal), w.window[0],
                                               w.window[1], dcode)
        need = fa.fa_fwd_splitkv_workspace_size(w.B, w.H, w.S, w.D, dcode, ns)
        ws = torch.empty(max(1, (need + 3) // 4), dtype=torch.float32, device=dev)
        n_splits = ns if ns > 1 else None
        paged = {"page_size": ps, "num_pages": num_pages, "pages_used": w.B * n_pg,
                 "placement": "seeded random permutation"}

        def step():
            fa.flash_attn_fwd_paged(qd, kp, vp, table, softmax_scale=w.scale, causal=w.causal,
                                    window_size=w.window, n_splits=ns, out=out, lse=lse,
                                    workspace=ws, stream=stream)
    elif args.splitkv >= 0:
        dcode = {torch.float32: fa.FA_DTYPE_FP32, torch.float16: fa.FA_DTYPE_FP16,
                 torch.bfloat16: fa.FA_DTYPE_BF16}[w.dtype]
        n_splits = args.splitkv or fa.fa_fwd_splitkv_auto_splits(
            w.B, w.H, w.S, w.D, int(w.causal), w.window[0], w.window[1], dcode)
        need = fa.fa_fwd_splitkv_workspace_size(w.B, w.H, w.S, w.D, dcode, n_splits)
        ws = torch.empty(max(1, (need + 3) // 4), dtype=torch.float32, device=dev)

        def step():
            fa.flash_attn_fwd_splitkv(qd, kd, vd, softmax_scale=w.scale, causal=w.causal,
                                      window_size=w.window, n_splits=n_splits, out=out, lse=lse,
                                      workspace=ws, stream=stream)
    else:
        def step():
            fa.flash_attn_fwd(qd, kd, vd, softmax_scale=w.scale, causal=w.causal,
                              window_size=w.window, out=out, lse=lse, stream=stream)

    # Timing protocol: before every launch (warm-up and timed alike) a 512 MiB
    # write evicts L2 and the 256 MB MALL and a read of the same buffer retires
    # the dirty lines it left, outside the HIP events; the events on the
    # launch's stream bracket the launch alone.  value and the
    # roofline use these cold launches (median and mean); inputs stay
    # resident in HBM throughout.
    flush = torch.empty(args.flush_mib << 18, dtype=torch.float32, device=dev) \
        if args.flush_mib > 0 else None

    def timed_launch(events=None):
        if flush is not None:
            flush.fill_(1.0)
            if args.flush_mode == "write-read":
                flush.sum()  # reads every line back; the scalar stays on the device
        if events is not None:
            events[0].record(stream)
        step()
        if events is not None:
            events[1].record(stream)

    for _ in range(args.warmup):
        timed_launch()
    torch.cuda.synchronize(dev)
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(args.steps)]
    torch.cuda.synchronize(dev)
    t0 = time.perf_counter()
    for e in ev:
        timed_launch(e)
    torch.cuda.synchronize(dev)
    wall = time.perf_counter() - t0
    launch_ms = [e0.elapsed_time(e1) for e0, e1 in ev]
    del flush
    # warm launches back to back after the timed region (caches hold K and V),
    # reported beside the headline
    warm_ms, warm_wall = [], None
    if args.warm_steps > 0:
        wev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
               for _ in range(args.warm_steps)]
        step()
        torch.cuda.synchronize(dev)
        tw = time.perf_counter()
        for e0, e1 in wev:
            e0.record(stream)
            step()
            e1.record(stream)
        torch.cuda.synchronize(dev)
        warm_wall = (time.perf_counter() - tw) * 1e3 / args.warm_steps
        warm_ms = [e0.elapsed_time(e1) for e0, e1 in wev]
    # (off by default: the default command launches only the warm-up and timed
    # launches, so a kernel trace of it averages exactly what achieved uses)
    sclk = sample_sclk(step, stream, float(np.median(launch_ms))) if args.clock else None

    if bs is not None:
        pairs = blocksparse_pairs(w.S, w.causal, w.window, bs[0][0], 128, 64)
    else:
        pairs = allowed_pairs(w.S, w.causal, w.window)
    s_eff = pairs / w.S
    # the backward's five products (S, dP, dV, dK, dQ) against the forward's two
    flops = (10.0 if args.backward else 4.0) * w.B * w.H * pairs * w.D
    ms_per_step = float(np.median(launch_ms))  # the median cold launch
    tflops = flops / (ms_per_step * 1e-3) / 1e12
    avg_launch_ms = float(np.mean(launch_ms))
    kern_tflops = flops / (avg_launch_ms * 1e-3) / 1e12
    esz = 4 if dt_name == "fp32" else 2
    if args.backward:  # read q, k, v, out, dO and LSE; write dQ, dK, dV; D out and back in
        alg_bytes = 8 * w.B * w.S * w.H * w.D * esz + 12 * w.B * w.H * w.S
    else:
        alg_bytes = 4 * w.B * w.S * w.H * w.D * esz + 4 * w.B * w.H * w.S
    ai = flops / alg_bytes
    peak = PEAK_MFMA_TFLOPS[dt_name]
    hbm_bound = ai < peak * 1e12 / (PEAK_HBM_GBS * 1e9)
    if hbm_bound:
        achieved = alg_bytes / (avg_launch_ms * 1e-3) / 1e9
        roof = {"bound": "hbm", "achieved": achieved, "peak": PEAK_HBM_GBS, "unit": "GB/s",
                "frac": achieved / PEAK_HBM_GBS}
    else:
        roof = {"bound": "mfma", "achieved": kern_tflops, "peak": peak, "unit": "TFLOP/s",
                "frac": kern_tflops / peak}
    # the recorded counters are those of fa_fwd on its default workload
    roof["traffic"] = (None if (args.backward or n_splits is not None or bs is not None or paged)
                       else measured_traffic(w.name))
    roof["kernel_ms"] = avg_launch_ms
    roof["kernel_ms_median"] = float(np.median(launch_ms))
    roof["kernel_ms_min"] = float(np.min(launch_ms))
    roof["timing"] = (f"{args.steps} launches on the launch's stream, each preceded outside the "
                      f"HIP events by a {args.flush_mib} MiB {args.flush_mode} flush that evicts "
                      f"L2 and the MALL "
                      f"({args.warmup} warm-up launches likewise); achieved uses the mean, value "
                      f"the median" if args.flush_mib > 0 else
                      f"{args.steps} back-to-back launches (no cache flush)")
    roof["warm"] = ({"kernel_ms_mean": float(np.mean(warm_ms)),
                     "kernel_ms_median": float(np.median(warm_ms)),
                     "kernel_ms_min": float(np.min(warm_ms)),
                     "wall_ms_per_step": warm_wall,
                     "tflops_at_median": flops / (float(np.median(warm_ms)) * 1e-3) / 1e12,
                     "frac_at_median": (flops / (float(np.median(warm_ms)) * 1e-3) / 1e12) / peak,
                     "launches": len(warm_ms),
                     "note": "back to back after the timed region, K and V resident in L2/MALL"}
                    if warm_ms else None)
    roof["algorithmic_flops_per_launch"] = flops
    roof["algorithmic_bytes_per_launch"] = alg_bytes
    # the same rate against the MFMA peak at the shader clock the chip ran at
    # (the published peak assumes 2.4 GHz)
    roof["sclk"] = sclk
    roof["frac_at_observed_sclk"] = (
        kern_tflops / (peak * sclk["median_mhz"] / 2400.0)
        if (sclk and not hbm_bound and sclk["median_mhz"] > 0) else None)

    # correctness of what was timed: sampled rows against the oracle are the
    # GPU tests' job; here only a finiteness check of the timed output
    timed = (dq, dk, dv) if args.backward else (out, lse)
    if not all(bool(torch.isfinite(t.float()).all()) for t in timed):
        print("bench.py: non-finite output", file=sys.stderr)
        return 1

    rec = {
        "metric": METRIC_BWD if args.backward else METRIC_BS if bs is not None else METRIC,
        "value": tflops,
        "unit": "TFLOPS",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": dt_name,
        "data": "synthetic",
        "pct_of_peak": 100.0 * tflops / peak,
        # the common S/2 count for a causal mask over the whole sequence, for
        # comparison with figures quoted that way (the value counts exact pairs)
        "tflops_causal_half_convention": (
            (10.0 if args.backward else 4.0) * w.B * w.H * w.S * (w.S / 2) * w.D
            / (ms_per_step * 1e-3) / 1e12
            if (w.causal and tuple(w.window) == (-1, -1) and bs is None) else None),
        "config": {"workload": w.name, "B": w.B, "H": w.H, "S": w.S, "D": w.D,
                   "causal": w.causal, "window": list(w.window), "S_eff": s_eff,
                   "flops_per_step": flops, "parallelism": "single GPU",
                   "entry": ("fa_bwd" if args.backward else "fa_fwd_blocksparse" if bs else
                             "fa_fwd_paged" if paged else
                             "fa_fwd" if n_splits is None else "fa_fwd_splitkv"),
                   **({} if n_splits is None else {"n_splits": n_splits}),
                   **({} if paged is None else {"paged_kv": paged}),
                   **({} if bs is None else {"block_mask": bs[1]})},
        "roofline": roof,
    }
    if args.no_cpu_baseline:
        rec["cpu_baseline"] = None
    elif bs is not None:
        rec["cpu_baseline"] = cpu_baseline_blocksparse(w, q, k, v, bs[0].numpy(), 128, 64)
    elif args.backward:
        rec["cpu_baseline"] = cpu_baseline_bwd(w, q, k, v, do_cpu)
    else:  # fa_fwd, fa_fwd_splitkv and fa_fwd_paged compute the same definition
        rec["cpu_baseline"] = cpu_baseline(w, q, k, v)
    print(json.dumps(rec), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
