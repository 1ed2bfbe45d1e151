"""Builds libfa_mi355x.so (the gfx950 kernels and the C ABI) in-tree with hipcc.

Runs on a machine without a GPU: hipcc cross-compiles for gfx950.
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
LIB = os.path.join(PKG, "libfa_mi355x.so")
SOURCES = ["fa_api.hip", "fa_fwd_kernels.hip", "fa_fwd_padded.hip", "fa_fwd_wide_bf16.hip",
           "fa_fwd_wide_fp16.hip", "fa_fwd_kvcache.hip", "fa_fwd_kvcache_padded.hip",
           "fa_bwd_kernels.hip", "fa_bwd_padded.hip"]

HIPCC_FLAGS = [
    "--offload-arch=gfx950",
    "-O3",
    "-std=c++17",
    "-shared",
    "-fPIC",
    "-fvisibility=hidden",
    "-Wall",
    # keep the compiler from forming packed-fp32 VALU ops (v_pk_*_f32)
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # MFMA results in VGPRs: the score tile feeds VALU code directly, with no
    # v_accvgpr_read copies
    "-Xarch_device", "-mllvm=-amdgpu-mfma-vgpr-form",
]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found: the ROCm toolchain is required to build libfa_mi355x")


def build(verbose: bool = False, extra_flags: list[str] | None = None) -> str:
    """Compile every HIP source into libfa_mi355x.so (always recompiles).  The
    sources compile to objects in parallel, then one link makes the library."""
    tag = ".tmp%d" % os.getpid()
    tmp = LIB + tag
    inc = ["-I", os.path.join(ROOT, "include"), "-I", CSRC]
    flags = [f for f in HIPCC_FLAGS if f not in ("-shared",)]
    objs, procs = [], []
    for s in SOURCES:
        obj = os.path.join(CSRC, s + tag + ".o")
        cmd = [hipcc(), *flags, *(extra_flags or []), *inc, "-c", os.path.join(CSRC, s), "-o", obj]
        if verbose:
            print(" ".join(cmd), flush=True)
        objs.append(obj)
        procs.append(subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT,
                                      text=True))
    outs = [(p, p.communicate()[0]) for p in procs]
    try:
        failed = False
        for (p, out), s in zip(outs, SOURCES):
            # hipcc's host pass warns that it does not know the packed-fp32 feature
            msgs = [ln for ln in out.splitlines() if "packed-fp32-ops" not in ln]
            if p.returncode != 0:
                sys.stderr.write(f"--- {s}\n" + "\n".join(msgs) + "\n")
                failed = True
            elif verbose and msgs:
                print("\n".join(msgs))
        if failed:
            raise RuntimeError("hipcc failed building libfa_mi355x.so")
        cmd = [hipcc(), "--offload-arch=gfx950", "-shared", "-fPIC", *objs, "-o", tmp]
        r = subprocess.run(cmd, capture_output=True, text=True)
        if r.returncode != 0:
            sys.stderr.write(r.stdout + r.stderr)
            raise RuntimeError(f"hipcc failed ({r.returncode}) linking libfa_mi355x.so")
    finally:
        for o in objs:
            if os.path.exists(o):
                os.remove(o)
    check_launch_stubs(tmp)
    os.replace(tmp, LIB)
    return LIB


def check_launch_stubs(path: str) -> None:
    """hipcc's host pass can drop a kernel's launch stub without a diagnostic
    (e.g. when a device-only builtin sits inside a lambda of a kernel
    template); the library then fails to load.  Refuse such a build."""
    r = subprocess.run(["nm", "-C", "--undefined-only", path], capture_output=True, text=True)
    missing = [ln.split(None, 1)[-1] for ln in r.stdout.splitlines() if "__device_stub__" in ln]
    if missing:
        os.remove(path)
        raise RuntimeError("hipcc emitted no host launch stub for: " + "; ".join(missing))


if __name__ == "__main__":
    print(build(verbose=True))
