"""Seeded synthetic inputs and the named workloads for exact-attention forward.

This module serves both the GPU library's tests/benchmark and the CPU oracle's
tests.  It holds no arithmetic of the method: it only draws i.i.d. N(0, 1)
values in fp32 from a seeded CPU generator and rounds them (round to nearest
even, torch's cast) to the workload's dtype, so the GPU path and the oracle see
identical bits.

Workload shapes follow the pages' own examples: a GPT-style causal call with
the default scale (FlashAttention技术解析 page, section 2.2), seq 4096 with
head_dim 64 (the benchmark row on the Flash-Attention compile-guide page,
section 性能与内存占用测试验证), the (128, 128) sliding window (same page,
section 滑动窗口注意力), and a 16K causal sequence (the V2 page's A100 16K
figure, section 二.2) with a 32K variant (table 1 of the first page).  Batch
and head counts are not stated on the pages and are fixed here.
"""
from __future__ import annotations

import math
from dataclasses import dataclass

import torch


@dataclass(frozen=True)
class Workload:
    name: str
    B: int
    H: int
    S: int
    D: int
    dtype: torch.dtype
    causal: bool
    window: tuple
    seed: int

    @property
    def scale(self) -> float:
        return 1.0 / math.sqrt(self.D)

    def describe(self) -> str:
        dt = {torch.float32: "fp32", torch.float16: "fp16", torch.bfloat16: "bf16"}[self.dtype]
        mask = "causal" if self.causal else "full"
        if self.window != (-1, -1):
            mask = f"window{self.window}" + ("+causal" if self.causal else "")
        return f"B{self.B} H{self.H} S{self.S} D{self.D} {dt} {mask}"


WORKLOADS = {
    "tiny_fp32": Workload("tiny_fp32", 1, 2, 128, 64, torch.float32, False, (-1, -1), 1),
    "gpt_causal_2k": Workload("gpt_causal_2k", 2, 16, 2048, 64, torch.bfloat16, True, (-1, -1), 2),
    "full_4k_d64": Workload("full_4k_d64", 4, 16, 4096, 64, torch.float16, False, (-1, -1), 3),
    "window_8k": Workload("window_8k", 2, 16, 8192, 128, torch.bfloat16, False, (128, 128), 4),
    "causal_16k": Workload("causal_16k", 1, 16, 16384, 128, torch.bfloat16, True, (-1, -1), 5),
    "causal_32k": Workload("causal_32k", 1, 16, 32768, 128, torch.bfloat16, True, (-1, -1), 6),
    # one GPU's share of causal_16k split by heads over 8 GPUs (2 of 16 heads):
    # a grid of one workgroup per compute unit, the case split-KV is for
    "causal_16k_h2": Workload("causal_16k_h2", 1, 2, 16384, 128, torch.bfloat16, True, (-1, -1), 7),
    # a million-token causal sequence, the long-context case block-sparse
    # attention is for (FlashAttention技术解析 page, section 5); only run under a
    # block mask
    "causal_1m_h8": Workload("causal_1m_h8", 1, 8, 1 << 20, 128, torch.bfloat16, True, (-1, -1), 8),
}


@dataclass(frozen=True)
class KvWorkload:
    """Decoding against a key/value cache: S_q new queries per sequence, a
    cache of S_k rows (all of them holding keys unless a test says otherwise)."""
    name: str
    B: int
    H: int
    S_q: int
    S_k: int
    D: int
    dtype: torch.dtype
    seed: int

    @property
    def scale(self) -> float:
        return 1.0 / math.sqrt(self.D)

    def describe(self) -> str:
        dt = {torch.float16: "fp16", torch.bfloat16: "bf16"}[self.dtype]
        return f"B{self.B} H{self.H} S_q{self.S_q} S_k{self.S_k} D{self.D} {dt} causal"


# One new token per sequence against a long cache: the inference step FlashDecoding
# serves (FlashAttention技术解析 page, section 5), at the 16K and 32K lengths of
# the forward workloads.  Batch and heads are not stated on the pages.
WORKLOADS_KV = {
    "decode_16k": KvWorkload("decode_16k", 8, 16, 1, 16384, 128, torch.bfloat16, 9),
    "decode_32k": KvWorkload("decode_32k", 4, 16, 1, 32768, 128, torch.bfloat16, 10),
}


def kv_workload_inputs(w: KvWorkload):
    """q [B, S_q, H, D] and the caches [B, S_k, H, D]: q from generator seed
    w.seed, k and v from seed w.seed + 1 (make_qkv's draws)."""
    q, _, _ = make_qkv(w.B, w.S_q, w.H, w.D, w.dtype, w.seed)
    _, k, v = make_qkv(w.B, w.S_k, w.H, w.D, w.dtype, w.seed + 1)
    return q, k, v


def make_qkv(B: int, S: int, H: int, D: int, dtype: torch.dtype, seed: int):
    """q, k, v as contiguous CPU tensors [B, S, H, D], drawn in that order from
    one torch CPU generator seeded with ``seed``, fp32 N(0, 1), then cast."""
    g = torch.Generator(device="cpu")
    g.manual_seed(int(seed))
    out = []
    for _ in range(3):
        t = torch.randn((B, S, H, D), generator=g, dtype=torch.float32)
        out.append(t.to(dtype).contiguous())
    return tuple(out)


def workload_qkv(w: Workload, seed: int | None = None):
    return make_qkv(w.B, w.S, w.H, w.D, w.dtype, w.seed if seed is None else seed)


# ---------------------------------------------------------------- block masks
# Which (query block, key block) pairs a block-sparse call keeps.  These only
# choose bytes of 0 / 1; what a kept block means is the method's business.
def random_block_mask(n_mask: int, n_qb: int, n_kb: int, density: float, seed: int) -> torch.Tensor:
    """uint8 [n_mask, n_qb, n_kb]: each block on with probability ``density``,
    from a torch CPU generator seeded with ``seed``."""
    g = torch.Generator(device="cpu")
    g.manual_seed(int(seed))
    u = torch.rand((n_mask, n_qb, n_kb), generator=g, dtype=torch.float32)
    return (u < density).to(torch.uint8).contiguous()


def local_global_block_mask(n_qb: int, n_kb: int, block_m: int, block_n: int, local_keys: int,
                            global_kb: int) -> torch.Tensor:
    """uint8 [1, n_qb, n_kb], the long-context pattern of a local band plus a few
    global key blocks: query block r keeps the first ``global_kb`` key blocks
    and every key block that overlaps the ``local_keys`` keys ending at the
    block's last query row (``local_keys`` >= 1)."""
    m = torch.zeros((1, n_qb, n_kb), dtype=torch.uint8)
    m[0, :, :global_kb] = 1
    for r in range(n_qb):
        last = (r + 1) * block_m - 1
        first = max(0, last - local_keys + 1)
        m[0, r, first // block_n: min(n_kb, last // block_n + 1)] = 1
    return m.contiguous()
