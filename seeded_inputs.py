"""Seeded synthetic inputs and the five workload definitions.

This module is shared by the oracle side (tests, the CPU baseline) and the
GPU side (tests, bench).  It holds no attention arithmetic: only the shapes
and parameters of the workloads and a deterministic bf16 N(0,1) generator.

Generator recipe (identical bits on every machine, independent of the number
of threads):
  * a tensor is drawn as a flat vector split into chunks of 2**22 values;
  * chunk ``i`` of tensor ``stream`` (0 = q, 1 = k, 2 = v) uses
    ``torch.Generator('cpu').manual_seed(seed * 1_000_003 + stream * 65_537 + i)``
    and ``torch.randn(n, dtype=float32)``;
  * the fp32 values are rounded to bfloat16 (round-to-nearest-even).
Chunks are drawn in a thread pool; torch releases the GIL inside randn.
"""
from __future__ import annotations

import concurrent.futures as _cf
import os
from dataclasses import dataclass, field
from typing import List, Optional, Tuple

import torch

CHUNK = 1 << 22


def _chunk(seed: int, stream: int, i: int, n: int) -> torch.Tensor:
    g = torch.Generator(device="cpu").manual_seed(seed * 1_000_003 + stream * 65_537 + i)
    return torch.randn(n, generator=g, dtype=torch.float32).to(torch.bfloat16)


def randn_bf16(shape, seed: int, stream: int, threads: Optional[int] = None) -> torch.Tensor:
    """bf16 tensor of i.i.d. N(0,1) values, deterministic in (seed, stream)."""
    numel = 1
    for s in shape:
        numel *= int(s)
    out = torch.empty(numel, dtype=torch.bfloat16)
    nchunks = (numel + CHUNK - 1) // CHUNK
    if nchunks == 0:
        return out.view(*shape)
    threads = threads or min(16, os.cpu_count() or 1)

    def work(i):
        lo = i * CHUNK
        hi = min(numel, lo + CHUNK)
        out[lo:hi] = _chunk(seed, stream, i, hi - lo)

    if nchunks == 1 or threads == 1:
        for i in range(nchunks):
            work(i)
    else:
        with _cf.ThreadPoolExecutor(max_workers=threads) as ex:
            list(ex.map(work, range(nchunks)))
    return out.view(*shape)


@dataclass
class Workload:
    """One attention workload.  ``q`` is [B,S,Hq,D] (varlen: [T,Hq,D])."""
    name: str
    B: int
    S: int
    Hq: int
    Hkv: int
    D: int
    impl: str                 # "basic" | "zigzag" | "stripe"
    ring_degree: int
    ulysses_degree: int = 1
    stripe_block: int = 1
    causal: bool = False
    window: int = 0           # 0 = no window; else number of keys incl. self
    n_sink: int = 0
    cu_seqlens: Optional[List[int]] = None   # varlen (then B == 1 and q is [T,H,D])
    softmax_scale: Optional[float] = None    # None = 1/sqrt(D)
    rank: int = -1            # -1 = every virtual rank; >=0 = that ring rank's share
    ulysses_rank: int = 0
    seed: int = 1000

    @property
    def varlen(self) -> bool:
        return self.cu_seqlens is not None

    @property
    def scale(self) -> float:
        return self.softmax_scale if self.softmax_scale is not None else self.D ** -0.5

    def q_shape(self) -> Tuple[int, ...]:
        return (self.S, self.Hq, self.D) if self.varlen else (self.B, self.S, self.Hq, self.D)

    def kv_shape(self) -> Tuple[int, ...]:
        return (self.S, self.Hkv, self.D) if self.varlen else (self.B, self.S, self.Hkv, self.D)

    def make_inputs(self, threads: Optional[int] = None):
        """(q, k, v) as CPU bf16 tensors in natural (unpermuted) order."""
        q = randn_bf16(self.q_shape(), self.seed, 0, threads)
        k = randn_bf16(self.kv_shape(), self.seed, 1, threads)
        v = randn_bf16(self.kv_shape(), self.seed, 2, threads)
        return q, k, v

    def scaled(self, **kw) -> "Workload":
        d = dict(self.__dict__)
        d.update(kw)
        return Workload(**d)


# The five workloads.  Shapes follow the ring sliding-window README examples
# (B=2, S=8192, 32 heads, D=128, window 1000; cu_seqlens [0,512,4000,8192])
# and the USP README's hybrid split (ulysses 2 x ring 4).
WORKLOADS = {
    "zigzag_causal_small": Workload(
        name="zigzag_causal_small", B=1, S=1024, Hq=4, Hkv=4, D=64, impl="zigzag",
        ring_degree=4, causal=True, softmax_scale=1.0 / 8.0, seed=1000),
    "ring_swa": Workload(
        name="ring_swa", B=2, S=8192, Hq=32, Hkv=32, D=128, impl="basic",
        ring_degree=8, window=1000, seed=1001),
    "varlen_streaming": Workload(
        name="varlen_streaming", B=1, S=8192, Hq=32, Hkv=32, D=128, impl="basic",
        ring_degree=4, window=1000, n_sink=4, cu_seqlens=[0, 512, 4000, 8192], seed=1002),
    "usp_zigzag_gqa": Workload(
        name="usp_zigzag_gqa", B=1, S=131072, Hq=32, Hkv=8, D=128, impl="zigzag",
        ring_degree=4, ulysses_degree=2, causal=True, rank=0, ulysses_rank=0, seed=1003),
    "stripe_mqa": Workload(
        name="stripe_mqa", B=1, S=1048576, Hq=8, Hkv=1, D=128, impl="stripe",
        ring_degree=8, stripe_block=1, causal=True, rank=0, seed=1004),
}

WORKLOAD_ORDER = ["zigzag_causal_small", "ring_swa", "varlen_streaming",
                  "usp_zigzag_gqa", "stripe_mqa"]
