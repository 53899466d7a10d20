"""Seeded synthetic workloads shared by the tests, the oracle checks and the bench.

This module holds only shapes and random numbers: none of the attention
arithmetic lives here, so both the GPU path and the CPU oracle can consume the
same inputs without sharing any computation.

Every input is drawn with PyTorch's CPU generator from a fixed seed, as float32
standard normals in the order Q, K, V, dO, multiplied by ``std`` and rounded to
the working dtype by round-to-nearest-even (``Tensor.to``).  The pages measure
only on random Gaussian tensors (claspmoon.cn "14 · 缩放定律与高效注意力" §3.5
and §6), so no dataset stands behind these shapes.
"""

from dataclasses import dataclass, replace
import math

import torch


@dataclass(frozen=True)
class Workload:
    name: str
    B: int
    Hq: int
    Hkv: int
    L: int
    d: int
    dtype: torch.dtype
    causal: bool
    window: int          # 0 = no window; w >= 1: |i - j| < w (keys i-w+1..i with causal)
    seed: int
    std: float = 1.0
    backward: bool = False
    global_tokens: tuple = ()   # positions seen by and seeing every position (negative: from the end)

    @property
    def scale(self) -> float:
        return 1.0 / math.sqrt(self.d)

    def with_(self, **kw) -> "Workload":
        return replace(self, **kw)


# The five workloads of the target, in the order they are listed there.
TINY_FP32 = Workload("tiny-fp32 B1 H2 L256 d64 non-causal", 1, 2, 2, 256, 64,
                     torch.float32, False, 0, seed=0)
LLAMA7B_CAUSAL = Workload("llama7b-layer B2 H32 L4096 d128 causal bf16", 2, 32, 32, 4096, 128,
                          torch.bfloat16, True, 0, seed=1, backward=True)
GQA_16K = Workload("gqa B1 Hq32 Hkv8 L16384 d128 causal bf16", 1, 32, 8, 16384, 128,
                   torch.bfloat16, True, 0, seed=2)
WINDOW_32K = Workload("sliding-window B1 H32 L32768 d128 w4096 bf16", 1, 32, 32, 32768, 128,
                      torch.bfloat16, True, 4096, seed=3, std=0.5)
LONG_FWD_128K = Workload("long-context fwd B1 H32 L131072 d128 causal bf16", 1, 32, 32, 131072, 128,
                         torch.bfloat16, True, 0, seed=4)
LONG_BWD_8K = Workload("long-context bwd B2 H32 L8192 d128 causal bf16", 2, 32, 32, 8192, 128,
                       torch.bfloat16, True, 0, seed=5, backward=True)

ALL = [TINY_FP32, LLAMA7B_CAUSAL, GQA_16K, WINDOW_32K, LONG_FWD_128K, LONG_BWD_8K]

# A general sparse mask: the hybrid configuration of kler.cn §5.1.2 (a window of
# 512 positions before and after each position, i.e. |i - j| < 513, the first
# and last token global, sequences of 131072 tokens, batch 2) on the
# llama7b-shaped heads (32 heads of 128).
# kler.cn §4.1.2's block-sparse pattern at full length: blocks of 128 tokens, each
# query block attending to its own and the two neighbouring key blocks (the
# banded block mask, radius 1), non-causal, on the same heads.
BLOCK_BAND_128K = Workload("block-band B2 H32 L131072 d128 block128 radius1 bf16", 2, 32, 32, 131072, 128,
                           torch.bfloat16, False, 0, seed=7, backward=True)
BLOCK_BAND_BLOCK = 128
BLOCK_BAND_RADIUS = 1

HYBRID_SPARSE_128K = Workload("hybrid-sparse B2 H32 L131072 d128 window513 global[0,-1] bf16", 2, 32, 32, 131072,
                              128, torch.bfloat16, False, 513, seed=6, backward=True, global_tokens=(0, -1))


def block_band_mask(L, block=64, radius=1):
    """The block-sparse pattern of kler.cn §4.1.2 as an input: query block a attends
    to key blocks b with |a - b| <= radius (each block sees itself and its
    neighbours).  A bool CPU tensor ``[nbm, nbm]`` with nbm = ceil(L / block)."""
    nbm = (int(L) + block - 1) // block
    idx = torch.arange(nbm)
    return (idx[:, None] - idx[None, :]).abs() <= int(radius)


def make_inputs(w: Workload, with_dout: bool = None):
    """Seeded CPU tensors ``(q, k, v, dout_or_None)`` for workload ``w``.

    Shapes: q ``[B,Hq,L,d]``, k and v ``[B,Hkv,L,d]``, dout like q.  Values are
    ``std * N(0,1)`` drawn in float32 then rounded to ``w.dtype``.
    """
    if with_dout is None:
        with_dout = w.backward
    g = torch.Generator().manual_seed(w.seed)

    def draw(h):
        x = torch.randn(w.B, h, w.L, w.d, generator=g, dtype=torch.float32)
        if w.std != 1.0:
            x = x * w.std
        return x.to(w.dtype)

    q = draw(w.Hq)
    k = draw(w.Hkv)
    v = draw(w.Hkv)
    do = draw(w.Hq) if with_dout else None
    return q, k, v, do


def small(name, B, Hq, Hkv, L, d, dtype=torch.bfloat16, causal=True, window=0,
          seed=100, std=1.0, backward=False) -> Workload:
    """An ad-hoc workload for parity cases (ragged L, odd heads, ...)."""
    return Workload(name, B, Hq, Hkv, L, d, dtype, causal, window, seed, std, backward)
