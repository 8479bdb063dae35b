"""Seeded synthetic inputs shared by the HIP path's tests/bench and the CPU oracle.

This module only draws numbers and lays them out: it holds none of the
arithmetic of softmax, online softmax or LayerNorm+GeLU.  Every tensor is
generated on the host with a seeded ``torch.Generator`` so that the GPU and the
oracle consume the same bytes.

Recipes (one per named workload; seeds are ``1000 + k``):

* ``tiny_f32_64x768``      x ~ N(0,1) [64,768] fp32; w = 1 + 0.1 N(0,1), b = 0.1 N(0,1)
* ``ln_gelu_f32_4096x768`` same recipe at [4096,768]
* ``softmax_f32_8192x1000`` x = 4 N(0,1) [8192,1000]; rows with i % 16 == 0 get +1000
* ``online_f32_64x262144`` x = 3 N(0,1) [64,262144]
* ``bf16_16384x4096``      x = bf16(N(0,1)) [16384,4096]; softmax input 8 x (exact in
  bf16); w, b as above rounded to bf16
* ``ln_long_f32_64x262144`` LayerNorm on rows too long for registers: x = N(0,1)
  [64,262144] fp32, rows i % 8 == 0 get +100 (a mean far from zero, where
  one-pass E[x^2] - E[x]^2 in fp32 would lose the variance); w, b as above

Draw order is always x, then w, then b.  bf16 values are produced by torch's
round-to-nearest-even cast of the fp32 draw.

Attention inputs (``attention_qkv``): q, k, v ~ N(0,1) of shape [B, H, T, d],
drawn in that order in fp32 and rounded to bf16 or fp16, seed given; the
pages benchmark B = 4, H = 32, d = 128, T = 128 ... 4096 in fp16.

RMSNorm runs on the same workloads: its input is ``x``, its weight ``w``; the
fused residual variant adds ``residual(name)``, an independent N(0,1) draw of
the workload's shape and dtype from seed ``seed + 100``.
"""
from __future__ import annotations

from dataclasses import dataclass

import torch

__all__ = ["Workload", "WORKLOADS", "make", "randn", "ln_params", "bf16_round", "residual",
           "attention_qkv"]


@dataclass(frozen=True)
class Workload:
    name: str
    seed: int
    M: int
    N: int
    dtype: torch.dtype
    ops: tuple  # which entry points the workload feeds
    x_scale: float = 1.0
    softmax_scale: float = 1.0  # extra scale applied to x for the softmax input
    offset_every: int = 0  # rows i % offset_every == 0 get +offset (0 = none)
    offset: float = 0.0


WORKLOADS = {
    "tiny_f32_64x768": Workload("tiny_f32_64x768", 1001, 64, 768, torch.float32,
                                ("softmax", "layernorm_gelu")),
    "ln_gelu_f32_4096x768": Workload("ln_gelu_f32_4096x768", 1002, 4096, 768, torch.float32,
                                     ("layernorm_gelu",)),
    "softmax_f32_8192x1000": Workload("softmax_f32_8192x1000", 1003, 8192, 1000, torch.float32,
                                      ("softmax",), x_scale=4.0, offset_every=16, offset=1000.0),
    "online_f32_64x262144": Workload("online_f32_64x262144", 1004, 64, 262144, torch.float32,
                                     ("online_softmax",), x_scale=3.0),
    "bf16_16384x4096": Workload("bf16_16384x4096", 1005, 16384, 4096, torch.bfloat16,
                                ("softmax", "layernorm_gelu"), softmax_scale=8.0),
    "ln_long_f32_64x262144": Workload("ln_long_f32_64x262144", 1006, 64, 262144, torch.float32,
                                      ("layernorm_gelu",), offset_every=8, offset=100.0),
}


def _gen(seed: int) -> torch.Generator:
    g = torch.Generator(device="cpu")
    g.manual_seed(int(seed))
    return g


def randn(M: int, N: int, seed: int, scale: float = 1.0, dtype=torch.float32,
          gen: torch.Generator | None = None) -> torch.Tensor:
    """``scale * N(0,1)`` of shape [M, N], drawn in fp32 and cast to ``dtype``."""
    g = gen if gen is not None else _gen(seed)
    x = torch.randn((M, N), generator=g, dtype=torch.float32)
    if scale != 1.0:
        x = x * scale
    return x.to(dtype)


def ln_params(N: int, gen: torch.Generator, dtype=torch.float32):
    """w = 1 + 0.1 N(0,1), b = 0.1 N(0,1), each [N], drawn w first."""
    w = 1.0 + 0.1 * torch.randn((N,), generator=gen, dtype=torch.float32)
    b = 0.1 * torch.randn((N,), generator=gen, dtype=torch.float32)
    return w.to(dtype), b.to(dtype)


def bf16_round(t: torch.Tensor) -> torch.Tensor:
    return t.to(torch.bfloat16)


def make(name: str, rows: int | None = None) -> dict:
    """Host tensors of a named workload.

    Returns a dict with ``x`` (LayerNorm input / base draw), ``x_softmax`` (the
    softmax input), and ``w``, ``b`` for LayerNorm.  ``rows`` truncates M (the
    first rows of the same draw), used for bounded CPU samples.
    """
    wl = WORKLOADS[name]
    g = _gen(wl.seed)
    base = torch.randn((wl.M, wl.N), generator=g, dtype=torch.float32)
    w, b = ln_params(wl.N, g, wl.dtype)
    if wl.x_scale != 1.0:
        base = base * wl.x_scale
    if wl.offset_every:
        base[:: wl.offset_every] += wl.offset
    x = base.to(wl.dtype)
    if wl.softmax_scale != 1.0:
        # Scaling by a power of two is exact in bf16 and fp32.
        xs = (x.float() * wl.softmax_scale).to(wl.dtype)
    else:
        xs = x
    if rows is not None:
        x, xs = x[:rows].contiguous(), xs[:rows].contiguous()
    return {"x": x, "x_softmax": xs, "w": w, "b": b, "workload": wl}


def residual(name: str, rows: int | None = None) -> torch.Tensor:
    """The residual-stream input paired with workload ``name``'s x: N(0,1) of
    the same shape and dtype, seed ``seed + 100`` (first ``rows`` rows if given)."""
    wl = WORKLOADS[name]
    r = randn(wl.M, wl.N, seed=wl.seed + 100, dtype=wl.dtype)
    return r if rows is None else r[:rows].contiguous()


def attention_qkv(B: int, H: int, T: int, d: int, dtype=torch.bfloat16, seed: int = 2001):
    """q, k, v ~ N(0,1) [B, H, T, d], drawn q, k, v in fp32, cast to dtype."""
    g = _gen(seed)
    return tuple(torch.randn((B, H, T, d), generator=g, dtype=torch.float32).to(dtype)
                 for _ in range(3))
