"""Seeded synthetic inputs for the Wall Attention forward workloads.

This module only draws random tensors; it holds none of the method's
arithmetic.  Both the fp64 oracle (through the tests) and the HIP path
(through the tests and the benchmark) take their inputs from here, so the two
sides always see the same numbers.

Recipe (one per workload):

* ``numpy.random.default_rng(seed)`` (PCG64) draws every value in float64 with
  ``standard_normal`` / ``uniform``, always in the order
  ``[segment lengths], q, k, v, x_g, x_gs, sink``.
* Gate inputs are transformed in float64: ``0.02 * x`` for the small
  random-walk gates of the README usage example, ``log(sigmoid(x))`` (computed
  as ``-logaddexp(0, -x)``) for the forgetting gates.
* Every tensor is then cast to the workload dtype by torch (round to nearest
  even).  The oracle receives these cast tensors upcast to float64.

The five named workloads mirror the shapes of the Wall Attention README usage
example (GQA, B=2, T=1024, HQ=8, H=4, K=V=64) and of the long-context,
options and varlen cases.  The long-context gate is bimodal (slow channels
0..63 from N(4,1), fast channels 64..127 from N(0,1) through log-sigmoid),
after the blog's observation that trained models split their channels into
static and fast-forgetting groups ("Bimodal channels" section).
"""

from __future__ import annotations

import dataclasses
from typing import Optional

import numpy as np
import torch

__all__ = ["WORKLOADS", "DECODE_WORKLOADS", "Workload", "WallInputs", "DecodeInputs", "make_inputs",
           "make_decode_inputs", "workload"]


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    seed: int
    B: int
    T: int
    HQ: int
    H: int
    K: int
    V: int
    dtype: str  # "float32" | "bfloat16"
    gate: str  # "small" | "bimodal" | "logsig4"
    window: Optional[int] = None
    g_scalar: bool = False
    sink: bool = False
    nseq: Optional[int] = None  # varlen packing (B must be 1)


WORKLOADS = {
    w.name: w
    for w in [
        Workload("tiny_fp32", 1, 1, 128, 1, 1, 64, 64, "float32", "small"),
        Workload("gqa_bf16", 2, 2, 1024, 8, 4, 64, 64, "bfloat16", "small"),
        Workload("long_bf16", 3, 1, 8192, 16, 4, 128, 128, "bfloat16", "bimodal"),
        Workload("options_bf16", 4, 4, 4096, 32, 8, 128, 128, "bfloat16", "logsig4",
                 window=1024, g_scalar=True, sink=True),
        Workload("varlen_bf16", 5, 1, 32768, 32, 8, 128, 128, "bfloat16", "logsig4",
                 nseq=8),
    ]
}


# Decode: one new token per sequence against a cache of T rows (the newest
# token's row included), the README's decode example at the long-context
# shapes with a batch of 16 sequences.
DECODE_WORKLOADS = {
    w.name: w
    for w in [
        Workload("decode_bf16", 6, 16, 8192, 16, 4, 128, 128, "bfloat16", "bimodal"),
    ]
}


def workload(name: str, **overrides) -> Workload:
    """The named workload, optionally with some fields replaced (e.g. a shorter T)."""
    table = DECODE_WORKLOADS if name in DECODE_WORKLOADS else WORKLOADS
    return dataclasses.replace(table[name], **overrides)


@dataclasses.dataclass
class WallInputs:
    q: torch.Tensor  # [B, T, HQ, K]
    k: torch.Tensor  # [B, T, H, K]
    v: torch.Tensor  # [B, T, H, V]
    g: torch.Tensor  # [B, T, HQ, K] natural-log gate
    g_scalar: Optional[torch.Tensor]  # [B, T, HQ]
    sink_bias: Optional[torch.Tensor]  # [HQ] float32
    cu_seqlens: Optional[torch.Tensor]  # [N+1] int32
    window_size: Optional[int]
    scale: float
    spec: Workload

    def to(self, device) -> "WallInputs":
        mv = lambda t: None if t is None else t.to(device)
        return dataclasses.replace(
            self, q=mv(self.q), k=mv(self.k), v=mv(self.v), g=mv(self.g),
            g_scalar=mv(self.g_scalar), sink_bias=mv(self.sink_bias),
            cu_seqlens=mv(self.cu_seqlens))


def _logsigmoid(x: np.ndarray) -> np.ndarray:
    return -np.logaddexp(0.0, -x)


def varlen_lengths(rng: np.random.Generator, total: int, nseq: int,
                   lo: float = 512.0, hi: float = 8192.0) -> np.ndarray:
    """Segment lengths uniform in [lo, hi), rescaled so they add up to ``total``."""
    u = rng.uniform(lo, hi, size=nseq)
    lens = np.floor(u * total / u.sum()).astype(np.int64)
    lens[-1] += total - lens.sum()
    return lens


def make_inputs(spec: Workload | str, **overrides) -> WallInputs:
    """Draw the inputs of one workload on the CPU (see the module docstring)."""
    if isinstance(spec, str):
        spec = workload(spec, **overrides)
    elif overrides:
        spec = dataclasses.replace(spec, **overrides)
    rng = np.random.default_rng(spec.seed)
    B, T, HQ, H, K, V = spec.B, spec.T, spec.HQ, spec.H, spec.K, spec.V
    dt = {"float32": torch.float32, "bfloat16": torch.bfloat16}[spec.dtype]

    cu = None
    if spec.nseq is not None:
        assert B == 1, "varlen packing needs B == 1"
        lens = varlen_lengths(rng, T, spec.nseq)
        cu = torch.tensor(np.concatenate([[0], np.cumsum(lens)]), dtype=torch.int32)

    def draw(shape):
        return rng.standard_normal(size=shape)

    q = draw((B, T, HQ, K))
    k = draw((B, T, H, K))
    v = draw((B, T, H, V))
    x_g = draw((B, T, HQ, K))
    if spec.gate == "small":
        g = 0.02 * x_g
    elif spec.gate == "bimodal":
        x_g[..., : K // 2] += 4.0  # slow channels: x ~ N(4, 1)
        g = _logsigmoid(x_g)  # fast channels keep x ~ N(0, 1)
    elif spec.gate == "logsig4":
        g = _logsigmoid(x_g + 4.0)
    else:
        raise ValueError(spec.gate)
    gs = None
    if spec.g_scalar:
        gs = _logsigmoid(draw((B, T, HQ)) + 3.0)
    sink = None
    if spec.sink:
        sink = torch.from_numpy(draw((HQ,))).to(torch.float32)

    cast = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(dt)
    return WallInputs(
        q=cast(q), k=cast(k), v=cast(v), g=cast(g),
        g_scalar=None if gs is None else cast(gs),
        sink_bias=sink, cu_seqlens=cu, window_size=spec.window,
        scale=float(K) ** -0.5, spec=spec)


@dataclasses.dataclass
class DecodeInputs:
    q: torch.Tensor  # [B, 1, HQ, K] the newest token of each sequence
    k: torch.Tensor  # [B, T, H, K]
    v: torch.Tensor  # [B, T, H, V]
    g: torch.Tensor  # [B, T, HQ, K] natural-log gate
    sink_bias: Optional[torch.Tensor]  # [HQ] float32
    scale: float
    chunk_size: int
    spec: Workload

    def to(self, device) -> "DecodeInputs":
        mv = lambda t: None if t is None else t.to(device)
        return dataclasses.replace(self, q=mv(self.q), k=mv(self.k), v=mv(self.v), g=mv(self.g),
                                   sink_bias=mv(self.sink_bias))


def make_decode_inputs(spec: Workload | str, chunk_size: int = 64, **overrides) -> DecodeInputs:
    """Draw the inputs of one decode workload on the CPU: the same recipe as
    make_inputs, drawn one sequence at a time (q of the newest token, then k,
    v, x_g of all T rows) so that host memory stays bounded, then the sink."""
    if isinstance(spec, str):
        spec = workload(spec, **overrides)
    elif overrides:
        spec = dataclasses.replace(spec, **overrides)
    rng = np.random.default_rng(spec.seed)
    B, T, HQ, H, K, V = spec.B, spec.T, spec.HQ, spec.H, spec.K, spec.V
    dt = {"float32": torch.float32, "bfloat16": torch.bfloat16}[spec.dtype]
    cast = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(dt)
    q = torch.empty((B, 1, HQ, K), dtype=dt)
    k = torch.empty((B, T, H, K), dtype=dt)
    v = torch.empty((B, T, H, V), dtype=dt)
    g = torch.empty((B, T, HQ, K), dtype=dt)
    for b in range(B):
        q[b] = cast(rng.standard_normal(size=(1, HQ, K)))
        k[b] = cast(rng.standard_normal(size=(T, H, K)))
        v[b] = cast(rng.standard_normal(size=(T, H, V)))
        x_g = rng.standard_normal(size=(T, HQ, K))
        if spec.gate == "small":
            gb = 0.02 * x_g
        elif spec.gate == "bimodal":
            x_g[..., : K // 2] += 4.0
            gb = _logsigmoid(x_g)
        elif spec.gate == "logsig4":
            gb = _logsigmoid(x_g + 4.0)
        else:
            raise ValueError(spec.gate)
        g[b] = cast(gb)
    sink = torch.from_numpy(rng.standard_normal(size=(HQ,))).to(torch.float32) if spec.sink else None
    return DecodeInputs(q=q, k=k, v=v, g=g, sink_bias=sink, scale=float(K) ** -0.5,
                        chunk_size=int(chunk_size), spec=spec)
