"""Seeded synthetic inputs for the KDA forward workloads.

This module only draws random numbers and lays them out; it holds none of the
method's arithmetic (no convolution, no recurrence).  Both the GPU path and the
oracle consume what it returns, so the two sides always see identical values.

Recipe (all draws from ``torch.Generator(device).manual_seed(seed)``, float32
normal/uniform draws, then rounded once, round-to-nearest-even, to the storage
dtype; "N(0, s)" means standard deviation s):

* raw q/k/v projections    N(0, 1)                       bf16   [T, H*D]
* short-conv weights       N(0, 0.5)                     bf16   [H*D, 4]
* log-decay g              lb * sigmoid(N(0, gate_std))  fp32   [T, H, D]
  (lb = -5, gate_std = 1 for the standard workloads; lb = -8, gate_std = 2 for the
  long-context stress workload)
* beta                     sigmoid(N(0, 1))              fp32   [T, H]
* initial state            N(0, 0.05)                    fp32   [N, H, D, D]
* pre-processed q/k        N(0, 1) scaled to unit L2 length per (token, head)
  (the decode and tiny workloads feed the recurrence directly)
* fused-gate inputs (make_gate, seed + 1000): pre-activation z N(0, gate_std) in
  the activation dtype [T, H, D], A_log N(0, 0.3) fp32 [H], dt_bias N(0, 0.5)
  fp32 [H, D]
* output-epilogue inputs (make_epilogue, seed + 2000): output-gate pre-activation
  N(0, 1) in the activation dtype [T, H, DV], norm weight 1 + N(0, 0.1) fp32 [DV]
* per-head decay for the GDN variant (make_head_gate, seed + 4000): lb * sigmoid(N(0,
  gate_std)) fp32 [T, H] (decode: [B, H] per step, make_decode_step's generator)
* decode with the conv (make_decode_conv, seed + 3000): conv weights N(0, 0.5) and
  initial conv caches N(0, 1) (raw inputs) in the activation dtype; per step
  (make_decode_conv_step) raw projections N(0, 1) and g, beta as above

The pages' own workloads are a Kimi-K3 KDA layer: 96 heads of 128x128 state,
width-4 short conv, gate floor -5; they publish no dataset or benchmark inputs.
"""
from __future__ import annotations

from dataclasses import dataclass, field
from typing import Dict, List, Optional

import torch

# Packed sequence lengths of the variable-length prefill workload.
VARLEN_LENGTHS = [512, 1024, 2048, 3072, 4096, 6144, 7680, 8192]


@dataclass
class PrefillSpec:
    name: str
    lengths: List[int]
    heads: int = 96
    dk: int = 128
    dv: int = 128
    chunk: int = 64
    dtype: torch.dtype = torch.bfloat16
    conv: bool = True              # raw projections pass through conv4 + SiLU (+ q/k L2)
    gate_lb: float = -5.0
    gate_std: float = 1.0
    h0_std: Optional[float] = None  # None: zero initial state
    scale: Optional[float] = None   # None: dk ** -0.5
    seed: int = 0

    @property
    def total_tokens(self) -> int:
        return int(sum(self.lengths))

    @property
    def read_scale(self) -> float:
        return self.dk ** -0.5 if self.scale is None else float(self.scale)


@dataclass
class DecodeSpec:
    name: str
    batch: int = 64
    heads: int = 96
    dk: int = 128
    dv: int = 128
    steps: int = 256
    dtype: torch.dtype = torch.bfloat16
    gate_lb: float = -5.0
    state_std: float = 0.05
    seed: int = 3


def standard_specs() -> Dict[str, object]:
    """The five workloads: tiny fp32 check, prefill, decode, varlen, long context."""
    return {
        "tiny_fp32": PrefillSpec("tiny_fp32 B=1 H=1 T=64 d=16 chunk=16 fp32", [64], heads=1, dk=16,
                                 dv=16, chunk=16, dtype=torch.float32, conv=False, scale=1.0,
                                 seed=1),
        "prefill": PrefillSpec("prefill B=1 T=4096 H=96 d=128 bf16", [4096], seed=2),
        "decode": DecodeSpec("decode 64 seq x H=96 d=128, 256 steps bf16"),
        "varlen": PrefillSpec("varlen 8 seq T=32768 H=96 d=128 bf16 h0", list(VARLEN_LENGTHS),
                              h0_std=0.05, seed=4),
        "long": PrefillSpec("long B=1 T=131072 H=96 d=128 bf16 g>=-8", [131072], gate_lb=-8.0,
                            gate_std=2.0, seed=5),
    }


def _gen(device, seed: int) -> torch.Generator:
    gen = torch.Generator(device=device)
    gen.manual_seed(int(seed))
    return gen


def _normal(shape, gen, device, std=1.0):
    x = torch.randn(shape, generator=gen, device=device, dtype=torch.float32)
    return x * std if std != 1.0 else x


def _unit_rows(x: torch.Tensor) -> torch.Tensor:
    """Scale each last-axis vector to unit Euclidean length (fp64 intermediate)."""
    xd = x.double()
    return (xd / xd.norm(dim=-1, keepdim=True)).to(x.dtype)


def cu_seqlens_of(lengths: List[int]) -> List[int]:
    out = [0]
    for L in lengths:
        out.append(out[-1] + int(L))
    return out


def make_prefill(spec: PrefillSpec, device="cpu") -> Dict[str, torch.Tensor]:
    """Inputs of one prefill call.

    Returns raw projections ``q_raw, k_raw, v_raw`` [T, H*D] and conv weights
    ``w_q, w_k, w_v`` [H*D, 4] when ``spec.conv``; otherwise ready ``q, k, v``
    [T, H, D] (q, k unit-length).  Always ``g`` [T, H, DK] fp32, ``beta`` [T, H]
    fp32, ``cu_seqlens`` int32 [N+1] and ``h0`` [N, H, DK, DV] fp32 or None.
    """
    gen = _gen(device, spec.seed)
    T, H, DK, DV = spec.total_tokens, spec.heads, spec.dk, spec.dv
    out: Dict[str, torch.Tensor] = {}
    if spec.conv:
        out["q_raw"] = _normal((T, H * DK), gen, device).to(spec.dtype)
        out["k_raw"] = _normal((T, H * DK), gen, device).to(spec.dtype)
        out["v_raw"] = _normal((T, H * DV), gen, device).to(spec.dtype)
        out["w_q"] = _normal((H * DK, 4), gen, device, 0.5).to(spec.dtype)
        out["w_k"] = _normal((H * DK, 4), gen, device, 0.5).to(spec.dtype)
        out["w_v"] = _normal((H * DV, 4), gen, device, 0.5).to(spec.dtype)
    else:
        out["q"] = _unit_rows(_normal((T, H, DK), gen, device)).to(spec.dtype)
        out["k"] = _unit_rows(_normal((T, H, DK), gen, device)).to(spec.dtype)
        out["v"] = _normal((T, H, DV), gen, device).to(spec.dtype)
    z = _normal((T, H, DK), gen, device, spec.gate_std)
    out["g"] = (spec.gate_lb * torch.sigmoid(z)).float()
    out["beta"] = torch.sigmoid(_normal((T, H), gen, device)).float()
    N = len(spec.lengths)
    out["h0"] = (None if spec.h0_std is None
                 else _normal((N, H, DK, DV), gen, device, spec.h0_std).float())
    out["cu_seqlens"] = torch.tensor(cu_seqlens_of(spec.lengths), dtype=torch.int32,
                                     device=device)
    return out


def make_head_gate(spec: PrefillSpec, device="cpu") -> torch.Tensor:
    """One log-decay per (token, head) for the GDN variant: g [T, H] fp32 (own seed)."""
    gen = _gen(device, spec.seed + 4000)
    z = _normal((spec.total_tokens, spec.heads), gen, device, spec.gate_std)
    return (spec.gate_lb * torch.sigmoid(z)).float()


def make_epilogue(spec: PrefillSpec, device="cpu") -> Dict[str, torch.Tensor]:
    """Inputs of the output epilogue for the same call: the output gate's
    pre-activation ``gate`` [T, H, DV] (activation dtype) and the norm ``weight``
    [DV] fp32 (own seed)."""
    gen = _gen(device, spec.seed + 2000)
    T, H, DV = spec.total_tokens, spec.heads, spec.dv
    return {
        "gate": _normal((T, H, DV), gen, device).to(spec.dtype),
        "weight": (1.0 + _normal((DV,), gen, device, 0.1)).float(),
    }


def make_gate(spec: PrefillSpec, device="cpu") -> Dict[str, torch.Tensor]:
    """Inputs of the fused bounded gate for the same call: ``z`` [T, H, DK] in the
    activation dtype, ``a_log`` [H] and ``dt_bias`` [H, DK] fp32 (own seed)."""
    gen = _gen(device, spec.seed + 1000)
    T, H, DK = spec.total_tokens, spec.heads, spec.dk
    return {
        "z": _normal((T, H, DK), gen, device, spec.gate_std).to(spec.dtype),
        "a_log": _normal((H,), gen, device, 0.3).float(),
        "dt_bias": _normal((H, DK), gen, device, 0.5).float(),
    }


def make_decode_conv(spec: DecodeSpec, device="cpu") -> Dict[str, torch.Tensor]:
    """Conv weights ``w_q, w_k, w_v`` [H*D, 4] and initial conv caches ``conv_q,
    conv_k, conv_v`` [B, 3, H*D] (the last three raw inputs) of a decode batch."""
    gen = _gen(device, spec.seed + 3000)
    B, H, DK, DV = spec.batch, spec.heads, spec.dk, spec.dv
    out = {}
    for name, D in (("q", DK), ("k", DK), ("v", DV)):
        out["w_" + name] = _normal((H * D, 4), gen, device, 0.5).to(spec.dtype)
    for name, D in (("q", DK), ("k", DK), ("v", DV)):
        out["conv_" + name] = _normal((B, 3, H * D), gen, device).to(spec.dtype)
    return out


def make_decode_conv_step(spec: DecodeSpec, step: int, device="cpu") -> Dict[str, torch.Tensor]:
    """Inputs of fused decode step ``step``: raw projections ``q_raw, k_raw`` [B, H*DK],
    ``v_raw`` [B, H*DV] (before the conv), ``g`` [B, H, DK] and ``beta`` [B, H]."""
    gen = _gen(device, (spec.seed + 3000) * 1_000_003 + 7919 * (step + 1))
    B, H, DK, DV = spec.batch, spec.heads, spec.dk, spec.dv
    return {
        "q_raw": _normal((B, H * DK), gen, device).to(spec.dtype),
        "k_raw": _normal((B, H * DK), gen, device).to(spec.dtype),
        "v_raw": _normal((B, H * DV), gen, device).to(spec.dtype),
        "g": (spec.gate_lb * torch.sigmoid(_normal((B, H, DK), gen, device))).float(),
        "beta": torch.sigmoid(_normal((B, H), gen, device)).float(),
    }


def make_decode_state(spec: DecodeSpec, device="cpu") -> torch.Tensor:
    gen = _gen(device, spec.seed)
    return _normal((spec.batch, spec.heads, spec.dk, spec.dv), gen, device,
                   spec.state_std).float()


def make_decode_step(spec: DecodeSpec, step: int, device="cpu") -> Dict[str, torch.Tensor]:
    """Inputs of decode step ``step``: one token per sequence, already conv-processed."""
    gen = _gen(device, spec.seed * 1_000_003 + 7919 * (step + 1))
    B, H, DK, DV = spec.batch, spec.heads, spec.dk, spec.dv
    return {
        "q": _unit_rows(_normal((B, H, DK), gen, device)).to(spec.dtype),
        "k": _unit_rows(_normal((B, H, DK), gen, device)).to(spec.dtype),
        "v": _normal((B, H, DV), gen, device).to(spec.dtype),
        "g": (spec.gate_lb * torch.sigmoid(_normal((B, H, DK), gen, device))).float(),
        "beta": torch.sigmoid(_normal((B, H), gen, device)).float(),
    }
