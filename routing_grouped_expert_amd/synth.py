"""Seeded synthetic MoE-layer inputs.

This module only draws random tensors and lays them out; it holds none of the
layer's arithmetic (no top-k, no softmax, no activation, no GEMM).  Both the
CPU oracle tests and the HIP path take their inputs from here, so the two sides
see identical bits.

Recipe (one ``torch.Generator('cpu')`` per layer, seeded; every draw is fp32 and
then rounded to the layer dtype with torch's round-to-nearest-even cast):

1. router logits ``[N, E]`` ~ N(0, 1)
2. activations ``x [N, H]`` ~ N(0, 1)
3. gated layers: ``gate [E, I, H]`` then ``up [E, I, H]`` ~ N(0, sigma13);
   non-gated (ReLU^2): ``up [E, I, H]`` only
4. ``w2 [E, H, I]`` ~ N(0, sigma2)
5. skewed layers only: ``perm = randperm(E)`` and a per-expert logit bias
   ``-s * ln(perm[e] + 1)`` (a Zipf(s) prior in log space over a seeded rank
   permutation), added to the logits before rounding.

Expert-parallel share layers (``n_local`` set) draw the logits over all E
experts and the weights (steps 3-4) for their ``n_local`` experts only: one
GPU's share [local_offset, local_offset + n_local) of a layer.

``w13`` is built from the same gate/up draws in either layout: packed rows
``[gate; up]`` or interleaved rows ``[g0, u0, g1, u1, ...]``, the two gated
layouts described in the vLLM PR #47106 report (section on the w13 reorder
helper).  Building both from one draw makes layout invariance testable.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field, replace
from typing import Optional

import torch

DTYPES = {"f32": torch.float32, "bf16": torch.bfloat16}


@dataclass(frozen=True)
class LayerSpec:
    """Shape and numerics of one synthetic MoE layer."""

    name: str
    n_tokens: int
    hidden: int
    inter: int
    n_experts: int
    topk: int
    dtype: str = "bf16"            # "f32" or "bf16": x, weights, logits, outputs
    act: str = "silu"              # "silu" | "swiglu_oai" | "relu2"
    layout: str = "packed"         # "packed" | "interleaved" (gated acts only)
    sigma13: Optional[float] = None  # None -> 1/sqrt(hidden)
    sigma2: Optional[float] = None   # None -> 1/sqrt(inter)
    alpha: Optional[float] = None
    beta: Optional[float] = None
    limit: Optional[float] = None
    zipf_s: Optional[float] = None   # skewed logit bias strength
    seed: int = 0
    local_offset: int = 0            # expert-parallel share: first local expert
    n_local: Optional[int] = None    # share size; None -> the whole layer

    @property
    def n_weights(self) -> int:
        """Experts whose weights this GPU holds."""
        return self.n_experts if self.n_local is None else self.n_local

    @property
    def gated(self) -> bool:
        return self.act != "relu2"

    @property
    def w13_rows(self) -> int:
        return (2 if self.gated else 1) * self.inter

    def with_(self, **kw) -> "LayerSpec":
        return replace(self, **kw)


def _cfg_tiny() -> LayerSpec:
    return LayerSpec("tiny_f32", n_tokens=33, hidden=128, inter=256, n_experts=8, topk=2,
                     dtype="f32", act="silu", layout="packed")


def _cfg_minimind(n_experts: int = 8) -> LayerSpec:
    return LayerSpec(f"minimind_e{n_experts}", n_tokens=8 * 512, hidden=512, inter=1408,
                     n_experts=n_experts, topk=1, dtype="bf16", act="silu", layout="packed")


def _cfg_gptoss(n_tokens: int = 4096) -> LayerSpec:
    return LayerSpec(f"gptoss_n{n_tokens}", n_tokens=n_tokens, hidden=2880, inter=2880,
                     n_experts=128, topk=4, dtype="bf16", act="swiglu_oai",
                     layout="interleaved", sigma13=0.02, sigma2=0.02,
                     alpha=1.702, beta=1.0, limit=7.0)


def _cfg_skewed(act: str = "silu") -> LayerSpec:
    return LayerSpec(f"skewed_{act}", n_tokens=16384, hidden=4096, inter=1536, n_experts=64,
                     topk=8, dtype="bf16", act=act, layout="packed", zipf_s=1.1)


def layer_spec(family: str, **overrides) -> LayerSpec:
    """Named workloads: tiny_f32, minimind, gptoss, skewed; ``overrides`` replace
    fields of the family's default spec (n_tokens, n_experts, act, name, ...)."""
    base = {
        "tiny_f32": _cfg_tiny,
        "minimind": _cfg_minimind,
        "gptoss": _cfg_gptoss,
        "skewed": _cfg_skewed,
    }[family]()
    return base.with_(**overrides) if overrides else base


# Routing-only sweep: (n_tokens, n_experts, topk), bf16 logits.
ROUTING_SWEEP = [(n, e, k) for n in (1, 33, 512, 16384, 65536) for (e, k) in ((32, 4), (128, 4))]


def _std(v: Optional[float], fan_in: int) -> float:
    return v if v is not None else 1.0 / math.sqrt(fan_in)


def draw_logits(gen: torch.Generator, n_tokens: int, n_experts: int) -> torch.Tensor:
    return torch.randn(n_tokens, n_experts, generator=gen, dtype=torch.float32)


def zipf_bias(gen: torch.Generator, n_experts: int, s: float) -> torch.Tensor:
    """Per-expert additive logit bias -s*ln(rank+1) over a seeded rank permutation."""
    perm = torch.randperm(n_experts, generator=gen)
    return -s * torch.log(perm.to(torch.float32) + 1.0)


def routing_logits(n_tokens: int, n_experts: int, dtype: str = "bf16", seed: int = 0,
                   zipf_s: Optional[float] = None) -> torch.Tensor:
    """Gaussian router logits on the CPU, rounded to ``dtype``."""
    gen = torch.Generator("cpu").manual_seed(seed)
    lg = draw_logits(gen, n_tokens, n_experts)
    if zipf_s is not None:
        lg = lg + zipf_bias(gen, n_experts, zipf_s)[None, :]
    return lg.to(DTYPES[dtype])


def router_inputs(n_tokens: int, n_experts: int, hidden: int, dtype: str = "bf16",
                  seed: int = 0, sigma: Optional[float] = None):
    """Token rows ``x [N, H]`` ~ N(0, 1) and the router's gate weight
    ``w_gate [E, H]`` ~ N(0, sigma) (default 1/sqrt(H), so the logits are about
    N(0, 1) like ``routing_logits``), drawn in that order and rounded to dtype."""
    gen = torch.Generator("cpu").manual_seed(seed)
    x = torch.randn(n_tokens, hidden, generator=gen, dtype=torch.float32)
    w = torch.randn(n_experts, hidden, generator=gen, dtype=torch.float32) * _std(sigma, hidden)
    return x.to(DTYPES[dtype]), w.to(DTYPES[dtype])


def pack_w13(gate: torch.Tensor, up: torch.Tensor, layout: str) -> torch.Tensor:
    """Lay gate/up rows out as ``[E, 2I, H]``: packed [gate; up] or interleaved."""
    if layout == "packed":
        return torch.cat([gate, up], dim=1).contiguous()
    if layout == "interleaved":
        e, i, h = gate.shape
        w = torch.empty(e, 2 * i, h, dtype=gate.dtype)
        w[:, 0::2] = gate
        w[:, 1::2] = up
        return w
    raise ValueError(layout)


@dataclass
class Layer:
    spec: LayerSpec
    logits: torch.Tensor          # [N, E]
    x: torch.Tensor               # [N, H]
    w13: torch.Tensor             # [E, nI, H] in spec.layout
    w2: torch.Tensor              # [E, H, I]
    gate: Optional[torch.Tensor] = None   # [E, I, H] (gated only)
    up: Optional[torch.Tensor] = None     # [E, I, H]
    extra: dict = field(default_factory=dict)


def make_layer(spec: LayerSpec, keep_parts: bool = False) -> Layer:
    """Draw one layer's inputs on the CPU, in the documented order."""
    dt = DTYPES[spec.dtype]
    gen = torch.Generator("cpu").manual_seed(spec.seed)
    E, I, H, N = spec.n_experts, spec.inter, spec.hidden, spec.n_tokens
    EW = spec.n_weights
    lg = draw_logits(gen, N, E)
    x = torch.randn(N, H, generator=gen, dtype=torch.float32).to(dt)
    s13 = _std(spec.sigma13, H)
    s2 = _std(spec.sigma2, I)
    gate = None
    if spec.gated:
        gate = _randn_cast(gen, (EW, I, H), s13, dt)
    up = _randn_cast(gen, (EW, I, H), s13, dt)
    w2 = _randn_cast(gen, (EW, H, I), s2, dt)
    if spec.zipf_s is not None:
        lg = lg + zipf_bias(gen, E, spec.zipf_s)[None, :]
    logits = lg.to(dt)
    if spec.gated:
        w13 = pack_w13(gate, up, spec.layout)
    else:
        w13 = up.contiguous()
    layer = Layer(spec, logits, x, w13, w2)
    if keep_parts:
        layer.gate, layer.up = gate, up
    return layer


def _randn_cast(gen: torch.Generator, shape, std: float, dt: torch.dtype) -> torch.Tensor:
    """N(0, std) drawn in fp32 one expert at a time (bounded peak memory), then cast."""
    out = torch.empty(shape, dtype=dt)
    for e in range(shape[0]):
        out[e] = (torch.randn(shape[1:], generator=gen, dtype=torch.float32) * std).to(dt)
    return out


def act_params(spec: LayerSpec) -> dict:
    """Activation parameters that the layer actually sets (unset ones are omitted)."""
    return {k: v for k, v in (("alpha", spec.alpha), ("beta", spec.beta), ("limit", spec.limit))
            if v is not None}
