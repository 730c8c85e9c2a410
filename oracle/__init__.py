"""CPU oracle for the MoE layer forward: TEST INFRASTRUCTURE ONLY.

A plain, slow, obviously-correct numpy (float64) statement of what the GPU path
computes.  Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline``
leg of ``bench.py`` may import it.  It shares no code with the HIP library or its
Python binding, and imports neither.

* :mod:`oracle.routing` -- top-k gating with softmax over the selected logits and
  the routing metadata built from it (bitmatrix, per-expert histogram, ragged
  offsets, stable expert-sorted gather/scatter indices, permuted gate weights).
* :mod:`oracle.ffn` -- the expert FFN (SiLU-gated, SwiGLU-OAI, ReLU^2) run as the
  masked per-expert loop, the weighted combine, and the sorted-dispatch variant.
* :mod:`oracle.ffn` also gives the layer with the routing weight on the input
  rows (``moe_ffn_weighted_input``).
* :mod:`oracle.quant` -- MXFP4 expert weights: E2M1 codes with one E8M0 scale
  per 32 weights along K (quantise, dequantise).
* :mod:`oracle.routing` also gives the router logits from the gate weight
  (``gate_logits``, ``route_gate``).
* both also give one GPU's expert-parallel share (``route_ep``,
  ``moe_ffn_share``): the selected experts remapped to local ids, -1 outside.

Every function is pinned by ``tests/test_oracle_*.py`` against brute force,
library routines, closed forms, invariants and the hand-derived fixtures in
``tests/golden/``; the one part with no such pin (the SwiGLU-OAI formula relative
to the pages) is marked "parity unpinned" where it is defined.
"""
from .routing import (RoutingRef, bitmatrix, gate_logits, histogram, offsets_from_hist,
                      remap_to_share, route, route_ep, route_gate, round_to_dtype, sorted_indices,
                      topk_select, topk_softmax)
from .quant import dequantize_mxfp4, e2m1_decode, e2m1_encode, quantize_mxfp4
from .ffn import (activation, moe_ffn, moe_ffn_share, moe_ffn_sorted,
                  moe_ffn_weighted_input, split_gate_up)

__all__ = [
    "RoutingRef", "route", "topk_select", "topk_softmax", "bitmatrix", "histogram",
    "offsets_from_hist", "sorted_indices", "round_to_dtype", "remap_to_share", "route_ep",
    "gate_logits", "route_gate",
    "activation", "split_gate_up", "moe_ffn", "moe_ffn_sorted", "moe_ffn_share",
    "moe_ffn_weighted_input", "quantize_mxfp4", "dequantize_mxfp4", "e2m1_encode",
    "e2m1_decode",
]
