"""Expert-FFN oracle (test infrastructure only; see the package docstring).

The layer output is computed the way the minimind issue #835 page describes its
``MOEFeedForward.forward`` (section "Summary"): loop over experts, select the
tokens routed to each one with a mask, run the expert FFN on those rows, scale
each row by its routing weight, and add it into the output at its token.  The
sorted-dispatch variant (same page, "It is removable in plain PyTorch") feeds
each expert a contiguous slice of the stably expert-sorted rows instead; the page
reports the two bit-identical, and ``moe_ffn_sorted`` is kept to check that.

Everything is float64.  Inputs (x, weights, routing weights) are taken exactly
as given; no intermediate is rounded to the layer dtype -- lower-precision
intermediates are the kernel's choice and are covered by the test tolerance.

Expert FFN, per routed row ``x`` of expert e (weights in nn.Linear out x in form):
``h = W13[e] @ x``; gated activations split h into gate/up rows (packed
``[gate; up]`` or interleaved ``[g0, u0, g1, u1, ...]``, the two layouts of the
w13 reorder helper in the vLLM PR #47106 report, section "key source snippets");
``a = act(...)``; ``y = W2[e] @ a``.

Activation kinds and their parameters (PR #47106 report, "implementation
breakdown" and the ``apply`` snippet; parameters left unset keep the plain SwiGLU
defaults alpha=1, beta=0, no clamp, "review highlights"):

* ``silu``:  g' = min(g, L), u' = clip(u, -L, L), a = g' * sigmoid(g') * u'
  (only the clamp limit L applies to SiLU; with no limit this is silu(g) * u);
* ``swiglu_oai``: a = g' * sigmoid(alpha * g') * (u' + beta), same clamps.
  parity unpinned: the pages name alpha/beta/limit and the 1.702/1.0/7.0
  values but print no formula; this is the public gpt-oss definition;
* ``relu2``: non-gated, a = max(h, 0)^2, no parameters.
"""
from __future__ import annotations

import numpy as np

from .routing import to_f64

_ACTS = ("silu", "swiglu_oai", "relu2")


def _sigmoid(z: np.ndarray) -> np.ndarray:
    with np.errstate(over="ignore"):
        return 1.0 / (1.0 + np.exp(-z))


def activation(act: str, g: np.ndarray, u: np.ndarray | None = None,
               params: dict | None = None) -> np.ndarray:
    """Elementwise activation in float64; ``g`` is the gate (or the only) input."""
    params = params or {}
    if act == "relu2":
        r = np.maximum(g, 0.0)
        return r * r
    lim = params.get("limit", np.inf)
    gc = np.minimum(g, lim)
    uc = np.clip(u, -lim, lim)
    if act == "silu":
        return gc * _sigmoid(gc) * uc
    if act == "swiglu_oai":
        alpha = params.get("alpha", 1.0)
        beta = params.get("beta", 0.0)
        return gc * _sigmoid(alpha * gc) * (uc + beta)
    raise ValueError(f"unknown activation {act!r}")


def split_gate_up(h: np.ndarray, layout: str):
    """Split the GEMM1 output rows into (gate, up) by w13 layout."""
    n2 = h.shape[-1]
    if n2 % 2:
        raise ValueError("gated w13 needs an even number of rows")
    if layout == "packed":
        return h[..., : n2 // 2], h[..., n2 // 2:]
    if layout == "interleaved":
        return h[..., 0::2], h[..., 1::2]
    raise ValueError(f"unknown layout {layout!r}")


def expert_ffn(xr: np.ndarray, w13e: np.ndarray, w2e: np.ndarray, act: str, layout: str,
               params: dict | None) -> np.ndarray:
    """One expert's FFN on rows ``xr [r, H]`` -> ``[r, H]`` (float64)."""
    h = xr @ w13e.T
    if act == "relu2":
        a = activation(act, h)
    else:
        g, u = split_gate_up(h, layout)
        a = activation(act, g, u, params)
    return a @ w2e.T


def _check(act, layout, w13, w2):
    if act not in _ACTS:
        raise ValueError(act)
    if act == "relu2" and layout != "packed":
        raise ValueError("relu2 is non-gated; only the packed (single up matrix) layout applies")


def moe_ffn(x, topk_idx, topk_w, w13, w2, act: str, layout: str = "packed",
            params: dict | None = None, tokens=None) -> np.ndarray:
    """Layer output ``[N, H]`` (float64) by the masked per-expert loop.

    ``tokens`` optionally restricts the computation to those token rows (the
    result then has one row per listed token, in the listed order).
    """
    _check(act, layout, w13, w2)
    xs = to_f64(x)
    idx = np.asarray(topk_idx)
    w = np.asarray(topk_w, dtype=np.float64)
    if tokens is not None:
        tokens = np.asarray(tokens, dtype=np.int64)
        xs, idx, w = xs[tokens], idx[tokens], w[tokens]
    n_experts = w13.shape[0]
    out = np.zeros((xs.shape[0], w2.shape[1]), dtype=np.float64)
    for e in range(n_experts):
        mask = idx == e                      # [n, k]
        if not mask.any():
            continue
        rows = np.flatnonzero(mask.any(axis=1))
        wt = np.where(mask, w, 0.0).sum(axis=1)[rows]   # a token names e at most once
        y = expert_ffn(xs[rows], to_f64(w13[e]), to_f64(w2[e]), act, layout, params)
        out[rows] += wt[:, None] * y
    return out


def moe_ffn_sorted(x, topk_idx, topk_w, w13, w2, act: str, layout: str = "packed",
                   params: dict | None = None) -> np.ndarray:
    """Same output by sorted dispatch: stable sort of the flat expert ids, group
    bounds by right-searchsorted, token of entry = flat index // k, each expert
    gets a contiguous slice, results scattered back with their weights."""
    _check(act, layout, w13, w2)
    xs = to_f64(x)
    idx = np.asarray(topk_idx)
    n, k = idx.shape
    flat = idx.reshape(-1)
    order = np.argsort(flat, kind="stable")
    ends = np.searchsorted(flat[order], np.arange(w13.shape[0]), side="right")
    tok = order // k
    wsort = np.asarray(topk_w, dtype=np.float64).reshape(-1)[order]
    xsorted = xs[tok]
    out = np.zeros((n, w2.shape[1]), dtype=np.float64)
    lo = 0
    for e, hi in enumerate(ends):
        if hi > lo:
            y = expert_ffn(xsorted[lo:hi], to_f64(w13[e]), to_f64(w2[e]), act, layout, params)
            out[tok[lo:hi]] += wsort[lo:hi, None] * y
        lo = hi
    return out


def moe_ffn_share(x, topk_idx, topk_w, w13, w2, act: str, local_offset: int,
                  layout: str = "packed", params: dict | None = None,
                  tokens=None) -> np.ndarray:
    """Contribution of one expert-parallel share: ``w13``/``w2`` hold the
    experts [local_offset, local_offset + len(w13)) and ``topk_idx`` the global
    selection.  The selection is remapped to local ids (-1 outside the share)
    and the masked per-expert loop runs over the local experts, so slots routed
    elsewhere add nothing and a token with none of them gets a zero row."""
    from .routing import remap_to_share
    loc = remap_to_share(topk_idx, local_offset, int(w13.shape[0]))
    return moe_ffn(x, loc, topk_w, w13, w2, act, layout, params, tokens=tokens)


def moe_ffn_weighted_input(x, topk_idx, topk_w, w13, w2, act: str, dtype: str,
                           layout: str = "packed", params: dict | None = None) -> np.ndarray:
    """Layer output ``[N, H]`` (float64) with the routing weight applied to the
    input rows (the ``apply_router_weight_on_input`` flag of the experts
    ``apply`` in the vLLM PR #47106 report, section "key source snippets"):
    masked per-expert loop as in ``moe_ffn``, but each routed row's input is
    ``x[t] * w[t, j]`` rounded once to the layer ``dtype`` and the expert
    output is added unweighted."""
    from .routing import round_to_dtype
    _check(act, layout, w13, w2)
    xs = to_f64(x)
    idx = np.asarray(topk_idx)
    w = np.asarray(topk_w, dtype=np.float64)
    out = np.zeros((xs.shape[0], w2.shape[1]), dtype=np.float64)
    for e in range(w13.shape[0]):
        mask = idx == e
        if not mask.any():
            continue
        rows = np.flatnonzero(mask.any(axis=1))
        wt = np.where(mask, w, 0.0).sum(axis=1)[rows]   # a token names e at most once
        xin = round_to_dtype(xs[rows] * wt[:, None], dtype)
        out[rows] += expert_ffn(xin, to_f64(w13[e]), to_f64(w2[e]), act, layout, params)
    return out
