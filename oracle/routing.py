"""Routing oracle (test infrastructure only; see the package docstring).

What is computed, and where the pages define it:

* top-k over each token's router logits, then softmax over the k selected
  logits only -- the ``topk(logits, k, apply_softmax=True)`` call in the parity
  test of the vLLM PR #45457 report (section "key source snippets");
* the expert bitmatrix, the per-expert column sums (``col_sum``), the row- and
  column-sorted index arrays and ``gate_scal = vals.flatten()[col_sorted]`` --
  the ``mask_metadata`` fields that ``routing_data_from_sparse_topk`` reads, same
  report, sections "implementation breakdown" and "key source snippets";
* the ragged per-expert offsets ``[0] + cumulative counts`` -- the segment bounds
  of the sorted dispatch in the minimind issue #835 page, section "It is
  removable in plain PyTorch" (stable sort by expert, group ends by
  ``searchsorted(right=True)``);
* the router logits themselves (``gate_logits``): the router's gate matmul
  ``x . W_gate^T``, the step just before the top-k that the PR #45457 report
  leaves to its own kernel (section "motivation");
* the expert-parallel share (``route_ep``): the selected expert ids remapped to
  the ids local to one GPU's experts, then the bitmatrix re-packed and the
  metadata rebuilt from the remapped ids -- the expert-map branch of the PR
  #45457 report ("implementation breakdown"); the share is the
  (local_expert_offset, num_local_experts) pair of the kernel call in the vLLM
  PR #47106 report ("key source snippets").

Readings where the pages are silent:
ties in top-k go to the lowest expert index; slots are ordered by descending
logit, ties by ascending index; -0.0 equals +0.0; logits must be finite;
softmax is evaluated in float64 and rounded once (nearest-even) to the weight
dtype, which is the logits dtype because ``gate_scal`` inherits the gating
output dtype (PR #45457 report, "risks and impact", item 1).
"""
from __future__ import annotations

from dataclasses import dataclass

import numpy as np


# --------------------------------------------------------------------------
# float helpers
# --------------------------------------------------------------------------

def to_f64(t) -> np.ndarray:
    """Exact float64 copy of a torch tensor (fp32/bf16) or numpy array."""
    try:
        import torch
        if isinstance(t, torch.Tensor):
            return t.detach().to("cpu", torch.float64).numpy()
    except ImportError:  # pragma: no cover
        pass
    return np.asarray(t, dtype=np.float64)


def _bf16_round(x: np.ndarray) -> np.ndarray:
    """Round float64 values to the nearest bfloat16 value, ties to even.

    Candidates are the bfloat16 grid points bracketing ``x`` (found from the
    fp32 bit pattern of ``x`` truncated to its top 16 bits, and its neighbours);
    the nearest candidate in exact float64 distance wins, a tie goes to the one
    whose last mantissa bit is 0.  Finite inputs of bf16 range only.
    """
    x = np.asarray(x, dtype=np.float64)
    f = x.astype(np.float32)
    hi16 = (f.view(np.uint32) & np.uint32(0xFFFF0000)).astype(np.int64)
    best = np.full(x.shape, np.nan)
    best_bits = np.zeros(x.shape, dtype=np.int64)
    best_dist = np.full(x.shape, np.inf)
    for step in (-0x10000, 0, 0x10000):
        cb = (hi16 + step) & 0xFFFFFFFF
        c = cb.astype(np.uint32).view(np.float32).astype(np.float64)
        d = np.abs(x - c)
        even = ((cb >> 16) & 1) == 0
        better = (d < best_dist) | ((d == best_dist) & even & (((best_bits >> 16) & 1) == 1))
        better &= np.isfinite(c)
        best = np.where(better, c, best)
        best_bits = np.where(better, cb, best_bits)
        best_dist = np.where(better, d, best_dist)
    return best


def round_to_dtype(x: np.ndarray, dtype: str) -> np.ndarray:
    """Round float64 values once, nearest-even, to ``dtype`` ('f32' or 'bf16');
    the result is returned as float64 holding exactly representable values."""
    if dtype == "f32":
        return np.asarray(x, dtype=np.float64).astype(np.float32).astype(np.float64)
    if dtype == "bf16":
        return _bf16_round(x)
    raise ValueError(dtype)


# --------------------------------------------------------------------------
# the routing steps
# --------------------------------------------------------------------------

def topk_select(v: np.ndarray, k: int) -> np.ndarray:
    """Top-k expert indices per token, ``[N, k]`` int32.

    k rounds; each round takes, among the experts not yet chosen, the one with
    the largest logit -- ``np.argmax`` returns the first maximum, so an equal
    value goes to the lowest expert index.  Slot j therefore holds the j-th
    expert in (descending value, ascending index) order.
    """
    v = np.asarray(v, dtype=np.float64) + 0.0      # -0.0 + 0.0 == +0.0
    n, e = v.shape
    if not (1 <= k <= e):
        raise ValueError("need 1 <= k <= n_experts")
    if not np.all(np.isfinite(v)):
        raise ValueError("logits must be finite")
    idx = np.zeros((n, k), dtype=np.int32)
    taken = np.zeros((n, e), dtype=bool)
    rows = np.arange(n)
    for j in range(k):
        cand = np.where(taken, -np.inf, v)
        pick = np.argmax(cand, axis=1)
        idx[:, j] = pick
        taken[rows, pick] = True
    return idx


def topk_softmax(v: np.ndarray, idx: np.ndarray, w_dtype: str) -> np.ndarray:
    """Softmax over each token's k selected logits, rounded to ``w_dtype``.

    ``w[t, j] = exp(v[t, idx[t, j]] - m_t) / sum_j' exp(v[t, idx[t, j']] - m_t)``
    with ``m_t`` the token's largest selected logit, evaluated in float64.
    """
    v = np.asarray(v, dtype=np.float64)
    sel = np.take_along_axis(v, idx.astype(np.int64), axis=1)
    m = sel.max(axis=1, keepdims=True)
    ex = np.exp(sel - m)
    w = ex / ex.sum(axis=1, keepdims=True)
    return round_to_dtype(w, w_dtype)


def bitmatrix(idx: np.ndarray, n_experts: int) -> np.ndarray:
    """``[N, ceil(E/32)]`` uint32; bit (e % 32) of word e // 32 in row t is set iff
    token t selected expert e.  Bits past E are zero; an id of -1 (a slot whose
    expert is outside an expert-parallel share) sets no bit."""
    n, k = idx.shape
    words = (n_experts + 31) // 32
    bm = np.zeros((n, words), dtype=np.uint64)
    for j in range(k):
        e = idx[:, j].astype(np.int64)
        rows = np.flatnonzero(e >= 0)
        e = e[rows]
        np.bitwise_or.at(bm, (rows, e // 32), (np.uint64(1) << (e % 32).astype(np.uint64)))
    return bm.astype(np.uint32)


def histogram(idx: np.ndarray, n_experts: int) -> np.ndarray:
    """``col_sum[e]`` = number of (token, slot) pairs routed to expert e, int32.
    One masked count per expert, the shape of the per-expert loop."""
    return np.array([int(np.count_nonzero(idx == e)) for e in range(n_experts)], dtype=np.int32)


def offsets_from_hist(col_sum: np.ndarray) -> np.ndarray:
    """Ragged segment bounds ``[E+1]``: 0, then the running total of col_sum."""
    off = np.zeros(len(col_sum) + 1, dtype=np.int64)
    for e, c in enumerate(col_sum):
        off[e + 1] = off[e] + int(c)
    return off.astype(np.int32)


def sorted_indices(idx: np.ndarray, n_experts: int):
    """Stable expert-major order of the flat (token, slot) entries.

    ``col_sorted[p]`` is the flat index f = t*k + j of the p-th entry when entries
    are grouped by expert (ascending) and kept in flat order inside a group;
    ``row_sorted[f]`` is the position p of entry f (its inverse permutation).
    Built with one masked scan per expert, which is stable by construction.
    Entries with id -1 (outside an expert-parallel share) get no position:
    ``col_sorted`` then lists only the others and their ``row_sorted`` is -1.
    """
    flat = idx.reshape(-1)
    parts = [np.flatnonzero(flat == e) for e in range(n_experts)]
    col_sorted = (np.concatenate(parts) if parts else np.zeros(0, np.int64)).astype(np.int64)
    row_sorted = np.full(flat.size, -1, dtype=np.int64)
    row_sorted[col_sorted] = np.arange(col_sorted.size)
    return col_sorted.astype(np.int32), row_sorted.astype(np.int32)


@dataclass
class RoutingRef:
    topk_idx: np.ndarray     # [N, k] int32
    topk_w: np.ndarray       # [N, k] float64 holding w_dtype values
    bitmatrix: np.ndarray    # [N, ceil(E/32)] uint32
    col_sum: np.ndarray      # [E] int32
    offsets: np.ndarray      # [E+1] int32
    col_sorted: np.ndarray   # [N*k] int32 (gather source / scatter destination)
    row_sorted: np.ndarray   # [N*k] int32 (gather destination / scatter source)
    gate_scal: np.ndarray    # [N*k] float64 holding w_dtype values

    @property
    def token_of_row(self) -> np.ndarray:
        """Token feeding sorted row p: col_sorted[p] // k (rows past an expert
        share's last local entry hold col_sorted -1 and have no token)."""
        k = self.topk_idx.shape[1]
        return self.col_sorted // k


def route(logits, topk: int, w_dtype: str) -> RoutingRef:
    """All routing outputs for one layer from its ``[N, E]`` router logits."""
    v = to_f64(logits)
    n, e = v.shape
    idx = topk_select(v, topk)
    w = topk_softmax(v, idx, w_dtype)
    cs = histogram(idx, e)
    col_sorted, row_sorted = sorted_indices(idx, e)
    return RoutingRef(
        topk_idx=idx,
        topk_w=w,
        bitmatrix=bitmatrix(idx, e),
        col_sum=cs,
        offsets=offsets_from_hist(cs),
        col_sorted=col_sorted,
        row_sorted=row_sorted,
        gate_scal=w.reshape(-1)[col_sorted],
    )


def remap_to_share(idx: np.ndarray, local_offset: int, n_local: int) -> np.ndarray:
    """Global expert ids -> ids local to the share [local_offset, local_offset +
    n_local): ``e - local_offset`` inside the share, -1 outside."""
    g = np.asarray(idx, dtype=np.int64)
    inside = (g >= local_offset) & (g < local_offset + n_local)
    return np.where(inside, g - local_offset, -1).astype(np.int32)


def route_ep(logits, topk: int, w_dtype: str, local_offset: int, n_local: int) -> RoutingRef:
    """Routing of one GPU's expert share [local_offset, local_offset + n_local).

    Top-k and softmax over all E logits (``topk_idx`` keeps the global ids);
    then the selected ids are remapped to local ids (-1 outside the share) and
    the bitmatrix, histogram, offsets and sorted indices are built from the
    remapped ids over the n_local experts.  ``col_sorted`` and ``gate_scal`` keep
    their N*k length: positions past the M_local = offsets[n_local] local entries
    hold -1 and 0.
    """
    v = to_f64(logits)
    n, e = v.shape
    if not (0 <= local_offset and 1 <= n_local and local_offset + n_local <= e):
        raise ValueError("expert share outside [0, n_experts)")
    idx = topk_select(v, topk)
    w = topk_softmax(v, idx, w_dtype)
    loc = remap_to_share(idx, local_offset, n_local)
    cs = histogram(loc, n_local)
    col, row_sorted = sorted_indices(loc, n_local)
    m, ml = n * topk, col.size
    col_sorted = np.full(m, -1, dtype=np.int32)
    col_sorted[:ml] = col
    gate = np.zeros(m, dtype=np.float64)
    gate[:ml] = w.reshape(-1)[col]
    return RoutingRef(
        topk_idx=idx,
        topk_w=w,
        bitmatrix=bitmatrix(loc, n_local),
        col_sum=cs,
        offsets=offsets_from_hist(cs),
        col_sorted=col_sorted,
        row_sorted=row_sorted,
        gate_scal=gate,
    )


def gate_logits(x, w_gate, dtype: str) -> np.ndarray:
    """Router logits ``[N, E]``: ``x [N, H]`` times the gate weight ``w_gate [E, H]``
    (nn.Linear out x in) transposed, evaluated in float64 and rounded once,
    nearest-even, to ``dtype`` (the router's output dtype)."""
    return round_to_dtype(to_f64(x) @ to_f64(w_gate).T, dtype)


def route_gate(x, w_gate, topk: int, w_dtype: str):
    """Logits from the router's gate matmul, then the routing of those logits;
    returns ``(logits, RoutingRef)``."""
    lg = gate_logits(x, w_gate, w_dtype)
    return lg, route(lg, topk, w_dtype)
