"""Plant plausible mistakes in the CPU oracle and check that the pins catch each.

Every mutation replaces one oracle function (monkeypatch, CPU only) with a
subtly wrong version; the test passes only if at least one pin in the given
group then fails.  This guards against pins too weak to notice a dropped term, a
wrong sign or index, or a transposed operand.
"""
import numpy as np
import pytest

import oracle.ffn as offn
import oracle.quant as oquant
import oracle.routing as orout
from tests import pins

_orig_topk = orout.topk_select
_orig_sorted = orout.sorted_indices
_orig_act = offn.activation
_orig_split = offn.split_gate_up
_orig_round = orout.round_to_dtype
_orig_expert = offn.expert_ffn
_orig_bm = orout.bitmatrix


def topk_ties_high(v, k):
    # ties broken towards the highest expert index
    vv = np.asarray(v, dtype=np.float64)[:, ::-1]
    idx = _orig_topk(vv, k)
    return (vv.shape[1] - 1 - idx).astype(np.int32)


def topk_signed_zero(v, k):
    # -0.0 ranked below +0.0 (compare by sign bit as well as value)
    vv = np.asarray(v, dtype=np.float64)
    vv = np.where((vv == 0) & np.signbit(vv), -1e-300, vv)
    return _orig_topk(vv, k)


def sorted_unstable(idx, e):
    col, row = _orig_sorted(idx, e)
    hist = orout.histogram(idx, e)
    off = orout.offsets_from_hist(hist)
    col = col.copy()
    for ex in range(e):
        col[off[ex]:off[ex + 1]] = col[off[ex]:off[ex + 1]][::-1]
    row = np.empty_like(col)
    row[col] = np.arange(col.size)
    return col, row


def hist_shifted(idx, e):
    return np.array([int(np.count_nonzero(idx == (x + 1) % e)) for x in range(e)], dtype=np.int32)


def offsets_exclusive(cs):
    off = np.zeros(len(cs) + 1, dtype=np.int32)
    off[1:] = np.concatenate([[0], np.cumsum(cs)[:-1]])
    return off


def softmax_all_logits(v, idx, w_dtype):
    v = np.asarray(v, dtype=np.float64)
    ex = np.exp(v - v.max(axis=1, keepdims=True))
    p = ex / ex.sum(axis=1, keepdims=True)
    return orout.round_to_dtype(np.take_along_axis(p, idx.astype(np.int64), axis=1), w_dtype)


def round_truncate(x, dtype):
    if dtype == "bf16":
        f = np.asarray(x, dtype=np.float32)
        return (f.view(np.uint32) & np.uint32(0xFFFF0000)).view(np.float32).astype(np.float64)
    return _orig_round(x, dtype)


def bitmatrix_off_by_one(idx, e):
    return _orig_bm(np.minimum(idx + 1, e - 1), e)


def split_swapped(h, layout):
    g, u = _orig_split(h, layout)
    return (u, g) if layout == "packed" else (g, u)


def split_interleave_odd(h, layout):
    g, u = _orig_split(h, layout)
    return (u, g) if layout == "interleaved" else (g, u)


def act_drop_beta(act, g, u=None, params=None):
    p = dict(params or {})
    p.pop("beta", None)
    return _orig_act(act, g, u, p)


def act_drop_alpha(act, g, u=None, params=None):
    p = dict(params or {})
    p.pop("alpha", None)
    return _orig_act(act, g, u, p)


def act_clamp_gate_both(act, g, u=None, params=None):
    p = params or {}
    if act != "relu2" and "limit" in p:
        g = np.clip(g, -p["limit"], p["limit"])
    return _orig_act(act, g, u, params)


def act_relu_no_square(act, g, u=None, params=None):
    if act == "relu2":
        return np.maximum(g, 0.0)
    return _orig_act(act, g, u, params)


def act_sigmoid_sign(act, g, u=None, params=None):
    if act == "silu":
        p = params or {}
        lim = p.get("limit", np.inf)
        gc = np.minimum(g, lim)
        return gc / (1.0 + np.exp(gc)) * np.clip(u, -lim, lim)
    return _orig_act(act, g, u, params)


def expert_transposed_w2(xr, w13e, w2e, act, layout, params):
    if w2e.shape[0] == w2e.shape[1]:
        w2e = w2e.T
    else:
        w2e = w2e.reshape(w2e.shape[1], w2e.shape[0]).T
    return _orig_expert(xr, w13e, w2e, act, layout, params)


def moe_ffn_no_weight(x, topk_idx, topk_w, *a, **kw):
    return _orig_moe(x, topk_idx, np.ones_like(np.asarray(topk_w, dtype=np.float64)), *a, **kw)


_orig_moe = offn.moe_ffn
_orig_remap = orout.remap_to_share


_orig_gate = orout.gate_logits


def gate_not_rounded(x, w, dtype):
    return orout.to_f64(x) @ orout.to_f64(w).T


def gate_rows_swapped(x, w, dtype):
    # the first two gate rows trade places (a wrong expert index)
    w = orout.to_f64(w).copy()
    w[[0, 1]] = w[[1, 0]]
    return _orig_gate(x, w, dtype)


def gate_dropped_last_column(x, w, dtype):
    return _orig_gate(orout.to_f64(x)[:, :-1], orout.to_f64(w)[:, :-1], dtype)


_orig_wi = offn.moe_ffn_weighted_input


def weighted_input_unrounded(x, idx, w, w13, w2, act, dtype, layout="packed", params=None):
    # the scaled input rows kept in float64 (the rounding to the layer dtype dropped)
    xs, idx, w = orout.to_f64(x), np.asarray(idx), np.asarray(w, dtype=np.float64)
    out = np.zeros((xs.shape[0], w2.shape[1]))
    for e in range(w13.shape[0]):
        mask = idx == e
        if mask.any():
            rows = np.flatnonzero(mask.any(axis=1))
            wt = np.where(mask, w, 0.0).sum(axis=1)[rows]
            out[rows] += offn.expert_ffn(xs[rows] * wt[:, None], orout.to_f64(w13[e]),
                                         orout.to_f64(w2[e]), act, layout, params)
    return out


def weighted_input_on_output(x, idx, w, w13, w2, act, dtype, layout="packed", params=None):
    return offn.moe_ffn(x, idx, w, w13, w2, act, layout, params)


_orig_enc = oquant.e2m1_encode
_orig_q = oquant.quantize_mxfp4


def e2m1_ties_away(v):
    # ties rounded away from zero instead of to the even code
    v = np.asarray(v, dtype=np.float64)
    a = np.abs(v)
    d = np.abs(a[..., None] - oquant.E2M1)
    best = 7 - np.argmin(d[..., ::-1], axis=-1)   # last minimum: the larger magnitude
    best = np.where(a > 6.0, 7, best)
    return (best.astype(np.uint8) | (np.signbit(v).astype(np.uint8) << 3)).astype(np.uint8)


def mxfp4_scale_off_by_one(w):
    # X = floor(log2 amax) - 1: the block's max lands in [2, 4)
    q, s = _orig_q(np.asarray(w, dtype=np.float64) / 2.0)
    return q, s + 1


def mxfp4_nibbles_swapped(w):
    q, s = _orig_q(w)
    return ((q >> 4) | (q << 4)).astype(np.uint8), s


def remap_off_by_one(idx, lo, nl):
    r = _orig_remap(idx, lo, nl)
    return np.where(r >= 0, np.minimum(r + 1, nl - 1), -1).astype(np.int32)


def remap_upper_inclusive(idx, lo, nl):
    g = np.asarray(idx, dtype=np.int64)
    inside = (g >= lo) & (g <= lo + nl)
    return np.where(inside, g - lo, -1).astype(np.int32)


def remap_none(idx, lo, nl):
    # global ids used as local ones
    return np.asarray(idx, dtype=np.int32)

MUTATIONS = [
    ("topk ties high", orout, "topk_select", topk_ties_high, "routing"),
    ("signed zero", orout, "topk_select", topk_signed_zero, "routing"),
    ("unstable sort", orout, "sorted_indices", sorted_unstable, "routing"),
    ("histogram shifted", orout, "histogram", hist_shifted, "routing"),
    ("offsets exclusive", orout, "offsets_from_hist", offsets_exclusive, "routing"),
    ("softmax over all", orout, "topk_softmax", softmax_all_logits, "routing"),
    ("bf16 truncation", orout, "round_to_dtype", round_truncate, "routing"),
    ("bitmatrix off by one", orout, "bitmatrix", bitmatrix_off_by_one, "routing"),
    ("packed gate/up swapped", offn, "split_gate_up", split_swapped, "ffn"),
    ("interleaved odd/even swapped", offn, "split_gate_up", split_interleave_odd, "ffn"),
    ("beta dropped", offn, "activation", act_drop_beta, "ffn"),
    ("alpha dropped", offn, "activation", act_drop_alpha, "ffn"),
    ("gate clamped below", offn, "activation", act_clamp_gate_both, "ffn"),
    ("relu not squared", offn, "activation", act_relu_no_square, "ffn"),
    ("sigmoid sign", offn, "activation", act_sigmoid_sign, "ffn"),
    ("w2 transposed", offn, "expert_ffn", expert_transposed_w2, "ffn"),
    ("routing weight dropped", offn, "moe_ffn", moe_ffn_no_weight, "ffn"),
    ("share remap off by one", orout, "remap_to_share", remap_off_by_one, "routing"),
    ("share upper bound inclusive", orout, "remap_to_share", remap_upper_inclusive, "routing"),
    ("share ids not remapped (routing)", orout, "remap_to_share", remap_none, "routing"),
    ("share ids not remapped (ffn)", orout, "remap_to_share", remap_none, "ffn"),
    ("share remap off by one (ffn)", orout, "remap_to_share", remap_off_by_one, "ffn"),
    ("gate logits not rounded", orout, "gate_logits", gate_not_rounded, "routing"),
    ("e2m1 ties away from zero", oquant, "e2m1_encode", e2m1_ties_away, "quant"),
    ("mxfp4 scale exponent off by one", oquant, "quantize_mxfp4", mxfp4_scale_off_by_one,
     "quant"),
    ("mxfp4 nibble order swapped", oquant, "quantize_mxfp4", mxfp4_nibbles_swapped, "quant"),
    ("weighted input not rounded", offn, "moe_ffn_weighted_input", weighted_input_unrounded,
     "ffn"),
    ("weight on output instead of input", offn, "moe_ffn_weighted_input",
     weighted_input_on_output, "ffn"),
    ("gate rows swapped", orout, "gate_logits", gate_rows_swapped, "routing"),
    ("gate last hidden unit dropped", orout, "gate_logits", gate_dropped_last_column, "routing"),
]


def _some_pin_fails(group):
    group_pins = {"routing": pins.ROUTING_PINS, "ffn": pins.FFN_PINS,
                  "quant": pins.QUANT_PINS}[group]
    failed = []
    for pin in group_pins:
        try:
            pin()
        except Exception:  # an assertion or a shape error both count as caught
            failed.append(pin.__name__)
    return failed


@pytest.mark.parametrize("name,mod,attr,fn,group", MUTATIONS, ids=[m[0] for m in MUTATIONS])
def test_mutation_is_caught(monkeypatch, name, mod, attr, fn, group):
    monkeypatch.setattr(mod, attr, fn)
    failed = _some_pin_fails(group)
    assert failed, f"planted mistake '{name}' passed every {group} pin"


def test_unmutated_oracle_passes_all_pins():
    assert not _some_pin_fails("routing")
    assert not _some_pin_fails("ffn")
    assert not _some_pin_fails("quant")
