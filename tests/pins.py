"""Checks that pin the CPU oracle to something other than itself.

Each ``pin_*`` function raises AssertionError when the oracle disagrees with an
independent statement of the same fact: brute-force enumeration, a different
library routine, a closed form, an invariant, or a hand-derived fixture.  The
oracle is always reached through its module attributes, so the mutation tests
can plant a mistake in it (monkeypatch) and check that some pin fails.
"""
from __future__ import annotations

import itertools
import json
import math
import os

import numpy as np
import torch

import oracle.ffn as offn
import oracle.quant as oquant
import oracle.routing as orout

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def sigmoid_tanh(z: float) -> float:
    """Logistic function through the identity sigmoid(z) = (1 + tanh(z/2)) / 2 for
    z >= 0, and e^z / (1 + e^z) below 0 (where 1 + tanh would cancel)."""
    if z >= 0:
        return 0.5 * (1.0 + math.tanh(0.5 * z))
    ez = math.exp(z)
    return ez / (1.0 + ez)


# --------------------------------------------------------------------------
# routing pins
# --------------------------------------------------------------------------

def pin_golden_routing():
    with open(os.path.join(GOLDEN, "routing_tiny.json")) as f:
        g = json.load(f)
    r = orout.route(np.array(g["logits"], dtype=np.float64), g["topk"], g["w_dtype"])
    for key in ("topk_idx", "bitmatrix", "col_sum", "offsets", "col_sorted", "row_sorted"):
        got = np.asarray(getattr(r, key)).astype(np.int64)
        exp = np.asarray(g[key], dtype=np.int64)
        assert got.shape == exp.shape and np.array_equal(got, exp), f"{key}: {got.tolist()} != {exp.tolist()}"
    for key in ("topk_w", "gate_scal"):
        got = np.asarray(getattr(r, key))
        exp = np.asarray(g[key], dtype=np.float64)
        assert np.array_equal(got, exp), f"{key}: {got.tolist()} != {exp.tolist()}"


def brute_topk(row: np.ndarray, k: int) -> list[int]:
    """The unique k-subset S that dominates its complement (a selected logit is
    larger, or equal with a lower index, than every unselected one), listed in
    (descending value, ascending index) order."""
    e = len(row)
    found = []
    for s in itertools.combinations(range(e), k):
        rest = [o for o in range(e) if o not in s]
        if all(row[i] > row[o] or (row[i] == row[o] and i < o) for i in s for o in rest):
            found.append(s)
    assert len(found) == 1, f"dominating subset not unique: {found}"
    return sorted(found[0], key=lambda i: (-row[i], i))


def pin_topk_bruteforce(seed: int = 0, trials: int = 300):
    rng = np.random.default_rng(seed)
    for _ in range(trials):
        e = int(rng.integers(1, 9))
        k = int(rng.integers(1, min(e, 3) + 1))
        # integer-valued logits in a narrow range force many ties; signed zeros too
        row = rng.integers(-2, 3, size=e).astype(np.float64)
        row[row == 0] *= rng.choice([-1.0, 1.0], size=int((row == 0).sum()))
        got = orout.topk_select(row[None, :], k)[0].tolist()
        exp = brute_topk(row, k)
        assert got == exp, f"row={row.tolist()} k={k}: {got} != {exp}"


def pin_topk_lexsort(n=3000, e=128, k=4, seed=1):
    """bf16 Gaussian logits (ties from bf16 spacing are common) against a stable
    lexicographic sort keyed on (-value, index)."""
    g = torch.Generator().manual_seed(seed)
    v = torch.randn(n, e, generator=g).to(torch.bfloat16).double().numpy()
    got = orout.topk_select(v, k)
    order = np.lexsort((np.broadcast_to(np.arange(e), v.shape), -v), axis=-1)[:, :k]
    assert np.array_equal(got, order), "top-k differs from lexsort"
    ties = sum(len(set(r)) < len(r) for r in v[np.arange(n)[:, None], order])
    return ties


def pin_topk_special_cases():
    v = np.full((3, 7), 0.25)
    for k in (1, 3, 7):
        assert orout.topk_select(v, k).tolist() == [list(range(k))] * 3
    rng = np.random.default_rng(3)
    v = rng.integers(-3, 4, size=(50, 9)).astype(np.float64)
    full = orout.topk_select(v, 9)
    for t in range(50):
        assert full[t].tolist() == sorted(range(9), key=lambda i: (-v[t, i], i))


def pin_bf16_rounding(seed=4):
    """Rounding to bf16 against torch's fp32->bf16 cast (round-to-nearest-even)
    on fp32 inputs, including exact halfway cases."""
    rng = np.random.default_rng(seed)
    bits = rng.integers(0x30000000, 0x4F000000, size=20000, dtype=np.uint64).astype(np.uint32)
    bits[:5000] = (bits[:5000] & np.uint32(0xFFFF0000)) | np.uint32(0x8000)   # ties
    vals = bits.view(np.float32)
    vals[::2] *= -1
    ref = torch.from_numpy(vals.copy()).to(torch.bfloat16).double().numpy()
    got = orout.round_to_dtype(vals.astype(np.float64), "bf16")
    assert np.array_equal(got, ref), "bf16 rounding differs from torch's RNE cast"


def pin_weights_closed_forms():
    rng = np.random.default_rng(5)
    # k = 1: the single weight is exactly 1
    v = rng.normal(size=(40, 16))
    r = orout.route(v, 1, "f32")
    assert np.all(r.topk_w == 1.0)
    # equal selected logits: every weight is exactly 1/k
    for k in (2, 4, 8):
        v = np.zeros((5, 16))
        v[:, :k] = 3.0
        for wd in ("f32", "bf16"):
            w = orout.route(v, k, wd).topk_w
            assert np.all(w == 1.0 / k), (k, wd, w)
    # k = 2: w0 = sigmoid(l0 - l1), through the tanh identity
    v = rng.normal(size=(200, 8)).astype(np.float32).astype(np.float64)
    r = orout.route(v, 2, "f32")
    for t in range(200):
        d = v[t, r.topk_idx[t, 0]] - v[t, r.topk_idx[t, 1]]
        s0 = sigmoid_tanh(d)
        assert abs(r.topk_w[t, 0] - s0) <= 2 ** -24 * s0 * 1.01, (t, r.topk_w[t, 0], s0)
        assert abs(r.topk_w[t, 1] - (1 - s0)) <= 2 ** -24 * 1.01
    # the weights sum to 1 within k rounding steps of the weight dtype
    v = rng.normal(size=(300, 32))
    for k in (3, 4, 8):
        w = orout.route(v, k, "bf16").topk_w
        assert np.all(np.abs(w.sum(axis=1) - 1.0) <= k * 2 ** -9), k
        assert np.all(np.diff(w, axis=1) <= 0), "weights must follow descending logits"


def pin_metadata_invariants(n=700, e=32, k=4, seed=6, w_dtype="bf16"):
    g = torch.Generator().manual_seed(seed)
    v = torch.randn(n, e, generator=g).to(torch.bfloat16).double().numpy()
    r = orout.route(v, k, w_dtype)
    m = n * k
    flat = r.topk_idx.reshape(-1).astype(np.int64)
    # bitmatrix: popcount k per row; decoded set is the token's top-k set
    words = (e + 31) // 32
    assert r.bitmatrix.shape == (n, words)
    for t in range(0, n, 7):
        bits = [w * 32 + b for w in range(words) for b in range(32) if (int(r.bitmatrix[t, w]) >> b) & 1]
        assert sorted(bits) == sorted(r.topk_idx[t].tolist()), t
    # histogram (library routine) and its total
    assert np.array_equal(r.col_sum, np.bincount(flat, minlength=e))
    assert int(r.col_sum.sum()) == m
    # offsets: [0] + cumsum, and the right-searchsorted group ends of a stable sort
    assert np.array_equal(r.offsets, np.concatenate([[0], np.cumsum(np.bincount(flat, minlength=e))]))
    srt = np.sort(flat, kind="stable")
    ends = np.searchsorted(srt, np.arange(e), side="right")
    assert np.array_equal(r.offsets[1:], ends) and r.offsets[0] == 0 and r.offsets[-1] == m
    # stable expert-major order
    assert np.array_equal(r.col_sorted, np.argsort(flat, kind="stable"))
    assert np.array_equal(flat[r.col_sorted], np.repeat(np.arange(e), r.col_sum))
    for ex in range(e):
        seg = r.col_sorted[r.offsets[ex]:r.offsets[ex + 1]]
        assert np.all(np.diff(seg) > 0)
    # mutual inverse permutations
    assert np.array_equal(r.row_sorted[r.col_sorted], np.arange(m))
    assert np.array_equal(r.col_sorted[r.row_sorted], np.arange(m))
    # permuted gate weights
    assert np.array_equal(r.gate_scal, r.topk_w.reshape(-1)[r.col_sorted])
    # token of each sorted row
    assert np.array_equal(r.token_of_row, np.argsort(flat, kind="stable") // k)


def pin_empty_experts():
    """N*k < E leaves experts with no rows: zero counts and empty segments."""
    v = np.random.default_rng(7).normal(size=(3, 64))
    r = orout.route(v, 2, "f32")
    assert int((r.col_sum > 0).sum()) <= 6
    assert r.offsets[-1] == 6 and len(r.col_sorted) == 6
    r0 = orout.route(np.zeros((0, 8)), 2, "bf16")
    assert r0.topk_idx.shape == (0, 2) and r0.col_sorted.size == 0
    assert np.array_equal(r0.offsets, np.zeros(9, dtype=np.int32))


def pin_share_routing(seed=14):
    """An expert share's routing against the whole layer's (which the pins above
    fix): the share's sorted entries are the contiguous slice of the layer's
    expert-major order between offsets[lo] and offsets[lo + n]; counts and
    offsets are the layer's restricted and rebased; a slot's position moves down
    by offsets[lo], or is -1 when its expert is outside the share; local bit l
    of the bitmatrix is the layer's bit lo + l (unpacked little-endian)."""
    rng = np.random.default_rng(seed)
    cases = [(300, 64, 4, "bf16", [(0, 64), (0, 8), (8, 8), (56, 8), (5, 37), (63, 1), (30, 2)]),
             (97, 8, 2, "f32", [(0, 1), (3, 4), (7, 1), (0, 8)]),
             (40, 128, 8, "bf16", [(96, 32), (17, 33), (0, 128)])]
    for n, e, k, wdt, shares in cases:
        v = rng.normal(size=(n, e))
        if wdt == "bf16":
            v = torch.from_numpy(v).to(torch.bfloat16).double().numpy()
        g = orout.route(v, k, wdt)
        flat = g.topk_idx.reshape(-1)
        gb = np.unpackbits(g.bitmatrix.view(np.uint8), axis=1, bitorder="little")[:, :e]
        for lo, nl in shares:
            r = orout.route_ep(v, k, wdt, lo, nl)
            a, b = int(g.offsets[lo]), int(g.offsets[lo + nl])
            assert np.array_equal(r.topk_idx, g.topk_idx) and np.array_equal(r.topk_w, g.topk_w)
            assert np.array_equal(r.col_sum, g.col_sum[lo:lo + nl])
            assert np.array_equal(r.offsets, g.offsets[lo:lo + nl + 1] - a)
            assert r.col_sorted.shape == (n * k,) and r.gate_scal.shape == (n * k,)
            assert np.array_equal(r.col_sorted[:b - a], g.col_sorted[a:b])
            assert np.all(r.col_sorted[b - a:] == -1)
            assert np.array_equal(r.gate_scal[:b - a], g.gate_scal[a:b])
            assert np.all(r.gate_scal[b - a:] == 0)
            inside = (flat >= lo) & (flat < lo + nl)
            assert np.array_equal(r.row_sorted, np.where(inside, g.row_sorted - a, -1))
            assert r.bitmatrix.shape == (n, (nl + 31) // 32)
            lb = np.unpackbits(r.bitmatrix.view(np.uint8), axis=1, bitorder="little")
            assert np.array_equal(lb[:, :nl], gb[:, lo:lo + nl]) and not lb[:, nl:].any()
        whole = orout.route_ep(v, k, wdt, 0, e)
        for f in ("topk_idx", "topk_w", "bitmatrix", "col_sum", "offsets", "col_sorted",
                  "row_sorted", "gate_scal"):
            assert np.array_equal(getattr(whole, f), getattr(g, f)), f


def pin_gate_logits(seed=16):
    """Router logits against scalar dot products summed with math.fsum (inputs
    on the bf16 grid, so every product is exact and fsum gives the exactly
    rounded sum), on non-square shapes in both dtypes; an identity gate gives
    x's first E columns exactly; route_gate routes exactly those logits."""
    rng = np.random.default_rng(seed)
    bf = lambda a: orout.round_to_dtype(a, "bf16")
    for n, e, h, dt in [(5, 3, 7, "f32"), (4, 6, 9, "bf16"), (3, 8, 40, "f32")]:
        x, w = bf(rng.normal(size=(n, h))), bf(rng.normal(size=(e, h)) * 0.3)
        lg = orout.gate_logits(x, w, dt)
        assert lg.shape == (n, e)
        for t in range(n):
            for ex in range(e):
                v = math.fsum(float(x[t, c]) * float(w[ex, c]) for c in range(h))
                assert lg[t, ex] == orout.round_to_dtype(np.array([v]), dt)[0], (t, ex)
    x = bf(rng.normal(size=(8, 16)))
    assert np.array_equal(orout.gate_logits(x, np.eye(16)[:5], "bf16"), x[:, :5])
    w = bf(rng.normal(size=(6, 16)))
    lg, r = orout.route_gate(x, w, 2, "bf16")
    ref = orout.route(lg, 2, "bf16")
    assert np.array_equal(r.topk_idx, ref.topk_idx) and np.array_equal(r.col_sorted, ref.col_sorted)


# --------------------------------------------------------------------------
# FFN pins
# --------------------------------------------------------------------------

def _scalar_act(act, g, u, params):
    """Scalar activation through math.* and the tanh form of the logistic."""
    if act == "relu2":
        return max(g, 0.0) ** 2
    lim = params.get("limit", math.inf)
    gc = min(g, lim)
    uc = max(-lim, min(u, lim))
    if act == "silu":
        return gc * sigmoid_tanh(gc) * uc
    a = params.get("alpha", 1.0)
    b = params.get("beta", 0.0)
    return gc * sigmoid_tanh(a * gc) * (uc + b)


def brute_ffn(x, idx, w, w13, w2, act, layout, params):
    """Token-major scalar loops: for each token, each slot, each hidden output,
    sum over intermediate units of w2 * act(gate dot x, up dot x)."""
    n, hdim = x.shape
    k = idx.shape[1]
    inter = w2.shape[2]
    out = [[0.0] * hdim for _ in range(n)]
    for t in range(n):
        for j in range(k):
            e = int(idx[t, j])
            acts = []
            for i in range(inter):
                if act == "relu2":
                    gr = w13[e, i]
                    ur = None
                elif layout == "packed":
                    gr, ur = w13[e, i], w13[e, inter + i]
                else:
                    gr, ur = w13[e, 2 * i], w13[e, 2 * i + 1]
                gv = math.fsum(float(gr[c]) * float(x[t, c]) for c in range(hdim))
                uv = 0.0 if ur is None else math.fsum(float(ur[c]) * float(x[t, c]) for c in range(hdim))
                acts.append(_scalar_act(act, gv, uv, params))
            for o in range(hdim):
                y = math.fsum(float(w2[e, o, i]) * acts[i] for i in range(inter))
                out[t][o] += float(w[t, j]) * y
    return np.array(out)


def _tiny_case(rng, act, layout, n=6, h=5, inter=4, e=3, k=2):
    x = rng.normal(size=(n, h))
    rows = inter if act == "relu2" else 2 * inter
    w13 = rng.normal(size=(e, rows, h)) * 0.7
    w2 = rng.normal(size=(e, h, inter)) * 0.5
    v = rng.normal(size=(n, e))
    r = orout.route(v, k, "f32")
    return x, r, w13, w2


ACT_CASES = [
    ("silu", "packed", {}),
    ("silu", "interleaved", {}),
    ("silu", "packed", {"limit": 0.6}),
    ("swiglu_oai", "interleaved", {"alpha": 1.702, "beta": 1.0, "limit": 0.9}),
    ("swiglu_oai", "packed", {"alpha": 1.702, "beta": 1.0, "limit": 7.0}),
    ("swiglu_oai", "packed", {}),
    ("relu2", "packed", {}),
]


def pin_ffn_bruteforce(seed=8):
    rng = np.random.default_rng(seed)
    for act, layout, params in ACT_CASES:
        x, r, w13, w2 = _tiny_case(rng, act, layout)
        got = offn.moe_ffn(x, r.topk_idx, r.topk_w, w13, w2, act, layout, params)
        exp = brute_ffn(x, r.topk_idx, r.topk_w, w13, w2, act, layout, params)
        err = np.max(np.abs(got - exp)) / max(1e-300, np.max(np.abs(exp)))
        assert err < 1e-12, (act, layout, params, err)


def pin_ffn_masked_equals_sorted(seed=9):
    """The masked loop and the sorted dispatch agree bit for bit."""
    rng = np.random.default_rng(seed)
    for act, layout, params in ACT_CASES:
        for e, k in ((1, 1), (4, 1), (4, 2), (8, 2), (8, 3)):
            x, r, w13, w2 = _tiny_case(rng, act, layout, n=37, h=16, inter=12, e=e, k=k)
            a = offn.moe_ffn(x, r.topk_idx, r.topk_w, w13, w2, act, layout, params)
            b = offn.moe_ffn_sorted(x, r.topk_idx, r.topk_w, w13, w2, act, layout, params)
            assert np.array_equal(a, b), (act, layout, e, k)


def pin_ffn_layout_invariance(seed=10):
    """Packed [gate; up] and interleaved [g0, u0, ...] rows of the same gate/up
    weights give the same layer output."""
    rng = np.random.default_rng(seed)
    n, h, inter, e, k = 29, 24, 16, 4, 2
    x = rng.normal(size=(n, h))
    gate = rng.normal(size=(e, inter, h)) * 0.3
    up = rng.normal(size=(e, inter, h)) * 0.3
    w2 = rng.normal(size=(e, h, inter)) * 0.3
    packed = np.concatenate([gate, up], axis=1)
    inter_l = np.empty((e, 2 * inter, h))
    inter_l[:, 0::2] = gate
    inter_l[:, 1::2] = up
    r = orout.route(rng.normal(size=(n, e)), k, "f32")
    for act, params in (("silu", {}), ("swiglu_oai", {"alpha": 1.702, "beta": 1.0, "limit": 0.8})):
        a = offn.moe_ffn(x, r.topk_idx, r.topk_w, packed, w2, act, "packed", params)
        b = offn.moe_ffn(x, r.topk_idx, r.topk_w, inter_l, w2, act, "interleaved", params)
        assert np.allclose(a, b, rtol=1e-13, atol=1e-13 * np.max(np.abs(a))), act


def pin_ffn_dense_special_case(seed=11):
    """All experts holding one weight set reduce the layer to a dense FFN scaled
    by each token's weight sum; the dense FFN here is torch's functional API."""
    import torch.nn.functional as F
    rng = np.random.default_rng(seed)
    n, h, inter, e, k = 23, 12, 10, 5, 3
    x = rng.normal(size=(n, h))
    gate = rng.normal(size=(inter, h)) * 0.4
    up = rng.normal(size=(inter, h)) * 0.4
    w2 = rng.normal(size=(h, inter)) * 0.4
    r = orout.route(rng.normal(size=(n, e)), k, "f32")
    wsum = r.topk_w.sum(axis=1, keepdims=True)
    xt = torch.from_numpy(x)
    gt, ut, w2t = map(torch.from_numpy, (gate, up, w2))
    dense = {
        "silu": F.linear(F.silu(F.linear(xt, gt)) * F.linear(xt, ut), w2t),
        "relu2": F.linear(F.relu(F.linear(xt, ut)) ** 2, w2t),
    }
    w13s = {"silu": np.concatenate([gate, up], 0), "relu2": up}
    for act in ("silu", "relu2"):
        w13 = np.broadcast_to(w13s[act], (e,) + w13s[act].shape)
        w2e = np.broadcast_to(w2, (e, h, inter))
        got = offn.moe_ffn(x, r.topk_idx, r.topk_w, w13, w2e, act, "packed", {})
        exp = dense[act].numpy() * wsum
        assert np.allclose(got, exp, rtol=1e-12, atol=1e-12), act
    # single expert, top-1: the weight is exactly 1 and the layer is the dense FFN
    r1 = orout.route(rng.normal(size=(n, 1)), 1, "bf16")
    got = offn.moe_ffn(x, r1.topk_idx, r1.topk_w, w13s["silu"][None], w2[None], "silu", "packed", {})
    assert np.allclose(got, dense["silu"].numpy(), rtol=1e-12, atol=1e-12)


def pin_activation_closed_forms():
    act = offn.activation
    a = np.array
    assert act("relu2", a([-1.0]))[0] == 0.0 and act("relu2", a([3.0]))[0] == 9.0
    assert act("silu", a([0.0]), a([5.0]))[0] == 0.0
    # SwiGLU-OAI at g=10, u=-9 with alpha 1.702, beta 1, limit 7: gate clamps to 7,
    # up clamps to -7, so a = 7 * sigmoid(1.702 * 7) * (-7 + 1)
    p = {"alpha": 1.702, "beta": 1.0, "limit": 7.0}
    exp = 7.0 * sigmoid_tanh(1.702 * 7.0) * (-6.0)
    got = act("swiglu_oai", a([10.0]), a([-9.0]), p)[0]
    assert abs(got - exp) <= 1e-14 * abs(exp), (got, exp)
    # gate below the limit is untouched; only the upper side of the gate clamps
    got = act("swiglu_oai", a([-10.0]), a([0.5]), p)[0]
    exp = -10.0 * sigmoid_tanh(-17.02) * 1.5
    assert abs(got - exp) <= 1e-14 * abs(exp)
    # unset parameters reduce SwiGLU-OAI to SiLU-gated (torch's silu)
    import torch.nn.functional as F
    g = np.linspace(-6, 6, 41)
    u = np.linspace(3, -3, 41)
    ref = (F.silu(torch.from_numpy(g)) * torch.from_numpy(u)).numpy()
    assert np.allclose(act("swiglu_oai", g, u, {}), ref, rtol=1e-14, atol=1e-15)
    assert np.allclose(act("silu", g, u, {}), ref, rtol=1e-14, atol=1e-15)
    # SiLU with a clamp: gate capped from above, up clipped both ways
    got = act("silu", a([9.0]), a([-8.0]), {"limit": 7.0})[0]
    exp = 7.0 * sigmoid_tanh(7.0) * (-7.0)
    assert abs(got - exp) <= 1e-14 * abs(exp)
    # SiLU ignores alpha/beta (only the limit applies to it)
    assert np.array_equal(act("silu", g, u, {"alpha": 3.0, "beta": 2.0}), act("silu", g, u, {}))


def pin_ffn_linearity(seed=12):
    rng = np.random.default_rng(seed)
    x, r, w13, w2 = _tiny_case(rng, "swiglu_oai", "interleaved", n=15, h=8, inter=6, e=4, k=2)
    p = {"alpha": 1.702, "beta": 1.0, "limit": 7.0}
    a = offn.moe_ffn(x, r.topk_idx, r.topk_w, w13, w2, "swiglu_oai", "interleaved", p)
    b = offn.moe_ffn(x, r.topk_idx, r.topk_w, w13, 2.0 * w2, "swiglu_oai", "interleaved", p)
    assert np.array_equal(2.0 * a, b)


def pin_ffn_token_subset(seed=13):
    rng = np.random.default_rng(seed)
    x, r, w13, w2 = _tiny_case(rng, "silu", "packed", n=40, h=8, inter=6, e=5, k=2)
    full = offn.moe_ffn(x, r.topk_idx, r.topk_w, w13, w2, "silu", "packed", {})
    sel = np.array([39, 0, 17, 17, 5])
    sub = offn.moe_ffn(x, r.topk_idx, r.topk_w, w13, w2, "silu", "packed", {}, tokens=sel)
    assert np.allclose(sub, full[sel], rtol=1e-13, atol=1e-13)


def pin_ffn_shares(seed=15):
    """Expert shares: their contributions summed over a partition of the experts
    give the whole layer; one share equals the brute-force token loop with the
    weights of slots outside the share set to zero; a share that no token chose
    gives zero rows."""
    rng = np.random.default_rng(seed)
    for act, layout, params in [("silu", "packed", {}), ("relu2", "packed", {}),
                                ("swiglu_oai", "interleaved",
                                 {"alpha": 1.702, "beta": 1.0, "limit": 0.9})]:
        x, r, w13, w2 = _tiny_case(rng, act, layout, n=12, h=6, inter=4, e=5, k=2)
        full = offn.moe_ffn(x, r.topk_idx, r.topk_w, w13, w2, act, layout, params)
        tot = np.zeros_like(full)
        for lo, nl in [(0, 2), (2, 1), (3, 2)]:
            tot += offn.moe_ffn_share(x, r.topk_idx, r.topk_w, w13[lo:lo + nl], w2[lo:lo + nl],
                                      act, lo, layout, params)
        assert np.allclose(tot, full, rtol=1e-12, atol=1e-12)
        lo, nl = 1, 3
        idx = r.topk_idx
        wz = np.where((idx >= lo) & (idx < lo + nl), r.topk_w, 0.0)
        bf = brute_ffn(x, idx, wz, w13, w2, act, layout, params)
        sh = offn.moe_ffn_share(x, idx, r.topk_w, w13[lo:lo + nl], w2[lo:lo + nl], act, lo,
                                layout, params)
        assert np.allclose(sh, bf, rtol=1e-11, atol=1e-11)
    x, r, w13, w2 = _tiny_case(rng, "silu", "packed", n=9, h=4, inter=4, e=4, k=2)
    v = rng.normal(size=(9, 4))
    v[:, 3] = -50.0                                   # expert 3 is never in a top-2
    r = orout.route(v, 2, "f32")
    z = offn.moe_ffn_share(x, r.topk_idx, r.topk_w, w13[3:], w2[3:], "silu", 3)
    assert z.shape == x.shape and not z.any()


def pin_ffn_weighted_input(seed=17):
    """Routing weight on the input rows: a scalar token loop that scales and
    rounds each slot's input row explicitly; the power-of-two closed form (for
    ReLU^2, h(w x) = w^2 h(x) exactly when w is a power of two, so the result is
    the output-weighted layer with weights w^2, bit for bit); top-1 with weight
    1 is the plain layer."""
    rng = np.random.default_rng(seed)
    for act, layout, params, dt in [("silu", "packed", {}, "bf16"),
                                    ("swiglu_oai", "interleaved",
                                     {"alpha": 1.702, "beta": 1.0, "limit": 0.9}, "f32"),
                                    ("relu2", "packed", {}, "bf16")]:
        x, r, w13, w2 = _tiny_case(rng, act, layout, n=7, h=5, inter=4, e=3, k=2)
        got = offn.moe_ffn_weighted_input(x, r.topk_idx, r.topk_w, w13, w2, act, dt, layout,
                                          params)
        n, k = r.topk_idx.shape
        want = np.zeros_like(got)
        for t in range(n):
            for j in range(k):
                xin = orout.round_to_dtype(x[t:t + 1] * float(r.topk_w[t, j]), dt)
                one = np.ones((1, 1))
                want[t] += brute_ffn(xin, r.topk_idx[t:t + 1, j:j + 1], one, w13, w2, act, layout,
                                     params)[0]
        assert np.allclose(got, want, rtol=1e-11, atol=1e-11), act
    x, r, w13, w2 = _tiny_case(rng, "relu2", "packed", n=9, h=6, inter=5, e=4, k=2)
    pw = 2.0 ** rng.integers(-3, 2, size=r.topk_w.shape)
    a = offn.moe_ffn_weighted_input(x, r.topk_idx, pw, w13, w2, "relu2", "f32")
    xr = orout.round_to_dtype(x, "f32")
    b = offn.moe_ffn(xr, r.topk_idx, pw * pw, w13, w2, "relu2")
    assert np.array_equal(a, b)
    v = rng.normal(size=(9, 4))
    r1 = orout.route(v, 1, "f32")
    assert np.all(r1.topk_w == 1.0)
    xb = orout.round_to_dtype(x, "bf16")
    assert np.array_equal(
        offn.moe_ffn_weighted_input(xb, r1.topk_idx, r1.topk_w, w13, w2, "relu2", "bf16"),
        offn.moe_ffn(xb, r1.topk_idx, r1.topk_w, w13, w2, "relu2"))


ROUTING_PINS = [pin_golden_routing, pin_topk_bruteforce, pin_topk_lexsort, pin_topk_special_cases,
                pin_bf16_rounding, pin_weights_closed_forms, pin_metadata_invariants,
                pin_empty_experts, pin_share_routing, pin_gate_logits]
FFN_PINS = [pin_ffn_bruteforce, pin_ffn_masked_equals_sorted, pin_ffn_layout_invariance,
            pin_ffn_dense_special_case, pin_activation_closed_forms, pin_ffn_linearity,
            pin_ffn_token_subset, pin_ffn_shares, pin_ffn_weighted_input]


# --------------------------------------------------------------------------
# MXFP4 weight pins
# --------------------------------------------------------------------------

def _e2m1_value(code: int) -> float:
    """FP4 E2M1 value from its bit fields: sign, 2 exponent bits (bias 1), 1
    mantissa bit; exponent 0 is subnormal (m * 0.5)."""
    sgn, e, m = code >> 3, (code >> 1) & 3, code & 1
    mag = m * 0.5 if e == 0 else 2.0 ** (e - 1) * (1 + m / 2)
    return -mag if sgn else mag


def _e2m1_nearest(v: float) -> int:
    """Brute force: the code nearest to v (magnitude capped at the largest value),
    ties to the code with an even lowest bit, the sign of v kept."""
    mags = [abs(_e2m1_value(m)) for m in range(8)]
    a = min(abs(v), max(mags))
    d = [abs(a - mg) for mg in mags]
    cands = [m for m in range(8) if d[m] == min(d)]
    m = cands[0] if len(cands) == 1 else [c for c in cands if c % 2 == 0][0]
    return m | (8 if math.copysign(1.0, v) < 0 else 0)


def pin_mxfp4_codes():
    """Decoding matches the E2M1 bit-field formula for all 16 codes; encoding of
    every multiple of 1/64 in [-10, 10] matches brute force (ties included)."""
    for c in range(16):
        assert float(oquant.e2m1_decode(np.uint8(c))) == _e2m1_value(c), c
    vals = np.arange(-640, 641) / 64.0
    got = oquant.e2m1_encode(vals)
    for v, c in zip(vals, got):
        assert int(c) == _e2m1_nearest(float(v)), (v, int(c), _e2m1_nearest(float(v)))


def pin_mxfp4_blocks(seed=18):
    """Block quantisation: the scale puts each block's largest magnitude in
    [4, 8); every element is the brute-force nearest code at that scale, even
    element in the low nibble; quantising the dequantised weights gives the same
    bytes back; a block of representable values round-trips exactly; an all-zero
    block gets scale byte 0 and zero codes."""
    rng = np.random.default_rng(seed)
    w = rng.normal(size=(6, 96)) * np.array([1e-3, 1.0, 50.0, 0.3, 7.0, 1e-30])[:, None]
    w[0, :32] = 0.0
    grid = np.array([_e2m1_value(c) for c in range(16)])
    w[1, 32:64] = rng.choice(grid, size=32) * 2.0 ** -3
    w[1, 32] = 6.0 * 2.0 ** -3                   # the block's max decides X = -3
    q, s = oquant.quantize_mxfp4(w)
    assert q.shape == (6, 48) and s.shape == (6, 3) and q.dtype == np.uint8
    deq = oquant.dequantize_mxfp4(q, s)
    for r in range(6):
        for b in range(3):
            blk = w[r, 32 * b:32 * b + 32]
            x = int(s[r, b]) - 127
            amax = np.abs(blk).max()
            if amax == 0:
                assert s[r, b] == 0 and not q[r, 16 * b:16 * b + 16].any()
                continue
            assert 4.0 <= amax / 2.0 ** x < 8.0, (r, b, x, amax)
            for i in range(32):
                c = _e2m1_nearest(blk[i] / 2.0 ** x)
                byte = int(q[r, 16 * b + i // 2])
                assert (byte >> (4 * (i % 2))) & 15 == c, (r, b, i)
                assert deq[r, 32 * b + i] == _e2m1_value(c) * 2.0 ** x
    q2, s2 = oquant.quantize_mxfp4(deq)
    assert np.array_equal(q, q2) and np.array_equal(s, s2)
    assert np.array_equal(deq[1, 32:64], w[1, 32:64])


QUANT_PINS = [pin_mxfp4_codes, pin_mxfp4_blocks]
