"""GPU router GEMM + routing (moe_gate_route / moe_gate_forward) against the CPU
oracle.

The logits are checked against the float64 product x . W_gate^T within the
error bound of fp32 accumulation plus the final rounding (derived below); the
routing is then checked bit-exact against the oracle's routing of the GPU's own
logits, so both sides take the top-k decision on the same values."""
import numpy as np
import pytest
import torch

import oracle
from routing_grouped_expert_amd import (moe_forward, moe_gate_forward, moe_gate_route, moe_route,
                                        MoeError)
from routing_grouped_expert_amd.synth import layer_spec, make_layer, router_inputs
from tests.gpu_util import INT_FIELDS, assert_output_close, assert_routing_equal

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def _ulp(v: np.ndarray, dt: str) -> np.ndarray:
    """Spacing of the dtype's values at |v| (normal range)."""
    mant = 7 if dt == "bf16" else 23
    e = np.floor(np.log2(np.maximum(np.abs(v), 2.0 ** -126)))
    return 2.0 ** (e - mant)


def assert_logits_close(gpu: torch.Tensor, x: torch.Tensor, w: torch.Tensor, dt: str,
                        rows=None, where="logits") -> dict:
    """|gpu - exact| <= (H + 2) 2^-24 sum_h |x w| + ulp/2.  The first term bounds
    fp32 accumulation of H products (exact for bf16 inputs, one rounding each
    for fp32 ones: gamma_(H+1) of the absolute sum, with margin); the second is
    the single rounding of the fp32 sum to the dtype."""
    g = gpu.detach().cpu().double().numpy()
    x64 = x.double().numpy() if rows is None else x.double().numpy()[rows]
    if rows is not None:
        g = g[rows]
    w64 = w.double().numpy()
    exact = x64 @ w64.T
    h = x64.shape[1]
    bound = (h + 2) * 2.0 ** -24 * (np.abs(x64) @ np.abs(w64).T) \
        + 0.5 * _ulp(np.maximum(np.abs(g), np.abs(exact)), dt)
    err = np.abs(g - exact)
    assert np.all(np.isfinite(g)), f"{where}: non-finite"
    assert np.all(err <= bound), f"{where}: {int((err > bound).sum())} logits beyond the bound; " \
                                 f"worst excess {float((err - bound).max())}"
    ref = oracle.gate_logits(x64, w64, dt)
    return {"differs_from_oracle_rounding": int((g != ref).sum()), "n": int(g.size)}


def _gate_case(n, e, h, k, dt):
    print(f"[gate] N={n} E={e} H={h} k={k} {dt}", flush=True)
    x, w = router_inputs(n, e, h, dt, seed=n + 7 * e + h)
    lg, routing = moe_gate_route(x.to(DEV), w.to(DEV), k)
    torch.cuda.synchronize()
    stats = assert_logits_close(lg, x, w, dt, None, f"logits N={n} E={e} H={h}")
    ref = oracle.route(lg.cpu(), k, dt)
    assert_routing_equal(routing, ref, f"gate-routing N={n} E={e}")
    print(f"[gate] {stats}", flush=True)
    return x, w, lg, routing


GATE_CASES = [
    (1, 128, 2880, 4, "bf16"),      # decode: a wave per expert row, then the one-wave routing
    (1, 33, 1000, 3, "f32"),        # one token, fp32, E odd, a ragged last piece per lane
    (1, 6, 136, 2, "bf16"),         # one token, fewer experts than a workgroup's waves
    (1, 32, 2880, 4, "bf16"),       # one token, gpt-oss-20b-sized router
    (1, 16, 1000, 2, "f32"),        # one token, fp32, a ragged last piece per lane
    (2, 128, 2880, 4, "bf16"),      # two tokens: a wave per expert row, both tokens' logits
    (3, 33, 1000, 3, "f32"),        # three tokens, fp32
    (4, 256, 7168, 8, "bf16"),      # four tokens, DeepSeek-sized router
    (5, 128, 2880, 4, "bf16"),      # five tokens: split over K, sums in the routing prologue
    (33, 8, 128, 2, "f32"),         # the tiny fp32 layer's router
    (64, 32, 512, 4, "bf16"),       # largest batch of the prologue path
    (65, 32, 512, 4, "bf16"),       # first batch of the separate GEMM kernel (4 K-slices)
    (65, 128, 2880, 4, "bf16"),     # first batch of the split over token tiles and K-groups
    (300, 6, 136, 2, "bf16"),       # E off the 32/8 grids; H leaves a 16-byte K tail
    (777, 256, 264, 8, "bf16"),     # largest expert count, multi-block routing
    (1000, 33, 1000, 3, "f32"),     # fp32, multi-block, split over K (16 groups)
    (4096, 8, 512, 1, "bf16"),      # small-model router (too few K-slices to split)
    (4096, 128, 2880, 4, "bf16"),   # gpt-oss-sized router: 4 K-groups of 6, 6, 6 and 5 slices
    (4097, 128, 2880, 4, "bf16"),   # first batch past the split: the separate GEMM kernel
    (700, 256, 7168, 8, "bf16"),    # DeepSeek-sized router at a prefill batch (11 tiles)
    (2, 16, 8200, 2, "bf16"),       # two tokens, a wave per expert row over a long row
    (5, 16, 8200, 2, "bf16"),       # split-K over 65 slices: three rounds of the group sum
    (5, 16, 32776, 2, "bf16"),      # more K-slices (257) than the split-K path takes: full prologue
    (8, 128, 2880, 4, "bf16"),      # split-K sums past the prologue's share: reduction kernel
    (4, 32, 2880, 4, "bf16"),       # four tokens: still a wave per expert row
    (6, 32, 2880, 4, "bf16"),       # split-K sums added up in the routing kernel's prologue
    (40, 256, 4096, 8, "bf16"),     # split-K with the widest expert bucket
    (1, 256, 7168, 8, "bf16"),      # DeepSeek-sized router, decode (a wave per expert row)
    (64, 256, 7168, 8, "bf16"),     # the same at the largest split-K batch
    (17, 64, 1000, 6, "f32"),       # fp32 split-K through the reduction kernel
    (2000, 64, 3000, 4, "f32"),     # fp32, K-groups of 6 slices (the last 5), K tail
    (300, 6, 2000, 2, "bf16"),      # E off the 32/8 grids through the split
]


@pytest.mark.parametrize("n,e,h,k,dt", GATE_CASES,
                         ids=[f"n{a}-e{b}-h{c}-k{d}-{f}" for a, b, c, d, f in GATE_CASES])
def test_gate_route(n, e, h, k, dt):
    _gate_case(n, e, h, k, dt)


@pytest.mark.timeout(600)
def test_gate_route_largest_batch():
    _gate_case(65536, 128, 2880, 4, "bf16")


# batches that take the 64-token tile (at least 64 tokens per compute unit, fewer
# than 128) and the 32-token tile just below it
@pytest.mark.parametrize("n,e,h,k,dt", [(20000, 64, 512, 8, "bf16"), (17000, 33, 264, 3, "f32"),
                                        (16000, 128, 1024, 4, "bf16")])
def test_gate_route_mid_batches(n, e, h, k, dt):
    _gate_case(n, e, h, k, dt)


def test_gate_route_equals_route_on_its_logits():
    x, w = router_inputs(3000, 64, 256, "bf16", seed=3)
    lg, r1 = moe_gate_route(x.to(DEV), w.to(DEV), 4)
    r2 = moe_route(lg, 4)
    torch.cuda.synchronize()
    for f in INT_FIELDS + ("topk_w", "gate_scal"):
        assert torch.equal(getattr(r1, f), getattr(r2, f)), f


@pytest.mark.parametrize("family,kw", [("minimind", dict(n_tokens=700, hidden=256, inter=512,
                                                          n_experts=8, topk=1)),
                                        ("tiny_f32", {}),
                                        ("gptoss", dict(n_tokens=48, hidden=256, inter=256,
                                                        n_experts=16))])
def test_gate_forward(family, kw):
    spec = layer_spec(family, **kw)
    print(f"[gate-fwd] {spec}", flush=True)
    layer = make_layer(spec)
    dt = spec.dtype
    _, w_gate = router_inputs(spec.n_tokens, spec.n_experts, spec.hidden, dt, seed=5)
    d = {f: getattr(layer, f).to(DEV) for f in ("x", "w13", "w2")}
    from routing_grouped_expert_amd.synth import act_params
    p = act_params(spec)
    out, lg, routing = moe_gate_forward(d["x"], w_gate.to(DEV), d["w13"], d["w2"], spec.topk,
                                        spec.act, spec.layout, p)
    out2, _ = moe_forward(d["x"], lg, d["w13"], d["w2"], spec.topk, spec.act, spec.layout, p)
    torch.cuda.synchronize()
    assert torch.equal(out, out2)
    assert_logits_close(lg, layer.x, w_gate, dt)
    ref_r = oracle.route(lg.cpu(), spec.topk, dt)
    assert_routing_equal(routing, ref_r, "gate-forward routing")
    ref = oracle.moe_ffn(layer.x, ref_r.topk_idx, ref_r.topk_w, layer.w13, layer.w2, spec.act,
                         spec.layout, p)
    assert_output_close(out, ref, f"gate-forward {spec.name}")


def test_gate_argument_checks():
    x, w = router_inputs(16, 8, 64, "bf16")
    with pytest.raises(ValueError):
        moe_gate_route(x.to(DEV), w[:, :32].contiguous().to(DEV), 2)   # hidden mismatch
    with pytest.raises(MoeError):
        moe_gate_route(x[:, :60].contiguous().to(DEV), w[:, :60].contiguous().to(DEV), 2)
