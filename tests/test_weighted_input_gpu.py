"""GPU routing weight on the input rows (moe_experts_weighted_input) against the
CPU oracle, and a HIP-graph-captured stack of layers against its eager run."""
import numpy as np
import pytest
import torch

import oracle
from routing_grouped_expert_amd import (moe_experts, moe_experts_weighted_input, moe_gate_forward,
                                        moe_route, moe_workspace_bytes, Routing)
from routing_grouped_expert_amd.synth import LayerSpec, act_params, make_layer, router_inputs
from tests.gpu_util import assert_output_close

pytestmark = pytest.mark.gpu
DEV = "cuda:0"

CASES = [
    # (name, N, H, I, E, k, dtype, act, layout, params, custom weights)
    ("top1-sigmoidlike", 600, 256, 384, 8, 1, "bf16", "silu", "packed", {}, True),
    ("top2", 300, 128, 256, 6, 2, "bf16", "silu", "packed", {}, False),
    ("oai-top4", 129, 264, 72, 8, 4, "bf16", "swiglu_oai", "interleaved",
     {"alpha": 1.702, "beta": 1.0, "limit": 7.0}, False),
    ("relu2-f32", 77, 40, 24, 3, 2, "f32", "relu2", "packed", {}, True),
    ("ktail-f32", 90, 136, 80, 4, 1, "f32", "swiglu_oai", "packed", {"limit": 0.8}, True),
]


def _routing(layer, k, custom, seed):
    r = moe_route(layer.logits.to(DEV), k)
    if custom:  # caller-supplied weights in (0, 1), not a softmax (e.g. a sigmoid router)
        g = torch.Generator().manual_seed(seed)
        w = (torch.rand(r.topk_w.shape, generator=g) * 0.9 + 0.05).to(r.topk_w.dtype).to(DEV)
        r.topk_w.copy_(w)
        r.gate_scal.copy_(w.reshape(-1)[r.col_sorted.long()])
    return r


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_weighted_input(case):
    name, n, h, i, e, k, dt, act, layout, params, custom = case
    spec = LayerSpec(name, n_tokens=n, hidden=h, inter=i, n_experts=e, topk=k, dtype=dt, act=act,
                     layout=layout, alpha=params.get("alpha"), beta=params.get("beta"),
                     limit=params.get("limit"), seed=n + h)
    print(f"[wi] {spec}", flush=True)
    layer = make_layer(spec)
    r = _routing(layer, k, custom, n)
    out = moe_experts_weighted_input(layer.x.to(DEV), layer.w13.to(DEV), layer.w2.to(DEV), r, act,
                                     layout, act_params(spec))
    torch.cuda.synchronize()
    w64 = r.topk_w.cpu().double().numpy()
    ref = oracle.moe_ffn_weighted_input(layer.x, r.topk_idx.cpu().numpy(), w64, layer.w13,
                                        layer.w2, act, dt, layout, act_params(spec))
    print(f"[wi] {name}: {assert_output_close(out, ref, name)}", flush=True)


def test_weighted_input_unit_weights_equal_plain():
    # top-1 softmax weights are exactly 1: scaling the input changes nothing
    spec = LayerSpec("wi-unit", n_tokens=800, hidden=256, inter=256, n_experts=8, topk=1,
                     dtype="bf16", seed=2)
    layer = make_layer(spec)
    d = {f: getattr(layer, f).to(DEV) for f in ("x", "w13", "w2")}
    r = moe_route(layer.logits.to(DEV), 1)
    a = moe_experts_weighted_input(d["x"], d["w13"], d["w2"], r, "silu")
    b = moe_experts(d["x"], d["w13"], d["w2"], r, "silu")
    torch.cuda.synchronize()
    assert torch.equal(a, b)


def test_graph_captured_layer_stack():
    """Four layers chained as in decoding (router GEMM + routing + experts,
    each layer's output the next one's input) record into one HIP graph; every
    replay equals the eager chain bit for bit, with eager work in between."""
    L, n, h, i, e, k = 4, 8, 256, 256, 16, 4
    p = {"alpha": 1.702, "beta": 1.0, "limit": 7.0}
    layers = []
    for l in range(L):
        spec = LayerSpec(f"stack{l}", n_tokens=n, hidden=h, inter=i, n_experts=e, topk=k,
                         dtype="bf16", act="swiglu_oai", layout="interleaved", sigma13=0.05,
                         sigma2=0.05, seed=100 + l)
        lay = make_layer(spec)
        _, wg = router_inputs(n, e, h, "bf16", seed=200 + l)
        layers.append((wg.to(DEV), lay.w13.to(DEV), lay.w2.to(DEV)))
    x0 = make_layer(LayerSpec("x0", n, h, i, e, k, seed=7)).x.to(DEV)
    bufs = [x0] + [torch.empty_like(x0) for _ in range(L)]
    logits = torch.empty(n, e, dtype=torch.bfloat16, device=DEV)
    routing = Routing.empty(n, e, k, torch.bfloat16, DEV)
    ws = torch.empty(moe_workspace_bytes(n, e, k, h, i), dtype=torch.uint8, device=DEV)

    def chain():
        for l, (wg, w13, w2) in enumerate(layers):
            moe_gate_forward(bufs[l], wg, w13, w2, k, "swiglu_oai", "interleaved", p,
                             out=bufs[l + 1], logits=logits, routing=routing, workspace=ws)

    chain()
    torch.cuda.synchronize()
    eager = [b.clone() for b in bufs[1:]]
    assert eager[-1].abs().sum() > 0
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        chain()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        chain()
    for rep in range(3):
        for b in bufs[1:]:
            b.fill_(float("nan"))
        g.replay()
        torch.cuda.synchronize()
        for l in range(L):
            assert torch.equal(bufs[l + 1], eager[l]), f"replay {rep} layer {l}"
        _ = (x0.float() * 3).sum().item()  # eager work between replays
