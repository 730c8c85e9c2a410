"""GPU layer forward (moe_forward / moe_experts) against the CPU oracle.

Every layer, the full-size ones included, is compared element by element over
its whole output (every row of every expert's m-tiles, ragged tails and
work-split boundaries included), with the routing of the same call checked
bit-exact in full.
"""
import numpy as np
import pytest
import torch

import oracle
from routing_grouped_expert_amd import Routing, moe_experts, moe_forward, moe_route
from routing_grouped_expert_amd.synth import LayerSpec, act_params, layer_spec, make_layer
from tests.gpu_util import assert_output_close, assert_routing_equal

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def _dt(spec):
    return "bf16" if spec.dtype == "bf16" else "f32"


def _to_dev(layer):
    return {k: getattr(layer, k).to(DEV) for k in ("x", "logits", "w13", "w2")}


def run_layer(spec: LayerSpec, check_routing=True):
    print(f"[moe] {spec}", flush=True)
    layer = make_layer(spec)
    d = _to_dev(layer)
    out, routing = moe_forward(d["x"], d["logits"], d["w13"], d["w2"], spec.topk, spec.act,
                               spec.layout, act_params(spec))
    torch.cuda.synchronize()
    ref_r = oracle.route(layer.logits, spec.topk, _dt(spec))
    if check_routing:
        assert_routing_equal(routing, ref_r, f"{spec.name}.routing")
    ref = oracle.moe_ffn(layer.x, ref_r.topk_idx, ref_r.topk_w, layer.w13, layer.w2, spec.act,
                         spec.layout, act_params(spec))
    stats = assert_output_close(out, ref, spec.name)
    print(f"[moe] {spec.name}: {stats}", flush=True)
    return out, routing, layer


# ---------------------------------------------------------------- the 5 configs

def test_tiny_f32():
    run_layer(layer_spec("tiny_f32"))


@pytest.mark.parametrize("e", [4, 8, 16])
def test_minimind_bf16(e):
    run_layer(layer_spec("minimind", n_experts=e, name=f"minimind_e{e}"))


@pytest.mark.timeout(900)
@pytest.mark.parametrize("n", [1, 33, 512, 4096])
def test_gptoss_bf16(n):
    run_layer(layer_spec("gptoss", n_tokens=n, name=f"gptoss_n{n}"))


@pytest.mark.timeout(900)
@pytest.mark.parametrize("act", ["silu", "relu2"])
def test_skewed_bf16(act):
    run_layer(layer_spec("skewed", act=act, name=f"skewed_{act}"))


# ---------------------------------------------------------------- variants and edges

SMALL = [
    # (name, N, H, I, E, k, dtype, act, layout, params)
    ("silu-ktail", 300, 136, 200, 6, 2, "bf16", "silu", "packed", {}),
    ("silu-clamp", 257, 192, 136, 5, 2, "bf16", "silu", "interleaved", {"limit": 0.5}),
    ("oai", 129, 264, 72, 4, 3, "bf16", "swiglu_oai", "interleaved",
     {"alpha": 1.702, "beta": 1.0, "limit": 7.0}),
    ("oai-packed", 200, 128, 128, 8, 2, "bf16", "swiglu_oai", "packed",
     {"alpha": 1.702, "beta": 1.0, "limit": 0.8}),
    ("oai-unset", 64, 64, 64, 3, 1, "bf16", "swiglu_oai", "packed", {}),
    ("relu2", 333, 96, 160, 7, 2, "bf16", "relu2", "packed", {}),
    ("f32-oai", 90, 64, 80, 4, 2, "f32", "swiglu_oai", "interleaved",
     {"alpha": 1.702, "beta": 1.0, "limit": 7.0}),
    ("f32-relu2", 77, 40, 24, 3, 3, "f32", "relu2", "packed", {}),
    ("empty-experts", 5, 128, 128, 64, 2, "bf16", "silu", "packed", {}),
    ("one-expert", 130, 64, 128, 1, 1, "bf16", "silu", "packed", {}),
    ("k-equals-e", 70, 64, 64, 4, 4, "bf16", "silu", "interleaved", {}),
    ("many-tiles", 1500, 256, 384, 3, 2, "bf16", "silu", "packed", {}),
]


@pytest.mark.parametrize("case", SMALL, ids=[c[0] for c in SMALL])
def test_variants(case):
    name, n, h, i, e, k, dt, act, layout, params = case
    spec = LayerSpec(name, n_tokens=n, hidden=h, inter=i, n_experts=e, topk=k, dtype=dt,
                     act=act, layout=layout, alpha=params.get("alpha"),
                     beta=params.get("beta"), limit=params.get("limit"), seed=n + h)
    run_layer(spec)


# Layers of 48 - 176 rows an expert on average (gated: 96 - 176) with K a
# multiple of 64 take the
# register-weight tiles (192 rows, 128 gated / 256 plain output columns a
# tile): skewed routing gives some experts more than 192 rows (several
# m-tiles) and leaves others nearly empty; the output widths leave ragged
# n-tiles; one K-slice (K = 64) makes each tile a single slice.
RW = [
    # (name, N, H, I, E, k, act, layout, zipf_s)
    ("rw-skew-multitile", 640, 192, 320, 8, 2, "silu", "interleaved", 1.2),
    ("rw-packed-ragged", 700, 320, 200, 8, 2, "swiglu_oai", "packed", None),
    ("rw-relu2", 480, 256, 136, 6, 2, "relu2", "packed", 0.8),
    ("rw-one-slice", 500, 64, 64, 8, 2, "silu", "packed", None),
    ("rw-topk1", 700, 128, 192, 5, 1, "silu", "interleaved", 1.0),
    # gated, about 208 rows an expert over 16 n-tiles: the 256-row register-weight
    # tile (skew puts some experts past 256 rows: a second m-tile)
    ("rw256-gated", 1664, 128, 2048, 16, 2, "swiglu_oai", "interleaved", 0.5),
    ("rw256-gated-packed", 1700, 192, 2048, 16, 2, "silu", "packed", None),
    # plain w2 at about 260 rows an expert with 256-row tiles covering the CUs
    # (the four-wave 256 x 256 LDS tile past the 256-row mark)
    ("l256-plain-w2", 4160, 768, 128, 64, 4, "relu2", "packed", 0.3),
    # below 48 rows an expert with the tiles covering the CUs: plain w2 at about
    # 20 rows an expert, gated w13 at about 36
    ("rw-low-plain-w2", 640, 1792, 128, 64, 2, "silu", "packed", 0.4),
    ("rw-low-gated", 1152, 128, 768, 64, 2, "swiglu_oai", "interleaved", None),
    # plain w2 at about 80 rows an expert over 4 n-tiles: the 128-row
    # register-weight tile (skew gives some experts a second m-tile)
    ("rw128-plain-w2", 2560, 1024, 128, 64, 2, "silu", "packed", 0.6),
]


@pytest.mark.parametrize("case", RW, ids=[c[0] for c in RW])
def test_register_weight_tiles(case):
    name, n, h, i, e, k, act, layout, zs = case
    spec = LayerSpec(name, n_tokens=n, hidden=h, inter=i, n_experts=e, topk=k, act=act,
                     layout=layout, zipf_s=zs, seed=n + i,
                     alpha=1.702 if act == "swiglu_oai" else None,
                     beta=1.0 if act == "swiglu_oai" else None,
                     limit=7.0 if act == "swiglu_oai" else None)
    _, routing, _ = run_layer(spec)
    counts = routing.col_sum.cpu()
    print(f"[moe] {name}: rows per expert {counts.tolist()}", flush=True)


def test_layouts_bit_identical_on_gpu():
    """Packed and interleaved w13 built from the same gate/up draws give the same
    output bit for bit (the kernel de-interleaves on the way into LDS)."""
    spec = LayerSpec("lay", n_tokens=700, hidden=256, inter=192, n_experts=8, topk=2,
                     act="swiglu_oai", layout="packed", alpha=1.702, beta=1.0, limit=7.0)
    layer = make_layer(spec, keep_parts=True)
    from routing_grouped_expert_amd.synth import pack_w13
    x, lg, w2 = layer.x.to(DEV), layer.logits.to(DEV), layer.w2.to(DEV)
    p = act_params(spec)
    a, _ = moe_forward(x, lg, pack_w13(layer.gate, layer.up, "packed").to(DEV), w2, 2,
                       "swiglu_oai", "packed", p)
    b, _ = moe_forward(x, lg, pack_w13(layer.gate, layer.up, "interleaved").to(DEV), w2, 2,
                       "swiglu_oai", "interleaved", p)
    torch.cuda.synchronize()
    assert torch.equal(a, b)


def test_forward_equals_route_then_experts_and_is_deterministic():
    spec = layer_spec("minimind", n_experts=8).with_(n_tokens=2000, topk=2)
    d = _to_dev(make_layer(spec))
    out1, r1 = moe_forward(d["x"], d["logits"], d["w13"], d["w2"], 2, "silu")
    r2 = moe_route(d["logits"], 2)
    out2 = moe_experts(d["x"], d["w13"], d["w2"], r2, "silu")
    out3, _ = moe_forward(d["x"], d["logits"], d["w13"], d["w2"], 2, "silu")
    torch.cuda.synchronize()
    assert torch.equal(out1, out2) and torch.equal(out1, out3)
    assert torch.equal(r1.col_sorted, r2.col_sorted)


def test_empty_batch():
    x = torch.empty(0, 64, dtype=torch.bfloat16, device=DEV)
    lg = torch.empty(0, 4, dtype=torch.bfloat16, device=DEV)
    w13 = torch.zeros(4, 128, 64, dtype=torch.bfloat16, device=DEV)
    w2 = torch.zeros(4, 64, 64, dtype=torch.bfloat16, device=DEV)
    out, r = moe_forward(x, lg, w13, w2, 2, "silu")
    torch.cuda.synchronize()
    assert out.shape == (0, 64)


def test_no_host_sync_graph_capture():
    """The whole layer records into a HIP graph (a host sync inside would break
    capture) and replays to the eager result, several times, with eager work in
    between."""
    spec = layer_spec("minimind", n_experts=8).with_(n_tokens=1024, topk=2)
    d = _to_dev(make_layer(spec))
    from routing_grouped_expert_amd import moe_workspace_bytes
    ws = torch.empty(moe_workspace_bytes(1024, 8, 2, spec.hidden, spec.inter), dtype=torch.uint8,
                     device=DEV)
    routing = Routing.empty(1024, 8, 2, torch.bfloat16, DEV)
    out = torch.empty_like(d["x"])
    eager, _ = moe_forward(d["x"], d["logits"], d["w13"], d["w2"], 2, "silu")
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        moe_forward(d["x"], d["logits"], d["w13"], d["w2"], 2, "silu", out=out, routing=routing,
                    workspace=ws)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        moe_forward(d["x"], d["logits"], d["w13"], d["w2"], 2, "silu", out=out, routing=routing,
                    workspace=ws)
    for i in range(3):
        out.fill_(float("nan"))
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, eager), f"replay {i}"
        _ = (d["x"].float() * 2).sum().item()  # eager work between replays
