"""moe_forward_noalloc (the layer with its intermediates in the library's static
per-GPU scratch, for callers that cannot allocate) against moe_forward: the
same kernels, so the same bits.  Two calls in a row, the second smaller, show
that a call does not depend on what the previous one left in the scratch."""
import pytest
import torch

from routing_grouped_expert_amd import (MoeError, Routing, moe_forward, moe_forward_noalloc,
                                        moe_workspace_bytes)
from routing_grouped_expert_amd import _native as N
from routing_grouped_expert_amd.synth import LayerSpec, act_params, layer_spec, make_layer

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
FIELDS = ("topk_idx", "topk_w", "bitmatrix", "col_sum", "offsets", "col_sorted", "row_sorted",
          "gate_scal")


def _dev(layer):
    return [getattr(layer, f).to(DEV) for f in ("x", "logits", "w13", "w2")]


def _check_same(spec):
    print(f"[noalloc] {spec}", flush=True)
    assert moe_workspace_bytes(spec.n_tokens, spec.n_experts, spec.topk, spec.hidden,
                               spec.inter, torch.bfloat16 if spec.dtype == "bf16"
                               else torch.float32) <= N.MOE_NOALLOC_SCRATCH_BYTES
    x, lg, w13, w2 = _dev(make_layer(spec))
    p = act_params(spec)
    want, r_want = moe_forward(x, lg, w13, w2, spec.topk, spec.act, spec.layout, p)
    routing = Routing.empty(spec.n_tokens, spec.n_experts, spec.topk, x.dtype, DEV)
    out = torch.full_like(x, float("nan"))
    got, r_got = moe_forward_noalloc(x, lg, w13, w2, spec.topk, spec.act, spec.layout, p,
                                     out=out, routing=routing)
    torch.cuda.synchronize()
    assert got is out and r_got is routing
    assert torch.equal(got, want), f"{spec.name}: output differs from moe_forward"
    for f in FIELDS:
        assert torch.equal(getattr(r_got, f), getattr(r_want, f)), f"{spec.name}: {f}"


def test_two_calls_second_smaller():
    big = layer_spec("gptoss", n_tokens=1200, name="gptoss_n1200")      # ~55 MB of scratch
    small = LayerSpec("small", n_tokens=300, hidden=256, inter=192, n_experts=16, topk=4,
                      act="swiglu_oai", layout="interleaved", alpha=1.702, beta=1.0, limit=7.0,
                      seed=5)
    _check_same(big)
    _check_same(small)


def test_decode_and_top1_shapes():
    _check_same(layer_spec("gptoss", n_tokens=33, name="gptoss_n33"))
    _check_same(layer_spec("minimind", n_experts=8, name="minimind_e8"))
    _check_same(layer_spec("tiny_f32"))


def test_rejects_sizes_past_the_scratch():
    spec = layer_spec("gptoss", n_tokens=4096, name="gptoss_n4096")
    x = torch.empty(spec.n_tokens, spec.hidden, dtype=torch.bfloat16, device=DEV)
    lg = torch.empty(spec.n_tokens, spec.n_experts, dtype=torch.bfloat16, device=DEV)
    w13 = torch.empty(spec.n_experts, 2 * spec.inter, spec.hidden, dtype=torch.bfloat16,
                      device=DEV)
    w2 = torch.empty(spec.n_experts, spec.hidden, spec.inter, dtype=torch.bfloat16, device=DEV)
    with pytest.raises(MoeError) as ei:
        moe_forward_noalloc(x, lg, w13, w2, spec.topk, "swiglu_oai", "interleaved")
    assert ei.value.status == N.MOE_ERR_SCRATCH


def test_graph_capture_replays():
    """A caller that cannot allocate: the call recorded into a HIP graph (after
    one eager call has resolved the scratch address) replays to the eager bits,
    several times, with eager work in between."""
    spec = layer_spec("gptoss", n_tokens=64, name="gptoss_n64")
    x, lg, w13, w2 = _dev(make_layer(spec))
    p = act_params(spec)
    routing = Routing.empty(spec.n_tokens, spec.n_experts, spec.topk, x.dtype, DEV)
    out = torch.empty_like(x)
    eager, _ = moe_forward(x, lg, w13, w2, spec.topk, spec.act, spec.layout, p)
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        moe_forward_noalloc(x, lg, w13, w2, spec.topk, spec.act, spec.layout, p, out=out,
                            routing=routing)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        moe_forward_noalloc(x, lg, w13, w2, spec.topk, spec.act, spec.layout, p, out=out,
                            routing=routing)
    for i in range(3):
        out.fill_(float("nan"))
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, eager), f"replay {i}"
        _ = (x.float() * 2).sum().item()
