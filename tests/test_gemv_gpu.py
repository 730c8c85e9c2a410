"""Decode-sized layers (at most 128 tokens, bf16, few rows per expert), which run
the expert GEMMs as grouped matrix-vector products, against the CPU oracle.

The cases cover every epilogue (gated with and without the clamp, ReLU^2, the
routing weight into sorted rows and, with one expert per token, straight into
the output), both w13 layouts, K from one partial piece a lane up to 4096
(8 pieces a lane), output widths that end inside a workgroup's column block,
experts holding more rows than one LDS group (all tokens on one expert), an
expert-parallel share, and the routing weight on the input rows.
"""
import numpy as np
import pytest
import torch

import oracle
from routing_grouped_expert_amd import moe_experts, moe_experts_weighted_input, moe_route
from routing_grouped_expert_amd.synth import LayerSpec, act_params, layer_spec
from tests.test_ep_gpu import _share_spec, run_share
from tests.test_moe_gpu import run_layer
from tests.gpu_util import assert_output_close

pytestmark = pytest.mark.gpu
DEV = "cuda:0"

CASES = [
    # (name, N, H, I, E, k, act, layout, params)
    ("n1-silu-packed", 1, 136, 200, 6, 2, "silu", "packed", {}),
    ("n2-oai-interleaved", 2, 2880, 2880, 32, 4, "swiglu_oai", "interleaved",
     {"alpha": 1.702, "beta": 1.0, "limit": 7.0}),
    ("n3-oai-packed", 3, 264, 72, 8, 3, "swiglu_oai", "packed",
     {"alpha": 1.702, "beta": 1.0, "limit": 0.8}),
    ("n5-relu2-top1", 5, 520, 1032, 5, 1, "relu2", "packed", {}),
    ("n8-silu-top1", 8, 64, 64, 3, 1, "silu", "interleaved", {"limit": 0.5}),
    ("n7-relu2-k2", 7, 96, 160, 7, 2, "relu2", "packed", {}),
    ("n4-ragged-cols", 4, 1032, 520, 9, 2, "silu", "packed", {}),
    ("n24-k2", 24, 256, 384, 16, 2, "silu", "packed", {}),
    ("n32-top1", 32, 136, 200, 16, 1, "relu2", "packed", {}),
    # 4-5 rows an expert: w13 on the MFMA tiles, w2 as matrix-vector products
    ("n20-w2-only", 20, 256, 384, 8, 2, "silu", "packed", {}),
    ("n9-oai-w2-only", 9, 264, 200, 9, 4, "swiglu_oai", "interleaved",
     {"alpha": 1.702, "beta": 1.0, "limit": 7.0}),
]

# Skewed logits send nearly every token to one expert: that expert holds more
# rows than one LDS group (K = 4096 stages 6 rows at a time, smaller K 8).
SKEWED = [
    ("skew-n32-k4096", 32, 4096, 256, 16, 1, "silu", "interleaved", {}),
    ("skew-n32-i4096", 32, 256, 4096, 24, 2, "swiglu_oai", "packed",
     {"alpha": 1.702, "beta": 1.0, "limit": 7.0}),
    ("skew-n20-small", 20, 128, 136, 24, 3, "silu", "packed", {}),
]


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_decode_layer(case):
    name, n, h, i, e, k, act, layout, params = case
    spec = LayerSpec(name, n_tokens=n, hidden=h, inter=i, n_experts=e, topk=k, dtype="bf16",
                     act=act, layout=layout, alpha=params.get("alpha"), beta=params.get("beta"),
                     limit=params.get("limit"), seed=7 * n + h)
    run_layer(spec)


@pytest.mark.parametrize("case", SKEWED, ids=[c[0] for c in SKEWED])
def test_decode_skewed(case):
    name, n, h, i, e, k, act, layout, params = case
    spec = LayerSpec(name, n_tokens=n, hidden=h, inter=i, n_experts=e, topk=k, dtype="bf16",
                     act=act, layout=layout, alpha=params.get("alpha"), beta=params.get("beta"),
                     limit=params.get("limit"), zipf_s=6.0, seed=5 * n + h)
    _, routing, _ = run_layer(spec)
    assert int(routing.col_sum.max()) > 8, "the skew should overfill one LDS group"


@pytest.mark.parametrize("n", [1, 8, 32, 96])
def test_decode_gptoss(n):
    run_layer(layer_spec("gptoss", n_tokens=n, name=f"gptoss_n{n}"))


def test_decode_deterministic():
    spec = layer_spec("gptoss", n_tokens=3, name="gptoss_n3")
    a, _, layer = run_layer(spec)
    b, _, _ = run_layer(spec)
    assert torch.equal(a, b)


@pytest.mark.parametrize("lo,nl", [(0, 5), (9, 7)])
def test_decode_share(lo, nl):
    run_share(_share_spec("gptoss", lo, nl, n_tokens=2, hidden=256, inter=384, n_experts=16))


def test_decode_weighted_input():
    spec = LayerSpec("wi-n4", n_tokens=4, hidden=264, inter=136, n_experts=8, topk=2,
                     dtype="bf16", act="swiglu_oai", layout="interleaved", alpha=1.702, beta=1.0,
                     limit=7.0, seed=11)
    from routing_grouped_expert_amd.synth import make_layer
    layer = make_layer(spec)
    r = moe_route(layer.logits.to(DEV), 2)
    out = moe_experts_weighted_input(layer.x.to(DEV), layer.w13.to(DEV), layer.w2.to(DEV), r,
                                     "swiglu_oai", "interleaved", act_params(spec))
    torch.cuda.synchronize()
    ref = oracle.moe_ffn_weighted_input(layer.x, r.topk_idx.cpu().numpy(),
                                        r.topk_w.cpu().double().numpy(), layer.w13, layer.w2,
                                        "swiglu_oai", "bf16", "interleaved", act_params(spec))
    print(f"[gemv] wi: {assert_output_close(out, ref, 'wi-n4')}", flush=True)
