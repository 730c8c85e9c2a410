"""GEMM2 and the scatter-combine as separate calls (moe_experts_w2_rows then
moe_combine) give the same bits as moe_experts_w2, which runs them in one
call; moe_combine alone sums each token's slots as the layer's definition
says (the weighted expert outputs added back into the token rows, minimind
issue #835, "Summary")."""
import numpy as np
import pytest
import torch

import oracle
from routing_grouped_expert_amd import (moe_combine, moe_experts_w13, moe_experts_w2,
                                        moe_experts_w2_rows, moe_route, moe_route_ep)
from routing_grouped_expert_amd.synth import LayerSpec, act_params, make_layer

pytestmark = pytest.mark.gpu
DEV = "cuda:0"

CASES = [
    # (name, N, H, I, E, k, dtype, share)
    ("top1-direct", 700, 256, 192, 8, 1, "bf16", None),
    ("k2-tiles", 1500, 256, 384, 6, 2, "bf16", None),
    ("k4-decode", 6, 2880, 2880, 32, 4, "bf16", None),      # w2 and combine in one kernel
    ("k8-f32", 300, 128, 96, 16, 8, "f32", None),
    ("k4-share", 400, 128, 256, 16, 4, "bf16", (4, 6)),    # slots outside the share skipped
]


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_rows_then_combine_equals_w2(case):
    name, n, h, i, e, k, dt, share = case
    spec = LayerSpec(name, n_tokens=n, hidden=h, inter=i, n_experts=e, topk=k, dtype=dt,
                     seed=n + k)
    print(f"[combine] {spec} share={share}", flush=True)
    layer = make_layer(spec)
    x, lg = layer.x.to(DEV), layer.logits.to(DEV)
    w13, w2 = layer.w13.to(DEV), layer.w2.to(DEV)
    if share:
        lo, nl = share
        r = moe_route_ep(lg, k, lo, nl)
        w13, w2 = w13[lo:lo + nl].contiguous(), w2[lo:lo + nl].contiguous()
    else:
        r = moe_route(lg, k)
    a = moe_experts_w13(x, w13, r, "silu")
    want = moe_experts_w2(a, w2, r)
    y = torch.zeros(n * k, h, dtype=x.dtype, device=DEV)
    moe_experts_w2_rows(a, w2, r, y_sorted=y)
    got = moe_combine(y, r)
    torch.cuda.synchronize()
    assert torch.equal(got, want), f"{name}: rows + combine != moe_experts_w2"


@pytest.mark.parametrize("dt,k", [("bf16", 8), ("bf16", 3), ("f32", 16)])
def test_combine_sums_slots(dt, k):
    """out[t] is the sum of the token's k sorted rows: within one rounding of
    the float64 sum (an fp32 sum of at most 16 terms is far inside one ulp of
    the output dtype, so only a value next to a rounding boundary can land one
    step away in bf16; fp32 keeps the fp32 sum's own bound)."""
    n, e, h = 1000, 32, 136
    spec = LayerSpec("comb", n_tokens=n, hidden=h, inter=8, n_experts=e, topk=k, dtype=dt,
                     seed=7)
    layer = make_layer(spec)
    r = moe_route(layer.logits.to(DEV), k)
    g = torch.Generator("cpu").manual_seed(3)
    y = torch.randn(n * k, h, generator=g).to(layer.x.dtype)
    out = moe_combine(y.to(DEV), r)
    torch.cuda.synchronize()
    ref_r = oracle.route(layer.logits, k, dt)
    y64 = y.double().numpy()
    ref = y64[ref_r.row_sorted.reshape(n, k)].sum(axis=1)
    got = out.double().cpu().numpy()
    if dt == "bf16":
        ulp = np.exp2(np.floor(np.log2(np.maximum(np.abs(ref), 1e-30))) - 7)
        assert np.all(np.abs(got - ref) <= ulp * 1.0 + 1e-30), "combine off by more than 1 ulp"
    else:
        bound = k * 2.0 ** -24 * np.abs(y64[ref_r.row_sorted.reshape(n, k)]).sum(axis=1)
        assert np.all(np.abs(got - ref) <= bound + 1e-30)
