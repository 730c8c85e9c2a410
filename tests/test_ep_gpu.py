"""GPU expert-parallel share (moe_route_ep / moe_experts_ep / moe_forward_ep)
against the CPU oracle (route_ep, moe_ffn_share): routing metadata bit-exact,
layer contributions within the layer tolerance, shares summing to the layer."""
import pytest
import torch

import oracle
from routing_grouped_expert_amd import (moe_experts_ep, moe_forward, moe_forward_ep, moe_route,
                                        moe_route_ep, MoeError)
from routing_grouped_expert_amd.synth import act_params, layer_spec, make_layer, routing_logits
from tests.gpu_util import INT_FIELDS, assert_output_close, assert_routing_equal

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
ALL_FIELDS = INT_FIELDS + ("topk_w", "gate_scal")


def _wdt(t):
    return "bf16" if t.dtype == torch.bfloat16 else "f32"


def _route(lg, k, lo, nl, where):
    print(f"[ep-route] {where} N={lg.shape[0]} E={lg.shape[1]} k={k} share=({lo},{nl}) "
          f"{lg.dtype}", flush=True)
    ref = oracle.route_ep(lg, k, _wdt(lg), lo, nl)
    gpu = moe_route_ep(lg.to(DEV), k, lo, nl)
    torch.cuda.synchronize()
    assert_routing_equal(gpu, ref, where)
    return gpu, ref


ROUTE_CASES = [
    (200, 64, 4, "bf16", 8, 8),        # single-workgroup path
    (256, 32, 4, "bf16", 5, 11),       # single workgroup, share not word aligned
    (257, 32, 4, "bf16", 0, 1),        # block path, one local expert
    (3000, 128, 4, "bf16", 96, 32),    # last share of an EP4 group
    (3000, 128, 4, "bf16", 17, 45),    # share straddling bitmatrix words
    (1000, 6, 2, "bf16", 2, 3),        # E not a multiple of the vector: scalar loads
    (777, 8, 4, "f32", 6, 2),          # fp32 logits, fewer local experts than k
    (1500, 256, 8, "bf16", 200, 56),   # largest expert count
    (40, 64, 8, "bf16", 60, 4),
    (5000, 16, 1, "bf16", 12, 4),      # top-1
    (65536, 128, 4, "bf16", 16, 16),   # EP8 share at the largest routing batch
    (1, 128, 4, "bf16", 17, 45),       # one token (single-wave kernel), share across words
    (1, 256, 16, "bf16", 224, 32),     # one token, last share of the widest layer
    (1, 32, 4, "f32", 8, 8),           # one token, fp32
]


@pytest.mark.parametrize("n,e,k,dt,lo,nl", ROUTE_CASES,
                         ids=[f"n{a}-e{b}-k{c}-{d}-s{f}x{g}" for a, b, c, d, f, g in ROUTE_CASES])
def test_route_ep_bit_exact(n, e, k, dt, lo, nl):
    _route(routing_logits(n, e, dt, seed=3 * n + e + lo), k, lo, nl, "share")


@pytest.mark.parametrize("n", [1, 100, 3000])
def test_route_ep_whole_layer_equals_route(n):
    lg = routing_logits(n, 64, "bf16", seed=n).to(DEV)
    a = moe_route(lg, 4)
    b = moe_route_ep(lg, 4, 0, 64)
    torch.cuda.synchronize()
    for f in ALL_FIELDS:
        assert torch.equal(getattr(a, f), getattr(b, f)), f


@pytest.mark.parametrize("n", [1, 150, 2000])
def test_route_ep_share_nobody_chose(n):
    lg = routing_logits(n, 32, "f32", seed=5)
    lg[:, 8:16] = -40.0                        # never in any token's top-4
    gpu, ref = _route(lg, 4, 8, 8, "unchosen")
    assert int(ref.offsets[-1]) == 0
    assert (gpu.row_sorted == -1).all() and (gpu.col_sorted == -1).all()


def test_route_ep_argument_checks():
    lg = routing_logits(64, 16, "bf16").to(DEV)
    for lo, nl in [(-1, 4), (0, 0), (13, 4), (16, 1)]:
        with pytest.raises((MoeError, ValueError)):
            moe_route_ep(lg, 2, lo, nl)


def _share_spec(family, lo, nl, **kw):
    base = layer_spec(family, **kw)
    return base.with_(local_offset=lo, n_local=nl, name=f"{base.name}_s{lo}x{nl}")


def run_share(spec):
    print(f"[ep-moe] {spec}", flush=True)
    layer = make_layer(spec)
    lo, nl = spec.local_offset, spec.n_local
    d = {k: getattr(layer, k).to(DEV) for k in ("x", "logits", "w13", "w2")}
    out, routing = moe_forward_ep(d["x"], d["logits"], d["w13"], d["w2"], spec.topk, lo, spec.act,
                                  spec.layout, act_params(spec))
    torch.cuda.synchronize()
    ref_r = oracle.route_ep(layer.logits, spec.topk, spec.dtype, lo, nl)
    assert_routing_equal(routing, ref_r, f"{spec.name}.routing")
    ref = oracle.moe_ffn_share(layer.x, ref_r.topk_idx, ref_r.topk_w, layer.w13, layer.w2,
                               spec.act, lo, spec.layout, act_params(spec))
    stats = assert_output_close(out, ref, spec.name)
    print(f"[ep-moe] {spec.name}: {stats}", flush=True)
    # tokens with no slot in the share get exact zero rows
    none_local = (ref_r.row_sorted.reshape(spec.n_tokens, -1) < 0).all(axis=1)
    if none_local.any():
        assert not out[torch.from_numpy(none_local).to(DEV)].any()
    return out, routing, layer


SHARES = [
    ("silu_k4", dict(family="minimind", n_tokens=300, hidden=128, inter=256, n_experts=16,
                     topk=4), (4, 5)),
    ("relu2_k2", dict(family="minimind", n_tokens=700, hidden=256, inter=192, n_experts=8,
                      topk=2, act="relu2"), (0, 3)),
    ("oai_interleaved", dict(family="gptoss", n_tokens=333, hidden=256, inter=384, n_experts=16),
     (12, 4)),
    ("top1", dict(family="minimind", n_tokens=1000, hidden=128, inter=128, n_experts=8), (2, 3)),
    ("tiny_f32", dict(family="tiny_f32"), (1, 2)),
    ("fewer_local_than_k", dict(family="minimind", n_tokens=500, hidden=128, inter=128,
                                n_experts=8, topk=4), (3, 2)),
]


@pytest.mark.parametrize("case", SHARES, ids=[c[0] for c in SHARES])
def test_share_layer(case):
    name, kw, (lo, nl) = case
    kw = dict(kw)
    run_share(_share_spec(kw.pop("family"), lo, nl, **kw))


@pytest.mark.timeout(600)
def test_gptoss_ep8_share_full_size():
    # one GPU of an EP8 group over gpt-oss-sized experts: 16 of 128 experts
    run_share(_share_spec("gptoss", 0, 16, n_tokens=4096))


@pytest.mark.parametrize("k,dt", [(2, "bf16"), (1, "f32"), (4, "f32")])
def test_shares_sum_to_layer(k, dt):
    spec = layer_spec("minimind", n_tokens=600, hidden=128, inter=256, n_experts=16, topk=k,
                      dtype=dt)
    print(f"[ep-sum] {spec}", flush=True)
    layer = make_layer(spec)
    d = {f: getattr(layer, f).to(DEV) for f in ("x", "logits", "w13", "w2")}
    full, _ = moe_forward(d["x"], d["logits"], d["w13"], d["w2"], k, "silu")
    tot = torch.zeros(spec.n_tokens, spec.hidden, dtype=torch.float64, device=DEV)
    for lo in range(0, 16, 4):
        o, _ = moe_forward_ep(d["x"], d["logits"], d["w13"][lo:lo + 4].contiguous(),
                              d["w2"][lo:lo + 4].contiguous(), k, lo, "silu")
        tot += o.double()
    torch.cuda.synchronize()
    ref_r = oracle.route(layer.logits, k, dt)
    ref = oracle.moe_ffn(layer.x, ref_r.topk_idx, ref_r.topk_w, layer.w13, layer.w2, "silu")
    assert_output_close(tot.to(full.dtype), ref, "sum of shares")
    if k == 1:  # one slot per token: exactly one share writes each row
        assert torch.equal(tot.to(full.dtype), full)


def test_forward_ep_equals_route_then_experts():
    spec = _share_spec("minimind", 3, 6, n_tokens=900, hidden=128, inter=256, n_experts=12,
                       topk=3)
    layer = make_layer(spec)
    d = {f: getattr(layer, f).to(DEV) for f in ("x", "logits", "w13", "w2")}
    o1, r1 = moe_forward_ep(d["x"], d["logits"], d["w13"], d["w2"], 3, 3, "silu")
    r2 = moe_route_ep(d["logits"], 3, 3, 6)
    o2 = moe_experts_ep(d["x"], d["w13"], d["w2"], r2, "silu")
    torch.cuda.synchronize()
    assert torch.equal(o1, o2)
    for f in ALL_FIELDS:
        assert torch.equal(getattr(r1, f), getattr(r2, f)), f
