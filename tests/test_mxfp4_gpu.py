"""GPU MXFP4 weights: the quantiser bit-exact against the oracle."""
import numpy as np
import pytest
import torch

import oracle
from routing_grouped_expert_amd import moe_quantize_mxfp4

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def _weights(e, rows, k, dt, seed):
    g = torch.Generator().manual_seed(seed)
    w = torch.randn(e, rows, k, generator=g) * 0.02
    w[0, 0, :32] = 0.0                                           # all-zero block
    if k >= 64:
        grid = torch.tensor([0, .5, 1, 1.5, 2, 3, 4, 6, -0., -.5, -1, -1.5, -2, -3, -4, -6])
        w[0, 1, 32:64] = grid[torch.randint(0, 16, (32,), generator=g)] * 2.0 ** -5
        w[0, 1, 32] = 6 * 2.0 ** -5                              # representable block
    w[-1, -1, -32:] *= 1e4                                       # large block
    w[-1, 0, :32] *= 1e-20                                       # tiny block
    return w.to({"bf16": torch.bfloat16, "f32": torch.float32}[dt])


@pytest.mark.parametrize("e,rows,k,dt", [(3, 40, 96, "bf16"), (2, 64, 2880, "bf16"),
                                        (4, 33, 64, "f32"), (1, 1, 32, "bf16")])
def test_quantize_bit_exact(e, rows, k, dt):
    print(f"[mxfp4-q] E={e} rows={rows} K={k} {dt}", flush=True)
    w = _weights(e, rows, k, dt, seed=e * rows + k)
    q, s = moe_quantize_mxfp4(w.to(DEV))
    torch.cuda.synchronize()
    rq, rs = oracle.quantize_mxfp4(w)
    gq, gs = q.cpu().numpy(), s.cpu().numpy().transpose(0, 2, 1)  # -> [E, rows, K/32]
    assert gq.shape == rq.shape and gs.shape == rs.shape
    bad = np.argwhere(gq != rq)
    assert bad.size == 0, f"{len(bad)} code bytes differ, first {tuple(bad[0])}: " \
                          f"gpu {gq[tuple(bad[0])]:#x} oracle {rq[tuple(bad[0])]:#x}"
    assert np.array_equal(gs, rs), f"{int((gs != rs).sum())} scale bytes differ"


# ---------------------------------------------------------------- MXFP4 layers

from routing_grouped_expert_amd import moe_experts, moe_forward_mxfp4, moe_experts_mxfp4  # noqa: E402
from routing_grouped_expert_amd.synth import LayerSpec, act_params, layer_spec, make_layer  # noqa: E402
from tests.gpu_util import assert_output_close, assert_routing_equal  # noqa: E402


class _Dequantised:
    """Expert weights dequantised one expert at a time (float64), for the oracle."""

    def __init__(self, q, s):
        self.q, self.s = q.cpu().numpy(), s.cpu().numpy()
        self.shape = (self.q.shape[0], self.q.shape[1], self.q.shape[2] * 2)

    def __getitem__(self, e):
        return oracle.dequantize_mxfp4(self.q[e], self.s[e].T)


def _quantised(layer):
    w13q, w13s = moe_quantize_mxfp4(layer.w13.to(DEV))
    w2q, w2s = moe_quantize_mxfp4(layer.w2.to(DEV))
    return w13q, w13s, w2q, w2s


MX = [
    # (name, N, H, I, E, k, act, layout, params)
    ("silu-packed", 33, 128, 256, 8, 2, "silu", "packed", {}),
    ("oai-interleaved", 100, 256, 192, 16, 4, "swiglu_oai", "interleaved",
     {"alpha": 1.702, "beta": 1.0, "limit": 7.0}),
    ("relu2", 77, 96, 160, 4, 2, "relu2", "packed", {}),
    ("top1", 300, 128, 128, 8, 1, "silu", "packed", {"limit": 3.0}),
    ("ktail", 64, 160, 96, 4, 3, "silu", "interleaved", {}),
    ("many-rows", 2048, 128, 128, 4, 2, "silu", "packed", {}),
    # decode-sized batches (matrix-vector kernel); the packed ones read the
    # scales of two row runs
    ("n1-oai-packed", 1, 256, 192, 16, 4, "swiglu_oai", "packed",
     {"alpha": 1.702, "beta": 1.0, "limit": 7.0}),
    ("n3-silu-interleaved", 3, 160, 96, 8, 3, "silu", "interleaved", {}),
    ("n8-relu2-top1", 8, 96, 160, 8, 1, "relu2", "packed", {}),
    # 2-3 rows an expert: w13 on the MFMA tiles, w2 as matrix-vector products
    ("n6-w2-only", 6, 128, 160, 8, 4, "silu", "packed", {}),
    ("n10-oai-w2-only", 10, 256, 192, 16, 4, "swiglu_oai", "interleaved",
     {"alpha": 1.702, "beta": 1.0, "limit": 7.0}),
    ("n24-skew-k4096", 24, 4096, 128, 32, 1, "silu", "packed", {"zipf_s": 6.0}),
    # prefill-sized: the 128-row ping-pong tiles for both GEMMs
    ("mq-oai-interleaved", 2500, 1024, 512, 4, 2, "swiglu_oai", "interleaved",
     {"alpha": 1.702, "beta": 1.0, "limit": 7.0}),
    ("mq-silu-packed-ktail", 2600, 1024, 416, 4, 2, "silu", "packed", {}),
    ("mq-relu2-top1", 5000, 1024, 512, 4, 1, "relu2", "packed", {}),
]


def _bf16_register_weight_low(m, e, nout, kdim, plain):
    """The bf16 layer's choice below 48 rows an expert: a register-weight tile
    (128 rows for plain layers from 16 rows an expert, 192 for gated ones from
    32), for K a multiple of 64, when its expected tiles cover the CUs (the
    host rule)."""
    if kdim % 64 or not ((16 if plain else 32) * e <= m < 48 * e):
        return False
    bm, bn = (128, 256) if plain else (192, 128)
    tiles = (m // bm + (min(m, e) + 1) // 2) * ((nout + bn - 1) // bn)
    return tiles >= torch.cuda.get_device_properties(0).multi_processor_count


def _same_kernels(n, k, e, h, i, act):
    """True when the MXFP4 and the bf16 layer take the same kernel for each of
    the two GEMMs (then the results are the same bits): both the matrix-vector
    kernel (at most 128 tokens and few rows an expert: w13 n * k <= 1.5 E for
    MXFP4 and <= 3 E for bf16, w2 <= 3 E and <= 5 E), or both the one-wave /
    32-row MFMA tiles (n * k < 48 E, outside the matrix-vector range, unless
    the bf16 layer takes its register-weight tile there)."""
    m = n * k

    def same(gv_mx, gv_16, rw):
        return (gv_mx and gv_16) or (not gv_mx and not gv_16 and m < 48 * e and not rw)

    small = n <= 128
    rw13 = _bf16_register_weight_low(m, e, i, h, act == "relu2")
    rw2 = _bf16_register_weight_low(m, e, h, i, True)
    # (at k > 1 and m <= E the bf16 layer folds the combine into its w2 kernel
    # and the MXFP4 layer does not: the fused kernel is built to give the same
    # bits, which this comparison then checks)
    return (same(small and 2 * m <= 3 * e, small and m <= 3 * e, rw13)
            and same(small and m <= 3 * e, small and m <= 5 * e, rw2))


@pytest.mark.parametrize("case", MX, ids=[c[0] for c in MX])
def test_mxfp4_layer(case):
    name, n, h, i, e, k, act, layout, params = case
    spec = LayerSpec(name, n_tokens=n, hidden=h, inter=i, n_experts=e, topk=k, dtype="bf16",
                     act=act, layout=layout, alpha=params.get("alpha"), beta=params.get("beta"),
                     limit=params.get("limit"), zipf_s=params.get("zipf_s"), seed=n + 3 * h)
    print(f"[mxfp4] {spec}", flush=True)
    layer = make_layer(spec)
    w = _quantised(layer)
    x, lg = layer.x.to(DEV), layer.logits.to(DEV)
    out, routing = moe_forward_mxfp4(x, lg, *w, k, act, layout, act_params(spec))
    torch.cuda.synchronize()
    ref_r = oracle.route(layer.logits, k, "bf16")
    assert_routing_equal(routing, ref_r, f"{name}.routing")
    d13, d2 = _Dequantised(w[0], w[1]), _Dequantised(w[2], w[3])
    ref = oracle.moe_ffn(layer.x, ref_r.topk_idx, ref_r.topk_w, d13, d2, act, layout,
                         act_params(spec))
    print(f"[mxfp4] {name}: {assert_output_close(out, ref, name)}", flush=True)
    if _same_kernels(n, k, e, h, i, act):
        deq13 = torch.stack([torch.from_numpy(d13[j]) for j in range(e)]).to(torch.bfloat16)
        deq2 = torch.stack([torch.from_numpy(d2[j]) for j in range(e)]).to(torch.bfloat16)
        ref16 = moe_experts(x, deq13.to(DEV), deq2.to(DEV), routing, act, layout,
                            act_params(spec))
        torch.cuda.synchronize()
        assert torch.equal(out, ref16), "MXFP4 path != bf16 path on the dequantised weights"


@pytest.mark.timeout(900)
@pytest.mark.parametrize("n", [1, 33, 512, 4096])
def test_mxfp4_gptoss(n):
    spec = layer_spec("gptoss", n_tokens=n, name=f"gptoss_n{n}_mxfp4")
    print(f"[mxfp4] {spec}", flush=True)
    layer = make_layer(spec)
    w = _quantised(layer)
    x, lg = layer.x.to(DEV), layer.logits.to(DEV)
    out, routing = moe_forward_mxfp4(x, lg, *w, spec.topk, spec.act, spec.layout,
                                     act_params(spec))
    torch.cuda.synchronize()
    ref_r = oracle.route(layer.logits, spec.topk, "bf16")
    assert_routing_equal(routing, ref_r, "gptoss mxfp4 routing")
    ref = oracle.moe_ffn(layer.x, ref_r.topk_idx, ref_r.topk_w, _Dequantised(w[0], w[1]),
                         _Dequantised(w[2], w[3]), spec.act, spec.layout, act_params(spec))
    print(f"[mxfp4] gptoss n={n}: {assert_output_close(out, ref, spec.name)}", flush=True)


def test_mxfp4_argument_checks():
    from routing_grouped_expert_amd import MoeError, moe_route
    spec = LayerSpec("chk", n_tokens=16, hidden=128, inter=128, n_experts=4, topk=2,
                     dtype="bf16", seed=1)
    layer = make_layer(spec)
    w = _quantised(layer)
    r = moe_route(layer.logits.to(DEV), 2)
    with pytest.raises(TypeError):  # fp32 layers are not supported with MXFP4 weights
        moe_experts_mxfp4(layer.x.float().to(DEV), *w, r, "silu")
    with pytest.raises(ValueError):
        moe_experts_mxfp4(layer.x.to(DEV), w[0], w[1][:, :2].contiguous(), w[2], w[3], r, "silu")
