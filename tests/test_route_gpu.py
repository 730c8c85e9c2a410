"""GPU routing (moe_route) against the CPU oracle: integer metadata bit-exact."""
import numpy as np
import pytest
import torch

import oracle
from routing_grouped_expert_amd import moe_route, Routing
from routing_grouped_expert_amd.synth import ROUTING_SWEEP, routing_logits
from tests.gpu_util import assert_routing_equal

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def _run(logits_cpu: torch.Tensor, k: int, where: str):
    print(f"[route] {where} N={logits_cpu.shape[0]} E={logits_cpu.shape[1]} k={k} "
          f"dtype={logits_cpu.dtype}", flush=True)
    ref = oracle.route(logits_cpu, k, "bf16" if logits_cpu.dtype == torch.bfloat16 else "f32")
    gpu = moe_route(logits_cpu.to(DEV), k)
    torch.cuda.synchronize()
    return assert_routing_equal(gpu, ref, where), gpu


@pytest.mark.parametrize("n,e,k", ROUTING_SWEEP, ids=[f"n{n}-e{e}-k{k}" for n, e, k in ROUTING_SWEEP])
def test_routing_sweep_bit_exact(n, e, k):
    _run(routing_logits(n, e, "bf16", seed=n + e), k, "sweep")


EDGE = [
    (256, 32, 4, "bf16"),    # exactly one block (fused single launch)
    (255, 32, 4, "bf16"),
    (257, 32, 4, "bf16"),    # two blocks, ragged tail
    (1000, 6, 2, "bf16"),    # E not a multiple of the 16-byte vector: scalar loads
    (777, 33, 3, "bf16"),
    (33, 8, 2, "f32"),       # fp32 logits (tiny layer)
    (600, 5, 5, "f32"),      # k == E
    (700, 64, 16, "bf16"),   # largest top-k
    (1500, 256, 8, "bf16"),  # largest expert count
    (300, 1, 1, "bf16"),     # single expert
    (40, 64, 8, "bf16"),     # N*k < E-ish: many empty experts
    (5000, 128, 1, "f32"),
    (4096, 32, 2, "bf16"),   # compact single-workgroup path at its limits
    (4097, 8, 1, "bf16"),    # one token past it: multi-block
    (4096, 16, 1, "f32"),    # compact path, fp32 logits
    (2049, 3, 2, "bf16"),    # compact path, scalar loads, ragged 64-token groups
    (8191, 256, 16, "bf16"),   # 64-token blocks: widest layer, ragged last block
    (12345, 256, 16, "bf16"),  # one lane a token from 8192 tokens at 256 experts
    (16385, 32, 4, "bf16"),  # first batch back on 256-token blocks, one-token tail
    (129, 128, 4, "bf16"),   # past 128 tokens, more than 64 experts: 64-token blocks
    (256, 256, 8, "bf16"),   # the same at the one-workgroup path's former limit
    (200, 128, 4, "f32"),    # fp32 logits on that path
    (256, 64, 16, "bf16"),   # 64 experts stay on the one-workgroup path up to 256 tokens
    # one token: the single-wave kernel
    (1, 256, 16, "bf16"),    # widest layer, largest top-k
    (1, 33, 3, "bf16"),      # scalar loads (E not a multiple of the 16-byte vector)
    (1, 200, 8, "f32"),      # fp32 logits over all 64 lanes
    (1, 5, 5, "f32"),        # k == E
    (1, 1, 1, "bf16"),       # single expert
    # one lane a token (32768 tokens and more, a power-of-two expert count)
    (32768 + 29, 256, 16, "bf16"),  # widest layer, largest top-k, ragged last block
    (32768, 8, 1, "bf16"),   # one chunk a row, top-1
    (70001, 64, 8, "bf16"),  # more than 1024 blocks: two rounds of the count scan
    (32800, 40, 3, "bf16"),  # not a power of two: back on the cooperative top-k
    (32768 + 1, 32, 4, "bf16"),   # rows of four chunks, one-token tail, staged scatter
    (32767, 32, 4, "bf16"),       # one token short of it: cooperative top-k
    (8192, 256, 8, "bf16"),       # the lane path's first batch at 256 experts
    (12287, 128, 4, "bf16"),      # 128 experts: cooperative one token short of 12288
    (12288, 128, 4, "bf16"),      # and the lane path from there
    (16385, 64, 8, "bf16"),       # 64 experts: the lane path past 64-token blocks
    (40000, 128, 2, "bf16"),      # two phases of 64 experts, top-2 vector stores
    (33000, 16, 8, "bf16"),       # top-8 of 16 experts (vector stores, staged scatter)
    (65536, 256, 8, "bf16"),      # four phases, two-word-vector bitmatrix rows
    # cooperative top-k past 256 blocks of 256 tokens: count rows prefix-summed once
    (65536 + 257, 40, 3, "bf16"),   # 258 blocks, ragged last one, odd expert count
    (70001, 128, 4, "f32"),         # fp32 logits
    (300000, 32, 8, "f32"),         # 1172 blocks: two rounds of the count scan
]


@pytest.mark.parametrize("n,e,k,dt", EDGE, ids=[f"n{a}-e{b}-k{c}-{d}" for a, b, c, d in EDGE])
def test_routing_edges(n, e, k, dt):
    _run(routing_logits(n, e, dt, seed=7 * n + e), k, "edge")


def test_routing_forced_ties_and_signed_zero():
    g = torch.Generator().manual_seed(3)
    lg = torch.randint(-2, 3, (3000, 48), generator=g).to(torch.float32)
    lg[lg == 0] = torch.where(torch.rand(int((lg == 0).sum()), generator=g) < 0.5, -0.0, 0.0)
    for dt in (torch.bfloat16, torch.float32):
        _run(lg.to(dt), 4, f"ties-{dt}")
    _run(torch.full((500, 16), 0.75).to(torch.bfloat16), 3, "all-equal")
    # one token: ties and signed zeros through the single-wave kernel
    for dt in (torch.bfloat16, torch.float32):
        _run(lg[:1].to(dt), 4, f"ties-one-{dt}")
        _run(torch.tensor([[0.0, -0.0, 1.0, 1.0, -0.0, 0.0, 1.0, -2.0, 0.0]]).to(dt), 6,
             f"signed-zero-one-{dt}")
    _run(torch.full((1, 40), -1.5).to(torch.bfloat16), 7, "all-equal-one")


def test_routing_lane_path_ties_and_share():
    """Forced ties and signed zeros, and an expert share, on the one-lane-a-token
    path."""
    g = torch.Generator().manual_seed(5)
    lg = torch.randint(-2, 3, (40000, 64), generator=g).to(torch.float32)
    lg[lg == 0] = torch.where(torch.rand(int((lg == 0).sum()), generator=g) < 0.5, -0.0, 0.0)
    _run(lg.to(torch.bfloat16), 6, "lane-ties")
    from routing_grouped_expert_amd import moe_route_ep
    lg = routing_logits(50001, 128, "bf16", seed=9)
    for lo, nl in ((5, 37), (0, 128), (96, 32)):
        print(f"[route] lane-share N=50001 E=128 k=4 share=[{lo},{lo + nl})", flush=True)
        ref = oracle.route_ep(lg, 4, "bf16", lo, nl)
        gpu = moe_route_ep(lg.to(DEV), 4, lo, nl)
        torch.cuda.synchronize()
        assert_routing_equal(gpu, ref, f"lane-share[{lo},{lo + nl})")


def test_routing_skewed_zipf():
    _run(routing_logits(16384, 64, "bf16", seed=0, zipf_s=1.1), 8, "zipf")


def test_routing_empty_is_noop():
    lg = torch.empty(0, 32, dtype=torch.bfloat16, device=DEV)
    r = moe_route(lg, 4)
    torch.cuda.synchronize()
    assert r.topk_idx.shape == (0, 4)


def test_routing_deterministic():
    lg = routing_logits(65536, 128, "bf16", seed=11).to(DEV)
    a = moe_route(lg, 4)
    b = moe_route(lg, 4)
    torch.cuda.synchronize()
    for f in ("topk_idx", "topk_w", "bitmatrix", "col_sum", "offsets", "col_sorted",
              "row_sorted", "gate_scal"):
        assert torch.equal(getattr(a, f), getattr(b, f)), f
