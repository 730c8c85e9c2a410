"""MoE-layer forward benchmark on one MI355X.

    python bench.py [--steps K] [--warmup W] [--workload NAME]

One step is one pass of the whole layer over one batch of seeded synthetic
inputs already resident in HBM: moe_route (top-k, softmax, bitmatrix,
histogram, offsets, sorted indices), moe_experts_w13 (grouped GEMM + activation)
and moe_experts_w2 (grouped GEMM + routing weight + combine), back to back on
one stream.  HIP events between the three calls give per-stage device times;
events around the K steps give the step time.  Rank 0 prints one JSON line.

The default workload is the small-model layer (8 x 512 tokens, hidden 512,
intermediate 1408, top-1, 8 experts, SiLU-gated, bf16).  ``--workload`` picks
another named layer for study (tiny_f32, minimind_e4/e8/e16, gptoss_n{1,33,512,4096},
skewed_silu, skewed_relu2).
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import torch

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

from routing_grouped_expert_amd import (Routing, moe_workspace_bytes, prepare_experts_w13,  # noqa: E402
                                        prepare_experts_w2, prepare_route)
from routing_grouped_expert_amd.synth import act_params, layer_spec, make_layer  # noqa: E402

METRIC = "MoE layer tokens/s + routing µs/layer; % MFMA bf16 peak and % HBM BW"
PEAK_HBM_GBS = 8000.0
PEAK_TFLOPS = {"bf16": 2500.0, "f32": 157.3}


def workload(name: str):
    if name.startswith("minimind_e"):
        return layer_spec("minimind", n_experts=int(name[len("minimind_e"):]), name=name)
    if name.startswith("gptoss_n"):
        return layer_spec("gptoss", n_tokens=int(name[len("gptoss_n"):]), name=name)
    if name.startswith("skewed_"):
        return layer_spec("skewed", act=name[len("skewed_"):], name=name)
    if name == "tiny_f32":
        return layer_spec("tiny_f32")
    raise SystemExit(f"unknown workload {name!r}")


def describe(spec) -> str:
    extra = f" zipf_s={spec.zipf_s}" if spec.zipf_s else ""
    return (f"N={spec.n_tokens} H={spec.hidden} I={spec.inter} E={spec.n_experts} "
            f"k={spec.topk} {spec.act} {spec.layout} {spec.dtype}{extra}")


def algorithmic(spec, col_sum):
    """Algorithmic flops / bytes per launch of each stage (weights of touched
    experts read once, activations read and written once)."""
    s = 2 if spec.dtype == "bf16" else 4
    n, h, i, e, k = spec.n_tokens, spec.hidden, spec.inter, spec.n_experts, spec.topk
    m = n * k
    g = 2 if spec.act != "relu2" else 1
    et = int((col_sum > 0).sum())
    words = (e + 31) // 32
    route_b = n * e * s + n * k * (4 + s + 4 + 4 + s) + n * words * 4 + (2 * e + 1) * 4
    w13_f = 2 * m * g * i * h
    w13_b = et * g * i * h * s + n * h * s + m * i * s
    w2_f = 2 * m * h * i
    w2_b = et * h * i * s + m * i * s + m * h * s + (m * h * s + m * 4 + n * h * s if k > 1 else 0)
    return {"route": (0, route_b), "w13": (w13_f, w13_b), "w2": (w2_f, w2_b)}, et


def roofline(spec, flops, nbytes, ms):
    ridge = PEAK_TFLOPS[spec.dtype] * 1e12 / (PEAK_HBM_GBS * 1e9)
    if flops and flops / nbytes >= ridge:
        ach = flops / (ms * 1e-3) / 1e12
        return {"bound": "mfma", "achieved": round(ach, 2), "peak": PEAK_TFLOPS[spec.dtype],
                "unit": "TFLOP/s", "frac": round(ach / PEAK_TFLOPS[spec.dtype], 4)}
    ach = nbytes / (ms * 1e-3) / 1e9
    return {"bound": "hbm", "achieved": round(ach, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
            "frac": round(ach / PEAK_HBM_GBS, 4)}


def cpu_baseline(spec, layer, budget_s: float):
    """The CPU oracle as it stands, on this host, over a bounded token sample."""
    import numpy as np
    import oracle
    try:
        from threadpoolctl import threadpool_info
        threads = max([p.get("num_threads", 1) for p in threadpool_info()] or [1])
    except Exception:  # pragma: no cover
        threads = os.cpu_count()
    wd = "bf16" if spec.dtype == "bf16" else "f32"
    n = spec.n_tokens
    # a contiguous token sample sized so one oracle pass takes a few seconds at most
    sample = min(n, max(1, int(4096 * 512 * 1408 / (spec.hidden * spec.inter))))
    lg, x = layer.logits[:sample], layer.x[:sample]
    done, t0 = 0, time.perf_counter()
    reps = 0
    while True:
        r = oracle.route(lg, spec.topk, wd)
        oracle.moe_ffn(x, r.topk_idx, r.topk_w, layer.w13, layer.w2, spec.act, spec.layout,
                       act_params(spec))
        done += sample
        reps += 1
        if time.perf_counter() - t0 >= budget_s:
            break
    dt = time.perf_counter() - t0
    return {"value": round(done / dt, 1), "unit": "tokens/s", "cores": threads, "kind": "oracle",
            "sample": f"first {sample} of {n} tokens of the same layer (numpy float64 oracle: "
                      f"routing + masked per-expert FFN loop), {reps} passes in {dt:.1f} s"}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default="minimind_e8")
    ap.add_argument("--cpu-seconds", type=float, default=12.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py runs on one GPU only: this build has no multi-GPU path "
              "(see DESIGN.md on how the layer would shard)", file=sys.stderr)
        sys.exit(2)

    spec = workload(args.workload)
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    layer = make_layer(spec)
    x, lg = layer.x.to(dev), layer.logits.to(dev)
    w13, w2 = layer.w13.to(dev), layer.w2.to(dev)
    n, e, k = spec.n_tokens, spec.n_experts, spec.topk
    dt = x.dtype
    routing = Routing.empty(n, e, k, dt, dev)
    act = torch.empty(n * k, spec.inter, dtype=dt, device=dev)
    out = torch.empty_like(x)
    ws = torch.empty(moe_workspace_bytes(n, e, k, spec.hidden, spec.inter, dt), dtype=torch.uint8,
                     device=dev)
    stream = torch.cuda.current_stream(dev)
    p_route = prepare_route(lg, k, routing=routing, workspace=ws, stream=stream)
    p_w13 = prepare_experts_w13(x, w13, routing, spec.act, spec.layout, act_params(spec),
                                act_out=act, stream=stream)
    p_w2 = prepare_experts_w2(act, w2, routing, out=out, workspace=ws, stream=stream)

    K, W = args.steps, args.warmup
    for _ in range(W):
        p_route(); p_w13(); p_w2()
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(K)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(K):
        ev[i][0].record(stream)
        p_route()
        ev[i][1].record(stream)
        p_w13()
        ev[i][2].record(stream)
        p_w2()
        ev[i][3].record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    total_ms = ev[0][0].elapsed_time(ev[K - 1][3])
    stage_ms = {name: sum(ev[i][j].elapsed_time(ev[i][j + 1]) for i in range(K)) / K
                for j, name in enumerate(("route", "w13", "w2"))}
    ms_step = total_ms / K
    col_sum = routing.col_sum.cpu()
    work, et = algorithmic(spec, col_sum)
    # the w13 grouped GEMM is one kernel and the largest of the layer (it has
    # n_sets x the flops of the w2 GEMM); its launch is bracketed by events
    dom = "w13"
    f, b = work[dom]
    roof = roofline(spec, f, b, stage_ms[dom])
    roof.update({"kernel": "grouped_gemm (w13 + activation)", "traffic": None,
                 "algorithmic_bytes": b, "algorithmic_flops": f,
                 "avg_launch_us": round(stage_ms[dom] * 1e3, 2)})
    result = {
        "metric": METRIC,
        "value": round(n / (ms_step * 1e-3), 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": W,
        "ms_per_step": round(ms_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": spec.dtype,
        "data": "synthetic (seeded Gaussian inputs, random-init weights)",
        "config": {"workload": f"{spec.name}: {describe(spec)}", "n_tokens": n,
                   "experts_touched": et, "max_expert_rows": int(col_sum.max())},
        "routing_us_per_layer": round(stage_ms["route"] * 1e3, 2),
        "stage_us": {s: round(v * 1e3, 2) for s, v in stage_ms.items()},
        "wall_ms_per_step": round(wall / K * 1e3, 4),
        "roofline": roof,
    }
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(spec, layer, args.cpu_seconds)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
