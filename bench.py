"""MoE-layer forward benchmark on one MI355X.

    python bench.py [--steps K] [--warmup W] [--workload NAME]

One step is one pass of the whole layer over one batch of seeded synthetic
inputs already resident in HBM: one moe_forward call through the C ABI, which
enqueues the routing kernels (top-k, softmax, bitmatrix, histogram, offsets,
sorted indices), the w13 grouped GEMM with the activation, the w2 grouped GEMM
with the routing weight, and the combine.  W untimed steps, then K steps
between two HIP events on the launch stream give the step time.

Per-kernel device times: K back-to-back calls of each stage's C call
(moe_route, moe_experts_w13, moe_experts_w2_rows -- GEMM2 alone --,
moe_combine) captured in a HIP graph on a stream of their own and replayed
between two events on that stream, so no host launch cost sits between the
calls; a stage's average still includes the short gap between consecutive
kernels.  The stage with the longest single-kernel time is the dominant kernel
of the roofline line.  Rank 0 prints one JSON line.

The default workload is the largest layer: 16384 tokens, hidden 4096,
intermediate 1536, 64 experts, top-8, Zipf-skewed router logits, SiLU-gated,
bf16.  ``--workload`` picks another named layer (tiny_f32, minimind_e4/e8/e16,
gptoss_n{1,33,512,4096}, skewed_silu, skewed_relu2, ...).
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

from routing_grouped_expert_amd import (Routing, moe_workspace_bytes,  # noqa: E402
                                        prepare_combine, prepare_experts_w13,
                                        prepare_experts_w2, prepare_experts_w2_rows,
                                        prepare_forward, prepare_forward_ep,
                                        prepare_gate_forward, prepare_gate_route, prepare_route,
                                        prepare_route_ep, moe_quantize_mxfp4,
                                        prepare_experts_mxfp4, prepare_forward_mxfp4)
from routing_grouped_expert_amd.synth import (act_params, layer_spec, make_layer,  # noqa: E402
                                              router_inputs, routing_logits)

METRIC = "MoE layer tokens/s + routing µs/layer; % MFMA bf16 peak and % HBM BW"
PEAK_HBM_GBS = 8000.0
PEAK_TFLOPS = {"bf16": 2500.0, "f32": 157.3}


def workload(name: str):
    if name.endswith("_mxfp4"):  # the same layer with MXFP4 expert weights
        return workload(name[:-len("_mxfp4")]).with_(name=name)
    if name.startswith("gptoss_ep"):
        # one GPU of an expert-parallel group of G: the first E/G experts of the
        # gpt-oss-sized layer, every token routed over all E
        g, n = name[len("gptoss_ep"):].split("_n")
        base = layer_spec("gptoss", n_tokens=int(n))
        return base.with_(name=name, local_offset=0, n_local=base.n_experts // int(g))
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
    if spec.n_local is not None:
        extra += f" share=experts[{spec.local_offset}:{spec.local_offset + spec.n_local}]"
    return (f"N={spec.n_tokens} H={spec.hidden} I={spec.inter} E={spec.n_experts} "
            f"k={spec.topk} {spec.act} {spec.layout} {spec.dtype}{extra}")


def algorithmic(spec, col_sum):
    """Algorithmic flops / bytes per launch of each stage (weights of touched
    experts read once, activations read and written once).  ``col_sum`` is the
    measured histogram; its total is the number of routed rows (N*k, or the
    rows of the local experts for an expert-parallel share)."""
    s = 2 if spec.dtype == "bf16" else 4
    n, h, i, e, k = spec.n_tokens, spec.hidden, spec.inter, spec.n_experts, spec.topk
    m = int(col_sum.sum())
    g = 2 if spec.act != "relu2" else 1
    et = int((col_sum > 0).sum())
    words = (spec.n_weights + 31) // 32
    route_b = n * e * s + n * k * (4 + s + 4 + 4 + s) + n * words * 4 + (2 * e + 1) * 4
    w13_f = 2 * m * g * i * h
    w13_b = et * g * i * h * s + n * h * s + m * i * s
    w2_f = 2 * m * h * i
    # GEMM2 writes the weighted sorted rows (k > 1) or, with one slot a token,
    # the output rows themselves
    w2_b = et * h * i * s + m * i * s + m * h * s
    work = {"route": (0, route_b), "w13": (w13_f, w13_b), "w2": (w2_f, w2_b)}
    if k > 1:  # each token's k rows read (with their positions) and its row written once
        work["combine"] = (0, m * h * s + n * k * 4 + n * h * s)
    return work, et


MXFP4_BYTES = 17 / 32  # bytes per weight: a 4-bit code plus a 1-byte scale per 32


def algorithmic_mxfp4(spec, col_sum):
    """Flops / bytes of one experts call (both grouped GEMMs) with MXFP4 weights:
    the touched experts' codes and scales read once, activations read and
    written once."""
    n, h, i, k = spec.n_tokens, spec.hidden, spec.inter, spec.topk
    m = int(col_sum.sum())
    g = 2 if spec.act != "relu2" else 1
    et = int((col_sum > 0).sum())
    flops = 2 * m * g * i * h + 2 * m * h * i
    nbytes = int(et * (g * i * h + h * i) * MXFP4_BYTES) + n * h * 2 + 2 * m * i * 2 + \
        (2 * m * h * 2 + m * 4 + n * h * 2 if k > 1 else n * h * 2)
    return flops, nbytes, et


def roofline(spec, flops, nbytes, ms):
    ridge = PEAK_TFLOPS[spec.dtype] * 1e12 / (PEAK_HBM_GBS * 1e9)
    if flops and flops / nbytes >= ridge:
        ach = flops / (ms * 1e-3) / 1e12
        return {"bound": "mfma", "achieved": round(ach, 2), "peak": PEAK_TFLOPS[spec.dtype],
                "unit": "TFLOP/s", "frac": round(ach / PEAK_TFLOPS[spec.dtype], 4)}
    ach = nbytes / (ms * 1e-3) / 1e9
    return {"bound": "hbm", "achieved": round(ach, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
            "frac": round(ach / PEAK_HBM_GBS, 4)}


def host_info() -> dict:
    """The host this run is on: CPU model and hardware threads, ROCm and HIP
    versions, GPU name and compute-unit count (the same GPU model on different
    hosts can time differently, so the record names the host)."""
    info = {"cpu_model": None, "cpu_threads": os.cpu_count(), "rocm": None,
            "hip_runtime": getattr(torch.version, "hip", None), "gpu": None, "gpu_cus": None}
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    info["cpu_model"] = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    try:
        with open("/opt/rocm/.info/version") as f:
            info["rocm"] = f.read().strip()
    except OSError:
        pass
    if torch.cuda.is_available():
        p = torch.cuda.get_device_properties(0)
        info["gpu"] = f"{p.name} ({getattr(p, 'gcnArchName', '?')})"
        info["gpu_cus"] = p.multi_processor_count
    return info


class ClockSampler:
    """Samples the GPU's current graphics clock (MHz, the mean over the XCDs)
    from the SMI library on a background thread.  Started early, since the
    library is slow to start; only samples taken in the clock pass (sustained())
    count.  Reports their median and range (None when the SMI library is not
    usable here)."""

    def __init__(self, period_s: float = 0.005):
        import threading
        self.period = period_s
        self.seconds, self.settle = 0.0, 0.0
        self.samples = []           # (perf_counter time, MHz)
        self.window = [None, None]
        self.error = None
        self._stop = threading.Event()
        self._thread = threading.Thread(target=self._run, daemon=True)

    def _read(self, smi, h):
        vals = []
        try:
            cur = smi.amdsmi_get_gpu_metrics_info(h).get("current_gfxclks")
            if isinstance(cur, (list, tuple)):
                vals = [v for v in cur if isinstance(v, (int, float)) and 0 < v < 10000]
        except Exception:
            vals = []
        if not vals:
            vals = [smi.amdsmi_get_clock_info(h, smi.AmdSmiClkType.GFX)["clk"]]
        return sum(vals) / len(vals)

    def _run(self):
        try:
            import amdsmi as smi
            smi.amdsmi_init()
            try:
                hs = smi.amdsmi_get_processor_handles()
                if len(hs) != 1:
                    raise RuntimeError(f"{len(hs)} GPUs visible to the SMI library")
                while not self._stop.is_set():
                    self.samples.append((time.perf_counter(), self._read(smi, hs[0])))
                    self._stop.wait(self.period)
            finally:
                smi.amdsmi_shut_down()
        except Exception as exc:  # no SMI access: the record says why
            self.error = f"{type(exc).__name__}: {exc}"[:160]

    def start(self):
        self._thread.start()
        return self

    def sustained(self, fn, seconds: float, settle: float = 1.2):
        """Runs fn back to back for `seconds` (after the timed region) and keeps
        the samples taken after the first `settle` seconds.  The SMI table is
        refreshed about once a second and holds its value in between, so a timed
        region of a few hundred milliseconds mostly reads the clock from before
        the load; this pass gives the clock the same step sustains."""
        self.seconds, self.settle = seconds, min(settle, seconds / 2)
        if seconds <= 0:
            self.error = self.error or "clock pass disabled"
            self._stop.set()
            return
        torch.cuda.synchronize()
        t = time.perf_counter()
        fn()
        torch.cuda.synchronize()
        # launch in chunks of ~20 ms of work, synchronising between them
        chunk = max(1, min(10000, int(0.02 / max(time.perf_counter() - t, 1e-6))))
        t0 = time.perf_counter()
        self.window[0] = t0 + self.settle
        while time.perf_counter() - t0 < seconds:
            for _ in range(chunk):
                fn()
            torch.cuda.synchronize()
        self.window[1] = time.perf_counter()
        self._stop.set()
        self._thread.join(timeout=5)

    def summary(self) -> dict:
        t0, t1 = self.window
        v = sorted(m for t, m in self.samples if t0 is not None and t1 is not None and t0 <= t <= t1)
        if not v:
            return {"median_mhz": None, "error": self.error or "no samples in the clock pass"}
        # the reading moves in steps (the SMI table holds a value for up to a
        # second), so few distinct values: median and range
        return {"median_mhz": round(v[len(v) // 2]), "min_mhz": round(v[0]),
                "max_mhz": round(v[-1]), "samples": len(v),
                "source": f"SMI graphics clock (mean over XCDs) while the step ran back to back "
                          f"for {self.seconds:g} s after the timed region, samples after the "
                          f"first {self.settle:g} s"}


def _oracle_threads() -> int:
    """Threads the oracle's numpy (BLAS) calls run on."""
    try:
        from threadpoolctl import threadpool_info
        return max([p.get("num_threads", 1) for p in threadpool_info()] or [1])
    except Exception:  # pragma: no cover
        return os.cpu_count()


def cpu_baseline(spec, layer, budget_s: float):
    """The CPU oracle as it stands, on this host, over a bounded token sample."""
    import oracle
    threads = _oracle_threads()
    wd = "bf16" if spec.dtype == "bf16" else "f32"
    n = spec.n_tokens
    share = spec.n_local is not None
    # a contiguous token sample sized so one oracle pass takes a few seconds at most
    sample = min(n, max(1, int(4096 * 512 * 1408 / (spec.hidden * spec.inter))))
    lg, x = layer.logits[:sample], layer.x[:sample]
    done, t0 = 0, time.perf_counter()
    reps = 0
    while True:
        if share:
            r = oracle.route_ep(lg, spec.topk, wd, spec.local_offset, spec.n_local)
            oracle.moe_ffn_share(x, r.topk_idx, r.topk_w, layer.w13, layer.w2, spec.act,
                                 spec.local_offset, spec.layout, act_params(spec))
        else:
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


def expert_kernel(spec, mxfp4: bool) -> str:
    """Which kernel family runs the expert GEMMs of this layer: the library takes
    the matrix-vector kernel for decode-sized bf16 batches (at most 128 tokens,
    N * topk <= 3 E for w13 (5 E for w2), or <= 1.5 E with MXFP4 weights;
    K <= 4096) and the MFMA tiles otherwise.  The label names the w13 kernel.
    Used for labels only."""
    n, m, e = spec.n_tokens, spec.n_tokens * spec.topk, spec.n_local or spec.n_experts
    fits = spec.dtype == "bf16" and n <= 128 and max(spec.hidden, spec.inter) <= 4096 and \
        (2 * m <= 3 * e if mxfp4 else m <= 3 * e)
    return "grouped_gemv" if fits else "grouped_gemm"


def stored_traffic(workload_name: str, stage: str):
    """HBM bytes per launch of a stage's kernel from the committed rocprofv3
    counter summary (FETCH_SIZE + WRITE_SIZE, each scaled by what the counter
    reads for a copy kernel of known size), or None when there is none or when
    the kernel's source file has changed since the counters were taken."""
    import hashlib
    import re
    path = os.path.join(ROOT, "profiles", "gemm_counters.md")
    try:
        text = open(path).read()
    except OSError:
        return None
    for m in re.finditer(r"traffic: workload=(\S+) stage=(\S+) src=(\S+) src_sha256=(\S+) "
                         r"fetch_bytes=(\d+) write_bytes=(\d+)", text):
        if m.group(1) != workload_name or m.group(2) != stage:
            continue
        src = os.path.join(ROOT, "routing_grouped_expert_amd", "csrc", m.group(3))
        try:
            sha = hashlib.sha256(open(src, "rb").read()).hexdigest()[:16]
        except OSError:
            return None
        if m.group(4) == sha:
            return int(m.group(5)) + int(m.group(6))
    return None


def step_stats(fn, steps: int, stream) -> dict:
    """Mean, and median / p10 / p90 over batches, of back-to-back step times."""
    # batches: the largest divisor of steps up to 20 that leaves >= 5 steps each,
    # so exactly `steps` steps are timed
    nb = max([d for d in range(1, 21) if steps % d == 0 and steps // d >= 5] or [1])
    per = steps // nb
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(nb + 1)]
    torch.cuda.synchronize()
    ev[0].record(stream)
    for bi in range(nb):
        for _ in range(per):
            fn()
        ev[bi + 1].record(stream)
    torch.cuda.synchronize()
    batch = sorted(ev[bi].elapsed_time(ev[bi + 1]) / per for bi in range(nb))
    q = lambda f: batch[min(nb - 1, int(f * nb))]
    return {"mean": ev[0].elapsed_time(ev[nb]) / (nb * per), "p10": q(0.1), "p50": q(0.5),
            "p90": q(0.9), "steps": nb * per}


def cold_stats(fns, reps: int, stream, dev) -> list:
    """Median time of each fn() run alone after a 512 MB write (more than the
    256 MB Infinity Cache and the L2s), outside the timed window."""
    flush = torch.empty(512 << 20, dtype=torch.uint8, device=dev)
    out = []
    for fn in fns:
        ts = []
        for _ in range(reps):
            flush.fill_(1)
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record(stream)
            fn()
            b.record(stream)
            torch.cuda.synchronize()
            ts.append(a.elapsed_time(b))
        ts.sort()
        out.append(ts[len(ts) // 2])
    del flush
    return out


def bench_route_only(args, name: str):
    """Routing-metadata workloads: route_n<N>_e<E>_k<k> (bf16 logits), with a
    _f32 suffix fp32 logits and weights."""
    import re
    m = re.fullmatch(r"route_n(\d+)_e(\d+)_k(\d+)(_f32)?", name)
    if not m:
        raise SystemExit(f"unknown workload {name!r}")
    n, e, k = (int(v) for v in m.groups()[:3])
    f32 = m.group(4) is not None
    clock = ClockSampler().start()
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    lg_cpu = routing_logits(n, e, "f32" if f32 else "bf16", seed=0)
    lg = lg_cpu.to(dev)
    routing = Routing.empty(n, e, k, torch.float32 if f32 else torch.bfloat16, dev)
    ws = torch.empty(max(1, moe_workspace_bytes(n, e, k)), dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream(dev)
    p_route = prepare_route(lg, k, routing=routing, workspace=ws, stream=stream)
    for _ in range(args.warmup):
        p_route()
    t0 = time.perf_counter()
    st = step_stats(p_route, args.steps, stream)
    wall = time.perf_counter() - t0
    clock.sustained(p_route, args.clock_seconds)
    cold = cold_stats([p_route], 20, stream, dev)[0]
    words = (e + 31) // 32
    es = 4 if f32 else 2  # logit and weight bytes
    nbytes = n * e * es + n * k * (4 + es + 4 + 4 + es) + n * words * 4 + (2 * e + 1) * 4
    ach = nbytes / (st["mean"] * 1e-3) / 1e9
    result = {
        "metric": METRIC, "value": round(n / (st["mean"] * 1e-3), 1), "unit": "tokens/s",
        "n_gpus": 1, "steps": st["steps"], "warmup": args.warmup,
        "ms_per_step": round(st["mean"], 5), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "f32" if f32 else "bf16", "data": "synthetic (seeded Gaussian logits)",
        "config": {"workload": f"{name}: routing metadata only, N={n} E={e} k={k} {'fp32' if f32 else 'bf16'} logits"},
        "routing_us_per_layer": round(st["mean"] * 1e3, 2),
        "step_us": {q: round(st[q] * 1e3, 2) for q in ("p10", "p50", "p90")},
        "cold_routing_us": round(cold * 1e3, 2),
        "wall_ms_per_step": round(wall / st["steps"] * 1e3, 4),
        "roofline": {"bound": "hbm", "achieved": round(ach, 1), "peak": PEAK_HBM_GBS,
                     "unit": "GB/s", "frac": round(ach / PEAK_HBM_GBS, 4),
                     "kernel": "routing (all routing kernels of one moe_route call)",
                     "traffic": None, "algorithmic_bytes": nbytes,
                     "avg_launch_us": round(st["mean"] * 1e3, 2)},
        "gpu_clock": clock.summary(),
        "host": host_info(),
    }
    if not args.no_cpu_baseline:
        import oracle
        sample = min(n, 4096)
        t0, reps = time.perf_counter(), 0
        while True:
            oracle.route(lg_cpu[:sample], k, "f32" if f32 else "bf16")
            reps += 1
            if time.perf_counter() - t0 >= args.cpu_seconds:
                break
        dt = time.perf_counter() - t0
        result["cpu_baseline"] = {"value": round(sample * reps / dt, 1), "unit": "tokens/s",
                                  "cores": 1, "kind": "oracle",
                                  "sample": f"first {sample} of {n} tokens, routing oracle, "
                                            f"{reps} passes in {dt:.1f} s"}
    print(json.dumps(result), flush=True)


def bench_gate_route(args, name: str):
    """Router GEMM + routing workloads: gate_n<N>_e<E>_h<H>_k<k> (bf16): x [N, H]
    and the gate weight [E, H] in, logits and routing metadata out, one
    moe_gate_route call per step; moe_route on the same logits is timed beside
    it (the routing alone)."""
    import re
    m = re.fullmatch(r"gate_n(\d+)_e(\d+)_h(\d+)_k(\d+)", name)
    if not m:
        raise SystemExit(f"unknown workload {name!r}")
    n, e, h, k = (int(v) for v in m.groups())
    clock = ClockSampler().start()
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    x_cpu, w_cpu = router_inputs(n, e, h, "bf16", seed=0)
    x, w = x_cpu.to(dev), w_cpu.to(dev)
    lg = torch.empty(n, e, dtype=torch.bfloat16, device=dev)
    routing = Routing.empty(n, e, k, torch.bfloat16, dev)
    ws = torch.empty(max(1, moe_workspace_bytes(n, e, k, h)), dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream(dev)
    p_gate = prepare_gate_route(x, w, k, logits=lg, routing=routing, workspace=ws, stream=stream)
    p_route = prepare_route(lg, k, routing=routing, workspace=ws, stream=stream)
    for _ in range(args.warmup):
        p_gate()
    t0 = time.perf_counter()
    st = step_stats(p_gate, args.steps, stream)
    wall = time.perf_counter() - t0
    st_route = step_stats(p_route, args.steps, stream)
    clock.sustained(p_gate, args.clock_seconds)
    cold = cold_stats([p_gate], 20, stream, dev)[0]
    words = (e + 31) // 32
    route_b = n * e * 2 + n * k * (4 + 2 + 4 + 4 + 2) + n * words * 4 + (2 * e + 1) * 4
    nbytes = n * h * 2 + e * h * 2 + n * e * 2 + route_b   # x, gate weight, logits out, routing
    flops = 2 * n * e * h
    spec_like = type("S", (), {"dtype": "bf16"})()
    roof = roofline(spec_like, flops, nbytes, st["mean"])
    roof.update({"kernel": "router GEMM + routing (all kernels of one moe_gate_route call)",
                 "traffic": None, "algorithmic_bytes": nbytes, "algorithmic_flops": flops,
                 "avg_launch_us": round(st["mean"] * 1e3, 2)})
    result = {
        "metric": METRIC, "value": round(n / (st["mean"] * 1e-3), 1), "unit": "tokens/s",
        "n_gpus": 1, "steps": st["steps"], "warmup": args.warmup,
        "ms_per_step": round(st["mean"], 5), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic (seeded Gaussian token rows and gate weight)",
        "config": {"workload": f"{name}: router GEMM + routing, N={n} E={e} H={h} k={k} bf16"},
        "routing_us_per_layer": round(st["mean"] * 1e3, 2),
        "route_only_us": round(st_route["mean"] * 1e3, 2),
        "step_us": {q: round(st[q] * 1e3, 2) for q in ("p10", "p50", "p90")},
        "cold_routing_us": round(cold * 1e3, 2),
        "wall_ms_per_step": round(wall / st["steps"] * 1e3, 4),
        "roofline": roof,
        "gpu_clock": clock.summary(),
        "host": host_info(),
    }
    if not args.no_cpu_baseline:
        import oracle
        sample = min(n, 2048)
        t0, reps = time.perf_counter(), 0
        while True:
            oracle.route_gate(x_cpu[:sample], w_cpu, k, "bf16")
            reps += 1
            if time.perf_counter() - t0 >= args.cpu_seconds:
                break
        dt = time.perf_counter() - t0
        result["cpu_baseline"] = {"value": round(sample * reps / dt, 1), "unit": "tokens/s",
                                  "cores": _oracle_threads(), "kind": "oracle",
                                  "sample": f"first {sample} of {n} tokens, router logits + "
                                            f"routing oracle, {reps} passes in {dt:.1f} s"}
    print(json.dumps(result), flush=True)


def bench_decode_stack(args, name: str):
    """decode<L>_n<N>: L chained layers shaped as gpt-oss-20b's MoE layers (32
    experts, top-4, H = I = 2880, SwiGLU-OAI interleaved), N tokens, each layer
    router GEMM + routing + experts (moe_gate_forward), its output the next
    layer's input.  One step = the L layers; timed eager (L prepared calls) and
    as one captured HIP graph replay, to show what capture saves on launches."""
    import re
    m = re.fullmatch(r"decode(\d+)_n(\d+)(_mxfp4)?", name)
    if not m:
        raise SystemExit(f"unknown workload {name!r}")
    L, n, mx = int(m.group(1)), int(m.group(2)), m.group(3) is not None
    e, k, h, i = 32, 4, 2880, 2880
    prm = {"alpha": 1.702, "beta": 1.0, "limit": 7.0}
    clock = ClockSampler().start()
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    gen = torch.Generator(device=dev)

    def draw(shape, std, seed):  # seeded on the GPU, one expert at a time, cast to bf16
        gen.manual_seed(seed)
        out = torch.empty(shape, dtype=torch.bfloat16, device=dev)
        for j in range(shape[0]):
            out[j] = (torch.randn(shape[1:], generator=gen, device=dev) * std).to(torch.bfloat16)
        return out

    layers = []
    for l in range(L):
        wg, w13, w2 = (draw((e, h), h ** -0.5, 3 * l), draw((e, 2 * i, h), 0.02, 3 * l + 1),
                       draw((e, h, i), 0.02, 3 * l + 2))
        if mx:  # MXFP4 expert weights (the router stays bf16)
            w13, w2 = moe_quantize_mxfp4(w13), moe_quantize_mxfp4(w2)
            torch.cuda.synchronize()
        layers.append((wg, w13, w2))
    x0, _ = router_inputs(n, e, h, "bf16", seed=0)
    bufs = [x0.to(dev)] + [torch.empty(n, h, dtype=torch.bfloat16, device=dev) for _ in range(L)]
    logits = torch.empty(n, e, dtype=torch.bfloat16, device=dev)
    routing = Routing.empty(n, e, k, torch.bfloat16, dev)
    ws = torch.empty(moe_workspace_bytes(n, e, k, h, i), dtype=torch.uint8, device=dev)

    def prepared(stream):
        if not mx:
            return [prepare_gate_forward(bufs[l], wg, w13, w2, k, "swiglu_oai", "interleaved",
                                         prm, out=bufs[l + 1], logits=logits, routing=routing,
                                         workspace=ws, stream=stream)
                    for l, (wg, w13, w2) in enumerate(layers)]
        calls = []
        for l, (wg, (q13, s13), (q2, s2)) in enumerate(layers):
            calls.append(prepare_gate_route(bufs[l], wg, k, logits=logits, routing=routing,
                                            workspace=ws, stream=stream))
            calls.append(prepare_experts_mxfp4(bufs[l], q13, s13, q2, s2, routing, "swiglu_oai",
                                               "interleaved", prm, out=bufs[l + 1],
                                               workspace=ws, stream=stream))
        return calls

    stream = torch.cuda.current_stream(dev)
    eager = prepared(stream)

    def step():
        for c in eager:
            c()
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    ref = bufs[-1].clone()
    st_eager = step_stats(step, args.steps, stream)
    g = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(stream)
    with torch.cuda.stream(side):
        for c in prepared(side):
            c()
    stream.wait_stream(side)
    torch.cuda.synchronize()
    with torch.cuda.graph(g):
        captured = prepared(torch.cuda.current_stream(dev))
        for c in captured:
            c()
    for _ in range(args.warmup):
        g.replay()
    torch.cuda.synchronize()
    same = bool(torch.equal(bufs[-1], ref))
    st_graph = step_stats(g.replay, args.steps, stream)
    clock.sustained(g.replay, args.clock_seconds)
    # weights of the experts each layer's tokens touch, read once (counted in an
    # untimed eager pass that reads every layer's histogram)
    touched = []
    for j, c in enumerate(eager):
        c()
        if not mx or j % 2 == 0:
            touched.append(int((routing.col_sum > 0).sum()))
    wb = MXFP4_BYTES if mx else 2  # bytes per expert weight
    nbytes = sum(int(t * 3 * i * h * wb) + e * h * 2 + n * h * 2 * 2 for t in touched)
    ms = st_graph["mean"]
    ach = nbytes / (ms * 1e-3) / 1e9
    result = {
        "metric": METRIC, "value": round(n / (ms * 1e-3), 1), "unit": "tokens/s",
        "n_gpus": 1, "steps": st_graph["steps"], "warmup": args.warmup,
        "ms_per_step": round(ms, 5), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic (seeded Gaussian token rows; weights drawn on the GPU from seeded "
                "generators)",
        "config": {"workload": f"{name}: {L} chained gpt-oss-20b-shaped MoE layers "
                               f"(E=32 k=4 H=I=2880 swiglu_oai interleaved bf16"
                               f"{', MXFP4 expert weights' if mx else ''}), N={n}, "
                               f"router GEMM + routing + experts per layer"},
        "graph_us_per_step": round(ms * 1e3, 2),
        "eager_us_per_step": round(st_eager["mean"] * 1e3, 2),
        "graph_us_per_layer": round(ms * 1e3 / L, 2),
        "eager_us_per_layer": round(st_eager["mean"] * 1e3 / L, 2),
        "graph_replay_equals_eager": same,
        "experts_touched_per_layer": touched,
        "roofline": {"bound": "hbm", "achieved": round(ach, 1), "peak": PEAK_HBM_GBS,
                     "unit": "GB/s", "frac": round(ach / PEAK_HBM_GBS, 4),
                     "kernel": "whole step (graph replay)", "traffic": None,
                     "algorithmic_bytes": nbytes, "avg_launch_us": round(ms * 1e3, 2)},
        "gpu_clock": clock.summary(),
        "host": host_info(),
    }
    print(json.dumps(result), flush=True)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default="skewed_silu")
    ap.add_argument("--cpu-seconds", type=float, default=12.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--clock-seconds", type=float, default=3.0,
                    help="length of the clock pass after the timed region (0: none)")
    ap.add_argument("--calibrate-copy", type=int, default=0, metavar="MB",
                    help="first copy MB mebibytes device to device three times: a plain copy "
                         "of known size that hardware byte counters can be scaled by")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py runs on one GPU only: the library drives a single GPU and has no "
              "multi-GPU path", file=sys.stderr)
        sys.exit(2)

    if args.calibrate_copy > 0:
        src = torch.ones(args.calibrate_copy << 20, dtype=torch.uint8, device="cuda:0")
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
    if args.workload.startswith("route_"):
        return bench_route_only(args, args.workload)
    if args.workload.startswith("gate_"):
        return bench_gate_route(args, args.workload)
    if args.workload.startswith("decode"):
        return bench_decode_stack(args, args.workload)
    spec = workload(args.workload)
    mx = spec.name.endswith("_mxfp4")
    # the SMI library is slow to start: start the sampler before the layer is built
    clock = ClockSampler().start()
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    layer = make_layer(spec)
    x, lg = layer.x.to(dev), layer.logits.to(dev)
    w13, w2 = layer.w13.to(dev), layer.w2.to(dev)
    if mx:  # quantised once, outside the timed region, as a model load would
        wq = moe_quantize_mxfp4(w13) + moe_quantize_mxfp4(w2)
        del w13, w2
        torch.cuda.synchronize()
    n, e, k = spec.n_tokens, spec.n_experts, spec.topk
    share = spec.n_local is not None
    dt = x.dtype
    routing = Routing.empty(n, spec.n_weights, k, dt, dev)
    act = torch.empty(n * k, spec.inter, dtype=dt, device=dev)
    out = torch.empty_like(x)
    ws = torch.empty(moe_workspace_bytes(n, e, k, spec.hidden, spec.inter, dt), dtype=torch.uint8,
                     device=dev)
    stream = torch.cuda.current_stream(dev)
    if mx:
        p_route = prepare_route(lg, k, routing=routing, workspace=ws, stream=stream)
        p_fwd = prepare_forward_mxfp4(x, lg, *wq, k, spec.act, spec.layout, act_params(spec),
                                      out=out, routing=routing, workspace=ws, stream=stream)
    elif share:
        p_route = prepare_route_ep(lg, k, spec.local_offset, spec.n_local, routing=routing,
                                   workspace=ws, stream=stream)
        p_fwd = prepare_forward_ep(x, lg, w13, w2, k, spec.local_offset, spec.act, spec.layout,
                                   act_params(spec), out=out, routing=routing, workspace=ws,
                                   stream=stream)
    else:
        p_route = prepare_route(lg, k, routing=routing, workspace=ws, stream=stream)
        p_fwd = prepare_forward(x, lg, w13, w2, k, spec.act, spec.layout, act_params(spec),
                                out=out, routing=routing, workspace=ws, stream=stream)
    # the split calls run the kernels of the full call: GEMM1 + activation,
    # GEMM2 + routing weight into sorted rows, then the combine (k > 1); with one
    # slot a token GEMM2 writes the output rows itself
    y_rows = torch.empty(n * k, spec.hidden, dtype=dt, device=dev) if not mx and k > 1 else None

    def stage_calls(st):
        """The layer's stages as prepared C calls on stream st, in order."""
        calls = [("route", prepare_route_ep(lg, k, spec.local_offset, spec.n_local,
                                            routing=routing, workspace=ws, stream=st)
                  if share else prepare_route(lg, k, routing=routing, workspace=ws, stream=st))]
        if mx:
            return calls + [("experts", prepare_experts_mxfp4(
                x, *wq, routing, spec.act, spec.layout, act_params(spec), out=out, workspace=ws,
                stream=st))]
        calls.append(("w13", prepare_experts_w13(x, w13, routing, spec.act, spec.layout,
                                                 act_params(spec), act_out=act, stream=st)))
        if k > 1:
            calls.append(("w2", prepare_experts_w2_rows(act, w2, routing, y_sorted=y_rows,
                                                        stream=st)))
            calls.append(("combine", prepare_combine(y_rows, routing, out=out, stream=st)))
        else:
            calls.append(("w2", prepare_experts_w2(act, w2, routing, out=out, workspace=ws,
                                                   stream=st)))
        return calls

    K, W = args.steps, args.warmup

    def graph_timed(fn, reps, gstream):
        """Device time of one call (ms): reps back-to-back calls captured in a HIP
        graph on gstream, replayed between two events on gstream (no host launch
        cost between the calls); the best of three replays."""
        with torch.cuda.stream(gstream):
            fn()
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=gstream):
            for _ in range(reps):
                fn()
        best = None
        for _ in range(3):
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            torch.cuda.synchronize()
            with torch.cuda.stream(gstream):
                a.record(gstream)
                g.replay()
                b.record(gstream)
            torch.cuda.synchronize()
            t = a.elapsed_time(b) / reps
            best = t if best is None else min(best, t)
        del g
        return best

    for _ in range(W):
        p_fwd()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    st = step_stats(p_fwd, K, stream)
    wall = time.perf_counter() - t0
    clock.sustained(p_fwd, args.clock_seconds)
    ms_step = st["mean"]
    # stages (the routing metadata of the last step stays valid for the others),
    # each timed as a captured graph of K calls on a stream of its own
    gstream = torch.cuda.Stream(device=dev)
    stage_ms = {name: graph_timed(fn, K, gstream) for name, fn in stage_calls(gstream)}
    eager = dict(stage_calls(stream))
    p_comb = eager.get("combine")
    cold_fns = [p_fwd, p_route] + ([p_comb] if not mx and k > 1 else [])
    cold = cold_stats(cold_fns, 20, stream, dev)
    col_sum = routing.col_sum.cpu()
    stage_roof = {}
    if mx:
        # MXFP4 workloads: both grouped GEMMs of one experts call, weight bytes
        # at 17/32 byte a weight
        f, b, et = algorithmic_mxfp4(spec, col_sum)
        roof = roofline(spec, f, b, stage_ms["experts"])
        roof.update({"kernel": f"{expert_kernel(spec, True)} w13 + w2 (MXFP4 weights, one "
                               "experts call)",
                     "traffic": None, "algorithmic_bytes": b, "algorithmic_flops": f,
                     "avg_launch_us": round(stage_ms["experts"] * 1e3, 2)})
    else:
        work, et = algorithmic(spec, col_sum)
        for name in stage_ms:
            sf, sb = work[name]
            r = roofline(spec, sf, sb, stage_ms[name])
            stage_roof[name] = {"bound": r["bound"], "frac": r["frac"], "achieved": r["achieved"],
                                "unit": r["unit"]}
        # the dominant kernel: the longest of the single-kernel stages
        dom = max(("w13", "w2", "combine"), key=lambda s_: stage_ms.get(s_, -1.0))
        f, b = work[dom]
        label = {"w13": f"{expert_kernel(spec, False)} (w13 + activation)",
                 "w2": f"{expert_kernel(spec, False)} (w2 + routing weight"
                       f"{' into sorted rows' if k > 1 else ', to the output rows'})",
                 "combine": "combine_kernel (scatter-combine)"}[dom]
        roof = roofline(spec, f, b, stage_ms[dom])
        roof.update({"kernel": label, "stage": dom,
                     "traffic": stored_traffic(spec.name, dom),
                     "algorithmic_bytes": b, "algorithmic_flops": f,
                     "avg_launch_us": round(stage_ms[dom] * 1e3, 2)})
    cold_us = {"step": round(cold[0] * 1e3, 2), "route": round(cold[1] * 1e3, 2)}
    if len(cold) > 2:
        cold_us["combine"] = round(cold[2] * 1e3, 2)
        cb = work["combine"][1]
        cold_us["combine_gbs"] = round(cb / (cold[2] * 1e-3) / 1e9, 1)
        cold_us["combine_warm_gbs"] = round(cb / (stage_ms["combine"] * 1e-3) / 1e9, 1)
    result = {
        "metric": METRIC,
        "value": round(n / (ms_step * 1e-3), 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": st["steps"],
        "warmup": W,
        "ms_per_step": round(ms_step, 5),
        "step_us": {q: round(st[q] * 1e3, 2) for q in ("p10", "p50", "p90")},
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": spec.dtype,
        "data": "synthetic (seeded Gaussian inputs, random-init weights)",
        "config": {"workload": f"{spec.name}: {describe(spec)}", "n_tokens": n,
                   "experts_touched": et, "max_expert_rows": int(col_sum.max())},
        "routing_us_per_layer": round(stage_ms["route"] * 1e3, 2),
        "stage_us": {s_: round(v * 1e3, 2) for s_, v in stage_ms.items()},
        "stage_roofline": stage_roof,
        "cold_us": cold_us,
        "wall_ms_per_step": round(wall / K * 1e3, 4),
        "roofline": roof,
        "gpu_clock": clock.summary(),
        "host": host_info(),
    }
    if not args.no_cpu_baseline and not mx:
        result["cpu_baseline"] = cpu_baseline(spec, layer, args.cpu_seconds)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
