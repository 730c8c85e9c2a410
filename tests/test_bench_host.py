"""Host-side pieces of bench.py (no GPU): workload names, the clock summary's
window, the stored hardware-counter traffic and its source-hash guard, and the
one-GPU refusal."""
import hashlib
import os
import re
import subprocess
import sys

import pytest

import bench


def test_workload_names():
    s = bench.workload("skewed_silu")
    assert (s.n_tokens, s.hidden, s.inter, s.n_experts, s.topk, s.act) == \
        (16384, 4096, 1536, 64, 8, "silu")
    assert bench.workload("skewed_relu2").act == "relu2"
    g = bench.workload("gptoss_n4096")
    assert (g.n_tokens, g.hidden, g.inter, g.n_experts, g.topk) == (4096, 2880, 2880, 128, 4)
    ep = bench.workload("gptoss_ep8_n4096")
    assert (ep.local_offset, ep.n_local, ep.n_weights) == (0, 16, 16)
    assert bench.workload("minimind_e16").n_experts == 16
    assert bench.workload("gptoss_n33_mxfp4").name == "gptoss_n33_mxfp4"
    with pytest.raises(SystemExit):
        bench.workload("no_such_layer")


def test_clock_summary_keeps_only_the_window():
    c = bench.ClockSampler()
    c.samples = [(0.5, 100.0), (1.0, 1800.0), (1.5, 1850.0), (2.0, 1900.0), (2.5, 120.0)]
    c.window = [0.9, 2.1]
    c.seconds, c.settle = 3.0, 1.2
    s = c.summary()
    assert (s["median_mhz"], s["min_mhz"], s["max_mhz"], s["samples"]) == (1850, 1800, 1900, 3)
    c.window = [3.0, 4.0]
    assert c.summary()["median_mhz"] is None


def test_clock_pass_disabled_reports_why():
    c = bench.ClockSampler()
    c.sustained(lambda: None, 0.0)
    s = c.summary()
    assert s["median_mhz"] is None and "disabled" in s["error"]


def _traffic_lines():
    text = open(os.path.join(bench.ROOT, "profiles", "gemm_counters.md")).read()
    return re.findall(r"traffic: workload=(\S+) stage=(\S+) src=(\S+) src_sha256=(\S+) "
                      r"fetch_bytes=(\d+) write_bytes=(\d+)", text)


def test_stored_traffic_is_for_the_current_sources():
    """The default bench line's roofline.traffic comes from counters taken on
    the kernel sources as they are: every stored line for the headline layer
    names the current hash of its source file (re-take the counters after a
    kernel change)."""
    lines = [l for l in _traffic_lines() if l[0] == "skewed_silu"]
    assert {l[1] for l in lines} >= {"w13", "w2", "combine"}
    for w, st, src, sha, fb, wb in lines:
        path = os.path.join(bench.ROOT, "routing_grouped_expert_amd", "csrc", src)
        assert hashlib.sha256(open(path, "rb").read()).hexdigest()[:16] == sha, (st, src)
        assert bench.stored_traffic(w, st) == int(fb) + int(wb)


def test_stored_traffic_is_none_for_unknown_or_changed(tmp_path, monkeypatch):
    assert bench.stored_traffic("skewed_silu", "no_such_stage") is None
    # a copy of the tree whose kernel source differs by one byte: no traffic
    root = tmp_path / "r"
    (root / "profiles").mkdir(parents=True)
    (root / "routing_grouped_expert_amd" / "csrc").mkdir(parents=True)
    (root / "profiles" / "gemm_counters.md").write_text(
        open(os.path.join(bench.ROOT, "profiles", "gemm_counters.md")).read())
    for w, st, src, sha, fb, wb in _traffic_lines():
        dst = root / "routing_grouped_expert_amd" / "csrc" / src
        if not dst.exists():
            data = open(os.path.join(bench.ROOT, "routing_grouped_expert_amd", "csrc", src),
                        "rb").read()
            dst.write_bytes(data + b"\n")
    monkeypatch.setattr(bench, "ROOT", str(root))
    assert bench.stored_traffic("skewed_silu", "w13") is None


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(bench.ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=300)
    assert r.returncode == 2 and "one GPU" in r.stderr
