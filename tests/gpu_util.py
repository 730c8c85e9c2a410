"""Comparison helpers for the GPU parity tests (HIP path vs CPU oracle)."""
from __future__ import annotations

import numpy as np
import torch

import oracle

INT_FIELDS = ("topk_idx", "bitmatrix", "col_sum", "offsets", "col_sorted", "row_sorted")


def _ulp_dist(gpu: torch.Tensor, ref64: np.ndarray) -> np.ndarray:
    """Distance in units of the last place between a GPU float tensor and
    float64 reference values exactly representable in the same dtype (>= 0)."""
    ref = torch.from_numpy(np.ascontiguousarray(ref64)).to(gpu.dtype)
    if gpu.dtype == torch.bfloat16:
        a = gpu.cpu().view(torch.int16).numpy().astype(np.int64)
        b = ref.view(torch.int16).numpy().astype(np.int64)
    else:
        a = gpu.cpu().view(torch.int32).numpy().astype(np.int64)
        b = ref.view(torch.int32).numpy().astype(np.int64)
    return np.abs(a - b)


def assert_routing_equal(gpu, ref: "oracle.RoutingRef", where: str = "routing") -> dict:
    """Integer metadata bit-exact (path-qualified messages); weights within one
    bf16 ulp, or 8 + k fp32 ulps; gate_scal equal to topk_w permuted, exactly.

    The fp32 bound: the kernel's exp is within ~1 ulp, rounding the argument
    v - max (|v - max| <= 8 for these inputs) moves exp by up to 8 * 2^-24
    relative (4 ulp), the k-term sum adds up to (k - 1) / 2 ulp and the divide
    half an ulp.  In bf16 those fp32 errors (~2^-20 relative) only matter when
    the exact weight sits next to a bf16 rounding boundary: one bf16 ulp."""
    for f in INT_FIELDS:
        g = getattr(gpu, f).cpu().numpy()
        r = getattr(ref, f)
        if f == "bitmatrix":
            g = g.view(np.uint32)
        assert g.shape == r.shape, f"{where}.{f}: shape {g.shape} != {r.shape}"
        if not np.array_equal(g.astype(np.int64), r.astype(np.int64)):
            bad = np.argwhere(g.astype(np.int64) != r.astype(np.int64))
            i = tuple(bad[0])
            raise AssertionError(f"{where}.{f}: {len(bad)} mismatches, first at {i}: "
                                 f"gpu {g[i]} != oracle {r[i]}")
    tol = 1 if gpu.topk_w.dtype == torch.bfloat16 else 8 + gpu.topk_idx.shape[1]
    stats = {}
    for f in ("topk_w", "gate_scal"):
        d = _ulp_dist(getattr(gpu, f), getattr(ref, f))
        stats[f + "_max_ulp"] = int(d.max()) if d.size else 0
        stats[f + "_n_off"] = int((d > 0).sum())
        assert d.size == 0 or d.max() <= tol, f"{where}.{f}: {d.max()} ulp off (tolerance {tol})"
    # inside the GPU result, gate_scal is exactly topk_w in sorted order (and 0
    # past an expert share's local entries, where col_sorted is -1)
    tw = gpu.topk_w.reshape(-1)
    cs = gpu.col_sorted.long()
    live = cs >= 0
    assert torch.equal(gpu.gate_scal[live], tw[cs[live]]), \
        f"{where}.gate_scal != topk_w.flat[col_sorted]"
    assert not gpu.gate_scal[~live].any(), f"{where}.gate_scal past the local entries != 0"
    return stats


def cosine(a: np.ndarray, b: np.ndarray) -> float:
    a = a.ravel().astype(np.float64)
    b = b.ravel().astype(np.float64)
    na, nb = np.linalg.norm(a), np.linalg.norm(b)
    if na == 0 and nb == 0:
        return 1.0
    return float(a @ b / (na * nb))


def assert_output_close(gpu: torch.Tensor, ref: np.ndarray, where: str = "out") -> dict:
    """fp32: max|gpu - ref| <= 1e-4 * max|ref|.  bf16: |gpu - ref| <= 3e-2 +
    3e-2 |ref| elementwise, and cosine similarity >= 0.99 (a zero or
    misdirected output can pass the absolute test alone)."""
    g = gpu.detach().cpu().double().numpy()
    assert g.shape == ref.shape, f"{where}: shape {g.shape} != {ref.shape}"
    assert np.all(np.isfinite(g)), f"{where}: non-finite values"
    scale = float(np.max(np.abs(ref))) if ref.size else 0.0
    err = np.abs(g - ref)
    stats = {"max_abs_err": float(err.max()) if err.size else 0.0, "ref_scale": scale,
             "cosine": cosine(g, ref)}
    if gpu.dtype == torch.float32:
        assert stats["max_abs_err"] <= 1e-4 * scale, f"{where}: {stats}"
    else:
        bad = err > 3e-2 + 3e-2 * np.abs(ref)
        assert not bad.any(), f"{where}: {int(bad.sum())} elements out of atol/rtol 3e-2; {stats}"
        assert stats["cosine"] >= 0.99, f"{where}: cosine {stats['cosine']}"
    return stats
