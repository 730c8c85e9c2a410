"""MI355X (gfx950) MoE-layer forward: routing metadata, grouped expert FFN and
combine, all in hand-written HIP kernels behind the C ABI of ``libmoe.so``.

This module is a thin binding over that ABI: it checks tensor placement and
dtypes, allocates outputs and workspaces with torch, and passes raw device
pointers plus the current HIP stream.  Every step of the layer runs in the
library's kernels; there is no other implementation behind these functions, and
they raise if the library is missing.

    routing = moe_route(logits, topk)
    out = moe_experts(x, w13, w2, routing, act="silu", layout="packed")
    out, routing = moe_forward(x, logits, w13, w2, topk, act="swiglu_oai",
                               layout="interleaved",
                               params={"alpha": 1.702, "beta": 1.0, "limit": 7.0})

With the router's gate weight ``w_gate [E, H]`` the routing step also computes
the logits (router GEMM): ``logits, routing = moe_gate_route(x, w_gate, topk)``;
``moe_gate_forward`` runs the whole layer from ``x`` and ``w_gate``.

One GPU of an expert-parallel group (experts [lo, lo + n) of the layer's E,
weights w13 [n, ...], w2 [n, ...]) uses the ``_ep`` variants; summing their
outputs over the group's shares gives the layer output:

    routing = moe_route_ep(logits, topk, lo, n)
    out = moe_experts_ep(x, w13, w2, routing, act="silu")
    out, routing = moe_forward_ep(x, logits, w13, w2, topk, lo, act="silu")
"""
from __future__ import annotations

import ctypes
from dataclasses import dataclass, fields
from typing import Optional

import torch

from . import _native as N

__all__ = ["Routing", "MoeError", "Prepared", "moe_route", "moe_experts", "moe_experts_w13",
           "moe_experts_w2", "moe_experts_w2_rows", "moe_combine", "prepare_experts_w2_rows",
           "prepare_combine", "moe_forward", "moe_forward_noalloc", "prepare_forward_noalloc",
           "prepare_route", "prepare_experts",
           "prepare_experts_w13", "prepare_experts_w2", "prepare_forward",
           "moe_route_ep", "moe_experts_ep", "moe_forward_ep", "prepare_route_ep",
           "prepare_experts_ep", "prepare_forward_ep", "moe_gate_route", "moe_gate_forward",
           "prepare_gate_route", "prepare_gate_forward", "moe_experts_weighted_input",
           "prepare_experts_weighted_input", "moe_quantize_mxfp4", "moe_experts_mxfp4",
           "moe_forward_mxfp4", "prepare_experts_mxfp4", "prepare_forward_mxfp4",
           "moe_workspace_bytes", "moe_status_str", "ACTS", "LAYOUTS"]

_DT = {torch.float32: N.MOE_F32, torch.bfloat16: N.MOE_BF16}
ACTS = {"silu": N.MOE_ACT_SILU, "swiglu_oai": N.MOE_ACT_SWIGLU_OAI, "relu2": N.MOE_ACT_RELU2}
LAYOUTS = {"packed": N.MOE_W13_PACKED, "interleaved": N.MOE_W13_INTERLEAVED}
_PBITS = {"alpha": N.MOE_PARAM_ALPHA, "beta": N.MOE_PARAM_BETA, "limit": N.MOE_PARAM_LIMIT}


class MoeError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: {moe_status_str(status)} (status {status})")


def moe_status_str(status: int) -> str:
    return N.load().moe_status_str(status).decode()


def _check(status: int, where: str):
    if status != N.MOE_OK:
        raise MoeError(status, where)


def _dt(t: torch.Tensor) -> int:
    if t.dtype not in _DT:
        raise TypeError(f"unsupported dtype {t.dtype}; expected float32 or bfloat16")
    return _DT[t.dtype]


def _dev(*ts: torch.Tensor):
    dev = ts[0].device
    for t in ts:
        if t.device.type != "cuda" or t.device != dev:
            raise ValueError("all tensors must be on the same GPU")
        if not t.is_contiguous():
            raise ValueError("tensors must be contiguous")
    return dev


def _shapes(x, w13, w2, act, out=None, logits=None, n_experts=None):
    """Every buffer size the kernels assume, checked before any launch.
    ``n_experts`` is the logits' expert count when w13/w2 hold only a share."""
    if act not in ACTS:
        raise ValueError(f"unknown activation {act!r}")
    if x.dim() != 2 or w13.dim() != 3 or w2.dim() != 3:
        raise ValueError("expected x [N, H], w13 [E, nI, H], w2 [E, H, I]")
    n, hidden = x.shape
    e, h2, inter = w2.shape
    rows = inter if act == "relu2" else 2 * inter
    if h2 != hidden or tuple(w13.shape) != (e, rows, hidden):
        raise ValueError(f"w13 {tuple(w13.shape)} / w2 {tuple(w2.shape)} do not match "
                         f"x {tuple(x.shape)} and act {act!r}")
    if not (x.dtype == w13.dtype == w2.dtype):
        raise TypeError("x, w13 and w2 must share a dtype")
    if out is not None and (tuple(out.shape) != (n, hidden) or out.dtype != x.dtype):
        raise ValueError("out must be [N, H] in the layer dtype")
    if logits is not None and (logits.dim() != 2 or
                               tuple(logits.shape) != (n, e if n_experts is None else n_experts)):
        raise ValueError("logits must be [N, E]")


def _check_routing(routing: "Routing", n: int, e: int, k: int):
    m = n * k
    want = {"topk_idx": (n, k), "topk_w": (n, k), "bitmatrix": (n, (e + 31) // 32),
            "col_sum": (e,), "offsets": (e + 1,), "col_sorted": (m,), "row_sorted": (m,),
            "gate_scal": (m,)}
    for f, shp in want.items():
        t = getattr(routing, f)
        if tuple(t.shape) != shp or not t.is_contiguous():
            raise ValueError(f"routing.{f} must be contiguous {shp}, got {tuple(t.shape)}")
    if routing.gate_scal.dtype != routing.topk_w.dtype:
        raise TypeError("routing.topk_w and gate_scal must share a dtype")


def _stream(dev, stream) -> ctypes.c_void_p:
    s = stream if stream is not None else torch.cuda.current_stream(dev)
    return ctypes.c_void_p(s.cuda_stream)


@dataclass
class Routing:
    """Routing metadata of one layer (device tensors); field meanings as in moe.h."""

    topk_idx: torch.Tensor    # [N, k] int32
    topk_w: torch.Tensor      # [N, k] logits dtype
    bitmatrix: torch.Tensor   # [N, ceil(E/32)] int32 (uint32 bit patterns)
    col_sum: torch.Tensor     # [E] int32
    offsets: torch.Tensor     # [E+1] int32
    col_sorted: torch.Tensor  # [N*k] int32
    row_sorted: torch.Tensor  # [N*k] int32
    gate_scal: torch.Tensor   # [N*k] logits dtype

    @classmethod
    def empty(cls, n_tokens: int, n_experts: int, topk: int, dtype: torch.dtype,
              device) -> "Routing":
        i32 = dict(dtype=torch.int32, device=device)
        m = n_tokens * topk
        return cls(
            topk_idx=torch.empty(n_tokens, topk, **i32),
            topk_w=torch.empty(n_tokens, topk, dtype=dtype, device=device),
            bitmatrix=torch.empty(n_tokens, (n_experts + 31) // 32, **i32),
            col_sum=torch.empty(n_experts, **i32),
            offsets=torch.empty(n_experts + 1, **i32),
            col_sorted=torch.empty(m, **i32),
            row_sorted=torch.empty(m, **i32),
            gate_scal=torch.empty(m, dtype=dtype, device=device),
        )

    @property
    def n_experts(self) -> int:
        return self.col_sum.numel()

    @property
    def topk(self) -> int:
        return self.topk_idx.shape[1]

    def as_c(self) -> N.MoeRouting:
        return N.MoeRouting(*(getattr(self, f.name).data_ptr() for f in fields(self)),
                            _dt(self.topk_w))


def _params(params: Optional[dict]) -> Optional[N.MoeActParams]:
    if not params:
        return None
    p = N.MoeActParams(1.0, 0.0, 0.0, 0)
    for k, v in params.items():
        if k not in _PBITS:
            raise ValueError(f"unknown activation parameter {k!r}")
        if v is None:
            continue  # unset: the kernel keeps its plain-SwiGLU default
        setattr(p, k, float(v))
        p.set |= _PBITS[k]
    return p


def moe_workspace_bytes(n_tokens: int, n_experts: int, topk: int, hidden: int = 0,
                        inter: int = 0, dtype: torch.dtype = torch.bfloat16) -> int:
    b = N.load().moe_workspace_bytes(n_tokens, n_experts, topk, hidden, inter, _DT[dtype])
    if b == 0:
        raise MoeError(N.MOE_ERR_SHAPE, "moe_workspace_bytes")
    return b


def _workspace(ws, nbytes: int, device) -> torch.Tensor:
    if ws is None:
        return torch.empty(nbytes, dtype=torch.uint8, device=device)
    if ws.numel() * ws.element_size() < nbytes:
        raise MoeError(N.MOE_ERR_WORKSPACE, "workspace")
    return ws


class Prepared:
    """One validated C-ABI call with its arguments marshalled once; calling it
    re-enqueues the same work (same buffers, same stream) without re-checking
    or re-converting anything on the Python side."""

    def __init__(self, name: str, args: tuple, keep: tuple, result):
        self._fn = getattr(N.load(), name)
        self._name = name
        self._args = args
        self._keep = keep          # ctypes structs and tensors the pointers refer to
        self.result = result

    def __call__(self):
        st = self._fn(*self._args)
        if st != N.MOE_OK:
            raise MoeError(st, self._name)
        return self.result


def _nbytes(t: torch.Tensor) -> int:
    return t.numel() * t.element_size()


def _share(e: int, local_offset: int, n_local: int):
    if not (0 <= local_offset and 1 <= n_local and local_offset + n_local <= e):
        raise ValueError(f"expert share [{local_offset}, {local_offset + n_local}) is not "
                         f"inside [0, {e})")


def prepare_route(logits: torch.Tensor, topk: int, *, routing: Optional[Routing] = None,
                  workspace: Optional[torch.Tensor] = None, stream=None,
                  _share_of: Optional[tuple] = None) -> Prepared:
    dev = _dev(logits)
    if logits.dim() != 2:
        raise ValueError("logits must be [N, E]")
    n, e = logits.shape
    lo, nl = _share_of if _share_of is not None else (0, e)
    _share(e, lo, nl)
    if routing is None:
        routing = Routing.empty(n, nl, topk, logits.dtype, dev)
    _check_routing(routing, n, nl, topk)
    ws = _workspace(workspace, moe_workspace_bytes(n, e, topk, 0, 0, logits.dtype), dev)
    r = routing.as_c()
    if _share_of is None:
        args = (logits.data_ptr(), _dt(logits), n, e, topk, ctypes.byref(r), ws.data_ptr(),
                _nbytes(ws), _stream(dev, stream))
        return Prepared("moe_route", args, (r, logits, ws, routing), routing)
    args = (logits.data_ptr(), _dt(logits), n, e, topk, lo, nl, ctypes.byref(r), ws.data_ptr(),
            _nbytes(ws), _stream(dev, stream))
    return Prepared("moe_route_ep", args, (r, logits, ws, routing), routing)


def prepare_route_ep(logits: torch.Tensor, topk: int, local_offset: int, n_local: int, *,
                     routing: Optional[Routing] = None, workspace: Optional[torch.Tensor] = None,
                     stream=None) -> Prepared:
    return prepare_route(logits, topk, routing=routing, workspace=workspace, stream=stream,
                         _share_of=(local_offset, n_local))


def moe_route_ep(logits: torch.Tensor, topk: int, local_offset: int, n_local: int, *,
                 routing: Optional[Routing] = None, workspace: Optional[torch.Tensor] = None,
                 stream=None) -> Routing:
    """Routing for the expert share [local_offset, local_offset + n_local) of
    ``logits [N, E]``: global top-k, metadata over the local experts (moe.h)."""
    return prepare_route_ep(logits, topk, local_offset, n_local, routing=routing,
                            workspace=workspace, stream=stream)()


def moe_route(logits: torch.Tensor, topk: int, *, routing: Optional[Routing] = None,
              workspace: Optional[torch.Tensor] = None, stream=None) -> Routing:
    """Top-k gating and routing metadata for ``logits [N, E]`` (see moe.h)."""
    return prepare_route(logits, topk, routing=routing, workspace=workspace, stream=stream)()


def prepare_experts(x, w13, w2, routing: Routing, act: str, layout: str = "packed",
                    params: Optional[dict] = None, *, out=None, workspace=None,
                    stream=None, _ep: bool = False) -> Prepared:
    dev = _dev(x, w13, w2)
    _shapes(x, w13, w2, act, out)
    n, hidden = x.shape
    e, inter = w2.shape[0], w2.shape[2]
    k = routing.topk
    _check_routing(routing, n, e, k)
    if out is None:
        out = torch.empty_like(x)
    # the experts' workspace does not depend on the expert count (any E >= k)
    ws = _workspace(workspace, moe_workspace_bytes(n, max(e, k), k, hidden, inter, x.dtype),
                    dev)
    r = routing.as_c()
    p = _params(params)
    args = (x.data_ptr(), _dt(x), n, hidden, w13.data_ptr(), w2.data_ptr(), e, inter, k,
            ACTS[act], LAYOUTS[layout], ctypes.byref(p) if p else None, ctypes.byref(r),
            out.data_ptr(), ws.data_ptr(), _nbytes(ws), _stream(dev, stream))
    return Prepared("moe_experts_ep" if _ep else "moe_experts", args,
                    (r, p, x, w13, w2, out, ws, routing), out)


def prepare_experts_ep(x, w13, w2, routing: Routing, act: str, layout: str = "packed",
                       params: Optional[dict] = None, *, out=None, workspace=None,
                       stream=None) -> Prepared:
    return prepare_experts(x, w13, w2, routing, act, layout, params, out=out,
                           workspace=workspace, stream=stream, _ep=True)


def moe_experts_ep(x: torch.Tensor, w13: torch.Tensor, w2: torch.Tensor, routing: Routing,
                   act: str, layout: str = "packed", params: Optional[dict] = None, *,
                   out: Optional[torch.Tensor] = None, workspace: Optional[torch.Tensor] = None,
                   stream=None) -> torch.Tensor:
    """Expert FFN of one expert share (w13/w2 hold its n_local experts) from a
    moe_route_ep routing; tokens with no slot in the share get zero rows."""
    return prepare_experts_ep(x, w13, w2, routing, act, layout, params, out=out,
                              workspace=workspace, stream=stream)()


def moe_experts(x: torch.Tensor, w13: torch.Tensor, w2: torch.Tensor, routing: Routing,
                act: str, layout: str = "packed", params: Optional[dict] = None, *,
                out: Optional[torch.Tensor] = None, workspace: Optional[torch.Tensor] = None,
                stream=None) -> torch.Tensor:
    """Grouped expert FFN + weighted combine from existing routing metadata."""
    return prepare_experts(x, w13, w2, routing, act, layout, params, out=out,
                           workspace=workspace, stream=stream)()


def prepare_experts_w13(x, w13, routing: Routing, act: str, layout: str = "packed",
                        params: Optional[dict] = None, *, act_out=None,
                        stream=None) -> Prepared:
    dev = _dev(x, w13)
    n, hidden = x.shape
    e, k = routing.n_experts, routing.topk
    inter = w13.shape[1] if act == "relu2" else w13.shape[1] // 2
    _shapes(x, w13, torch.empty(e, hidden, inter, device="meta", dtype=x.dtype), act)
    _check_routing(routing, n, e, k)
    if act_out is None:
        act_out = torch.empty(n * k, inter, dtype=x.dtype, device=dev)
    if tuple(act_out.shape) != (n * k, inter) or act_out.dtype != x.dtype:
        raise ValueError("act_out must be [N*k, inter] in the layer dtype")
    r = routing.as_c()
    p = _params(params)
    args = (x.data_ptr(), _dt(x), n, hidden, w13.data_ptr(), e, inter, k, ACTS[act],
            LAYOUTS[layout], ctypes.byref(p) if p else None, ctypes.byref(r),
            act_out.data_ptr(), _stream(dev, stream))
    return Prepared("moe_experts_w13", args, (r, p, x, w13, act_out, routing), act_out)


def moe_experts_w13(x: torch.Tensor, w13: torch.Tensor, routing: Routing, act: str,
                    layout: str = "packed", params: Optional[dict] = None, *,
                    act_out: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    """Grouped GEMM with w13 + activation; returns the sorted activation rows
    ``[N*k, inter]`` that moe_experts_w2 consumes."""
    return prepare_experts_w13(x, w13, routing, act, layout, params, act_out=act_out,
                               stream=stream)()


def prepare_experts_w2(act_in, w2, routing: Routing, *, out=None, workspace=None,
                       stream=None) -> Prepared:
    dev = _dev(act_in, w2)
    e, hidden, inter = w2.shape
    k = routing.topk
    n = routing.topk_idx.shape[0]
    if tuple(act_in.shape) != (n * k, inter) or act_in.dtype != w2.dtype:
        raise ValueError("act_in must be [N*k, inter] in the layer dtype")
    _check_routing(routing, n, e, k)
    if out is None:
        out = torch.empty(n, hidden, dtype=w2.dtype, device=dev)
    if tuple(out.shape) != (n, hidden) or out.dtype != w2.dtype:
        raise ValueError("out must be [N, hidden] in the layer dtype")
    ws = _workspace(workspace, moe_workspace_bytes(n, e, k, hidden, inter, w2.dtype), dev)
    r = routing.as_c()
    args = (act_in.data_ptr(), _dt(act_in), n, hidden, w2.data_ptr(), e, inter, k,
            ctypes.byref(r), out.data_ptr(), ws.data_ptr(), _nbytes(ws), _stream(dev, stream))
    return Prepared("moe_experts_w2", args, (r, act_in, w2, out, ws, routing), out)


def moe_experts_w2(act_in: torch.Tensor, w2: torch.Tensor, routing: Routing, *,
                   out: Optional[torch.Tensor] = None, workspace: Optional[torch.Tensor] = None,
                   stream=None) -> torch.Tensor:
    """Grouped GEMM with w2 + routing weight + combine into ``out [N, hidden]``."""
    return prepare_experts_w2(act_in, w2, routing, out=out, workspace=workspace,
                              stream=stream)()


def prepare_experts_w2_rows(act_in, w2, routing: Routing, *, y_sorted=None,
                            stream=None) -> Prepared:
    dev = _dev(act_in, w2)
    e, hidden, inter = w2.shape
    k = routing.topk
    n = routing.topk_idx.shape[0]
    if tuple(act_in.shape) != (n * k, inter) or act_in.dtype != w2.dtype:
        raise ValueError("act_in must be [N*k, inter] in the layer dtype")
    _check_routing(routing, n, e, k)
    if y_sorted is None:
        y_sorted = torch.empty(n * k, hidden, dtype=w2.dtype, device=dev)
    if tuple(y_sorted.shape) != (n * k, hidden) or y_sorted.dtype != w2.dtype:
        raise ValueError("y_sorted must be [N*k, hidden] in the layer dtype")
    _dev(act_in, y_sorted)
    r = routing.as_c()
    args = (act_in.data_ptr(), _dt(act_in), n, hidden, w2.data_ptr(), e, inter, k,
            ctypes.byref(r), y_sorted.data_ptr(), _stream(dev, stream))
    return Prepared("moe_experts_w2_rows", args, (r, act_in, w2, y_sorted, routing), y_sorted)


def moe_experts_w2_rows(act_in: torch.Tensor, w2: torch.Tensor, routing: Routing, *,
                        y_sorted: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    """Grouped GEMM with w2 + routing weight into the sorted rows ``[N*k, hidden]``
    (no combine); rows past the routed ones are left as they were."""
    return prepare_experts_w2_rows(act_in, w2, routing, y_sorted=y_sorted, stream=stream)()


def prepare_combine(y_sorted, routing: Routing, *, out=None, stream=None) -> Prepared:
    dev = _dev(y_sorted)
    n, k = routing.topk_idx.shape
    if y_sorted.dim() != 2 or y_sorted.shape[0] != n * k:
        raise ValueError("y_sorted must be [N*k, hidden]")
    hidden = y_sorted.shape[1]
    rs = routing.row_sorted
    if tuple(rs.shape) != (n * k,) or rs.dtype != torch.int32 or not rs.is_contiguous():
        raise ValueError("routing.row_sorted must be contiguous int32 [N*k]")
    if out is None:
        out = torch.empty(n, hidden, dtype=y_sorted.dtype, device=dev)
    if tuple(out.shape) != (n, hidden) or out.dtype != y_sorted.dtype:
        raise ValueError("out must be [N, hidden] in the dtype of y_sorted")
    _dev(y_sorted, out, rs)
    r = routing.as_c()
    args = (y_sorted.data_ptr(), _dt(y_sorted), n, hidden, k, ctypes.byref(r), out.data_ptr(),
            _stream(dev, stream))
    return Prepared("moe_combine", args, (r, y_sorted, out, routing), out)


def moe_combine(y_sorted: torch.Tensor, routing: Routing, *, out: Optional[torch.Tensor] = None,
                stream=None) -> torch.Tensor:
    """Scatter-combine ``out[t] = sum_j y_sorted[row_sorted[t*k + j]]`` (slot order,
    fp32 sum, one rounding; slots with row_sorted = -1 skipped)."""
    return prepare_combine(y_sorted, routing, out=out, stream=stream)()


def prepare_forward(x, logits, w13, w2, topk: int, act: str, layout: str = "packed",
                    params: Optional[dict] = None, *, out=None, routing=None, workspace=None,
                    stream=None) -> Prepared:
    dev = _dev(x, logits, w13, w2)
    _shapes(x, w13, w2, act, out, logits)
    n, hidden = x.shape
    e, inter = w2.shape[0], w2.shape[2]
    if logits.dtype != x.dtype:
        raise TypeError("moe_forward takes logits in the layer dtype")
    if routing is None:
        routing = Routing.empty(n, e, topk, logits.dtype, dev)
    _check_routing(routing, n, e, topk)
    if out is None:
        out = torch.empty_like(x)
    ws = _workspace(workspace, moe_workspace_bytes(n, e, topk, hidden, inter, x.dtype), dev)
    r = routing.as_c()
    p = _params(params)
    args = (x.data_ptr(), logits.data_ptr(), _dt(x), n, hidden, w13.data_ptr(), w2.data_ptr(),
            e, inter, topk, ACTS[act], LAYOUTS[layout], ctypes.byref(p) if p else None,
            ctypes.byref(r), out.data_ptr(), ws.data_ptr(), _nbytes(ws), _stream(dev, stream))
    return Prepared("moe_forward", args, (r, p, x, logits, w13, w2, out, ws, routing),
                    (out, routing))


def prepare_forward_noalloc(x, logits, w13, w2, topk: int, act: str, layout: str = "packed",
                            params: Optional[dict] = None, *, out=None, routing=None,
                            stream=None) -> Prepared:
    dev = _dev(x, logits, w13, w2)
    _shapes(x, w13, w2, act, out, logits)
    n, hidden = x.shape
    e, inter = w2.shape[0], w2.shape[2]
    if logits.dtype != x.dtype:
        raise TypeError("moe_forward_noalloc takes logits in the layer dtype")
    if routing is None:
        routing = Routing.empty(n, e, topk, logits.dtype, dev)
    _check_routing(routing, n, e, topk)
    if out is None:
        out = torch.empty_like(x)
    r = routing.as_c()
    p = _params(params)
    args = (x.data_ptr(), logits.data_ptr(), _dt(x), n, hidden, w13.data_ptr(), w2.data_ptr(),
            e, inter, topk, ACTS[act], LAYOUTS[layout], ctypes.byref(p) if p else None,
            ctypes.byref(r), out.data_ptr(), _stream(dev, stream))
    return Prepared("moe_forward_noalloc", args, (r, p, x, logits, w13, w2, out, routing),
                    (out, routing))


def moe_forward_noalloc(x: torch.Tensor, logits: torch.Tensor, w13: torch.Tensor,
                        w2: torch.Tensor, topk: int, act: str, layout: str = "packed",
                        params: Optional[dict] = None, *, out: Optional[torch.Tensor] = None,
                        routing: Optional[Routing] = None, stream=None):
    """moe_forward with no workspace argument: the intermediates live in the
    library's static per-GPU scratch (MOE_NOALLOC_SCRATCH_BYTES).  With ``out``
    and ``routing`` given, nothing is allocated; calls that overlap on one GPU
    race.  Returns (out, routing)."""
    return prepare_forward_noalloc(x, logits, w13, w2, topk, act, layout, params, out=out,
                                   routing=routing, stream=stream)()


def prepare_forward_ep(x, logits, w13, w2, topk: int, local_offset: int, act: str,
                       layout: str = "packed", params: Optional[dict] = None, *, out=None,
                       routing=None, workspace=None, stream=None) -> Prepared:
    dev = _dev(x, logits, w13, w2)
    n, hidden = x.shape
    e = logits.shape[1]
    nl, inter = w2.shape[0], w2.shape[2]
    _shapes(x, w13, w2, act, out, logits, n_experts=e)
    _share(e, local_offset, nl)
    if logits.dtype != x.dtype:
        raise TypeError("moe_forward_ep takes logits in the layer dtype")
    if routing is None:
        routing = Routing.empty(n, nl, topk, logits.dtype, dev)
    _check_routing(routing, n, nl, topk)
    if out is None:
        out = torch.empty_like(x)
    ws = _workspace(workspace, moe_workspace_bytes(n, e, topk, hidden, inter, x.dtype), dev)
    r = routing.as_c()
    p = _params(params)
    args = (x.data_ptr(), logits.data_ptr(), _dt(x), n, hidden, w13.data_ptr(), w2.data_ptr(),
            e, local_offset, nl, inter, topk, ACTS[act], LAYOUTS[layout],
            ctypes.byref(p) if p else None, ctypes.byref(r), out.data_ptr(), ws.data_ptr(),
            _nbytes(ws), _stream(dev, stream))
    return Prepared("moe_forward_ep", args, (r, p, x, logits, w13, w2, out, ws, routing),
                    (out, routing))


def moe_forward_ep(x: torch.Tensor, logits: torch.Tensor, w13: torch.Tensor, w2: torch.Tensor,
                   topk: int, local_offset: int, act: str, layout: str = "packed",
                   params: Optional[dict] = None, *, out: Optional[torch.Tensor] = None,
                   routing: Optional[Routing] = None, workspace: Optional[torch.Tensor] = None,
                   stream=None):
    """moe_route_ep then moe_experts_ep for the share of w13/w2's experts that
    starts at ``local_offset``; returns ``(out, routing)``."""
    return prepare_forward_ep(x, logits, w13, w2, topk, local_offset, act, layout, params,
                              out=out, routing=routing, workspace=workspace, stream=stream)()


def moe_forward(x: torch.Tensor, logits: torch.Tensor, w13: torch.Tensor, w2: torch.Tensor,
                topk: int, act: str, layout: str = "packed", params: Optional[dict] = None, *,
                out: Optional[torch.Tensor] = None, routing: Optional[Routing] = None,
                workspace: Optional[torch.Tensor] = None, stream=None):
    """Routing then experts on one stream; returns ``(out, routing)``."""
    return prepare_forward(x, logits, w13, w2, topk, act, layout, params, out=out,
                           routing=routing, workspace=workspace, stream=stream)()


def _gate_args(x, w_gate, logits):
    dev = _dev(x, w_gate)
    if x.dim() != 2 or w_gate.dim() != 2 or x.shape[1] != w_gate.shape[1]:
        raise ValueError("expected x [N, H] and w_gate [E, H]")
    if x.dtype != w_gate.dtype:
        raise TypeError("x and w_gate must share a dtype")
    n, e = x.shape[0], w_gate.shape[0]
    if logits is None:
        logits = torch.empty(n, e, dtype=x.dtype, device=dev)
    _dev(x, logits)
    if tuple(logits.shape) != (n, e) or logits.dtype != x.dtype:
        raise ValueError("logits must be [N, E] in the layer dtype")
    return dev, n, e, logits


def prepare_gate_route(x: torch.Tensor, w_gate: torch.Tensor, topk: int, *,
                       logits: Optional[torch.Tensor] = None, routing: Optional[Routing] = None,
                       workspace: Optional[torch.Tensor] = None, stream=None) -> Prepared:
    dev, n, e, logits = _gate_args(x, w_gate, logits)
    if routing is None:
        routing = Routing.empty(n, e, topk, x.dtype, dev)
    _check_routing(routing, n, e, topk)
    ws = _workspace(workspace, moe_workspace_bytes(n, e, topk, x.shape[1], 0, x.dtype), dev)
    r = routing.as_c()
    args = (x.data_ptr(), w_gate.data_ptr(), _dt(x), n, x.shape[1], e, topk, logits.data_ptr(),
            ctypes.byref(r), ws.data_ptr(), _nbytes(ws), _stream(dev, stream))
    return Prepared("moe_gate_route", args, (r, x, w_gate, logits, ws, routing),
                    (logits, routing))


def moe_gate_route(x: torch.Tensor, w_gate: torch.Tensor, topk: int, *,
                   logits: Optional[torch.Tensor] = None, routing: Optional[Routing] = None,
                   workspace: Optional[torch.Tensor] = None, stream=None):
    """Router GEMM ``logits = x . w_gate^T`` then the routing step; returns
    ``(logits, routing)`` (see moe.h)."""
    return prepare_gate_route(x, w_gate, topk, logits=logits, routing=routing,
                              workspace=workspace, stream=stream)()


def prepare_gate_forward(x, w_gate, w13, w2, topk: int, act: str, layout: str = "packed",
                         params: Optional[dict] = None, *, out=None, logits=None, routing=None,
                         workspace=None, stream=None) -> Prepared:
    dev, n, e, logits = _gate_args(x, w_gate, logits)
    _dev(x, w13, w2)
    _shapes(x, w13, w2, act, out, logits)
    hidden, inter = x.shape[1], w2.shape[2]
    if routing is None:
        routing = Routing.empty(n, e, topk, x.dtype, dev)
    _check_routing(routing, n, e, topk)
    if out is None:
        out = torch.empty_like(x)
    ws = _workspace(workspace, moe_workspace_bytes(n, e, topk, hidden, inter, x.dtype), dev)
    r = routing.as_c()
    p = _params(params)
    args = (x.data_ptr(), w_gate.data_ptr(), _dt(x), n, hidden, w13.data_ptr(), w2.data_ptr(),
            e, inter, topk, ACTS[act], LAYOUTS[layout], ctypes.byref(p) if p else None,
            logits.data_ptr(), ctypes.byref(r), out.data_ptr(), ws.data_ptr(), _nbytes(ws),
            _stream(dev, stream))
    return Prepared("moe_gate_forward", args,
                    (r, p, x, w_gate, w13, w2, out, logits, ws, routing), (out, logits, routing))


def moe_gate_forward(x: torch.Tensor, w_gate: torch.Tensor, w13: torch.Tensor, w2: torch.Tensor,
                     topk: int, act: str, layout: str = "packed", params: Optional[dict] = None,
                     *, out: Optional[torch.Tensor] = None, logits: Optional[torch.Tensor] = None,
                     routing: Optional[Routing] = None, workspace: Optional[torch.Tensor] = None,
                     stream=None):
    """The whole layer from the token rows and the router's gate weight;
    returns ``(out, logits, routing)``."""
    return prepare_gate_forward(x, w_gate, w13, w2, topk, act, layout, params, out=out,
                                logits=logits, routing=routing, workspace=workspace,
                                stream=stream)()


def prepare_experts_weighted_input(x, w13, w2, routing: Routing, act: str,
                                   layout: str = "packed", params: Optional[dict] = None, *,
                                   out=None, workspace=None, stream=None) -> Prepared:
    dev = _dev(x, w13, w2)
    _shapes(x, w13, w2, act, out)
    n, hidden = x.shape
    e, inter = w2.shape[0], w2.shape[2]
    k = routing.topk
    _check_routing(routing, n, e, k)
    if out is None:
        out = torch.empty_like(x)
    # the scaled input rows xs [N*k, hidden] follow the experts' workspace
    need = moe_workspace_bytes(n, max(e, k), k, hidden, inter, x.dtype) \
        + (n * k * hidden * x.element_size() + 255) // 256 * 256
    ws = _workspace(workspace, need, dev)
    r = routing.as_c()
    p = _params(params)
    args = (x.data_ptr(), _dt(x), n, hidden, w13.data_ptr(), w2.data_ptr(), e, inter, k,
            ACTS[act], LAYOUTS[layout], ctypes.byref(p) if p else None, ctypes.byref(r),
            out.data_ptr(), ws.data_ptr(), _nbytes(ws), _stream(dev, stream))
    return Prepared("moe_experts_weighted_input", args, (r, p, x, w13, w2, out, ws, routing), out)


def moe_experts_weighted_input(x: torch.Tensor, w13: torch.Tensor, w2: torch.Tensor,
                               routing: Routing, act: str, layout: str = "packed",
                               params: Optional[dict] = None, *,
                               out: Optional[torch.Tensor] = None,
                               workspace: Optional[torch.Tensor] = None,
                               stream=None) -> torch.Tensor:
    """Expert FFN with the routing weight applied to each entry's input row
    (rounded to the layer dtype) instead of its output (see moe.h)."""
    return prepare_experts_weighted_input(x, w13, w2, routing, act, layout, params, out=out,
                                          workspace=workspace, stream=stream)()


def moe_quantize_mxfp4(w: torch.Tensor, *, stream=None):
    """MXFP4 expert weights from ``w [E, rows, K]`` (K a multiple of 32): returns
    ``(q [E, rows, K/2] uint8, scales [E, K/32, rows] uint8)`` (see moe.h)."""
    dev = _dev(w)
    if w.dim() != 3:
        raise ValueError("expected w [E, rows, K]")
    e, rows, k = w.shape
    q = torch.empty(e, rows, k // 2, dtype=torch.uint8, device=dev)
    sc = torch.empty(e, k // 32, rows, dtype=torch.uint8, device=dev)
    _check(N.load().moe_quantize_mxfp4(w.data_ptr(), _dt(w), e, rows, k, q.data_ptr(),
                                       sc.data_ptr(), _stream(dev, stream)), "moe_quantize_mxfp4")
    return q, sc


def _mxfp4_shapes(x, w13_q, w13_s, w2_q, w2_s, act):
    """Codes and scales as moe_quantize_mxfp4 lays them out; returns (E, inter)."""
    if x.dtype != torch.bfloat16:
        raise TypeError("MXFP4 weights run a bf16 layer")
    for t in (w13_q, w13_s, w2_q, w2_s):
        if t.dtype != torch.uint8 or t.dim() != 3:
            raise TypeError("MXFP4 codes and scales are 3-D uint8 tensors")
    n, h = x.shape
    e, hh, half_i = w2_q.shape
    inter = 2 * half_i
    rows = inter if act == "relu2" else 2 * inter
    want = {"w13_q": (e, rows, h // 2), "w13_s": (e, h // 32, rows),
            "w2_q": (e, h, inter // 2), "w2_s": (e, inter // 32, h)}
    got = {"w13_q": w13_q, "w13_s": w13_s, "w2_q": w2_q, "w2_s": w2_s}
    if hh != h or h % 32 or inter % 32:
        raise ValueError("hidden and inter must be multiples of 32 and match x")
    for k, shp in want.items():
        if tuple(got[k].shape) != shp:
            raise ValueError(f"{k} must be {shp}, got {tuple(got[k].shape)}")
    return e, inter


def prepare_experts_mxfp4(x, w13_q, w13_s, w2_q, w2_s, routing: Routing, act: str,
                          layout: str = "packed", params: Optional[dict] = None, *, out=None,
                          workspace=None, stream=None) -> Prepared:
    dev = _dev(x, w13_q, w13_s, w2_q, w2_s)
    if act not in ACTS:
        raise ValueError(f"unknown activation {act!r}")
    e, inter = _mxfp4_shapes(x, w13_q, w13_s, w2_q, w2_s, act)
    n, hidden = x.shape
    k = routing.topk
    _check_routing(routing, n, e, k)
    if out is None:
        out = torch.empty_like(x)
    ws = _workspace(workspace, moe_workspace_bytes(n, max(e, k), k, hidden, inter, x.dtype), dev)
    r = routing.as_c()
    p = _params(params)
    args = (x.data_ptr(), _dt(x), n, hidden, w13_q.data_ptr(), w13_s.data_ptr(), w2_q.data_ptr(),
            w2_s.data_ptr(), e, inter, k, ACTS[act], LAYOUTS[layout],
            ctypes.byref(p) if p else None, ctypes.byref(r), out.data_ptr(), ws.data_ptr(),
            _nbytes(ws), _stream(dev, stream))
    return Prepared("moe_experts_mxfp4", args,
                    (r, p, x, w13_q, w13_s, w2_q, w2_s, out, ws, routing), out)


def moe_experts_mxfp4(x: torch.Tensor, w13_q: torch.Tensor, w13_s: torch.Tensor,
                      w2_q: torch.Tensor, w2_s: torch.Tensor, routing: Routing, act: str,
                      layout: str = "packed", params: Optional[dict] = None, *,
                      out: Optional[torch.Tensor] = None,
                      workspace: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    """moe_experts with MXFP4 expert weights (codes and scales from
    moe_quantize_mxfp4); bf16 layer (see moe.h)."""
    return prepare_experts_mxfp4(x, w13_q, w13_s, w2_q, w2_s, routing, act, layout, params,
                                 out=out, workspace=workspace, stream=stream)()


def prepare_forward_mxfp4(x, logits, w13_q, w13_s, w2_q, w2_s, topk: int, act: str,
                          layout: str = "packed", params: Optional[dict] = None, *, out=None,
                          routing=None, workspace=None, stream=None) -> Prepared:
    dev = _dev(x, logits, w13_q, w13_s, w2_q, w2_s)
    if act not in ACTS:
        raise ValueError(f"unknown activation {act!r}")
    e, inter = _mxfp4_shapes(x, w13_q, w13_s, w2_q, w2_s, act)
    n, hidden = x.shape
    if logits.dtype != x.dtype or tuple(logits.shape) != (n, e):
        raise ValueError("logits must be [N, E] in the layer dtype")
    if routing is None:
        routing = Routing.empty(n, e, topk, x.dtype, dev)
    _check_routing(routing, n, e, topk)
    if out is None:
        out = torch.empty_like(x)
    ws = _workspace(workspace, moe_workspace_bytes(n, e, topk, hidden, inter, x.dtype), dev)
    r = routing.as_c()
    p = _params(params)
    args = (x.data_ptr(), logits.data_ptr(), _dt(x), n, hidden, w13_q.data_ptr(),
            w13_s.data_ptr(), w2_q.data_ptr(), w2_s.data_ptr(), e, inter, topk, ACTS[act],
            LAYOUTS[layout], ctypes.byref(p) if p else None, ctypes.byref(r), out.data_ptr(),
            ws.data_ptr(), _nbytes(ws), _stream(dev, stream))
    return Prepared("moe_forward_mxfp4", args,
                    (r, p, x, logits, w13_q, w13_s, w2_q, w2_s, out, ws, routing),
                    (out, routing))


def moe_forward_mxfp4(x: torch.Tensor, logits: torch.Tensor, w13_q: torch.Tensor,
                      w13_s: torch.Tensor, w2_q: torch.Tensor, w2_s: torch.Tensor, topk: int,
                      act: str, layout: str = "packed", params: Optional[dict] = None, *,
                      out: Optional[torch.Tensor] = None, routing: Optional[Routing] = None,
                      workspace: Optional[torch.Tensor] = None, stream=None):
    """Routing then the MXFP4-weight experts on one stream; returns ``(out, routing)``."""
    return prepare_forward_mxfp4(x, logits, w13_q, w13_s, w2_q, w2_s, topk, act, layout, params,
                                 out=out, routing=routing, workspace=workspace, stream=stream)()
