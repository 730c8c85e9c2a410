"""ctypes view of libmoe.so (declarations mirror include/moe.h)."""
from __future__ import annotations

import ctypes
import os

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libmoe.so")

c_i32, c_i64, c_u32, c_sz, c_vp, c_f = (ctypes.c_int32, ctypes.c_int64, ctypes.c_uint32,
                                        ctypes.c_size_t, ctypes.c_void_p, ctypes.c_float)

# moe_status_t
MOE_OK, MOE_ERR_NULL, MOE_ERR_SHAPE, MOE_ERR_DTYPE = 0, -1, -2, -3
MOE_ERR_UNSUPPORTED, MOE_ERR_ALIGN, MOE_ERR_WORKSPACE, MOE_ERR_HIP = -4, -5, -6, -7
MOE_ERR_SCRATCH = -8
MOE_NOALLOC_SCRATCH_BYTES = 64 << 20
# moe_dtype_t, moe_act_t, moe_w13_layout_t
MOE_F32, MOE_BF16 = 0, 1
MOE_ACT_SILU, MOE_ACT_SWIGLU_OAI, MOE_ACT_RELU2 = 0, 1, 2
MOE_W13_PACKED, MOE_W13_INTERLEAVED = 0, 1
MOE_PARAM_ALPHA, MOE_PARAM_BETA, MOE_PARAM_LIMIT = 1, 2, 4


class MoeActParams(ctypes.Structure):
    _fields_ = [("alpha", c_f), ("beta", c_f), ("limit", c_f), ("set", c_u32)]


class MoeRouting(ctypes.Structure):
    _fields_ = [("topk_idx", c_vp), ("topk_w", c_vp), ("bitmatrix", c_vp), ("col_sum", c_vp),
                ("offsets", c_vp), ("col_sorted", c_vp), ("row_sorted", c_vp),
                ("gate_scal", c_vp), ("w_dtype", c_i32)]


_P_ROUTING = ctypes.POINTER(MoeRouting)
_P_PARAMS = ctypes.POINTER(MoeActParams)

# name -> (restype, argtypes); every function include/moe.h declares
SIGNATURES = {
    "moe_workspace_bytes": (c_sz, [c_i64, c_i32, c_i32, c_i32, c_i32, c_i32]),
    "moe_route": (c_i32, [c_vp, c_i32, c_i64, c_i32, c_i32, _P_ROUTING, c_vp, c_sz, c_vp]),
    "moe_experts": (c_i32, [c_vp, c_i32, c_i64, c_i32, c_vp, c_vp, c_i32, c_i32, c_i32, c_i32,
                            c_i32, _P_PARAMS, _P_ROUTING, c_vp, c_vp, c_sz, c_vp]),
    "moe_experts_w13": (c_i32, [c_vp, c_i32, c_i64, c_i32, c_vp, c_i32, c_i32, c_i32, c_i32,
                                c_i32, _P_PARAMS, _P_ROUTING, c_vp, c_vp]),
    "moe_experts_w2": (c_i32, [c_vp, c_i32, c_i64, c_i32, c_vp, c_i32, c_i32, c_i32, _P_ROUTING,
                               c_vp, c_vp, c_sz, c_vp]),
    "moe_experts_w2_rows": (c_i32, [c_vp, c_i32, c_i64, c_i32, c_vp, c_i32, c_i32, c_i32,
                                    _P_ROUTING, c_vp, c_vp]),
    "moe_combine": (c_i32, [c_vp, c_i32, c_i64, c_i32, c_i32, _P_ROUTING, c_vp, c_vp]),
    "moe_forward": (c_i32, [c_vp, c_vp, c_i32, c_i64, c_i32, c_vp, c_vp, c_i32, c_i32, c_i32,
                            c_i32, c_i32, _P_PARAMS, _P_ROUTING, c_vp, c_vp, c_sz, c_vp]),
    "moe_forward_noalloc": (c_i32, [c_vp, c_vp, c_i32, c_i64, c_i32, c_vp, c_vp, c_i32, c_i32,
                                    c_i32, c_i32, c_i32, _P_PARAMS, _P_ROUTING, c_vp, c_vp]),
    "moe_route_ep": (c_i32, [c_vp, c_i32, c_i64, c_i32, c_i32, c_i32, c_i32, _P_ROUTING, c_vp,
                             c_sz, c_vp]),
    "moe_experts_ep": (c_i32, [c_vp, c_i32, c_i64, c_i32, c_vp, c_vp, c_i32, c_i32, c_i32,
                               c_i32, c_i32, _P_PARAMS, _P_ROUTING, c_vp, c_vp, c_sz, c_vp]),
    "moe_forward_ep": (c_i32, [c_vp, c_vp, c_i32, c_i64, c_i32, c_vp, c_vp, c_i32, c_i32, c_i32,
                               c_i32, c_i32, c_i32, c_i32, _P_PARAMS, _P_ROUTING, c_vp, c_vp,
                               c_sz, c_vp]),
    "moe_gate_route": (c_i32, [c_vp, c_vp, c_i32, c_i64, c_i32, c_i32, c_i32, c_vp, _P_ROUTING,
                               c_vp, c_sz, c_vp]),
    "moe_gate_forward": (c_i32, [c_vp, c_vp, c_i32, c_i64, c_i32, c_vp, c_vp, c_i32, c_i32,
                                 c_i32, c_i32, c_i32, _P_PARAMS, c_vp, _P_ROUTING, c_vp, c_vp,
                                 c_sz, c_vp]),
    "moe_experts_weighted_input": (c_i32, [c_vp, c_i32, c_i64, c_i32, c_vp, c_vp, c_i32, c_i32,
                                           c_i32, c_i32, c_i32, _P_PARAMS, _P_ROUTING, c_vp,
                                           c_vp, c_sz, c_vp]),
    "moe_quantize_mxfp4": (c_i32, [c_vp, c_i32, c_i32, c_i32, c_i32, c_vp, c_vp, c_vp]),
    "moe_experts_mxfp4": (c_i32, [c_vp, c_i32, c_i64, c_i32, c_vp, c_vp, c_vp, c_vp, c_i32, c_i32,
                                  c_i32, c_i32, c_i32, _P_PARAMS, _P_ROUTING, c_vp, c_vp, c_sz,
                                  c_vp]),
    "moe_forward_mxfp4": (c_i32, [c_vp, c_vp, c_i32, c_i64, c_i32, c_vp, c_vp, c_vp, c_vp, c_i32,
                                  c_i32, c_i32, c_i32, c_i32, _P_PARAMS, _P_ROUTING, c_vp, c_vp,
                                  c_sz, c_vp]),
    "moe_status_str": (ctypes.c_char_p, [c_i32]),
}

_lib = None


def load(path: str | None = None) -> ctypes.CDLL:
    """Load libmoe.so once; raise if it has not been built."""
    global _lib
    if _lib is not None and path is None:
        return _lib
    p = path or LIB_PATH
    if not os.path.exists(p):
        raise RuntimeError(
            f"{p} is missing: build the HIP library first "
            "(python -m routing_grouped_expert_amd.build, or __graft_entry__.build())")
    lib = ctypes.CDLL(p)
    for name, (res, args) in SIGNATURES.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    if path is None:
        _lib = lib
    return lib
