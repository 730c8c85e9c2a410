"""libmoe.so loads, exports every function moe.h declares, and rejects bad
arguments with the documented status before any HIP call (CPU only: nothing here
launches a kernel or touches device memory; the non-NULL pointers are never
dereferenced because every call returns an error first)."""
import ctypes
import os
import re

import pytest

from routing_grouped_expert_amd import _native as N

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "moe.h")

FAKE = 0x10000          # aligned, never dereferenced
MISALIGNED = 0x10008


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(N.LIB_PATH):
        from routing_grouped_expert_amd.build import build
        build()
    return N.load()


def declared_functions():
    txt = open(HEADER).read()
    txt = re.sub(r"/\*.*?\*/", "", txt, flags=re.S)
    return sorted(set(re.findall(r"\b(moe_[a-z0-9_]+)\s*\(", txt)))


def test_every_declared_symbol_is_exported(lib):
    names = declared_functions()
    assert set(names) == set(N.SIGNATURES), names
    for name in names:
        assert hasattr(lib, name), name


def test_status_strings(lib):
    for code in range(0, -9, -1):
        s = lib.moe_status_str(code).decode()
        assert s and s != "unknown status", code
    assert lib.moe_status_str(-99).decode() == "unknown status"


def test_workspace_sizes(lib):
    ok = lib.moe_workspace_bytes(4096, 8, 1, 512, 1408, N.MOE_BF16)
    assert ok >= 4096 * 1408 * 2
    # k > 1 adds the weighted expert-output rows
    assert lib.moe_workspace_bytes(33, 8, 2, 128, 256, N.MOE_F32) >= 66 * (256 + 128) * 4
    assert lib.moe_workspace_bytes(65536, 128, 4, 0, 0, N.MOE_BF16) > 0   # routing only
    for bad in [(-1, 8, 1, 512, 512), (16, 0, 1, 512, 512), (16, 8, 9, 512, 512),
                (16, 300, 4, 512, 512), (16, 32, 17, 512, 512), (16, 8, 2, 500, 512),
                (16, 8, 2, 512, 12)]:
        assert lib.moe_workspace_bytes(*bad, N.MOE_BF16) == 0, bad
    assert lib.moe_workspace_bytes(16, 8, 2, 512, 512, 7) == 0


def test_workspace_sizes_router_gemm(lib):
    # hidden given: room for the router GEMM's split-K partial sums as well; every
    # batch size is defined, the empty batch included
    for n in (0, 1, 64, 65, 4096, 4097, 65536):
        assert lib.moe_workspace_bytes(n, 128, 4, 2880, 0, N.MOE_BF16) > 0, n
        assert lib.moe_workspace_bytes(n, 128, 4, 2880, 2880, N.MOE_BF16) > 0, n
    assert lib.moe_workspace_bytes(0, 8, 2, 128, 256, N.MOE_F32) > 0
    # five tokens: fp32 sums of 23 K-slices (2880 bf16 values in 256-byte slices)
    # for each token and each of the 128 experts (up to four tokens need none)
    assert lib.moe_workspace_bytes(5, 128, 4, 2880, 0, N.MOE_BF16) >= 23 * 5 * 128 * 4


def routing(fields=None, w_dtype=N.MOE_BF16, ptr=FAKE):
    r = N.MoeRouting(*([ptr] * 8), w_dtype)
    for k, v in (fields or {}).items():
        setattr(r, k, v)
    return r


def route(lib, logits=FAKE, dt=N.MOE_BF16, n=33, e=32, k=4, r=None, ws=FAKE, wsb=1 << 30):
    r = r if r is not None else routing(w_dtype=dt)
    return lib.moe_route(logits, dt, n, e, k, ctypes.byref(r), ws, wsb, None)


def test_route_argument_checks(lib):
    assert route(lib, n=0, logits=None, ws=None) == N.MOE_OK          # empty: nothing enqueued
    assert route(lib, logits=None) == N.MOE_ERR_NULL
    assert route(lib, r=routing({"col_sorted": None})) == N.MOE_ERR_NULL
    assert lib.moe_route(FAKE, N.MOE_BF16, 5, 8, 2, None, FAKE, 1 << 20, None) == N.MOE_ERR_NULL
    assert route(lib, k=0) == N.MOE_ERR_SHAPE
    assert route(lib, k=9, e=8) == N.MOE_ERR_SHAPE
    assert route(lib, k=17, e=64) == N.MOE_ERR_SHAPE
    assert route(lib, e=257) == N.MOE_ERR_SHAPE
    assert route(lib, n=-1) == N.MOE_ERR_SHAPE
    assert route(lib, n=1 << 30, k=4) == N.MOE_ERR_SHAPE               # N*k >= 2^31
    assert route(lib, dt=5) == N.MOE_ERR_DTYPE
    assert route(lib, r=routing(w_dtype=N.MOE_F32)) == N.MOE_ERR_DTYPE  # weights inherit
    assert route(lib, logits=MISALIGNED) == N.MOE_ERR_ALIGN
    assert route(lib, r=routing({"gate_scal": MISALIGNED})) == N.MOE_ERR_ALIGN
    # small batches route inside one workgroup with no scratch, so the
    # workspace checks use a batch that needs it
    assert lib.moe_workspace_bytes(4096, 8, 2, 0, 0, N.MOE_BF16) > 16
    assert route(lib, n=4096, ws=None) == N.MOE_ERR_WORKSPACE
    assert route(lib, n=4096, wsb=16) == N.MOE_ERR_WORKSPACE


def experts(lib, n=33, h=128, e=8, i=256, k=2, act=N.MOE_ACT_SILU, layout=N.MOE_W13_PACKED,
            params=None, x=FAKE, r=None, ws=FAKE, wsb=1 << 30, dt=N.MOE_BF16):
    r = r if r is not None else routing(w_dtype=dt)
    p = ctypes.byref(params) if params is not None else None
    return lib.moe_experts(x, dt, n, h, FAKE, FAKE, e, i, k, act, layout, p, ctypes.byref(r),
                           FAKE, ws, wsb, None)


def test_experts_argument_checks(lib):
    assert experts(lib, n=0, x=None, ws=None) == N.MOE_OK
    assert experts(lib, x=None) == N.MOE_ERR_NULL
    assert experts(lib, r=routing({"offsets": None})) == N.MOE_ERR_NULL
    assert experts(lib, h=100) == N.MOE_ERR_SHAPE
    assert experts(lib, i=0) == N.MOE_ERR_SHAPE
    assert experts(lib, k=3, e=2) == N.MOE_ERR_SHAPE
    # sorted expert outputs n * k * hidden * 2 bytes = 2^32: over the 2^31 limit
    assert experts(lib, n=1 << 19, h=1024, i=8, k=4) == N.MOE_ERR_SHAPE
    assert experts(lib, dt=9) == N.MOE_ERR_DTYPE
    assert experts(lib, act=7) == N.MOE_ERR_UNSUPPORTED
    assert experts(lib, layout=2) == N.MOE_ERR_UNSUPPORTED
    assert experts(lib, act=N.MOE_ACT_RELU2, layout=N.MOE_W13_INTERLEAVED) == N.MOE_ERR_UNSUPPORTED
    assert experts(lib, params=N.MoeActParams(1, 0, 0, 8)) == N.MOE_ERR_UNSUPPORTED
    nan = float("nan")
    assert experts(lib, params=N.MoeActParams(1, 0, nan, N.MOE_PARAM_LIMIT)) == N.MOE_ERR_SHAPE
    assert experts(lib, params=N.MoeActParams(1, 0, -1.0, N.MOE_PARAM_LIMIT)) == N.MOE_ERR_SHAPE
    assert experts(lib, act=N.MOE_ACT_SWIGLU_OAI,
                   params=N.MoeActParams(nan, 0, 7, N.MOE_PARAM_ALPHA)) == N.MOE_ERR_SHAPE
    assert experts(lib, x=MISALIGNED) == N.MOE_ERR_ALIGN
    assert experts(lib, ws=None) == N.MOE_ERR_WORKSPACE
    assert experts(lib, wsb=1024) == N.MOE_ERR_WORKSPACE


def test_forward_argument_checks(lib):
    r = routing()
    args = lambda **kw: dict(dict(x=FAKE, lg=FAKE, n=33, e=8, k=2, act=N.MOE_ACT_SILU,
                                  layout=N.MOE_W13_PACKED, ws=FAKE, wsb=1 << 30), **kw)

    def fwd(x, lg, n, e, k, act, layout, ws, wsb):
        return lib.moe_forward(x, lg, N.MOE_BF16, n, 128, FAKE, FAKE, e, 256, k, act, layout,
                               None, ctypes.byref(r), FAKE, ws, wsb, None)
    assert fwd(**args(n=0, x=None, lg=None, ws=None)) == N.MOE_OK
    assert fwd(**args(lg=None)) == N.MOE_ERR_NULL
    assert fwd(**args(x=None)) == N.MOE_ERR_NULL
    assert fwd(**args(k=0)) == N.MOE_ERR_SHAPE
    assert fwd(**args(act=N.MOE_ACT_RELU2, layout=N.MOE_W13_INTERLEAVED)) == N.MOE_ERR_UNSUPPORTED
    assert fwd(**args(wsb=256)) == N.MOE_ERR_WORKSPACE


def test_half_entry_points_argument_checks(lib):
    r = routing()
    w13 = lambda **kw: lib.moe_experts_w13(
        kw.get("x", FAKE), N.MOE_BF16, kw.get("n", 33), 128, FAKE, 8, 256, kw.get("k", 2),
        kw.get("act", N.MOE_ACT_SILU), kw.get("layout", N.MOE_W13_PACKED), None,
        ctypes.byref(r), kw.get("a", FAKE), None)
    assert w13(n=0, x=None, a=None) == N.MOE_OK
    assert w13(a=None) == N.MOE_ERR_NULL
    assert w13(a=MISALIGNED) == N.MOE_ERR_ALIGN
    assert w13(k=9) == N.MOE_ERR_SHAPE
    assert w13(act=N.MOE_ACT_RELU2, layout=N.MOE_W13_INTERLEAVED) == N.MOE_ERR_UNSUPPORTED
    w2 = lambda **kw: lib.moe_experts_w2(
        kw.get("a", FAKE), N.MOE_BF16, kw.get("n", 33), 128, FAKE, 8, 256, kw.get("k", 2),
        ctypes.byref(r), FAKE, kw.get("ws", FAKE), kw.get("wsb", 1 << 30), None)
    assert w2(n=0, a=None, ws=None) == N.MOE_OK
    assert w2(a=None) == N.MOE_ERR_NULL
    assert w2(ws=None) == N.MOE_ERR_WORKSPACE            # topk 2 needs the weighted rows
    assert w2(wsb=64) == N.MOE_ERR_WORKSPACE


def test_noalloc_forward_argument_checks(lib):
    r = routing()

    def fwd(n=33, e=8, k=2, h=128, i=256, x=FAKE, lg=FAKE, out=FAKE, dt=N.MOE_BF16):
        return lib.moe_forward_noalloc(x, lg, dt, n, h, FAKE, FAKE, e, i, k, N.MOE_ACT_SILU,
                                       N.MOE_W13_PACKED, None, ctypes.byref(r), out, None)
    assert fwd(n=0, x=None, lg=None, out=None) == N.MOE_OK   # empty: nothing enqueued
    assert fwd(x=None) == N.MOE_ERR_NULL
    assert fwd(lg=MISALIGNED) == N.MOE_ERR_ALIGN
    assert fwd(k=0) == N.MOE_ERR_SHAPE
    assert fwd(h=100) == N.MOE_ERR_SHAPE
    assert fwd(dt=6) == N.MOE_ERR_DTYPE
    # past the static scratch: rejected before any device call
    assert lib.moe_workspace_bytes(4096, 128, 4, 2880, 2880, N.MOE_BF16) > \
        N.MOE_NOALLOC_SCRATCH_BYTES
    assert fwd(n=4096, e=128, k=4, h=2880, i=2880) == N.MOE_ERR_SCRATCH
    assert fwd(n=1457, e=128, k=4, h=2880, i=2880) == N.MOE_ERR_SCRATCH


def test_w2_rows_and_combine_argument_checks(lib):
    r = routing()
    rows = lambda **kw: lib.moe_experts_w2_rows(
        kw.get("a", FAKE), kw.get("dt", N.MOE_BF16), kw.get("n", 33), kw.get("h", 128), FAKE,
        kw.get("e", 8), 256, kw.get("k", 2), ctypes.byref(kw.get("r", r)), kw.get("y", FAKE),
        None)
    assert rows(n=0, a=None, y=None) == N.MOE_OK
    assert rows(a=None) == N.MOE_ERR_NULL
    assert rows(y=None) == N.MOE_ERR_NULL
    assert rows(y=MISALIGNED) == N.MOE_ERR_ALIGN
    assert rows(r=routing({"gate_scal": None})) == N.MOE_ERR_NULL
    assert rows(h=100) == N.MOE_ERR_SHAPE
    assert rows(k=17) == N.MOE_ERR_SHAPE
    assert rows(dt=3) == N.MOE_ERR_DTYPE
    comb = lambda **kw: lib.moe_combine(
        kw.get("y", FAKE), kw.get("dt", N.MOE_BF16), kw.get("n", 33), kw.get("h", 128),
        kw.get("k", 2), kw.get("rp", ctypes.byref(kw.get("r", r))), kw.get("out", FAKE), None)
    assert comb(n=0, y=None, out=None) == N.MOE_OK
    assert comb(y=None) == N.MOE_ERR_NULL
    assert comb(out=None) == N.MOE_ERR_NULL
    assert comb(rp=None) == N.MOE_ERR_NULL
    assert comb(r=routing({"row_sorted": None})) == N.MOE_ERR_NULL
    assert comb(r=routing({"row_sorted": MISALIGNED})) == N.MOE_ERR_ALIGN
    assert comb(out=MISALIGNED) == N.MOE_ERR_ALIGN
    assert comb(h=12) == N.MOE_ERR_SHAPE
    assert comb(k=0) == N.MOE_ERR_SHAPE
    assert comb(k=17) == N.MOE_ERR_SHAPE
    assert comb(n=1 << 30, k=4) == N.MOE_ERR_SHAPE
    assert comb(dt=4) == N.MOE_ERR_DTYPE


def test_share_entry_points_argument_checks(lib):
    r = routing()

    def route_ep(lo, nl, n=33, e=32, k=4, lg=FAKE, ws=FAKE):
        return lib.moe_route_ep(lg, N.MOE_BF16, n, e, k, lo, nl, ctypes.byref(r), ws, 1 << 30,
                                None)
    assert route_ep(0, 8, n=0, lg=None, ws=None) == N.MOE_OK          # empty: nothing enqueued
    for lo, nl in [(-1, 4), (0, 0), (29, 4), (32, 1), (0, 33), (1 << 30, 8)]:
        assert route_ep(lo, nl) == N.MOE_ERR_SHAPE, (lo, nl)
    assert route_ep(0, 8, k=33) == N.MOE_ERR_SHAPE                    # k > E still rejected
    assert route_ep(0, 8, lg=None) == N.MOE_ERR_NULL
    assert route_ep(0, 8, lg=MISALIGNED) == N.MOE_ERR_ALIGN
    assert route_ep(0, 8, n=4096, ws=None) == N.MOE_ERR_WORKSPACE

    def experts_ep(nl=2, k=4, n=33, x=FAKE, wsb=1 << 30):
        return lib.moe_experts_ep(x, N.MOE_BF16, n, 128, FAKE, FAKE, nl, 256, k, N.MOE_ACT_SILU,
                                  N.MOE_W13_PACKED, None, ctypes.byref(r), FAKE, FAKE, wsb, None)
    assert experts_ep(n=0, x=None) == N.MOE_OK
    assert experts_ep(nl=0) == N.MOE_ERR_SHAPE
    assert experts_ep(nl=257) == N.MOE_ERR_SHAPE
    assert experts_ep(k=17) == N.MOE_ERR_SHAPE
    assert experts_ep(x=None) == N.MOE_ERR_NULL
    assert experts_ep(wsb=1024) == N.MOE_ERR_WORKSPACE

    def fwd_ep(lo, nl, e=16, k=4, n=33):
        return lib.moe_forward_ep(FAKE, FAKE, N.MOE_BF16, n, 128, FAKE, FAKE, e, lo, nl, 256, k,
                                  N.MOE_ACT_SILU, N.MOE_W13_PACKED, None, ctypes.byref(r), FAKE,
                                  FAKE, 1 << 30, None)
    assert fwd_ep(4, 4, n=0) == N.MOE_OK
    assert fwd_ep(13, 4) == N.MOE_ERR_SHAPE
    assert fwd_ep(-2, 4) == N.MOE_ERR_SHAPE
    assert fwd_ep(0, 4, k=17) == N.MOE_ERR_SHAPE


def test_gate_entry_points_argument_checks(lib):
    r = routing()

    def gate(n=33, h=128, e=16, k=4, x=FAKE, wg=FAKE, lg=FAKE, dt=N.MOE_BF16, ws=FAKE):
        return lib.moe_gate_route(x, wg, dt, n, h, e, k, lg, ctypes.byref(r), ws, 1 << 30, None)
    assert gate(n=0, x=None, wg=None, lg=None, ws=None) == N.MOE_OK
    assert gate(x=None) == N.MOE_ERR_NULL
    assert gate(wg=None) == N.MOE_ERR_NULL
    assert gate(lg=None) == N.MOE_ERR_NULL
    assert gate(lg=MISALIGNED) == N.MOE_ERR_ALIGN
    assert gate(h=100) == N.MOE_ERR_SHAPE                        # not a multiple of 8
    assert gate(e=257) == N.MOE_ERR_SHAPE
    assert gate(k=17) == N.MOE_ERR_SHAPE
    assert gate(n=1 << 20, h=1 << 11) == N.MOE_ERR_SHAPE         # x over 2^31 bytes
    assert gate(dt=7) == N.MOE_ERR_DTYPE
    assert gate(n=4096, ws=None) == N.MOE_ERR_WORKSPACE

    def gfwd(n=33, x=FAKE, act=N.MOE_ACT_SILU, layout=N.MOE_W13_PACKED, wsb=1 << 30):
        return lib.moe_gate_forward(x, FAKE, N.MOE_BF16, n, 128, FAKE, FAKE, 8, 256, 2, act,
                                    layout, None, FAKE, ctypes.byref(r), FAKE, FAKE, wsb, None)
    assert gfwd(n=0) == N.MOE_OK
    assert gfwd(x=None) == N.MOE_ERR_NULL
    assert gfwd(act=N.MOE_ACT_RELU2, layout=N.MOE_W13_INTERLEAVED) == N.MOE_ERR_UNSUPPORTED
    assert gfwd(wsb=256) == N.MOE_ERR_WORKSPACE
