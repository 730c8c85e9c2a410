// C-ABI entry points of libmoe.so: argument checks, workspace layout, launch
// order.  Every check runs before the first launch, so a rejected call writes
// nothing.  No entry point allocates, frees, synchronises or keeps state.
#include <math.h>

#include <initializer_list>
#include <mutex>

#include "moe_common.h"

namespace {

using moe::ActParams;

inline size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }
inline bool aligned16(const void *p) { return ((uintptr_t)p & 15u) == 0; }
inline bool dtype_ok(int d) { return d == MOE_F32 || d == MOE_BF16; }
inline size_t dsize(int d) { return d == MOE_BF16 ? 2 : 4; }
// moe_combine sees no expert count: the size check takes the largest one
constexpr int32_t kCombineAnyExperts = moe::kMaxExperts;

// Sizes shared by all entry points.  An expert-parallel share may hold fewer
// experts than a token selects (k_le_e = false for its expert count).
moe_status_t check_sizes(int64_t n, int32_t e, int32_t k, bool k_le_e = true) {
  if (n < 0 || e < 1 || e > moe::kMaxExperts || k < 1 || k > moe::kMaxTopk || (k_le_e && k > e))
    return MOE_ERR_SHAPE;
  if (n > (int64_t)0x7fffffff / k) return MOE_ERR_SHAPE;
  return MOE_OK;
}

moe_status_t check_ffn_sizes(int32_t hidden, int32_t inter) {
  if (hidden < 8 || inter < 8 || hidden % 8 || inter % 8) return MOE_ERR_SHAPE;
  if (hidden > (1 << 24) || inter > (1 << 24)) return MOE_ERR_SHAPE;
  return MOE_OK;
}

size_t experts_ws_bytes(int64_t n, int32_t k, int32_t hidden, int32_t inter, int dt) {
  const size_t m = (size_t)n * k;
  size_t b = align256(m * inter * dsize(dt));  // activation rows a[M, inter]
  if (k > 1) b += align256(m * hidden * dsize(dt));  // weighted expert outputs y[M, hidden]
  return b;
}

moe_status_t check_routing_struct(const moe_routing_t *r, bool for_route, int64_t n) {
  if (!r) return MOE_ERR_NULL;
  if (!dtype_ok(r->w_dtype)) return MOE_ERR_DTYPE;
  if (n == 0) return MOE_OK;
  const void *need_exp[] = {r->offsets, r->col_sorted, r->row_sorted, r->gate_scal};
  for (const void *p : need_exp) {
    if (!p) return MOE_ERR_NULL;
    if (!aligned16(p)) return MOE_ERR_ALIGN;
  }
  if (for_route) {
    const void *need_rt[] = {r->topk_idx, r->topk_w, r->bitmatrix, r->col_sum};
    for (const void *p : need_rt) {
      if (!p) return MOE_ERR_NULL;
      if (!aligned16(p)) return MOE_ERR_ALIGN;
    }
  }
  return MOE_OK;
}

moe_status_t act_params(moe_act_t act, moe_w13_layout_t layout, const moe_act_params_t *p,
                        ActParams *out) {
  if (act != MOE_ACT_SILU && act != MOE_ACT_SWIGLU_OAI && act != MOE_ACT_RELU2)
    return MOE_ERR_UNSUPPORTED;
  if (layout != MOE_W13_PACKED && layout != MOE_W13_INTERLEAVED) return MOE_ERR_UNSUPPORTED;
  if (act == MOE_ACT_RELU2 && layout != MOE_W13_PACKED) return MOE_ERR_UNSUPPORTED;
  const uint32_t set = p ? p->set : 0u;
  if (set & ~(MOE_PARAM_ALPHA | MOE_PARAM_BETA | MOE_PARAM_LIMIT)) return MOE_ERR_UNSUPPORTED;
  // unset fields keep the plain-SwiGLU defaults; SiLU reads only the limit
  out->alpha = 1.f;
  out->beta = 0.f;
  out->limit = INFINITY;
  if (act == MOE_ACT_RELU2) return MOE_OK;
  if (set & MOE_PARAM_LIMIT) {
    if (!(p->limit >= 0.f)) return MOE_ERR_SHAPE;  // also rejects NaN
    out->limit = p->limit;
  }
  if (act == MOE_ACT_SWIGLU_OAI) {
    if (set & MOE_PARAM_ALPHA) out->alpha = p->alpha;
    if (set & MOE_PARAM_BETA) out->beta = p->beta;
    if (!isfinite(out->alpha) || !isfinite(out->beta)) return MOE_ERR_SHAPE;
  }
  return MOE_OK;
}

// Checks shared by the expert entry points: sizes, dtype, activation, routing.
moe_status_t check_expert_args(moe_dtype_t dtype, int64_t n, int32_t hidden, int32_t e,
                               int32_t inter, int32_t k, moe_act_t act, moe_w13_layout_t layout,
                               const moe_act_params_t *params, const moe_routing_t *routing,
                               ActParams *prm, bool share = false) {
  moe_status_t st = check_sizes(n, e, k, !share);
  if (st != MOE_OK) return st;
  if ((st = check_ffn_sizes(hidden, inter)) != MOE_OK) return st;
  if (!dtype_ok(dtype)) return MOE_ERR_DTYPE;
  // the GEMMs address one expert's w13 / w2 block, x and the activation rows
  // with 32-bit byte offsets
  const int64_t lim = 0x7fffffff, es = (int64_t)dsize(dtype);
  if ((int64_t)2 * inter * hidden * es > lim || n * hidden * es > lim ||
      n * k * (int64_t)inter * es > lim || n * k * (int64_t)hidden * es > lim)
    return MOE_ERR_SHAPE;
  if ((st = act_params(act, layout, params, prm)) != MOE_OK) return st;
  return check_routing_struct(routing, false, n);
}

moe_status_t check_ptrs(std::initializer_list<const void *> ptrs) {
  for (const void *p : ptrs) {
    if (!p) return MOE_ERR_NULL;
    if (!aligned16(p)) return MOE_ERR_ALIGN;
  }
  return MOE_OK;
}

moe_status_t check_ws(const void *ws, size_t have, size_t need) {
  if (need == 0) return MOE_OK;
  if (!ws) return MOE_ERR_WORKSPACE;
  if (!aligned16(ws)) return MOE_ERR_ALIGN;
  return have < need ? MOE_ERR_WORKSPACE : MOE_OK;
}

size_t y_bytes(int64_t n, int32_t k, int32_t hidden, int dt) {
  return k > 1 ? align256((size_t)n * k * hidden * dsize(dt)) : 0;
}

moe_status_t check_experts(const void *x, moe_dtype_t dtype, int64_t n, int32_t hidden,
                           const void *w13, const void *w2, int32_t e, int32_t inter, int32_t k,
                           moe_act_t act, moe_w13_layout_t layout, const moe_act_params_t *params,
                           const moe_routing_t *routing, void *out, void *ws, size_t ws_bytes,
                           ActParams *prm, bool share = false) {
  moe_status_t st = check_expert_args(dtype, n, hidden, e, inter, k, act, layout, params,
                                      routing, prm, share);
  if (st != MOE_OK || n == 0) return st;
  if ((st = check_ptrs({x, w13, w2, out})) != MOE_OK) return st;
  return check_ws(ws, ws_bytes, experts_ws_bytes(n, k, hidden, inter, dtype));
}

moe_status_t check_route(const void *logits, moe_dtype_t dt, int64_t n, int32_t e, int32_t k,
                         const moe_routing_t *out, void *ws, size_t ws_bytes) {
  moe_status_t st = check_sizes(n, e, k);
  if (st != MOE_OK) return st;
  if (!dtype_ok(dt)) return MOE_ERR_DTYPE;
  if ((st = check_routing_struct(out, true, n)) != MOE_OK) return st;
  if (out->w_dtype != dt) return MOE_ERR_DTYPE;  // the weights inherit the gating dtype
  if (n == 0) return MOE_OK;
  if (!logits) return MOE_ERR_NULL;
  if (!aligned16(logits)) return MOE_ERR_ALIGN;
  if (!ws) return MOE_ERR_WORKSPACE;
  if (!aligned16(ws)) return MOE_ERR_ALIGN;
  if (ws_bytes < moe::route_scratch_bytes(n, e, k)) return MOE_ERR_WORKSPACE;
  return MOE_OK;
}

// Router GEMM operands: x [n, hidden], w_gate [e, hidden], logits_out [n, e].
moe_status_t check_gate(const void *x, const void *w_gate, moe_dtype_t dt, int64_t n,
                        int32_t hidden, int32_t e, void *logits_out) {
  if (!dtype_ok(dt)) return MOE_ERR_DTYPE;
  if (hidden < 8 || hidden % 8 || hidden > (1 << 24) || e < 1 || e > moe::kMaxExperts || n < 0)
    return MOE_ERR_SHAPE;
  const int64_t lim = 0x7fffffff, es = (int64_t)dsize(dt);
  if (n * hidden * es > lim || n * e * es > lim || (int64_t)e * hidden * es > lim)
    return MOE_ERR_SHAPE;
  if (n == 0) return MOE_OK;
  return check_ptrs({x, w_gate, logits_out});
}

// The expert-parallel share [lo, lo + nl) must lie inside [0, e).
moe_status_t check_share(int32_t e, int32_t lo, int32_t nl) {
  if (lo < 0 || nl < 1 || lo > e - nl) return MOE_ERR_SHAPE;
  return MOE_OK;
}

hipError_t run_w13(const void *x, moe_dtype_t dtype, int64_t n, int32_t hidden, const void *w13,
                   int32_t e, int32_t inter, int32_t k, moe_act_t act, moe_w13_layout_t layout,
                   const ActParams &prm, const moe_routing_t *r, void *a, hipStream_t s,
                   const void *w13_scale = nullptr) {
  return moe::launch_gemm1(x, w13, a, r->offsets, r->col_sorted, dtype, n, k, e, hidden, inter,
                           act, layout, prm, s, false,
                           reinterpret_cast<const uint8_t *>(w13_scale));
}

hipError_t run_w2(const void *a, moe_dtype_t dtype, int64_t n, int32_t hidden, const void *w2,
                  int32_t e, int32_t inter, int32_t k, const moe_routing_t *r, void *out, void *y,
                  hipStream_t s, bool share = false, bool unit_gate = false,
                  const void *w2_scale = nullptr) {
  const bool direct = k == 1;  // one row per token: GEMM2 writes the output rows itself
  if (!direct && moe::gemm2_combine_fits(dtype, n, k, e, hidden, inter, w2_scale != nullptr))
    return moe::launch_gemm2_combine(a, w2, out, r->offsets, r->row_sorted,
                                     unit_gate ? nullptr : r->gate_scal, (moe_dtype_t)r->w_dtype,
                                     n, k, e, hidden, inter, s,
                                     reinterpret_cast<const uint8_t *>(w2_scale));
  hipError_t err = moe::launch_gemm2(a, w2, direct ? out : y, r->offsets, r->col_sorted,
                                     unit_gate ? nullptr : r->gate_scal,
                                     (moe_dtype_t)r->w_dtype, dtype, n, k, e, hidden, inter,
                                     direct, s, reinterpret_cast<const uint8_t *>(w2_scale));
  if (err != hipSuccess) return err;
  // an expert share leaves the rows of tokens routed elsewhere to be zeroed
  if (direct) return share ? moe::launch_zero_unrouted(r->row_sorted, out, dtype, n, hidden, s)
                           : err;
  return moe::launch_combine(y, r->row_sorted, out, dtype, n, k, hidden, s);
}

moe_status_t run_experts(const void *x, moe_dtype_t dtype, int64_t n, int32_t hidden,
                         const void *w13, const void *w2, int32_t e, int32_t inter, int32_t k,
                         moe_act_t act, moe_w13_layout_t layout, const ActParams &prm,
                         const moe_routing_t *r, void *out, void *ws, hipStream_t s,
                         bool share = false, const void *w13_scale = nullptr,
                         const void *w2_scale = nullptr) {
  // workspace: activation rows a[M, inter], then (topk > 1) weighted rows y[M, hidden]
  char *base = reinterpret_cast<char *>(ws);
  void *a = base;
  void *y = base + align256((size_t)n * k * inter * dsize(dtype));
  if (run_w13(x, dtype, n, hidden, w13, e, inter, k, act, layout, prm, r, a, s, w13_scale) !=
      hipSuccess)
    return MOE_ERR_HIP;
  if (run_w2(a, dtype, n, hidden, w2, e, inter, k, r, out, y, s, share, false, w2_scale) !=
      hipSuccess)
    return MOE_ERR_HIP;
  return MOE_OK;
}

// Scratch of moe_forward_noalloc, for callers that cannot allocate device
// memory: a file-scope device array of MOE_NOALLOC_SCRATCH_BYTES.  Every GPU
// the library runs on holds its own copy, at its own address, until the
// process ends.  In host code the array's name is only a stand-in, never a
// device address: kernels receive the address hipGetSymbolAddress returns for
// the device, resolved once per device with that device current.
constexpr int kMaxDevices = 64;
struct ScratchSlot {
  std::once_flag once;
  void *ptr = nullptr;
  hipError_t err = hipSuccess;
};
ScratchSlot g_scratch[kMaxDevices];

}  // namespace

static __device__ __align__(256) char scratch[MOE_NOALLOC_SCRATCH_BYTES];

namespace {

// Device address of `scratch` on the device that runs stream s (the current
// device for the null stream).  The first call on a device makes that device
// current for the lookup and restores the caller's device.
hipError_t noalloc_scratch(hipStream_t s, void **out) {
  int cur = 0;
  hipError_t e = hipGetDevice(&cur);
  if (e != hipSuccess) return e;
  int dev = cur;
  if (s != nullptr) {
    hipDevice_t d = 0;
    if ((e = hipStreamGetDevice(s, &d)) != hipSuccess) return e;
    dev = (int)d;
  }
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  ScratchSlot &slot = g_scratch[dev];
  std::call_once(slot.once, [&] {
    if (dev != cur && (slot.err = hipSetDevice(dev)) != hipSuccess) return;
    slot.err = hipGetSymbolAddress(&slot.ptr, HIP_SYMBOL(scratch));
    if (dev != cur) {
      const hipError_t back = hipSetDevice(cur);
      if (slot.err == hipSuccess) slot.err = back;
    }
  });
  if (slot.err != hipSuccess) return slot.err;
  *out = slot.ptr;
  return hipSuccess;
}

}  // namespace

extern "C" {

size_t moe_workspace_bytes(int64_t n_tokens, int32_t n_experts, int32_t topk, int32_t hidden,
                           int32_t inter, moe_dtype_t dtype) {
  if (check_sizes(n_tokens, n_experts, topk) != MOE_OK || !dtype_ok(dtype)) return 0;
  if (inter != 0 && check_ffn_sizes(hidden, inter) != MOE_OK) return 0;
  if (inter == 0 && hidden != 0 && check_ffn_sizes(hidden, 8) != MOE_OK) return 0;
  // routing scratch, plus the router GEMM's when hidden is given; the expert
  // intermediates reuse the same bytes once the routing has run
  const size_t route = moe::route_scratch_bytes(n_tokens, n_experts, topk) +
                       (hidden ? moe::gate_scratch_bytes(n_tokens, n_experts, hidden, dtype) : 0);
  size_t ffn = 0;
  if (inter != 0) ffn = experts_ws_bytes(n_tokens, topk, hidden, inter, dtype);
  const size_t b = route > ffn ? route : ffn;
  return b ? b : 256;
}

moe_status_t moe_route(const void *logits, moe_dtype_t logits_dtype, int64_t n_tokens,
                       int32_t n_experts, int32_t topk, const moe_routing_t *out,
                       void *workspace, size_t ws_bytes, void *stream) {
  moe_status_t st =
      check_route(logits, logits_dtype, n_tokens, n_experts, topk, out, workspace, ws_bytes);
  if (st != MOE_OK || n_tokens == 0) return st;
  if (moe::launch_route(logits, logits_dtype, n_tokens, n_experts, topk, 0, n_experts, out,
                        workspace, (hipStream_t)stream) != hipSuccess)
    return MOE_ERR_HIP;
  return MOE_OK;
}

moe_status_t moe_experts(const void *x, moe_dtype_t dtype, int64_t n_tokens, int32_t hidden,
                         const void *w13, const void *w2, int32_t n_experts, int32_t inter,
                         int32_t topk, moe_act_t act, moe_w13_layout_t layout,
                         const moe_act_params_t *params, const moe_routing_t *routing, void *out,
                         void *workspace, size_t ws_bytes, void *stream) {
  ActParams prm;
  moe_status_t st = check_experts(x, dtype, n_tokens, hidden, w13, w2, n_experts, inter, topk,
                                  act, layout, params, routing, out, workspace, ws_bytes, &prm);
  if (st != MOE_OK || n_tokens == 0) return st;
  return run_experts(x, dtype, n_tokens, hidden, w13, w2, n_experts, inter, topk, act, layout,
                     prm, routing, out, workspace, (hipStream_t)stream);
}

moe_status_t moe_experts_w13(const void *x, moe_dtype_t dtype, int64_t n_tokens, int32_t hidden,
                             const void *w13, int32_t n_experts, int32_t inter, int32_t topk,
                             moe_act_t act, moe_w13_layout_t layout,
                             const moe_act_params_t *params, const moe_routing_t *routing,
                             void *act_out, void *stream) {
  ActParams prm;
  moe_status_t st = check_expert_args(dtype, n_tokens, hidden, n_experts, inter, topk, act,
                                      layout, params, routing, &prm);
  if (st != MOE_OK || n_tokens == 0) return st;
  if ((st = check_ptrs({x, w13, act_out})) != MOE_OK) return st;
  return run_w13(x, dtype, n_tokens, hidden, w13, n_experts, inter, topk, act, layout, prm,
                 routing, act_out, (hipStream_t)stream) == hipSuccess
             ? MOE_OK
             : MOE_ERR_HIP;
}

moe_status_t moe_experts_w2(const void *act_in, moe_dtype_t dtype, int64_t n_tokens,
                            int32_t hidden, const void *w2, int32_t n_experts, int32_t inter,
                            int32_t topk, const moe_routing_t *routing, void *out,
                            void *workspace, size_t ws_bytes, void *stream) {
  ActParams prm;
  moe_status_t st = check_expert_args(dtype, n_tokens, hidden, n_experts, inter, topk,
                                      MOE_ACT_SILU, MOE_W13_PACKED, nullptr, routing, &prm);
  if (st != MOE_OK || n_tokens == 0) return st;
  if ((st = check_ptrs({act_in, w2, out})) != MOE_OK) return st;
  if ((st = check_ws(workspace, ws_bytes, y_bytes(n_tokens, topk, hidden, dtype))) != MOE_OK)
    return st;
  return run_w2(act_in, dtype, n_tokens, hidden, w2, n_experts, inter, topk, routing, out,
                workspace, (hipStream_t)stream) == hipSuccess
             ? MOE_OK
             : MOE_ERR_HIP;
}

moe_status_t moe_experts_w2_rows(const void *act_in, moe_dtype_t dtype, int64_t n_tokens,
                                 int32_t hidden, const void *w2, int32_t n_experts, int32_t inter,
                                 int32_t topk, const moe_routing_t *routing, void *y_sorted,
                                 void *stream) {
  ActParams prm;
  moe_status_t st = check_expert_args(dtype, n_tokens, hidden, n_experts, inter, topk,
                                      MOE_ACT_SILU, MOE_W13_PACKED, nullptr, routing, &prm, true);
  if (st != MOE_OK || n_tokens == 0) return st;
  if ((st = check_ptrs({act_in, w2, y_sorted})) != MOE_OK) return st;
  return moe::launch_gemm2(act_in, w2, y_sorted, routing->offsets, routing->col_sorted,
                           routing->gate_scal, (moe_dtype_t)routing->w_dtype, dtype, n_tokens,
                           topk, n_experts, hidden, inter, false, (hipStream_t)stream) ==
                 hipSuccess
             ? MOE_OK
             : MOE_ERR_HIP;
}

moe_status_t moe_combine(const void *y_sorted, moe_dtype_t dtype, int64_t n_tokens,
                         int32_t hidden, int32_t topk, const moe_routing_t *routing, void *out,
                         void *stream) {
  moe_status_t st = check_sizes(n_tokens, kCombineAnyExperts, topk, false);
  if (st != MOE_OK) return st;
  if (check_ffn_sizes(hidden, 8) != MOE_OK) return MOE_ERR_SHAPE;
  if (!dtype_ok(dtype)) return MOE_ERR_DTYPE;
  // one thread per 16-byte chunk of out: the grid must stay below 2^31 workgroups of 256
  if (n_tokens * hidden * (int64_t)dsize(dtype) / 16 > 0x7fffffffLL * 256) return MOE_ERR_SHAPE;
  if (!routing) return MOE_ERR_NULL;
  if (n_tokens == 0) return MOE_OK;
  if ((st = check_ptrs({y_sorted, routing->row_sorted, out})) != MOE_OK) return st;
  return moe::launch_combine(y_sorted, routing->row_sorted, out, dtype, n_tokens, topk, hidden,
                             (hipStream_t)stream) == hipSuccess
             ? MOE_OK
             : MOE_ERR_HIP;
}

moe_status_t moe_forward(const void *x, const void *logits, moe_dtype_t dtype, int64_t n_tokens,
                         int32_t hidden, const void *w13, const void *w2, int32_t n_experts,
                         int32_t inter, int32_t topk, moe_act_t act, moe_w13_layout_t layout,
                         const moe_act_params_t *params, const moe_routing_t *routing_out,
                         void *out, void *workspace, size_t ws_bytes, void *stream) {
  ActParams prm;
  moe_status_t st = check_route(logits, dtype, n_tokens, n_experts, topk, routing_out, workspace,
                                ws_bytes);
  if (st != MOE_OK) return st;
  st = check_experts(x, dtype, n_tokens, hidden, w13, w2, n_experts, inter, topk, act, layout,
                     params, routing_out, out, workspace, ws_bytes, &prm);
  if (st != MOE_OK || n_tokens == 0) return st;
  hipStream_t s = (hipStream_t)stream;
  // the routing scratch is dead once the routing kernels ran (stream order), so
  // the expert intermediates reuse the same workspace bytes
  if (moe::launch_route(logits, dtype, n_tokens, n_experts, topk, 0, n_experts, routing_out,
                        workspace, s) != hipSuccess)
    return MOE_ERR_HIP;
  return run_experts(x, dtype, n_tokens, hidden, w13, w2, n_experts, inter, topk, act, layout,
                     prm, routing_out, out, workspace, s);
}

moe_status_t moe_forward_noalloc(const void *x, const void *logits, moe_dtype_t dtype,
                                 int64_t n_tokens, int32_t hidden, const void *w13,
                                 const void *w2, int32_t n_experts, int32_t inter, int32_t topk,
                                 moe_act_t act, moe_w13_layout_t layout,
                                 const moe_act_params_t *params, const moe_routing_t *routing_out,
                                 void *out, void *stream) {
  // the sizes must fit the static scratch; checked before anything else
  const size_t need = moe_workspace_bytes(n_tokens, n_experts, topk, hidden, inter, dtype);
  if (need == 0) return check_sizes(n_tokens, n_experts, topk) != MOE_OK ? MOE_ERR_SHAPE
                        : !dtype_ok(dtype)                            ? MOE_ERR_DTYPE
                                                                      : MOE_ERR_SHAPE;
  if (need > (size_t)MOE_NOALLOC_SCRATCH_BYTES) return MOE_ERR_SCRATCH;
  // every check of moe_forward, with a stand-in for the workspace (never
  // dereferenced by the checks) of the scratch's size
  void *const ws_stand_in = reinterpret_cast<void *>((uintptr_t)256);
  ActParams prm;
  moe_status_t st = check_route(logits, dtype, n_tokens, n_experts, topk, routing_out,
                                ws_stand_in, MOE_NOALLOC_SCRATCH_BYTES);
  if (st != MOE_OK) return st;
  st = check_experts(x, dtype, n_tokens, hidden, w13, w2, n_experts, inter, topk, act, layout,
                     params, routing_out, out, ws_stand_in, MOE_NOALLOC_SCRATCH_BYTES, &prm);
  if (st != MOE_OK || n_tokens == 0) return st;
  hipStream_t s = (hipStream_t)stream;
  void *ws = nullptr;
  if (noalloc_scratch(s, &ws) != hipSuccess) return MOE_ERR_HIP;
  // the same launches as moe_forward, into this GPU's copy of the scratch
  if (moe::launch_route(logits, dtype, n_tokens, n_experts, topk, 0, n_experts, routing_out, ws,
                        s) != hipSuccess)
    return MOE_ERR_HIP;
  return run_experts(x, dtype, n_tokens, hidden, w13, w2, n_experts, inter, topk, act, layout,
                     prm, routing_out, out, ws, s);
}

moe_status_t moe_route_ep(const void *logits, moe_dtype_t logits_dtype, int64_t n_tokens,
                          int32_t n_experts, int32_t topk, int32_t local_offset, int32_t n_local,
                          const moe_routing_t *out, void *workspace, size_t ws_bytes,
                          void *stream) {
  moe_status_t st = check_share(n_experts, local_offset, n_local);
  if (st != MOE_OK) return st;
  st = check_route(logits, logits_dtype, n_tokens, n_experts, topk, out, workspace, ws_bytes);
  if (st != MOE_OK || n_tokens == 0) return st;
  if (moe::launch_route(logits, logits_dtype, n_tokens, n_experts, topk, local_offset, n_local,
                        out, workspace, (hipStream_t)stream) != hipSuccess)
    return MOE_ERR_HIP;
  return MOE_OK;
}

moe_status_t moe_experts_ep(const void *x, moe_dtype_t dtype, int64_t n_tokens, int32_t hidden,
                            const void *w13, const void *w2, int32_t n_local, int32_t inter,
                            int32_t topk, moe_act_t act, moe_w13_layout_t layout,
                            const moe_act_params_t *params, const moe_routing_t *routing,
                            void *out, void *workspace, size_t ws_bytes, void *stream) {
  ActParams prm;
  moe_status_t st = check_experts(x, dtype, n_tokens, hidden, w13, w2, n_local, inter, topk, act,
                                  layout, params, routing, out, workspace, ws_bytes, &prm, true);
  if (st != MOE_OK || n_tokens == 0) return st;
  return run_experts(x, dtype, n_tokens, hidden, w13, w2, n_local, inter, topk, act, layout, prm,
                     routing, out, workspace, (hipStream_t)stream, true);
}

moe_status_t moe_forward_ep(const void *x, const void *logits, moe_dtype_t dtype,
                            int64_t n_tokens, int32_t hidden, const void *w13, const void *w2,
                            int32_t n_experts, int32_t local_offset, int32_t n_local,
                            int32_t inter, int32_t topk, moe_act_t act, moe_w13_layout_t layout,
                            const moe_act_params_t *params, const moe_routing_t *routing_out,
                            void *out, void *workspace, size_t ws_bytes, void *stream) {
  ActParams prm;
  moe_status_t st = check_share(n_experts, local_offset, n_local);
  if (st != MOE_OK) return st;
  st = check_route(logits, dtype, n_tokens, n_experts, topk, routing_out, workspace, ws_bytes);
  if (st != MOE_OK) return st;
  st = check_experts(x, dtype, n_tokens, hidden, w13, w2, n_local, inter, topk, act, layout,
                     params, routing_out, out, workspace, ws_bytes, &prm, true);
  if (st != MOE_OK || n_tokens == 0) return st;
  hipStream_t s = (hipStream_t)stream;
  if (moe::launch_route(logits, dtype, n_tokens, n_experts, topk, local_offset, n_local,
                        routing_out, workspace, s) != hipSuccess)
    return MOE_ERR_HIP;
  return run_experts(x, dtype, n_tokens, hidden, w13, w2, n_local, inter, topk, act, layout, prm,
                     routing_out, out, workspace, s, true);
}

moe_status_t moe_gate_route(const void *x, const void *w_gate, moe_dtype_t dtype,
                            int64_t n_tokens, int32_t hidden, int32_t n_experts, int32_t topk,
                            void *logits_out, const moe_routing_t *out, void *workspace,
                            size_t ws_bytes, void *stream) {
  moe_status_t st = check_gate(x, w_gate, dtype, n_tokens, hidden, n_experts, logits_out);
  if (st != MOE_OK) return st;
  st = check_route(logits_out, dtype, n_tokens, n_experts, topk, out, workspace, ws_bytes);
  if (st != MOE_OK || n_tokens == 0) return st;
  if (ws_bytes < moe::route_scratch_bytes(n_tokens, n_experts, topk) +
                     moe::gate_scratch_bytes(n_tokens, n_experts, hidden, dtype))
    return MOE_ERR_WORKSPACE;
  if (moe::launch_route(logits_out, dtype, n_tokens, n_experts, topk, 0, n_experts, out,
                        workspace, (hipStream_t)stream, x, w_gate, hidden) != hipSuccess)
    return MOE_ERR_HIP;
  return MOE_OK;
}

moe_status_t moe_gate_forward(const void *x, const void *w_gate, moe_dtype_t dtype,
                              int64_t n_tokens, int32_t hidden, const void *w13, const void *w2,
                              int32_t n_experts, int32_t inter, int32_t topk, moe_act_t act,
                              moe_w13_layout_t layout, const moe_act_params_t *params,
                              void *logits_out, const moe_routing_t *routing_out, void *out,
                              void *workspace, size_t ws_bytes, void *stream) {
  ActParams prm;
  moe_status_t st = check_gate(x, w_gate, dtype, n_tokens, hidden, n_experts, logits_out);
  if (st != MOE_OK) return st;
  st = check_route(logits_out, dtype, n_tokens, n_experts, topk, routing_out, workspace,
                   ws_bytes);
  if (st != MOE_OK) return st;
  st = check_experts(x, dtype, n_tokens, hidden, w13, w2, n_experts, inter, topk, act, layout,
                     params, routing_out, out, workspace, ws_bytes, &prm);
  if (st != MOE_OK || n_tokens == 0) return st;
  if (ws_bytes < moe::route_scratch_bytes(n_tokens, n_experts, topk) +
                     moe::gate_scratch_bytes(n_tokens, n_experts, hidden, dtype))
    return MOE_ERR_WORKSPACE;
  hipStream_t s = (hipStream_t)stream;
  if (moe::launch_route(logits_out, dtype, n_tokens, n_experts, topk, 0, n_experts, routing_out,
                        workspace, s, x, w_gate, hidden) != hipSuccess)
    return MOE_ERR_HIP;
  return run_experts(x, dtype, n_tokens, hidden, w13, w2, n_experts, inter, topk, act, layout,
                     prm, routing_out, out, workspace, s);
}

moe_status_t moe_experts_weighted_input(const void *x, moe_dtype_t dtype, int64_t n_tokens,
                                        int32_t hidden, const void *w13, const void *w2,
                                        int32_t n_experts, int32_t inter, int32_t topk,
                                        moe_act_t act, moe_w13_layout_t layout,
                                        const moe_act_params_t *params,
                                        const moe_routing_t *routing, void *out, void *workspace,
                                        size_t ws_bytes, void *stream) {
  ActParams prm;
  moe_status_t st = check_expert_args(dtype, n_tokens, hidden, n_experts, inter, topk, act,
                                      layout, params, routing, &prm);
  if (st != MOE_OK || n_tokens == 0) return st;
  if ((st = check_ptrs({x, w13, w2, out})) != MOE_OK) return st;
  const size_t base = experts_ws_bytes(n_tokens, topk, hidden, inter, dtype);
  const size_t xs_bytes = align256((size_t)n_tokens * topk * hidden * dsize(dtype));
  if ((st = check_ws(workspace, ws_bytes, base + xs_bytes)) != MOE_OK) return st;
  // workspace: a[M, inter], (topk > 1) y[M, hidden], then the scaled rows xs[M, hidden]
  hipStream_t s = (hipStream_t)stream;
  char *ws = reinterpret_cast<char *>(workspace);
  void *a = ws;
  void *y = ws + align256((size_t)n_tokens * topk * inter * dsize(dtype));
  void *xs = ws + base;
  if (moe::launch_scale_gather(x, routing->col_sorted, routing->gate_scal,
                               (moe_dtype_t)routing->w_dtype, routing->offsets, n_experts, dtype,
                               n_tokens, topk, hidden, xs, s) != hipSuccess ||
      moe::launch_gemm1(xs, w13, a, routing->offsets, routing->col_sorted, dtype, n_tokens, topk,
                        n_experts, hidden, inter, act, layout, prm, s, true) != hipSuccess ||
      run_w2(a, dtype, n_tokens, hidden, w2, n_experts, inter, topk, routing, out, y, s, false,
             true) != hipSuccess)
    return MOE_ERR_HIP;
  return MOE_OK;
}

moe_status_t moe_quantize_mxfp4(const void *w, moe_dtype_t dtype, int32_t n_experts,
                                int32_t rows, int32_t k, void *q, void *scales, void *stream) {
  if (!dtype_ok(dtype)) return MOE_ERR_DTYPE;
  if (n_experts < 1 || rows < 1 || k < 32 || k % 32 || k > (1 << 24)) return MOE_ERR_SHAPE;
  if ((int64_t)n_experts * rows * k * (int64_t)dsize(dtype) > 0x7fffffffLL * 8)
    return MOE_ERR_SHAPE;
  moe_status_t st = check_ptrs({w, q});
  if (st != MOE_OK) return st;
  if (!scales) return MOE_ERR_NULL;
  return moe::launch_quantize_mxfp4(w, dtype, n_experts, rows, k, q, scales,
                                    (hipStream_t)stream) == hipSuccess
             ? MOE_OK
             : MOE_ERR_HIP;
}

namespace {
// MXFP4 weights: bf16 layer, K of both GEMMs (hidden, inter) a multiple of 32,
// codes and scales present and 16-byte aligned.
moe_status_t check_mxfp4(moe_dtype_t dtype, int32_t hidden, int32_t inter, const void *w13_s,
                         const void *w2_s) {
  if (dtype != MOE_BF16) return MOE_ERR_UNSUPPORTED;
  if (hidden % 32 || inter % 32) return MOE_ERR_SHAPE;
  return check_ptrs({w13_s, w2_s});
}
}  // namespace

moe_status_t moe_experts_mxfp4(const void *x, moe_dtype_t dtype, int64_t n_tokens,
                               int32_t hidden, const void *w13_q, const void *w13_s,
                               const void *w2_q, const void *w2_s, int32_t n_experts,
                               int32_t inter, int32_t topk, moe_act_t act,
                               moe_w13_layout_t layout, const moe_act_params_t *params,
                               const moe_routing_t *routing, void *out, void *workspace,
                               size_t ws_bytes, void *stream) {
  ActParams prm;
  moe_status_t st = check_experts(x, dtype, n_tokens, hidden, w13_q, w2_q, n_experts, inter,
                                  topk, act, layout, params, routing, out, workspace, ws_bytes,
                                  &prm);
  if (st != MOE_OK) return st;
  if ((st = check_mxfp4(dtype, hidden, inter, w13_s, w2_s)) != MOE_OK || n_tokens == 0)
    return st;
  return run_experts(x, dtype, n_tokens, hidden, w13_q, w2_q, n_experts, inter, topk, act, layout,
                     prm, routing, out, workspace, (hipStream_t)stream, false, w13_s, w2_s);
}

moe_status_t moe_forward_mxfp4(const void *x, const void *logits, moe_dtype_t dtype,
                               int64_t n_tokens, int32_t hidden, const void *w13_q,
                               const void *w13_s, const void *w2_q, const void *w2_s,
                               int32_t n_experts, int32_t inter, int32_t topk, moe_act_t act,
                               moe_w13_layout_t layout, const moe_act_params_t *params,
                               const moe_routing_t *routing_out, void *out, void *workspace,
                               size_t ws_bytes, void *stream) {
  ActParams prm;
  moe_status_t st = check_route(logits, dtype, n_tokens, n_experts, topk, routing_out, workspace,
                                ws_bytes);
  if (st != MOE_OK) return st;
  st = check_experts(x, dtype, n_tokens, hidden, w13_q, w2_q, n_experts, inter, topk, act,
                     layout, params, routing_out, out, workspace, ws_bytes, &prm);
  if (st != MOE_OK) return st;
  if ((st = check_mxfp4(dtype, hidden, inter, w13_s, w2_s)) != MOE_OK || n_tokens == 0)
    return st;
  hipStream_t s = (hipStream_t)stream;
  if (moe::launch_route(logits, dtype, n_tokens, n_experts, topk, 0, n_experts, routing_out,
                        workspace, s) != hipSuccess)
    return MOE_ERR_HIP;
  return run_experts(x, dtype, n_tokens, hidden, w13_q, w2_q, n_experts, inter, topk, act, layout,
                     prm, routing_out, out, workspace, s, false, w13_s, w2_s);
}

const char *moe_status_str(moe_status_t status) {
  switch (status) {
    case MOE_OK: return "ok";
    case MOE_ERR_NULL: return "required pointer is NULL";
    case MOE_ERR_SHAPE: return "size out of range or inconsistent";
    case MOE_ERR_DTYPE: return "unknown or mismatched dtype";
    case MOE_ERR_UNSUPPORTED: return "unsupported activation/layout combination";
    case MOE_ERR_ALIGN: return "pointer not 16-byte aligned";
    case MOE_ERR_WORKSPACE: return "workspace missing or too small";
    case MOE_ERR_HIP: return "HIP launch failed";
    case MOE_ERR_SCRATCH:
      return "sizes need more than the library's static scratch (MOE_NOALLOC_SCRATCH_BYTES)";
  }
  return "unknown status";
}

}  // extern "C"
