// Routing weight applied to the input rows (the experts apply() flag
// apply_router_weight_on_input of the vLLM PR #47106 report, "key source
// snippets"): every routed entry p gets its own input row, the token's row
// scaled by the entry's weight and rounded once to the layer dtype, written in
// the expert-sorted order so GEMM1 reads it without the gather index.  One
// thread per 16-byte chunk; HBM bound (reads and writes M * hidden elements).
#include "moe_common.h"

namespace moe {
namespace {

template <typename T, typename G>
__global__ __launch_bounds__(256) void scale_gather_kernel(
    const T *__restrict__ x, const int32_t *__restrict__ col_sorted, const G *__restrict__ gate,
    const int32_t *__restrict__ offsets, int E, int64_t M, int K, int H, T *__restrict__ xs) {
  constexpr int CH = 16 / sizeof(T);  // elements per 16-byte chunk
  const int nch = H / CH;
  const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= M * nch) return;
  const int64_t p = idx / nch;
  if (p >= offsets[E]) return;  // past the routed entries (an expert share has fewer)
  const int c = (int)(idx - p * nch);
  const int64_t t = col_sorted[p] / K;
  const float g = to_f32(gate[p]);
  const u32x4_t v = *reinterpret_cast<const u32x4_t *>(x + t * H + (int64_t)c * CH);
  u32x4_t o;
  if constexpr (sizeof(T) == 2) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float lo = g * __uint_as_float(v[i] << 16), hi = g * __uint_as_float(v[i] & 0xffff0000u);
      o[i] = (uint32_t)bf16_rne(lo) | ((uint32_t)bf16_rne(hi) << 16);
    }
  } else {
#pragma unroll
    for (int i = 0; i < 4; ++i) o[i] = __float_as_uint(g * __uint_as_float(v[i]));
  }
  *reinterpret_cast<u32x4_t *>(xs + p * H + (int64_t)c * CH) = o;
}

template <typename T>
hipError_t launch_t(const void *x, const int32_t *col_sorted, const void *gate, bool gate_bf16,
                    const int32_t *offsets, int E, int64_t M, int K, int H, void *xs,
                    hipStream_t s) {
  const int64_t total = M * (H / (16 / (int)sizeof(T)));
  const dim3 grid((unsigned)((total + 255) / 256));
  const T *xt = reinterpret_cast<const T *>(x);
  T *o = reinterpret_cast<T *>(xs);
  if (gate_bf16)
    hipLaunchKernelGGL((scale_gather_kernel<T, bf16_t>), grid, dim3(256), 0, s, xt, col_sorted,
                       reinterpret_cast<const bf16_t *>(gate), offsets, E, M, K, H, o);
  else
    hipLaunchKernelGGL((scale_gather_kernel<T, float>), grid, dim3(256), 0, s, xt, col_sorted,
                       reinterpret_cast<const float *>(gate), offsets, E, M, K, H, o);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_scale_gather(const void *x, const int32_t *col_sorted, const void *gate_scal,
                               moe_dtype_t gate_dt, const int32_t *offsets, int n_experts,
                               moe_dtype_t dt, int64_t n_tokens, int topk, int hidden, void *xs,
                               hipStream_t s) {
  const int64_t M = n_tokens * topk;
  const bool gb = gate_dt == MOE_BF16;
  if (dt == MOE_BF16)
    return launch_t<bf16_t>(x, col_sorted, gate_scal, gb, offsets, n_experts, M, topk, hidden, xs,
                            s);
  return launch_t<float>(x, col_sorted, gate_scal, gb, offsets, n_experts, M, topk, hidden, xs, s);
}

}  // namespace moe
