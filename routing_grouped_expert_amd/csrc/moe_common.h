// Shared device helpers for the gfx950 MoE kernels (bf16 storage, vector types,
// launch-size constants).  Internal to libmoe.so.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "moe.h"

namespace moe {

typedef uint16_t bf16_t;  // bfloat16 storage
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));  // one 16-byte chunk

constexpr int kMaxExperts = 256;
constexpr int kMaxTopk = 16;

__device__ __forceinline__ float to_f32(bf16_t b) { return __uint_as_float((uint32_t)b << 16); }
__device__ __forceinline__ float to_f32(float f) { return f; }

// fp32 -> bf16, round to nearest, ties to even (NaN kept quiet).
__device__ __forceinline__ bf16_t bf16_rne(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return (bf16_t)((u >> 16) | 0x40u);
  u += 0x7fffu + ((u >> 16) & 1u);
  return (bf16_t)(u >> 16);
}

template <typename T> __device__ __forceinline__ T from_f32(float f);
template <> __device__ __forceinline__ float from_f32<float>(float f) { return f; }
template <> __device__ __forceinline__ bf16_t from_f32<bf16_t>(float f) { return bf16_rne(f); }

__device__ __forceinline__ int popc64(unsigned long long x) { return __popcll(x); }

// Inclusive prefix sum over the 64 lanes of a wave, all in DPP (no LDS round
// trips): shifts by 1, 2, 4 and 8 inside each 16-lane row (lanes shifted in
// from outside the row add 0), then the last lane of rows 0 and 2 is added to
// rows 1 and 3 (row_bcast:15) and the last lane of row 1 to rows 2 and 3
// (row_bcast:31).  Needs every lane of the wave active.
__device__ __forceinline__ int wave_inclusive_sum(int v) {
  v += __builtin_amdgcn_update_dpp(0, v, 0x111, 0xf, 0xf, false);  // row_shr:1
  v += __builtin_amdgcn_update_dpp(0, v, 0x112, 0xf, 0xf, false);  // row_shr:2
  v += __builtin_amdgcn_update_dpp(0, v, 0x114, 0xf, 0xf, false);  // row_shr:4
  v += __builtin_amdgcn_update_dpp(0, v, 0x118, 0xf, 0xf, false);  // row_shr:8
  v += __builtin_amdgcn_update_dpp(0, v, 0x142, 0xa, 0xf, false);  // row_bcast:15
  v += __builtin_amdgcn_update_dpp(0, v, 0x143, 0xc, 0xf, false);  // row_bcast:31
  return v;
}

}  // namespace moe

// Host-side launchers (one per kernel family).  Each returns hipSuccess or the
// launch error; argument checking happens in moe_api.hip before these run.
namespace moe {
constexpr int kRouteThreads = 256;
constexpr int kRouteTokens = 256;  // tokens per routing block (one per thread in the rank phase)

size_t route_scratch_bytes(int64_t n_tokens, int n_experts, int topk);
// Scratch the router GEMM of moe_gate_route needs besides route_scratch_bytes
// (the split-K partial sums of batches up to 4096 tokens; the two are never
// live together).
size_t gate_scratch_bytes(int64_t n_tokens, int n_experts, int hidden, moe_dtype_t dt);
// Routing for the expert share [local_offset, local_offset + n_local) of the
// n_experts (0 and n_experts for the whole layer).  With x != nullptr the
// logits [N, E] are first computed as x [N, hidden] . w_gate [E, hidden]^T and
// written to `logits` (router GEMM).
hipError_t launch_route(const void *logits, moe_dtype_t dt, int64_t n_tokens, int n_experts,
                        int topk, int local_offset, int n_local, const moe_routing_t *r,
                        void *scratch, hipStream_t s, const void *x = nullptr,
                        const void *w_gate = nullptr, int hidden = 0);

struct ActParams {
  float alpha, beta, limit;
};

// GEMM1: a[M, inter] = act(xs[M, hidden] . W13[e]^T) for every expert segment.
// With w13_scale (bf16 only) W13 holds MXFP4 codes [E, rows, hidden / 2] and
// w13_scale the scales [E, hidden / 32, rows]; GEMM2 likewise with w2_scale.
hipError_t launch_gemm1(const void *x, const void *w13, void *act_out, const int32_t *offsets,
                        const int32_t *col_sorted, moe_dtype_t dt, int64_t n_tokens, int topk,
                        int n_experts, int hidden, int inter, moe_act_t act,
                        moe_w13_layout_t layout, ActParams p, hipStream_t s,
                        bool sorted_rows = false, const uint8_t *w13_scale = nullptr);
// GEMM2: y = gate_scal[p] * (a[p] . W2[e]^T) (gate_scal NULL: weight 1); stored
// to y_sorted[M, hidden], or (topk == 1) straight to out[token(p)].
hipError_t launch_gemm2(const void *act_in, const void *w2, void *y, const int32_t *offsets,
                        const int32_t *col_sorted, const void *gate_scal, moe_dtype_t gate_dt,
                        moe_dtype_t dt, int64_t n_tokens, int topk, int n_experts, int hidden,
                        int inter, bool direct_out, hipStream_t s,
                        const uint8_t *w2_scale = nullptr);
// Decode-sized layers with topk > 1 and about one row per expert: GEMM2 and
// the combine in one kernel (true when launch_gemm2_combine takes the shape).
bool gemm2_combine_fits(moe_dtype_t dt, int64_t n_tokens, int topk, int n_experts, int hidden,
                        int inter, bool mxfp4);
// out[t] = RNE(sum_j RNE(gate_scal[p] * (a[p] . W2[e(p)]^T))), p = row_sorted[t*topk + j]
// in slot order (slots with p = -1 skipped): the same bits as launch_gemm2 into
// y_sorted followed by launch_combine.
hipError_t launch_gemm2_combine(const void *act_in, const void *w2, void *out,
                                const int32_t *offsets, const int32_t *row_sorted,
                                const void *gate_scal, moe_dtype_t gate_dt, int64_t n_tokens,
                                int topk, int n_experts, int hidden, int inter, hipStream_t s,
                                const uint8_t *w2_scale = nullptr);
// out[t] = sum_j y_sorted[row_sorted[t*topk + j]] (fp32, slot order), slots
// with row_sorted = -1 skipped.
hipError_t launch_combine(const void *y_sorted, const int32_t *row_sorted, void *out,
                          moe_dtype_t dt, int64_t n_tokens, int topk, int hidden, hipStream_t s);
// xs[p] = RNE(gate_scal[p] * x[col_sorted[p] / topk]) for the routed rows
// p < offsets[n_experts]: the input rows of each entry, in sorted order and
// scaled by the entry's routing weight.
hipError_t launch_scale_gather(const void *x, const int32_t *col_sorted, const void *gate_scal,
                               moe_dtype_t gate_dt, const int32_t *offsets, int n_experts,
                               moe_dtype_t dt, int64_t n_tokens, int topk, int hidden, void *xs,
                               hipStream_t s);
// MXFP4: w [E, rows, k] -> codes q [E, rows, k/2], scales [E, k/32, rows].
hipError_t launch_quantize_mxfp4(const void *w, moe_dtype_t dt, int n_experts, int rows, int k,
                                 void *q, void *scales, hipStream_t s);
// topk == 1: out[t] = 0 where row_sorted[t] = -1.
hipError_t launch_zero_unrouted(const int32_t *row_sorted, void *out, moe_dtype_t dt,
                                int64_t n_tokens, int hidden, hipStream_t s);
}  // namespace moe
