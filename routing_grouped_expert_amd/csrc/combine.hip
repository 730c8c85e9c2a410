// Weighted scatter-combine: out[t] = sum over slots j of y_sorted[row_sorted[t*k + j]].
//
// The expert outputs were already scaled by their routing weights in GEMM2's
// epilogue; this kernel adds each token's k rows back together, the step the
// minimind issue #835 page does with index_add_ ("Summary").  That page notes
// index_add_ uses atomics on the GPU when k > 1; here each thread owns one
// 16-byte chunk of one output row and sums the k chunks in slot order in fp32,
// so the result is deterministic.  The loads are 16-byte vectors; each token
// row is read from k places and written once (HBM bound).  A slot with
// row_sorted = -1 (its expert is outside this GPU's expert-parallel share)
// adds nothing; a token with no slot in the share gets a zero row.
#include "moe_common.h"

#include <type_traits>

namespace moe {
namespace {

__device__ __forceinline__ void add_chunk(float (&acc)[8], u32x4_t v, bf16_t) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    acc[2 * i] += __uint_as_float(v[i] << 16);
    acc[2 * i + 1] += __uint_as_float(v[i] & 0xffff0000u);
  }
}
__device__ __forceinline__ void add_chunk(float (&acc)[4], u32x4_t v, float) {
#pragma unroll
  for (int i = 0; i < 4; ++i) acc[i] += __uint_as_float(v[i]);
}
__device__ __forceinline__ u32x4_t pack_chunk(const float (&acc)[8], bf16_t) {
  u32x4_t o;
#pragma unroll
  for (int i = 0; i < 4; ++i)
    o[i] = (uint32_t)bf16_rne(acc[2 * i]) | ((uint32_t)bf16_rne(acc[2 * i + 1]) << 16);
  return o;
}
__device__ __forceinline__ u32x4_t pack_chunk(const float (&acc)[4], float) {
  u32x4_t o;
#pragma unroll
  for (int i = 0; i < 4; ++i) o[i] = __float_as_uint(acc[i]);
  return o;
}

// KK: the number of slots when it is known at compile time (2, 4, 6, 8): all
// KK index loads and then all KK row loads go out back to back; 0: any k.
// The sum runs in slot order either way, so both give the same bits.  The
// expert rows are read once and the output written once, so both go
// non-temporal: on the skewed 64-expert layer (16384 tokens, k = 8, 1 GB of
// rows) 242 -> 219 us, fp32 k = 6 94 -> 81 us.
template <typename T, int KK>
__global__ __launch_bounds__(256) void combine_kernel(const T *__restrict__ y,
                                                      const int32_t *__restrict__ row_sorted,
                                                      T *__restrict__ out, int64_t N, int K,
                                                      int H) {
  constexpr int CH = 16 / sizeof(T);  // elements per 16-byte chunk
  const int nch = H / CH;
  const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= N * nch) return;
  const int64_t t = idx / nch;
  const int c = (int)(idx - t * nch);
  float acc[CH];
#pragma unroll
  for (int i = 0; i < CH; ++i) acc[i] = 0.f;
  if constexpr (KK > 0) {
    int32_t p[KK];
#pragma unroll
    for (int j = 0; j < KK; ++j) p[j] = row_sorted[t * KK + j];
    u32x4_t v[KK];
#pragma unroll
    for (int j = 0; j < KK; ++j)
      v[j] = p[j] >= 0 ? __builtin_nontemporal_load(reinterpret_cast<const u32x4_t *>(
                             y + (int64_t)p[j] * H + (int64_t)c * CH))
                       : u32x4_t{0u, 0u, 0u, 0u};
#pragma unroll
    for (int j = 0; j < KK; ++j)
      if (p[j] >= 0) add_chunk(acc, v[j], T());
  } else {
    for (int j = 0; j < K; ++j) {
      const int64_t p = row_sorted[t * K + j];
      if (p >= 0)
        add_chunk(acc, *reinterpret_cast<const u32x4_t *>(y + p * H + (int64_t)c * CH), T());
    }
  }
  __builtin_nontemporal_store(pack_chunk(acc, T()),
                              reinterpret_cast<u32x4_t *>(out + t * H + (int64_t)c * CH));
}

// Top-1 layer of an expert-parallel share: GEMM2 writes the rows of tokens
// whose expert is local; this kernel writes zero rows for the others
// (row_sorted = -1).  The two write disjoint rows, so their order is free.
__global__ __launch_bounds__(256) void zero_unrouted_kernel(const int32_t *__restrict__ row_sorted,
                                                            u32x4_t *__restrict__ out, int64_t N,
                                                            int nch) {
  const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= N * nch) return;
  const int64_t t = idx / nch;
  if (row_sorted[t] < 0) out[idx] = u32x4_t{0u, 0u, 0u, 0u};
}

}  // namespace

hipError_t launch_zero_unrouted(const int32_t *row_sorted, void *out, moe_dtype_t dt,
                                int64_t n_tokens, int hidden, hipStream_t s) {
  const int nch = hidden / (dt == MOE_BF16 ? 8 : 4);  // 16-byte chunks per row
  const int64_t total = n_tokens * nch;
  hipLaunchKernelGGL(zero_unrouted_kernel, dim3((unsigned)((total + 255) / 256)), dim3(256), 0, s,
                     row_sorted, reinterpret_cast<u32x4_t *>(out), n_tokens, nch);
  return hipGetLastError();
}

hipError_t launch_combine(const void *y_sorted, const int32_t *row_sorted, void *out,
                          moe_dtype_t dt, int64_t n_tokens, int topk, int hidden, hipStream_t s) {
  const int ch = dt == MOE_BF16 ? 8 : 4;
  const int64_t total = n_tokens * (hidden / ch);
  const unsigned blocks = (unsigned)((total + 255) / 256);
  auto go = [&](auto kk) {
    constexpr int KK = decltype(kk)::value;
    if (dt == MOE_BF16)
      hipLaunchKernelGGL((combine_kernel<bf16_t, KK>), dim3(blocks), dim3(256), 0, s,
                         reinterpret_cast<const bf16_t *>(y_sorted), row_sorted,
                         reinterpret_cast<bf16_t *>(out), n_tokens, topk, hidden);
    else
      hipLaunchKernelGGL((combine_kernel<float, KK>), dim3(blocks), dim3(256), 0, s,
                         reinterpret_cast<const float *>(y_sorted), row_sorted,
                         reinterpret_cast<float *>(out), n_tokens, topk, hidden);
  };
  switch (topk) {
    case 2: go(std::integral_constant<int, 2>()); break;
    case 4: go(std::integral_constant<int, 4>()); break;
    case 6: go(std::integral_constant<int, 6>()); break;
    case 8: go(std::integral_constant<int, 8>()); break;
    default: go(std::integral_constant<int, 0>()); break;
  }
  return hipGetLastError();
}

}  // namespace moe
