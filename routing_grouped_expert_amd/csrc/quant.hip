// MXFP4 quantisation of expert weights: FP4 E2M1 codes with one E8M0 scale per
// 32 consecutive weights along K.  The gpt-oss experts of the vLLM PR #45457
// report run with MXFP4 weights ("key source snippets", the MXFP4 experts
// forward); the pages name the format only, so the definition is the public
// OCP microscaling one: X = floor(log2 max|w|) - 2 per block (an all-zero
// block: -127), each weight w * 2^-X to the nearest E2M1 value (0, 0.5, 1,
// 1.5, 2, 3, 4, 6), ties to the code with an even lowest bit, saturating at 6,
// sign kept.  Codes pack two to a byte, the even element in the low nibble;
// scales are stored block-major per expert ([E][K/32][rows]) so that the rows
// of a GEMM tile find one K-block's scales side by side.
#include "moe_common.h"

namespace moe {
namespace {

// E2M1 code of a value already divided by the block scale: the thresholds are
// the midpoints between neighbouring values, a midpoint going to the even code.
__device__ __forceinline__ uint32_t e2m1_code(float v) {
  const float a = fabsf(v);
  const uint32_t c = a <= 0.25f ? 0u
                   : a < 0.75f  ? 1u
                   : a <= 1.25f ? 2u
                   : a < 1.75f  ? 3u
                   : a <= 2.5f  ? 4u
                   : a < 3.5f   ? 5u
                   : a <= 5.0f  ? 6u
                                : 7u;
  return c | (signbit(v) ? 8u : 0u);
}

// One thread per 32-weight block of one row.
template <typename T>
__global__ __launch_bounds__(256) void quantize_mxfp4_kernel(const T *__restrict__ w,
                                                             int64_t nrows, int rows, int K,
                                                             uint8_t *__restrict__ q,
                                                             uint8_t *__restrict__ s) {
  const int nb = K / 32;
  const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= nrows * nb) return;
  const int64_t rg = idx / nb;
  const int b = (int)(idx - rg * nb);
  constexpr int PER = 16 / (int)sizeof(T);  // elements per 16-byte load
  const u32x4_t *src = reinterpret_cast<const u32x4_t *>(w + rg * K + b * 32);
  float v[32];
#pragma unroll
  for (int c = 0; c < 32 / PER; ++c) {
    const u32x4_t x = src[c];
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      const uint32_t word = x[i * (int)sizeof(T) / 4];
      v[c * PER + i] = sizeof(T) == 2 ? __uint_as_float((i & 1) ? (word & 0xffff0000u) : (word << 16))
                                      : __uint_as_float(word);
    }
  }
  float amax = 0.f;
#pragma unroll
  for (int i = 0; i < 32; ++i) amax = fmaxf(amax, fabsf(v[i]));
  int x = amax > 0.f ? ilogbf(amax) - 2 : -127;
  x = x < -127 ? -127 : (x > 127 ? 127 : x);
  u32x4_t packed = {0u, 0u, 0u, 0u};
#pragma unroll
  for (int i = 0; i < 32; ++i) packed[i / 8] |= e2m1_code(ldexpf(v[i], -x)) << (4 * (i % 8));
  *reinterpret_cast<u32x4_t *>(q + rg * (K / 2) + b * 16) = packed;
  const int64_t e = rg / rows, r = rg - e * rows;
  s[(e * nb + b) * rows + r] = (uint8_t)(x + 127);
}

}  // namespace

hipError_t launch_quantize_mxfp4(const void *w, moe_dtype_t dt, int n_experts, int rows, int k,
                                 void *q, void *scales, hipStream_t s) {
  const int64_t nrows = (int64_t)n_experts * rows;
  const int64_t total = nrows * (k / 32);
  const dim3 grid((unsigned)((total + 255) / 256));
  uint8_t *qq = reinterpret_cast<uint8_t *>(q), *ss = reinterpret_cast<uint8_t *>(scales);
  if (dt == MOE_BF16)
    hipLaunchKernelGGL(quantize_mxfp4_kernel<bf16_t>, grid, dim3(256), 0, s,
                       reinterpret_cast<const bf16_t *>(w), nrows, rows, k, qq, ss);
  else
    hipLaunchKernelGGL(quantize_mxfp4_kernel<float>, grid, dim3(256), 0, s,
                       reinterpret_cast<const float *>(w), nrows, rows, k, qq, ss);
  return hipGetLastError();
}

}  // namespace moe
