// Definitions shared by the grouped expert GEMM kernels (the MFMA tiles of
// grouped_gemm.hip and the decode-sized kernel of gemv.hip): launch arguments,
// epilogue kinds, the activation and the MXFP4 weight decode.  Internal to
// libmoe.so.
#pragma once

#include "moe_common.h"

namespace moe {

// Epilogue kinds: GEMM1 applies the activation (gated without or with the
// clamp, or ReLU^2); GEMM2 scales by the routing weight and writes the sorted
// row (EPI_Y) or, with one expert per token, the token's output row (EPI_OUT).
enum { EPI_GATED = 0, EPI_Y = 1, EPI_OUT = 2, EPI_GATED_CLAMP = 3, EPI_RELU2 = 4 };

struct GemmArgs {
  const void *A;                 // GEMM1: x [N, K]; GEMM2: a [M, K]
  const void *W;                 // [E, NSETS * Nout, K]
  void *C;                       // output rows
  const int32_t *offsets;        // [E + 1]
  const int32_t *col_sorted;     // [M]
  const void *gate_scal;         // [M] (GEMM2)
  uint32_t a_bytes;              // bytes of A (buffer range)
  uint32_t c_bytes;              // bytes of C
  int gate_bf16, E, K, Nout, topk, gather, interleaved, act;
  ActParams prm;
  // MXFP4 weights: W holds E2M1 codes [E, NSETS * Nout, K / 2] and wscale the
  // E8M0 scales [E, K / 32, NSETS * Nout] (nullptr: W is in the A dtype)
  const uint8_t *wscale;
  const int32_t *row_sorted;     // [N * topk] (w2 with the combine folded in)
};

// 8 E2M1 codes (element i in nibble i of `word`) times the scale `sc`, as the
// bf16 fragment of 8 consecutive K elements.  The hardware conversion takes
// byte b and yields its low nibble's value first.
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ bf16x8_t fp4x8_to_bf16(uint32_t word, float sc) {
  u32x4_t w;
  w[0] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(word, sc, 0));
  w[1] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(word, sc, 1));
  w[2] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(word, sc, 2));
  w[3] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(word, sc, 3));
  return __builtin_bit_cast(bf16x8_t, w);
}

// Activation of one (gate, up) pair.  Gated kinds evaluate the logistic
// function as 1 / (1 + 2^(nal * g)) with nal = -alpha * log2(e), using the
// hardware exp2 and reciprocal (about 1 ulp each); the clamp variant first
// limits the gate from above and the up value to [-limit, limit].
template <int EPI>
__device__ __forceinline__ float act_val(float g, float u, float nal, const ActParams &p) {
  if constexpr (EPI == EPI_RELU2) {
    const float r = fmaxf(g, 0.f);
    return r * r;
  } else {
    if constexpr (EPI == EPI_GATED_CLAMP) {
      g = fminf(g, p.limit);
      u = fminf(fmaxf(u, -p.limit), p.limit);
    }
    const float e = __builtin_amdgcn_exp2f(nal * g);
    return g * __builtin_amdgcn_rcpf(1.f + e) * (u + p.beta);
  }
}

// Decode-sized batches run the expert GEMMs as grouped matrix-vector
// products (gemv.hip): bf16 activations, at most kGemvMaxTokens tokens, and
// few rows per expert on average -- N * topk <= 3 E for w13 with bf16 weights
// (5 E for the plain w2), <= 1.5 E for w13 with MXFP4 weights, whose FP4
// decode is repeated for every row (3 E for their w2).  Above that the MFMA
// tiles are faster (measured on gpt-oss-sized layers, E = 32 and 128, up to
// 128 tokens: at 4-5 rows an expert the gated bf16 w13 is 3-6 % slower as
// matrix-vector products, the plain bf16 w2 6-19 % faster; the MXFP4 w2 gains
// up to 2-3 rows an expert and loses past 4).  True when that kernel takes a
// launch of this shape; plain: the w2 launch.
constexpr int kGemvMaxTokens = 128;
bool gemv_fits(moe_dtype_t dt, int64_t n_tokens, int topk, int n_experts, int K, int Nout,
               bool mxfp4, bool plain = false);
// nsets: weight sets per output column (2 gated, 1 plain); epi: the epilogue
// kind; M: rows of the launch (n_tokens * topk).
hipError_t launch_gemv(const GemmArgs &a, int nsets, int epi, int64_t n_tokens, int64_t M,
                       hipStream_t s);

}  // namespace moe
