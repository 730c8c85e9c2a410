// Grouped expert GEMMs over ragged expert segments, MFMA on gfx950.
//
// The expert FFN it runs -- w13 projection, gated (SiLU / SwiGLU-OAI) or
// non-gated (ReLU^2) activation, w2 projection, routing weight on the expert
// output -- is the one described by the minimind issue #835 page ("Summary":
// the weight multiplies each expert's output before it is added in) and the
// vLLM PR #47106 report (activation kinds, parameters, w13 layouts).
//
// Design (this file's own):
//  * One workgroup computes a BM x BN tile of one expert's output.  The m-tiles
//    of all experts are numbered expert by expert; a workgroup finds its expert
//    from the device-side offsets (a 64-lane scan of ceil(count / BM) per
//    expert and a binary search), so the host never learns the counts.  The
//    grid is an upper bound (floor(M/BM) + min(E, M) m-tiles); surplus
//    workgroups return at once.
//  * GEMM1 gathers its A rows straight from x: sorted row p reads token
//    col_sorted[p] / topk.  No gathered copy of x is ever written.
//  * Both operands are K-contiguous.  Tiles of 128-byte K-slices are staged
//    through LDS (double buffered, one barrier per K step) with the 16-byte
//    chunk index XOR-swizzled by the row, so the 16-byte fragment reads of a
//    32-row MFMA operand hit distinct banks.
//  * Gated GEMM1 tiles hold BN gate rows and the BN matching up rows of w13,
//    picked by layout (packed: rows n and inter+n; interleaved: 2n and 2n+1),
//    so gate and up of one output land in the same lane and register of two
//    accumulators and the activation runs in the epilogue from fp32.
//  * bf16 uses v_mfma_f32_32x32x16_bf16, fp32 uses v_mfma_f32_32x32x2_f32.
#include "moe_common.h"

namespace moe {
namespace {

constexpr int BM = 128;         // rows per tile
constexpr int BN = 128;         // output columns per tile
constexpr int kThreads = 256;   // 4 waves, 2 (rows) x 2 (columns), 64 x 64 each
constexpr int kRowBytes = 128;  // one K-slice row in LDS
constexpr int kChunks = kRowBytes / 16;

enum { EPI_ACT = 0, EPI_Y = 1, EPI_OUT = 2 };

template <typename T> struct Mma;
template <> struct Mma<bf16_t> {
  static constexpr int BK = 64;  // K elements per LDS slice
  static constexpr int KS = 16;  // K per instruction
  static constexpr int EPL = 8;  // K elements per lane fragment
  typedef bf16x8_t Frag;
  __device__ static Frag ld(const char *p) { return *reinterpret_cast<const bf16x8_t *>(p); }
  __device__ static f32x16_t mma(Frag a, Frag b, f32x16_t c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
  }
};
template <> struct Mma<float> {
  static constexpr int BK = 32;
  static constexpr int KS = 2;
  static constexpr int EPL = 1;
  typedef float Frag;
  __device__ static Frag ld(const char *p) { return *reinterpret_cast<const float *>(p); }
  __device__ static f32x16_t mma(Frag a, Frag b, f32x16_t c) {
    return __builtin_amdgcn_mfma_f32_32x32x2f32(a, b, c, 0, 0, 0);
  }
};

// 16-byte LDS slot of (row, chunk) after the XOR swizzle.
__device__ __forceinline__ int swz(int row, int chunk) { return row * kChunks + (chunk ^ (row & 7)); }

__device__ __forceinline__ float act_fn(int act, float g, float u, const ActParams &p) {
  if (act == MOE_ACT_RELU2) {
    const float r = fmaxf(g, 0.f);
    return r * r;
  }
  const float gc = fminf(g, p.limit);
  const float uc = fminf(fmaxf(u, -p.limit), p.limit);
  return gc * (1.f / (1.f + expf(-p.alpha * gc))) * (uc + p.beta);
}

template <typename T, int NSETS, int EPI>
__global__ __launch_bounds__(kThreads) void grouped_gemm(
    const T *__restrict__ A, const T *__restrict__ W, T *__restrict__ C,
    const int32_t *__restrict__ offsets, const int32_t *__restrict__ col_sorted,
    const void *__restrict__ gate_scal, int gate_bf16, int E, int K, int Nout, int topk,
    int gather, int interleaved, int act, ActParams prm) {
  using Mm = Mma<T>;
  using Frag = typename Mm::Frag;
  constexpr int BK = Mm::BK;
  constexpr int NB = NSETS * BN;  // B rows per tile
  constexpr int A_CH = BM * kChunks / kThreads;
  constexpr int B_CH = NB * kChunks / kThreads;

  __shared__ u32x4_t sA[2][BM * kChunks];
  __shared__ u32x4_t sB[2][NB * kChunks];
  __shared__ int s_ts[kMaxExperts + 1];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;

  // ---- which expert and rows this workgroup owns ---------------------------
  if (wave == 0) {
    int v[4], s = 0;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int e = lane * 4 + q;
      v[q] = (e < E) ? (offsets[e + 1] - offsets[e] + BM - 1) / BM : 0;
      s += v[q];
    }
    int incl = s;
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
      const int o = __shfl_up(incl, d);
      if (lane >= d) incl += o;
    }
    int run = incl - s;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int e = lane * 4 + q;
      if (e < E) s_ts[e] = run;
      run += v[q];
    }
    if (lane == 63) s_ts[E] = incl;
  }
  __syncthreads();
  const int n_ntiles = (Nout + BN - 1) / BN;
  const int mt = blockIdx.x / n_ntiles;  // n-tiles of one m-tile are adjacent
  const int nt = blockIdx.x - mt * n_ntiles;
  if (mt >= s_ts[E]) return;  // uniform: surplus tile slot
  int lo = 0, hi = E - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (s_ts[mid] <= mt) lo = mid; else hi = mid - 1;
  }
  const int e = lo;
  const int row0 = offsets[e] + (mt - s_ts[e]) * BM;
  const int rows = min(BM, offsets[e + 1] - row0);
  const int n0 = nt * BN;
  const T *We = W + (int64_t)e * NSETS * Nout * K;

  // ---- per-thread global sources of its 16-byte chunks ---------------------
  // A: byte offsets from A (gathered rows for GEMM1), -1 for rows past the
  // segment; B: byte offsets inside this expert's weight block, -1 past Nout.
  int64_t a_off[A_CH];
  int b_off[B_CH];
#pragma unroll
  for (int i = 0; i < A_CH; ++i) {
    const int c = tid + i * kThreads, r = c / kChunks, ch = c % kChunks;
    a_off[i] = -1;
    if (r < rows) {
      const int p = row0 + r;
      const int64_t arow = gather ? (int64_t)(col_sorted[p] / topk) : (int64_t)p;
      a_off[i] = arow * K * (int64_t)sizeof(T) + ch * 16;
    }
  }
#pragma unroll
  for (int i = 0; i < B_CH; ++i) {
    const int c = tid + i * kThreads, r = c / kChunks, ch = c % kChunks;
    const int set = r / BN, n = n0 + r % BN;
    b_off[i] = -1;
    if (n < Nout) {
      const int grow = NSETS == 1 ? n : (interleaved ? 2 * n + set : set * Nout + n);
      b_off[i] = grow * K * (int)sizeof(T) + ch * 16;
    }
  }
  const char *Ab = reinterpret_cast<const char *>(A);
  const char *Bb = reinterpret_cast<const char *>(We);

  const int kbytes = K * (int)sizeof(T);
  const int nk = (K + BK - 1) / BK;
  u32x4_t ra[A_CH], rb[B_CH];
  const u32x4_t zero = {0u, 0u, 0u, 0u};

#define MOE_GLOAD(kt_)                                                                        \
  do {                                                                                        \
    const int kb_ = (kt_) * kRowBytes;                                                        \
    _Pragma("unroll") for (int i = 0; i < A_CH; ++i) {                                        \
      const int ch_ = (tid + i * kThreads) % kChunks;                                         \
      ra[i] = (a_off[i] >= 0 && kb_ + ch_ * 16 < kbytes)                                      \
                  ? *reinterpret_cast<const u32x4_t *>(Ab + a_off[i] + kb_) : zero;             \
    }                                                                                         \
    _Pragma("unroll") for (int i = 0; i < B_CH; ++i) {                                        \
      const int ch_ = (tid + i * kThreads) % kChunks;                                         \
      rb[i] = (b_off[i] >= 0 && kb_ + ch_ * 16 < kbytes)                                      \
                  ? *reinterpret_cast<const u32x4_t *>(Bb + b_off[i] + kb_) : zero;             \
    }                                                                                         \
  } while (0)
#define MOE_SSTORE(st_)                                                                       \
  do {                                                                                        \
    _Pragma("unroll") for (int i = 0; i < A_CH; ++i) {                                        \
      const int c_ = tid + i * kThreads;                                                      \
      sA[(st_)][swz(c_ / kChunks, c_ % kChunks)] = ra[i];                                     \
    }                                                                                         \
    _Pragma("unroll") for (int i = 0; i < B_CH; ++i) {                                        \
      const int c_ = tid + i * kThreads;                                                      \
      sB[(st_)][swz(c_ / kChunks, c_ % kChunks)] = rb[i];                                     \
    }                                                                                         \
  } while (0)

  const int wm = wave & 1, wn = wave >> 1;
  f32x16_t acc[2][2][NSETS];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int s = 0; s < NSETS; ++s)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[i][j][s][r] = 0.f;

  MOE_GLOAD(0);
  MOE_SSTORE(0);
  for (int kt = 0; kt < nk; ++kt) {
    __syncthreads();
    const int st = kt & 1;
    if (kt + 1 < nk) MOE_GLOAD(kt + 1);
    const char *la = reinterpret_cast<const char *>(sA[st]);
    const char *lb = reinterpret_cast<const char *>(sB[st]);
#pragma unroll
    for (int ks = 0; ks < BK / Mm::KS; ++ks) {
      const int byte = (ks * Mm::KS + (lane >> 5) * Mm::EPL) * (int)sizeof(T);
      const int ch = byte >> 4, inner = byte & 15;
      Frag fa[2], fb[2][NSETS];
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        const int row = wm * 64 + i * 32 + (lane & 31);
        fa[i] = Mm::ld(la + swz(row, ch) * 16 + inner);
      }
#pragma unroll
      for (int j = 0; j < 2; ++j)
#pragma unroll
        for (int s = 0; s < NSETS; ++s) {
          const int row = s * BN + wn * 64 + j * 32 + (lane & 31);
          fb[j][s] = Mm::ld(lb + swz(row, ch) * 16 + inner);
        }
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
          for (int s = 0; s < NSETS; ++s) acc[i][j][s] = Mm::mma(fa[i], fb[j][s], acc[i][j][s]);
    }
    if (kt + 1 < nk) MOE_SSTORE((kt + 1) & 1);
  }
#undef MOE_GLOAD
#undef MOE_SSTORE

  // ---- epilogue: lane holds column (lane % 32) and 16 rows of each 32x32 ----
#pragma unroll
  for (int i = 0; i < 2; ++i) {
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int row = wm * 64 + i * 32 + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
      if (row >= rows) continue;
      const int p = row0 + row;
      float g = 1.f;
      int64_t orow = p;
      if (EPI != EPI_ACT) {
        g = gate_bf16 ? to_f32(reinterpret_cast<const bf16_t *>(gate_scal)[p])
                      : reinterpret_cast<const float *>(gate_scal)[p];
        if (EPI == EPI_OUT) orow = col_sorted[p];  // topk == 1: entry index == token
      }
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const int col = n0 + wn * 64 + j * 32 + (lane & 31);
        if (col >= Nout) continue;
        float v;
        if (EPI == EPI_ACT)
          v = act_fn(act, acc[i][j][0][r], NSETS == 2 ? acc[i][j][NSETS - 1][r] : 0.f, prm);
        else
          v = acc[i][j][0][r] * g;
        C[orow * Nout + col] = from_f32<T>(v);
      }
    }
  }
}

template <typename T, int NSETS, int EPI>
hipError_t launch_t(const void *A, const void *W, void *C, const int32_t *offsets,
                    const int32_t *col_sorted, const void *gate_scal, int gate_bf16, int64_t M,
                    int E, int K, int Nout, int topk, int gather, int interleaved, int act,
                    ActParams prm, hipStream_t s) {
  const int64_t mtiles = M / BM + (M < E ? M : E);
  const dim3 grid((unsigned)(mtiles * ((Nout + BN - 1) / BN)));
  hipLaunchKernelGGL((grouped_gemm<T, NSETS, EPI>), grid, dim3(kThreads), 0, s,
                     reinterpret_cast<const T *>(A), reinterpret_cast<const T *>(W),
                     reinterpret_cast<T *>(C), offsets, col_sorted, gate_scal, gate_bf16, E, K,
                     Nout, topk, gather, interleaved, act, prm);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_gemm1(const void *x, const void *w13, void *act_out, const int32_t *offsets,
                        const int32_t *col_sorted, moe_dtype_t dt, int64_t n_tokens, int topk,
                        int n_experts, int hidden, int inter, moe_act_t act,
                        moe_w13_layout_t layout, ActParams p, hipStream_t s) {
  const int64_t M = n_tokens * topk;
  const int il = layout == MOE_W13_INTERLEAVED;
  const bool gated = act != MOE_ACT_RELU2;
  if (dt == MOE_BF16) {
    return gated ? launch_t<bf16_t, 2, EPI_ACT>(x, w13, act_out, offsets, col_sorted, nullptr, 0, M,
                                               n_experts, hidden, inter, topk, 1, il, act, p, s)
                 : launch_t<bf16_t, 1, EPI_ACT>(x, w13, act_out, offsets, col_sorted, nullptr, 0, M,
                                               n_experts, hidden, inter, topk, 1, il, act, p, s);
  }
  return gated ? launch_t<float, 2, EPI_ACT>(x, w13, act_out, offsets, col_sorted, nullptr, 0, M,
                                            n_experts, hidden, inter, topk, 1, il, act, p, s)
               : launch_t<float, 1, EPI_ACT>(x, w13, act_out, offsets, col_sorted, nullptr, 0, M,
                                            n_experts, hidden, inter, topk, 1, il, act, p, s);
}

hipError_t launch_gemm2(const void *act_in, const void *w2, void *y, const int32_t *offsets,
                        const int32_t *col_sorted, const void *gate_scal, moe_dtype_t gate_dt,
                        moe_dtype_t dt, int64_t n_tokens, int topk, int n_experts, int hidden,
                        int inter, bool direct_out, hipStream_t s) {
  const int64_t M = n_tokens * topk;
  const int gb = gate_dt == MOE_BF16;
  const ActParams none{1.f, 0.f, 0.f};
  if (dt == MOE_BF16) {
    return direct_out
               ? launch_t<bf16_t, 1, EPI_OUT>(act_in, w2, y, offsets, col_sorted, gate_scal, gb, M,
                                              n_experts, inter, hidden, topk, 0, 0, 0, none, s)
               : launch_t<bf16_t, 1, EPI_Y>(act_in, w2, y, offsets, col_sorted, gate_scal, gb, M,
                                            n_experts, inter, hidden, topk, 0, 0, 0, none, s);
  }
  return direct_out
             ? launch_t<float, 1, EPI_OUT>(act_in, w2, y, offsets, col_sorted, gate_scal, gb, M,
                                           n_experts, inter, hidden, topk, 0, 0, 0, none, s)
             : launch_t<float, 1, EPI_Y>(act_in, w2, y, offsets, col_sorted, gate_scal, gb, M,
                                         n_experts, inter, hidden, topk, 0, 0, 0, none, s);
}

}  // namespace moe
