// Routing kernels for gfx950: top-k gating + softmax over the selected logits,
// expert bitmatrix, per-expert histogram, ragged offsets, and the stable
// expert-sorted gather/scatter indices with permuted gate weights.
//
// What is computed follows the topk / routing_data_from_sparse_topk description
// in the vLLM PR #45457 report ("implementation breakdown", "key source
// snippets") and the stable sort-by-expert of the minimind issue #835 page ("It
// is removable in plain PyTorch").  How it is computed is this file's own design:
//
//  * route_topk_rank: one workgroup per 256 tokens.  A token's logits row is
//    read by a group of G lanes with 16-byte loads (G = E / values-per-load,
//    rounded up to a power of two), each logit becomes an order-preserving
//    integer key (value bits, then the inverted expert index, so equal values
//    rank the lower index higher), and k rounds of an in-group max reduction
//    (xor shuffles) pick the top-k.  Then every wave builds, with one ballot per
//    expert, the 64-bit mask of its tokens that chose that expert; popcounts of
//    those masks give per-wave counts and the stable in-wave rank of every
//    entry, and a prefix over the four waves gives the rank within the block.
//    No atomics: the result is the same on every run.
//  * route_scatter: per-expert totals and this block's prefix over earlier
//    blocks, an exclusive scan into offsets, and the scatter of every entry to
//    p = offsets[e] + (entries of e in earlier blocks) + rank in block.
//  * When all tokens fit one block, route_topk_rank does the scan and scatter
//    itself (one launch for the whole routing step).
#include "moe_common.h"

namespace moe {
namespace {

template <typename T> struct Logit;

// bf16 logits: key = ordered 16 value bits << 16 | (0xffff - expert).
template <> struct Logit<bf16_t> {
  typedef uint32_t Key;
  static constexpr int kVec = 8;  // values per 16-byte load
  __device__ static Key key(uint32_t bits, int e) {
    if (bits == 0x8000u) bits = 0u;  // -0 ranks as +0
    const uint32_t ord = (bits & 0x8000u) ? (~bits & 0xffffu) : (bits | 0x8000u);
    return (ord << 16) | (uint32_t)(0xffff - e);
  }
  __device__ static int expert(Key k) { return 0xffff - (int)(k & 0xffffu); }
  __device__ static float value(Key k) {
    const uint32_t ord = k >> 16;
    const uint32_t bits = (ord & 0x8000u) ? (ord & 0x7fffu) : (~ord & 0xffffu);
    return __uint_as_float(bits << 16);
  }
  __device__ static void load(const bf16_t *row, int e0, int E, bool vec, Key (&k)[kVec]) {
    if (vec) {
      const u32x4_t v = *reinterpret_cast<const u32x4_t *>(row + e0);
      const uint32_t w[4] = {v[0], v[1], v[2], v[3]};
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        k[2 * i] = key(w[i] & 0xffffu, e0 + 2 * i);
        k[2 * i + 1] = key(w[i] >> 16, e0 + 2 * i + 1);
      }
    } else {
#pragma unroll
      for (int i = 0; i < kVec; ++i) k[i] = (e0 + i < E) ? key(row[e0 + i], e0 + i) : 0u;
    }
  }
};

// fp32 logits: key = ordered 32 value bits << 32 | (0xffff - expert).
template <> struct Logit<float> {
  typedef unsigned long long Key;
  static constexpr int kVec = 4;
  __device__ static Key key(uint32_t bits, int e) {
    if (bits == 0x80000000u) bits = 0u;
    const uint32_t ord = (bits & 0x80000000u) ? ~bits : (bits | 0x80000000u);
    return ((Key)ord << 32) | (Key)(uint32_t)(0xffff - e);
  }
  __device__ static int expert(Key k) { return 0xffff - (int)(k & 0xffffu); }
  __device__ static float value(Key k) {
    const uint32_t ord = (uint32_t)(k >> 32);
    const uint32_t bits = (ord & 0x80000000u) ? (ord & 0x7fffffffu) : ~ord;
    return __uint_as_float(bits);
  }
  __device__ static void load(const float *row, int e0, int E, bool vec, Key (&k)[kVec]) {
    if (vec) {
      const u32x4_t v = *reinterpret_cast<const u32x4_t *>(row + e0);
      k[0] = key(v[0], e0);
      k[1] = key(v[1], e0 + 1);
      k[2] = key(v[2], e0 + 2);
      k[3] = key(v[3], e0 + 3);
    } else {
#pragma unroll
      for (int i = 0; i < kVec; ++i)
        k[i] = (e0 + i < E) ? key(__float_as_uint(row[e0 + i]), e0 + i) : 0ull;
    }
  }
};

__device__ __forceinline__ uint32_t shfl_xor_key(uint32_t v, int m) {
  return (uint32_t)__shfl_xor((int)v, m);
}
__device__ __forceinline__ unsigned long long shfl_xor_key(unsigned long long v, int m) {
  const uint32_t lo = (uint32_t)__shfl_xor((int)(uint32_t)v, m);
  const uint32_t hi = (uint32_t)__shfl_xor((int)(uint32_t)(v >> 32), m);
  return ((unsigned long long)hi << 32) | lo;
}

// Exclusive scan of in[0..E) into out[0..E], out[E] = total; E <= 256.  Wave 0
// does the work (four elements per lane + a shuffle scan); all threads sync.
__device__ void block_exclusive_scan(const int *in, int *out, int E) {
  if (threadIdx.x < 64) {
    const int lane = threadIdx.x;
    int v[4];
    int s = 0;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int e = lane * 4 + q;
      v[q] = (e < E) ? in[e] : 0;
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
      if (e < E) out[e] = run;
      run += v[q];
    }
    if (lane == 63) out[E] = incl;
  }
  __syncthreads();
}

template <typename T>
__global__ __launch_bounds__(kRouteThreads) void route_topk_rank(
    const T *__restrict__ logits, int64_t N, int E, int K, int logG, int vec,
    int32_t *__restrict__ topk_idx, T *__restrict__ topk_w, uint32_t *__restrict__ bitmatrix,
    int32_t *__restrict__ blk_cnt, uint8_t *__restrict__ blk_rank, int fused,
    int32_t *__restrict__ col_sum, int32_t *__restrict__ offsets,
    int32_t *__restrict__ col_sorted, int32_t *__restrict__ row_sorted,
    T *__restrict__ gate_scal) {
  using L = Logit<T>;
  using Key = typename L::Key;
  constexpr int V = L::kVec;
  constexpr int kWords = kMaxExperts / 32;

  __shared__ uint32_t s_bits[kRouteTokens][kWords];
  __shared__ uint8_t s_sel[kRouteTokens * kMaxTopk];
  __shared__ uint8_t s_rank[kRouteTokens * kMaxTopk];
  __shared__ T s_w[kRouteTokens * kMaxTopk];
  __shared__ unsigned long long s_mask[kRouteThreads / 64][kMaxExperts];
  __shared__ int s_cnt[kRouteThreads / 64][kMaxExperts];
  __shared__ int s_tot[kMaxExperts];
  __shared__ int s_off[kMaxExperts + 1];

  const int tid = threadIdx.x;
  const int wave = tid >> 6, lane = tid & 63;
  const int G = 1 << logG;
  const int tpp = 64 >> logG;  // tokens per wave pass
  const int grp = lane >> logG, lg = lane & (G - 1);
  const int words = (E + 31) >> 5;
  const int64_t tok0 = (int64_t)blockIdx.x * kRouteTokens;

  // ---- phase A: top-k + softmax + bitmatrix, G lanes per token ------------
  for (int pass = 0; pass < G; ++pass) {
    const int tl = wave * 64 + pass * tpp + grp;  // token within the block
    const int64_t t = tok0 + tl;
    const bool live = t < N;
    const int e0 = lg * V;
    Key key[V];
    if (live && e0 < E) {
      L::load(logits + t * E, e0, E, vec != 0, key);
    } else {
#pragma unroll
      for (int i = 0; i < V; ++i) key[i] = 0;
    }
    int sel_e[kMaxTopk];
    float sel_v[kMaxTopk];
#pragma unroll
    for (int j = 0; j < kMaxTopk; ++j) {
      sel_e[j] = 0;
      sel_v[j] = 0.f;
      if (j < K) {
        Key m = key[0];
#pragma unroll
        for (int i = 1; i < V; ++i) m = key[i] > m ? key[i] : m;
        for (int d = 1; d < G; d <<= 1) {
          const Key o = shfl_xor_key(m, d);
          m = o > m ? o : m;
        }
        const int e = L::expert(m);
        sel_e[j] = e;
        sel_v[j] = L::value(m);
#pragma unroll
        for (int i = 0; i < V; ++i)
          if (e0 + i == e) key[i] = 0;  // only the owning lane matches
      }
    }
    // softmax over the selected logits (slot 0 holds the maximum)
    float ex[kMaxTopk];
    float ssum = 0.f;
#pragma unroll
    for (int j = 0; j < kMaxTopk; ++j) {
      ex[j] = 0.f;
      if (j < K) {
        ex[j] = expf(sel_v[j] - sel_v[0]);
        ssum += ex[j];
      }
    }
    if (live) {
#pragma unroll
      for (int j = 0; j < kMaxTopk; ++j) {
        if (j < K) {
          const T w = from_f32<T>(ex[j] / ssum);
          if ((j & (G - 1)) == lg) {
            topk_idx[t * K + j] = sel_e[j];
            topk_w[t * K + j] = w;
          }
          if (lg == 0) {
            s_sel[tl * K + j] = (uint8_t)sel_e[j];
            s_w[tl * K + j] = w;
          }
        }
      }
#pragma unroll
      for (int wd = 0; wd < kWords; ++wd) {
        if (wd < words && (wd & (G - 1)) == lg) {
          uint32_t word = 0;
#pragma unroll
          for (int j = 0; j < kMaxTopk; ++j)
            if (j < K && (sel_e[j] >> 5) == wd) word |= 1u << (sel_e[j] & 31);
          bitmatrix[t * words + wd] = word;
          s_bits[tl][wd] = word;
        }
      }
    } else {
#pragma unroll
      for (int wd = 0; wd < kWords; ++wd)
        if (wd < words && (wd & (G - 1)) == lg) s_bits[tl][wd] = 0u;
    }
  }
  __syncthreads();

  // ---- phase B: per-wave expert masks by ballot; thread tid owns token tid --
  {
    uint32_t myb[kWords];
#pragma unroll
    for (int wd = 0; wd < kWords; ++wd) myb[wd] = (wd < words) ? s_bits[tid][wd] : 0u;
    unsigned long long mk[kMaxExperts / 64] = {0ull, 0ull, 0ull, 0ull};
#pragma unroll
    for (int wd = 0; wd < kWords; ++wd) {
      if (wd < words) {
#pragma unroll
        for (int b = 0; b < 32; ++b) {
          const int e = wd * 32 + b;
          if (e < E) {
            const unsigned long long m = __ballot((myb[wd] >> b) & 1u);
            if (lane == (e & 63)) mk[wd >> 1] = m;
          }
        }
      }
    }
#pragma unroll
    for (int q = 0; q < kMaxExperts / 64; ++q) {
      const int e = q * 64 + lane;
      if (e < E) {
        s_mask[wave][e] = mk[q];
        s_cnt[wave][e] = popc64(mk[q]);
      }
    }
  }
  __syncthreads();
  for (int e = tid; e < E; e += kRouteThreads) {
    int run = 0;
#pragma unroll
    for (int w = 0; w < kRouteThreads / 64; ++w) {
      const int c = s_cnt[w][e];
      s_cnt[w][e] = run;  // exclusive prefix over the block's waves
      run += c;
    }
    s_tot[e] = run;
  }
  __syncthreads();
  {
    const int64_t t = tok0 + tid;
    if (t < N) {
      const unsigned long long below = lane ? (~0ull >> (64 - lane)) : 0ull;
#pragma unroll
      for (int j = 0; j < kMaxTopk; ++j) {
        if (j < K) {
          const int e = s_sel[tid * K + j];
          const int r = s_cnt[wave][e] + popc64(s_mask[wave][e] & below);
          if (fused)
            s_rank[tid * K + j] = (uint8_t)r;
          else
            blk_rank[t * K + j] = (uint8_t)r;
        }
      }
    }
  }
  if (!fused) {
    for (int e = tid; e < E; e += kRouteThreads) blk_cnt[(int64_t)blockIdx.x * E + e] = s_tot[e];
    return;
  }

  // ---- fused tail (a single block holds every token) -----------------------
  __syncthreads();
  block_exclusive_scan(s_tot, s_off, E);
  for (int e = tid; e <= E; e += kRouteThreads) {
    offsets[e] = s_off[e];
    if (e < E) col_sum[e] = s_tot[e];
  }
  const int M = (int)N * K;
  for (int f = tid; f < M; f += kRouteThreads) {
    const int p = s_off[s_sel[f]] + s_rank[f];
    col_sorted[p] = f;
    row_sorted[f] = p;
    gate_scal[p] = s_w[f];
  }
}

template <typename T>
__global__ __launch_bounds__(kRouteThreads) void route_scatter(
    int64_t N, int E, int K, int nblocks, const int32_t *__restrict__ blk_cnt,
    const uint8_t *__restrict__ blk_rank, const int32_t *__restrict__ topk_idx,
    const T *__restrict__ topk_w, int32_t *__restrict__ col_sum, int32_t *__restrict__ offsets,
    int32_t *__restrict__ col_sorted, int32_t *__restrict__ row_sorted,
    T *__restrict__ gate_scal) {
  __shared__ int s_tot[kMaxExperts];
  __shared__ int s_base[kMaxExperts];
  __shared__ int s_off[kMaxExperts + 1];
  const int tid = threadIdx.x;
  const int b = blockIdx.x;
  for (int e = tid; e < E; e += kRouteThreads) {
    int pre = 0, post = 0;
    for (int bb = 0; bb < b; ++bb) pre += blk_cnt[(int64_t)bb * E + e];
    for (int bb = b; bb < nblocks; ++bb) post += blk_cnt[(int64_t)bb * E + e];
    s_tot[e] = pre + post;
    s_base[e] = pre;
  }
  __syncthreads();
  block_exclusive_scan(s_tot, s_off, E);
  if (b == 0) {
    for (int e = tid; e <= E; e += kRouteThreads) {
      offsets[e] = s_off[e];
      if (e < E) col_sum[e] = s_tot[e];
    }
  }
  for (int e = tid; e < E; e += kRouteThreads) s_base[e] += s_off[e];
  __syncthreads();
  const int64_t f0 = (int64_t)b * kRouteTokens * K;
  const int64_t tend = ((int64_t)(b + 1) * kRouteTokens < N) ? (int64_t)(b + 1) * kRouteTokens : N;
  const int64_t f1 = tend * K;
  for (int64_t f = f0 + tid; f < f1; f += kRouteThreads) {
    const int p = s_base[topk_idx[f]] + blk_rank[f];
    col_sorted[p] = (int32_t)f;
    row_sorted[f] = p;
    gate_scal[p] = topk_w[f];
  }
}

inline size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

template <typename T>
hipError_t launch_route_t(const T *logits, int64_t N, int E, int K, const moe_routing_t *r,
                          void *scratch, hipStream_t s) {
  constexpr int V = Logit<T>::kVec;
  const int need = (E + V - 1) / V;
  int logG = 0;
  while ((1 << logG) < need) ++logG;
  const int vec = (E % V) == 0;
  const int64_t nb = (N + kRouteTokens - 1) / kRouteTokens;
  const int fused = nb == 1;
  int32_t *blk_cnt = reinterpret_cast<int32_t *>(scratch);
  uint8_t *blk_rank = reinterpret_cast<uint8_t *>(scratch) + align256((size_t)nb * E * 4);
  T *tw = reinterpret_cast<T *>(r->topk_w);
  T *gs = reinterpret_cast<T *>(r->gate_scal);
  hipLaunchKernelGGL(route_topk_rank<T>, dim3((unsigned)nb), dim3(kRouteThreads), 0, s, logits,
                     N, E, K, logG, vec, r->topk_idx, tw, r->bitmatrix, blk_cnt, blk_rank, fused,
                     r->col_sum, r->offsets, r->col_sorted, r->row_sorted, gs);
  if (!fused) {
    hipLaunchKernelGGL(route_scatter<T>, dim3((unsigned)nb), dim3(kRouteThreads), 0, s, N, E, K,
                       (int)nb, blk_cnt, blk_rank, r->topk_idx, tw, r->col_sum, r->offsets,
                       r->col_sorted, r->row_sorted, gs);
  }
  return hipGetLastError();
}

}  // namespace

size_t route_scratch_bytes(int64_t n_tokens, int n_experts, int topk) {
  const int64_t nb = (n_tokens + kRouteTokens - 1) / kRouteTokens;
  return align256((size_t)nb * n_experts * 4) + align256((size_t)n_tokens * topk);
}

hipError_t launch_route(const void *logits, moe_dtype_t dt, int64_t n_tokens, int n_experts,
                        int topk, const moe_routing_t *r, void *scratch, hipStream_t s) {
  if (dt == MOE_BF16)
    return launch_route_t<bf16_t>(reinterpret_cast<const bf16_t *>(logits), n_tokens, n_experts,
                                  topk, r, scratch, s);
  return launch_route_t<float>(reinterpret_cast<const float *>(logits), n_tokens, n_experts,
                               topk, r, scratch, s);
}

}  // namespace moe
