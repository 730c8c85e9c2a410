// Routing kernels for gfx950: top-k gating + softmax over the selected logits,
// expert bitmatrix, per-expert histogram, ragged offsets, and the stable
// expert-sorted gather/scatter indices with permuted gate weights.
//
// What is computed follows the topk / routing_data_from_sparse_topk description
// in the vLLM PR #45457 report ("implementation breakdown", "key source
// snippets") and the stable sort-by-expert of the minimind issue #835 page ("It
// is removable in plain PyTorch").  How it is computed is this file's own design:
//
//  * route_topk_rank: one workgroup of 1024 threads per 256 tokens.  A
//    token's logits row is read by a group of G lanes with 16-byte loads, one
//    or two per lane (G = E / values-per-lane, rounded up to a power of two),
//    each logit
//    becomes an order-preserving integer key (value bits, then the inverted
//    expert index, so equal values rank the lower index higher), and k rounds
//    of an in-group max reduction (DPP row permutes, then shuffles) pick the
//    top-k.  Then, per wave of 64 tokens, one ballot per expert gives the mask
//    of the tokens that chose it; popcounts of those masks give per-wave counts
//    and the stable in-wave rank of every entry, and a prefix over the waves
//    gives the rank within the block.  No atomics: every run gives the same
//    result.
//  * route_scatter: per-expert totals and this block's prefix over earlier
//    blocks, an exclusive scan into offsets, and the scatter of every entry to
//    p = offsets[e] + (entries of e in earlier blocks) + rank in block.
//  * route_fused: batches of up to 256 tokens run both phases in one
//    workgroup of 1024 threads with every per-entry value kept in LDS (one
//    launch for the whole routing step).
//  * route_one: a single token, in one wave's registers (no workgroup
//    barrier; offsets and positions are prefix popcounts of its experts).
//
// Router GEMM (moe_gate_route): the logits are computed from the token rows and
// the router's gate weight (logits = x . W_gate^T, fp32 accumulation on MFMA,
// rounded once to the layer dtype) and written out; top-k then runs on them.
// The router's own matmul is the step ahead of the routing that the vLLM PR
// #45457 report leaves as a separate kernel ("motivation").  Up to
// kGateGemvTokens tokens take a wave per expert row (gate_gemv).  Batches of up
// to kGateSplitTokens tokens
// split the product over 64-token tiles and K-groups
// (gate_partial, about one workgroup a compute unit) and add the fp32 group
// sums up in the routing kernel's prologue (one token, or a few with little to
// add) or in gate_reduce; rows too short to split and larger batches run the
// whole product per token tile, in the prologue of the one-workgroup routing
// kernel (at most kGateFusedTokens tokens) or as gate_gemm ahead of the
// routing kernels.
//
// Expert-parallel share: every kernel takes the share [lo, lo + nl) of the E
// experts that this GPU holds (lo = 0, nl = E for the whole layer).  Top-k and
// softmax run over all E logits; the selected ids are then remapped to local
// ids e - lo, and the bitmatrix, counts, ranks, offsets and sorted indices are
// over the nl local experts only.  A slot whose expert lies outside the share
// gets row_sorted = -1 and no sorted position; sorted positions past the last
// local entry get col_sorted = -1 and gate weight 0.  The remap and re-packing
// of the bitmatrix follow the expert-map branch described in the vLLM PR
// #45457 report ("implementation breakdown"), with the share given as the
// (local_expert_offset, num_local_experts) pair of the kernel call in the PR
// #47106 report ("key source snippets").
#include <type_traits>

#include "lds_dma.h"
#include "moe_common.h"

namespace moe {
namespace {

template <typename T> struct Logit;

// 16 bytes of one token's logits row (values e0 .. e0 + kVec - 1), zero past E.
__device__ __forceinline__ uint32_t bits_of(bf16_t v) { return v; }
__device__ __forceinline__ uint32_t bits_of(float v) { return __float_as_uint(v); }

template <typename T>
__device__ __forceinline__ u32x4_t fetch16(const T *row, int e0, int E, bool vec) {
  if (vec) return *reinterpret_cast<const u32x4_t *>(row + e0);
  constexpr int V = 16 / sizeof(T), PW = 4 / sizeof(T);  // values per 32-bit word
  u32x4_t r = {0u, 0u, 0u, 0u};
#pragma unroll
  for (int i = 0; i < V; ++i)
    if (e0 + i < E) r[i / PW] |= bits_of(row[e0 + i]) << (32 / PW * (i % PW));
  return r;
}

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
  // keys of values e0 .. e0 + 7; values past E (zero-filled) get key 0
  __device__ static void decode(u32x4_t v, int e0, int E, Key (&k)[kVec]) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      k[2 * i] = (e0 + 2 * i < E) ? key(v[i] & 0xffffu, e0 + 2 * i) : 0u;
      k[2 * i + 1] = (e0 + 2 * i + 1 < E) ? key(v[i] >> 16, e0 + 2 * i + 1) : 0u;
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
  __device__ static void decode(u32x4_t v, int e0, int E, Key (&k)[kVec]) {
#pragma unroll
    for (int i = 0; i < 4; ++i) k[i] = (e0 + i < E) ? key(v[i], e0 + i) : 0ull;
  }
};

// ---- in-group maximum of order keys -----------------------------------------
// Groups of G lanes (G a power of two, aligned).  Steps inside a 16-lane row
// use DPP row permutes (register-only): swap neighbours, swap pairs, mirror
// each half-row, mirror the row.  After each step every lane holds the max of
// a block twice as large.  Wider groups finish with cross-row shuffles.
template <int CTRL> __device__ __forceinline__ uint32_t dpp32(uint32_t v) {
  return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, CTRL, 0xf, 0xf, false);
}
template <int CTRL> __device__ __forceinline__ uint32_t dpp(uint32_t v) { return dpp32<CTRL>(v); }
template <int CTRL> __device__ __forceinline__ unsigned long long dpp(unsigned long long v) {
  return ((unsigned long long)dpp32<CTRL>((uint32_t)(v >> 32)) << 32) | dpp32<CTRL>((uint32_t)v);
}
__device__ __forceinline__ uint32_t xshfl(uint32_t v, int m) { return (uint32_t)__shfl_xor((int)v, m); }
__device__ __forceinline__ unsigned long long xshfl(unsigned long long v, int m) {
  return ((unsigned long long)xshfl((uint32_t)(v >> 32), m) << 32) | xshfl((uint32_t)v, m);
}
template <typename K> __device__ __forceinline__ K kmax(K a, K b) { return a > b ? a : b; }

template <typename K> __device__ __forceinline__ K group_max(K m, int G) {
  if (G >= 2) m = kmax(m, dpp<0xB1>(m));    // quad_perm [1,0,3,2]
  if (G >= 4) m = kmax(m, dpp<0x4E>(m));    // quad_perm [2,3,0,1]
  if (G >= 8) m = kmax(m, dpp<0x141>(m));   // row_half_mirror
  if (G >= 16) m = kmax(m, dpp<0x140>(m));  // row_mirror
  if (G >= 32) m = kmax(m, xshfl(m, 16));
  if (G >= 64) m = kmax(m, xshfl(m, 32));
  return m;
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
    const int incl = wave_inclusive_sum(s);
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

// LDS of one routing chunk: NT tokens, at most MAXE experts and MAXK slots.
template <typename T, int NT, int MAXE = kMaxExperts, int MAXK = kMaxTopk> struct ChunkLds {
  static constexpr int kTokens = NT, kExperts = MAXE, kSlots = MAXK, kWords = (MAXE + 31) / 32;
  uint32_t bits[NT][kWords];               // bitmatrix rows of the chunk
  uint8_t sel[NT * MAXK];                  // selected experts, slot order
  T w[NT * MAXK];                          // their weights (layer dtype)
  float val[NT * MAXK];                    // their logits
  unsigned long long mask[NT / 64][MAXE];  // per-wave ballot masks
  int cnt[NT / 64][MAXE];                  // per-wave counts -> exclusive wave bases
  int tot[MAXE];                           // chunk counts per expert
};

// Phase A for tokens [tok0, tok0 + NT): top-k, softmax, topk_idx / topk_w /
// bitmatrix rows to HBM, selected experts and bitmatrix rows to LDS.
// C: 16-byte logit chunks per lane (C * kVec consecutive experts per lane), so
// G = ceil(E / (C * kVec)) lanes serve one token.  Fewer lanes per token cost
// fewer VALU lane-operations per selection round, so wide expert sets use C = 2.
template <typename T, int THREADS, int C, typename Lds>
__device__ __forceinline__ void topk_chunk(const T *logits, int64_t N, int E, int K,
                                           int lo, int nl, int logG, int vec, int64_t tok0,
                                           int32_t *__restrict__ topk_idx,
                                           T *__restrict__ topk_w,
                                           uint32_t *__restrict__ bitmatrix, Lds &L) {
  constexpr int NT = Lds::kTokens;
  using Lg = Logit<T>;
  using Key = typename Lg::Key;
  constexpr int V = Lg::kVec;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int G = 1 << logG;
  const int tpp = 64 >> logG;  // tokens per wave pass
  const int grp = lane >> logG, lg = lane & (G - 1);
  const int words = (nl + 31) >> 5;  // bitmatrix words over the local experts
  // Whole passes are dealt round-robin over the NW = THREADS / 64 waves: pass
  // p of wave w is pass q = p * NW + w of the chunk, whose group grp holds
  // chunk token q * tpp + grp.  A partial chunk then fills the passes of the
  // first waves and the rest stop at once: a wave's pass costs the same
  // instructions however many of its groups hold a token, so spreading a few
  // tokens over every wave multiplied the selection's VALU work (32 tokens of
  // 4 lanes each: 16 wave passes instead of 2).
  constexpr int NW = THREADS / 64;
  const int npass = (NT / NW + tpp - 1) / tpp;
  // A lane's 16-byte logit chunks for kBatch passes are fetched before any is
  // used, so their loads overlap.  The batch is kept small: these kernels run
  // their code once per wave, so every extra unrolled copy is paid in cold
  // instruction-cache misses.
  constexpr int kBatch = 4;
  // A pass whose first token (group 0) is past N has no live token, nor has
  // any later pass of the wave: the wave stops there (the rank phase treats
  // chunk tokens past N as empty).
  auto first_tok = [&](int p) { return tok0 + ((int64_t)p * NW + wave) * tpp; };
  for (int pass0 = 0; pass0 < npass && first_tok(pass0) < N; pass0 += kBatch) {
    u32x4_t raw[kBatch][C];
#pragma unroll
    for (int q = 0; q < kBatch; ++q) {
      const int tl = ((pass0 + q) * NW + wave) * tpp + grp;  // token within the chunk
      const int64_t t = tok0 + tl;
#pragma unroll
      for (int c = 0; c < C; ++c) {
        const int ec = (lg * C + c) * V;
        raw[q][c] = u32x4_t{0u, 0u, 0u, 0u};
        if (tl < NT && t < N && ec < E) raw[q][c] = fetch16(logits + t * E, ec, E, vec != 0);
      }
    }
#pragma unroll
    for (int q = 0; q < kBatch; ++q) {
      if (pass0 + q < npass && first_tok(pass0 + q) < N) {
        const int tl = ((pass0 + q) * NW + wave) * tpp + grp;
        const int64_t t = tok0 + tl;
        const bool inwave = tl < NT;
        const bool live = inwave && t < N;
        const int e0 = lg * C * V;  // this lane's experts: e0 .. e0 + C * V - 1
        Key key[C * V];
#pragma unroll
        for (int c = 0; c < C; ++c) {
          Key kc[V];
          Lg::decode(raw[q][c], e0 + c * V, live ? E : 0, kc);
#pragma unroll
          for (int i = 0; i < V; ++i) key[c * V + i] = kc[i];
        }
        // k rounds: the group's largest remaining key; its owner clears it.
        // Slot j's expert and logit go to LDS (the group's lanes share them).
        uint32_t word = 0;  // bitmatrix word lg of this token (local expert ids)
        for (int j = 0; j < K; ++j) {
          Key m = key[0];
#pragma unroll
          for (int i = 1; i < C * V; ++i) m = kmax(m, key[i]);
          m = group_max(m, G);
          const int e = Lg::expert(m);
#pragma unroll
          for (int i = 0; i < C * V; ++i)
            if (e0 + i == e) key[i] = 0;  // only the owning lane matches
          const int l = e - lo;
          if ((unsigned)l < (unsigned)nl && (l >> 5) == lg) word |= 1u << (l & 31);
          if (lg == 0 && inwave) {
            L.sel[tl * K + j] = (uint8_t)e;
            L.val[tl * K + j] = Lg::value(m);
          }
        }
        if (live) {
          // softmax over the selected logits, summed in slot order; slot 0 is the max
          const float* vals = &L.val[tl * K];
          const float vmax = vals[0];
          float ssum = 0.f;
          for (int j = 0; j < K; ++j) ssum += expf(vals[j] - vmax);
          for (int j = lg; j < K; j += G) {
            const T w = from_f32<T>(expf(vals[j] - vmax) / ssum);
            topk_idx[t * K + j] = L.sel[tl * K + j];
            topk_w[t * K + j] = w;
            L.w[tl * K + j] = w;
          }
          if (lg < words) {
            bitmatrix[t * words + lg] = word;
            L.bits[tl][lg] = word;
          }
        }
      }
    }
  }
}

// Phase B: per-wave ballot masks per expert, exclusive wave bases in L.cnt,
// chunk totals in L.tot.  Ends synchronised.  With at least as many waves as
// 64-token groups, group tw is handled by THREADS / NT waves, each taking a
// contiguous share of the experts, so the per-expert ballot loop runs in
// parallel; with fewer waves, each wave takes whole groups, all experts.
template <int THREADS, typename Lds>
__device__ __forceinline__ void rank_chunk(int E, int nlive, Lds &L) {
  constexpr int NT = Lds::kTokens, TW = NT / 64, NWV = THREADS / 64;
  constexpr int PARTS = NWV >= TW ? NWV / TW : 1;
  static_assert(NWV >= TW ? PARTS * TW == NWV && PARTS >= (Lds::kExperts + 127) / 128
                          : TW % NWV == 0 && Lds::kExperts <= 128,
                "rank split: at most 128 experts a share");
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int part = NWV >= TW ? wave / TW : 0;                 // wave-uniform
  const int per = (E + PARTS - 1) / PARTS;
  const int e_beg = part * per, e_end = min(E, e_beg + per);
  for (int tw = NWV >= TW ? wave % TW : wave; tw < TW; tw += NWV >= TW ? TW : NWV) {
    const int tok = tw * 64 + lane;  // chunk token of this lane
    if (tw * 64 >= nlive) {
      // no live token in this group: empty masks and zero counts
      for (int e = e_beg + lane; e < e_end; e += 64) {
        L.mask[tw][e] = 0ull;
        L.cnt[tw][e] = 0;
      }
      continue;
    }
    // Lane l keeps the masks of the (at most two) experts e of this share with
    // e % 64 == l in registers and stores them after the loop, so the loop
    // body touches no LDS (one bitmatrix word is read per 32 experts).
    const bool has = tok < nlive;  // chunk tokens past N chose nothing
    unsigned long long m0 = 0, m1 = 0;
    for (int wi = e_beg >> 5; wi <= ((e_end - 1) >> 5) && e_beg < e_end; ++wi) {
      const uint32_t w = has ? L.bits[tok][wi] : 0u;
      const int lo = max(e_beg, wi * 32), hi = min(e_end, wi * 32 + 32);
      for (int e = lo; e < hi; ++e) {  // a runtime loop keeps the code small
        const unsigned long long m = __ballot((w >> (e & 31)) & 1u);
        if (lane == (e & 63)) {
          if (e - e_beg < 64) m0 = m; else m1 = m;
        }
      }
    }
    const int ea = e_beg + ((lane - e_beg) & 63);  // this lane's experts: ea, ea + 64
    if (ea < e_end) {
      L.mask[tw][ea] = m0;
      L.cnt[tw][ea] = popc64(m0);
    }
    if (ea + 64 < e_end) {
      L.mask[tw][ea + 64] = m1;
      L.cnt[tw][ea + 64] = popc64(m1);
    }
  }
  __syncthreads();
  // exclusive prefix over the chunk's (at most four) groups: one thread per
  // expert walks them in order
  static_assert(TW <= 4, "a short serial prefix over the groups");
  for (int e = tid; e < E; e += THREADS) {
    int run = 0;
#pragma unroll
    for (int g = 0; g < TW; ++g) {
      const int c = L.cnt[g][e];
      L.cnt[g][e] = run;
      run += c;
    }
    L.tot[e] = run;
  }
  __syncthreads();
}

// Rank within the chunk of an entry of chunk token t for expert e.
template <typename Lds>
__device__ __forceinline__ int chunk_rank(const Lds &L, int t, int e) {
  const int tw = t >> 6, ln = t & 63;
  const unsigned long long below = ln ? (~0ull >> (64 - ln)) : 0ull;
  return L.cnt[tw][e] + popc64(L.mask[tw][e] & below);
}


// ---- router GEMM -------------------------------------------------------------
// MFMA of the router matmul: bf16 v_mfma_f32_32x32x16_bf16 (16 K per step,
// 8 per lane), fp32 v_mfma_f32_32x32x2_f32 (2 K per step, 1 per lane).
template <typename T> struct GateMma;
template <> struct GateMma<bf16_t> {
  static constexpr int KS = 16, EPL = 8;
  typedef bf16x8_t Frag;
  __device__ static Frag ld(const char *p) { return *reinterpret_cast<const bf16x8_t *>(p); }
  __device__ static f32x16_t mma(Frag a, Frag b, f32x16_t c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
  }
};
template <> struct GateMma<float> {
  static constexpr int KS = 2, EPL = 1;
  typedef float Frag;
  __device__ static Frag ld(const char *p) { return *reinterpret_cast<const float *>(p); }
  __device__ static f32x16_t mma(Frag a, Frag b, f32x16_t c) {
    return __builtin_amdgcn_mfma_f32_32x32x2f32(a, b, c, 0, 0, 0);
  }
};

constexpr int kGateRowBytes = 256;  // one K-slice of a row in LDS (preferred)
// Token tile of the split router GEMM, and the largest batch whose whole
// product may run in the one-workgroup routing kernel's prologue.  kGateSplitK:
// split over K-groups where it pays (gate_split), instead of computing a
// tile's whole product on one compute unit.
constexpr int kGateFusedTokens = 64;
constexpr bool kGateSplitK = true;

// Experts rounded up to the gate-row bucket the kernels are built for.
inline int gate_bucket(int e) { return e <= 32 ? 32 : e <= 64 ? 64 : e <= 128 ? 128 : 256; }
// Ring depth that fits `budget` LDS bytes with rows of rb bytes (at most 8).
constexpr int gate_stages(int nt, int epb, int budget, int rb) {
  return budget / ((nt + epb) * rb) < 8 ? budget / ((nt + epb) * rb) : 8;
}
// Row bytes of a tile: the preferred slice unless two stages of it do not fit.
constexpr int gate_row_bytes(int nt, int epb, int budget) {
  return gate_stages(nt, epb, budget, kGateRowBytes) >= 2 ? kGateRowBytes : 128;
}

// Byte offset of 16-byte chunk c of LDS row r.  A ds_read_b128 serves 16
// lanes at a time from 256 bytes of banks, i.e. from 256 / kGateRowBytes rows;
// XOR-ing the chunk with (r / (256 / kGateRowBytes)) % (kGateRowBytes / 16)
// puts the 16 lanes of a fragment read (16 consecutive rows, same chunk) in
// different bank groups.
template <int RB> __device__ __forceinline__ int gate_swz(int r, int c) {
  return r * RB + ((c ^ ((r / (256 / RB)) % (RB / 16))) << 4);
}

// logits[t][e] for tokens t in [tok0, min(tok0 + NT, N)) and the E <= EPB
// experts: sum over h of x[t][h] * wg[e][h] in fp32, rounded once to T.
// Every K-slice of RB bytes of the NT token rows and EPB gate rows (rows past
// N or E read as zero) goes from memory straight into an S-stage LDS ring with
// 16-byte DMA loads, issued S - 1 slices ahead by waves 0-3; every wave then
// multiplies 32x32 output blocks on MFMA (gate rows as the first operand, so a
// lane ends up holding one token and runs of 4 experts).  Uses S * (NT + EPB) *
// RB bytes of `lds` and ends with every thread past a barrier, the logits
// stored.  PART: only the K-slices [zb, ze) are summed and the fp32 sums are
// stored to part[(t - tok0) * E + e] instead.
template <typename T, int NT, int THREADS, int EPB, int S, int RB, bool PART = false>
__device__ __forceinline__ void gate_logits(const T *__restrict__ x, const T *__restrict__ wg,
                                            int64_t N, int H, int E, int64_t tok0,
                                            T *__restrict__ logits, char *lds, int zb = 0,
                                            int ze = -1, float *__restrict__ part = nullptr) {
  using Mm = GateMma<T>;
  constexpr int NW = THREADS / 64;
  constexpr int RS = NT + EPB;                 // LDS rows of one stage
  constexpr int STAGE = RS * RB;
  constexpr int NWI = 4;                       // waves issuing the DMA loads
  constexpr int CPR = RB / 16;                 // 16-byte chunks per row
  constexpr int RPI = 64 / CPR;                // rows per 1 KB load
  constexpr int PER = RS / RPI / NWI;          // 1 KB loads per issuing wave per slice
  static_assert(RS % (RPI * NWI) == 0 && NT % RPI == 0 && NW >= NWI, "loads per issuing wave");
  static_assert(S >= 2 && (S - 2) * PER < 64, "ring depth / vmcnt range");
  // 32x32 output blocks over the whole NT x EPB tile (rows past N or E hold
  // zeros and their results are not stored), dealt to the waves: block
  // b = wave + j * NW is token block b % TBS, expert block b / TBS.  A fixed
  // deal keeps the MFMA loop free of branches, so fragment reads overlap it.
  constexpr int TBS = NT / 32, NBS = TBS * (EPB / 32);
  constexpr int MAXB = (NBS + NW - 1) / NW;       // output blocks a wave
  constexpr bool SAME_TB = NW % TBS == 0;         // one token block per wave
  constexpr int KSTEPS = RB / (Mm::KS * (int)sizeof(T));
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int live = (int)min<int64_t>(NT, N - tok0);
  const int rowb = H * (int)sizeof(T);  // bytes of one x / gate row (a multiple of 16)
  if (ze < 0) ze = (rowb + RB - 1) / RB;
  const int nslice = ze - zb;  // slices of this call
  // buffer views: this chunk's token rows, and the gate weight
  const __amdgpu_buffer_rsrc_t rx = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<T *>(x) + tok0 * H, (short)0, live * rowb, kRsrcWord3);
  const __amdgpu_buffer_rsrc_t rw =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<T *>(wg), (short)0, E * rowb, kRsrcWord3);
  // per load j of this wave: RPI stage rows from RPI * i for i = wave * PER + j;
  // the lane fills physical chunk lane % CPR of row RPI * i + lane / CPR with
  // the logical chunk that the swizzle puts there
  uint32_t voff[PER], coff[PER];
#pragma unroll
  for (int j = 0; j < PER; ++j) {
    const int r = (wave * PER + j) * RPI + lane / CPR;
    const int c = (gate_swz<RB>(r, lane % CPR) - r * RB) >> 4;  // XOR is an involution
    coff[j] = (uint32_t)c * 16;
    const bool ok = r < NT ? r < live : r - NT < E;
    voff[j] = ok ? (uint32_t)(r < NT ? r : r - NT) * (uint32_t)rowb + coff[j] : kOOB;
  }
  auto issue = [&](int z) {
    const uint32_t kb = (uint32_t)(zb + z) * RB;
    const bool tail = (int)kb + RB > rowb;
    char *base = lds + (z % S) * STAGE;
#pragma unroll
    for (int j = 0; j < PER; ++j) {
      uint32_t off = voff[j] + kb;  // kOOB + kb stays out of range
      if (tail && (int)(kb + coff[j]) >= rowb) off = kOOB;
      dma16((wave * PER + j) * RPI < NT ? rx : rw, base + (wave * PER + j) * 1024, off);
    }
  };

  f32x16_t acc[MAXB];
#pragma unroll
  for (int j = 0; j < MAXB; ++j)
#pragma unroll
    for (int i = 0; i < 16; ++i) acc[j][i] = 0.f;
  const bool busy = wave < NBS;  // waves past the block count only load and wait
  if (wave < NWI) {
#pragma unroll
    for (int z = 0; z < S - 1; ++z)
      if (z < nslice) issue(z);
  }
  for (int z = 0; z < nslice; ++z) {
    if (wave < NWI) wait_pending<PER, 0, S - 2>(min(S - 2, nslice - 1 - z), false);
    barrier();  // slice z is in LDS for every wave; slot (z - 1) % S is free
    if (wave < NWI && z + S - 1 < nslice) issue(z + S - 1);
    const char *st = lds + (z % S) * STAGE;
    if (busy) {
#pragma unroll
      for (int ks = 0; ks < KSTEPS; ++ks) {
        const int bo = (ks * Mm::KS + (lane >> 5) * Mm::EPL) * (int)sizeof(T);
        typename Mm::Frag fa[MAXB], fx[MAXB];
#pragma unroll
        for (int j = 0; j < MAXB; ++j) {
          const int b = min(wave + j * NW, NBS - 1);  // a wave's spare blocks repeat its last
          const int ra = NT + (b / TBS) * 32 + (lane & 31);
          fa[j] = Mm::ld(st + gate_swz<RB>(ra, bo >> 4) + (bo & 15));
          if (!SAME_TB || j == 0) {
            const int rt = (b % TBS) * 32 + (lane & 31);
            fx[j] = Mm::ld(st + gate_swz<RB>(rt, bo >> 4) + (bo & 15));
          }
        }
#pragma unroll
        for (int j = 0; j < MAXB; ++j) acc[j] = Mm::mma(fa[j], fx[SAME_TB ? 0 : j], acc[j]);
      }
    }
  }
  // lane: token tb*32 + lane%32; register r: expert eb*32 + 8(r/4) + 4(lane/32) + r%4
#pragma unroll
  for (int j = 0; j < MAXB; ++j) {
    const int b = wave + j * NW;
    if (b < NBS) {
      const int tb = b % TBS, eb = b / TBS;
      const int64_t t = tok0 + tb * 32 + (lane & 31);
      if (t < N) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int e = eb * 32 + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
          if (e < E) {
            if constexpr (PART)
              part[(t - tok0) * E + e] = acc[j][r];
            else
              logits[t * E + e] = from_f32<T>(acc[j][r]);
          }
        }
      }
    }
  }
  __syncthreads();  // logits visible to the workgroup; the ring's LDS may be reused
}

// Router GEMM split over K for batches of up to kGateSplitTokens: workgroup
// (z, y) sums K-group z (g consecutive K-slices) of token tile y
// (kGateFusedTokens tokens) over all experts and stores the fp32 sums to
// part[(z * N + t) * E + e] (group-major: a workgroup writes whole rows, and a
// group's sums of consecutive logits are adjacent); gate_reduce or the routing
// kernel adds them up.  The gate weight is then
// read by about kGateSplitWGs compute units at once, each with a ring of slices
// in flight, instead of by one workgroup per token tile.
constexpr int kGateMaxParts = 256;  // more K-slices than this: no split over K
constexpr int64_t kGateSplitTokens = 4096;
constexpr int kGateSplitWGs = 256;
// Past one token tile, a row of fewer K-slices than this does not gain from
// the split (the extra reduction launch costs more: E = 8, H = 512, 4096
// tokens 14.1 -> 15.4 us).
constexpr int kGateSplitMinSlices = 8;
// Split-K sums up to this many bytes are added up in the routing kernel's
// prologue; more take a reduction kernel of their own first.
constexpr int64_t kGateSumInlineBytes = 32 * 1024;
template <typename T, int EPB>
__global__ __launch_bounds__(256) void gate_partial(const T *__restrict__ x,
                                                    const T *__restrict__ wg, int64_t N, int H,
                                                    int E, float *__restrict__ part, int g);

// Logit i of the split-K router GEMM: its nparts K-group sums (group z at
// part[z * ne + i]) added in group order from zero in fp32 (rounded by the
// caller).  The loads of 32 groups are all issued before their additions (a
// wider round costs more in cold instruction-cache misses than it saves).
__device__ __forceinline__ float gate_group_sum(const float *__restrict__ part, int64_t i,
                                                int64_t ne, int nparts) {
  constexpr int Z = 32;
  float acc = 0.f;
  for (int z0 = 0; z0 < nparts; z0 += Z) {
    float v[Z];
#pragma unroll
    for (int u = 0; u < Z; ++u) v[u] = z0 + u < nparts ? part[(z0 + u) * ne + i] : 0.f;
#pragma unroll
    for (int u = 0; u < Z; ++u)
      if (z0 + u < nparts) acc += v[u];
  }
  return acc;
}

// The split-K sums of ne logits added up over many workgroups, one logit a
// thread, when there are too many for the routing kernel's prologue (a single
// workgroup) to read quickly.
constexpr int kGateReduceThreads = 256;
template <typename T>
__global__ __launch_bounds__(kGateReduceThreads) void gate_reduce(const float *__restrict__ part,
                                                                  int64_t ne, int nparts,
                                                                  T *__restrict__ logits) {
  const int64_t i = (int64_t)blockIdx.x * kGateReduceThreads + threadIdx.x;
  if (i < ne) logits[i] = from_f32<T>(gate_group_sum(part, i, ne, nparts));
}

// Router GEMM alone: one workgroup of 256 threads per NT tokens, all experts.
constexpr int kGateThreads = 256;
constexpr int kGateLdsBudget = 150 * 1024;
template <typename T, int NT, int EPB>
__global__ __launch_bounds__(kGateThreads) void gate_gemm(const T *__restrict__ x,
                                                          const T *__restrict__ wg, int64_t N,
                                                          int H, int E, T *__restrict__ logits) {
  constexpr int RB = gate_row_bytes(NT, EPB, kGateLdsBudget);
  constexpr int S = gate_stages(NT, EPB, kGateLdsBudget, RB);
  __shared__ __align__(16) char lds[S * (NT + EPB) * RB];
  gate_logits<T, NT, kGateThreads, EPB, S, RB>(x, wg, N, H, E, (int64_t)blockIdx.x * NT, logits,
                                               lds);
}

// Row bytes of the split-K router GEMM's slices, and the number of slices of a
// row of rowb bytes.
constexpr int gate_part_rb(int epb) { return gate_row_bytes(kGateFusedTokens, epb, kGateLdsBudget); }
inline int gate_parts(int e, int rowb) {
  const int rb = gate_part_rb(gate_bucket(e));
  return (rowb + rb - 1) / rb;
}
// Whether the router GEMM of n tokens with rows of nsl K-slices splits over K.
inline bool gate_split(int64_t n, int nsl) {
  return kGateSplitK && nsl <= kGateMaxParts &&
         (n <= kGateFusedTokens || (n <= kGateSplitTokens && nsl >= kGateSplitMinSlices));
}
// K-groups for N tokens and nsl slices: about kGateSplitWGs workgroups over the
// token tiles, each group the same whole number of slices (the last one fewer);
// a batch of one tile gets one slice a group.
inline int gate_groups(int64_t n, int nsl) {
  const int64_t tiles = (n + kGateFusedTokens - 1) / kGateFusedTokens;
  if (tiles <= 1) return nsl;  // (an empty batch included)
  const int ng = (int)std::min<int64_t>(nsl, (kGateSplitWGs + tiles - 1) / tiles);
  const int g = (nsl + ng - 1) / ng;
  return (nsl + g - 1) / g;
}
template <typename T, int EPB>
__global__ __launch_bounds__(256) void gate_partial(const T *__restrict__ x,
                                                    const T *__restrict__ wg, int64_t N, int H,
                                                    int E, float *__restrict__ part, int g) {
  constexpr int RB = gate_part_rb(EPB);
  constexpr int S = gate_stages(kGateFusedTokens, EPB, kGateLdsBudget, RB);
  __shared__ __align__(16) char lds[S * (kGateFusedTokens + EPB) * RB];
  const int z = blockIdx.x, nsl = (H * (int)sizeof(T) + RB - 1) / RB;
  const int64_t tok0 = (int64_t)blockIdx.y * kGateFusedTokens;
  gate_logits<T, kGateFusedTokens, kGateThreads, EPB, S, RB, true>(
      x, wg, N, H, E, tok0, nullptr, lds, z * g, min(z * g + g, nsl), part + (z * N + tok0) * E);
}

// Batches of at most NT tokens: one workgroup, one launch.  Every per-entry
// value stays in LDS; the scan and the scatter follow the rank phase directly.
// GATE: the logits are first computed from x and the gate weight (router GEMM
// prologue) and stored to `logits`, which the top-k phase then reads.
// (The logits pointer carries no __restrict__: with GATE the same buffer is
// written through logits_out first.)  With GATE the GEMM's LDS ring and the
// routing phases' LDS share one buffer: the ring is dead once the logits are
// stored.
constexpr int kFusedGateRing = 140 * 1024;
// GATE: 0 logits given; 1 router GEMM in the prologue; 2 the prologue adds up
// the K-group sums of gate_partial (nparts groups) into the logits.
template <typename T, int THREADS, int C, typename Lds, int GATE = 0, int EPB = 32>
__global__ __launch_bounds__(THREADS) void route_fused(
    const T *logits, int64_t N, int E, int K, int lo, int nl, int logG, int vec,
    int32_t *__restrict__ topk_idx, T *__restrict__ topk_w, uint32_t *__restrict__ bitmatrix,
    int32_t *__restrict__ col_sum, int32_t *__restrict__ offsets,
    int32_t *__restrict__ col_sorted, int32_t *__restrict__ row_sorted,
    T *__restrict__ gate_scal, const T *__restrict__ x = nullptr, const T *__restrict__ wg = nullptr,
    int H = 0, T *logits_out = nullptr, const float *__restrict__ part = nullptr,
    int nparts = 0) {
  constexpr int NT = Lds::kTokens;
  constexpr int GRB = gate_row_bytes(kGateFusedTokens, EPB, kFusedGateRing);
  constexpr int GS = gate_stages(kGateFusedTokens, EPB, kFusedGateRing, GRB);
  constexpr int RING = GATE == 1 ? GS * (kGateFusedTokens + EPB) * GRB : 0;
  constexpr int RAW = RING > (int)sizeof(Lds) ? RING : (int)sizeof(Lds);
  __shared__ __align__(16) char s_raw[RAW];
  Lds &L = *reinterpret_cast<Lds *>(s_raw);
  __shared__ uint16_t s_rank[NT * Lds::kSlots];
  __shared__ int s_off[Lds::kExperts + 1];
  const int tid = threadIdx.x;
  if constexpr (GATE == 1)  // N <= kGateFusedTokens
    gate_logits<T, kGateFusedTokens, THREADS, EPB, GS, GRB>(x, wg, N, H, E, 0, logits_out, s_raw);
  if constexpr (GATE == 2) {  // groups summed in order, rounded once
    const int ne = (int)N * E;
    for (int i = tid; i < ne; i += THREADS)
      logits_out[i] = from_f32<T>(gate_group_sum(part, i, ne, nparts));
    __syncthreads();
  }
  topk_chunk<T, THREADS, C>(logits, N, E, K, lo, nl, logG, vec, 0, topk_idx, topk_w, bitmatrix,
                            L);
  __syncthreads();
  rank_chunk<THREADS>(nl, (int)N, L);
  const int M = (int)N * K;
  // in-chunk ranks, one entry a thread on waves 1.., while wave 0 scans the
  // chunk totals into offsets
  if (tid >= 64) {
    for (int f = tid - 64; f < M; f += THREADS - 64) {
      const int l = (int)L.sel[f] - lo;
      if ((unsigned)l < (unsigned)nl) s_rank[f] = (uint16_t)chunk_rank(L, f / K, l);
    }
  }
  block_exclusive_scan(L.tot, s_off, nl);  // synchronises
  for (int e = tid; e <= nl; e += THREADS) {
    offsets[e] = s_off[e];
    if (e < nl) col_sum[e] = L.tot[e];
  }
  const int m_local = s_off[nl];
  for (int f = tid; f < M; f += THREADS) {
    const int l = (int)L.sel[f] - lo;
    if ((unsigned)l < (unsigned)nl) {
      const int p = s_off[l] + s_rank[f];
      col_sorted[p] = f;
      row_sorted[f] = p;
      gate_scal[p] = L.w[f];
    } else {
      row_sorted[f] = -1;
    }
  }
  for (int p = m_local + tid; p < M; p += THREADS) {
    col_sorted[p] = -1;
    gate_scal[p] = from_f32<T>(0.f);
  }
}

// Router GEMM of NT <= kGateGemvTokens tokens: a wave per expert row computes
// logits[t][e] = sum_h x[t][h] w[e][h] in fp32 -- each lane its 16-byte pieces
// h in [V (lane + 64 c), V (lane + 64 c + 1)), the weight piece loaded once
// for all NT tokens, multiply-adds in element order, then a butterfly sum over
// the wave -- rounded once.  The logits go straight to the routing kernel, with
// no partial sums in between.
constexpr int kGateGemvWaves = 4, kGateGemvTokens = 4;
template <typename T, int NT>
__global__ __launch_bounds__(64 * kGateGemvWaves) void gate_gemv(const T *__restrict__ x,
                                                                 const T *__restrict__ wg, int H,
                                                                 int E, T *__restrict__ logits) {
  constexpr int V = 16 / (int)sizeof(T);  // values a 16-byte piece
  constexpr int PW = 4 / (int)sizeof(T);  // values a dword
  const int lane = threadIdx.x & 63;
  const int e = (int)blockIdx.x * kGateGemvWaves + (int)(threadIdx.x >> 6);
  if (e >= E) return;  // whole waves
  const int npc = H / V;  // pieces of a row (H a multiple of 8)
  const u32x4_t *wr = reinterpret_cast<const u32x4_t *>(wg + (size_t)e * H);
  // the loads of kBatch pieces a lane go out before their multiply-adds
  constexpr int kBatch = NT == 1 ? 8 : 4;
  float acc[NT];
#pragma unroll
  for (int t = 0; t < NT; ++t) acc[t] = 0.f;
  for (int c0 = lane; c0 < npc; c0 += 64 * kBatch) {
    u32x4_t a[NT][kBatch], b[kBatch];
#pragma unroll
    for (int u = 0; u < kBatch; ++u) {
      const int c = c0 + 64 * u;
#pragma unroll
      for (int t = 0; t < NT; ++t)
        a[t][u] = c < npc ? reinterpret_cast<const u32x4_t *>(x + (size_t)t * H)[c]
                          : u32x4_t{0u, 0u, 0u, 0u};
      b[u] = c < npc ? wr[c] : u32x4_t{0u, 0u, 0u, 0u};
    }
#pragma unroll
    for (int u = 0; u < kBatch; ++u) {
      if (c0 + 64 * u >= npc) break;
#pragma unroll
      for (int i = 0; i < V; ++i) {
        const uint32_t sh = 32 / PW * (i % PW);
        float wb;
        if constexpr (sizeof(T) == 2)
          wb = __uint_as_float(((b[u][i / PW] >> sh) & 0xffffu) << 16);
        else
          wb = __uint_as_float(b[u][i]);
#pragma unroll
        for (int t = 0; t < NT; ++t) {
          float xa;
          if constexpr (sizeof(T) == 2)
            xa = __uint_as_float(((a[t][u][i / PW] >> sh) & 0xffffu) << 16);
          else
            xa = __uint_as_float(a[t][u][i]);
          acc[t] = fmaf(xa, wb, acc[t]);
        }
      }
    }
  }
#pragma unroll
  for (int t = 0; t < NT; ++t) {
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) acc[t] += __shfl_xor(acc[t], m);
    if (lane == 0) logits[(size_t)t * E + e] = from_f32<T>(acc[t]);
  }
}

// One token: a single wave runs the whole routing step in registers, with no
// workgroup barrier.  Lane l holds the 16-byte logit chunk of experts
// [l V, l V + V); k rounds of a wave-wide key maximum select the experts (the
// keys and tie rule of topk_chunk, so the same choices), and the softmax adds
// up the same terms in the same slot order.  With at most one entry per expert,
// an entry's sorted position and every offset are prefix popcounts of the
// selected-expert mask, whose bitmatrix word w lane w holds.
template <typename T>
__global__ __launch_bounds__(64) void route_one(
    const T *logits, int E, int K, int lo, int nl, int vec, int32_t *__restrict__ topk_idx,
    T *__restrict__ topk_w, uint32_t *__restrict__ bitmatrix, int32_t *__restrict__ col_sum,
    int32_t *__restrict__ offsets, int32_t *__restrict__ col_sorted,
    int32_t *__restrict__ row_sorted, T *__restrict__ gate_scal) {
  using Lg = Logit<T>;
  using Key = typename Lg::Key;
  constexpr int V = Lg::kVec;
  const int lane = threadIdx.x, e0 = lane * V;
  u32x4_t raw = {0u, 0u, 0u, 0u};
  if (e0 < E) raw = fetch16(logits, e0, E, vec != 0);
  Key key[V];
  Lg::decode(raw, e0, E, key);
  int my_e = -1;  // lane j: slot j's expert and logit
  float my_v = 0.f, vmax = 0.f, ssum = 0.f;
  uint32_t word = 0;  // lane w: bitmatrix word w (local expert ids)
  for (int j = 0; j < K; ++j) {
    Key m = key[0];
#pragma unroll
    for (int i = 1; i < V; ++i) m = kmax(m, key[i]);
    m = group_max(m, 64);
    const int e = Lg::expert(m);
    const float v = Lg::value(m);
#pragma unroll
    for (int i = 0; i < V; ++i)
      if (e0 + i == e) key[i] = 0;  // only the owning lane matches
    if (j == 0) vmax = v;           // slot 0 holds the maximum
    ssum += expf(v - vmax);
    if (lane == j) {
      my_e = e;
      my_v = v;
    }
    const int l = e - lo;
    if ((unsigned)l < (unsigned)nl && (l >> 5) == lane) word |= 1u << (l & 31);
  }
  // selected local experts below local id x (x <= nl <= kMaxExperts): the
  // popcount prefix of the words before x / 32 plus the bits of that word below
  // x.  Shuffles: every lane calls this with the same trip count.
  const int pc = __popc(word), excl = wave_inclusive_sum(pc) - pc;
  auto below = [&](int x, uint32_t &w) {
    w = (uint32_t)__shfl((int)word, x >> 5);
    return __shfl(excl, x >> 5) + __popc(w & ((1u << (x & 31)) - 1u));
  };
  for (int x0 = 0; x0 <= kMaxExperts; x0 += 64) {
    const int x = x0 + lane;
    uint32_t w;
    const int r = below(min(x, nl), w);
    if (x <= nl) offsets[x] = r;
    if (x < nl) col_sum[x] = (w >> (x & 31)) & 1u;
  }
  const int words = (nl + 31) >> 5;
  if (lane < words) bitmatrix[lane] = word;
  const int l = my_e - lo;
  const bool local = lane < K && (unsigned)l < (unsigned)nl;
  uint32_t w;
  const int p = below(local ? l : 0, w);
  uint32_t wn;
  const int m_local = below(nl, wn);
  if (lane < K) {
    const T wt = from_f32<T>(expf(my_v - vmax) / ssum);
    topk_idx[lane] = my_e;
    topk_w[lane] = wt;
    if (local) {
      col_sorted[p] = lane;
      row_sorted[lane] = p;
      gate_scal[p] = wt;
    } else {
      row_sorted[lane] = -1;
    }
    if (lane >= m_local) {  // positions no local entry fills
      col_sorted[lane] = -1;
      gate_scal[lane] = from_f32<T>(0.f);
    }
  }
}

// Multi-block path, kernel 1: one chunk of NTB tokens per workgroup (64 or 256);
// per-block expert counts and per-entry in-block ranks to the workspace.
// THREADS: 1024, or 256 for 64-token blocks of few experts.
constexpr int kTopkThreads = 1024;

template <typename T, int C, int NTB, int THREADS = kTopkThreads>
__global__ __launch_bounds__(THREADS) void route_topk_rank(
    const T *__restrict__ logits, int64_t N, int E, int K, int lo, int nl, int logG, int vec,
    int32_t *__restrict__ topk_idx, T *__restrict__ topk_w, uint32_t *__restrict__ bitmatrix,
    int32_t *__restrict__ blk_cnt, int nbp, uint8_t *__restrict__ blk_rank) {
  __shared__ ChunkLds<T, NTB> L;
  const int tid = threadIdx.x;
  const int64_t tok0 = (int64_t)blockIdx.x * NTB;
  topk_chunk<T, THREADS, C>(logits, N, E, K, lo, nl, logG, vec, tok0, topk_idx, topk_w,
                                 bitmatrix, L);
  __syncthreads();
  rank_chunk<THREADS>(nl, (int)min<int64_t>(NTB, N - tok0), L);
  const int64_t t = tok0 + tid;
  if (tid < NTB && t < N) {
#pragma unroll
    for (int j = 0; j < kMaxTopk; ++j) {
      if (j < K) {
        // slots outside the share get rank 0; the scatter never places them
        const int l = (int)L.sel[tid * K + j] - lo;
        blk_rank[t * K + j] = (unsigned)l < (unsigned)nl ? (uint8_t)chunk_rank(L, tid, l) : 0;
      }
    }
  }
  // expert-major, row stride nbp (a multiple of 4): the scatter sums rows
  for (int e = tid; e < nl; e += THREADS) blk_cnt[(int64_t)e * nbp + blockIdx.x] = L.tot[e];
}

// Multi-block path, kernel 2: workgroup b scatters routing block b.  It sums
// the per-block counts (expert-major rows of nbp ints: totals over all blocks
// and the prefix over the blocks before b) with 16-byte loads spread over all
// threads, scans the totals into offsets (workgroup 0 writes col_sum /
// offsets), and places every entry of its block at offsets[e] + (entries of e
// in earlier blocks) + rank in the block.
constexpr int kScatterThreads = 1024;

// PRE: route_count_scan has already turned the count rows into exclusive
// prefixes over the blocks and written the totals to tot, so the workgroup
// reads its own column and the totals (linear in the number of blocks
// overall) instead of summing the rows (quadratic).
template <typename T, int NTB, bool PRE = false>
__global__ __launch_bounds__(kScatterThreads) void route_scatter(
    int64_t N, int K, int lo, int nl, int nblocks, int nbp, const int32_t *__restrict__ blk_cnt,
    const int32_t *__restrict__ tot, const uint8_t *__restrict__ blk_rank,
    const int32_t *__restrict__ topk_idx,
    const T *__restrict__ topk_w, int32_t *__restrict__ col_sum, int32_t *__restrict__ offsets,
    int32_t *__restrict__ col_sorted, int32_t *__restrict__ row_sorted,
    T *__restrict__ gate_scal) {
  constexpr int kParts = kScatterThreads / 32;  // at most this many threads per expert
  __shared__ int s_tot[kMaxExperts];
  __shared__ int s_base[kMaxExperts];
  __shared__ int s_off[kMaxExperts + 1];
  __shared__ int s_pre[kParts][kMaxExperts];
  __shared__ int s_all[kParts][kMaxExperts];
  const int tid = threadIdx.x;
  const int b = blockIdx.x;
  // the block's entries: token t = b * NTB + tid, slots 0..K-1.  They do not
  // depend on the counts, so their loads go out first and overlap the sums.
  const int64_t t = (int64_t)b * NTB + tid;
  const bool own = tid < NTB && t < N;
  int ex[kMaxTopk], rk[kMaxTopk];
  T w[kMaxTopk];
  if (own) {
#pragma unroll
    for (int j = 0; j < kMaxTopk; ++j) {
      if (j < K) {
        ex[j] = topk_idx[t * K + j] - lo;  // local id; outside the share if not in [0, nl)
        rk[j] = blk_rank[t * K + j];
        w[j] = topk_w[t * K + j];
      }
    }
  }
  const int E = nl;  // counts, offsets and positions are over the local experts
  if constexpr (PRE) {
    for (int x = tid; x < E; x += kScatterThreads) {
      s_base[x] = blk_cnt[(int64_t)x * nbp + b];
      s_tot[x] = tot[x];
    }
    __syncthreads();
  } else {
  // thread (e, part): part-th share of row e, in 4-int chunks
  const int parts = min(kParts, kScatterThreads / E);
  const int e = tid % E, part = tid / E;
  const int nch = nbp / 4;                       // 16-byte chunks per row
  const int per = (nch + parts - 1) / parts;
  if (part < parts) {
    int pre = 0, all = 0;
    const u32x4_t *row = reinterpret_cast<const u32x4_t *>(blk_cnt + (int64_t)e * nbp);
    constexpr int U = 4;
    for (int c0 = part * per; c0 < min(nch, (part + 1) * per); c0 += U) {
      u32x4_t v[U];
#pragma unroll
      for (int u = 0; u < U; ++u)
        v[u] = (c0 + u < min(nch, (part + 1) * per)) ? row[c0 + u] : u32x4_t{0u, 0u, 0u, 0u};
#pragma unroll
      for (int u = 0; u < U; ++u)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int bb = (c0 + u) * 4 + q;  // block index; entries past nblocks are padding
          const int c = bb < nblocks ? (int)v[u][q] : 0;
          all += c;
          if (bb < b) pre += c;
        }
    }
    s_pre[part][e] = pre;
    s_all[part][e] = all;
  }
  __syncthreads();
  for (int x = tid; x < E; x += kScatterThreads) {
    int pre = 0, all = 0;
    for (int q = 0; q < parts; ++q) {
      pre += s_pre[q][x];
      all += s_all[q][x];
    }
    s_base[x] = pre;
    s_tot[x] = all;
  }
  __syncthreads();
  }
  block_exclusive_scan(s_tot, s_off, E);
  if (b == 0) {
    for (int x = tid; x <= E; x += kScatterThreads) {
      offsets[x] = s_off[x];
      if (x < E) col_sum[x] = s_tot[x];
    }
  }
  for (int x = tid; x < E; x += kScatterThreads) s_base[x] += s_off[x];
  __syncthreads();
  if (own) {
#pragma unroll
    for (int j = 0; j < kMaxTopk; ++j) {
      if (j < K) {
        if ((unsigned)ex[j] < (unsigned)E) {
          const int p = s_base[ex[j]] + rk[j];
          col_sorted[p] = (int32_t)(t * K + j);
          row_sorted[t * K + j] = p;
          gate_scal[p] = w[j];
        } else {
          row_sorted[t * K + j] = -1;
        }
      }
    }
  }
  // sorted positions past the local entries: this block clears its share of
  // [m_local, N*K), the positions [b*NTB*K, (b+1)*NTB*K)
  const int64_t M = N * K, m_local = s_off[E];
  const int64_t p_end = min(M, ((int64_t)b + 1) * NTB * K);
  for (int64_t p = max(m_local, (int64_t)b * NTB * K) + tid; p < p_end;
       p += kScatterThreads) {
    col_sorted[p] = -1;
    gate_scal[p] = from_f32<T>(0.f);
  }
}

// ---- Large batches of bf16 logits: one lane per token ------------------------
// Each lane runs the whole top-k of its token.  A bf16 logit becomes a signed
// order key: the two's complement of its sign-magnitude bits (so -0 and +0 are
// the same value) in the high half, the inverted expert index in the low half,
// so keys order by value and then by lower expert index (the same order, and
// so the same choices, as the unsigned keys of topk_chunk).  Keys are unique,
// and the lane keeps its best L as a sorted list t[0] > t[1] > ... > t[L-1]
// into which each key x enters as t'[0] = max(t[0], x), t'[j] = med3(t[j-1],
// t[j], x): one max and L - 1 median-of-three instructions a key, all from the
// old list.  Three kernels:
//  * route_lane_topk: 64-token blocks (one wave each, four a workgroup): top-k,
//    softmax, topk_idx / topk_w / bitmatrix rows; then each token ORs its bit
//    into an LDS mask per chosen local expert, whose popcount is the block's
//    count (stored expert-major) and whose popcount below a lane is that
//    entry's stable rank in the block.
//  * route_count_scan: one wave per expert turns its row of block counts into
//    exclusive prefixes over the blocks (linear in the number of blocks) and
//    stores the expert's total.
//  * route_lane_scatter: per block, the totals' exclusive scan gives the
//    offsets; an entry goes to offsets[e] + (entries of e in earlier blocks) +
//    its rank.  No atomics: every run gives the same result.
constexpr int kLaneBlock = 64;   // tokens of a routing block (one wave)
constexpr int kLaneWaves = 4;    // blocks (waves) of a workgroup
constexpr int kLaneMaxWords = (kMaxExperts + 31) / 32;

__device__ __forceinline__ int key_med3(int a, int b, int c) {
  return max(min(a, b), min(max(a, b), c));  // v_med3_i32
}

// Keys of the 8 logits of a 16-byte chunk (experts e0 .. e0 + 7) inserted in
// the sorted list t; values past E are skipped.
template <int L, bool FULL>
__device__ __forceinline__ void lane_insert_chunk(int (&t)[L], u32x4_t v, int e0, int E) {
  typedef short s16x2 __attribute__((ext_vector_type(2)));
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    // the element goes through a scalar first: hipcc miscompiles a bit_cast of
    // an ext_vector element (every i read element 0)
    const uint32_t wi = v[i];
    const s16x2 h = __builtin_bit_cast(s16x2, wi);
    const s16x2 m = h >> (s16x2){15, 15};
    const s16x2 tt = ((h & (s16x2){0x7fff, 0x7fff}) ^ m) - m;  // signed value order, -0 == +0
    const uint32_t u = __builtin_bit_cast(uint32_t, tt);
    const int e = e0 + 2 * i;
    const int kk[2] = {(int)((u << 16) | (uint32_t)(0xffff - e)),
                       (int)((u & 0xffff0000u) | (uint32_t)(0xffff - e - 1))};
#pragma unroll
    for (int q = 0; q < 2; ++q) {
      if (FULL || e + q < E) {
        const int x = kk[q];
        int n[L];
        n[0] = max(t[0], x);
#pragma unroll
        for (int j = 1; j < L; ++j) n[j] = key_med3(t[j - 1], t[j], x);
#pragma unroll
        for (int j = 0; j < L; ++j) t[j] = n[j];
      }
    }
  }
}

__device__ __forceinline__ int lane_key_expert(int k) { return 0xffff - (k & 0xffff); }
__device__ __forceinline__ float lane_key_value(int k) {
  const int tv = k >> 16;  // signed value order
  const uint32_t bits = tv < 0 ? ((uint32_t)(-tv) | 0x8000u) : (uint32_t)tv;
  return __uint_as_float(bits << 16);
}

// Logits of a block in LDS with fewer than 8 chunks a row (CH = 2^lch): token
// t's 16-byte chunk c sits in slot t * CH + (c + rot(t)) % CH, rot(t) =
// t / (16 / CH), so the 16 lanes of a ds_read_b128 (16 tokens, one chunk each)
// hit 16 distinct bank groups.
__device__ __forceinline__ int lane_rot(int t, int lch) { return t >> (4 - lch); }

// Logits of a block with 8 or more chunks a row sit in phases of 8 chunks
// (64 experts): phase h holds chunks 8h + [0, 8) of all 64 tokens, token t's
// chunk 8h + c in slot 512 h + 8 t + (c + t / 2) % 8.  A load instruction
// fills 64 slots, 8 tokens' whole 128-byte pieces (fully coalesced), so phase
// h arrives with loads 8h .. 8h + 7, and its keys are ranked while the later
// phases are in flight.  16 lanes of a ds_read_b128 (16 tokens, one chunk)
// hit 16 distinct bank groups: 8 (t % 2) + (c + t / 2) % 8.
template <int N> __device__ __forceinline__ void wait_lds_loads() {
  wait_vm<N>();
  asm volatile("" ::: "memory");  // no LDS read moves above the wait
  __builtin_amdgcn_wave_barrier();
}
// wait until at most 8 r of this wave's loads are outstanding (r < 4)
__device__ __forceinline__ void wait_phases(int r) {
  if (r >= 3) wait_lds_loads<24>();
  else if (r == 2) wait_lds_loads<16>();
  else if (r == 1) wait_lds_loads<8>();
  else wait_lds_loads<0>();
}

// NB bytes (a power of two, 2 - 64) from w to p, p aligned to min(NB, 16):
// 16-byte stores, or one of 8, 4 or 2 bytes.
template <int NB, typename P>
__device__ __forceinline__ void store_bytes(P *p, const uint32_t *w) {
  typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));
  char *c = reinterpret_cast<char *>(p);
  if constexpr (NB >= 16) {
#pragma unroll
    for (int i = 0; i < NB / 16; ++i)
      *reinterpret_cast<u32x4_t *>(c + 16 * i) = u32x4_t{w[4 * i], w[4 * i + 1], w[4 * i + 2],
                                                          w[4 * i + 3]};
  } else if constexpr (NB == 8) {
    *reinterpret_cast<u32x2_t *>(c) = u32x2_t{w[0], w[1]};
  } else if constexpr (NB == 4) {
    *reinterpret_cast<uint32_t *>(c) = w[0];
  } else {
    static_assert(NB == 2, "bytes");
    *reinterpret_cast<uint16_t *>(c) = (uint16_t)w[0];
  }
}
__device__ __forceinline__ bool aligned_to(const void *p, int n) {
  return ((uintptr_t)p & (uintptr_t)(n - 1)) == 0;
}

// L: list length, a power of two >= topk.  One wave per 64-token block b.
// E is a power of two from 8 (whole 16-byte chunks, 2^lch a row); the
// block's rows are copied to LDS with direct-to-LDS loads, fully coalesced,
// then each lane reads its own row from there, a phase at a time from 64
// experts a row.  A token's outputs are written as whole vectors where K = L
// (phases and vector stores: 65536 tokens, 128 experts, top-4 19.6 -> 18.5 us;
// 256 experts, top-8 35.3 -> 30.6 us).
template <int L>
__global__ __launch_bounds__(64 * kLaneWaves) void route_lane_topk(
    const bf16_t *__restrict__ logits, int64_t N, int E, int lch, int K, int lo, int nl,
    int32_t *__restrict__ topk_idx, bf16_t *__restrict__ topk_w,
    uint32_t *__restrict__ bitmatrix, int32_t *__restrict__ blk_cnt, int nbp,
    uint8_t *__restrict__ blk_rank) {
  extern __shared__ __attribute__((aligned(16))) char s_rows[];  // kLaneWaves * 64 * E * 2 bytes
  __shared__ unsigned long long s_mask[kLaneWaves][kMaxExperts];
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int64_t b = (int64_t)blockIdx.x * kLaneWaves + wave;
  const int64_t tok0 = b * kLaneBlock;
  if (tok0 >= N) return;  // whole wave: no token of this block exists
  const int64_t t = tok0 + lane;
  const bool live = t < N;
  const int ch = 1 << lch;                           // 16-byte chunks a row (E / 8)
  const int rowb = E * 2;
  char *rows = s_rows + wave * kLaneBlock * rowb;
  {
    // DMA instruction i fills LDS slots [64 i, 64 i + 64); lane l fetches the
    // chunk that belongs in slot 64 i + l.  Tokens past N read zeros.
    const int ntok = (int)min<int64_t>(kLaneBlock, N - tok0);
    const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<bf16_t *>(logits + tok0 * E), (short)0, ntok * rowb, kRsrcWord3);
    for (int i = 0; i < ch; ++i) {
      int tt, c;
      if (lch >= 3) {  // phases of 8 chunks
        const int sl = (i & 7) * 64 + lane;
        tt = sl >> 3;
        c = (i & ~7) + (((sl & 7) - (tt >> 1)) & 7);
      } else {
        const int slot = i * 64 + lane, pos = slot & (ch - 1);
        tt = slot >> lch;
        c = (pos - lane_rot(tt, lch)) & (ch - 1);
      }
      const uint32_t off = tt < ntok ? (uint32_t)(tt * rowb + c * 16) : kOOB;
      dma16(rs, rows + i * 1024, off);
    }
  }
  int key[L];
#pragma unroll
  for (int j = 0; j < L; ++j) key[j] = (int)0x80000000;  // below every real key: no-ops
  if (lch >= 3) {
    // each wave reads only its own rows: its own loads' waits suffice
    const char *mine = rows + lane * 128;
    const int rot = (lane >> 1) & 7;
    for (int h = 0; h < (ch >> 3); ++h) {
      wait_phases((ch >> 3) - 1 - h);
      if (live) {
        u32x4_t raw[8];
#pragma unroll
        for (int c = 0; c < 8; ++c)
          raw[c] = *reinterpret_cast<const u32x4_t *>(mine + h * 8192 + ((c + rot) & 7) * 16);
#pragma unroll
        for (int c = 0; c < 8; ++c) lane_insert_chunk<L, true>(key, raw[c], (8 * h + c) * 8, E);
      }
    }
  } else {
    wait_lds_loads<0>();
    if (live) {
      const char *myrow = rows + lane * rowb;
      const int rot = lane_rot(lane, lch);
      u32x4_t raw[4];
#pragma unroll
      for (int c = 0; c < 4; ++c)
        if (c < ch) raw[c] = *reinterpret_cast<const u32x4_t *>(myrow + ((c + rot) & (ch - 1)) * 16);
#pragma unroll
      for (int c = 0; c < 4; ++c)
        if (c < ch) lane_insert_chunk<L, true>(key, raw[c], c * 8, E);
    }
  }
  // softmax over the selected logits in slot order (the arithmetic of
  // topk_chunk, so the same weights), outputs, bitmatrix words over local ids
  const int words = (nl + 31) >> 5;
  uint32_t word[kLaneMaxWords];
#pragma unroll
  for (int w = 0; w < kLaneMaxWords; ++w) word[w] = 0u;
  int sel[L];
  // K == L: a token's outputs go out as whole vectors (their offsets are
  // multiples of their sizes; the bases are checked)
  const bool vk = K == L && aligned_to(topk_idx, min(4 * L, 16)) &&
                  aligned_to(topk_w, min(2 * L, 16)) && aligned_to(blk_rank, min(L, 16));
  const bool vw = (words & (words - 1)) == 0 && aligned_to(bitmatrix, min(4 * words, 16));
  if (live) {
    const float vmax = lane_key_value(key[0]);
    float ssum = 0.f;
#pragma unroll
    for (int j = 0; j < L; ++j)
      if (j < K) ssum += expf(lane_key_value(key[j]) - vmax);
    uint32_t wi[L], ww[L / 2];
#pragma unroll
    for (int j = 0; j < L; ++j) {
      sel[j] = lane_key_expert(key[j]);
      if (j < K) {
        const bf16_t wj = from_f32<bf16_t>(expf(lane_key_value(key[j]) - vmax) / ssum);
        wi[j] = (uint32_t)sel[j];
        const uint32_t wb = (uint32_t)__builtin_bit_cast(uint16_t, wj);
        if (j & 1) ww[j / 2] |= wb << 16;
        else ww[j / 2] = wb;
        if (!vk) {
          topk_idx[t * K + j] = sel[j];
          topk_w[t * K + j] = wj;
        }
        const int l = sel[j] - lo;
        if ((unsigned)l < (unsigned)nl) {
#pragma unroll
          for (int w = 0; w < kLaneMaxWords; ++w)
            if ((l >> 5) == w) word[w] |= 1u << (l & 31);
        }
      }
    }
    if (vk) {
      store_bytes<4 * L>(topk_idx + t * L, wi);
      store_bytes<2 * L>(topk_w + t * L, ww);
    }
    if (vw && words == 4) store_bytes<16>(bitmatrix + t * 4, word);
    else if (vw && words == 8) store_bytes<32>(bitmatrix + t * 8, word);
    else if (vw && words == 2) store_bytes<8>(bitmatrix + t * 2, word);
    else {
#pragma unroll
      for (int w = 0; w < kLaneMaxWords; ++w)
        if (w < words) bitmatrix[t * words + w] = word[w];
    }
  }
  // per local expert l: the mask of this block's tokens that chose it, built
  // in LDS by OR-ing each token's bit into the masks of the experts it chose
  // (OR does not depend on the order of the updates, so every run builds the
  // same masks); its popcount is the block's count, its popcount below a lane
  // that entry's stable rank
  auto wave_sync = [&]() {  // this wave's LDS operations done and visible to it
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  };
#pragma unroll
  for (int q = 0; q < kMaxExperts / 64; ++q) {
    const int l = q * 64 + lane;
    if (l < nl) s_mask[wave][l] = 0ull;
  }
  wave_sync();
  if (live) {
#pragma unroll
    for (int j = 0; j < L; ++j) {
      const int l = sel[j] - lo;
      if (j < K && (unsigned)l < (unsigned)nl) atomicOr(&s_mask[wave][l], 1ull << lane);
    }
  }
  wave_sync();
#pragma unroll
  for (int q = 0; q < kMaxExperts / 64; ++q) {
    const int l = q * 64 + lane;
    if (l < nl) blk_cnt[(int64_t)l * nbp + b] = popc64(s_mask[wave][l]);
  }
  if (live) {
    const unsigned long long below = lane ? (~0ull >> (64 - lane)) : 0ull;
    uint32_t rb[(L + 3) / 4];
#pragma unroll
    for (int j = 0; j < L; ++j) {
      if (j < K) {
        // slots outside the share get rank 0; the scatter never places them
        const int l = sel[j] - lo;
        const uint32_t r =
            (unsigned)l < (unsigned)nl ? (uint32_t)popc64(s_mask[wave][l] & below) : 0u;
        if (j % 4 == 0) rb[j / 4] = r;
        else rb[j / 4] |= r << (8 * (j % 4));
        if (!vk) blk_rank[t * K + j] = (uint8_t)r;
      }
    }
    if (vk) store_bytes<L>(blk_rank + t * L, rb);
  }
}

// One wave per local expert l: the block counts blk_cnt[l][0 .. nb) become
// exclusive prefixes over the blocks, in place; tot[l] gets the total.  A
// round covers 1024 blocks (16 a lane, all loaded before any is used).
constexpr int kScanWaves = 4;
// The multi-block scatter sums every earlier block's counts itself up to this
// many blocks (65536 tokens in 256-token blocks), and reads prefixes that
// route_count_scan made beyond (fp32 logits, expert counts that are no power
// of two): 131072 fp32-routed tokens over 128 experts sum 512 x 128 counts in
// each of 512 workgroups otherwise.
constexpr int64_t kScanBlocks = 256;
__global__ __launch_bounds__(64 * kScanWaves) void route_count_scan(int32_t *__restrict__ blk_cnt,
                                                                    int nbp, int nb, int nl,
                                                                    int32_t *__restrict__ tot) {
  const int lane = threadIdx.x & 63;
  const int l = blockIdx.x * kScanWaves + __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  if (l >= nl) return;  // whole wave
  u32x4_t *row = reinterpret_cast<u32x4_t *>(blk_cnt + (int64_t)l * nbp);
  int carry = 0;
  for (int c0 = 0; c0 < nb; c0 += 1024) {
    const int base = c0 + 16 * lane;  // this lane's 16 blocks
    u32x4_t v[4];
#pragma unroll
    for (int u = 0; u < 4; ++u)
      v[u] = base + 4 * u < nbp ? row[base / 4 + u] : u32x4_t{0u, 0u, 0u, 0u};
    int c[16], s = 0;
#pragma unroll
    for (int u = 0; u < 4; ++u)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        c[4 * u + q] = base + 4 * u + q < nb ? (int)v[u][q] : 0;  // padding was never written
        s += c[4 * u + q];
      }
    const int incl = wave_inclusive_sum(s);
    int run = carry + incl - s;
#pragma unroll
    for (int u = 0; u < 4; ++u) {
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        v[u][q] = (uint32_t)run;
        run += c[4 * u + q];
      }
      if (base + 4 * u < nbp) row[base / 4 + u] = v[u];
    }
    carry += __shfl(incl, 63);
  }
  if (lane == 0) tot[l] = carry;
}

// Per 64-token block (a wave): offsets from the totals, then every entry of
// the block to offsets[e] + (entries of e in earlier blocks) + rank.  The
// workgroup's four blocks are consecutive, so for each expert their entries
// fill one contiguous range of the sorted order; the entries are staged in
// LDS in that order (expert by expert, then by position) and written out by
// consecutive lanes to consecutive positions (STAGED), instead of each lane
// storing its own entries at scattered positions.  Staging pays from top-4
// (65536 tokens: 256 experts top-8 30.9 -> 28.9 us, 64 experts top-8 19.6 ->
// 17.9, 128 experts top-16 43.4 -> 37.4, top-4 18.2 -> 17.9) and costs its two
// barriers below that (8 experts top-1 9.8 -> 10.5 us).
constexpr int kScatterStage = kLaneWaves * kLaneBlock * kMaxTopk;  // entries of a workgroup
template <bool STAGED>
__global__ __launch_bounds__(64 * kLaneWaves) void route_lane_scatter(
    int64_t N, int K, int lo, int nl, int nbp, const int32_t *__restrict__ blk_pre,
    const int32_t *__restrict__ tot, const uint8_t *__restrict__ blk_rank,
    const int32_t *__restrict__ topk_idx, const bf16_t *__restrict__ topk_w,
    int32_t *__restrict__ col_sum, int32_t *__restrict__ offsets, int32_t *__restrict__ col_sorted,
    int32_t *__restrict__ row_sorted, bf16_t *__restrict__ gate_scal) {
  constexpr int NS = STAGED ? kScatterStage : 1;
  __shared__ int s_base[kLaneWaves][kMaxExperts];  // a block's first position of each expert
  __shared__ int s_qoff[kMaxExperts];              // staging index minus position, per expert
  __shared__ int s_nq;                             // entries staged
  __shared__ int s_p[NS];                          // staged entries: position,
  __shared__ int s_c[NS];                          // slot,
  __shared__ bf16_t s_w[NS];                       // routing weight
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int64_t b0 = (int64_t)blockIdx.x * kLaneWaves;
  const int64_t b = b0 + wave;
  const int64_t tok0 = b * kLaneBlock;
  const bool blk = tok0 < N;  // (uniform) this wave's block exists; every wave meets the barriers
  const int64_t t = tok0 + lane;
  const bool own = t < N;
  // the block's entries first: they do not depend on the counts
  int ex[kMaxTopk], rk[kMaxTopk];
  bf16_t w[kMaxTopk];
  // K = 4 or 8: a token's entries come in as whole vectors (offsets are
  // multiples of their sizes; the bases are checked)
  const int kv = (K == 4 || K == 8) && aligned_to(topk_idx, 16) && aligned_to(topk_w, 2 * K) &&
                         aligned_to(blk_rank, K) && aligned_to(row_sorted, 16)
                     ? K
                     : 0;
  auto load_vec = [&](auto kc) {
    constexpr int KV = decltype(kc)::value;
    typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));
    const u32x4_t *pi = reinterpret_cast<const u32x4_t *>(topk_idx + t * KV);
    uint32_t wr[KV / 2], rr[KV / 4];
    if constexpr (KV == 4) {
      const u32x2_t a = *reinterpret_cast<const u32x2_t *>(topk_w + t * KV);
      wr[0] = a[0];
      wr[1] = a[1];
      rr[0] = *reinterpret_cast<const uint32_t *>(blk_rank + t * KV);
    } else {
      const u32x4_t a = *reinterpret_cast<const u32x4_t *>(topk_w + t * KV);
      const u32x2_t r = *reinterpret_cast<const u32x2_t *>(blk_rank + t * KV);
#pragma unroll
      for (int i = 0; i < 4; ++i) wr[i] = a[i];
      rr[0] = r[0];
      rr[1] = r[1];
    }
#pragma unroll
    for (int q = 0; q < KV / 4; ++q) {
      const u32x4_t v = pi[q];
#pragma unroll
      for (int i = 0; i < 4; ++i) ex[4 * q + i] = (int)v[i] - lo;
    }
#pragma unroll
    for (int j = 0; j < KV; ++j) {
      rk[j] = (int)((rr[j / 4] >> (8 * (j % 4))) & 0xffu);
      w[j] = (bf16_t)(wr[j / 2] >> (16 * (j % 2)));
    }
  };
  if (own) {
    if (kv == 4) {
      load_vec(std::integral_constant<int, 4>());
    } else if (kv == 8) {
      load_vec(std::integral_constant<int, 8>());
    } else {
#pragma unroll
      for (int j = 0; j < kMaxTopk; ++j) {
        if (j < K) {
          ex[j] = topk_idx[t * K + j] - lo;  // local id; outside the share if not in [0, nl)
          rk[j] = blk_rank[t * K + j];
          w[j] = topk_w[t * K + j];
        }
      }
    }
  }
  // totals of the local experts (four a lane) -> exclusive scan -> offsets
  int v[4], off[4], s = 0;
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int l = lane * 4 + q;
    v[q] = l < nl ? tot[l] : 0;
    s += v[q];
  }
  const int incl = wave_inclusive_sum(s);
  {
    int run = incl - s;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      off[q] = run;
      run += v[q];
    }
  }
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int l = lane * 4 + q;
    if (l < nl) {
      if (blk) s_base[wave][l] = off[q] + blk_pre[(int64_t)l * nbp + b];
      if (b == 0) {
        offsets[l] = off[q];
        col_sum[l] = v[q];
      }
    }
  }
  const int m_local = __shfl(incl, 63);
  if (b == 0 && lane == 0) offsets[nl] = m_local;
  if (STAGED && wave == 0) {
    // the workgroup's range of each expert: [off + pre[b0], off + pre[b0 + 4]),
    // pre past the last block being the total; staged expert by expert
    int c[4], p0[4], cs = 0;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int l = lane * 4 + q;
      p0[q] = 0;
      c[q] = 0;
      if (l < nl) {
        p0[q] = blk_pre[(int64_t)l * nbp + b0];
        c[q] = (b0 + kLaneWaves < nbp ? blk_pre[(int64_t)l * nbp + b0 + kLaneWaves] : v[q]) - p0[q];
      }
      cs += c[q];
    }
    const int ci = wave_inclusive_sum(cs);
    int run = ci - cs;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int l = lane * 4 + q;
      if (l < nl) s_qoff[l] = run - (off[q] + p0[q]);
      run += c[q];
    }
    if (lane == 63) s_nq = ci;
  }
  if (STAGED) {
    __syncthreads();
  } else {  // each wave reads only its own block's bases
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  }
  if (own) {
    uint32_t rs[kMaxTopk];
#pragma unroll
    for (int j = 0; j < kMaxTopk; ++j) {
      if (j < K) {
        int p = -1;
        if ((unsigned)ex[j] < (unsigned)nl) {
          p = s_base[wave][ex[j]] + rk[j];
          if (STAGED) {
            const int q = s_qoff[ex[j]] + p;
            s_p[q] = p;
            s_c[q] = (int)(t * K + j);
            s_w[q] = w[j];
          } else {
            col_sorted[p] = (int32_t)(t * K + j);
            gate_scal[p] = w[j];
          }
        }
        rs[j] = (uint32_t)p;
        if (!kv) row_sorted[t * K + j] = p;
      }
    }
    if (kv == 4) store_bytes<16>(row_sorted + t * 4, rs);
    else if (kv == 8) store_bytes<32>(row_sorted + t * 8, rs);
  }
  if (STAGED) {
    __syncthreads();
    const int nq = s_nq;
    for (int q = threadIdx.x; q < nq; q += 64 * kLaneWaves) {
      const int p = s_p[q];
      col_sorted[p] = s_c[q];
      gate_scal[p] = s_w[q];
    }
  }
  // sorted positions past the local entries: each block clears its share of
  // [m_local, N*K), the positions [b*64*K, (b+1)*64*K)
  if (blk) {
    const int64_t M = N * K;
    const int64_t p_end = min(M, (b + 1) * kLaneBlock * K);
    for (int64_t p = max((int64_t)m_local, b * kLaneBlock * K) + lane; p < p_end; p += 64) {
      col_sorted[p] = -1;
      gate_scal[p] = from_f32<bf16_t>(0.f);
    }
  }
}

inline size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

// Which routing path a batch takes: one workgroup for small batches (see
// route_path), otherwise one workgroup per block of 64 or 256 tokens plus the
// scatter kernel.  (One workgroup for up to 4096 tokens of a few experts was
// measured slower than the two kernels: 16.8 against 11.1 us at N = 4096,
// E = 8.)
constexpr int kFusedTokens = 256;
// Batches of at most 64 tokens (decode) use a one-group chunk: the rank phase
// then spreads the experts over all 16 waves of the workgroup.
constexpr int kSmallTokens = 64;
static_assert(kGateFusedTokens <= kSmallTokens, "the router-GEMM prologue paths use the small chunk");
// Past kFusedWideTokens tokens, layers of more than kFusedWideExperts experts
// (two or more 16-byte logit chunks per lane-group row) take the multi-block
// path: the one-workgroup top-k is then VALU-bound on one CU (E = 128 at 256
// tokens: 15.3 us fused, 11.4 us in 64-token blocks; E = 256, k = 8: 35.5 vs
// 20.6), while few experts stay cheaper in one launch (E = 32 at 256 tokens:
// 7.4 vs 10.4 us; E = 64, k = 16 at 150 tokens: 15.7 vs 17.4).
constexpr int kFusedWideTokens = 128, kFusedWideExperts = 64;
enum RoutePath { kPathFused, kPathBlocks };
inline RoutePath route_path(int64_t N, int E, int K) {
  (void)K;
  if (N <= kFusedWideTokens) return kPathFused;
  return N <= kFusedTokens && E <= kFusedWideExperts ? kPathFused : kPathBlocks;
}
// Tokens per block of the multi-block path.  A block's top-k runs on one CU,
// so batches too small to fill the CUs with 256-token blocks take 64-token
// blocks (one pass of 16 lanes a token at E = 128): 4x the workgroups.
constexpr int64_t kSmallBlocksUpTo = 16384;
inline int route_block_tokens(int64_t N) { return N <= kSmallBlocksUpTo ? 64 : kRouteTokens; }

// The lane-per-token path takes bf16 logits of a power-of-two expert count
// from 8 in batches of at least lane_tokens(E) tokens, where it is faster (32768
// tokens, 128 experts: 22.9 -> 19.8 us; 65536: 27.7 -> 23.2 us; 32 experts
// even) and its count scan is linear in the number of blocks, where
// route_scatter's re-summing of all earlier blocks grows with their square
// (262144 tokens: 146 -> 54 us).  Smaller batches keep the cooperative top-k
// above: with few tokens a CU the lane path leaves SIMDs idle, which costs
// less the more experts a token ranks.  Where the two cross (same builds,
// interleaved): 256 experts top-8 from 8192 tokens (25.9 -> 23.5 us; 12288:
// 29.4 -> 23.7), 128 experts top-4 from 12288 (15.9 -> 15.4; 10240: 15.2
// against 15.5; 24576: 21.8 -> 15.6), 64 experts past the cooperative path's
// 64-token blocks (16384 top-4: 12.8 against 13.4; 20480: 16.5 -> 13.5, top-8
// 22.5 -> 16.3); 32 experts even from 20480 to 28672 tokens, 16 behind up to
// 28672: 32768 for those.
inline int64_t lane_tokens(int E) {
  return E >= 256 ? 8192 : E >= 128 ? 12288 : E >= 64 ? kSmallBlocksUpTo + 1 : 32768;
}
inline bool lane_path(int64_t N, int E) {
  return E >= 8 && (E & (E - 1)) == 0 && N >= lane_tokens(E) && N * E * 2 < ((int64_t)1 << 31);
}

// With x != nullptr (router GEMM), `logits` is written from x and the gate
// weight wg [E, H] before the top-k reads it.
template <typename T>
hipError_t launch_route_t(const T *logits, int64_t N, int E, int K, int lo, int nl,
                          const moe_routing_t *r, void *scratch, hipStream_t s,
                          const T *x = nullptr, const T *wg = nullptr, int H = 0) {
  constexpr int V = Logit<T>::kVec;
  // two chunks a lane when one would need more than 8 lanes a token, unless the
  // batch is so small that spreading it over more lanes matters more
  const RoutePath path = route_path(N, E, K);
  const int ntb = route_block_tokens(N);
  const bool wide = (E + V - 1) / V > 8 && N > 64 && !(path == kPathBlocks && ntb == 64);
  const int C = wide ? 2 : 1;
  const int need = (E + C * V - 1) / (C * V);
  int logG = 0;
  while ((1 << logG) < need) ++logG;
  const int vec = (E % V) == 0;
  T *tw = reinterpret_cast<T *>(r->topk_w);
  T *gs = reinterpret_cast<T *>(r->gate_scal);
  T *lw = const_cast<T *>(logits);
  const int gate_nsl = x ? gate_parts(E, H * (int)sizeof(T)) : 0;
  if (x && N <= kGateGemvTokens) {
    // a few tokens: the router GEMM as a wave per expert row, then the routing
    // kernels below on its logits
    const dim3 grid((unsigned)((E + kGateGemvWaves - 1) / kGateGemvWaves)), block(64 * kGateGemvWaves);
    switch (N) {
      case 1: hipLaunchKernelGGL((gate_gemv<T, 1>), grid, block, 0, s, x, wg, H, E, lw); break;
      case 2: hipLaunchKernelGGL((gate_gemv<T, 2>), grid, block, 0, s, x, wg, H, E, lw); break;
      case 3: hipLaunchKernelGGL((gate_gemv<T, 3>), grid, block, 0, s, x, wg, H, E, lw); break;
      default: hipLaunchKernelGGL((gate_gemv<T, 4>), grid, block, 0, s, x, wg, H, E, lw); break;
    }
    const hipError_t err = hipGetLastError();
    if (err != hipSuccess) return err;
  } else if (x && gate_split(N, gate_nsl)) {
    // split-K router GEMM into the scratch; the sums are added up by gate_reduce
    // or, for a small batch, in the routing kernel's prologue
    float *part = reinterpret_cast<float *>(scratch);
    const int ep = gate_bucket(E), np = gate_groups(N, gate_nsl);
    const int g = (gate_nsl + np - 1) / np;
    const unsigned tiles = (unsigned)((N + kGateFusedTokens - 1) / kGateFusedTokens);
    auto partial = [&](auto kern) {
      hipLaunchKernelGGL(kern, dim3((unsigned)np, tiles), dim3(256), 0, s, x, wg, N, H, E, part,
                         g);
    };
    switch (ep) {
      case 32: partial(gate_partial<T, 32>); break;
      case 64: partial(gate_partial<T, 64>); break;
      case 128: partial(gate_partial<T, 128>); break;
      default: partial(gate_partial<T, 256>); break;
    }
    hipError_t err = hipGetLastError();
    if (err != hipSuccess) return err;
    const int64_t ne = N * E;
    if (N <= kSmallTokens && ne * np * 4 <= kGateSumInlineBytes) {
      hipLaunchKernelGGL((route_fused<T, 1024, 1, ChunkLds<T, kSmallTokens>, 2>), dim3(1),
                         dim3(1024), 0, s, logits, N, E, K, lo, nl, logG, vec, r->topk_idx, tw,
                         r->bitmatrix, r->col_sum, r->offsets, r->col_sorted, r->row_sorted, gs,
                         x, wg, H, lw, part, np);
      return hipGetLastError();
    }
    hipLaunchKernelGGL(gate_reduce<T>,
                       dim3((unsigned)((ne + kGateReduceThreads - 1) / kGateReduceThreads)),
                       dim3(kGateReduceThreads), 0, s, part, ne, np, lw);
    err = hipGetLastError();
    if (err != hipSuccess) return err;
    // the logits are in place: the routing kernels below
  } else if (x && N <= kGateFusedTokens) {  // router GEMM in the routing kernel's prologue
    // (batches this small take one logit chunk a lane: `wide` is false)
    auto fused = [&](auto kern) {
      hipLaunchKernelGGL(kern, dim3(1), dim3(1024), 0, s, logits, N, E, K, lo, nl, logG, vec,
                         r->topk_idx, tw, r->bitmatrix, r->col_sum, r->offsets, r->col_sorted,
                         r->row_sorted, gs, x, wg, H, lw, nullptr, 0);
    };
    using L = ChunkLds<T, kSmallTokens>;
    switch (gate_bucket(E)) {
      case 32: fused(route_fused<T, 1024, 1, L, 1, 32>); break;
      case 64: fused(route_fused<T, 1024, 1, L, 1, 64>); break;
      case 128: fused(route_fused<T, 1024, 1, L, 1, 128>); break;
      default: fused(route_fused<T, 1024, 1, L, 1, 256>); break;
    }
    return hipGetLastError();
  } else if (x) {  // router GEMM as a kernel of its own, then the routing kernels
    // The largest tile (32, 64 or 128 tokens) that still gives every compute
    // unit a workgroup: larger tiles read the gate weight less often, but a
    // launch with fewer workgroups than CUs leaves the x stream short of
    // loads in flight (128-token tiles at 8192 tokens: 63 us; 32-token: ~51)
    int dev = 0, cus = 0;
    if (hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
        cus <= 0)
      cus = 256;
    const int nt = N >= 128 * (int64_t)cus ? 128 : N >= 64 * (int64_t)cus ? 64 : 32;
    const unsigned g = (unsigned)((N + nt - 1) / nt);
    auto gemm = [&](auto kern) {
      hipLaunchKernelGGL(kern, dim3(g), dim3(kGateThreads), 0, s, x, wg, N, H, E, lw);
    };
    switch (gate_bucket(E) * 1000 + nt) {
      case 32032: gemm(gate_gemm<T, 32, 32>); break;
      case 64032: gemm(gate_gemm<T, 32, 64>); break;
      case 128032: gemm(gate_gemm<T, 32, 128>); break;
      case 256032: gemm(gate_gemm<T, 32, 256>); break;
      case 32064: gemm(gate_gemm<T, 64, 32>); break;
      case 64064: gemm(gate_gemm<T, 64, 64>); break;
      case 128064: gemm(gate_gemm<T, 64, 128>); break;
      case 256064: gemm(gate_gemm<T, 64, 256>); break;
      case 32128: gemm(gate_gemm<T, 128, 32>); break;
      case 64128: gemm(gate_gemm<T, 128, 64>); break;
      case 128128: gemm(gate_gemm<T, 128, 128>); break;
      default: gemm(gate_gemm<T, 128, 256>); break;
    }
    const hipError_t err = hipGetLastError();
    if (err != hipSuccess) return err;
  }
  if (path == kPathFused) {
    if (N == 1)
      hipLaunchKernelGGL((route_one<T>), dim3(1), dim3(64), 0, s, logits, E, K, lo, nl, vec,
                         r->topk_idx, tw, r->bitmatrix, r->col_sum, r->offsets, r->col_sorted,
                         r->row_sorted, gs);
    else if (N <= kSmallTokens)  // (`wide` needs N > 64)
      hipLaunchKernelGGL((route_fused<T, 1024, 1, ChunkLds<T, kSmallTokens>>), dim3(1), dim3(1024),
                         0, s, logits, N, E, K, lo, nl, logG, vec, r->topk_idx, tw, r->bitmatrix,
                         r->col_sum, r->offsets, r->col_sorted, r->row_sorted, gs);
    else if (wide)
      hipLaunchKernelGGL((route_fused<T, 1024, 2, ChunkLds<T, kFusedTokens>>), dim3(1), dim3(1024),
                         0, s, logits, N, E, K, lo, nl, logG, vec, r->topk_idx, tw, r->bitmatrix,
                         r->col_sum, r->offsets, r->col_sorted, r->row_sorted, gs);
    else
      hipLaunchKernelGGL((route_fused<T, 1024, 1, ChunkLds<T, kFusedTokens>>), dim3(1), dim3(1024),
                         0, s, logits, N, E, K, lo, nl, logG, vec, r->topk_idx, tw, r->bitmatrix,
                         r->col_sum, r->offsets, r->col_sorted, r->row_sorted, gs);
    return hipGetLastError();
  }
  if constexpr (std::is_same<T, bf16_t>::value) {
    if (lane_path(N, E)) {
    // bf16 logits: one lane per token (route_lane_topk, route_count_scan,
    // route_lane_scatter).  Scratch: block counts [nl][nbp] (then their
    // prefixes), the local experts' totals, the entries' in-block ranks.
    const int64_t nb = (N + kLaneBlock - 1) / kLaneBlock;
    const int nbp = (int)((nb + 3) / 4 * 4);
    int32_t *blk_cnt = reinterpret_cast<int32_t *>(scratch);
    int32_t *tot = reinterpret_cast<int32_t *>(reinterpret_cast<char *>(scratch) +
                                               align256((size_t)nbp * E * 4));
    uint8_t *blk_rank = reinterpret_cast<uint8_t *>(tot) + align256((size_t)E * 4);
    const unsigned wgs = (unsigned)((nb + kLaneWaves - 1) / kLaneWaves);
    const size_t lds = (size_t)kLaneWaves * kLaneBlock * E * 2;
    auto topk = [&](auto kern) {
      int lch = 0;
      while ((8 << lch) < E) ++lch;
      hipLaunchKernelGGL(kern, dim3(wgs), dim3(64 * kLaneWaves), lds, s, logits, N, E, lch, K, lo,
                         nl, r->topk_idx, tw, r->bitmatrix, blk_cnt, nbp, blk_rank);
    };
    if (K <= 2) topk(route_lane_topk<2>);
    else if (K <= 4) topk(route_lane_topk<4>);
    else if (K <= 8) topk(route_lane_topk<8>);
    else topk(route_lane_topk<16>);
    hipLaunchKernelGGL(route_count_scan, dim3((unsigned)((nl + kScanWaves - 1) / kScanWaves)),
                       dim3(64 * kScanWaves), 0, s, blk_cnt, nbp, (int)nb, nl, tot);
    hipLaunchKernelGGL(K >= 4 ? route_lane_scatter<true> : route_lane_scatter<false>, dim3(wgs),
                       dim3(64 * kLaneWaves), 0, s, N, K, lo, nl, nbp, blk_cnt, tot, blk_rank,
                       r->topk_idx, tw, r->col_sum, r->offsets, r->col_sorted, r->row_sorted, gs);
    return hipGetLastError();
    }
  }
  const int64_t nb = (N + ntb - 1) / ntb;
  const int nbp = (int)((nb + 3) / 4 * 4);
  // scratch: block counts [nl][nbp], the totals, the entries' in-block ranks
  int32_t *blk_cnt = reinterpret_cast<int32_t *>(scratch);
  int32_t *tot = reinterpret_cast<int32_t *>(reinterpret_cast<char *>(scratch) +
                                             align256((size_t)nbp * E * 4));
  uint8_t *blk_rank = reinterpret_cast<uint8_t *>(tot) + align256((size_t)E * 4);
  // past kScanBlocks blocks the counts are prefix-summed once (route_count_scan)
  // instead of by every scatter workgroup
  const bool pre = nb > kScanBlocks;
  auto blocks = [&](auto topk_kern, auto scatter_kern, auto scatter_pre, int tt) {
    hipLaunchKernelGGL(topk_kern, dim3((unsigned)nb), dim3(tt), 0, s, logits, N, E, K, lo, nl,
                       logG, vec, r->topk_idx, tw, r->bitmatrix, blk_cnt, nbp, blk_rank);
    if (pre)
      hipLaunchKernelGGL(route_count_scan, dim3((unsigned)((nl + kScanWaves - 1) / kScanWaves)),
                         dim3(64 * kScanWaves), 0, s, blk_cnt, nbp, (int)nb, nl, tot);
    hipLaunchKernelGGL(pre ? scatter_pre : scatter_kern, dim3((unsigned)nb), dim3(kScatterThreads),
                       0, s, N, K, lo, nl, (int)nb, nbp, blk_cnt, tot, blk_rank, r->topk_idx, tw,
                       r->col_sum, r->offsets, r->col_sorted, r->row_sorted, gs);
  };
  // 64-token blocks of tokens that need at most four lanes each (up to 32 bf16
  // or 16 fp32 experts) fill a quarter of a 1024-thread workgroup in the top-k
  // phase: 256-thread workgroups for it (E = 8 at 4096 tokens 9.1 -> 8.1 us,
  // E = 32 at 16384 tokens 12.6 -> 10.9 us; the scatter kept at 1024 threads
  // measured best)
  if (ntb == 64 && logG <= 2)
    blocks(route_topk_rank<T, 1, 64, 256>, route_scatter<T, 64>, route_scatter<T, 64, true>, 256);
  else if (ntb == 64)
    blocks(route_topk_rank<T, 1, 64>, route_scatter<T, 64>, route_scatter<T, 64, true>,
           kTopkThreads);
  else if (wide)
    blocks(route_topk_rank<T, 2, kRouteTokens>, route_scatter<T, kRouteTokens>,
           route_scatter<T, kRouteTokens, true>, kTopkThreads);
  else
    blocks(route_topk_rank<T, 1, kRouteTokens>, route_scatter<T, kRouteTokens>,
           route_scatter<T, kRouteTokens, true>, kTopkThreads);
  return hipGetLastError();
}

}  // namespace

size_t gate_scratch_bytes(int64_t n_tokens, int n_experts, int hidden, moe_dtype_t dt) {
  const int nsl = gate_parts(n_experts, hidden * (dt == MOE_BF16 ? 2 : 4));
  if (n_tokens <= kGateGemvTokens || !gate_split(n_tokens, nsl)) return 0;  // gate_gemv
  const int np = gate_groups(n_tokens, nsl);
  return align256((size_t)np * n_tokens * n_experts * 4);
}

size_t route_scratch_bytes(int64_t n_tokens, int n_experts, int topk) {
  if (route_path(n_tokens, n_experts, topk) != kPathBlocks) return 0;
  // the most either multi-block path needs: the 64-token blocks of the
  // lane-per-token path (at least as many blocks as route_block_tokens gives)
  // plus its expert totals
  const int64_t nb = (n_tokens + kLaneBlock - 1) / kLaneBlock;
  const int64_t nbp = (nb + 3) / 4 * 4;
  return align256((size_t)nbp * n_experts * 4) + align256((size_t)n_experts * 4) +
         align256((size_t)n_tokens * topk);
}

hipError_t launch_route(const void *logits, moe_dtype_t dt, int64_t n_tokens, int n_experts,
                        int topk, int local_offset, int n_local, const moe_routing_t *r,
                        void *scratch, hipStream_t s, const void *x, const void *w_gate,
                        int hidden) {
  if (dt == MOE_BF16)
    return launch_route_t<bf16_t>(reinterpret_cast<const bf16_t *>(logits), n_tokens, n_experts,
                                  topk, local_offset, n_local, r, scratch, s,
                                  reinterpret_cast<const bf16_t *>(x),
                                  reinterpret_cast<const bf16_t *>(w_gate), hidden);
  return launch_route_t<float>(reinterpret_cast<const float *>(logits), n_tokens, n_experts,
                               topk, local_offset, n_local, r, scratch, s,
                               reinterpret_cast<const float *>(x),
                               reinterpret_cast<const float *>(w_gate), hidden);
}

}  // namespace moe
