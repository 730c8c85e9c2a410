// Grouped expert GEMMs over ragged expert segments, MFMA on gfx950.
//
// The expert FFN it runs -- w13 projection, gated (SiLU / SwiGLU-OAI) or
// non-gated (ReLU^2) activation, w2 projection, routing weight on the expert
// output -- is the one described by the minimind issue #835 page ("Summary":
// the weight multiplies each expert's output before it is added in) and the
// vLLM PR #47106 report (activation kinds, parameters, w13 layouts).
//
// Design (this file's own):
//  * Persistent workgroups.  The m-tiles of all experts are numbered expert by
//    expert; every workgroup derives the tile starts from the device-side
//    offsets (a 64-lane scan of ceil(count / BM) per expert), so the host never
//    learns the counts, and loops over (m-tile, n-tile) pairs with a stride of
//    the grid size.  Only real tiles are visited; the grid is sized to the
//    machine, not to a host-side upper bound.
//  * Operands go from HBM straight into LDS with buffer_load ... lds (16 bytes
//    per lane, no VGPR staging) through an S-stage ring: at step kt a workgroup
//    waits for slice kt, passes one barrier, issues slice kt + S - 1 into the
//    slot freed by step kt - 1, and runs the MFMAs of slice kt.  Lanes whose
//    chunk lies past the expert's rows, past the output columns, or past K get
//    an out-of-range buffer offset and the hardware writes zeros, so tails need
//    no separate code.
//  * The 32-row tiles (taken when experts hold fewer than 48 rows, i.e. when
//    the layer streams its weights) load bf16 / fp32 weight slices non-
//    temporally: 5-7 % faster on a gpt-oss-sized layer at 200-512 tokens and
//    on a 32-token decode stack.  Larger tiles keep the default policy: their
//    weight slices are re-read by neighbouring m-tiles through L2 (non-
//    temporal there measured 18-30 % slower), and so do MXFP4 code slices
//    (15-35 % slower non-temporal, even on the 32-row tiles).
//  * GEMM1 gathers its A rows straight from x: sorted row p reads token
//    col_sorted[p] / topk.  No gathered copy of x is ever written.
//  * Tiles are 128-byte K-slices per row with the 16-byte chunk index XOR-
//    swizzled by the row; each lane of a load fetches the chunk that belongs in
//    its fixed LDS slot, and the 16-byte fragment reads of a 32-row MFMA operand
//    hit distinct banks.
//  * Gated GEMM1 tiles hold BN gate rows and the BN matching up rows of w13,
//    picked by layout (packed: rows n and inter + n; interleaved: 2n and
//    2n + 1), so gate and up of one output land in the same lane and register
//    of two accumulators and the activation runs in the epilogue from fp32.
//  * bf16 uses v_mfma_f32_32x32x16_bf16, fp32 uses v_mfma_f32_32x32x2_f32.
#include <cmath>
#include <type_traits>
#include <utility>

#include "gemm_common.h"
#include "lds_dma.h"

namespace moe {
namespace {


template <typename T> struct Mma;
template <> struct Mma<bf16_t> {
  static constexpr int KS = 16;  // K per instruction
  static constexpr int EPL = 8;  // K elements per lane fragment
  typedef bf16x8_t Frag;
  __device__ static Frag ld(const char *p) { return *reinterpret_cast<const bf16x8_t *>(p); }
  __device__ static f32x16_t mma(Frag a, Frag b, f32x16_t c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
  }
};
template <> struct Mma<float> {
  static constexpr int KS = 2;
  static constexpr int EPL = 1;
  typedef float Frag;
  __device__ static Frag ld(const char *p) { return *reinterpret_cast<const float *>(p); }
  __device__ static f32x16_t mma(Frag a, Frag b, f32x16_t c) {
    return __builtin_amdgcn_mfma_f32_32x32x2f32(a, b, c, 0, 0, 0);
  }
};

// LDS rows are RB bytes (one K-slice of one operand row).  A ds_read_b128 is
// served 16 lanes at a time from 64 four-byte banks (256 bytes), i.e. from
// 256 / RB rows at once, and the 16 lanes of a fragment read hit 16
// consecutive rows at the same logical chunk.  XOR-ing the chunk index with
// (row / (256 / RB)) % (RB / 16) spreads those 16 reads over all 16 bank
// groups: row % (256 / RB) picks the group's row in the bank line and the key
// the chunk.
template <int RB> __device__ __forceinline__ int swz_key(int row) {
  return (row / (256 / RB)) % (RB / 16);
}
template <int RB> __device__ __forceinline__ int swz(int row, int chunk) {
  return row * RB + ((chunk ^ swz_key<RB>(row)) << 4);
}

// Two fp32 values as two bf16 (round to nearest even, v_cvt_pk_bf16_f32), the
// first in the low half.
__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
  typedef __bf16 bf16x2v_t __attribute__((ext_vector_type(2)));
  const bf16x2v_t p = {(__bf16)a, (__bf16)b};
  return __builtin_bit_cast(uint32_t, p);
}

// Four consecutive output elements of one row.
typedef int32_t i32x2_t __attribute__((ext_vector_type(2)));
typedef int32_t i32x4_t __attribute__((ext_vector_type(4)));
__device__ __forceinline__ void store4(__amdgpu_buffer_rsrc_t r, uint32_t off, const float (&v)[4],
                                       bf16_t) {
  typedef __bf16 bf16x4_t __attribute__((ext_vector_type(4)));
  // v_cvt_pk_bf16_f32: round to nearest even, as bf16_rne
  const bf16x4_t b = {(__bf16)v[0], (__bf16)v[1], (__bf16)v[2], (__bf16)v[3]};
  __builtin_amdgcn_raw_buffer_store_b64(__builtin_bit_cast(i32x2_t, b), r, (int)off, 0, 0);
}
__device__ __forceinline__ void store4(__amdgpu_buffer_rsrc_t r, uint32_t off, const float (&v)[4],
                                       float) {
  i32x4_t d;
#pragma unroll
  for (int t = 0; t < 4; ++t) d[t] = __float_as_int(v[t]);
  __builtin_amdgcn_raw_buffer_store_b128(d, r, (int)off, 0, 0);
}

// Where tile L of the expert-major tile order lives: expert e, output-column
// tile nt, and the rows [row0, row0 + rows) of the expert's sorted segment.
// Inside an expert, tiles are walked in blocks of GM m-tiles x GN n-tiles
// (n-block outer, m-block inner, m-tile fastest inside a block), so the 32
// workgroups one XCD runs at a time share each row tile GN ways and each weight
// tile GM ways.
constexpr int GM = 8, GN = 4;

struct TileInfo {
  int e, row0, rows, n0;
};

template <int BM, int BN>
__device__ __forceinline__ TileInfo tile_info(int L, const int *s_ts, const int *s_off, int E,
                                              int n_nt) {
  const int q = L / n_nt;  // s_ts[e] <= q < s_ts[e + 1] exactly when L is in expert e
  int lo = 0, hi = E - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (s_ts[mid] <= q) lo = mid; else hi = mid - 1;
  }
  const int me = s_ts[lo + 1] - s_ts[lo];  // m-tiles of this expert
  const int l = L - s_ts[lo] * n_nt;
  const int nb = l / (GN * me);
  const int gn = min(GN, n_nt - nb * GN);
  const int r = l - nb * GN * me;
  const int mb = r / (GM * gn);
  const int gm = min(GM, me - mb * GM);
  const int r2 = r - mb * GM * gn;
  const int mt = mb * GM + r2 % gm;
  const int nt = nb * GN + r2 / gm;
  TileInfo ti;
  ti.e = lo;
  ti.row0 = s_off[lo] + mt * BM;
  ti.rows = min(BM, s_off[lo + 1] - ti.row0);
  ti.n0 = nt * BN;
  return ti;
}

// First m-tile of each expert (s_ts[0 .. E], s_ts[E] = all m-tiles) and the
// routing offsets (s_off[0 .. E]) in LDS, from the device-side offsets: one
// wave, four experts a lane.
template <int BM>
__device__ __forceinline__ void tile_starts(const GemmArgs &g, int *s_ts, int *s_off, int lane) {
  const int E = g.E;
  int v[4], s = 0;
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int e = lane * 4 + q;
    const int o0 = e < E ? g.offsets[e] : 0;
    const int o1 = e < E ? g.offsets[e + 1] : 0;
    if (e < E) s_off[e] = o0;
    v[q] = (e < E) ? (o1 - o0 + BM - 1) / BM : 0;
    s += v[q];
  }
  const int incl = wave_inclusive_sum(s);
  int run = incl - s;
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int e = lane * 4 + q;
    if (e < E) s_ts[e] = run;
    run += v[q];
  }
  if (lane == 63) {
    s_ts[E] = incl;
    s_off[E] = g.offsets[E];
  }
}

// f(integral_constant<int, I>) for I = 0 .. N - 1, unrolled at compile time
// (register arrays indexed by I stay in registers).
template <typename F, int... I>
__device__ __forceinline__ void static_for_impl(F &f, std::integer_sequence<int, I...>) {
  (f(std::integral_constant<int, I>{}), ...);
}
template <int N, typename F> __device__ __forceinline__ void static_for(F &&f) {
  static_for_impl(f, std::make_integer_sequence<int, N>{});
}

// This workgroup's share of `total` tiles: first + i * stride, i < count.  The
// tile order is cut into 8 contiguous chunks, one per XCD (the dispatcher
// places workgroup b on XCD b % 8); the XCD's workgroups stride through it.
struct TileShare {
  int first, stride, count;
};
__device__ __forceinline__ TileShare tile_share(int total) {
  const int gx = (int)gridDim.x / 8;  // workgroups per XCD (grid is a multiple of 8)
  const int xcd = (int)blockIdx.x % 8, qx = (int)blockIdx.x / 8;
  const int chunk = (total + 7) / 8;
  const int cbeg = min(total, xcd * chunk), cend = min(total, cbeg + chunk);
  TileShare t;
  t.first = cbeg + qx;
  t.stride = gx;
  t.count = t.first < cend ? (cend - t.first + gx - 1) / gx : 0;
  return t;
}

// Tile of BM rows x BN output columns; WM x WN waves; S-stage LDS ring of
// RB-byte K-slices.
//
// Work split: tiles are ordered expert by expert (within an expert n-tile-
// major, m-tile fastest) and cut into 8 contiguous chunks, one per XCD; the
// dispatcher places workgroup b on XCD b % 8, so the workgroups of one XCD --
// which share that XCD's L2 -- walk one chunk together: concurrently they hold
// neighbouring m-tiles of the same weight tile, or neighbouring n-tiles of the
// same rows.  A workgroup's tiles form one stream of K-slices: the ring keeps
// loading S - 1 slices ahead across tile boundaries, so a tile's epilogue runs
// while the next tile's first slices are in flight.
//
// Eight-wave tiles run a ping-pong schedule: waves 0-3 and 4-7 (one of each
// on every SIMD) alternate between a memory phase -- issue this wave's share
// of a future slice, read all fragments of the current slice into registers
// -- and an MFMA phase on those registers, one group a barrier behind the
// other, so each SIMD's matrix core is fed by one wave while the other waits
// on LDS and HBM.  Four-wave tiles keep one phase per slice and overlap the
// fragment reads of k-step ks + 1 with the MFMAs of k-step ks.
//
// The MFMA takes the weight fragment as its first operand, so the 32 x 32
// accumulator comes out transposed: lane l holds sorted row (l % 32) of the
// sub-tile and each group of four registers four consecutive output columns.
// The epilogue then writes 8-byte (bf16) or 16-byte (fp32) pieces of a row,
// and needs one output-row index and one routing weight per lane.
//
// WQ (MXFP4 weights, bf16 activations): a stage holds the A
// rows, each weight row's E2M1 codes for the slice (RB / 4 bytes: the same K
// range) and the slice's E8M0 scales, tile rows in weight-row order per K-block
// (4-byte loads: the rows of a tile are one or, packed and gated, two
// contiguous runs of the block-major scale array).  A weight fragment is one
// 4-byte read of 8 codes and one scale byte, turned into 8 bf16 values with
// the hardware's scaled FP4 conversion (exact: a code times a power of two).
template <typename T, int NSETS, int EPI, int BM, int BN, int WM, int WN, int S, int RB,
          bool WQ>
__device__ __forceinline__ void gemm_body(const GemmArgs &g) {
  using Mm = Mma<T>;
  using Frag = typename Mm::Frag;
  constexpr int BK = RB / (int)sizeof(T);  // K elements per slice
  constexpr int NKS = BK / Mm::KS;         // MFMA k-steps per slice
  constexpr int CPR = RB / 16;             // 16-byte chunks per LDS row
  constexpr int RPI = 1024 / RB;           // rows per 1 KB load instruction
  constexpr int NW = WM * WN;
  constexpr int NB = NSETS * BN;           // B rows per tile
  constexpr int JA = BM / RPI / NW;        // load instructions per wave per slice
  constexpr int JB = NB / RPI / NW;
  constexpr int TM = BM / WM / 32;         // 32x32 sub-tiles per wave
  constexpr int TN = BN / WN / 32;
  constexpr int QRB = RB / 4;              // WQ: code bytes of a weight row's slice
  constexpr int QCPR = QRB / 16;           // WQ: 16-byte chunks of those
  constexpr int QRPI = 64 / (QCPR > 0 ? QCPR : 1);  // WQ: code rows per 1 KB load
  constexpr int JBQ = WQ ? NB / QRPI / NW : 0;      // WQ: code loads per wave per slice
  constexpr int SBK = BK / 32;             // WQ: scale blocks per slice
  constexpr int BQ = WQ ? NB * QRB : NB * RB;       // B bytes of a stage
  constexpr int SCL = WQ ? NW * 256 : 0;   // WQ: scale bytes of a stage (one 4-byte load a lane)
  constexpr int STAGE = BM * RB + BQ + SCL;
  constexpr int PER = WQ ? JA + JBQ + 1 : JA + JB;  // load instructions per wave per slice
  // stores per wave per epilogue (exact: the ring's vmcnt waits count them):
  // bf16 rows go out as 16-byte pieces, two per 32 x 32 sub-tile; fp32 four
  constexpr int NST = TM * TN * (std::is_same<T, bf16_t>::value ? 2 : 4);
  constexpr bool META = EPI == EPI_Y || EPI == EPI_OUT;
  constexpr bool PP = NW == 8;             // ping-pong schedule
  // four waves over 256-row tiles, one a SIMD: 128-row register blocks
  constexpr bool BIG = NW == 4 && BM == 256;
  static_assert(!BIG || !WQ, "four-wave tiles: bf16/fp32 weights");
  static_assert(!WQ || (std::is_same<T, bf16_t>::value && QCPR >= 1 && JBQ >= 1 &&
                        JBQ * QRPI * NW == NB && SBK * NB <= SCL && NB % 4 == 0),
                "MXFP4 weights: bf16 tiles whose code rows fill whole wave loads");
  // a tile's metadata is written when its first slice is issued (S - 1
  // slices ahead) and read by its epilogue; NSL slots keep the epilogue of
  // tile i clear of the set-up of tile i + NSL
  constexpr int NSL = S + 1;
  static_assert(RB == 64 || RB == 128 || RB == 256, "row bytes");
  static_assert(JA >= 1 && JB >= 1 && JA * RPI * NW == BM && JB * RPI * NW == NB,
                "tile rows vs waves");
  static_assert(TM * 32 * WM == BM && TN * 32 * WN == BN, "wave tiles");
  static_assert(BK % Mm::KS == 0, "slice vs instruction K");
  static_assert(S >= 2 && (S - 2) * PER < 64, "stages / vmcnt range");
  static_assert((EPI == EPI_RELU2 || EPI == EPI_Y || EPI == EPI_OUT) == (NSETS == 1),
                "gated epilogues take two weight sets");

  __shared__ __attribute__((aligned(16))) char smem[S * STAGE];
  __shared__ int s_ts[kMaxExperts + 1];   // first m-tile of each expert
  __shared__ int s_off[kMaxExperts + 1];  // the routing offsets
  __shared__ TileInfo s_tile[NSL];        // per slot: the tile
  // per slot: output row and routing weight of each tile row
  __shared__ i32x2_t s_meta[META ? NSL : 1][META ? BM : 1];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform: keeps LDS bases scalar
  const int E = g.E, K = g.K, Nout = g.Nout;

  // ---- tile starts per expert (same in every workgroup) ---------------------
  if (wave == 0) tile_starts<BM>(g, s_ts, s_off, lane);
  __syncthreads();

  const int n_nt = (Nout + BN - 1) / BN;
  // this workgroup's tiles: L = first + i * gx, i < my_tiles
  const TileShare share = tile_share(s_ts[E] * n_nt);
  const int first = share.first, gx = share.stride, my_tiles = share.count;

  const int kbytes = K * (int)sizeof(T);
  const int nk = (K + BK - 1) / BK;
  const int nz = my_tiles * nk;  // K-slices in this workgroup's stream (uniform)
  if (nz == 0) return;
  const int lrow = lane / CPR;   // row within a 1 KB load; the lane fills physical chunk lane % CPR
  const __amdgpu_buffer_rsrc_t ra = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<void *>(g.A), (short)0, (int)g.a_bytes, kRsrcWord3);
  const __amdgpu_buffer_rsrc_t rc =
      __builtin_amdgcn_make_buffer_rsrc(g.C, (short)0, (int)g.c_bytes, kRsrcWord3);
  const int wkbytes = WQ ? K / 2 : kbytes;  // bytes of one weight row
  const uint32_t w_bytes = (uint32_t)NSETS * Nout * wkbytes;
  const int nrows = NSETS * Nout;           // weight rows of one expert
  const int wm = wave % WM, wn = wave / WM;
  const float nal = -g.prm.alpha * 1.44269504088896341f;

  // issue side: the tile whose slices are being loaded.  A tile's weight
  // loads go out before its gather indices are read (the inline-asm loads are
  // compiler memory barriers, so the index loads stay behind them), and the
  // first weight slices travel while the indices make their round trip.
  uint32_t va[JA], vb[WQ ? JBQ : JB];
  __amdgpu_buffer_rsrc_t rb = ra, rs = ra;
  uint32_t vs = kOOB;  // WQ: this lane's scale offset at K-block 0 (4 rows)
  TileInfo cur;
  auto setup_b = [&](int i) {
    cur = tile_info<BM, BN>(first + i * gx, s_ts, s_off, E, n_nt);
    if (tid == 0) s_tile[i % NSL] = cur;
    rb = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<char *>(reinterpret_cast<const char *>(g.W)) + (size_t)cur.e * w_bytes,
        (short)0, (int)w_bytes, kRsrcWord3);
    if constexpr (WQ) {
#pragma unroll
      for (int j = 0; j < JBQ; ++j) {
        const int r = (wave * JBQ + j) * QRPI + lane / QCPR;
        const int set = r / BN, n = cur.n0 + r % BN;
        vb[j] = kOOB;
        if (n < Nout) {
          const int grow = NSETS == 1 ? n : (g.interleaved ? 2 * n + set : set * Nout + n);
          vb[j] = (uint32_t)grow * (uint32_t)wkbytes + (((lane % QCPR) ^ swz_key<QRB>(r)) << 4);
        }
      }
      // scales: stage byte o = 4 * (wave * 64 + lane) is K-block o / NB of the
      // slice, tile row o % NB in weight-row order (packed: the gate run, then
      // the up run; interleaved and plain: one run from the tile's first row)
      const uint32_t sbytes = (uint32_t)(K / 32) * (uint32_t)nrows;
      rs = __builtin_amdgcn_make_buffer_rsrc(
          const_cast<uint8_t *>(g.wscale) + (size_t)cur.e * sbytes, (short)0, (int)sbytes,
          kRsrcWord3);
      const int o = 4 * (wave * 64 + lane), blk = o / NB, rem = o % NB;
      int wrow, n;
      if (NSETS == 2 && !g.interleaved) {
        n = cur.n0 + rem % BN;
        wrow = (rem / BN) * Nout + n;
      } else {
        wrow = (NSETS == 2 ? 2 * cur.n0 : cur.n0) + rem;
        n = NSETS == 2 ? wrow / 2 : wrow;
      }
      vs = (blk < SBK && n < Nout) ? (uint32_t)blk * (uint32_t)nrows + (uint32_t)wrow : kOOB;
    } else {
#pragma unroll
      for (int j = 0; j < JB; ++j) {
        const int r = (wave * JB + j) * RPI + lrow;
        const int set = r / BN, n = cur.n0 + r % BN;
        vb[j] = kOOB;
        if (n < Nout) {
          const int grow = NSETS == 1 ? n : (g.interleaved ? 2 * n + set : set * Nout + n);
          vb[j] = (uint32_t)grow * (uint32_t)kbytes + (((lane % CPR) ^ swz_key<RB>(r)) << 4);
        }
      }
    }
  };
  auto setup_a = [&](int i) {
#pragma unroll
    for (int j = 0; j < JA; ++j) {
      const int r = (wave * JA + j) * RPI + lrow;
      va[j] = kOOB;
      if (r < cur.rows) {
        const int p = cur.row0 + r;
        const uint32_t arow = g.gather ? (uint32_t)(g.col_sorted[p] / g.topk) : (uint32_t)p;
        va[j] = arow * (uint32_t)kbytes + (((lane % CPR) ^ swz_key<RB>(r)) << 4);
        if (META && lane % CPR == 0) {
          // no gate weights: the routing weight was applied to the input rows
          const float gs = !g.gate_scal ? 1.f
                           : g.gate_bf16
                               ? to_f32(reinterpret_cast<const bf16_t *>(g.gate_scal)[p])
                               : reinterpret_cast<const float *>(g.gate_scal)[p];
          i32x2_t m;
          m[0] = EPI == EPI_OUT ? g.col_sorted[p] : p;  // topk == 1: entry index == token
          m[1] = __float_as_int(gs);
          s_meta[i % NSL][r] = m;
        }
      }
    }
  };
  auto issue = [&](int z) {  // load slice z of the stream into ring slot z % S
    const int i = z / nk, kt = z - i * nk;
    const uint32_t kb = (uint32_t)kt * RB;
    char *base = smem + (z % S) * STAGE;
    // kOOB + kb stays out of range, so invalid rows / columns need no test;
    // only a K-tail slice (kb + RB > row bytes) masks chunks past K.  Rows
    // are K * sizeof(T) bytes, a multiple of 16, so the tail is chunk-aligned.
    const bool tail = (int)kb + RB > kbytes;
    if (kt == 0) setup_b(i);
    if constexpr (WQ) {
      const uint32_t qb = (uint32_t)kt * QRB;
#pragma unroll
      for (int j = 0; j < JBQ; ++j) {
        uint32_t off = vb[j] + qb;
        if (tail) {
          const int r = (wave * JBQ + j) * QRPI + lane / QCPR;
          const int coff = ((lane % QCPR) ^ swz_key<QRB>(r)) << 4;
          off = (int)qb + coff < wkbytes ? off : kOOB;
        }
        dma16(rb, base + BM * RB + (wave * JBQ + j) * 1024, off);
      }
      // the slice's K-blocks kt * SBK + blk; blocks past K read as zero scales
      const int o = 4 * (wave * 64 + lane);
      const bool sin = kt * SBK + o / NB < K / 32;
      dma4(rs, base + BM * RB + BQ + wave * 256,
           sin ? vs + (uint32_t)(kt * SBK) * (uint32_t)nrows : kOOB);
    } else {
#pragma unroll
      for (int j = 0; j < JB; ++j) {
        uint32_t off = vb[j] + kb;
        if (tail) {
          const int coff = ((lane % CPR) ^ swz_key<RB>((wave * JB + j) * RPI + lrow)) << 4;
          off = (int)kb + coff < kbytes ? off : kOOB;
        }
        if constexpr (BM <= 32) dma16_nt(rb, base + BM * RB + (wave * JB + j) * 1024, off);
        else dma16(rb, base + BM * RB + (wave * JB + j) * 1024, off);
      }
    }
    if (kt == 0) setup_a(i);
#pragma unroll
    for (int j = 0; j < JA; ++j) {
      uint32_t off = va[j] + kb;
      if (tail) {
        const int coff = ((lane % CPR) ^ swz_key<RB>((wave * JA + j) * RPI + lrow)) << 4;
        off = (int)kb + coff < kbytes ? off : kOOB;
      }
      dma16(ra, base + (wave * JA + j) * 1024, off);
    }
  };

  f32x16_t acc[TM][TN][NSETS];
  int st_until = -1;  // last slice whose wait must also cover the latest epilogue's stores

  // Slice w is in LDS as far as this wave's loads go: at most the loads of
  // the slices issued after w (this wave has issued up to min(w + S - 2,
  // nz - 1)) may remain, plus an epilogue's stores if they were issued after
  // slice w's loads (an epilogue at slice z0 follows the loads of slices up to
  // z0 + S - 1).  Waits on ds operations too.
  auto wait_slice = [&](int w) {
    wait_pending<PER, NST, S - 2>(min(S - 2, nz - 1 - w), w <= st_until);
  };
  auto frag_addr = [&](int ks, int row) {  // byte in a slice of k-step ks, operand row
    const int byte = (ks * Mm::KS + (lane >> 5) * Mm::EPL) * (int)sizeof(T);
    return swz<RB>(row, byte >> 4) + (byte & 15);
  };
  // B fragment of k-step ks, tile row r: 8 bf16 weights, or (WQ) 8 codes (K
  // elements 16 ks + 8 (lane / 32) ..) times their block's scale
  auto bfrag = [&](const char *lb, int ks, int r) -> Frag {
    if constexpr (WQ) {
      const int qoff = ks * 8 + (lane >> 5) * 4;
      const uint32_t word =
          *reinterpret_cast<const uint32_t *>(lb + swz<QRB>(r, qoff >> 4) + (qoff & 15));
      const int sidx = (NSETS == 2 && g.interleaved) ? 2 * (r % BN) + r / BN : r;
      const uint32_t sb = reinterpret_cast<const uint8_t *>(lb + BQ)[(ks / 2) * NB + sidx];
      return fp4x8_to_bf16(word, __uint_as_float(sb << 23));
    } else {
      return Mm::ld(lb + frag_addr(ks, r));
    }
  };
  auto zero_acc = [&]() {
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
      for (int j = 0; j < TN; ++j)
#pragma unroll
        for (int s = 0; s < NSETS; ++s)
#pragma unroll
          for (int r = 0; r < 16; ++r) acc[i][j][s][r] = 0.f;
  };

  // ---- epilogue: lane holds row (lane % 32) and, in register group q, the
  // four columns 8q + 4 * (lane / 32) + [0, 4) of each 32 x 32 sub-tile ------
  auto epilogue = [&](int z) {
    const int ti_i = z / nk;
    const TileInfo ti = s_tile[ti_i % NSL];
#pragma unroll
    for (int i = 0; i < TM; ++i) {
      const int row = wm * (BM / WM) + i * 32 + (lane & 31);
      const bool ok = row < ti.rows;
      uint32_t orow = (uint32_t)(ti.row0 + row);
      float gs = 1.f;
      if (META) {
        const i32x2_t m = s_meta[ti_i % NSL][row];
        orow = (uint32_t)m[0];
        gs = __int_as_float(m[1]);
      }
#pragma unroll
      for (int j = 0; j < TN; ++j) {
        if constexpr (BIG) {
          // the accumulators stay in AGPRs up to here, so their copies to
          // VGPRs for this sub-tile's arithmetic cannot move earlier
#pragma unroll
          for (int s = 0; s < NSETS; ++s) asm volatile("" : "+a"(acc[i][j][s]));
        }
        auto value = [&](int q, float (&v)[4]) {
#pragma unroll
          for (int t = 0; t < 4; ++t) {
            if constexpr (META)
              v[t] = acc[i][j][0][4 * q + t] * gs;
            else
              v[t] = act_val<EPI>(acc[i][j][0][4 * q + t], acc[i][j][NSETS - 1][4 * q + t], nal,
                                  g.prm);
          }
        };
        if constexpr (std::is_same<T, bf16_t>::value) {
          // register groups q and q + 1 hold columns 8q + [0, 8) and 8q + [8, 16)
          // split between lanes l and l + 32; swapping the halves between the
          // two lanes (v_permlane32_swap) gives lane l the 8 columns 8q + [0, 8)
          // and lane l + 32 the 8 columns 8q + [8, 16): one 16-byte store each
#pragma unroll
          for (int q = 0; q < 4; q += 2) {
            float v0[4], v1[4];
            value(q, v0);
            value(q + 1, v1);
            u32x4_t o = {pack_bf16x2(v0[0], v0[1]), pack_bf16x2(v0[2], v0[3]),
                         pack_bf16x2(v1[0], v1[1]), pack_bf16x2(v1[2], v1[3])};
            const auto s0 = __builtin_amdgcn_permlane32_swap(o[0], o[2], false, false);
            const auto s1 = __builtin_amdgcn_permlane32_swap(o[1], o[3], false, false);
            o[0] = s0[0];
            o[2] = s0[1];
            o[1] = s1[0];
            o[3] = s1[1];
            const int col = ti.n0 + wn * (BN / WN) + j * 32 + 8 * q + 8 * (lane >> 5);
            // Nout is a multiple of 8, so col < Nout covers all eight columns
            const uint32_t off =
                (ok && col < Nout) ? (orow * (uint32_t)Nout + (uint32_t)col) * 2u : kOOB;
            __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(i32x4_t, o), rc, (int)off,
                                                   0, 0);
          }
        } else {
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const int col = ti.n0 + wn * (BN / WN) + j * 32 + 8 * q + 4 * (lane >> 5);
            float v[4];
            value(q, v);
            // Nout is a multiple of 8, so col < Nout covers all four columns
            const uint32_t off = (ok && col < Nout)
                                     ? (orow * (uint32_t)Nout + (uint32_t)col) * (uint32_t)sizeof(T)
                                     : kOOB;
            store4(rc, off, v, T());
          }
        }
        // one sub-tile at a time: hoisting every accumulator read would need
        // 256 more registers in the four-wave tiles
        if constexpr (BIG) __builtin_amdgcn_sched_barrier(0);
      }
    }
    // the four-wave loop issues slice z + S before this epilogue, the others z + S - 1
    st_until = z + S - 1 + (BIG ? 1 : 0);
  };

#pragma unroll
  for (int s = 0; s < S - 1; ++s)
    if (s < nz) issue(s);

  if constexpr (PP) {
    const int grp = wave >> 2;
    Frag fa[NKS][TM], fb[NKS][TN][NSETS];
    wait_slice(0);
    barrier();
    if (grp) barrier();  // group 1 runs one phase behind group 0
    for (int z = 0; z < nz; ++z) {
      // memory phase: next loads out, this slice's fragments in
      if (z + S - 1 < nz) issue(z + S - 1);
      const char *la = smem + (z % S) * STAGE;
      const char *lb = la + BM * RB;
#pragma unroll
      for (int ks = 0; ks < NKS; ++ks) {
#pragma unroll
        for (int i = 0; i < TM; ++i)
          fa[ks][i] = Mm::ld(la + frag_addr(ks, wm * (BM / WM) + i * 32 + (lane & 31)));
#pragma unroll
        for (int j = 0; j < TN; ++j)
#pragma unroll
          for (int s = 0; s < NSETS; ++s)
            fb[ks][j][s] = bfrag(lb, ks, s * BN + wn * (BN / WN) + j * 32 + (lane & 31));
      }
      if (grp && z + 1 < nz) wait_slice(z + 1);
      barrier();
      // MFMA phase
      __builtin_amdgcn_s_setprio(1);
      const int kt = z % nk;
      if (kt == 0) zero_acc();
#pragma unroll
      for (int ks = 0; ks < NKS; ++ks)
#pragma unroll
        for (int i = 0; i < TM; ++i)
#pragma unroll
          for (int j = 0; j < TN; ++j)
#pragma unroll
            for (int s = 0; s < NSETS; ++s)
              acc[i][j][s] = Mm::mma(fb[ks][j][s], fa[ks][i], acc[i][j][s]);
      __builtin_amdgcn_s_setprio(0);
      if (kt == nk - 1) epilogue(z);
      if (!grp && z + 1 < nz) wait_slice(z + 1);
      barrier();
    }
    if (!grp) barrier();
  } else if constexpr (BIG) {
    // One wave a SIMD: nothing else fills the matrix core while this wave
    // issues other work, and a wave issues at most one instruction every four
    // cycles, so the loop keeps its instructions few and each memory
    // instruction follows an MFMA (about seven free issue slots each).
    //  * k-step ks < NKS - 1: the fragments of k-step ks + 1 are read, one
    //    after each MFMA.
    //  * k-step NKS - 2, once its reads are out: the ring's bookkeeping, the
    //    wait for slice z + 1 and the barrier (after which no wave reads slot
    //    z % S again: its last fragments are in registers), then the first
    //    DMA loads of slice z + S into that slot, one after each MFMA.
    //  * last k-step: the remaining DMA loads, then the reads of slice
    //    z + 1's first fragments, spread over its MFMAs (DMA loads bunched in
    //    one k-step stall their issue: spreading them over two measured 1-2 %
    //    faster on every 256-row layer).
    // Every slice takes that path: a slice that starts a tile first sets up
    // the tile's load offsets, and slices past the end of the stream load
    // through an empty buffer (zeros into a slot nobody reads), so each wait
    // is one count.  Rows hold whole slices (no K tail: the host checks).
    constexpr int NM = TM * TN * NSETS;  // MFMAs a k-step
    constexpr int NFK = TM + TN * NSETS; // fragment reads a k-step
    constexpr int NDMA = JA + JB;         // DMA loads a slice
    static_assert(!BIG || (NFK + 2 <= NM && NKS % 2 == 0), "reads, bookkeeping and barrier in a k-step; k-step pairs");
    Frag fa[2][TM], fb[2][TN][NSETS];
    auto frag_read = [&](int buf, const char *la, int ks, int f) {
      if (f < TM) {
        fa[buf][f] = Mm::ld(la + frag_addr(ks, wm * (BM / WM) + f * 32 + (lane & 31)));
      } else {
        const int j = (f - TM) / NSETS, s = (f - TM) % NSETS;
        fb[buf][j][s] = bfrag(la + BM * RB, ks, s * BN + wn * (BN / WN) + j * 32 + (lane & 31));
      }
    };
    auto mma_one = [&](int buf, int m) {
      const int i = m / (TN * NSETS), j = (m / NSETS) % TN, s = m % NSETS;
      acc[i][j][s] = Mm::mma(fb[buf][j][s], fa[buf][i], acc[i][j][s]);
    };
    auto bar = [&]() {  // workgroup barrier; MFMAs may cross it
      asm volatile("" ::: "memory");
      __builtin_amdgcn_s_barrier();
      asm volatile("" ::: "memory");
    };
    // the loads of a slice past the stream's end: offsets outside every
    // buffer (zeros, or for rows already marked out of range other bytes of
    // the same buffers) into a slot no wave reads again
    static_assert(!BIG || (S & (S - 1)) == 0, "ring slots by mask");
    const uint32_t sbase = __builtin_amdgcn_readfirstlane(lds_addr(smem));  // LDS address of slot 0
    const uint32_t wb = (uint32_t)(BM * RB + wave * JB * 1024), wa = (uint32_t)(wave * JA * 1024);
    auto issue_past = [&](int zs) {
      const uint32_t d = sbase + ((uint32_t)zs & (S - 1)) * STAGE;
#pragma unroll
      for (int j = 0; j < JB; ++j) dma16a(rb, d + wb + j * 1024, vb[j], kOOB);
#pragma unroll
      for (int j = 0; j < JA; ++j) dma16a(ra, d + wa + j * 1024, va[j], kOOB);
    };
    // prologue: slices 0 .. S - 2 went out above (those that exist); the
    // others go out past the end, so S - 2 slices' loads follow every slice
    // and each wait below has one count
#pragma unroll
    for (int s = 1; s < S - 1; ++s)
      if (s >= nz) issue_past(s);
    wait_vm<vm_cap((S - 2) * PER)>();
    barrier();
    if (S - 1 < nz) issue(S - 1);  // a slot not read yet
    else issue_past(S - 1);
#pragma unroll
    for (int f = 0; f < NFK; ++f) frag_read(0, smem, 0, f);
    int z = 0;
    // where the loads of slice z + S stand: its tile and its place in it
    int in = (S - 1) / nk, kn = (S - 1) % nk;
#pragma nounroll
    for (int it = 0; it < my_tiles; ++it) {
      zero_acc();
#pragma nounroll
      for (int kt = 0; kt < nk; ++kt, ++z) {
        const char *la = smem + ((uint32_t)z & (S - 1)) * STAGE;
        uint32_t dst = 0, kb = 0;  // the DMA slot and K offset of slice z + S
        const char *nla = smem;    // where slice z + 1 sits
        bool live = false;
        auto dma = [&](int q) {  // DMA load q of slice z + S (B rows, then A rows)
          if (q < JB) dma16a(rb, dst + wb + q * 1024, vb[q], kb);
          else dma16a(ra, dst + wa + (q - JB) * 1024, va[q - JB], kb);
        };
#pragma unroll
        for (int ks = 0; ks + 1 < NKS; ++ks) {
          const int cb = ks & 1;
#pragma unroll
          for (int m = 0; m < NM; ++m) {
            mma_one(cb, m);
            if (m < NFK) frag_read(cb ^ 1, la, ks + 1, m);
            if (ks == NKS - 2) {
              if (m == NFK) {
                // the ring's bookkeeping, between MFMAs that carry no read
                if (++kn == nk) { kn = 0; ++in; }
                live = z + S < nz;
                dst = sbase + ((uint32_t)z & (S - 1)) * STAGE;  // slot of slices z and z + S
                kb = live ? (uint32_t)kn * RB : kOOB;           // past the end: as issue_past
                nla = smem + ((uint32_t)(z + 1) & (S - 1)) * STAGE;
              } else if (m == NFK + 1) {
                // this wave's reads of slot z % S are done (the wait covers
                // them); slice z + 1 has landed once every wave is here
                if (z + 1 <= st_until) wait_vm<vm_cap((S - 2) * PER + NST)>();
                else wait_vm<vm_cap((S - 2) * PER)>();
                bar();
                // (uniform) a new tile's load offsets and metadata, after the
                // barrier: its metadata slot may be the one an epilogue just read
                if (live && kn == 0) setup_b(in), setup_a(in);
              } else if (m > NFK + 1) {
                dma(m - NFK - 2);  // the first DMA loads go out here already
              }
            }
            __builtin_amdgcn_sched_barrier(0);
          }
        }
        constexpr int cb = (NKS - 1) & 1;
        // last k-step: the remaining DMA loads of slice z + S, then the reads
        // of slice z + 1's first fragments, spread over its MFMAs
        constexpr int D0 = NM - NFK - 2;            // DMA loads issued in the k-step before
        constexpr int NL = NDMA - D0 + NFK;         // memory instructions of this k-step
        static_assert(!BIG || (D0 >= 0 && D0 <= NDMA && NL <= 2 * NM), "memory instructions a MFMA");
#pragma unroll
        for (int m = 0; m < NM; ++m) {
          mma_one(cb, m);
          // memory instruction q follows MFMA q * NM / NL
#pragma unroll
          for (int q = 0; q < NL; ++q) {
            if (q * NM / NL != m) continue;
            if (q < NDMA - D0) dma(D0 + q);
            else frag_read(cb ^ 1, nla, 0, q - (NDMA - D0));
          }
          __builtin_amdgcn_sched_barrier(0);
        }
      }
      epilogue(z - 1);
    }
    wait_vm<0>();  // the loads past the end of the stream have landed
  } else {
    for (int z = 0; z < nz; ++z) {
      wait_slice(z);
      barrier();
      if (z + S - 1 < nz) issue(z + S - 1);
      const int kt = z % nk;
      if (kt == 0) zero_acc();
      const char *la = smem + (z % S) * STAGE;
      const char *lb = la + BM * RB;
      // fragments of k-step ks + 1 are read while the MFMAs of k-step ks run
      Frag fa[2][TM], fb[2][TN][NSETS];
      auto load_frags = [&](int buf, int ks) {
#pragma unroll
        for (int i = 0; i < TM; ++i)
          fa[buf][i] = Mm::ld(la + frag_addr(ks, wm * (BM / WM) + i * 32 + (lane & 31)));
#pragma unroll
        for (int j = 0; j < TN; ++j)
#pragma unroll
          for (int s = 0; s < NSETS; ++s)
            fb[buf][j][s] = bfrag(lb, ks, s * BN + wn * (BN / WN) + j * 32 + (lane & 31));
      };
      load_frags(0, 0);
#pragma unroll
      for (int ks = 0; ks < NKS; ++ks) {
        if (ks + 1 < NKS) load_frags((ks + 1) & 1, ks + 1);
#pragma unroll
        for (int i = 0; i < TM; ++i)
#pragma unroll
          for (int j = 0; j < TN; ++j)
#pragma unroll
            for (int s = 0; s < NSETS; ++s)
              acc[i][j][s] = Mm::mma(fb[ks & 1][j][s], fa[ks & 1][i], acc[i][j][s]);
      }
      if (kt == nk - 1) epilogue(z);
    }
  }
}

template <typename T, int NSETS, int EPI, int BM, int BN, int WM, int WN, int S, int RB,
          bool WQ = false>
__global__ __launch_bounds__(64 * WM * WN) void grouped_gemm(GemmArgs g) {
  gemm_body<T, NSETS, EPI, BM, BN, WM, WN, S, RB, WQ>(g);
}

// The four-wave 256-row tiles: one wave a SIMD, which may then hold the whole
// register file (256 accumulator registers for its 128-row block).
template <typename T, int NSETS, int EPI, int BM, int BN, int WM, int WN, int S, int RB>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 1))) void grouped_gemm_w4(
    GemmArgs g) {
  gemm_body<T, NSETS, EPI, BM, BN, WM, WN, S, RB, false>(g);
}

// ---- Register-weight tiles ---------------------------------------------------
// weight slices in the register ring, activation slices loaded ahead
constexpr int kRwD = 4, kRwDA = 2;
// weight-load cache policy: non-temporal for plain layers (gpt-oss-sized w2 at 4096
// tokens 502 -> 475 us), the default for gated ones (w13 933 -> 965 us non-temporal)
template <int NSETS> constexpr int kAuxW = NSETS == 1 ? 2 : 0;
//
// Layers with about 48 - 176 rows an expert stream their weights: each weight
// slice is read from HBM once per m-tile and used by few rows, and an LDS ring,
// which holds activation and weight slices together, keeps at most two weight
// slices in flight.  Here each of the four waves (one a SIMD) loads its own 64
// weight rows straight into registers, D - 1 slices ahead (a ring of D slices:
// 4 x D x 8 KB a CU), and only the activation rows go through LDS, by direct-
// to-LDS loads DA slices ahead into a ring of D slots.  Every wave covers all
// BM rows of the tile, so an expert with up to BM rows has one m-tile and each
// weight slice is streamed once for it.
//
// v_mfma_f32_16x16x32_bf16 with the weight fragment first: lane l supplies 16
// bytes (8 K elements) of weight row l % 16 at K chunk l / 16 of a 32-deep
// k-step (built from whole-line loads, below); the activation fragment is the
// same 16 bytes of row l % 16 of a 16-row block, read from LDS.  Lane l ends
// with weight positions 4 (l / 16) + [0, 4) of token row l % 16.  A wave's
// weight rows form 16-row half blocks h = 0, 1: position i of half h is output
// column 8 (i / 4) + 4 h + i % 4, so a lane holds 8 consecutive output columns
// of one row (one 16-byte store); gated layers load the gate rows of those
// columns into blocks 0, 1 and the up rows into blocks 2, 3 (the same lane and
// register for both halves of a pair).
//
// vmcnt retires loads in issue order, so a wait for one load is a wait for all
// older ones: the activation loads of a slice go out before its weight loads,
// DA < D slices ahead, and each slice's single barrier waits for the
// activation rows of the next slice only.  The weight loads are compiler-
// visible (it places their waits); the direct-to-LDS loads are not, and the
// barrier's wait counts every load issued after them.
template <int NSETS, int EPI, int BM, int D, int DA>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 1))) void grouped_gemm_rw(
    GemmArgs g) {
  constexpr int RB = 128;                   // bytes of a row's K-slice: 64 bf16, two k-steps
  constexpr int NKS = 2;
  constexpr int TMB = BM / 16;              // 16-row blocks
  constexpr int WC = 64 / NSETS;            // output columns of a wave
  constexpr int BN = 4 * WC;                // output columns of a tile
  constexpr int JA = BM * RB / 1024 / 4;    // 1 KB activation loads a wave a slice
  constexpr int NSL = DA + 3;               // metadata slots
  constexpr int SLOT = BM * RB;             // bytes of an LDS slot
  constexpr bool META = EPI == EPI_Y || EPI == EPI_OUT;
  static_assert(JA * 4 * 1024 == BM * RB, "tile rows");
  static_assert(D >= 2 && DA >= 1 && DA < D, "rings");
  static_assert((EPI == EPI_RELU2 || EPI == EPI_Y || EPI == EPI_OUT) == (NSETS == 1),
                "gated epilogues take two weight sets");
  typedef float f32x4_t __attribute__((ext_vector_type(4)));

  __shared__ __attribute__((aligned(16))) char s_a[D * SLOT];
  __shared__ int s_ts[kMaxExperts + 1];
  __shared__ int s_off[kMaxExperts + 1];
  __shared__ i32x2_t s_meta[META ? NSL : 1][META ? BM : 1];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int E = g.E, K = g.K, Nout = g.Nout;
  if (wave == 0) tile_starts<BM>(g, s_ts, s_off, lane);
  __syncthreads();
  const int n_nt = (Nout + BN - 1) / BN;
  const TileShare share = tile_share(s_ts[E] * n_nt);
  const int first = share.first, gx = share.stride, my_tiles = share.count;
  const int kbytes = K * 2;
  const int nk = K / 64;         // rows hold whole slices (the host checks)
  const int nz = my_tiles * nk;  // slices of this workgroup's stream
  if (nz == 0) return;
  const __amdgpu_buffer_rsrc_t ra = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<void *>(g.A), (short)0, (int)g.a_bytes, kRsrcWord3);
  const __amdgpu_buffer_rsrc_t rc =
      __builtin_amdgcn_make_buffer_rsrc(g.C, (short)0, (int)g.c_bytes, kRsrcWord3);
  const uint32_t w_bytes = (uint32_t)NSETS * Nout * kbytes;
  const float nal = -g.prm.alpha * 1.44269504088896341f;
  const int fi = lane & 15, fq = lane >> 4;  // fragment row and K chunk
  const uint32_t sbase = __builtin_amdgcn_readfirstlane(lds_addr(s_a));

  // ---- weights: 8 loads a lane a slice, register ring of D slices ----------
  // A 16-row weight block cb of a slice is two 1 KB loads of whole 128-byte
  // row pieces: X holds rows 0-7, Y rows 8-15 of the block; lane l takes row
  // l % 8 and, for lanes with bit 3 clear, chunks l / 16 (X) and 4 + l / 16
  // (Y), the other way round for lanes with bit 3 set.  Then k-step 0's
  // fragment (row l % 16, chunk l / 16) is X or Y in the lane's own register
  // (bit 3 picks), and k-step 1's (chunk 4 + l / 16) is the other choice
  // taken from lane l ^ 8 (a DPP rotate by 8 within each 16-lane row).  A
  // slice's loads go out together, D - 1 slices ahead, into the slot the
  // previous slice has finished with, and become fragments at the start of
  // their slice.  The K offset goes in the scalar offset field (a slice past
  // the stream's end: out of range, zeros).
  u32x4_t wr[D][NKS][4];  // [slot][X / Y, then k-step][block]
  __amdgpu_buffer_rsrc_t rb = ra;
  uint32_t vb[2][4];
  int ib = 0, kb = -1;  // tile and slice of the weight loads in progress
  bool blive = false;
  const bool hi8 = (lane & 8) != 0;
  auto setup_b = [&](int i) __attribute__((always_inline)) {
    const TileInfo t = tile_info<BM, BN>(first + i * gx, s_ts, s_off, E, n_nt);
    rb = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<char *>(reinterpret_cast<const char *>(g.W)) + (size_t)t.e * w_bytes,
        (short)0, (int)w_bytes, kRsrcWord3);
#pragma unroll
    for (int cb = 0; cb < 4; ++cb) {
#pragma unroll
      for (int xy = 0; xy < 2; ++xy) {
        const int pos = 8 * xy + (lane & 7);  // position in the block: its output column
        const int chunk = (lane >> 4) + ((((lane >> 3) & 1) ^ xy) ? 4 : 0);
        const int h = cb & 1, set = NSETS == 2 ? cb >> 1 : 0, pair = NSETS == 2 ? 0 : cb >> 1;
        const int col = t.n0 + wave * WC + 32 * pair + 8 * (pos >> 2) + 4 * h + (pos & 3);
        const int row = NSETS == 1 ? col
                        : g.interleaved ? 2 * col + set
                                        : set * Nout + col;
        vb[xy][cb] =
            col < Nout ? (uint32_t)row * (uint32_t)kbytes + (uint32_t)(chunk * 16) : kOOB;
      }
    }
  };
  auto advance_b = [&](int zb) __attribute__((always_inline)) {  // slice zb's weight loads begin
    if (++kb == nk) { kb = 0; ++ib; }
    blive = zb < nz;
    if (blive && kb == 0) setup_b(ib);
  };
  auto load_b = [&](int xy, int cb) __attribute__((always_inline)) -> u32x4_t {
    const uint32_t k = blive ? (uint32_t)(kb * RB) : kOOB;
    return __builtin_amdgcn_raw_buffer_load_b128(rb, vb[xy][cb], __builtin_amdgcn_readfirstlane(k),
                                                 kAuxW<NSETS>);
  };
  // X, Y of block cb in slot u -> k-step 0 and (still to rotate) k-step 1
  auto frag_select = [&](int u, int cb) __attribute__((always_inline)) {
    const u32x4_t x = wr[u][0][cb], y = wr[u][1][cb];
    u32x4_t f0, t;
#pragma unroll
    for (int d = 0; d < 4; ++d) {
      f0[d] = hi8 ? y[d] : x[d];
      t[d] = hi8 ? x[d] : y[d];
    }
    wr[u][0][cb] = f0;
    wr[u][1][cb] = t;
  };
  auto frag_rotate = [&](int u, int cb) __attribute__((always_inline)) {
#pragma unroll
    for (int d = 0; d < 4; ++d)
      wr[u][1][cb][d] = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)wr[u][1][cb][d],
                                                              0x128 /* row_ror:8 */, 0xf, 0xf,
                                                              false);
  };

  // ---- activations: JA direct-to-LDS loads a wave a slice --------------------
  // load j of wave w fills slot bytes [1024 (w JA + j), + 1024): row
  // 8 (w JA + j) + lane / 8, physical chunk lane % 8, which holds the row's
  // logical chunk (lane % 8) ^ key(row)
  uint32_t va[JA];
  int gidx[JA];   // the next tile's A row (or output row) per load, fetched a tile ahead
  float gsc[JA];  // and its routing weight (w2)
  int ia = 0, ka = -1;  // tile and slice of the activation loads in progress
  bool alive = false;
  auto arow_of = [&](int j) __attribute__((always_inline)) { return (wave * JA + j) * 8 + (lane >> 3); };
  auto fetch_idx = [&](int i) __attribute__((always_inline)) {  // gather indices / metadata of tile i
    if (i >= my_tiles) return;
    const TileInfo t = tile_info<BM, BN>(first + i * gx, s_ts, s_off, E, n_nt);
#pragma unroll
    for (int j = 0; j < JA; ++j) {
      const int p = t.row0 + min(arow_of(j), t.rows - 1);  // rows past the tile: any valid entry
      gidx[j] = (g.gather || EPI == EPI_OUT) ? g.col_sorted[p] : p;
      if constexpr (META)
        gsc[j] = !g.gate_scal ? 1.f
                 : g.gate_bf16 ? to_f32(reinterpret_cast<const bf16_t *>(g.gate_scal)[p])
                               : reinterpret_cast<const float *>(g.gate_scal)[p];
    }
  };
  auto setup_a = [&](int i) __attribute__((always_inline)) {
    const TileInfo t = tile_info<BM, BN>(first + i * gx, s_ts, s_off, E, n_nt);
#pragma unroll
    for (int j = 0; j < JA; ++j) {
      const int r = arow_of(j), p = t.row0 + r;
      const uint32_t arow = g.gather ? (uint32_t)(gidx[j] / g.topk) : (uint32_t)p;
      va[j] = r < t.rows ? arow * (uint32_t)kbytes + (uint32_t)(((lane & 7) ^ swz_key<RB>(r)) << 4)
                         : kOOB;
      if (META && (lane & 7) == 0 && r < t.rows) {
        i32x2_t m;
        m[0] = EPI == EPI_OUT ? gidx[j] : p;  // topk == 1: entry index == token
        m[1] = __float_as_int(gsc[j]);
        s_meta[i % NSL][r] = m;
      }
    }
    fetch_idx(i + 1);
  };
  auto advance_a = [&](int za) __attribute__((always_inline)) {  // slice za's activation loads begin
    if (++ka == nk) { ka = 0; ++ia; }
    alive = za < nz;
    if (alive && ka == 0) setup_a(ia);
  };
  auto dma_a = [&](int slot, int j) __attribute__((always_inline)) {
    const uint32_t k = alive ? (uint32_t)(ka * RB) : kOOB;
    dma16a(ra, sbase + (uint32_t)(slot * SLOT + (wave * JA + j) * 1024), va[j],
           __builtin_amdgcn_readfirstlane(k));
  };

  // ---- fragments: group q of a slice is k-step q / TMB, row block q % TMB;
  // a ring of FR registers read L groups ahead
  constexpr int NG = NKS * TMB, FR = 4, L = 3;
  static_assert(NG % FR == 0 && L < FR, "fragment ring");
  bf16x8_t af[FR];
  // row 16 i + fi has swizzle key fi / 2 for every block i; k-step 1's chunk
  // (4 + fq) flips bit 6 of k-step 0's address
  const int rbase = swz<RB>(fi, fq);
  auto read_frag = [&](int slot, int q) __attribute__((always_inline)) -> bf16x8_t {
    const int ks = q / TMB, i = q % TMB;
    return *reinterpret_cast<const bf16x8_t *>(s_a + slot * SLOT + i * 16 * RB +
                                              (ks ? (rbase ^ 64) : rbase));
  };

  f32x4_t acc[TMB][4];
  // zeros the compiler cannot see through: otherwise it folds them into the
  // next MFMAs and splits the stream into zeroed and running copies
  auto zero_acc = [&]() __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < TMB; ++i)
#pragma unroll
      for (int cb = 0; cb < 4; ++cb) {
        acc[i][cb] = f32x4_t{0.f, 0.f, 0.f, 0.f};
        asm volatile("" : "+a"(acc[i][cb]));
      }
  };
  int ic = 0, kc = 0;  // the tile and slice being multiplied
  int nrb = TMB;       // 16-row blocks of that tile holding rows (the others multiply zeros)

  auto epilogue = [&]() __attribute__((always_inline)) {
    const TileInfo t = tile_info<BM, BN>(first + ic * gx, s_ts, s_off, E, n_nt);
#pragma unroll
    for (int i = 0; i < TMB; ++i) {
#pragma unroll
      for (int cb = 0; cb < 4; ++cb) asm volatile("" : "+a"(acc[i][cb]));
      const int m = i * 16 + fi;
      const bool ok = m < t.rows;
      uint32_t orow = (uint32_t)(t.row0 + m);
      float gs = 1.f;
      if constexpr (META) {
        const i32x2_t md = s_meta[ic % NSL][ok ? m : 0];
        orow = (uint32_t)md[0];
        gs = __int_as_float(md[1]);
      }
#pragma unroll
      for (int pr = 0; pr < 2 / NSETS; ++pr) {
        float v[8];
#pragma unroll
        for (int q = 0; q < 8; ++q) {
          const float a0 = acc[i][2 * pr + (q >> 2)][q & 3];
          if constexpr (META) v[q] = a0 * gs;
          else v[q] = act_val<EPI>(a0, acc[i][NSETS == 2 ? 2 + (q >> 2) : 0][q & 3], nal, g.prm);
        }
        const u32x4_t o = {pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3]),
                           pack_bf16x2(v[4], v[5]), pack_bf16x2(v[6], v[7])};
        const int col = t.n0 + wave * WC + 32 * pr + 8 * fq;
        // Nout is a multiple of 8, so col < Nout covers all eight columns
        const uint32_t off =
            (ok && col < Nout) ? (orow * (uint32_t)Nout + (uint32_t)col) * 2u : kOOB;
        __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(i32x4_t, o), rc, (int)off, 0, 0);
      }
      __builtin_amdgcn_sched_barrier(0);
    }
  };

  // ---- the stream: per slice NG groups of four MFMAs, each followed by the
  // fragment read L groups ahead and at most one memory operation:
  //   groups [0, JA): slice z + DA's activation loads into slot (z + DA) % D;
  //   groups [G1, G1 + 8): the weight loads of slice z + D - 1 into the slot
  //     slice z - 1 used (X and Y of each block back to back);
  //   groups [1, 5): k-step 1's fragments rotated into place;
  //   at group NG - L (before the first read of slice z + 1): the wait for
  //     slice z + 1's activation rows and the barrier.
  constexpr int G1 = JA;
  static_assert(G1 + 8 <= NG - L, "memory operations a slice");
  // loads issued after slice z + 1's activation loads (slice z + 1 - DA) up to
  // that wait: the weight loads of that slice, then whole slices
  constexpr int VWAIT = 8 + (DA - 1) * (JA + 8);
  static_assert(VWAIT < 64, "vmcnt range");

  // prologue: activation rows of slices 0 .. DA - 1, weights of slices
  // 0 .. D - 2
  fetch_idx(0);
#pragma unroll
  for (int u = 0; u < DA; ++u) {
    advance_a(u);
#pragma unroll
    for (int j = 0; j < JA; ++j) dma_a(u, j);
  }
#pragma unroll
  for (int u = 0; u < D - 1; ++u) {
    advance_b(u);
#pragma unroll
    for (int cb = 0; cb < 4; ++cb)
#pragma unroll
      for (int xy = 0; xy < 2; ++xy) wr[u][xy][cb] = load_b(xy, cb);
  }
  zero_acc();
  wait_vm<0>();
  barrier();
#pragma unroll
  for (int q = 0; q < L; ++q) af[q % FR] = read_frag(0, q);

  const int nzp = (nz + D - 1) / D * D;
#pragma nounroll
  for (int z0 = 0; z0 < nzp; z0 += D) {
    static_for<D>([&](auto uc) __attribute__((always_inline)) {
      constexpr int u = decltype(uc)::value;
      const int z = z0 + u;
      if (kc == 0 && z < nz) {
        const TileInfo t = tile_info<BM, BN>(first + ic * gx, s_ts, s_off, E, n_nt);
        nrb = __builtin_amdgcn_readfirstlane((t.rows + 15) >> 4);
      }
      // this slice's weight fragments: k-step 0 by a select, before its MFMAs
#pragma unroll
      for (int cb = 0; cb < 4; ++cb) frag_select(u, cb);
      static_for<NG>([&](auto qc) __attribute__((always_inline)) {
        constexpr int q = decltype(qc)::value;
        constexpr int ks = q / TMB, i = q % TMB;
        // row blocks past the tile's rows are skipped (a uniform branch);
        // slices past the stream's end multiply zeros into accumulators that
        // no epilogue reads again
        if (i < nrb) {
#pragma unroll
          for (int cb = 0; cb < 4; ++cb)
            acc[i][cb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                __builtin_bit_cast(bf16x8_t, wr[u][ks][cb]), af[q % FR], acc[i][cb], 0, 0, 0);
        }
        if constexpr (q == NG - L) {
          // slice z + 1's activation rows (and this wave's LDS reads) are done
          wait_vm<VWAIT>();
          barrier();
        }
        if constexpr (q + L < NG) af[(q + L) % FR] = read_frag(u, q + L);
        else af[(q + L) % FR] = read_frag((u + 1) % D, q + L - NG);
        if constexpr (q < JA) {
          if constexpr (q == 0) advance_a(z + DA);
          dma_a((u + DA) % D, q);
        }
        if constexpr (q >= G1 && q < G1 + 8) {
          constexpr int cb = (q - G1) >> 1, xy = (q - G1) & 1;
          if constexpr (q == G1) advance_b(z + D - 1);
          wr[(u + D - 1) % D][xy][cb] = load_b(xy, cb);
        }
        // k-step 1's fragments rotated into place, one block a group
        if constexpr (q >= 1 && q < 5) frag_rotate(u, q - 1);
        __builtin_amdgcn_sched_barrier(0);
      });
      if (z < nz && kc == nk - 1) {
        epilogue();
        zero_acc();
      }
      if (++kc == nk) { kc = 0; ++ic; }
    });
  }
  wait_vm<0>();  // the loads past the end of the stream have landed
}

int device_cus() {
  int dev = 0, cus = 0;
  if (hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
      cus <= 0)
    cus = 256;
  return cus;
}

template <int BM_, int BN_, int WM_, int WN_, int S_, int RB_> struct Cfg {
  static constexpr int BM = BM_, BN = BN_, WM = WM_, WN = WN_, S = S_, RB = RB_;
};
// Tile configurations, largest first (rows x output columns, waves rows x
// columns, ring stages, LDS row bytes).  Gated tiles carry 2 * BN weight rows.
using GatedL = Cfg<256, 128, 4, 2, 4, 64>;  // 8 waves, 64 x (64 + 64) each
// the same tiles with 128-byte slices in a two-stage ring, for rows of at
// least kLongRowBytes: four MFMA k-steps a phase instead of two halves the
// barriers a slice, which pays once a tile's K loop is long (skewed 64-expert
// layer, 4096-wide rows: gated w13 3270 -> 3106 us, plain ReLU^2 w13 -6 %);
// with 1536-wide rows the single slice of lookahead loses (w2 +25 %)
using GatedL2 = Cfg<256, 128, 4, 2, 2, 128>;
using PlainL2 = Cfg<256, 256, 4, 2, 2, 128>;
constexpr int kLongRowBytes = 6144;
// The bf16 256-row tiles: four waves, one a SIMD, with 128 x (64 + 64) and
// 128 x 128 register blocks.  They read a third fewer LDS bytes a MFMA than
// the eight-wave tiles (whose LDS is busy 87 % of the time on the skewed
// 64-expert layer), at the price of a loop in which every other instruction
// has to issue between MFMAs.  Measured against the eight-wave tiles on that
// layer (bit-identical): gated w13 3110 -> 3035 us with 64-byte slices in a
// four-stage ring, plain w2 1840 -> 1690 us with 128-byte slices in a
// two-stage ring (w2: 1750 us with 64-byte slices).
using GatedB = Cfg<256, 128, 2, 2, 4, 64>;
using PlainB = Cfg<256, 256, 2, 2, 2, 128>;
using GatedM = Cfg<128, 128, 2, 4, 3, 128>; // 8 waves, 64 x (32 + 32) each
// 96 - 176 rows an expert (the gpt-oss-sized layer at 2048-4096 tokens): one
// 192-row plain tile holds all of an expert's rows, where 128-row tiles give
// about half the experts a second, nearly empty tile (w2 at 4096 tokens 568 ->
// 545 us; the gated 192-row tile measured no faster than the 128-row one)
using PlainX = Cfg<192, 256, 2, 4, 2, 128>; // 8 waves, 96 x 64 each
using GatedS = Cfg<32, 128, 1, 4, 4, 128>;  // 4 waves, 32 x (32 + 32) each
using PlainL = Cfg<256, 256, 4, 2, 4, 64>;  // 8 waves, 64 x 128 each
using PlainM = Cfg<128, 128, 2, 4, 3, 128>; // 8 waves, 64 x 32 each
using PlainS = Cfg<32, 128, 1, 4, 4, 128>;  // 4 waves, 32 x 32 each
// one wave: a handful of rows against many weight columns (decode-sized
// batches), where even 32 x 128 tiles leave CUs idle during weight streaming.
// 256-byte row slices: each weight row is read in runs twice as long as with
// 128 bytes, which streams the weights ~25 % faster (gpt-oss-sized layer, one
// token: w13 50 -> 37 us, w2 38 -> 30 us); two stages keep the LDS at 48 KB,
// three workgroups a CU.
using GatedT = Cfg<32, 32, 1, 1, 2, 256>;   // 1 wave, 32 x (32 + 32)
using PlainT = Cfg<32, 32, 1, 1, 2, 256>;   // 1 wave, 32 x 32
// MXFP4 weights: the same tile shapes; deeper rings (4/6 and 6/8 stages) were
// measured slower (LDS per workgroup costs occupancy) on the gpt-oss-sized
// layer at 1, 33 and 512 tokens
// prefill-sized batches: the 8-wave ping-pong tiles (the plain one 256
// columns wide, so its code rows fill whole 1 KB wave loads)
using GatedMQ = Cfg<128, 128, 2, 4, 3, 128>;
using PlainMQ = Cfg<128, 256, 2, 4, 3, 128>;
using GatedSQ = Cfg<32, 128, 1, 4, 4, 128>;
using PlainSQ = Cfg<32, 128, 1, 4, 4, 128>;
using GatedTQ = Cfg<32, 32, 1, 1, 2, 256>;
using PlainTQ = Cfg<32, 32, 1, 1, 2, 256>;

template <typename C, int NSETS, bool WQ = false> constexpr int lds_bytes() {
  return C::S * (C::BM * C::RB + NSETS * C::BN * (WQ ? C::RB / 4 : C::RB) +
                 (WQ ? C::WM * C::WN * 256 : 0)) +
         2 * (kMaxExperts + 1) * 4 + (C::S + 1) * (16 + C::BM * 8);
}

// Upper bound on the tiles of one launch: floor(M / BM) + min(E, M) m-tiles.
inline int64_t est_tiles(int64_t M, int E, int Nout, int BM, int BN) {
  return (M / BM + (M < E ? M : E)) * ((Nout + BN - 1) / BN);
}

template <typename T, int NSETS, int EPI, typename C, bool WQ = false>
hipError_t launch_cfg(const GemmArgs &a, int64_t M, int E, hipStream_t s) {
  constexpr int LDS = lds_bytes<C, NSETS, WQ>();
  constexpr int per_cu = (160 * 1024) / LDS > 0 ? (160 * 1024) / LDS : 1;
  const int64_t tiles = est_tiles(M, E, a.Nout, C::BM, C::BN);
  int64_t grid = (int64_t)device_cus() * (per_cu < 2 ? per_cu : 2);
  if (grid > tiles) grid = tiles;
  grid = (grid + 7) / 8 * 8;  // whole XCD rounds; surplus workgroups get no tiles
  static_assert(LDS <= 160 * 1024, "LDS budget");
  if constexpr (C::WM * C::WN == 4 && C::BM == 256 && !WQ)
    hipLaunchKernelGGL((grouped_gemm_w4<T, NSETS, EPI, C::BM, C::BN, C::WM, C::WN, C::S, C::RB>),
                       dim3((unsigned)grid), dim3(256), 0, s, a);
  else
    hipLaunchKernelGGL((grouped_gemm<T, NSETS, EPI, C::BM, C::BN, C::WM, C::WN, C::S, C::RB, WQ>),
                       dim3((unsigned)grid), dim3(64 * C::WM * C::WN), 0, s, a);
  return hipGetLastError();
}

// Register-weight tiles (bf16): one workgroup a CU (four waves, one a SIMD).
template <int NSETS, int EPI, int BM>
hipError_t launch_rw(const GemmArgs &a, int64_t M, int E, hipStream_t s) {
  constexpr int BN = 4 * 64 / NSETS;
  const int64_t tiles = est_tiles(M, E, a.Nout, BM, BN);
  int64_t grid = device_cus();
  if (grid > tiles) grid = tiles;
  grid = (grid + 7) / 8 * 8;  // whole XCD rounds; surplus workgroups get no tiles
  hipLaunchKernelGGL((grouped_gemm_rw<NSETS, EPI, BM, kRwD, kRwDA>), dim3((unsigned)grid),
                     dim3(256), 0, s, a);
  return hipGetLastError();
}

// Expected tiles when the M rows spread evenly over the experts: an expert's
// last m-tile is half full on average, so about M / BM + E / 2 m-tiles.
inline int64_t expected_tiles(int64_t M, int E, int Nout, int BM, int BN) {
  const int64_t e = M < E ? M : E;
  return (M / BM + (e + 1) / 2) * ((Nout + BN - 1) / BN);
}

// Relative duration of a launch: rounds of one tile per CU times the tile's
// MFMA work, with a surcharge for tiles whose fixed per-tile cost (set-up,
// epilogue, pipeline fill) is larger relative to that work.
inline double launch_cost(int64_t tiles, int64_t cus, int BM, int BN, double surcharge) {
  return (double)((tiles + cus - 1) / cus) * BM * BN * (1.0 + surcharge);
}

// Rows per expert below 48 take the 32-row tile (weight streaming, little MFMA
// waste), and so do launches too small to give half the CUs a 128-row tile;
// when even the 32 x 128 tiles number fewer than the CUs, the 32 x 32
// one-wave tile spreads the weight stream over more CUs.
// Plain (w2) launches of 96 to 176 rows an expert on average take the 192-row
// tile (one m-tile an expert).
// Plain (w2) layers take the 256-row tile whenever those tiles still cover the
// CUs: with up to one 256-row tile per expert on average it streams each
// expert's weights about once where 128-row tiles stream them about 1.5 times
// (gpt-oss-sized w2 at 128 rows per expert), and past that the cost model's
// near-ties chose the 128-row tile at a large loss (gpt-oss-sized w2 at 256,
// 384 and 512 rows an expert: 1247 -> 845, 1761 -> 1030, 2255 -> 1258 us).  Everything else takes
// whichever tile the cost model favours: the gated 256 x 128 tile at 64-128
// rows per expert is half empty and measured 6-14 % slower than the 128-row
// tile (gpt-oss-sized layer, 2048 and 4096 tokens), and 64 plain 256-row tiles
// leave most CUs idle (minimind-sized w2 at E = 32: 22 % slower).
// MXFP4 weights take the same thresholds with their own tiles: the 32-row
// and one-wave tiles for weight-streaming batches, the 128-row ping-pong tiles
// above (no 256-row tile: its 64-byte row slices hold 16 code bytes a row,
// too few to fill the wave loads).
template <typename T, int NSETS, int EPI>
hipError_t launch_wq(const GemmArgs &a, int64_t M, int E, hipStream_t s) {
  using Md = typename std::conditional<NSETS == 2, GatedMQ, PlainMQ>::type;
  using Sm = typename std::conditional<NSETS == 2, GatedSQ, PlainSQ>::type;
  using Tn = typename std::conditional<NSETS == 2, GatedTQ, PlainTQ>::type;
  const int64_t cus = device_cus();
  if (M < 48 * (int64_t)E || expected_tiles(M, E, a.Nout, Md::BM, Md::BN) < cus / 2) {
    if (expected_tiles(M, E, a.Nout, Sm::BM, Sm::BN) < cus)
      return launch_cfg<T, NSETS, EPI, Tn, true>(a, M, E, s);
    return launch_cfg<T, NSETS, EPI, Sm, true>(a, M, E, s);
  }
  return launch_cfg<T, NSETS, EPI, Md, true>(a, M, E, s);
}

template <typename T, int NSETS, int EPI>
hipError_t launch_t(const GemmArgs &a, int64_t M, int E, hipStream_t s) {
  using L = typename std::conditional<NSETS == 2, GatedL, PlainL>::type;
  using Md = typename std::conditional<NSETS == 2, GatedM, PlainM>::type;
  using Sm = typename std::conditional<NSETS == 2, GatedS, PlainS>::type;
  using Tn = typename std::conditional<NSETS == 2, GatedT, PlainT>::type;
  if constexpr (std::is_same<T, bf16_t>::value) {
    if (a.wscale) return launch_wq<T, NSETS, EPI>(a, M, E, s);
  }
  const int64_t cus = device_cus();
  const int64_t tm = expected_tiles(M, E, a.Nout, Md::BM, Md::BN);
  // below 48 rows an expert the 32-row tiles give every expert with more than
  // 32 rows a second m-tile (a second pass over its weights); a register-weight
  // tile keeps one where its tiles cover the CUs (gpt-oss-sized layer, w13 / w2
  // in us: 1024 tokens 863 / 602 -> 805 / 411, 1280 tokens 1064 / 773 -> 811 /
  // 427, 768 tokens w2 464 -> 401, 512 tokens w2 426 -> 386, all on the 192-row
  // tile; gated at 16 and 24 rows an expert it loses, 673 -> 796 and 715 ->
  // 799).  Plain layers of 16 - 96 rows an expert take the 128-row one (fewer
  // activation loads of padding rows: w2 at 768 - 3072 tokens 4 - 8 % faster
  // than on the 192-row tile, 464 -> 427 us at 2048), gated ones of 32 - 47 the
  // 192-row one (on the 128-row tile gated layers measured -4 % to +3 %).
  if constexpr (std::is_same<T, bf16_t>::value) {
    if constexpr (NSETS == 1) {
      if (a.K % 64 == 0 && M >= 16 * (int64_t)E && M <= 96 * (int64_t)E &&
          expected_tiles(M, E, a.Nout, 128, 4 * 64) >= cus)
        return launch_rw<NSETS, EPI, 128>(a, M, E, s);
    } else {
      if (a.K % 64 == 0 && M >= 32 * (int64_t)E && M < 48 * (int64_t)E &&
          expected_tiles(M, E, a.Nout, 192, 4 * 64 / NSETS) >= cus)
        return launch_rw<NSETS, EPI, 192>(a, M, E, s);
    }
  }
  if (M < 48 * (int64_t)E || tm < cus / 2) {
    if (expected_tiles(M, E, a.Nout, Sm::BM, Sm::BN) < cus)
      return launch_cfg<T, NSETS, EPI, Tn>(a, M, E, s);
    return launch_cfg<T, NSETS, EPI, Sm>(a, M, E, s);
  }
  // register-weight tiles (bf16, rows of whole 64-element slices): plain layers
  // of 48 - 176 rows an expert, gated ones of 96 - 176 (at 64 rows an expert
  // the gated 128-row ping-pong tile measured faster: gpt-oss-sized w13 at
  // 2048 tokens 791 vs 829 us; at 4096 tokens 986 vs 905 us)
  if constexpr (std::is_same<T, bf16_t>::value) {
    if (a.K % 64 == 0 && M >= (NSETS == 2 ? 96 : 48) * (int64_t)E && M <= 176 * (int64_t)E)
      return launch_rw<NSETS, EPI, 192>(a, M, E, s);
    // gated layers of 177 - 240 rows an expert: the 256-row register-weight
    // tile keeps one m-tile an expert (gpt-oss-sized w13 at 6144 tokens 1278 ->
    // 1159 us, 7168: 1353 -> 1172; the 256-row LDS tile 1167 / 1201; at 256
    // rows an expert it loses, 1587 -> 1615), where its tiles cover the CUs
    if constexpr (NSETS == 2) {
      if (a.K % 64 == 0 && M > 176 * (int64_t)E && M <= 240 * (int64_t)E &&
          expected_tiles(M, E, a.Nout, 256, 4 * 64 / NSETS) >= cus)
        return launch_rw<NSETS, EPI, 256>(a, M, E, s);
    }
  }
  if constexpr (NSETS == 1) {
    if (M >= 96 * (int64_t)E && M <= 176 * (int64_t)E &&
        expected_tiles(M, E, a.Nout, PlainX::BM, PlainX::BN) >= cus)
      return launch_cfg<T, NSETS, EPI, PlainX>(a, M, E, s);
  }
  // the 256-row tile: in bf16 the four-wave one (its loop takes rows of
  // whole slices), else the eight-wave one with 128-byte slices for long
  // bf16 rows; fp32 layers keep the 64-byte slices
  using L2 = typename std::conditional<NSETS == 2, GatedL2, PlainL2>::type;
  using B4 = typename std::conditional<NSETS == 2, GatedB, PlainB>::type;
  auto launch_l = [&]() {
    if constexpr (std::is_same<T, bf16_t>::value) {
      const int64_t rowb = (int64_t)a.K * (int64_t)sizeof(T);
      if (rowb % B4::RB == 0) return launch_cfg<T, NSETS, EPI, B4>(a, M, E, s);
      if (rowb >= kLongRowBytes) return launch_cfg<T, NSETS, EPI, L2>(a, M, E, s);
    }
    return launch_cfg<T, NSETS, EPI, L>(a, M, E, s);
  };
  if (NSETS == 1 && expected_tiles(M, E, a.Nout, L::BM, L::BN) >= cus) return launch_l();
  const double cl = launch_cost(expected_tiles(M, E, a.Nout, L::BM, L::BN), cus, L::BM, L::BN, 0.0);
  const double cm = launch_cost(tm, cus, Md::BM, Md::BN, 0.15);
  if (cl <= cm) return launch_l();
  return launch_cfg<T, NSETS, EPI, Md>(a, M, E, s);
}

}  // namespace

hipError_t launch_gemm1(const void *x, const void *w13, void *act_out, const int32_t *offsets,
                        const int32_t *col_sorted, moe_dtype_t dt, int64_t n_tokens, int topk,
                        int n_experts, int hidden, int inter, moe_act_t act,
                        moe_w13_layout_t layout, ActParams p, hipStream_t s, bool sorted_rows,
                        const uint8_t *w13_scale) {
  const int64_t M = n_tokens * topk;
  const size_t es = dt == MOE_BF16 ? 2 : 4;
  // A is x [N, hidden] read through the gather index, or (sorted_rows) rows
  // already in sorted order [M, hidden]
  const int64_t a_rows = sorted_rows ? M : n_tokens;
  GemmArgs a{x, w13, act_out, offsets, col_sorted, nullptr, (uint32_t)(a_rows * hidden * es),
             (uint32_t)(M * inter * es), 0, n_experts, hidden, inter, topk, sorted_rows ? 0 : 1,
             layout == MOE_W13_INTERLEAVED, act, p, w13_scale};
  const bool gated = act != MOE_ACT_RELU2;
  const bool clamp = std::isfinite(p.limit);  // an infinite limit clamps nothing
  if (gemv_fits(dt, n_tokens, topk, n_experts, hidden, inter, w13_scale != nullptr))
    return launch_gemv(a, gated ? 2 : 1, !gated ? EPI_RELU2 : clamp ? EPI_GATED_CLAMP : EPI_GATED,
                       n_tokens, M, s);
  if (dt == MOE_BF16)
    return !gated  ? launch_t<bf16_t, 1, EPI_RELU2>(a, M, n_experts, s)
           : clamp ? launch_t<bf16_t, 2, EPI_GATED_CLAMP>(a, M, n_experts, s)
                   : launch_t<bf16_t, 2, EPI_GATED>(a, M, n_experts, s);
  return !gated  ? launch_t<float, 1, EPI_RELU2>(a, M, n_experts, s)
         : clamp ? launch_t<float, 2, EPI_GATED_CLAMP>(a, M, n_experts, s)
                 : launch_t<float, 2, EPI_GATED>(a, M, n_experts, s);
}

hipError_t launch_gemm2(const void *act_in, const void *w2, void *y, const int32_t *offsets,
                        const int32_t *col_sorted, const void *gate_scal, moe_dtype_t gate_dt,
                        moe_dtype_t dt, int64_t n_tokens, int topk, int n_experts, int hidden,
                        int inter, bool direct_out, hipStream_t s, const uint8_t *w2_scale) {
  const int64_t M = n_tokens * topk;
  const size_t es = dt == MOE_BF16 ? 2 : 4;
  const int64_t c_rows = direct_out ? n_tokens : M;
  GemmArgs a{act_in, w2, y, offsets, col_sorted, gate_scal, (uint32_t)(M * inter * es),
             (uint32_t)(c_rows * hidden * es), gate_dt == MOE_BF16, n_experts, inter, hidden,
             topk, 0, 0, 0, ActParams{1.f, 0.f, 0.f}, w2_scale};
  if (gemv_fits(dt, n_tokens, topk, n_experts, inter, hidden, w2_scale != nullptr, true))
    return launch_gemv(a, 1, direct_out ? EPI_OUT : EPI_Y, n_tokens, M, s);
  if (dt == MOE_BF16)
    return direct_out ? launch_t<bf16_t, 1, EPI_OUT>(a, M, n_experts, s)
                      : launch_t<bf16_t, 1, EPI_Y>(a, M, n_experts, s);
  return direct_out ? launch_t<float, 1, EPI_OUT>(a, M, n_experts, s)
                    : launch_t<float, 1, EPI_Y>(a, M, n_experts, s);
}

}  // namespace moe
