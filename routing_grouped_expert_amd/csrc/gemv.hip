// Decode-sized grouped expert GEMMs on gfx950: a few rows per expert against
// the expert's whole weight matrix, as matrix-vector products.
//
// What is computed is the expert FFN of grouped_gemm.hip (w13 with the fused
// activation, or w2 with the routing weight), the one the minimind issue #835
// page ("Summary") and the vLLM PR #47106 report (activation kinds, w13
// layouts) describe.  With at most a handful of tokens the layer is a weight
// stream: every weight is read once and used by a few rows, so the
// kernel is shaped for bytes in flight, not for matrix-core reuse.
//
// Design (this file's own):
//  * One workgroup of four waves per (expert with rows, block of output
//    columns); grid.y counts the experts that have rows, and a workgroup finds
//    its expert with a scan of the device-side offsets.
//  * A wave owns RPW weight rows (the gate and up rows of its columns, or the
//    plain rows) and loads all of them, whole, into registers before anything
//    else: lane l holds the K elements 8 (l + 64 t) .. + 7 of every row, t < T.
//    That is ~23 KB a wave in flight at K = 2880 with bf16 weights (4 rows,
//    16-byte loads) and ~12 KB with MXFP4 weights (8 rows of E2M1 codes,
//    4-byte loads), so a few waves a CU cover HBM latency.  The weight loads
//    are non-temporal: each weight is read once.
//  * The A rows of the expert (the gathered token rows, or the sorted
//    activation rows) are staged in LDS, cb at a time; each lane reads the
//    16-byte pieces matching its weight pieces.  Products accumulate in fp32
//    with v_dot2_f32_bf16, two K elements per instruction, in the same order
//    for bf16 and for MXFP4 weights (the FP4 codes are first turned into bf16
//    with the hardware's scaled conversion, exactly).
//  * The RPW per-lane partial sums are reduced across the wave by halving:
//    each exchange step a lane keeps half of its values and adds its
//    partner's copy of that half, until a lane holds the gate and up sums of
//    one output column (or the one sum of a plain column); the remaining lane
//    bits are summed out.  Then one lane per column runs the epilogue.
//  * MXFP4 scales: the 4 lanes that share a K-block load the 8 scale bytes of
//    the wave's rows as dwords and broadcast them inside the quad with DPP, so
//    no lane loads single bytes.
#include "gemm_common.h"
#include "lds_dma.h"

namespace moe {
namespace {

constexpr int kGemvWaves = 4;
// Cache policy of the weight loads: non-temporal (nt).  Every weight is read
// once a layer, so keeping it out of the caches' retention leaves them to the
// activation rows and routing data: measured 10-11 % faster at 8-33 tokens of
// a gpt-oss-sized layer and 6 % on a 24-layer decode stack (cold weights).
constexpr int kWeightCpol = 2;
// weight rows a wave streams.  FP4 rows are a quarter of the bytes, but 16
// of them a wave (as many bytes in flight as 4 bf16 rows) measured 20 % slower
// than 8 at one token: the per-row decode and dot products, not the loads,
// bound those waves, and 8 rows give twice the workgroups.
constexpr int kRowsBf16 = 4, kRowsFp4 = 8;
template <bool WQ> constexpr int rows_per_wave() { return WQ ? kRowsFp4 : kRowsBf16; }
constexpr int kGemvLdsBudget = 48 * 1024;  // LDS for staged A rows

// acc + a.lo * b.lo + a.hi * b.hi on packed bf16 pairs (v_dot2_f32_bf16)
__device__ __forceinline__ float dot2(uint32_t a, uint32_t b, float acc) {
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, a),
                                         __builtin_bit_cast(bf16x2_t, b), acc, false);
}

// Cross-lane sum of V values per lane.  Halving steps (exchange distance 32,
// 16, ...) run until NKEEP values remain: a lane with the distance bit set
// keeps the upper half of its values, the others the lower half, each adding
// the partner's copy of the half it keeps.  The NKEEP survivors are then
// summed over the remaining lane bits.  On return v[0 .. NKEEP) of lane l are
// the full sums of the values with indices base .. base + NKEEP - 1, where
// base = sum over the halving steps of (V_step / 2 if lane l has that bit).
template <int V, int NKEEP>
__device__ __forceinline__ void wave_sum(float (&v)[V], int lane) {
  int m = 32;
#pragma unroll
  for (int n = V; n > NKEEP; n /= 2, m >>= 1) {
    const bool hi = (lane & m) != 0;
#pragma unroll
    for (int j = 0; j < n / 2; ++j) {
      const float send = hi ? v[j] : v[j + n / 2];
      const float keep = hi ? v[j + n / 2] : v[j];
      v[j] = keep + __shfl_xor(send, m);
    }
  }
#pragma unroll
  for (; m >= 1; m >>= 1)
#pragma unroll
    for (int j = 0; j < NKEEP; ++j) v[j] += __shfl_xor(v[j], m);
}

// Lane distance of the last halving step of wave_sum<V, NKEEP> (the lanes
// below it hold equal sums).
template <int V, int NKEEP> constexpr int last_halving() {
  int m = 64;
  for (int n = V; n > NKEEP; n /= 2) m >>= 1;
  return m;
}

template <int CTRL> __device__ __forceinline__ uint32_t dpp_b(uint32_t v) {
  return (uint32_t)__builtin_amdgcn_mov_dpp((int)v, CTRL, 0xf, 0xf, false);
}

// Workgroup (blockIdx.x, blockIdx.y): output columns [blockIdx.x * RC * 4,
// + RC * 4) of the blockIdx.y-th expert that has rows.  T: 8-element K pieces
// per lane and row (K <= 512 T).  cb: A rows staged in LDS at a time (<= 8).
template <int NSETS, int EPI, bool WQ, int T>
__global__ __launch_bounds__(64 * kGemvWaves) void grouped_gemv(GemmArgs g, int cb) {
  constexpr int NW = kGemvWaves;
  constexpr int RPW = rows_per_wave<WQ>();  // weight rows per wave
  constexpr int RC = RPW / NSETS;    // output columns per wave
  constexpr int CW = WQ ? 1 : 4;     // dwords per lane per 8-element piece
  constexpr bool META = EPI == EPI_Y || EPI == EPI_OUT;
  static_assert((EPI == EPI_RELU2 || META) == (NSETS == 1), "gated epilogues take two sets");
  // staged A rows: row r, piece ch at byte 16 (r * K / 8 + ch), filled by
  // direct-to-LDS loads in whole 1 KB wave instructions (plus 4 KB of slack)
  extern __shared__ __attribute__((aligned(16))) char s_a[];
  __shared__ int s_sel[3];  // expert, its first sorted row, its row count

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int E = g.E, K = g.K, Nout = g.Nout;

  // ---- the blockIdx.y-th expert with rows (wave 0: four experts a lane) ----
  if (wave == 0) {
    int o[5], c[4], n = 0;
#pragma unroll
    for (int q = 0; q < 5; ++q) o[q] = g.offsets[min(lane * 4 + q, E)];  // E + 1 entries
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      c[q] = lane * 4 + q < E ? o[q + 1] - o[q] : 0;
      n += c[q] > 0;
    }
    const int incl = wave_inclusive_sum(n);
    const int want = (int)blockIdx.y;
    int before = incl - n;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      if (c[q] > 0) {
        if (before == want) {
          s_sel[0] = lane * 4 + q;
          s_sel[1] = o[q];
          s_sel[2] = c[q];
        }
        ++before;
      }
    }
    if (lane == 63 && incl <= want) s_sel[0] = -1;
  }
  __syncthreads();
  const int e = __builtin_amdgcn_readfirstlane(s_sel[0]);
  if (e < 0) return;  // fewer experts with rows than grid.y (uniform)
  const int row0 = __builtin_amdgcn_readfirstlane(s_sel[1]);
  const int cnt = __builtin_amdgcn_readfirstlane(s_sel[2]);

  // sorted entry (gather: its col_sorted value) of group row lane % 8,
  // clamped to the group's rows; the division by topk comes after the
  // weight loads
  auto group_rows = [&](int a0) {
    const int p = row0 + a0 + min(lane & 7, cnt - a0 - 1);
    return g.gather ? g.col_sorted[p] : p;
  };
  // the first group's, loaded ahead of the weights: waiting for them later
  // then waits for nothing else (vector loads retire in order)
  int arv = group_rows(0);

  // ---- this wave's weight rows, whole, into registers ----------------------
  // Buffer loads with out-of-range offsets for missing columns and K pieces
  // (they read zeros), so every load is issued, unconditionally, back to back.
  const int n0 = ((int)blockIdx.x * NW + wave) * RC;  // first output column
  const int nch = K / 8;                              // 8-element pieces a row
  const int rowb = WQ ? K / 2 : 2 * K;                // bytes of a weight row
  const int nrows = NSETS * Nout;
  const uint32_t wbytes = (uint32_t)nrows * (uint32_t)rowb;
  const __amdgpu_buffer_rsrc_t rw = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<char *>(reinterpret_cast<const char *>(g.W)) + (size_t)e * wbytes, (short)0,
      (int)wbytes, kRsrcWord3);
  auto memrow = [&](int i, int s) {  // weight row of column n0 + i, set s
    const int n = n0 + i;
    return NSETS == 1 ? n : (g.interleaved ? 2 * n + s : s * Nout + n);
  };
  uint32_t w[RC][NSETS][T][CW];
#pragma unroll
  for (int i = 0; i < RC; ++i)
#pragma unroll
    for (int s = 0; s < NSETS; ++s) {
      const uint32_t rbase = (uint32_t)memrow(i, s) * (uint32_t)rowb;
      const bool col_ok = n0 + i < Nout;
#pragma unroll
      for (int t = 0; t < T; ++t) {
        const int ch = lane + 64 * t;
        const uint32_t off = (col_ok && ch < nch) ? rbase + (uint32_t)ch * (4 * CW) : kOOB;
        if constexpr (WQ) {
          w[i][s][t][0] = (uint32_t)__builtin_amdgcn_raw_buffer_load_b32(rw, (int)off, 0, kWeightCpol);
        } else {
          const u32x4_t v =
              __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(rw, (int)off, 0, kWeightCpol));
#pragma unroll
          for (int d = 0; d < 4; ++d) w[i][s][t][d] = v[d];
        }
      }
    }
  // MXFP4 scales: quad lane j = lane % 4 loads the 4 bytes of the wave's local
  // rows 4j' .. 4j' + 3, j' = j % (RPW / 4), at K-block (lane + 64 t) / 4.
  // Local row order: column-major pairs (interleaved and plain) or the gate
  // run then the up run (packed); either way 4 consecutive local rows are 4
  // consecutive weight rows, 4-byte aligned (Nout and n0 are multiples of 4).
  uint32_t scw[WQ ? T : 1], scq[WQ ? T : 1][4];
  const bool packed = NSETS == 2 && !g.interleaved;
  if constexpr (WQ) {
    const uint32_t sbytes = (uint32_t)(K / 32) * (uint32_t)nrows;
    const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint8_t *>(g.wscale) + (size_t)e * sbytes, (short)0, (int)sbytes, kRsrcWord3);
    static_assert(RPW == 8 || RPW == 16, "four-row scale dwords, one or two a quad lane");
    const int l0 = 4 * ((lane & 3) % (RPW / 4));
    const int i0 = packed ? l0 % RC : l0 / NSETS, s0 = packed ? l0 / RC : l0 % NSETS;
    const uint32_t mr = (uint32_t)memrow(i0, s0);
    const bool col_ok = n0 + i0 < Nout;
#pragma unroll
    for (int t = 0; t < T; ++t) {
      const int kb = (lane + 64 * t) >> 2;
      const uint32_t off = (col_ok && kb < K / 32) ? (uint32_t)kb * (uint32_t)nrows + mr : kOOB;
      scw[t] = (uint32_t)__builtin_amdgcn_raw_buffer_load_b32(rs, (int)off, 0, 0);
    }
  }

  const float nal = -g.prm.alpha * 1.44269504088896341f;
  constexpr int LH = last_halving<RPW, NSETS>();
  int base = 0;  // first value index this lane holds after wave_sum
  {
    int m = 32;
#pragma unroll
    for (int n = RPW; n > NSETS; n /= 2, m >>= 1)
      if (lane & m) base += n / 2;
  }
  const int my_col = n0 + base / NSETS;
  const bool writer = (lane & (LH - 1)) == 0 && my_col < Nout;

  const __amdgpu_buffer_rsrc_t ra = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<void *>(g.A), (short)0, (int)g.a_bytes, kRsrcWord3);
  const int arow_b = 2 * K;
  const int nj = (cb * nch + 64 * NW - 1) / (64 * NW);  // DMA instructions a wave per group
  for (int a0 = 0; a0 < cnt; a0 += cb) {
    const int na = min(cb, cnt - a0);
    if (a0 > 0) __syncthreads();  // every wave is done with the previous group
    // A rows of the group (DMA behind the weight loads)
    if (a0 > 0) arv = group_rows(a0);
    const int arow_l = g.gather ? arv / g.topk : arv;  // x row (gather) or sorted row
    for (int j = 0; j < nj; ++j) {
      const int q = (j * NW + wave) * 64 + lane;
      const int r = q / nch, ch = q - r * nch;
      const int arow = __shfl(arow_l, r & 7);
      const uint32_t off = r < na ? (uint32_t)arow * (uint32_t)arow_b + (uint32_t)ch * 16 : kOOB;
      dma16(ra, s_a + (j * NW + wave) * 1024, off);
    }
    if constexpr (WQ) {
      if (a0 == 0) {
        // every lane of a quad gets the quad's four scale dwords
#pragma unroll
        for (int t = 0; t < T; ++t) {
          scq[t][0] = dpp_b<0x00>(scw[t]);
          scq[t][1] = dpp_b<0x55>(scw[t]);
          scq[t][2] = dpp_b<0xAA>(scw[t]);
          scq[t][3] = dpp_b<0xFF>(scw[t]);
        }
      }
    }
    wait_vm<0>();
    barrier();
    for (int r = 0; r < na; ++r) {
      if constexpr (WQ) {
        // the decoded weights would not fit in registers: keep the compiler
        // from hoisting the FP4 decode out of this loop
#pragma unroll
        for (int t = 0; t < T; ++t)
#pragma unroll
          for (int q = 0; q < 4; ++q) asm volatile("" : "+v"(scq[t][q]));
      }
      u32x4_t a[T];
#pragma unroll
      for (int t = 0; t < T; ++t) {
        // pieces past K (T is rounded up to 4, 6 or 8) would read the next
        // row or unwritten LDS: zeroed, since 0 * inf or 0 * NaN is not 0
        a[t] = *reinterpret_cast<const u32x4_t *>(s_a + r * arow_b + (lane + 64 * t) * 16);
        if (lane + 64 * t >= nch) a[t] = u32x4_t{0u, 0u, 0u, 0u};
      }
      float acc[RPW];  // value index i * NSETS + s
#pragma unroll
      for (int i = 0; i < RC; ++i)
#pragma unroll
        for (int s = 0; s < NSETS; ++s) {
          float sum = 0.f;
#pragma unroll
          for (int t = 0; t < T; ++t) {
            uint32_t wv[4];
            if constexpr (WQ) {
              // the scale byte of local row l: quad lane l / 4, byte l % 4
              const int li = i * NSETS + s, lp = s * RC + i;
              const uint32_t src = packed ? scq[t][lp >> 2] : scq[t][li >> 2];
              const int sh = 8 * (packed ? (lp & 3) : (li & 3));
              const float sc = __uint_as_float(((src >> sh) & 0xffu) << 23);
              const u32x4_t d = __builtin_bit_cast(u32x4_t, fp4x8_to_bf16(w[i][s][t][0], sc));
#pragma unroll
              for (int q = 0; q < 4; ++q) wv[q] = d[q];
            } else {
#pragma unroll
              for (int q = 0; q < 4; ++q) wv[q] = w[i][s][t][q];
            }
#pragma unroll
            for (int q = 0; q < 4; ++q) sum = dot2(wv[q], a[t][q], sum);
          }
          acc[i * NSETS + s] = sum;
        }
      wave_sum<RPW, NSETS>(acc, lane);
      if (writer) {
        const int p = row0 + a0 + r;
        float v;
        uint32_t orow = (uint32_t)p;
        if constexpr (META) {
          const float gs = !g.gate_scal ? 1.f
                           : g.gate_bf16
                               ? to_f32(reinterpret_cast<const bf16_t *>(g.gate_scal)[p])
                               : reinterpret_cast<const float *>(g.gate_scal)[p];
          v = acc[0] * gs;
          if (EPI == EPI_OUT) orow = (uint32_t)g.col_sorted[p];  // topk == 1: entry == token
        } else {
          v = act_val<EPI>(acc[0], acc[NSETS - 1], nal, g.prm);
        }
        reinterpret_cast<bf16_t *>(g.C)[(size_t)orow * Nout + my_col] = bf16_rne(v);
      }
    }
  }
}

// GEMM2 with the combine folded in, for decode-sized layers with topk > 1:
// workgroup (blockIdx.x, t) computes output columns [blockIdx.x * 4 * CPW,
// + 4 * CPW) of token t.  Wave w streams, for each of the token's slots j, the
// CPW weight rows of its columns from the slot's expert (slots in batches of
// SB, all rows of a batch in flight at once), takes the dot products with the
// slot's activation row (staged in LDS), and the lane sums of all SB * CPW
// (slot, column) values go through one halving reduction.  Its addition tree
// is the same for every value, so each y = RNE(gate_scal * sum) has the bits
// the w2 kernel would store in y_sorted; the y of one column are then added
// in slot order in fp32 and rounded once, as the combine kernel does.
template <bool WQ, int T>
__global__ __launch_bounds__(64 * kGemvWaves) void gemv_w2_combine(GemmArgs g) {
  constexpr int NW = kGemvWaves;
  constexpr int CPW = WQ ? 2 : 1;  // output columns a wave
  constexpr int SB = 4;            // slots a batch
  constexpr int CW = WQ ? 1 : 4;   // dwords per lane per 8-element piece
  constexpr int V = SB * CPW;      // values a lane reduces per batch
  extern __shared__ __attribute__((aligned(16))) char s_a[];  // SB activation rows
  __shared__ int s_off[kMaxExperts + 1];
  __shared__ int s_p[kMaxTopk], s_e[kMaxTopk];
  __shared__ float s_gs[kMaxTopk];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int E = g.E, K = g.K, Nout = g.Nout, k = g.topk;
  const int t = (int)blockIdx.y;

  // ---- the token's slots: sorted row, expert (from offsets), routing weight
  for (int i = tid; i <= E; i += 64 * NW) s_off[i] = g.offsets[i];
  if (tid < k) {
    const int p = g.row_sorted[(size_t)t * k + tid];
    s_p[tid] = p;
    s_gs[tid] = p < 0 ? 0.f
                : !g.gate_scal ? 1.f
                : g.gate_bf16 ? to_f32(reinterpret_cast<const bf16_t *>(g.gate_scal)[p])
                              : reinterpret_cast<const float *>(g.gate_scal)[p];
  }
  __syncthreads();
  if (tid < k) {
    const int p = s_p[tid];
    int e = -1;
    if (p >= 0) {  // the expert whose segment holds p: last e with offsets[e] <= p
      int lo = 0, hi = E - 1;
      while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (s_off[mid] <= p) lo = mid; else hi = mid - 1;
      }
      e = lo;
    }
    s_e[tid] = e;
  }
  __syncthreads();

  const int col0 = ((int)blockIdx.x * NW + wave) * CPW;
  const int nch = K / 8;
  const int rowb = WQ ? K / 2 : 2 * K;
  const uint32_t wbytes = (uint32_t)Nout * (uint32_t)rowb;
  const uint32_t sbytes = (uint32_t)(K / 32) * (uint32_t)Nout;
  const __amdgpu_buffer_rsrc_t ra = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<void *>(g.A), (short)0, (int)g.a_bytes, kRsrcWord3);
  const int arow_b = 2 * K;
  const int nj = (SB * nch + 64 * NW - 1) / (64 * NW);  // DMA instructions a wave per batch
  // lane holding value v after the halving reduction: one lane bit per step
  auto value_lane = [](int v) {
    int l = 0, m = 32;
    for (int n = V; n > 1; n /= 2, m >>= 1)
      if (v & (n / 2)) { l += m; v -= n / 2; }
    return l;
  };
  float out_acc[CPW];
#pragma unroll
  for (int c = 0; c < CPW; ++c) out_acc[c] = 0.f;

  for (int j0 = 0; j0 < k; j0 += SB) {
    if (j0 > 0) __syncthreads();  // every wave is done with the previous batch's rows
    // weights of the batch's slots, all in flight
    uint32_t w[SB][CPW][T][CW];
    uint32_t sc[WQ ? SB : 1][T];
#pragma unroll
    for (int jj = 0; jj < SB; ++jj) {
      const int e = j0 + jj < k ? __builtin_amdgcn_readfirstlane(s_e[j0 + jj]) : -1;
      const __amdgpu_buffer_rsrc_t rw = __builtin_amdgcn_make_buffer_rsrc(
          const_cast<char *>(reinterpret_cast<const char *>(g.W)) + (size_t)(e < 0 ? 0 : e) * wbytes,
          (short)0, (int)wbytes, kRsrcWord3);
#pragma unroll
      for (int c = 0; c < CPW; ++c)
#pragma unroll
        for (int tt = 0; tt < T; ++tt) {
          const int ch = lane + 64 * tt;
          const uint32_t off = (e >= 0 && col0 + c < Nout && ch < nch)
                                   ? (uint32_t)(col0 + c) * (uint32_t)rowb + (uint32_t)ch * (4 * CW)
                                   : kOOB;
          if constexpr (WQ) {
            w[jj][c][tt][0] = (uint32_t)__builtin_amdgcn_raw_buffer_load_b32(rw, (int)off, 0, kWeightCpol);
          } else {
            const u32x4_t v = __builtin_bit_cast(
                u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(rw, (int)off, 0, kWeightCpol));
#pragma unroll
            for (int d = 0; d < 4; ++d) w[jj][c][tt][d] = v[d];
          }
        }
      if constexpr (WQ) {
        // the scale bytes of the wave's two columns at K-block (lane + 64 tt) / 4
        const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
            const_cast<uint8_t *>(g.wscale) + (size_t)(e < 0 ? 0 : e) * sbytes, (short)0,
            (int)sbytes, kRsrcWord3);
#pragma unroll
        for (int tt = 0; tt < T; ++tt) {
          const int kb = (lane + 64 * tt) >> 2;
          const uint32_t off = (e >= 0 && col0 < Nout && kb < K / 32)
                                   ? (uint32_t)kb * (uint32_t)Nout + (uint32_t)col0
                                   : kOOB;
          sc[jj][tt] = (uint32_t)(uint16_t)__builtin_amdgcn_raw_buffer_load_b16(rs, (int)off, 0, 0);
        }
      }
    }
    // the batch's activation rows (DMA behind the weight loads)
    for (int j = 0; j < nj; ++j) {
      const int q = (j * NW + wave) * 64 + lane;
      const int r = q / nch, ch = q - r * nch;
      const int p = r < SB && j0 + r < k ? s_p[j0 + r] : -1;
      const uint32_t off = p >= 0 ? (uint32_t)p * (uint32_t)arow_b + (uint32_t)ch * 16 : kOOB;
      dma16(ra, s_a + (j * NW + wave) * 1024, off);
    }
    wait_vm<0>();
    barrier();
    float acc[V];  // value index jj * CPW + c
#pragma unroll
    for (int jj = 0; jj < SB; ++jj) {
      u32x4_t a[T];
#pragma unroll
      for (int tt = 0; tt < T; ++tt) {
        a[tt] = *reinterpret_cast<const u32x4_t *>(s_a + jj * arow_b + (lane + 64 * tt) * 16);
        if (lane + 64 * tt >= nch) a[tt] = u32x4_t{0u, 0u, 0u, 0u};
      }
#pragma unroll
      for (int c = 0; c < CPW; ++c) {
        float sum = 0.f;
#pragma unroll
        for (int tt = 0; tt < T; ++tt) {
          uint32_t wv[4];
          if constexpr (WQ) {
            const float scl = __uint_as_float(((sc[jj][tt] >> (8 * c)) & 0xffu) << 23);
            const u32x4_t d = __builtin_bit_cast(u32x4_t, fp4x8_to_bf16(w[jj][c][tt][0], scl));
#pragma unroll
            for (int q = 0; q < 4; ++q) wv[q] = d[q];
          } else {
#pragma unroll
            for (int q = 0; q < 4; ++q) wv[q] = w[jj][c][tt][q];
          }
#pragma unroll
          for (int q = 0; q < 4; ++q) sum = dot2(wv[q], a[tt][q], sum);
        }
        acc[jj * CPW + c] = sum;
      }
    }
    wave_sum<V, 1>(acc, lane);
    // y of each (slot, column), added in slot order
#pragma unroll
    for (int jj = 0; jj < SB; ++jj) {
      const int j = j0 + jj;
      if (j < k && s_p[j] >= 0) {
        const float gs = s_gs[j];
#pragma unroll
        for (int c = 0; c < CPW; ++c) {
          const float y = __int_as_float(
              __builtin_amdgcn_readlane(__float_as_int(acc[0]), value_lane(jj * CPW + c)));
          out_acc[c] += to_f32(bf16_rne(y * gs));
        }
      }
    }
  }
  if (lane == 0) {
#pragma unroll
    for (int c = 0; c < CPW; ++c)
      if (col0 + c < Nout)
        reinterpret_cast<bf16_t *>(g.C)[(size_t)t * Nout + col0 + c] = bf16_rne(out_acc[c]);
  }
}

template <int NSETS, int EPI, bool WQ>
hipError_t launch_sets(const GemmArgs &a, int64_t M, int cb, hipStream_t s) {
  constexpr int RC = rows_per_wave<WQ>() / NSETS;
  const unsigned gx = (unsigned)((a.Nout + RC * kGemvWaves - 1) / (RC * kGemvWaves));
  const unsigned gy = (unsigned)(M < a.E ? M : a.E);
  const int nj = (cb * (a.K / 8) + 64 * kGemvWaves - 1) / (64 * kGemvWaves);
  // whole DMA instructions, and 4 KB more: the last row's (masked) reads run
  // up to 64 T - K / 8 < 256 pieces past its end
  const size_t lds = (size_t)(nj + 1) * kGemvWaves * 1024;
  const int t = (a.K + 511) / 512;
  if (t <= 4)
    hipLaunchKernelGGL((grouped_gemv<NSETS, EPI, WQ, 4>), dim3(gx, gy), dim3(64 * kGemvWaves), lds,
                       s, a, cb);
  else if (t <= 6)
    hipLaunchKernelGGL((grouped_gemv<NSETS, EPI, WQ, 6>), dim3(gx, gy), dim3(64 * kGemvWaves), lds,
                       s, a, cb);
  else
    hipLaunchKernelGGL((grouped_gemv<NSETS, EPI, WQ, 8>), dim3(gx, gy), dim3(64 * kGemvWaves), lds,
                       s, a, cb);
  return hipGetLastError();
}

template <int NSETS, int EPI>
hipError_t launch_epi(const GemmArgs &a, int64_t M, int cb, hipStream_t s) {
  return a.wscale ? launch_sets<NSETS, EPI, true>(a, M, cb, s)
                  : launch_sets<NSETS, EPI, false>(a, M, cb, s);
}

}  // namespace

bool gemv_fits(moe_dtype_t dt, int64_t n_tokens, int topk, int n_experts, int K, int Nout,
               bool mxfp4, bool plain) {
  if (dt != MOE_BF16 || n_tokens > kGemvMaxTokens || K % 8 != 0 || K > 4096 || Nout % 8 != 0)
    return false;
  const int64_t m = n_tokens * topk;
  const int64_t e = n_experts;
  if (mxfp4) return plain ? m <= 3 * e : 2 * m <= 3 * e;
  return m <= (plain ? 5 : 3) * e;
}

bool gemm2_combine_fits(moe_dtype_t dt, int64_t n_tokens, int topk, int n_experts, int hidden,
                        int inter, bool mxfp4) {
  // about one row per expert (each token reads its slots' weight rows itself);
  // bf16 weights only: with MXFP4 weights the fused kernel measured no faster
  // than the matrix-vector w2 plus the combine (one token, gpt-oss-sized layer)
  return !mxfp4 && topk > 1 && n_tokens * topk <= n_experts && hidden % 2 == 0 &&
         gemv_fits(dt, n_tokens, topk, n_experts, inter, hidden, mxfp4);
}

hipError_t launch_gemm2_combine(const void *act_in, const void *w2, void *out,
                                const int32_t *offsets, const int32_t *row_sorted,
                                const void *gate_scal, moe_dtype_t gate_dt, int64_t n_tokens,
                                int topk, int n_experts, int hidden, int inter, hipStream_t s,
                                const uint8_t *w2_scale) {
  if (n_tokens <= 0) return hipSuccess;
  const int64_t M = n_tokens * topk;
  GemmArgs a{act_in, w2, out, offsets, nullptr, gate_scal, (uint32_t)(M * inter * 2),
             (uint32_t)(n_tokens * hidden * 2), gate_dt == MOE_BF16, n_experts, inter, hidden,
             topk, 0, 0, 0, ActParams{1.f, 0.f, 0.f}, w2_scale, row_sorted};
  const bool wq = w2_scale != nullptr;
  const int cpw = wq ? 2 : 1;
  const unsigned gx = (unsigned)((hidden + cpw * kGemvWaves - 1) / (cpw * kGemvWaves));
  const int nj = (4 * (inter / 8) + 64 * kGemvWaves - 1) / (64 * kGemvWaves);
  const size_t lds = (size_t)(nj + 1) * kGemvWaves * 1024;  // + slack, as in grouped_gemv
  const dim3 grid(gx, (unsigned)n_tokens), block(64 * kGemvWaves);
  const int t = (inter + 511) / 512;
  if (wq) {
    if (t <= 4) hipLaunchKernelGGL((gemv_w2_combine<true, 4>), grid, block, lds, s, a);
    else if (t <= 6) hipLaunchKernelGGL((gemv_w2_combine<true, 6>), grid, block, lds, s, a);
    else hipLaunchKernelGGL((gemv_w2_combine<true, 8>), grid, block, lds, s, a);
  } else {
    if (t <= 4) hipLaunchKernelGGL((gemv_w2_combine<false, 4>), grid, block, lds, s, a);
    else if (t <= 6) hipLaunchKernelGGL((gemv_w2_combine<false, 6>), grid, block, lds, s, a);
    else hipLaunchKernelGGL((gemv_w2_combine<false, 8>), grid, block, lds, s, a);
  }
  return hipGetLastError();
}

hipError_t launch_gemv(const GemmArgs &a, int nsets, int epi, int64_t n_tokens, int64_t M,
                       hipStream_t s) {
  if (M <= 0) return hipSuccess;
  // an expert holds at most one row per token, so n_tokens rows cover it
  int64_t cb = kGemvLdsBudget / (2 * a.K);
  if (cb > n_tokens) cb = n_tokens;
  if (cb > 8) cb = 8;
  if (cb < 1) cb = 1;
  if (nsets == 2)
    return epi == EPI_GATED_CLAMP ? launch_epi<2, EPI_GATED_CLAMP>(a, M, (int)cb, s)
                                  : launch_epi<2, EPI_GATED>(a, M, (int)cb, s);
  return epi == EPI_RELU2 ? launch_epi<1, EPI_RELU2>(a, M, (int)cb, s)
         : epi == EPI_OUT ? launch_epi<1, EPI_OUT>(a, M, (int)cb, s)
                          : launch_epi<1, EPI_Y>(a, M, (int)cb, s);
}

}  // namespace moe
