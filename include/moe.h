/*
 * moe.h -- C ABI of the MI355X (gfx950) MoE-layer forward library, libmoe.so.
 *
 * Three entry points run the layer on one GPU, entirely on the device and with
 * no device-to-host synchronisation:
 *
 *   moe_route    router logits -> top-k + softmax + all routing metadata
 *   moe_experts  routing metadata + x -> grouped expert FFN -> weighted combine
 *   moe_forward  moe_route followed by moe_experts, on one stream
 *
 * with the router GEMM in front (moe_gate_route, moe_gate_forward: logits from
 * the token rows and the gate weight), and the expert-parallel-share variants
 * moe_route_ep, moe_experts_ep and moe_forward_ep (one GPU's contiguous share
 * of the experts; see below).
 *
 * moe_experts is also exported as its two halves, moe_experts_w13 (grouped
 * GEMM with w13 + activation) and moe_experts_w2 (grouped GEMM with w2 +
 * routing weight + combine), and the latter as moe_experts_w2_rows (GEMM2 +
 * routing weight into sorted rows) and moe_combine (the scatter-combine).
 *
 * Sources of the operations (the pages are cited by title and section):
 *  - top-k over the router logits with softmax over the selected values, and the
 *    metadata it yields -- expert bitmatrix, per-expert column sums (col_sum),
 *    row- and column-sorted indices, gate weights permuted into sorted order --
 *    follow the topk / routing_data_from_sparse_topk description in the vLLM PR
 *    #45457 report ("implementation breakdown", "key source snippets").  The
 *    gather index pair is (col_sorted, row_sorted) and the scatter pair is
 *    (row_sorted, col_sorted); gate_scal has the dtype of the gating output.
 *  - the stable sort by expert with contiguous per-expert row slices and
 *    segment bounds [0] + group ends follows the minimind issue #835 page
 *    ("It is removable in plain PyTorch"); here the bounds never leave the GPU.
 *  - the expert FFN activations (SiLU-gated with optional clamp, SwiGLU-OAI with
 *    alpha/beta/limit, non-gated ReLU^2), the rule that unset parameters keep
 *    plain-SwiGLU defaults, and the packed [gate; up] vs interleaved
 *    [g0, u0, g1, u1, ...] w13 layouts follow the vLLM PR #47106 report
 *    ("implementation breakdown", the apply and w13-reorder snippets, "review
 *    highlights").
 *  - the caller owns the output and the workspaces, as in the experts apply()
 *    signature of the PR #47106 report.
 *
 * Conventions for every entry point:
 *  - All tensor pointers are DEVICE pointers, row-major, contiguous, 16-byte
 *    aligned, allocated and owned by the caller.  The library never allocates,
 *    frees, synchronises, logs, or keeps state between calls; it is re-entrant.
 *  - `stream` is a hipStream_t (NULL = the default stream).  All work is
 *    enqueued on it; the call returns before the work finishes.
 *  - Arguments are checked before anything is enqueued; on error a negative
 *    moe_status_t is returned and nothing is written.  A launch failure returns
 *    MOE_ERR_HIP.  Asynchronous device faults surface at the caller's next sync.
 *  - n_tokens == 0 is valid: MOE_OK, nothing enqueued.
 *  - Limits: 1 <= n_experts <= 256, 1 <= topk <= min(n_experts, 16),
 *    n_tokens * topk < 2^31, hidden and inter positive multiples of 8.
 *    moe_experts* and moe_forward also need each of these below 2^31 bytes:
 *    one expert's w13 block (2 * inter * hidden elements), x (n_tokens *
 *    hidden), the activation rows (n_tokens * topk * inter) and the sorted
 *    expert outputs (n_tokens * topk * hidden).
 *  - Logits must be finite.  Ties between equal logits go to the lower expert
 *    index; -0.0 and +0.0 are equal.
 */
#ifndef MOE_H_
#define MOE_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  MOE_OK = 0,
  MOE_ERR_NULL = -1,        /* a required pointer is NULL                     */
  MOE_ERR_SHAPE = -2,       /* a size is out of range or inconsistent          */
  MOE_ERR_DTYPE = -3,       /* unknown dtype, or dtypes that must match do not */
  MOE_ERR_UNSUPPORTED = -4, /* unsupported (activation, layout) combination    */
  MOE_ERR_ALIGN = -5,       /* a pointer is not 16-byte aligned                */
  MOE_ERR_WORKSPACE = -6,   /* workspace NULL or smaller than required         */
  MOE_ERR_HIP = -7,         /* a HIP launch failed                             */
  MOE_ERR_SCRATCH = -8      /* moe_forward_noalloc: sizes exceed its scratch   */
} moe_status_t;

typedef enum { MOE_F32 = 0, MOE_BF16 = 1 } moe_dtype_t;

/* Expert activation.  g = gate row, u = up row of the GEMM1 output.
 *   MOE_ACT_SILU:       a = g' * sigmoid(g') * u'            (uses limit only)
 *   MOE_ACT_SWIGLU_OAI: a = g' * sigmoid(alpha*g') * (u' + beta)
 *     with g' = min(g, limit) and u' = clamp(u, -limit, limit);
 *   MOE_ACT_RELU2:      a = max(h, 0)^2, non-gated (w13 has inter rows), no params.
 * The SwiGLU-OAI formula is a reading: the PR #47106 report names only its
 * parameters alpha, beta and limit (with the 1.702 / 1.0 / 7.0 values) and
 * prints no formula; this is the public gpt-oss definition, which no passage of
 * the pages pins (only its reduction to SiLU-gated with the parameters unset). */
typedef enum { MOE_ACT_SILU = 0, MOE_ACT_SWIGLU_OAI = 1, MOE_ACT_RELU2 = 2 } moe_act_t;

/* Row order of a gated w13 [E, 2*inter, hidden]:
 *   PACKED:      rows [0, inter) are gate, rows [inter, 2*inter) are up;
 *   INTERLEAVED: even rows are gate, odd rows are up.
 * MOE_ACT_RELU2 requires MOE_W13_PACKED (its w13 is a single up matrix). */
typedef enum { MOE_W13_PACKED = 0, MOE_W13_INTERLEAVED = 1 } moe_w13_layout_t;

/* Activation parameters.  A field counts only if its bit is set in `set`; an
 * unset field keeps the plain-SwiGLU default (alpha 1, beta 0, no clamp).  The
 * library never substitutes other defaults.  SiLU reads only `limit`. */
#define MOE_PARAM_ALPHA 1u
#define MOE_PARAM_BETA 2u
#define MOE_PARAM_LIMIT 4u
typedef struct {
  float alpha;
  float beta;
  float limit;
  uint32_t set;
} moe_act_params_t;

/* Routing metadata buffers (device pointers, caller-allocated).  M = n_tokens*topk.
 * Flat entry index f = t*topk + j names slot j of token t; slots are ordered by
 * descending logit (ties: lower expert index first). */
typedef struct {
  int32_t *topk_idx;   /* [N, topk]  selected expert of each slot                 */
  void *topk_w;        /* [N, topk]  softmax over the selected logits (w_dtype)   */
  uint32_t *bitmatrix; /* [N, ceil(E/32)] bit e%32 of word e/32: token chose e    */
  int32_t *col_sum;    /* [E]        entries routed to each expert                */
  int32_t *offsets;    /* [E+1]      0, running sum of col_sum; offsets[E] = M    */
  int32_t *col_sorted; /* [M]        f of the p-th entry in expert-major order,
                                     token order kept inside an expert            */
  int32_t *row_sorted; /* [M]        position p of entry f (inverse of col_sorted)*/
  void *gate_scal;     /* [M]        topk_w flat [col_sorted[p]] (w_dtype)         */
  int32_t w_dtype;     /* moe_dtype_t of topk_w and gate_scal                      */
} moe_routing_t;

/* Bytes of device workspace sufficient for moe_route (pass hidden = inter = 0),
 * moe_gate_route (pass hidden, inter = 0), moe_experts, moe_forward and
 * moe_gate_forward (pass both) with these sizes.  Returns 0 on invalid sizes. */
size_t moe_workspace_bytes(int64_t n_tokens, int32_t n_experts, int32_t topk,
                           int32_t hidden, int32_t inter, moe_dtype_t dtype);

/* Top-k gating and routing metadata.
 *   logits  [N, E] in logits_dtype.
 *   out     every field of *out is written; out->w_dtype must equal logits_dtype
 *           (the weights inherit the gating dtype).
 *   The result is deterministic and bit-identical across runs. */
moe_status_t moe_route(const void *logits, moe_dtype_t logits_dtype, int64_t n_tokens,
                       int32_t n_experts, int32_t topk, const moe_routing_t *out,
                       void *workspace, size_t ws_bytes, void *stream);

/* Grouped expert FFN and weighted combine from existing routing metadata.
 *   x    [N, hidden]; w13 [E, 2*inter, hidden] (gated) or [E, inter, hidden]
 *   (ReLU^2); w2 [E, hidden, inter]; out [N, hidden].  x, w13, w2, out share
 *   `dtype`.  Reads routing->offsets, col_sorted, row_sorted, gate_scal.
 *   out[t] = sum over the token's slots j of gate * W2[e] act(W13[e] x[t]),
 *   summed in slot order with fp32 accumulation (deterministic). */
moe_status_t moe_experts(const void *x, moe_dtype_t dtype, int64_t n_tokens, int32_t hidden,
                         const void *w13, const void *w2, int32_t n_experts, int32_t inter,
                         int32_t topk, moe_act_t act, moe_w13_layout_t layout,
                         const moe_act_params_t *params, const moe_routing_t *routing,
                         void *out, void *workspace, size_t ws_bytes, void *stream);

/* The two halves of moe_experts, for callers that keep the activation rows
 * themselves (the experts apply() of the PR #47106 report likewise takes one
 * workspace for the w13 stage and one for the w2 stage).
 *
 * moe_experts_w13: grouped GEMM with w13 and the activation.
 *   act_out [N*topk, inter] in `dtype`; row p is the activation of sorted entry p
 *   (the expert-major order of routing->col_sorted).  Reads routing->offsets and
 *   col_sorted.  Needs no workspace. */
moe_status_t moe_experts_w13(const void *x, moe_dtype_t dtype, int64_t n_tokens, int32_t hidden,
                             const void *w13, int32_t n_experts, int32_t inter, int32_t topk,
                             moe_act_t act, moe_w13_layout_t layout,
                             const moe_act_params_t *params, const moe_routing_t *routing,
                             void *act_out, void *stream);

/* moe_experts_w2: grouped GEMM with w2, routing weight, and the combine.
 *   act_in [N*topk, inter] from moe_experts_w13; w2 [E, hidden, inter];
 *   out [N, hidden].  Reads routing->offsets, col_sorted, row_sorted, gate_scal.
 *   workspace: at least moe_workspace_bytes(...) bytes (it holds the weighted
 *   expert rows when topk > 1). */
moe_status_t moe_experts_w2(const void *act_in, moe_dtype_t dtype, int64_t n_tokens,
                            int32_t hidden, const void *w2, int32_t n_experts, int32_t inter,
                            int32_t topk, const moe_routing_t *routing, void *out,
                            void *workspace, size_t ws_bytes, void *stream);

/* moe_experts_w2 split further into its two kernels, GEMM2 and the combine
 * (the weighted expert outputs and the index_add_-style sum back into token
 * rows of the minimind issue #835 page, "Summary"), for callers that time or
 * overlap them separately.  moe_experts_w2 gives the same bits as the two in
 * sequence for any topk.
 *
 * moe_experts_w2_rows: y_sorted [N*topk, hidden] in `dtype`; row p receives
 *   gate_scal[p] * (W2[e] act_in[p]), accumulated in fp32 and rounded once
 *   (nearest-even), for the routed rows p < offsets[n_experts]; rows past it
 *   (an expert share's unrouted positions) are not written.  Reads
 *   routing->offsets, col_sorted, gate_scal.  n_experts may be smaller than
 *   topk (an expert share).  Needs no workspace.
 * moe_combine: out [N, hidden] in `dtype`; out[t] = sum over j < topk of
 *   y_sorted[row_sorted[t*topk + j]], in slot order with fp32 accumulation and
 *   one rounding; slots with row_sorted = -1 add nothing (a token with none
 *   gets a zero row).  Reads routing->row_sorted only; deterministic, no
 *   atomics.  Limits: 1 <= topk <= 16, n_tokens * topk < 2^31, hidden a
 *   positive multiple of 8. */
moe_status_t moe_experts_w2_rows(const void *act_in, moe_dtype_t dtype, int64_t n_tokens,
                                 int32_t hidden, const void *w2, int32_t n_experts, int32_t inter,
                                 int32_t topk, const moe_routing_t *routing, void *y_sorted,
                                 void *stream);
moe_status_t moe_combine(const void *y_sorted, moe_dtype_t dtype, int64_t n_tokens,
                         int32_t hidden, int32_t topk, const moe_routing_t *routing, void *out,
                         void *stream);

/* moe_route on `logits` (dtype `dtype`) into *routing_out, then moe_experts. */
moe_status_t moe_forward(const void *x, const void *logits, moe_dtype_t dtype,
                         int64_t n_tokens, int32_t hidden, const void *w13, const void *w2,
                         int32_t n_experts, int32_t inter, int32_t topk, moe_act_t act,
                         moe_w13_layout_t layout, const moe_act_params_t *params,
                         const moe_routing_t *routing_out, void *out, void *workspace,
                         size_t ws_bytes, void *stream);

/* ---- The layer without a workspace argument -----------------------------------
 * For callers that cannot allocate device memory: code under HIP graph
 * capture, tight serving loops, harnesses that forbid allocation.
 *
 * moe_forward_noalloc: moe_forward (same arguments less the workspace, same
 *   kernels, same bits) with its intermediates -- the routing scratch, the
 *   activation rows and the weighted expert rows -- in a static device array of
 *   MOE_NOALLOC_SCRATCH_BYTES inside the library.  Each GPU holds its own copy
 *   from the first call on it until the process ends; the call never allocates
 *   or frees memory.  Sizes whose moe_workspace_bytes(n_tokens, n_experts,
 *   topk, hidden, inter, dtype) exceed MOE_NOALLOC_SCRATCH_BYTES are rejected
 *   with MOE_ERR_SCRATCH before anything is enqueued (64 MiB: e.g. up to 1456
 *   tokens of a top-4, 2880-wide gpt-oss-shaped layer).
 *   Every call on one GPU uses that GPU's one array: calls that overlap on a
 *   GPU (two streams, two threads) race and give wrong results; serialise them.
 *   Nothing in the array needs to start at zero, so a call never depends on
 *   what an earlier call left there.  The first call on a GPU resolves the
 *   array's address (a runtime symbol lookup, not a stream operation); make it
 *   before capturing a graph that contains the call. */
#define MOE_NOALLOC_SCRATCH_BYTES (64u << 20)
moe_status_t moe_forward_noalloc(const void *x, const void *logits, moe_dtype_t dtype,
                                 int64_t n_tokens, int32_t hidden, const void *w13,
                                 const void *w2, int32_t n_experts, int32_t inter, int32_t topk,
                                 moe_act_t act, moe_w13_layout_t layout,
                                 const moe_act_params_t *params, const moe_routing_t *routing_out,
                                 void *out, void *stream);

/* ---- Routing weight on the input rows ---------------------------------------
 * moe_experts_weighted_input: the experts apply() of the vLLM PR #47106 report
 *   takes apply_router_weight_on_input ("key source snippets"); with it the
 *   routing weight scales the expert's input instead of its output:
 *     out[t] = sum over the token's slots j of W2[e] act(W13[e] xw),
 *     xw = x[t] * gate, multiplied in fp32 and rounded once (nearest-even) to
 *     `dtype`, the expert outputs summed in slot order with fp32 accumulation.
 *   Arguments as moe_experts; the workspace must hold moe_workspace_bytes(...)
 *   plus n_tokens * topk * hidden elements of `dtype` rounded up to 256 bytes
 *   (the scaled input rows).  Any topk (the pages' kernels use it with 1). */
moe_status_t moe_experts_weighted_input(const void *x, moe_dtype_t dtype, int64_t n_tokens,
                                        int32_t hidden, const void *w13, const void *w2,
                                        int32_t n_experts, int32_t inter, int32_t topk,
                                        moe_act_t act, moe_w13_layout_t layout,
                                        const moe_act_params_t *params,
                                        const moe_routing_t *routing, void *out, void *workspace,
                                        size_t ws_bytes, void *stream);

/* ---- Router GEMM ahead of the routing ----------------------------------------
 * The router's gate matmul, logits = x . w_gate^T, is the step just before
 * the top-k; the vLLM PR #45457 report leaves it to its own kernel
 * ("motivation").  Here it is part of the routing step.
 *
 * moe_gate_route: x [N, hidden] and w_gate [n_experts, hidden] (nn.Linear
 *   out x in, row-major) in `dtype`; logits_out [N, n_experts] in `dtype`
 *   receives logits[t][e] = sum_h x[t][h] * w_gate[e][h], accumulated in fp32
 *   and rounded once (nearest-even) to `dtype`; then everything moe_route
 *   computes from those logits goes to *out (out->w_dtype == dtype).  The same
 *   result as writing the logits and calling moe_route on them.  Workspace:
 *   moe_workspace_bytes(n_tokens, n_experts, topk, hidden, 0, dtype) (batches
 *   of 5 to 4096 tokens keep fp32 partial sums of the product over K-groups
 *   there); limits as
 *   moe_route; hidden a positive multiple of 8; x, w_gate and logits_out below
 *   2^31 bytes.
 * moe_gate_forward: moe_gate_route then moe_experts, on one stream. */
moe_status_t moe_gate_route(const void *x, const void *w_gate, moe_dtype_t dtype,
                            int64_t n_tokens, int32_t hidden, int32_t n_experts, int32_t topk,
                            void *logits_out, const moe_routing_t *out, void *workspace,
                            size_t ws_bytes, void *stream);
moe_status_t moe_gate_forward(const void *x, const void *w_gate, moe_dtype_t dtype,
                              int64_t n_tokens, int32_t hidden, const void *w13, const void *w2,
                              int32_t n_experts, int32_t inter, int32_t topk, moe_act_t act,
                              moe_w13_layout_t layout, const moe_act_params_t *params,
                              void *logits_out, const moe_routing_t *routing_out, void *out,
                              void *workspace, size_t ws_bytes, void *stream);

/* ---- Expert-parallel share ---------------------------------------------------
 * One GPU of an expert-parallel group holds the contiguous share of experts
 * [local_offset, local_offset + n_local) of the layer's n_experts and computes
 * those experts' contribution for every token; the group's outputs summed over
 * all shares give the layer output.  The share is the (local_expert_offset,
 * num_local_experts) pair the experts kernel call of the vLLM PR #47106 report
 * takes ("key source snippets"); remapping the selected expert ids to local
 * ids and re-packing the bitmatrix after the remap is the expert-map branch of
 * the vLLM PR #45457 report ("implementation breakdown").
 *
 * moe_route_ep: top-k and softmax over all n_experts logits, then
 *   topk_idx [N, topk]   selected experts, GLOBAL ids (as moe_route)
 *   topk_w   [N, topk]   softmax over the selected logits (as moe_route)
 *   bitmatrix [N, ceil(n_local/32)]  bit l: token chose local expert l
 *   col_sum [n_local], offsets [n_local+1]  over local experts; offsets[n_local]
 *            = M_local, the number of slots whose expert is in the share
 *   col_sorted [N*topk]  positions p < M_local as in moe_route (local experts
 *            in ascending order, token order inside each); p >= M_local: -1
 *   row_sorted [N*topk]  p for slots in the share, -1 for the others
 *   gate_scal [N*topk]   topk_w flat[col_sorted[p]] for p < M_local; 0 after
 *   Needs 0 <= local_offset, 1 <= n_local, local_offset + n_local <= n_experts
 *   (else MOE_ERR_SHAPE), and the workspace moe_workspace_bytes(n_tokens,
 *   n_experts, ...) gives.  local_offset = 0, n_local = n_experts gives exactly
 *   the moe_route result.
 *
 * moe_experts_ep: moe_experts over the n_local experts of a share, from a
 *   moe_route_ep routing: w13 [n_local, ...], w2 [n_local, ...].  out[t] is the
 *   weighted sum over the token's slots in the share (fp32, slot order); a
 *   token with none gets a zero row.  n_local may be smaller than topk.
 *   Workspace: moe_workspace_bytes(n_tokens, n_experts, topk, hidden, inter,
 *   dtype) with any n_experts >= topk.
 *
 * moe_forward_ep: moe_route_ep then moe_experts_ep, on one stream. */
moe_status_t moe_route_ep(const void *logits, moe_dtype_t logits_dtype, int64_t n_tokens,
                          int32_t n_experts, int32_t topk, int32_t local_offset, int32_t n_local,
                          const moe_routing_t *out, void *workspace, size_t ws_bytes,
                          void *stream);
moe_status_t moe_experts_ep(const void *x, moe_dtype_t dtype, int64_t n_tokens, int32_t hidden,
                            const void *w13, const void *w2, int32_t n_local, int32_t inter,
                            int32_t topk, moe_act_t act, moe_w13_layout_t layout,
                            const moe_act_params_t *params, const moe_routing_t *routing,
                            void *out, void *workspace, size_t ws_bytes, void *stream);
moe_status_t moe_forward_ep(const void *x, const void *logits, moe_dtype_t dtype,
                            int64_t n_tokens, int32_t hidden, const void *w13, const void *w2,
                            int32_t n_experts, int32_t local_offset, int32_t n_local,
                            int32_t inter, int32_t topk, moe_act_t act, moe_w13_layout_t layout,
                            const moe_act_params_t *params, const moe_routing_t *routing_out,
                            void *out, void *workspace, size_t ws_bytes, void *stream);

/* ---- MXFP4 expert weights ------------------------------------------------------
 * The gpt-oss experts of the vLLM PR #45457 report run with MXFP4 weights and
 * bf16 activations (the MXFP4 experts forward of "key source snippets"); the
 * pages name the format only.  Format (public OCP microscaling definition):
 * every 32 consecutive weights along K share a scale 2^X stored as the byte
 * X + 127, X = floor(log2 max|w|) - 2 (-127 for an all-zero block); each weight
 * is an FP4 E2M1 code (magnitudes 0, 0.5, 1, 1.5, 2, 3, 4, 6; bit 3 the sign)
 * for the nearest value of w * 2^-X, ties to the code with an even lowest bit,
 * saturating at 6.  Codes pack two to a byte, the even element in the low
 * nibble; scales are block-major per expert.
 *
 * moe_quantize_mxfp4: w [n_experts, rows, k] (dtype) -> q [n_experts, rows,
 *   k / 2] bytes and scales [n_experts, k / 32, rows] bytes.  k a multiple of
 *   32; w and q 16-byte aligned.  Deterministic, bit-exact. */
moe_status_t moe_quantize_mxfp4(const void *w, moe_dtype_t dtype, int32_t n_experts,
                                int32_t rows, int32_t k, void *q, void *scales, void *stream);

/* moe_experts_mxfp4 / moe_forward_mxfp4: moe_experts / moe_forward with MXFP4
 *   expert weights from moe_quantize_mxfp4: w13_q [E, w13 rows, hidden / 2] and
 *   w13_s [E, hidden / 32, w13 rows] (w13 rows = 2 * inter gated, in the same
 *   packed or interleaved order as a bf16 w13; inter for ReLU^2), w2_q
 *   [E, hidden, inter / 2] and w2_s [E, inter / 32, hidden].  The layer is bf16
 *   (dtype MOE_BF16, else MOE_ERR_UNSUPPORTED); hidden and inter multiples of
 *   32.  Each weight is its code's value times its block's scale, exactly
 *   representable in bf16, so the result is that of moe_experts on the
 *   dequantised bf16 weights (bit-identical when both take the same kernel for
 *   each GEMM: at most 128 tokens with N * topk <= 1.5 E take the
 *   matrix-vector kernels in both, and past the bf16 layer's matrix-vector
 *   range (3 E for w13, 5 E for w2) the 32-row / one-wave tiles are shared
 *   below 48 rows an expert, except where the bf16 layer takes its
 *   register-weight tiles there (bf16 K a multiple of 64, from 16 rows an
 *   expert for w2 and ReLU^2 w13, from 32 for gated w13, when those tiles
 *   cover the compute units); the 128-row MXFP4 tiles differ from the bf16
 *   ones).  Workspace and other arguments as moe_experts / moe_forward. */
moe_status_t moe_experts_mxfp4(const void *x, moe_dtype_t dtype, int64_t n_tokens,
                               int32_t hidden, const void *w13_q, const void *w13_s,
                               const void *w2_q, const void *w2_s, int32_t n_experts,
                               int32_t inter, int32_t topk, moe_act_t act,
                               moe_w13_layout_t layout, const moe_act_params_t *params,
                               const moe_routing_t *routing, void *out, void *workspace,
                               size_t ws_bytes, void *stream);
moe_status_t moe_forward_mxfp4(const void *x, const void *logits, moe_dtype_t dtype,
                               int64_t n_tokens, int32_t hidden, const void *w13_q,
                               const void *w13_s, const void *w2_q, const void *w2_s,
                               int32_t n_experts, int32_t inter, int32_t topk, moe_act_t act,
                               moe_w13_layout_t layout, const moe_act_params_t *params,
                               const moe_routing_t *routing_out, void *out, void *workspace,
                               size_t ws_bytes, void *stream);

/* Static, human-readable name of a status code. */
const char *moe_status_str(moe_status_t status);

#ifdef __cplusplus
}
#endif
#endif /* MOE_H_ */
