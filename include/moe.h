/*
 * moe.h -- C ABI of one GPU's mixture-of-experts (MoE) expert layer on
 * AMD MI355X (gfx950).
 *
 * The layer, as the MegaScale-MoE pages describe it:
 *   route    -- a trainable gate scores the E experts of each token and keeps
 *               the k best ("MegaScale-MoE: 大规模通信高效的生产级混合专家模型
 *               训练系统", §三 MoE layer structure / Fig. 2 and the training
 *               flow; DisagMoE page, §2.1 / Fig. 2(a));
 *   permute  -- a local scatter makes every expert's tokens contiguous,
 *               ordered by expert then by source (same review, §四 adaptive
 *               EP communication; MegaScale-MoE research digest, §3.3
 *               Diagram C);
 *   grouped  -- one GroupedGEMM runs every expert's SwiGLU FFN: FC1 (gate
 *               and up projections), SiLU(gate)*up, FC2 (review §三 core
 *               formulas and §四 selective activation recomputation; digest
 *               §3.3);
 *   combine  -- each token's k expert outputs are summed with the gate
 *               weights (review §三 training flow, token aggregation);
 *   backward -- FC2/FC1 gradients with FC2's input recomputed, FP32 weight
 *               gradients (review §四 selective recomputation, §三 parameter
 *               update);
 *   FP8      -- per-token E4M3 scales for activations (review §三
 *               communication-compression layer, §四 FP8 row; digest §3.4).
 *
 * Conventions for every call
 *   - Row-major, contiguous tensors; row-vector math y = x W.
 *   - Every tensor pointer is a DEVICE pointer owned by the caller.  The
 *     library allocates nothing on these paths, frees nothing, and keeps no
 *     pointer after the call returns.  Scratch memory comes from the caller
 *     as a workspace sized by the matching *_workspace_size() call.
 *   - Every call only validates its arguments on the host and enqueues
 *     kernels on `stream` (a hipStream_t; NULL = the null stream).  Nothing
 *     synchronizes the host and no count is copied back to the host.
 *   - Pointers must be 16-byte aligned.
 *   - Return value: MOE_OK, or a negative MOE_ERR_* code.  Arguments are
 *     checked before any launch; on an error nothing is enqueued and no
 *     output is touched.  moe_last_error() returns a message for the last
 *     failing call of the calling thread.
 *   - T = 0 (or rows = 0) is a successful no-op, except that moe_permute
 *     still writes zero counts and offsets when it builds an index, and the
 *     expert backward entry points still write zero weight gradients.
 */
#ifndef MOE_MI355X_H
#define MOE_MI355X_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define MOE_OK 0
#define MOE_ERR_ARG (-1)       /* NULL pointer, bad count, misaligned pointer */
#define MOE_ERR_DTYPE (-2)     /* unsupported element type or combination     */
#define MOE_ERR_SHAPE (-3)     /* dimension outside what the kernels support  */
#define MOE_ERR_WORKSPACE (-4) /* workspace missing or too small              */
#define MOE_ERR_HIP (-5)       /* a HIP launch or query failed                */

#define MOE_MAX_EXPERTS 256    /* E <= MOE_MAX_EXPERTS                         */
#define MOE_MAX_TOPK 16        /* k <= MOE_MAX_TOPK                            */

/* Element types. */
#define MOE_F32 0
#define MOE_BF16 1
#define MOE_FP8_E4M3 2         /* OCP E4M3FN: bias 7, max 448, no infinities   */

/*
 * Expert weights in the layout the GroupedGEMM reads (filled by
 * moe_pack_weights into caller-allocated buffers).
 *   w13  [E][2*h_ffn][h]  FC1 weights transposed (h contiguous).  Packed row
 *        p holds gate channel (p/64)*32 + p%32 when (p/32) is even and up
 *        channel (p/64)*32 + p%32 when it is odd, so every 64 packed rows
 *        hold 32 gate channels followed by the same 32 up channels.
 *   w2   [E][h][h_ffn]    FC2 weight transposed (h_ffn contiguous).
 *   w13_scale [E][2*h_ffn], w2_scale [E][h]: FP8 only, per packed row
 *        (= per output channel) dequantization scales; NULL otherwise.
 *   w13_bwd [E][h][2*h_ffn]: for the backward (BF16 or FP8): W1 and W3 side
 *        by side along h_ffn in the same 32-channel interleave as w13's rows
 *        (column p holds W1 or W3 column (p/64)*32 + p%32 by the parity of
 *        p/32).  NULL when no backward will run.
 *   w2_bwd  [E][h_ffn][h]: for the backward (BF16 or FP8), W2 as given (h
 *        contiguous); NULL when no backward will run.
 *   w13_bwd_scale [E][h], w2_bwd_scale [E][h_ffn]: FP8 backward copies only,
 *        one scale per row over that row (amax/448); NULL otherwise.
 *   dtype: MOE_F32, MOE_BF16 or MOE_FP8_E4M3.
 */
typedef struct {
  int dtype;
  int E, h, h_ffn;
  const void* w13;
  const void* w2;
  const float* w13_scale;
  const float* w2_scale;
  const void* w13_bwd;
  const void* w2_bwd;
  const float* w13_bwd_scale;
  const float* w2_bwd_scale;
} moe_weights;

/* Bytes needed for w13 (`which`=0), w2 (1), w13_scale (2), w2_scale (3),
 * w13_bwd (4), w2_bwd (5), w13_bwd_scale (6), w2_bwd_scale (7). */
size_t moe_packed_weight_bytes(int which, int E, int h, int h_ffn, int dtype);

/*
 * Pack (and for FP8, quantize) expert weights.  Set-up work, outside the
 * per-step path.
 *   w1, w3  [E][h][h_ffn]  gate / up projections, element type in_dtype
 *   w2      [E][h_ffn][h]  down projection
 *   in_dtype: MOE_F32 or MOE_BF16.  out_dtype: MOE_F32 (needs in F32),
 *   MOE_BF16 (needs in BF16) or MOE_FP8_E4M3 (needs in BF16).
 *   FP8: per output channel s = amax/448 over the input dimension (1 when the
 *   channel is all zero); codes = E4M3(w / s) rounded to nearest even with
 *   the division in fp32, saturating at +-448.
 *   Outputs: see moe_weights; scales are written only for FP8 (may be NULL
 *   otherwise).  w13_bwd / w2_bwd are written when non-NULL (BF16, or FP8
 *   with w13_bwd_scale / w2_bwd_scale: one scale per row over the row, the
 *   dimension the backward contracts).
 *   h and h_ffn must be multiples of 128.
 */
int moe_pack_weights(const void* w1, const void* w3, const void* w2, int in_dtype, int E, int h,
                     int h_ffn, int out_dtype, void* w13, void* w2_packed, float* w13_scale,
                     float* w2_scale, void* w13_bwd, void* w2_bwd, float* w13_bwd_scale,
                     float* w2_bwd_scale, void* stream);

/*
 * Router: gate GEMM, top-k and softmax over the k selected logits.
 *   x       [T][h] (MOE_F32 or MOE_BF16 = dtype), or NULL: then `logits` is
 *           an INPUT of fp32 router logits [T][E] and the gate GEMM is
 *           skipped (used to compare routing bit for bit against another
 *           implementation given identical logits).
 *   w_gate  [h][E] same dtype as x (ignored when x is NULL).
 *   bias    [E] fp32 added to the logits, or NULL for none.
 *   logits  [T][E] fp32: written when x != NULL and logits != NULL.
 *   topk_idx[T][k] int32: experts of each token by logit descending, equal
 *           logits by expert index ascending.
 *   topk_w  [T][k] fp32: softmax of the k selected logits (sums to 1; k = 1
 *           gives exactly 1).
 *   Logits are x W_g accumulated in fp32, then + bias in fp32.
 *   Limits: 1 <= k <= E <= MOE_MAX_EXPERTS, k <= MOE_MAX_TOPK; h a multiple
 *   of 64 when x != NULL.
 */
int moe_route(const void* x, const void* w_gate, const float* bias, float* logits, int T, int h,
              int E, int k, int dtype, int32_t* topk_idx, float* topk_w, void* stream);

/* Workspace bytes for moe_permute with index building (topk_idx != NULL). */
size_t moe_permute_workspace_size(int T, int E, int k);

/*
 * Dispatch: build the expert-contiguous index and copy rows into it.
 *   src      [T][h] element type src_dtype (MOE_F32 or MOE_BF16).
 *   topk_idx [T][k] int32 expert ids, or NULL to reuse an index built by an
 *            earlier call (then counts/offsets/src_tok are not touched and
 *            dst_row is an INPUT).  Ids outside [0, E) are dropped:
 *            dst_row = -1 and they are not counted.  A token may name one
 *            expert in several slots (moe_route never does): each such
 *            (t, j) pair is counted and gets its own row, the pairs of one
 *            token in slot order.
 *   row_scale[T][k] fp32 or NULL: when given, routed row (t, j) receives
 *            row_scale[t][j] * src[t] (the transpose of the weighted combine,
 *            used for the upstream gradient).
 *   counts   [E]   int32 rows per expert.
 *   offsets  [E+1] int32 exclusive prefix sum; offsets[E] = rows kept.
 *   dst_row  [T][k] int32 row of (t, j) in dst: offsets[e] + number of
 *            pairs (t', j') routed to e with t' < t, or t' = t and j' < j.
 *            As an input, entries outside [0, T*k) are skipped.
 *   src_tok  [T*k] int32 token of every routed row.
 *   dst      [T*k][h] element type dst_dtype: MOE_F32 (src F32), MOE_BF16
 *            (src BF16) or MOE_FP8_E4M3 (src BF16; per-token quantization:
 *            dst_scale[row] = amax_t / 448 (1 for an all-zero row), codes =
 *            E4M3(src / scale) with the division in fp32, nearest even,
 *            saturating).  With FP8 and row_scale the codes stay those of
 *            src[t] and dst_scale[row] = row_scale[t][j] * scale (fp32).
 *   dst_scale[T*k] fp32, FP8 only (NULL otherwise).
 *   ws / ws_bytes: workspace, at least moe_permute_workspace_size(T, E, k)
 *            bytes when topk_idx != NULL (may be NULL otherwise).
 *   h must be a multiple of 8.
 */
int moe_permute(const void* src, int src_dtype, const int32_t* topk_idx, const float* row_scale,
                int T, int h, int E, int k, int32_t* counts, int32_t* offsets, int32_t* dst_row,
                int32_t* src_tok, void* dst, int dst_dtype, float* dst_scale, void* ws,
                size_t ws_bytes, void* stream);

/*
 * moe_permute without a workspace, for callers that cannot allocate device
 * memory (code under HIP graph capture, tight serving loops, harnesses that
 * forbid hipMalloc).  Same arguments and results as moe_permute, minus ws and
 * ws_bytes: the index builder's per-block histograms live in a file-scope
 * device array of MOE_NOALLOC_SCRATCH_BYTES, one per GPU, held until the
 * process ends.  Nothing is allocated or freed.  Returns MOE_ERR_WORKSPACE
 * (nothing written) when the index needs more than that scratch:
 * ceil(T / 256) * E * 4 bytes (rounded up to 256) must fit, e.g. T up to
 * 262144 with E = 256.  Every call on one GPU shares that GPU's array, which
 * keeps the last call's contents (each call rewrites every byte it reads), so
 * calls that overlap on one GPU (different streams, or threads) race.
 */
#define MOE_NOALLOC_SCRATCH_BYTES (1 << 20)
int moe_permute_noalloc(const void* src, int src_dtype, const int32_t* topk_idx, const float* row_scale,
                        int T, int h, int E, int k, int32_t* counts, int32_t* offsets, int32_t* dst_row,
                        int32_t* src_tok, void* dst, int dst_dtype, float* dst_scale, void* stream);

/*
 * One GPU's share of expert parallelism (MegaScale-MoE research digest §3.2,
 * Diagram B: scatter to the local experts and drop the rest; paper review §四
 * adaptive EP communication): the dispatch of moe_permute restricted to the
 * experts [e_lo, e_lo + e_count) of an E-expert layer, renumbered from 0.
 * Pairs routed elsewhere get dst_row = -1 and are not counted; moe_combine
 * over this share's rows (y_dtype MOE_F32) is the share's partial output,
 * and the shares' partials add up to the layer's output (the reduce-scatter
 * of the all-gather path).  Rows of each local expert are ordered by token,
 * i.e. by (source rank, token) when source ranks hold contiguous token ranges
 * (the order the all-to-all path delivers).
 *   topk_idx [T][k] global expert ids; counts [e_count], offsets [e_count+1];
 *   dst_row [T][k]; src_tok [T*k] (entries past offsets[e_count] untouched);
 *   dst [T*k][h] (offsets[e_count] rows written); everything else as for
 *   moe_permute with topk_idx given.  0 <= e_lo, 1 <= e_count,
 *   e_lo + e_count <= E.
 */
size_t moe_permute_local_workspace_size(int T, int e_count, int k);
int moe_permute_local(const void* src, int src_dtype, const int32_t* topk_idx, const float* row_scale,
                      int T, int h, int E, int k, int e_lo, int e_count, int32_t* counts,
                      int32_t* offsets, int32_t* dst_row, int32_t* src_tok, void* dst, int dst_dtype,
                      float* dst_scale, void* ws, size_t ws_bytes, void* stream);

/*
 * Token dropping by affinity (MegaScale-MoE research digest §3.2: tokens are
 * dropped per GPU, as in DeepSeek-V2, which drops the lowest-affinity tokens
 * of each device until its budget is met).  A device is a group of `group`
 * consecutive experts (one GPU's share; group = 1 gives a per-expert
 * capacity).  Among the (t, j) pairs routed into a group, the `capacity`
 * pairs with the highest affinity s = softmax(logits[t])[e] (fp32, over all E
 * experts) are kept, equal affinities in dispatch order (expert, then token);
 * every other pair's id becomes -1 in topk_idx_out, which moe_permute then
 * drops (and with it the pair's share of the combine and of the backward).
 * Gate weights are not changed.
 *   topk_idx [T][k] int32 in; topk_idx_out [T][k] int32 out (may be the same
 *   buffer as topk_idx); logits [T][E] fp32 (bias included).
 *   group divides E; capacity >= 0 rows per group.
 */
size_t moe_capacity_drop_workspace_size(int T, int E, int k);
int moe_capacity_drop(const int32_t* topk_idx, const float* logits, int T, int E, int k, int group,
                      int capacity, int32_t* topk_idx_out, void* ws, size_t ws_bytes, void* stream);

/* Workspace bytes for moe_grouped_swiglu_fwd (rows = T*k). */
size_t moe_grouped_workspace_size(int rows, int h, int h_ffn, int E, int dtype);

/*
 * Forward GroupedGEMM of every expert's SwiGLU FFN over expert-contiguous rows.
 *   xp       [rows][h] routed rows, element type W->dtype (FP8: codes).
 *   xp_scale [rows] fp32 per-row scales (FP8 only, else NULL).
 *   W        packed weights (moe_pack_weights).
 *   offsets  [E+1] int32 device array from moe_permute; rows of expert e are
 *            offsets[e] .. offsets[e+1]-1; offsets[E] <= rows.
 *   h13_save [rows][2*h_ffn] bf16 or NULL (BF16 or FP8 weights): when given, FC1's output is kept
 *            for the backward, columns in the packed order of W->w13.
 *   yp       [rows][h] expert outputs, element type yp_dtype: MOE_F32 (any
 *            weights; FC2's fp32 sum is stored as it is) or MOE_BF16 (BF16
 *            or FP8 weights; rounded to nearest even).  Any other pairing
 *            returns MOE_ERR_DTYPE.
 *   Math: G = xp W1_e, U = xp W3_e (fp32 accumulation), A = SiLU(G) * U,
 *   yp = A W2_e.  FP8: G, U carry xp_scale[row] * w13_scale[e][channel]; A
 *   is quantized per row (amax/448 over the row's h_ffn values) before FC2,
 *   whose result carries that scale times w2_scale.
 *   Rows >= offsets[E] of yp are left untouched.  offsets is read on the
 *   device and clamped to [0, rows].
 *   Limits: h and h_ffn multiples of 128.
 */
int moe_grouped_swiglu_fwd(const void* xp, const float* xp_scale, const moe_weights* W,
                           const int32_t* offsets, int rows, void* h13_save, void* yp, int yp_dtype,
                           void* ws, size_t ws_bytes, void* stream);

/* Workspace bytes for moe_grouped_swiglu_bwd. */
size_t moe_grouped_bwd_workspace_size(int rows, int h, int h_ffn, int E, int dtype);

/*
 * Backward of the GroupedGEMM (BF16 weights with w13_bwd and w2_bwd packed),
 * routing held fixed.
 *   dyp      [rows][h] bf16: gradient of yp (the weighted dispatch of dY).
 *   xp       [rows][h] bf16: the forward's routed input (re-gathered).
 *   h13_save [rows][2*h_ffn] bf16: FC1's output kept by the forward.
 *   dxp      [rows][h] bf16 out: gradient of xp.
 *   dw1, dw3 [E][h][h_ffn] fp32 out; dw2 [E][h_ffn][h] fp32 out (zero for an
 *            expert without rows).
 *   Math: A = SiLU(G) * U is recomputed from h13_save; dA = dyp W2^T;
 *   dW2 = A^T dyp; dG = dA * U * s * (1 + G (1 - s)) with s = sigmoid(G);
 *   dU = dA * SiLU(G); dxp = dG W1^T + dU W3^T; dW1 = xp^T dG;
 *   dW3 = xp^T dU.  Products accumulate in fp32.
 */
int moe_grouped_swiglu_bwd(const void* dyp, const void* xp, const void* h13_save,
                           const moe_weights* W, const int32_t* offsets, int rows, void* dxp,
                           float* dw1, float* dw3, float* dw2, void* ws, size_t ws_bytes,
                           void* stream);

/*
 * Combine: y[t] = sum_{j<k} topk_w[t][j] * yp[dst_row[t][j]], accumulated in
 * fp32 in increasing j, then rounded (nearest even) to y_dtype.
 *   yp       [*][h] element type yp_dtype (MOE_F32 or MOE_BF16).
 *   dst_row  [T][k] int32 rows in [0, T*k); other entries are skipped.
 *   topk_w   [T][k] fp32, or NULL for weight 1 (the transpose of the
 *            dispatch copy, used for dX).
 *   y        [T][h] element type y_dtype (MOE_F32 or MOE_BF16).
 *   h must be a multiple of 8.
 */
int moe_combine(const void* yp, int yp_dtype, const int32_t* dst_row, const float* topk_w, int T,
                int h, int k, void* y, int y_dtype, void* stream);

/*
 * FP8 backward of the expert GroupedGEMM (MegaScale-MoE paper review §三:
 * FP8 training with per-token instead of per-tensor scales; research digest
 * §3.4: fp32 sums).  Same products as moe_grouped_swiglu_bwd, on E4M3 codes:
 *   dA  = dYp W2^T: dYp codes per routed row (dyp_q, dyp_scale, from
 *         moe_permute of dY to FP8 with row_scale = topk_w) and W2 per h_ffn
 *         row (W->w2_bwd, w2_bwd_scale); dG, dU and A as in the BF16 backward,
 *         kept in bf16;
 *   dXp = [dG|dU] W13^T: dG|dU quantized per routed row, W13 per h row
 *         (W->w13_bwd, w13_bwd_scale); dxp bf16;
 *   dW2 = A^T dYp, dW13 = Xp^T [dG|dU]: these sum over tokens, where a
 *         per-token scale cannot leave the sum, so both transposed operands
 *         are quantized per channel over the expert's rows; fp32 out.
 *   Every product is a rank-1 rescale of an fp32 MFMA sum.
 *   dyp [rows][h] bf16: w * dY in dispatch order (moe_permute with row_scale),
 *   for dW2; xp [rows][h] bf16; h13_save as for the BF16 backward.
 *   W: dtype MOE_FP8_E4M3 with w13_bwd, w2_bwd and their scales.
 */
size_t moe_grouped_bwd_fp8_workspace_size(int rows, int h, int h_ffn, int E);
int moe_grouped_swiglu_bwd_fp8(const void* dyp_q, const float* dyp_scale, const void* dyp,
                               const void* xp, const void* h13_save, const moe_weights* W,
                               const int32_t* offsets, int rows, void* dxp, float* dw1, float* dw3,
                               float* dw2, void* ws, size_t ws_bytes, void* stream);

/*
 * The same FP8 backward, same results bit for bit, reading dY and x in token
 * order in place of their routed bf16 copies dyp and xp: the weight-gradient
 * operands are gathered row by row where they are transposed and quantized
 * (each value of dYp formed as bf16(w * dY), as moe_permute with row_scale
 * forms it), so the caller dispatches neither copy.
 *   dy, x    [T][h] bf16.
 *   dst_row  [T][k] int32 (moe_permute's output; pairs outside [0, rows) are
 *            skipped), topk_w [T][k] fp32: each routed row's token and weight.
 *   rows <= T*k; a row in [0, rows) that no pair targets reads as zeros.
 *   Everything else, the workspace size included, as
 *   moe_grouped_swiglu_bwd_fp8.
 */
int moe_grouped_swiglu_bwd_fp8_tok(const void* dyp_q, const float* dyp_scale, const void* dy,
                                   const void* x, const int32_t* dst_row, const float* topk_w, int T,
                                   int k, const void* h13_save, const moe_weights* W,
                                   const int32_t* offsets, int rows, void* dxp, float* dw1, float* dw3,
                                   float* dw2, void* ws, size_t ws_bytes, void* stream);

/*
 * The index, the dispatch copy and the expert forward in one call, with the
 * copy and FC1 overlapped by tile arrival (MegaScale-MoE research digest
 * §3.3 Diagram C and paper review §四 intra-operator overlap: the GEMM starts
 * a tile as soon as its rows have arrived, flagged on the device, instead of
 * after the whole exchange).  On one GPU the dispatch copy plays the
 * exchange: it runs on a second stream of the library's own, in row order,
 * and releases each expert's rows as they land; FC1 waits until a tile's
 * expert has landed whole before loading the tile.  Results
 * are those of moe_permute (index and BF16 copy) followed by
 * moe_grouped_swiglu_fwd, bit for bit.
 *   x [T][h] bf16; topk_idx [T][k] as for moe_permute; counts, offsets,
 *   dst_row, src_tok: moe_permute's index outputs; xp [T*k][h] bf16 out.
 *   W: MOE_BF16 weights; h13_save, yp, yp_dtype as moe_grouped_swiglu_fwd.
 *   status: one int32 on the device, set to 0 by the call, and to 1 if a wait
 *   of FC1 for its rows gave up after ~0.5 s (the copy found no room beside
 *   it, e.g. another process filling the GPU): then yp and h13_save are not
 *   valid.
 *   The call returns once everything is enqueued on `stream`; later work on
 *   `stream` runs after the copy too.  The second stream is one per device,
 *   shared by all calls: copies of calls on different streams run one after
 *   another; calls that share ws, or any output, and overlap race.
 */
size_t moe_dispatch_swiglu_fwd_workspace_size(int T, int k, int h, int h_ffn, int E);
int moe_dispatch_swiglu_fwd(const void* x, const int32_t* topk_idx, int T, int k, int32_t* counts,
                            int32_t* offsets, int32_t* dst_row, int32_t* src_tok, const moe_weights* W,
                            void* xp, void* h13_save, void* yp, int yp_dtype, int32_t* status, void* ws,
                            size_t ws_bytes, void* stream);

/*
 * Test of FC1's bounded waits in moe_dispatch_swiglu_fwd (same arguments and
 * checks): the index is built and FC1 and FC2 run, but the dispatch copy is
 * left out and a wait gives up after 64 polls instead of 2^20, so every wait
 * gives up and *status must read 1 once the stream has finished; xp is not
 * written, and h13_save and yp hold FC1/FC2 of whatever xp held.  The kernels
 * end normally; a later moe_dispatch_swiglu_fwd clears the status and the
 * flags itself.
 */
int moe_dispatch_swiglu_fwd_wait_selftest(const void* x, const int32_t* topk_idx, int T, int k,
                                          int32_t* counts, int32_t* offsets, int32_t* dst_row,
                                          int32_t* src_tok, const moe_weights* W, void* xp,
                                          void* h13_save, void* yp, int yp_dtype, int32_t* status,
                                          void* ws, size_t ws_bytes, void* stream);

/*
 * Router backward: gradients of  sum_t <dY_t, y_t> + L_aux  through the gate
 * (MegaScale-MoE paper review, §三 MoE layer structure: the gating network is
 * trainable), with the top-k selection held fixed.  For each token t,
 *   dw[t][j]      = <dy[t], yp[dst_row[t][j]]>                 (fp32 sum over h)
 *   dL[t][idx_j] += w_j (dw_j - sum_i w_i dw_i)                (softmax over the top k)
 *   dL[t][e]     += s_te (g_e - sum_e' s_te' g_e')             (balance loss, alpha != 0)
 * with s_t = softmax(logits[t]) over all E experts and
 * g_e = alpha * E / (k T) * counts[e] / T (see moe_router_aux_loss).  Then
 *   dw_gate = x^T dL,   dbias = sum_t dL[t],   dx = dx_in + dL W_g^T.
 *   dy       [T][h] element type dtype (MOE_BF16 or MOE_F32): the upstream
 *            gradient.
 *   yp       [T*k][h] element type yp_dtype (MOE_BF16 or MOE_F32): the
 *            forward's expert outputs.
 *   dst_row, topk_idx [T][k] int32, topk_w [T][k] fp32, logits [T][E] fp32
 *            (bias included), counts [E] int32: the forward's routing.
 *   x [T][h], w_gate [h][E]: dtype.
 *   dx_in    [T][h] fp32 (the expert path's dX, e.g. from moe_combine with
 *            y_dtype MOE_F32) or NULL for zero; dx [T][h] out, dtype (may not
 *            alias dx_in).
 *   dlogits  [T][E] fp32 out, or NULL (then dL stays in the workspace).
 *   dw_gate  [h][E] fp32 out; dbias [E] fp32 out or NULL.
 *   h must be a multiple of 64.  Every sum over tokens runs in a fixed order:
 *   results are bit-for-bit repeatable.
 */
size_t moe_router_bwd_workspace_size(int T, int h, int E);
int moe_router_bwd(const void* dy, const void* yp, int yp_dtype, const int32_t* dst_row,
                   const int32_t* topk_idx,
                   const float* topk_w, const float* logits, const int32_t* counts, int T, int h,
                   int E, int k, float alpha, int dtype, const void* x, const void* w_gate,
                   const float* dx_in, void* dx, float* dlogits, float* dw_gate, float* dbias,
                   void* ws, size_t ws_bytes, void* stream);

/*
 * Load-balance loss (MegaScale-MoE research digest §3.2: an auxiliary loss
 * balances the experts, following DeepSeek-V2; the digest prints no formula, and
 * DeepSeek-V2's expert-level form is used):
 *   loss = alpha * sum_e f_e P_e,  f_e = E / (k T) * counts[e],
 *   P_e  = (1/T) sum_t softmax(logits[t])_e.
 *   logits [T][E] fp32, counts [E] int32 (from moe_permute), loss: one fp32
 *   written on the device.  T >= 1.
 */
size_t moe_router_aux_workspace_size(int T, int E);
int moe_router_aux_loss(const float* logits, const int32_t* counts, int T, int E, int k,
                        float alpha, float* loss, void* ws, size_t ws_bytes, void* stream);

/*
 * Kernel timing for benchmarks.  moe_timing_enable(1) starts recording a pair
 * of HIP events around every kernel this library launches (on the launch
 * stream); moe_timing_enable(0) stops.  moe_timing_report() waits for the
 * recorded events and writes one line per kernel kind, "name count total_ms",
 * into buf (NUL-terminated, truncated to len), then clears the record.
 * Recording adds host work per launch; leave it off outside measurements.
 */
int moe_timing_enable(int on);
int moe_timing_report(char* buf, size_t len);

/*
 * Self-test of the FP8 encoder.  The activation quantizers (dispatch copy,
 * A, dG|dU, the transposed weight-gradient operands) encode with the
 * hardware's packed fp32 -> E4M3 conversion; this runs, for every finite
 * fp32 of magnitude <= 464 (the quantizers pass at most 448 (1 + 2^-23)),
 * that conversion and the library's bit-level reference encoder (OCP
 * E4M3FN, round to nearest even, saturating), in pairs and quadruples, and
 * writes the number of disagreements to *mismatches (one uint64 in device
 * memory, written on the stream; 0 expected).  The count also includes the
 * quantizers' quotient encoder (codes of v / s from one reciprocal per
 * scale, with the division where a quotient lies near a rounding boundary)
 * against the plain division, on 2^30 hashed quadruples of bf16 values with
 * their scales.  About 2^32 + 2^32 values: tens of milliseconds.
 */
int moe_fp8_convert_selftest(unsigned long long* mismatches, void* stream);

/* Message of the last failing call on this thread ("" if none). */
const char* moe_last_error(void);

/* ABI version of this library. */
int moe_version(void);

#ifdef __cplusplus
}
#endif

#endif /* MOE_MI355X_H */
