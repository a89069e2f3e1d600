/*
 * moe.h -- C ABI of the MI355X (gfx950) MoE layer forward library.
 *
 * One MoE layer's forward pass on one GPU's share of the work:
 *
 *   route     H = x W_g (+ b),  G = Softmax(KeepTopK(H, k))
 *   dispatch  per-expert histogram, capacity, token-order positions, and the
 *             expert-contiguous send buffer the dispatch all-to-all would send
 *   expert    SwiGLU FFN of every expert on its rows (grouped GEMM)
 *   combine   y[t] = sum over kept s of G[t,s] * Expert_{idx[t,s]}(x[t])
 *
 * Sources (page title, section):
 *   [G]  "Mixture-of-Experts (MoE) Architecture and Expert Parallelism",
 *        section 2 "The Gating Network Formulation".
 *   [N]  "EP Math -- Expert Parallelism (MoE)", "Notation": T tokens on one
 *        device, d hidden size, k experts per token, D devices, T*k
 *        assignments per device.
 *   [DA] same page, "The dispatch all-to-all"; [CA] "The combine all-to-all";
 *   [CF] "Capacity factor"; [TD] "Token drop"; [PL] "Placing experts across
 *        devices".
 *   [M]  "MoE Expert Parallelism Sizing: Traffic, Capacity, Fabric":
 *        "Memory residency for the same shape" (gated three-matrix expert),
 *        "Capacity semantics decide what crosses the wire" (drop before the
 *        exchange), "First-order dispatch and combine bytes" (one input chunk
 *        per destination rank).
 *   [DP] same page, "Capacity semantics decide what crosses the wire" and its
 *        question on the capacity factor: with a capacity factor set, tokens
 *        beyond an expert's capacity are dropped by selected probability.
 *   [MC] same page, the DeepSpeed paragraph: C raised to a floor,
 *        min_capacity, whatever the capacity factor gives.
 *   [F8] same page, "What the bounds omit": FP8 rows on dispatch, bf16 on
 *        combine; per-row scales added to the traffic.
 *   [GL] same page, the traffic bounds: at most 4 nodes per token
 *        (DeepSeek-V3), exposed by Megatron as group-limited routing.
 *   [SE] same page, the token-assignment worksheet: the shared expert is
 *        replicated on every rank (compute and memory, no dispatch traffic).
 *   [RS] same page, "Rank-level skew and the straggler effect": the load
 *        imbalance ratio (max - mean) / mean.
 *
 * Conventions for every call
 *   - Tensor pointers are DEVICE pointers (HIP global memory) unless marked
 *     "host".  bf16 tensors are passed as raw 16-bit patterns (uint16_t).
 *     All tensors are dense row-major with the shapes given.  Every device
 *     pointer must be 16-byte aligned; the workspace 256-byte aligned.  A
 *     pointer to a tensor with no elements (T = 0, or send_rows = 0) may be
 *     NULL; every other required pointer must not be.
 *   - The caller owns every buffer, including the workspace sized by
 *     moe_query.  The library allocates nothing, frees nothing, keeps no
 *     state between calls and never synchronises the host with the device.
 *   - Work is enqueued on `stream` (a hipStream_t; NULL = the null stream)
 *     and runs in stream order.  Calls that share a workspace must not
 *     overlap in time.
 *   - Arguments are validated on the host before anything is enqueued; on
 *     an error nothing is enqueued and no output is touched.
 *   - Inputs must be finite.  Non-finite x, W_g or bias give unspecified
 *     routing.
 *   - Results are deterministic: the same inputs give bitwise-identical
 *     outputs on every run.
 */
#ifndef MOE_MI355X_H
#define MOE_MI355X_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Status codes returned by every call. */
#define MOE_OK 0
#define MOE_EINVAL (-1)       /* bad argument: null/misaligned pointer, bad size */
#define MOE_EUNSUPPORTED (-2) /* valid shape that no kernel here handles         */
#define MOE_EWORKSPACE (-3)   /* workspace NULL or smaller than moe_query says  */
#define MOE_EHIP (-4)         /* a HIP launch reported an error                 */
#define MOE_ESCRATCH (-5)     /* moe_dispatch_noalloc: the shape needs more     */
                              /* scratch than MOE_DISPATCH_SCRATCH_BYTES        */

/* Shape of one layer on one device, in the pages' notation [N][CF][PL][DP][MC][F8][GL][SE].
 *   T        tokens on this device (T >= 0; T = 0 enqueues nothing)
 *   d        hidden size (d > 0, d % 64 == 0)
 *   E        routed experts (1 <= E <= 1024, E % D == 0)
 *   k        experts per token (1 <= k <= E)
 *   H        SwiGLU hidden size of one expert (H > 0, H % 64 == 0)
 *   D        logical destination ranks (D >= 1); rank r owns the contiguous
 *            experts [r*E/D, (r+1)*E/D)  [PL]
 *   my_rank  this device's rank, 0 <= my_rank < D (only for byte accounting)
 *   drop_policy  which assignments an expert over capacity keeps:
 *            0: the first C by token index (token order);
 *            1: the C with the largest gate value G = topk_w[t,s], equal G
 *               going to the lower token index [DP].
 *            Either way the kept rows sit in ascending token order inside
 *            the expert's block, and the counts (so offsets, bytes and
 *            per-rank rows) are the same.  Other values -> MOE_EINVAL.
 *   min_capacity  >= 0: in capacity mode C = max(ceil(f*T*k/E), min_capacity)
 *            [MC]; 0 leaves C as computed.  Ignored when dropless.
 *   dispatch_fp8  0: the send buffer holds bf16 rows (d * 2 bytes each).
 *            1 [F8]: it holds OCP FP8 E4M3 rows (d bytes each) and a
 *            separate fp32 scale per row: s = amax/448 computed in fp32 (1 for
 *            an all-zero row), code = E4M3(x/s) with the quotient in fp32,
 *            rounded to nearest (ties to even), saturating at 448, sign kept.
 *            The expert sees code value * s; expert_out, h and the combine
 *            stay bf16.  Other values -> MOE_EINVAL.
 *   n_groups, group_limit  [GL]: with n_groups = G > 1 and group_limit =
 *            M < G, the experts form G contiguous groups of E/G; a group's
 *            score for a token is its largest logit, the M best groups are
 *            kept (ties to the lower group index) and KeepTopK picks among
 *            their experts only.  G must divide E and M*E/G >= k (else
 *            MOE_EINVAL); n_groups <= 1 or group_limit >= n_groups: no limit.
 *   shared_H  [SE]: SwiGLU hidden size of a shared expert applied to every
 *            token and added, with weight 1, to the combine; 0 = none;
 *            shared_H % 64 == 0 (else MOE_EUNSUPPORTED).
 *   capacity_factor  f > 0: capacity C = ceil(f*T*k/E), evaluated left to
 *            right in IEEE double [CF]; +INFINITY: dropless (no capacity).
 *            NaN, zero, negative -> MOE_EINVAL.
 */
typedef struct moe_shape {
    int32_t T, d, E, k, H, D, my_rank;
    int32_t drop_policy;
    int32_t min_capacity;
    int32_t dispatch_fp8;
    int32_t n_groups, group_limit;
    int32_t shared_H;
    double capacity_factor;
} moe_shape;

/* Device-resident counters written by moe_dispatch (and moe_layer_fwd).
 *   assignments           T*k  [N]
 *   kept                  assignments that reach an expert
 *   dropped               assignments - kept  [TD]
 *   padded                E*C - kept in capacity mode, 0 when dropless  [CF]
 *   capacity              C, or -1 when dropless
 *   send_rows             rows of the send buffer: E*C, or T*k when dropless
 *   dispatch_bytes        kept * row bytes: the token vectors that travel
 *                         [DA]; a row is d*2 bytes (bf16), or d + 4 under
 *                         FP8 dispatch (codes plus the row's scale) [F8]
 *   dispatch_wire_bytes   send_rows * row bytes in capacity mode (pads
 *                         included, the static [E, C, d] buffer), as
 *                         dispatch_bytes when dropless
 *   dispatch_remote_bytes kept rows bound for ranks other than my_rank,
 *                         times the row bytes
 *   combine_bytes         kept*d*2: the bf16 expert outputs that travel back
 *                         (combine reverses dispatch) [CA]
 *   max_expert_count      max over experts of the routed count n_e; with
 *                         the mean T*k/E it gives the load imbalance
 *                         (max - mean) / mean over experts [RS] (rank_rows
 *                         gives it over destination ranks)
 *   invalid_index         topk_idx entries outside [0, E), or repeating an
 *                         expert listed earlier for the same token; each is
 *                         treated as dropped (slot -1), never as an error
 */
typedef struct moe_stats {
    int64_t assignments, kept, dropped, padded, capacity, send_rows;
    int64_t dispatch_bytes, dispatch_wire_bytes, dispatch_remote_bytes;
    int64_t combine_bytes, max_expert_count, invalid_index;
} moe_stats;

/* Host-only size query.  Writes (host pointers, each may be NULL):
 *   send_rows        rows of send_buf / expert_out: E*C, or T*k if dropless
 *                    (C includes the minimum capacity)
 *   capacity         C, or -1 if dropless  [CF]
 *   workspace_bytes  bytes of device workspace every call below needs
 *                    (one size serves them all)
 * Returns MOE_OK, or MOE_EINVAL / MOE_EUNSUPPORTED for a bad shape. */
int moe_query(const moe_shape *shape, int64_t *send_rows, int64_t *capacity,
              size_t *workspace_bytes);

/* Router [G][GL]: logits H = x W_g (+ bias), fp32 accumulation of exact
 * bf16 products; then KeepTopK (within the token's best groups under a
 * group limit) + softmax over the kept logits.
 *   x           [T, d] bf16
 *   w_gate      [d, E] bf16 (d_model x E, as W_g is written on the page)
 *   logit_bias  [E] fp32 or NULL; added to H, so it enters selection and
 *               softmax alike
 *   logits_out  [T, E] fp32 or NULL (the fp32 logits the selection used)
 *   topk_idx    [T, k] int32 out: kept experts, descending logit, ties to
 *               the lower expert index
 *   topk_w      [T, k] fp32 out: gates G, summing to 1 per token
 *   workspace   device, workspace_bytes >= moe_query's size */
int moe_route(const moe_shape *shape, const uint16_t *x, const uint16_t *w_gate,
              const float *logit_bias, float *logits_out, int32_t *topk_idx, float *topk_w,
              void *workspace, size_t workspace_bytes, void *stream);

/* KeepTopK + softmax alone, on caller-given fp32 logits [T, E] [G].  Same
 * selection and gates as moe_route; lets routing be compared on identical
 * logits. */
int moe_topk_from_logits(const moe_shape *shape, const float *logits, int32_t *topk_idx,
                         float *topk_w, void *stream);

/* Dispatch [N][CF][TD][PL][M][DP][F8]: histogram n_e, capacity, positions,
 * slots and the send buffer.
 *   x             [T, d] bf16
 *   topk_idx      [T, k] int32 (entries outside [0, E), and repeats of an
 *                 expert already listed for the token, are counted in
 *                 stats->invalid_index and dropped)
 *   topk_w        [T, k] fp32 gates (as moe_route writes them): read only by
 *                 drop policy 1 in capacity mode, may be NULL otherwise
 *   send_buf      [send_rows, d] out: bf16, or E4M3 codes under FP8 dispatch
 *                 (the row of a kept assignment is its token's row, quantized
 *                 with that row's scale).  Expert e's kept rows are
 *                 [expert_offset[e], expert_offset[e] + expert_kept[e]), in
 *                 ascending token order; capacity mode gives expert e the
 *                 rows [e*C, (e+1)*C) and zero-fills the pad rows; when
 *                 dropless, rows [expert_offset[E], T*k) -- present only if
 *                 entries were invalid -- are zero-filled too.  Experts
 *                 are in ascending order, so rank r's chunk -- what the
 *                 dispatch all-to-all sends to rank r -- is rows
 *                 [expert_offset[r*E/D], expert_offset[(r+1)*E/D]).
 *   send_scale    [send_rows] fp32 out under FP8 dispatch (pad rows: 0), may
 *                 be NULL otherwise
 *   slot          [T, k] int32 out: send_buf row of assignment (t, s), or -1
 *                 if dropped
 *   expert_count  [E] int32 out: n_e, assignments routed to expert e
 *   expert_kept   [E] int32 out: min(n_e, C) (n_e when dropless)
 *   expert_offset [E+1] int32 out: first send_buf row of each expert
 *   rank_rows     [D] int32 out: kept rows per destination rank
 *   stats         one moe_stats, device memory, out
 *   workspace     device, >= moe_query's size */
int moe_dispatch(const moe_shape *shape, const uint16_t *x, const int32_t *topk_idx,
                 const float *topk_w, void *send_buf, float *send_scale, int32_t *slot, int32_t *expert_count, int32_t *expert_kept,
                 int32_t *expert_offset, int32_t *rank_rows, moe_stats *stats, void *workspace,
                 size_t workspace_bytes, void *stream);

/* moe_dispatch for callers that cannot allocate device memory: code under
 * HIP graph capture, tight serving loops, harnesses that forbid allocation.
 * Arguments, outputs and results are those of moe_dispatch (bit for bit);
 * there is no workspace argument.  The dispatch's scratch (per-chunk expert
 * counts and their scan, and under drop policy 1 the by-expert assignment
 * list) lives in a static device array of MOE_DISPATCH_SCRATCH_BYTES that
 * each GPU the library runs on holds until the process ends; its address is
 * looked up on the first call on a device.  Nothing is allocated, freed or
 * cleared with a memset.  Every call on one GPU shares that GPU's array, so
 * calls that overlap in time on one GPU (different streams, or different
 * host threads) race and must not be issued.  Returns MOE_ESCRATCH, before
 * anything is enqueued, for a shape whose scratch exceeds the array:
 * 8 * ceil(T/256) * E + 4 * ceil(T/256) bytes, plus 4 * (E + T*k) under drop
 * policy 1 in capacity mode, each region rounded up to 256 bytes. */
#define MOE_DISPATCH_SCRATCH_BYTES ((size_t)8 << 20)
int moe_dispatch_noalloc(const moe_shape *shape, const uint16_t *x, const int32_t *topk_idx,
                         const float *topk_w, void *send_buf, float *send_scale, int32_t *slot,
                         int32_t *expert_count, int32_t *expert_kept, int32_t *expert_offset,
                         int32_t *rank_rows, moe_stats *stats, void *stream);

/* Expert FFN [M]: for every expert e, on its kept rows X_e of send_buf,
 *   h = bf16(SiLU(X_e W1_e^T) * (X_e W3_e^T)),  out = bf16(h W2_e^T),
 * SiLU(z) = z / (1 + exp(-z)), fp32 accumulation on bf16 matrix cores.
 *   send_buf       [send_rows, d] bf16, or E4M3 codes under FP8 dispatch
 *   send_scale     [send_rows] fp32 row scales under FP8 dispatch, may be
 *                  NULL otherwise; the expert's input row is code * scale
 *   expert_offset  [E+1] int32, expert_kept [E] int32 (as moe_dispatch
 *                  writes them); an expert's rows [offset, offset + kept)
 *                  are clipped to [0, send_rows), a negative offset or count
 *                  gives none
 *   w1, w3         [E, H, d] bf16;  w2 [E, d, H] bf16
 *   expert_out     [send_rows, d] bf16 out; only kept rows are written
 *   workspace      device, >= moe_query's size (holds h) */
int moe_expert_ffn(const moe_shape *shape, const void *send_buf, const float *send_scale,
                   const int32_t *expert_offset,
                   const int32_t *expert_kept, const uint16_t *w1, const uint16_t *w3,
                   const uint16_t *w2, uint16_t *expert_out, void *workspace,
                   size_t workspace_bytes, void *stream);

/* The two halves of moe_expert_ffn, for callers that keep h themselves.
 * moe_expert_gate_up:  h = bf16(SiLU(X_e W1_e^T) * (X_e W3_e^T)) for every
 *   expert's kept rows; h is [send_rows, H] bf16, row r of h belongs to row r
 *   of send_buf; only kept rows are written.
 * moe_expert_down:     expert_out = bf16(h W2_e^T) on the same rows.
 * Arguments as in moe_expert_ffn.  moe_expert_down needs no workspace; for
 * moe_expert_gate_up it is optional (NULL, 0 allowed; otherwise at least
 * moe_query's size, and h must not lie inside it).  With dispatch_fp8 set
 * and an expected load of at least 512 rows per expert (C, or T*k/E when
 * dropless), a workspace lets the E4M3 rows be widened to bf16 in one pass
 * before the GEMM (moe_expert_ffn and moe_layer_fwd always do); without one
 * the GEMM widens them in registers.  Both give the same output bits. */
int moe_expert_gate_up(const moe_shape *shape, const void *send_buf, const float *send_scale,
                       const int32_t *expert_offset, const int32_t *expert_kept,
                       const uint16_t *w1, const uint16_t *w3, uint16_t *h, void *workspace,
                       size_t workspace_bytes, void *stream);
int moe_expert_down(const moe_shape *shape, const uint16_t *h, const int32_t *expert_offset,
                    const int32_t *expert_kept, const uint16_t *w2, uint16_t *expert_out,
                    void *stream);

/* Combine [G][CA][TD][SE]: y[t] = bf16(sum over s with slot[t,s] >= 0, in s
 * order, of topk_w[t,s] * expert_out[slot[t,s]], then + shared_out[t]) with
 * fp32 accumulation.  Dropped assignments add nothing; the residual is the
 * caller's to add.
 *   expert_out  [send_rows, d] bf16;  slot, topk_w [T, k];  a slot outside
 *               [0, send_rows) counts as dropped (never read past the rows)
 *   shared_out  [T, d] bf16 (the shared expert's output) or NULL;
 *   y [T, d] bf16 out */
int moe_combine(const moe_shape *shape, const uint16_t *expert_out, const int32_t *slot,
                const float *topk_w, const uint16_t *shared_out, uint16_t *y, void *stream);

/* Shared expert [SE][M]: shared_out = bf16(SiLU(x W1s^T) * (x W3s^T)) W2s^T
 * for every token (h rounded to bf16, fp32 accumulation), the same SwiGLU as
 * the routed experts, on x directly: it is replicated, so nothing is
 * dispatched for it.  Requires shape->shared_H > 0 (else MOE_EINVAL).
 *   x [T, d] bf16;  w1s, w3s [shared_H, d] bf16;  w2s [d, shared_H] bf16
 *   shared_out [T, d] bf16 out;  workspace >= moe_query's size */
int moe_shared_expert(const moe_shape *shape, const uint16_t *x, const uint16_t *w1s,
                      const uint16_t *w3s, const uint16_t *w2s, uint16_t *shared_out,
                      void *workspace, size_t workspace_bytes, void *stream);

/* The whole forward pass: moe_route, moe_dispatch, moe_expert_ffn,
 * moe_shared_expert (when shared_H > 0) and moe_combine enqueued back to
 * back on `stream`, with no host synchronisation; every intermediate lands
 * in the caller's buffers with the meaning given above.  logit_bias and
 * logits_out may be NULL; w1s, w3s, w2s and shared_out are required when
 * shared_H > 0 and may be NULL otherwise. */
int moe_layer_fwd(const moe_shape *shape, const uint16_t *x, const uint16_t *w_gate,
                  const float *logit_bias, const uint16_t *w1, const uint16_t *w3,
                  const uint16_t *w2, const uint16_t *w1s, const uint16_t *w3s,
                  const uint16_t *w2s, uint16_t *y, float *logits_out, int32_t *topk_idx,
                  float *topk_w, void *send_buf, float *send_scale, int32_t *slot,
                  int32_t *expert_count,
                  int32_t *expert_kept, int32_t *expert_offset, int32_t *rank_rows,
                  moe_stats *stats, uint16_t *expert_out, uint16_t *shared_out,
                  void *workspace, size_t workspace_bytes, void *stream);

/* Diagnostic decode of FP8 dispatch rows [F8]: out[r, i] = bf16(value of
 * E4M3 code codes[r*d + i] * scales[r]), with the product rounded to fp32
 * then to bf16 (nearest even); exact when every scale is a power of two.
 * It uses the same decode as the expert GEMM.
 *   codes   [rows, d] E4M3 (device); scales [rows] fp32 (device)
 *   rows >= 0; d > 0, d % 16 == 0;  out [rows, d] bf16 (device) */
int moe_fp8_rows_to_bf16(const void *codes, const float *scales, int64_t rows, int32_t d,
                         uint16_t *out, void *stream);

/* Diagnostic, not a step of the layer: reads bytes of device memory at
 * src once, with the non-temporal 16-byte loads that the expert GEMMs use
 * for their weights, so that a caller can time this device's streaming-read
 * rate beside the layer's kernels.  Each reading lane XORs the 32-bit words
 * it reads; a lane whose XOR equals MOE_STREAM_READ_MARK stores it to *sink,
 * and nothing else is written (so a buffer of zeros holding the mark in one
 * word sets *sink to the mark exactly when that word is read).
 *   src   device, 16-byte aligned; bytes % 16 == 0 (bytes == 0: no launch)
 *   sink  device uint32, 16-byte aligned
 * Returns MOE_EINVAL for a bad pointer or size, MOE_EHIP on a launch error. */
#define MOE_STREAM_READ_MARK 0x9E3779B9u
int moe_stream_read(const void *src, size_t bytes, uint32_t *sink, void *stream);

/* Diagnostic, not a step of the layer: writes value to every 32-bit word of
 * the bytes of device memory at dst, once, with the non-temporal 16-byte
 * stores that the permute and the expert GEMMs' epilogues write with, so
 * that a caller can time this device's streaming-store rate beside the
 * layer's kernels.
 *   dst   device, 16-byte aligned, caller-owned; bytes % 16 == 0 (0: no launch)
 * Returns MOE_EINVAL for a bad pointer or size, MOE_EHIP on a launch error. */
int moe_stream_write(void *dst, size_t bytes, uint32_t value, void *stream);

/* Diagnostic, not a step of the layer: the combine's memory traffic without
 * its arithmetic, out[t] = XOR over s < k of the 16-byte pieces of row
 * slot[t, s] of rows (a slot outside [0, nrows) adds nothing), with the
 * combine's access (a wavefront per token, or several sharing its row when
 * there are fewer than 4096 tokens; non-temporal 16-byte gathers, all k of
 * a piece in flight together for k <= 8), so that a caller can
 * time the rate of that access beside moe_combine.
 *   rows  [nrows, d] bf16 (device);  slot [T, k] int32 (device)
 *   out   [T, d] bf16 out (device);  d % 8 == 0, k >= 1
 * Returns MOE_EINVAL for a bad pointer or size, MOE_EHIP on a launch error. */
int moe_stream_gather(const void *rows, int64_t nrows, int32_t d, const int32_t *slot,
                      int64_t T, int32_t k, void *out, void *stream);

/* Static string naming a status code (never NULL). */
const char *moe_status_str(int status);

#ifdef __cplusplus
}
#endif

#endif /* MOE_MI355X_H */
