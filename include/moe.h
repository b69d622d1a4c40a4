/*
 * moe.h -- C ABI of the MI355X (gfx950) fused mixture-of-experts layer:
 * top-k routing, token sort into expert order (dispatch), grouped gate/up
 * GEMM with SwiGLU, grouped down GEMM, weighted combine, and the full
 * backward of that layer, for one GPU's share of the work.
 *
 * The operation is the one described on the pages
 *   "Prime Intellect's Prime Mega MoE Trains Giant AI Models 55% Faster"
 *     (section "Where MoE training loses time": dispatch tokens to their
 *     experts, run the expert MLPs, return outputs to their original
 *     positions; the backward repeats the exchange for gradients) and
 *   "Prime Intellect Fused MoE Kernel: 3.11x MoE Training Speed"
 *     (section "What a mixture-of-experts layer actually does": dispatch,
 *     both expert linear layers, SwiGLU and the combine), with the routing
 *     inputs of "Mario/overlap moe kernel integration" (prime-rl PR 3651,
 *     commit on GroupedExperts.forward: either per-expert token counts or
 *     top scores plus selected expert indices).
 *
 * Notation: T tokens, d hidden size, E experts, k experts per token, I expert
 * intermediate size, R = T*k routed rows.  All matrices are row-major and
 * densely packed (leading dimension = last extent).
 *
 * Math (per token t, slot j, expert e = topk_ids[t][j]):
 *   topk_ids[t]  = the k largest logits of row t, largest first, ties to the
 *                  lower expert index (-0.0 equals +0.0);
 *   topk_w[t][j] = exp(l_tj) / sum_{i<k} exp(l_ti)   (softmax over the k
 *                  selected logits = full softmax renormalised over top k);
 *   h = W_gate_up[e] x_t  (rows [0,I) gate g, rows [I,2I) up u),
 *   a = silu(g) * u,  y_tj = W_down[e] a,  out_t = sum_j topk_w[t][j] y_tj.
 *   The backward is the exact gradient of L = sum(dout * out).
 *
 * Ownership: the caller allocates every buffer (device memory unless noted)
 * and keeps it alive until the stream has finished the call.  The library
 * never allocates, frees or keeps device memory between calls, performs no
 * device-to-host copy and no stream synchronisation: every call only
 * enqueues kernels on `stream` (a hipStream_t; NULL = the default stream),
 * so calls may be captured into a HIP graph.  Calls on different streams
 * need separate workspaces and outputs.
 *
 * Errors: every argument check runs on the host before any HIP call; a
 * failing check returns a status and enqueues nothing.  moe_last_error()
 * gives a message for the last failure on the calling thread.  Device-side
 * contract violations in the ids-in form (an id outside [0, E), repeated ids
 * in a row, non-finite values) are not detected; ids are clamped into
 * [0, E) so that no access leaves its buffer, and results are then
 * unspecified.
 */
#ifndef MOE_MI355X_H
#define MOE_MI355X_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  MOE_OK = 0,
  MOE_ERR_INVALID_ARGUMENT = 1, /* null pointer, bad extent, k > E, ...     */
  MOE_ERR_UNSUPPORTED = 2,      /* valid but not built (dtype, alignment)   */
  MOE_ERR_WORKSPACE = 3,        /* workspace smaller than moe_workspace_bytes */
  MOE_ERR_HIP = 4               /* a kernel launch failed                   */
} moe_status;

typedef enum { MOE_F32 = 0, MOE_BF16 = 1 } moe_dtype;

/* Precision of the GEMM operands.  MOE_PREC_FP8_BLOCK: blockwise FP8
 * ("Prime Mega MoE Trains Giant AI Models 55% Faster", section "Precision and
 * hardware support": one scale shared by a block of values) as OCP e4m3 with
 * fp32 scales over 1x128 activation blocks and 128x128 weight blocks
 * (weight-gradient operands: 128-row blocks along the token dimension), fp32
 * accumulation.  MOE_PREC_MXFP8: the OCP microscaling format MXFP8 (same
 * section: smaller scaling groups than blockwise FP8; "Mario/overlap moe
 * kernel integration" overview: an mxfp8 precision option): e4m3 values in
 * blocks of 32 along every GEMM operand's contraction dimension, each block
 * with a power-of-two scale stored as an E8M0 byte (see
 * moe_quantize_mxfp8), fp32 accumulation.  MOE_PREC_FP8_BWD (the PR's
 * fp8_bwd option): FP8 in the backward only -- the forward of the bf16 layer,
 * then the backward of MOE_PREC_FP8_BLOCK on the saved bf16 H and Aw (the
 * backward quantises the weights itself).  The fp8 precisions require dtype
 * MOE_BF16, d and I multiples of 128 and T*k*max(d, 2I)/128 < 2^31; H and
 * Aw are stored in bf16, and dH is rounded to bf16 before it is encoded. */
typedef enum {
  MOE_PREC_NATIVE = 0,
  MOE_PREC_FP8_BLOCK = 1,
  MOE_PREC_MXFP8 = 2,
  MOE_PREC_FP8_BWD = 3
} moe_precision;

/* MOE_OP_BACKWARD_RECOMPUTE sizes a moe_backward call that gets saved ==
 * NULL and recomputes what moe_forward would have saved. */
typedef enum {
  MOE_OP_ROUTE = 0,
  MOE_OP_FORWARD = 1,
  MOE_OP_BACKWARD = 2,
  MOE_OP_BACKWARD_RECOMPUTE = 3
} moe_op;

typedef struct {
  int64_t T, d, E, k, I;
  int32_t dtype;        /* moe_dtype of x, weights, out, saved, dout, grads */
  int32_t logits_dtype; /* moe_dtype of logits and dlogits                  */
  int32_t precision;    /* moe_precision                                    */
  float swiglu_limit;   /* 0: SwiGLU; > 0 (finite): clamped SwiGLU, below   */
  int32_t flags;        /* moe_flags; unknown bits are rejected            */
} moe_shape;

/* MOE_FLAG_PERSISTENT: the bf16 GEMMs (gate/up and down forward, down and
 * gate/up data gradients, and, in MOE_PREC_NATIVE, both weight gradients;
 * also the forward of MOE_PREC_FP8_BWD) run as persistent kernels, one
 * work-group per CU walking its XCD's tiles, that issue the next tile's
 * first stage (its gathered token rows and weight slice, or for a weight
 * gradient its first 64 rows of both operands) during the current tile's
 * last K step, so that it loads while that step's MFMAs run and while the
 * epilogue stores: the one-GPU form of the overlapped pipeline in "Prime
 * Intellect's Prime Mega MoE Trains Giant AI Models 55% Faster", section
 * "One kernel overlaps the pipeline".  Results are bit-identical to the
 * default engine's (every tile runs at full height, with the same MFMA
 * order).  Other precisions and MOE_F32 ignore the flag. */
typedef enum { MOE_FLAG_PERSISTENT = 1 } moe_flags;

/* swiglu_limit > 0 selects the clamped SwiGLU that "Mario/overlap moe kernel
 * integration" names for DeepSeek V4 (commit on activations.ClampedSilu);
 * the pages give neither its form nor its constant, so the limit L is an
 * argument and the form is read as a = silu(min(g, L)) * clamp(u, -L, L),
 * with no gradient through an active clamp (g > L, |u| > L).  The pages'
 * other clamped variant (sigmoid of 1.702 g, up + 1) is not computed.  H in
 * `saved` holds the unclamped pre-activations. */

/* Limits checked by every call: 1 <= T <= 2^24, 1 <= k <= E <= 1024,
 * T*k <= 2^27, d and I multiples of 8 in [8, 16384]. */

/* Routing tensors (device pointers).  logits [T,E] in logits_dtype, or NULL
 * for the ids-in form, where topk_ids/topk_w are inputs used as given (no
 * renormalisation).  Otherwise topk_ids/topk_w are outputs.
 *   topk_ids [T,k] int32, topk_w [T,k] float32
 *   counts  [E]   int32  rows per expert
 *   offsets [E+1] int32  exclusive prefix sum of counts, offsets[E] = T*k
 *   row_of  [T*k] int32  flat entry t*k+j -> its row in expert order
 *   src_of  [T*k] int32  row -> flat entry; rows are ordered by expert, then
 *                        by flat entry (token order inside each expert) */
typedef struct {
  const void* logits;
  int32_t* topk_ids;
  float* topk_w;
  int32_t* counts;
  int32_t* offsets;
  int32_t* row_of;
  int32_t* src_of;
} moe_routing;

/* Bytes of device workspace a call with this shape needs (op: moe_op);
 * 0 when the shape or op is invalid (moe_last_error() says why).  The
 * caller owns the workspace: the pages' layer owns persistent buffers
 * ("Mario/overlap moe kernel integration", commit list: symmetric buffers
 * that the layer allocates and destroys itself),
 * whereas on one GPU nothing has to outlive a call, so here every call takes
 * its scratch memory from the caller. */
size_t moe_workspace_bytes(const moe_shape* shape, int op);

/* Bytes of the `saved` buffer written by moe_forward and read by
 * moe_backward (0 for an invalid shape): H [T*k, 2I] (gate|up
 * pre-activations) followed by Aw [T*k, I] (SwiGLU output times the row's
 * top-k weight), both in dtype, in expert-sorted row order.  With an fp8
 * forward (MOE_PREC_FP8_BLOCK, MOE_PREC_MXFP8) the buffer also holds the
 * e4m3 weight codes and scales that the backward's data gradients use (both
 * weights are quantised once, in the forward): for MOE_PREC_FP8_BLOCK the
 * forward's own encodings (a 128 x 128 block has one scale whichever axis
 * the contraction runs over), for MOE_PREC_MXFP8 a second, transposed
 * encoding (its 32-value blocks run along one axis).  The
 * forward keeps these so that the backward, which repeats the layer's
 * exchange for gradients ("Prime Mega MoE Trains Giant AI Models 55%
 * Faster", section "Where MoE training loses time"), need not recompute
 * them; moe_backward with saved == NULL recomputes instead. */
size_t moe_saved_bytes(const moe_shape* shape);

/* The same sizes with a status: MOE_OK and *bytes set, or the reason the
 * shape or op is rejected. */
moe_status moe_workspace_size(const moe_shape* shape, int op, size_t* bytes);
moe_status moe_saved_size(const moe_shape* shape, size_t* bytes);

/* Routing only: top-k (when logits != NULL), per-expert counts and offsets,
 * and the stable expert-order permutation.  The router sends each token to
 * a small subset of experts, and dispatch sorts the tokens into expert
 * order ("Prime Mega MoE Trains Giant AI Models 55% Faster", section "Where
 * MoE training loses time"); the routing tensors are the per-token top
 * scores and selected expert indices, or the per-expert token counts
 * ("Mario/overlap moe kernel integration", commit on
 * GroupedExperts.forward(x, *routing)).  Logits in: the k largest per
 * token, weights the softmax over them (see the math above); ids in
 * (logits == NULL): topk_ids and topk_w are read as given, and only counts,
 * offsets, row_of and src_of are written. */
moe_status moe_route(const moe_shape* shape, moe_routing* routing,
                     void* workspace, size_t workspace_bytes, void* stream);

/* moe_route for callers that cannot allocate device memory (code under HIP
 * graph capture, tight serving loops, harnesses that forbid allocation): the
 * same kernels and results, with no workspace argument.  The counting
 * sort's per-chunk histograms live in a 4 MiB array of device memory that
 * the library holds on each GPU it runs on until the process ends, so
 * 4 * ceil(T*k / 1024) * E must not exceed 4 MiB (T*k*E <= 2^30); larger
 * shapes get MOE_ERR_UNSUPPORTED before anything is enqueued.  Every call on
 * one GPU uses that GPU's one array: calls that overlap in time on the same
 * GPU (different streams, or host threads) race and must be serialised by
 * the caller.  The array needs no clearing between calls (each call writes
 * every histogram it reads).  The first call on a device looks the array up
 * (hipGetSymbolAddress); no call allocates. */
moe_status moe_route_noalloc(const moe_shape* shape, moe_routing* routing, void* stream);

/* Layer forward: routing as moe_route, then out [T,d] (dtype): dispatch
 * into expert order, both expert linear layers with SwiGLU, and the combine
 * that returns each token's k expert outputs to its position, weighted by
 * topk_w ("Prime Intellect Fused MoE Kernel: 3.11x MoE Training Speed",
 * section "What a mixture-of-experts layer actually does"; "Prime Mega MoE
 * Trains Giant AI Models 55% Faster", section "Where MoE training loses
 * time").  x [T,d], w_gate_up [E,2I,d], w_down [E,d,I] in dtype.  saved:
 * NULL, or a buffer of moe_saved_bytes bytes that moe_backward will read.
 * workspace: moe_workspace_bytes(shape, MOE_OP_FORWARD) bytes, 256-byte
 * aligned; x, the weights, out and saved 16-byte aligned. */
moe_status moe_forward(const moe_shape* shape, const void* x, moe_routing* routing,
                       const void* w_gate_up, const void* w_down, void* out,
                       void* saved, void* workspace, size_t workspace_bytes,
                       void* stream);

/* Layer backward from the routing and `saved` of a moe_forward call with
 * the same inputs.  dout [T,d] (dtype).  Outputs: dx [T,d],
 * dw_gate_up [E,2I,d], dw_down [E,d,I] (dtype; experts with no rows get
 * exact zeros), d_topk_w [T,k] float32, and dlogits [T,E] (logits_dtype;
 * zero outside the selected experts) or NULL.  dlogits requires the logits
 * form of routing (routing->logits != NULL).
 * saved == NULL selects recomputation (activation checkpointing, where a
 * layer costs two forwards and one backward: "Prime Intellect added the
 * missing backward pass to DeepSeek's fused MoE kernel ..."; "Prime Mega MoE
 * Trains Giant AI Models 55% Faster", section "Where MoE training loses
 * time"): the call first reruns the gate/up GEMM (and, with an fp8 forward,
 * the weight encodings) from x and the routing into its workspace, with the
 * same kernels as moe_forward, so the results equal those from a saved
 * buffer bit for bit; the workspace must then hold
 * moe_workspace_bytes(shape, MOE_OP_BACKWARD_RECOMPUTE) bytes. */
moe_status moe_backward(const moe_shape* shape, const void* dout, const void* x,
                        const moe_routing* routing, const void* w_gate_up,
                        const void* w_down, const void* saved, void* dx,
                        void* dw_gate_up, void* dw_down, float* d_topk_w,
                        void* dlogits, void* workspace, size_t workspace_bytes,
                        void* stream);

/* Dispatch alone ("token sorting": "Prime Mega MoE Trains Giant AI Models
 * 55% Faster", section "Where MoE training loses time"): xp[r] =
 * x[src_of[r] / k], xp [T*k, d] (dtype), rows in expert order; reads
 * routing->src_of and routing->row_of (as moe_route wrote them: each token's
 * row is copied to its k expert-sorted rows).  x and xp 16-byte aligned. */
moe_status moe_permute(const moe_shape* shape, const void* x,
                       const moe_routing* routing, void* xp, void* stream);

/* Combine alone (outputs returned to their original positions: "Prime Mega
 * MoE Trains Giant AI Models 55% Faster", section "Where MoE training loses
 * time"; the weighted sum of a token's expert outputs: "Prime Intellect
 * Fused MoE Kernel: 3.11x MoE Training Speed", section "What a
 * mixture-of-experts layer actually does"): out[t] = sum_j topk_w[t][j] *
 * rows[row_of[t*k+j]], summed in float32 in slot order; rows [T*k, d], out
 * [T,d] (dtype); reads routing->row_of and topk_w.  rows and out 16-byte
 * aligned. */
moe_status moe_combine(const moe_shape* shape, const void* rows,
                       const moe_routing* routing, void* out, void* stream);

/* Block quantisation to OCP e4m3 with fp32 scales, the operand encoding of
 * MOE_PREC_FP8_BLOCK ("Prime Mega MoE Trains Giant AI Models 55% Faster",
 * section "Precision and hardware support": one scale per block of values).
 * For a block with largest magnitude amax the scale is s = amax / 448 (1 for
 * an all-zero block) and each value x becomes the code of the e4m3 number
 * nearest to the float32 quotient x / s (ties to even, saturating at 448);
 * x is then represented as decode(code) * s.  src is bf16, q holds the
 * 8-bit codes, s the float32 scales (device pointers; src and q 16-byte
 * aligned).  Kinds:
 *   MOE_QUANT_ROWS:     src [n0, n1], 1 x 128 blocks along rows
 *                       -> q [n0, n1], s [n0, n1/128]; n1 % 128 == 0;
 *   MOE_QUANT_WEIGHT:   src [n0, n1, n2], 128 x 128 blocks of each [n1, n2]
 *                       matrix -> q [n0, n1, n2], s [n0, n1/128, n2/128];
 *   MOE_QUANT_WEIGHT_T: the same blocks written transposed
 *                       -> q [n0, n2, n1], s [n0, n2/128, n1/128].
 * n2 is ignored for MOE_QUANT_ROWS. */
typedef enum { MOE_QUANT_ROWS = 0, MOE_QUANT_WEIGHT = 1, MOE_QUANT_WEIGHT_T = 2 } moe_quant_kind;
moe_status moe_quantize_fp8(int kind, const void* src, int64_t n0, int64_t n1, int64_t n2,
                            uint8_t* q, float* s, void* stream);

/* Token-block quantisation of a weight-gradient operand (same encoding):
 * blocks are runs of 128 consecutive expert-sorted rows of one expert's
 * segment (counted from the expert's first row, the last run short) by one
 * column.  Row r of the operand is src[src_of[r] / k] when gather != 0 (src
 * [T, C], token rows) and src[r] otherwise (src [T*k, C], expert order).
 * Output transposed and padded: with nblk = ceil(T*k / 128) + E and
 * blk_off[e] = sum over e' < e of ceil(counts[e'] / 128), run i of expert e
 * is block b = blk_off[e] + i, q [C, 128 nblk] holds its codes at
 * q[c][128 b + j] (zero past the segment) and s [C, nblk] its scales at
 * s[c][b]; blocks b >= blk_off[E] are not written.  shape->dtype must be
 * MOE_BF16, C a multiple of 128; routing->offsets (and src_of when
 * gathering) are read; workspace as for moe_route. */
moe_status moe_quantize_tokens_fp8(const moe_shape* shape, const void* src, int64_t C, int gather,
                                   const moe_routing* routing, uint8_t* q, float* s,
                                   void* workspace, size_t workspace_bytes, void* stream);

/* MXFP8 encoding of MOE_PREC_MXFP8 (OCP microscaling: blocks of 32 values,
 * one E8M0 scale byte per block, e4m3 elements).  For a block with largest
 * magnitude amax the scale is 2^X with X the smallest integer such that
 * amax <= 448 * 2^X (the blockwise scale amax / 448 rounded up to a power of
 * two, so no value saturates), X >= -127, and X = 0 for an all-zero block;
 * the scale byte is X + 127 and each value x becomes the code of the e4m3
 * number nearest to x / 2^X (exact in float32; ties to even).  src is bf16,
 * q the 8-bit codes, s the scale bytes (device pointers; src and q 16-byte
 * aligned, s 4-byte aligned).  Kinds (moe_quant_kind):
 *   MOE_QUANT_ROWS:     src [n0, n1], blocks of 32 along each row
 *                       -> q [n0, n1], s [n0, n1/32]; n1 % 128 == 0;
 *   MOE_QUANT_WEIGHT:   src [n0, n1, n2], blocks of 32 along each row of
 *                       every [n1, n2] matrix (the forward GEMMs' encoding)
 *                       -> q [n0, n1, n2], s [n0, n1, n2/32];
 *   MOE_QUANT_WEIGHT_T: blocks of 32 down each column (the data-gradient
 *                       encoding), written transposed
 *                       -> q [n0, n2, n1], s [n0, n2, n1/32];
 *                       n1, n2 multiples of 128 for both weight kinds. */
moe_status moe_quantize_mxfp8(int kind, const void* src, int64_t n0, int64_t n1, int64_t n2,
                              uint8_t* q, uint8_t* s, void* stream);

/* MXFP8 token-block quantisation of a weight-gradient operand: as
 * moe_quantize_tokens_fp8 (same runs of 128 rows, same q layout), but each
 * run holds four blocks of 32 rows with their own E8M0 scales (a short last
 * run: blocks past the segment are all zero, scale byte 127), and
 * s [C, 4 nblk] bytes holds block m of run b of column c at s[c][4 b + m]. */
moe_status moe_quantize_tokens_mxfp8(const moe_shape* shape, const void* src, int64_t C,
                                     int gather, const moe_routing* routing, uint8_t* q,
                                     uint8_t* s, void* workspace, size_t workspace_bytes,
                                     void* stream);

const char* moe_status_string(moe_status status);
const char* moe_last_error(void);

/* Kernel timing for measurement: between moe_profile_begin and
 * moe_profile_end every kernel the library enqueues carries a start and a
 * stop HIP event on its stream, stamped by the runtime with the kernel's
 * own start and end (hipExtLaunchKernel), so timing adds no packets between
 * kernels.  moe_profile_end waits for those events and returns, per kernel
 * name, the number of launches and their summed duration. */
typedef struct {
  char name[48];
  int64_t launches;
  double total_ms;
} moe_kernel_stat;

moe_status moe_profile_begin(void);
moe_status moe_profile_end(moe_kernel_stat* stats, int capacity, int* count);

#ifdef __cplusplus
}
#endif

#endif /* MOE_MI355X_H */
