/*
 * moe.h -- C ABI of the fused, dropless mixture-of-experts expert layer for
 * training on one MI355X (gfx950).
 *
 * The layer (one GPU's share of the work):
 *   forward : top-k routing -> permute token rows into expert-contiguous order
 *             -> grouped GEMM with W1/W3 and a SwiGLU epilogue -> grouped GEMM
 *             with W2 -> gate-weighted combine back to token order;
 *   backward: combine-backward -> SwiGLU derivative -> grouped dgrad/wgrad
 *             GEMMs of the three expert matrices -> routing-weight gradient.
 * Sources: Prime Mega MoE news page, "How does the fused kernel work?" (one
 * call fusing dispatch, the two expert linear layers, SwiGLU and combine;
 * GPU-only scratch buffers instead of intermediate tensors; BF16/MXFP8 and an
 * fp8_bwd mode, BF16 forward with FP8 backward); TE dropless-MoE page,
 * "03 Specialised optimisations" and "Optimisation 1: Grouped GEMM" (no
 * token dropping or padding; grouped GEMM over the actual per-expert counts,
 * which stay on the device so that nothing waits on a device-to-host copy);
 * neurobober digest, "Overlapping Backward Pass" (activation gradients need
 * the expert weights, not the weight gradients).
 *
 * Conventions shared by every call
 *   - Every pointer argument named as "device" is a device pointer; dims and
 *     routing structs are host pointers read during the call only.
 *   - The caller owns all memory.  The library allocates nothing and keeps no
 *     global state, apart from the static routing scratch of
 *     moe_route_noalloc; calls with distinct workspaces may run concurrently.
 *   - Every call only enqueues work on `stream` (no host synchronisation, no
 *     device-to-host copy), so a call may be captured in a HIP graph.
 *   - Validation happens on the host before any launch: every status other
 *     than MOE_OK and MOE_ERR_LAUNCH means nothing was enqueued.
 *   - MOE_ERR_LAUNCH is the failure of one of the call's own kernel launches
 *     (the status hipLaunchKernel returned for it; an error left behind by an
 *     earlier, unrelated HIP call is neither reported nor cleared).  A call
 *     launches its kernels in order and stops at the first failure, so the
 *     kernels before it may already be enqueued: the outputs are then
 *     undefined, and the workspace and `saved` contents too.
 *   - Device pointers must be 256-byte aligned; buffers may not alias.
 *   - Results are deterministic: bitwise identical for identical inputs.
 *
 * Shapes: T tokens, H hidden, I expert intermediate, E experts, k experts per
 * token, M = T*k routed rows.  Activations and weights are row-major:
 *   x, dy, y, dx [T,H];  w13 [E,2I,H] (rows [0,I) = W1, [I,2I) = W3);
 *   w2 [E,H,I];  logits [T,E] fp32;  dw13 [E,2I,H] fp32;  dw2 [E,H,I] fp32.
 * Element type of x/dy/y/dx/w13/w2: fp32 in MOE_MODE_FP32, bf16 (raw 16-bit
 * patterns) otherwise.  Gates, gate/logit gradients and weight gradients are
 * always fp32.  Current limits: H and I multiples of 64 (H a multiple of 128
 * in MOE_MODE_FP8_BWD, H and I multiples of 128 in MOE_MODE_MXFP8), E <= 512,
 * k <= 32, and every activation-sized buffer below 2 GiB (the kernels address
 * each operand through 32-bit byte offsets; e.g. T = 32768 at H = 4096 needs
 * M*H*2 = 2 GiB for the permuted rows and is rejected): MOE_ERR_UNSUPPORTED
 * otherwise.
 */
#ifndef MOE_H_
#define MOE_H_

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  MOE_MODE_FP32 = 0,     /* fp32 activations/weights (debug and tiny shapes) */
  MOE_MODE_BF16 = 1,     /* bf16 storage, fp32 accumulation, MFMA GEMMs */
  MOE_MODE_MXFP8 = 2,    /* MXFP8 forward GEMMs and the fp8_bwd backward (see moe_forward) */
  MOE_MODE_FP8_BWD = 3   /* bf16 forward, MXFP8 backward GEMMs (see moe_backward) */
} moe_mode;

typedef enum {
  MOE_OK = 0,
  MOE_ERR_NULL = 1,         /* a required pointer is NULL */
  MOE_ERR_DIMS = 2,         /* a dimension <= 0, k > E, or sizes overflow */
  MOE_ERR_UNSUPPORTED = 3,  /* valid but outside this build's limits (mode, H/I % 64, E, k) */
  MOE_ERR_ALIGN = 4,        /* a device pointer is not 256-byte aligned */
  MOE_ERR_WORKSPACE = 5,    /* workspace smaller than moe_workspace_size reports */
  MOE_ERR_LAUNCH = 6        /* a kernel launch of the call failed; earlier kernels may be enqueued */
} moe_status;

typedef struct {
  int32_t T, H, I, E, k;
  int32_t mode;             /* a moe_mode value */
} moe_dims;

/* Routing state produced by moe_route and consumed by forward/backward.  All
 * members are device pointers owned by the caller. */
typedef struct {
  int32_t* topk_idx;        /* [T,k] expert of slot j of token t (slot 0 = largest logit) */
  float* gate;              /* [T,k] renormalised softmax over the k selected logits */
  int32_t* counts;          /* [E]   rows routed to each expert */
  int32_t* offsets;         /* [E+1] exclusive prefix sum of counts; offsets[E] = M */
  int32_t* sorted_to_flat;  /* [M]   row r of the expert-sorted order -> flat slot t*k+j */
  int32_t* flat_to_sorted;  /* [M]   inverse permutation */
} moe_routing;

/* Sizes in bytes of the buffers the caller provides (host-only, pure).
 *   route_ws : workspace of moe_route
 *   saved    : state written by moe_forward and read by moe_backward
 *   fwd_ws   : workspace of moe_forward
 *   bwd_ws   : workspace of moe_backward
 * Any output pointer may be NULL. */
moe_status moe_workspace_size(const moe_dims* dims, size_t* route_ws, size_t* saved,
                              size_t* fwd_ws, size_t* bwd_ws);

/* Top-k routing (TE dropless-MoE page, "01": the router sends each token to a
 * few experts; Prime Mega MoE news page, "Short": top-8 of 128).
 * For each token the k largest logits are chosen, ordered by (-logit, expert
 * id) so that ties go to the smaller id; gate = softmax over the k selected
 * logits.  counts/offsets/maps describe the stable sort of the flat slots by
 * expert (rows of one expert are in ascending token order).  Bit-exact and
 * deterministic.  logits: device [T,E] fp32, finite values. */
moe_status moe_route(const moe_dims* dims, const float* logits, const moe_routing* out,
                     void* ws, size_t ws_bytes, hipStream_t stream);

/* moe_route without a workspace argument, for callers that cannot allocate
 * device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc).  Same results, bit for bit, and the same
 * arguments otherwise.  The per-block expert partials and bases live in a
 * static device array of MOE_ROUTE_NOALLOC_MAX_BYTES that the library holds
 * on every GPU it runs on until the process ends (its address is looked up
 * on the first call on each device); the call allocates nothing.  Shapes
 * whose routing workspace (moe_workspace_size's route_ws, 2 * ceil(T*k /
 * 4096) * E * 4 bytes rounded up to 256) exceeds it return MOE_ERR_WORKSPACE.
 * Every call on one GPU shares that GPU's array: calls that overlap on one
 * GPU (other streams, other host threads) race and must be serialised by the
 * caller.  Nothing in the array needs clearing: each call writes every entry
 * it reads. */
#define MOE_ROUTE_NOALLOC_MAX_BYTES ((size_t)2 << 20)
moe_status moe_route_noalloc(const moe_dims* dims, const float* logits, const moe_routing* out,
                             hipStream_t stream);

/* Router projection, then moe_route (TE dropless-MoE page, "01 Why is MoE
 * training harder than dense training?": the router is a trained component):
 *   logits[t,e] = <x[t], w_router[e]>   (bf16 inputs, fp32 accumulation)
 * x: device [T,H] bf16; w_router: device [E,H] bf16; logits: device [T,E]
 * fp32, written (the top-k and gates are taken from these values exactly as
 * moe_route takes its input).  Modes with bf16 activations only
 * (MOE_ERR_UNSUPPORTED in MOE_MODE_FP32).  ws as for moe_route. */
moe_status moe_route_project(const moe_dims* dims, const void* x, const void* w_router, float* logits,
                             const moe_routing* out, void* ws, size_t ws_bytes, hipStream_t stream);

/* Backward of the router projection, after moe_backward produced dlogits and
 * dx:
 *   dx[t]      += sum_j dlogits[t, idx_j] w_router[idx_j]   (fp32 on top of
 *                 dx's bf16 value, rounded once; dlogits is zero off the
 *                 top-k set, so this is dlogits w_router)
 *   dw_router[e] = sum over the rows r of expert e, in a fixed order, of
 *                 dlogits[t(r), e] x[t(r)]                   (fp32, written)
 * dlogits: device [T,E] fp32 (moe_backward's); x, w_router as for
 * moe_route_project; dx: device [T,H] bf16, read and written; dw_router:
 * device [E,H] fp32.  No workspace.  MOE_ERR_UNSUPPORTED in MOE_MODE_FP32. */
moe_status moe_router_backward(const moe_dims* dims, const moe_routing* routing, const float* dlogits,
                               const void* x, const void* w_router, void* dx, float* dw_router,
                               hipStream_t stream);

/* Forward pass (Prime Mega MoE news page, "How does the fused kernel work?").
 *   G13[r] = x[t(r)] W13[e]^T,  A = SiLU(G1) * G3,  O = A W2[e]^T   (per expert e)
 *   y[t]   = sum_j gate[t,j] * O[flat_to_sorted[t*k+j]]               (fp32 sum in slot order)
 * x, w13, w2: device inputs; y: device output [T,H]; saved: device buffer of
 * the size reported (G13 of every routed row; in MOE_MODE_MXFP8 also the
 * backward's weight codes), to be passed unchanged to moe_backward.
 *
 * MOE_MODE_MXFP8 (Prime Mega MoE news page, "How does the fused kernel
 * work?": BF16 and MXFP8 precisions): both GEMMs read their operands as
 * MXFP8 quantised along K as moe_mxfp8_quantize describes (x and W13 along H,
 * A and W2 along I; A is quantised from its fp32 value inside GEMM W13);
 * SwiGLU, the combine and y stay as above.  Its backward is the
 * MOE_MODE_FP8_BWD backward.  Each weight is read once and quantised both
 * ways: the forward's row-wise copy, and the transposed copy of the backward
 * (W13 along 2I, W2 along H), which goes into `saved`; in this mode
 * moe_backward takes its weight operands from `saved` and reads w13/w2 only
 * through it, so the weights must not change between the two calls.
 *
 * saved may be NULL: the forward then keeps no state for a backward (G13 is
 * not stored; in MOE_MODE_MXFP8 the weights are quantised only along their
 * rows, for the forward's own GEMMs) and y is the same, bit for bit.  This is
 * the first forward of activation checkpointing, whose backward follows a
 * moe_forward_recompute. */
moe_status moe_forward(const moe_dims* dims, const void* x, const void* w13, const void* w2,
                       const moe_routing* routing, void* y, void* saved,
                       void* ws, size_t ws_bytes, hipStream_t stream);

/* The second forward of activation checkpointing (Prime Mega MoE news page,
 * "How fast is Prime Mega MoE?": the training runs use full activation
 * checkpointing, and the full-layer timing counts the forward twice).  Writes
 * `saved` exactly as moe_forward does (bit for bit, for a moe_backward that
 * follows) but no y: GEMM W2 and the combine, which only produce y, are
 * skipped (in MOE_MODE_MXFP8, W2 is still quantised, since `saved` holds its
 * transposed copy for the backward).  Arguments, sizes and errors as for
 * moe_forward without y; routing must be the one the first forward used. */
moe_status moe_forward_recompute(const moe_dims* dims, const void* x, const void* w13, const void* w2,
                                 const moe_routing* routing, void* saved,
                                 void* ws, size_t ws_bytes, hipStream_t stream);

/* Backward pass of <dy, y> (neurobober digest, "Overlapping Backward Pass":
 * the activation-gradient chain needs only the weights; the weight gradients
 * are independent of it).
 *   dA'  = dy[t(r)] W2[e];  dgate[t,j] = <dA'_r, A_r>;  dA = gate * dA'
 *   dG1  = dA * G3 * s * (1 + G1 (1 - s)),  dG3 = dA * SiLU(G1),  s = sigmoid(G1)
 *   dx[t] = sum_j (dG13 W13[e])[row of slot j]       (fp32 sum in slot order)
 *   dw2[e]  = sum_r dy[t(r)]^T (gate_r A_r)          (fp32 accumulate and output)
 *   dw13[e] = sum_r dG13_r^T x[t(r)]                 (fp32; zero for an empty expert)
 *     (an expert with more than moe_wgrad_chunk_rows() rows, 8192, sums these
 *     over chunks of that many rows, each accumulated in fp32, then added in
 *     chunk order: deterministic)
 *   dlogits[t,e] = gate_e (dgate_e - sum_j gate_j dgate_j) on the top-k set, else 0
 * dy, x, w13, w2: device inputs; saved: from moe_forward; dx: device [T,H];
 * dw13, dw2: device fp32, overwritten; dgate: device [T,k] fp32; dlogits:
 * device [T,E] fp32 or NULL to skip.
 *
 * MOE_MODE_FP8_BWD (Prime Mega MoE news page, "How does the fused kernel
 * work?": BF16 forward with FP8 backward; TE dropless-MoE page, "03
 * Specialised optimisations": group-aware MXFP8 quantisation and MXFP8
 * grouped GEMM): the four GEMMs above read both operands as MXFP8, each
 * quantised along that GEMM's reduction dimension as moe_mxfp8_quantize
 * describes: dy and W2 along H, dG13 and W13 along 2I, and for the weight
 * gradients dy, gate*A, dG13 and x along the tokens of each expert in blocks
 * that start at the expert's first row (moe_mxfp8_quantize_grouped).  dG13
 * and gate*A are quantised in fp32, inside the dgrad of W2 that produces
 * them (in this mode the forward saves G13 in fp32); dgate, the SwiGLU
 * derivative and the router gradient use the unquantised forward state. */
moe_status moe_backward(const moe_dims* dims, const void* dy, const void* x, const void* w13,
                        const void* w2, const moe_routing* routing, const void* saved,
                        void* dx, float* dw13, float* dw2, float* dgate, float* dlogits,
                        void* ws, size_t ws_bytes, hipStream_t stream);

/* moe_backward, except that the weight gradients are added to what dw13 and
 * dw2 hold (an fp32 main-gradient buffer accumulated over micro-batches):
 * dw[e] = ((dw_in[e] + chunk 0) + chunk 1) + ... in fp32, deterministic; an
 * empty expert leaves its entries unchanged.  All other outputs as in
 * moe_backward.  dw13, dw2: device fp32, read and written.  For training
 * loops that keep fp32 gradients across micro-batches (the weight gradients
 * are the backward's independent half: neurobober digest, "Overlapping
 * Backward Pass"). */
moe_status moe_backward_accumulate(const moe_dims* dims, const void* dy, const void* x, const void* w13,
                                   const void* w2, const moe_routing* routing, const void* saved,
                                   void* dx, float* dw13, float* dw2, float* dgate, float* dlogits,
                                   void* ws, size_t ws_bytes, hipStream_t stream);

/* Cached MXFP8 weights, for the two fp8 modes (Prime Mega MoE news page,
 * "How does the fused kernel work?": MXFP8 and fp8_bwd precisions; the
 * weights change once per optimizer step, while a training step runs the
 * forward twice under activation checkpointing and every micro-batch reuses
 * them, so their MXFP8 copies can be made once and kept by the caller).
 *   moe_weight_codes_size: bytes of the copies the mode uses (host-only):
 *     MOE_MODE_MXFP8: W13 along H and W2 along I (the forward's operands) and
 *       W13^T along 2I and W2^T along H (the backward's);
 *     MOE_MODE_FP8_BWD: W13^T and W2^T.
 *     Codes then scales per copy, each as moe_mxfp8_quantize writes them
 *     (along = 1 for the row-wise copies of the [E*2I, H] and [E*H, I]
 *     weights, along = 0 per expert for the transposed ones), each 256-byte
 *     aligned, in the order listed.  MOE_ERR_UNSUPPORTED in the other modes.
 *   moe_quantize_weights: writes them from w13, w2 (device bf16, as for
 *     moe_forward; each weight read once); codes: device buffer of at least
 *     that size (MOE_ERR_WORKSPACE otherwise), owned by the caller.
 *   moe_forward_cached / moe_backward_cached: moe_forward / moe_backward with
 *     the weight operands of the MXFP8 GEMMs taken from `codes` instead of
 *     quantised in the call.  Results are bit for bit those of moe_forward /
 *     moe_backward on the weights the codes were made from.  w13, w2: the
 *     bf16 weights, read by the bf16 forward GEMMs of MOE_MODE_FP8_BWD (in
 *     MOE_MODE_MXFP8 they are not read); the backward reads no bf16 weight.
 *     In MOE_MODE_MXFP8 the `saved` of moe_forward_cached holds G13 only, so
 *     its backward must be moe_backward_cached with the same codes.  Other
 *     arguments, sizes and errors as for moe_forward / moe_backward. */
moe_status moe_weight_codes_size(const moe_dims* dims, size_t* bytes);
moe_status moe_quantize_weights(const moe_dims* dims, const void* w13, const void* w2, void* codes, size_t bytes,
                                hipStream_t stream);
moe_status moe_forward_cached(const moe_dims* dims, const void* x, const void* w13, const void* w2,
                              const void* codes, const moe_routing* routing, void* y, void* saved, void* ws,
                              size_t ws_bytes, hipStream_t stream);
moe_status moe_backward_cached(const moe_dims* dims, const void* dy, const void* x, const void* codes,
                               const moe_routing* routing, const void* saved, void* dx, float* dw13, float* dw2,
                               float* dgate, float* dlogits, void* ws, size_t ws_bytes, hipStream_t stream);

/* Benchmarking variants of moe_forward / moe_backward: the same work, and in
 * addition events[0] is recorded on `stream` before the first kernel and
 * events[i+1] after kernel i, so that hipEventElapsedTime(events[i],
 * events[i+1]) is the duration of kernel i.  `events` is a host array of
 * n_events >= moe_num_kernels(...) + 1 events created by the caller
 * (MOE_ERR_NULL / MOE_ERR_DIMS otherwise).  Kernel order:
 *   forward : tile table, GEMM W13 + SwiGLU, GEMM W2, combine
 *   forward, MOE_MODE_MXFP8: tile table, quantise x, quantise W13, GEMM W13 +
 *             SwiGLU + quantise A, quantise W2, GEMM W2, combine
 *   backward: tile table, dgrad W2 + SwiGLU derivative, dgrad W13,
 *             unpermute-reduce, router backward, wgrad W2, wgrad W13, and
 *             (all modes but MOE_MODE_FP32) the split-K completion of the
 *             weight gradients
 *   backward, MOE_MODE_FP8_BWD: tile table, padded expert offsets,
 *             quantise W2^T, quantise dy, dgrad W2 + SwiGLU derivative +
 *             quantise dG13 and gate*A, quantise W13^T, dgrad W13,
 *             unpermute-reduce, router backward, quantise dy^T, wgrad W2,
 *             quantise x^T, wgrad W13, split-K completion
 *   backward, MOE_MODE_MXFP8: the same without quantise W2^T and quantise
 *             W13^T (their codes come from `saved`)
 *   forward, MOE_MODE_MXFP8, "quantise W13" / "quantise W2" write both
 *             copies of the weight */
moe_status moe_forward_timed(const moe_dims* dims, const void* x, const void* w13, const void* w2,
                             const moe_routing* routing, void* y, void* saved, void* ws, size_t ws_bytes,
                             hipStream_t stream, hipEvent_t* events, int n_events);
moe_status moe_backward_timed(const moe_dims* dims, const void* dy, const void* x, const void* w13,
                              const void* w2, const moe_routing* routing, const void* saved, void* dx,
                              float* dw13, float* dw2, float* dgate, float* dlogits, void* ws, size_t ws_bytes,
                              hipStream_t stream, hipEvent_t* events, int n_events);

/* Number of kernels a call with these dims launches: which = 0 route,
 * 1 forward, 2 backward (-1 for any other value or invalid dims).  Host-only. */
int moe_num_kernels(const moe_dims* dims, int which);

/* MXFP8 quantisation of a bf16 matrix (OCP microscaling format as the TE
 * dropless-MoE page, "03 Specialised optimisations", applies it: E4M3FN
 * elements with one E8M0 scale per 32 consecutive elements along the GEMM's
 * reduction dimension).  For a block with largest magnitude amax:
 *   X     = the smallest integer with amax <= 448 * 2^X, clamped to [-127, 127]
 *           (-127 for an all-zero block); scale byte = X + 127;
 *   codes = v / 2^X rounded to the nearest E4M3FN value, ties to the even
 *           code, magnitudes above 448 saturate to 448; the sign bit of v is
 *           kept, also when the value rounds to zero.
 * src: device bf16 [rows, cols] row-major.
 *   along = 1: blocks of 32 along each row (cols % 32 == 0):
 *              codes [rows, cols], scales [rows, cols/32];
 *   along = 0: blocks of 32 down each column (rows % 128 == 0), written
 *              transposed: codes [cols, rows], scales [cols, rows/32].
 * codes, scales: device outputs (bytes), 256-byte aligned.  Deterministic;
 * the codes are those of the exact definition for the given bf16 values. */
moe_status moe_mxfp8_quantize(const void* src, int32_t rows, int32_t cols, int32_t along, uint8_t* codes,
                              uint8_t* scales, hipStream_t stream);

/* Group-aware MXFP8 quantisation along the rows of expert-sorted data (TE
 * dropless-MoE page, "03 Specialised optimisations"): src: device bf16
 * [rows, cols] whose rows offsets[e] .. offsets[e+1]-1 belong to expert e
 * (offsets: device int32 [E+1], offsets[0] = 0, offsets[E] = rows).  Blocks
 * of 32 rows start at each expert's first row; an expert's last block is
 * zero-padded.  Output, transposed and padded: expert e's rows occupy
 * columns pad_off[e] .. of codes [cols, capacity] and scales
 * [cols, capacity/32], pad_off[e] = sum over e' < e of the counts rounded up
 * to 128 (pad_off: device int32 [E+1], written); columns from
 * pad_off[e] + count_e up to pad_off[e+1] hold zero codes.  capacity must be
 * a multiple of 128 and at least moe_mxfp8_grouped_capacity(rows, E). */
moe_status moe_mxfp8_quantize_grouped(const void* src, int32_t rows, int32_t cols, const int32_t* offsets,
                                      int32_t E, int32_t capacity, int32_t* pad_off, uint8_t* codes,
                                      uint8_t* scales, hipStream_t stream);
size_t moe_mxfp8_grouped_capacity(int32_t rows, int32_t E);

/* Rows per weight-gradient chunk.  An expert with more routed rows has its
 * weight gradients computed in chunks of this many rows (split along K) whose
 * fp32 partial sums are added in chunk order (so such an expert's dW differs
 * from a single-pass sum by fp32 rounding only).  A constant of the library
 * build; no GPU needed. */
int32_t moe_wgrad_chunk_rows(void);

/* Static, human-readable name of a status code. */
const char* moe_status_str(moe_status status);

#ifdef __cplusplus
}
#endif

#endif /* MOE_H_ */
