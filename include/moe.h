/*
 * moe.h -- C ABI of libmoe: the sparse Mixture-of-Experts feed-forward layer
 * on one AMD MI355X (gfx950) GPU.
 *
 * The layer (Qwen3.8-Flash-Next anatomy page on frontier-model-atlas,
 * "Decoder microscope", Feed-forward panel; "Expert fan-out"):
 *   router logits -> softmax -> top-k routed experts -> normalisation of the
 *   selected weights; one shared expert computed alongside the routed path
 *   and scaled by its own sigmoid gate.  Every expert, routed or shared, is a
 *   gated MLP with SiLU (llm-architectures-explained "Qwen3.8-Flash-Next",
 *   "Every architecture field", ffns.moe.gated; llm-atlas
 *   "Qwen3.8-Flash-Next", "Raw config fields", hidden_act).
 *
 * For token x_t (length d):
 *   l[t,e]   = x_t . W_r[e] + b[e]                  (binary32, fixed order*)
 *   idx[t,:] = the k largest l[t,.], descending; equal logits -> lower e
 *   w[t,j]   = softmax(l[t,.])[idx_j] / sum_j' softmax(l[t,.])[idx_j']
 *   s[t]     = sigmoid(g . x_t)
 *   E_e(x)   = W_dn[e] (silu(W_g[e] x) * (W_u[e] x))
 *   out[t]   = sum_j w[t,j] E_{idx_j}(x_t) + s[t] E_shared(x_t)
 * (*) the router logit is accumulated in binary32 in one fixed order: 64
 * partial sums; element kk feeds partial (kk mod 512) div 8; each partial
 * takes its elements in ascending kk with a fused multiply-add starting at
 * +0; the partials are then combined by acc[j] += acc[j+s] for
 * s = 32,16,8,4,2,1; the bias is added last.  This makes topk_idx
 * reproducible bit for bit.
 *
 * Conventions for every entry point:
 *   - Pointers are DEVICE pointers owned by the caller (e.g. allocated by
 *     PyTorch).  The library allocates no device memory and keeps no state
 *     between calls; work is enqueued on `stream` (a hipStream_t, NULL = the
 *     default stream) and returns before it completes.
 *   - Arrays are dense, row-major and 16-byte aligned.  Weights and x are in
 *     desc->dtype (MOE_BF16: bfloat16; MOE_F32: binary32).  out, topk_w,
 *     router bias and the shared-gate output are binary32; topk_idx is int32.
 *   - Layouts: x [T,d]; w_router [E,d]; router_bias [E] (NULL = zeros);
 *     w_gate_up [E,2F,d], rows 0..F-1 the gate projection (SiLU side), rows
 *     F..2F-1 the up projection; w_down [E,d,F]; w_sh_gate_up [2Fs,d];
 *     w_sh_down [d,Fs]; sh_gate [d]; out [T,d]; topk_idx/topk_w [T,k].
 *   - Argument errors are reported before any GPU work is enqueued.  T == 0
 *     is a no-op that returns MOE_OK once desc is valid (pointers unread).
 *     A failed launch returns MOE_ERR_HIP; a fault inside a kernel surfaces
 *     at the caller's next synchronisation.
 *   - out is combined without atomics in a fixed order, so results are
 *     deterministic run to run.
 *   - Calls on one stream are ordered.  Calls that may run concurrently must
 *     use distinct workspaces and outputs.
 */
#ifndef SPARSE_MOE_FEED_AMD_MOE_H
#define SPARSE_MOE_FEED_AMD_MOE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    MOE_OK = 0,
    MOE_ERR_INVALID_ARG = 1,  /* NULL / negative / out-of-range argument, misalignment */
    MOE_ERR_UNSUPPORTED = 2,  /* valid layer the kernels do not handle (see moe_desc) */
    MOE_ERR_WORKSPACE = 3,    /* ws NULL or ws_bytes < moe_workspace_size() */
    MOE_ERR_HIP = 4           /* a HIP launch or runtime call failed */
} moe_status;

typedef enum { MOE_F32 = 0, MOE_BF16 = 1 } moe_dtype;

/* Router algorithm (moe_desc.flags).  Both give the same topk_idx bit for
 * bit (the canonical binary32 logits decide); they differ in cost.
 *   0                        automatic: shortlist for MOE_BF16 with T >= 128
 *   MOE_FLAG_ROUTER_EXACT    canonical logits of every expert (vector ALUs)
 *   MOE_FLAG_ROUTER_SHORTLIST MFMA logits bound the canonical ones; only the
 *                            experts that can still reach the top k are
 *                            recomputed exactly (MOE_BF16 only) */
enum { MOE_FLAG_ROUTER_EXACT = 1, MOE_FLAG_ROUTER_SHORTLIST = 2 };

/* Layer shape.  d_model = d, n_experts = E, top_k = k, d_expert = F,
 * d_shared = Fs (0: no shared expert).
 * Valid: d, E, F >= 1; 1 <= k <= E; Fs >= 0; dtype MOE_F32 or MOE_BF16.
 * Supported: k <= 32; E <= 1024; d <= 16384; for MOE_BF16 additionally
 * d, F and Fs multiples of 64.  Anything valid but outside this returns
 * MOE_ERR_UNSUPPORTED.  flags: 0 or one MOE_FLAG_ROUTER_* value
 * (MOE_FLAG_ROUTER_SHORTLIST with MOE_F32 is unsupported). */
typedef struct {
    int32_t d_model;
    int32_t n_experts;
    int32_t top_k;
    int32_t d_expert;
    int32_t d_shared;
    int32_t dtype; /* moe_dtype */
    int32_t flags; /* MOE_FLAG_ROUTER_* or 0 */
} moe_desc;

/* Bytes of device workspace a call with T tokens needs (0 on an invalid or
 * unsupported desc).  The workspace holds the router logits, the routing
 * histogram and permutation, and the gated-MLP activations h (bf16 for
 * MOE_BF16); it is scratch, its contents are undefined between calls. */
size_t moe_workspace_size(const moe_desc *desc, int64_t T);

/* Byte offsets of the workspace regions, for inspection by tests.  Valid
 * after a call on the same stream has completed (y: moe_forward/moe_experts).
 *   logits   float [T, E+1]   router logits: exact router: canonical logits,
 *                             column E = g . x_t; shortlist router: the
 *                             MFMA logits f (no bias, column E unused) as
 *                             S partial sums [S, T, E+1] over consecutive
 *                             K slices, f = p_0 + p_1 (S = 2) if
 *                             d % 128 == 0, else S = 1
 *   gate     float [T]        s_t = sigmoid(g . x_t)
 *   counts   int32 [E+1]      tokens per expert; counts[E] = T (shared)
 *   offsets  int32 [E+1]      exclusive prefix of counts[0..E-1]
 *   perm     int32 [T*k]      row r of expert e (offsets[e] <= r < offsets[e+1])
 *                             holds the pair id t*k+j; rows of one expert are in
 *                             ascending pair id
 *   Exception: moe_forward / moe_forward_mx4 / moe_forward_prenorm with
 *   T <= 32 on the weight-streaming path and the exact router skip the
 *   permutation: counts[e] = 1 for each selected expert (0 otherwise),
 *   counts[E] = the number of selected experts, offsets and perm are not
 *   written, and the rows of h and y are the pair ids t*k+j.
 *   h        [T*k, F]         gated activations of the routed rows (bf16 / f32)
 *   h_shared [T, Fs]          gated activations of the shared expert
 *   y        [T*k, d]         w[t,j] * expert output of each routed row
 *                             (binary32); the combine adds a token's k rows to
 *                             the shared term in binary32
 *   xnorm    [T, d]           the normalised layer input of moe_forward_prenorm
 *                             (desc->dtype) */
typedef struct {
    size_t logits, gate, counts, offsets, perm, h, h_shared, y, xnorm, total;
} moe_workspace_layout;

moe_status moe_workspace_query(const moe_desc *desc, int64_t T,
                               moe_workspace_layout *layout);

/* Routing only: router logits, softmax, top-k, normalised weights.
 * Writes topk_idx, topk_w and, when sh_gate and sh_gate_out are both
 * non-NULL, sh_gate_out[t] = sigmoid(sh_gate . x_t).  Reads x, w_router,
 * router_bias, sh_gate. */
moe_status moe_route(const moe_desc *desc, int64_t T, const void *x,
                     const void *w_router, const float *router_bias,
                     const void *sh_gate, int32_t *topk_idx, float *topk_w,
                     float *sh_gate_out, void *ws, size_t ws_bytes,
                     void *stream);

/* The whole layer: routing as moe_route, then the routed experts and the
 * shared expert, combined into out (overwritten, binary32).  With
 * d_shared == 0 the shared pointers may be NULL and the shared term is
 * absent.  topk_idx and topk_w are outputs. */
moe_status moe_forward(const moe_desc *desc, int64_t T, const void *x,
                       const void *w_router, const float *router_bias,
                       const void *w_gate_up, const void *w_down,
                       const void *w_sh_gate_up, const void *w_sh_down,
                       const void *sh_gate, float *out, int32_t *topk_idx,
                       float *topk_w, void *ws, size_t ws_bytes, void *stream);

/* The expert stage alone, with the routing given: topk_idx (each entry in
 * [0,E), entries of one row distinct) and topk_w are INPUTS.  out is
 * overwritten.  Indices out of range make the result undefined; the kernels
 * clamp them and never access memory outside the weights. */
moe_status moe_experts(const moe_desc *desc, int64_t T, const void *x,
                       const void *w_gate_up, const void *w_down,
                       const void *w_sh_gate_up, const void *w_sh_down,
                       const void *sh_gate, const int32_t *topk_idx,
                       const float *topk_w, float *out, void *ws,
                       size_t ws_bytes, void *stream);

/* ---------------------------------------------------------------------------
 * Low-bit expert weights (MXFP4).
 *
 * The model's published weights are packed low-bit tensors (llm-atlas
 * "Qwen3.8-Flash-Next", "Modelled costs"; the encoding is not named there).
 * These entry points take the expert weights, routed and shared, in MXFP4 as
 * defined by the OCP Microscaling (MX) specification v1.0: every run of 32
 * consecutive elements of a weight row (along the reduction axis: d for the
 * gate/up matrices, F or Fs for the down matrices) shares one E8M0 scale
 * byte X, worth 2^(X-127); each element is an FP4 E2M1 code (sign bit 3,
 * exponent bits 2..1 with bias 1, mantissa bit 0: magnitudes 0, 0.5, 1, 1.5,
 * 2, 3, 4, 6).  Every element is decoded exactly (to bfloat16) and the layer
 * is then the MOE_BF16 layer on the decoded weights: x, w_router and sh_gate
 * are bfloat16, desc->dtype must be MOE_BF16, and the workspace is
 * moe_workspace_size(desc, T).
 *
 * Row-major MX form of a tensor of logical shape [R, K] (what moe_mx4_pack
 * reads):
 *   codes   uint8 [R, K/2]   element 2i of a row in bits 3..0 of byte i,
 *                            element 2i+1 in bits 7..4
 *   scales  uint8 [R, K/32]  the scale of elements 32b .. 32b+31 of a row
 * Packed form (what the layer reads; R % 16 == 0, K % 128 == 0): tiles of 16
 * rows x 128 elements, 1088 bytes each, tile (b, t) (rows 16b .. 16b+15,
 * elements 128t .. 128t+127) at byte offset (b * K/128 + t) * 1088:
 *   byte 16 (r + 16 c) + j, r < 16, c < 4, j < 16:  codes byte 64 t + 16 c + j
 *                            of row 16 b + r (elements 128 t + 32 c + 2 j and
 *                            + 1)
 *   byte 1024 + r + 16 c:    scales byte 4 t + c of row 16 b + r
 * so R K 17/32 bytes in all.  A tile is exactly what one 64-lane wave reads
 * with one 16-byte load per lane (plus one byte each for the scales), and
 * the tiles of a 16-row block follow each other along K.  The layer's
 * tensors, in this form: w_gate_up [E*2F, d], w_down [E*d, F], w_sh_gate_up
 * [2Fs, d], w_sh_down [d, Fs] (experts stacked along the rows).
 *
 * Supported: d, F and Fs multiples of 128, and T*k*max(d, F) and T*d below
 * 2^32; otherwise MOE_ERR_UNSUPPORTED, before any GPU work.  Up to 16 rows
 * per expert on average (T*k <= 16*E, e.g. decode) the weights are streamed
 * straight into registers; above that a grouped GEMM stages the packed tiles
 * in LDS and decodes them there.  Scale byte 255 (NaN) gives unspecified
 * results.  Errors as for moe_forward.
 * --------------------------------------------------------------------------- */

/* Bytes of the packed form of an [R, K] MXFP4 tensor (0 unless R > 0,
 * K > 0, R % 16 == 0 and K % 128 == 0). */
size_t moe_mx4_packed_bytes(int64_t rows, int64_t K);

/* Packs a row-major MXFP4 tensor [rows, K] (codes 16-byte aligned, scales
 * any alignment) into `packed` (16-byte aligned, moe_mx4_packed_bytes(rows,
 * K) bytes), enqueued on `stream`.  A pure byte permutation, done once per
 * weight tensor.  MOE_ERR_INVALID_ARG for NULL or misaligned pointers, rows
 * or K not positive or not multiples of 16 and 128. */
moe_status moe_mx4_pack(const uint8_t *codes, const uint8_t *scales, int64_t rows,
                        int64_t K, void *packed, void *stream);

/* The whole layer with packed MXFP4 expert weights; as moe_forward
 * otherwise (same arguments, the four expert weight pointers being packed
 * tensors). */
moe_status moe_forward_mx4(const moe_desc *desc, int64_t T, const void *x,
                           const void *w_router, const float *router_bias,
                           const void *w_gate_up, const void *w_down,
                           const void *w_sh_gate_up, const void *w_sh_down,
                           const void *sh_gate, float *out, int32_t *topk_idx,
                           float *topk_w, void *ws, size_t ws_bytes, void *stream);

/* The expert stage alone with packed MXFP4 expert weights and the routing
 * given (topk_idx, topk_w are INPUTS); as moe_experts otherwise. */
moe_status moe_experts_mx4(const moe_desc *desc, int64_t T, const void *x,
                           const void *w_gate_up, const void *w_down,
                           const void *w_sh_gate_up, const void *w_sh_down,
                           const void *sh_gate, const int32_t *topk_idx,
                           const float *topk_w, float *out, void *ws,
                           size_t ws_bytes, void *stream);

/* ---------------------------------------------------------------------------
 * Pre-FFN RMSNorm.
 *
 * The model's norm is RMSNorm with eps 1e-6 (llm-atlas "Qwen3.8-Flash-Next",
 * "Key facts" Norm and "Raw config fields" rms_norm_eps); its placement is
 * not disclosed and is read as the usual pre-norm in front of the layer:
 *   x[t] = h[t] / sqrt(mean_k h[t,k]^2 + eps) * norm_weight
 * The normalised rows decide the integer top-k, so they are computed in one
 * fixed binary32 order: ss = sum_k h_k^2 in the router logit's canonical
 * order (above, no bias); mean = ss / d; v = mean + eps; r = 1 / sqrt(v);
 * x_k = (h_k * r) * norm_weight_k, every step rounded once to nearest; then
 * rounded to desc->dtype (bfloat16: nearest even).  eps is binary32, finite
 * and >= 0 (else MOE_ERR_INVALID_ARG); a zero row with eps = 0 gives NaN.
 * h and norm_weight ([d]) are in desc->dtype.
 * --------------------------------------------------------------------------- */

/* x_out [T, d] = RMSNorm(h) as above (x_out may not alias h). */
moe_status moe_rmsnorm(const moe_desc *desc, int64_t T, const void *h,
                       const void *norm_weight, float eps, void *x_out, void *stream);

/* Expert weight formats of moe_forward_prenorm. */
enum { MOE_WEIGHTS_DTYPE = 0, MOE_WEIGHTS_MX4 = 1 };

/* The layer on the normalised rows: RMSNorm(h) is written to the workspace
 * (region xnorm) and the layer runs on it, with expert weights in
 * desc->dtype (weight_format MOE_WEIGHTS_DTYPE, as moe_forward) or packed
 * MXFP4 (MOE_WEIGHTS_MX4, as moe_forward_mx4, with its limits).  One call;
 * out, topk_idx and topk_w as for moe_forward.
 *
 * resid (nullable, binary32 [T, d], 16-byte aligned, aliasing neither out
 * nor h): the residual stream the layer's output joins.  The model feeds the
 * output into its gated residual streams (frontier-model-atlas anatomy page,
 * "Residual topology", Gated Residual); their gates are the caller's.  With
 * resid given, the combine that finishes out also adds it to the stream in
 * the same pass: resid[t,c] = resid[t,c] + out[t,c], one binary32 rounding
 * (the gate-1 single-stream case; a caller with gates scales out itself).
 * out is written as well. */
moe_status moe_forward_prenorm(const moe_desc *desc, int64_t T, const void *h,
                               const void *norm_weight, float eps, int32_t weight_format,
                               const void *w_router, const float *router_bias,
                               const void *w_gate_up, const void *w_down,
                               const void *w_sh_gate_up, const void *w_sh_down,
                               const void *sh_gate, float *out, int32_t *topk_idx,
                               float *topk_w, float *resid, void *ws, size_t ws_bytes,
                               void *stream);

/* ---------------------------------------------------------------------------
 * Training forward: moe_forward plus the gate/up pre-activations that
 * moe_backward would otherwise recompute (reading every touched expert's
 * gate/up weights again).  `saved` (moe_saved_bytes bytes, 16-byte aligned)
 * receives [a | u] = [W_g x | W_u x] (desc->dtype) of every routed row in
 * the permuted order the routing implies (the rows of expert e, ascending
 * pair id t*k+j, after those of experts < e), each row 2F wide, then the
 * shared expert's [a | u] per token (2Fs wide).  When the layer routes with
 * the shortlist router (bf16 layers of 128 tokens or more, unless a flag
 * picks the exact router), the router logits follow, at the next multiple
 * of 256 bytes: binary32 [S][T][E + 1], S = 2 K-slice partial sums (1 when
 * d % 128 != 0) of x W_r^T (no bias), the shared gate's logit x . g in
 * column E of slice 0 and zeros in the other slices' column E; moe_backward
 * then reads them instead of recomputing them.  With T > 256 the layer's
 * permutation follows, int32, each part at the next multiple of 256 bytes:
 * rank [T k] (the permuted row of pair t*k+j), perm [T k] (the pair of each
 * permuted row) and the rows per expert [E + 1] (the last = T); moe_backward
 * then builds only its tile map.  It stays valid while the routing and x
 * are unchanged.  Everything else as moe_forward.
 * --------------------------------------------------------------------------- */
size_t moe_saved_bytes(const moe_desc *desc, int64_t T);

moe_status moe_forward_train(const moe_desc *desc, int64_t T, const void *x,
                             const void *w_router, const float *router_bias,
                             const void *w_gate_up, const void *w_down,
                             const void *w_sh_gate_up, const void *w_sh_down,
                             const void *sh_gate, float *out, int32_t *topk_idx,
                             float *topk_w, void *saved, size_t saved_bytes, void *ws,
                             size_t ws_bytes, void *stream);

/* ---------------------------------------------------------------------------
 * Backward pass (training).
 *
 * Gradients of  Lambda = sum_t dout[t] . out[t] + L_aux  for the layer of
 * moe_forward with the routing (topk_idx, topk_w) given, as moe_forward
 * returned it.  The top-k selection is piecewise constant and carries no
 * gradient; the router is reached through the normalised weights of the
 * selected experts (w = softmax over the selected logits) and through the
 * router's auxiliary load-balancing loss.  The pages give only that loss's
 * coefficient, 0.001 (llm-atlas "Qwen3.8-Flash-Next", "Raw config fields",
 * router_aux_loss_coef); the loss is read as the usual
 *   L_aux = aux_coef * E * sum_e f_e * P_e,
 *   f_e = (number of (t, j) with topk_idx[t,j] = e) / (T k),
 *   P_e = (1/T) sum_t softmax(l_t)_e   (softmax over all E logits + bias).
 * aux_coef = 0 gives the plain layer gradient.
 *
 * Inputs: the moe_forward operands, topk_idx / topk_w [T,k], dout [T,d]
 * (binary32, the gradient arriving at out), and `saved`: NULL (the gate/up
 * pre-activations, the router logits and the permutation are recomputed) or
 * the buffer moe_forward_train filled for this x and routing (with the same
 * desc).  The entries of one topk_idx row
 * must be distinct experts in [0,E) (else the result is undefined; every
 * access stays in bounds).
 * Outputs (all overwritten, none may alias an input):
 *   dx [T,d] binary32;
 *   dw_router [E,d], dw_gate_up [E,2F,d], dw_down [E,d,F], dw_sh_gate_up
 *   [2Fs,d], dw_sh_down [d,Fs], dsh_gate [d] in desc->dtype (bfloat16 layers
 *   round each gradient once to nearest even); the shared ones only with
 *   d_shared > 0 (else they may be NULL); experts no token chose get zeros;
 *   aux_loss (nullable, device pointer to one float, 4-byte aligned) = L_aux.
 * The router bias gets no gradient (it is an input of the workload, not a
 * weight).  Arithmetic: binary32 accumulation throughout; bfloat16 layers
 * feed the MFMA with bfloat16 operands (dout and the intermediate gradients
 * rounded to bfloat16 once).  T == 0 returns MOE_OK and writes nothing.
 * The workspace (moe_backward_workspace_size bytes) is scratch.
 * --------------------------------------------------------------------------- */
size_t moe_backward_workspace_size(const moe_desc *desc, int64_t T);

moe_status moe_backward(const moe_desc *desc, int64_t T, const void *x,
                        const void *w_router, const float *router_bias,
                        const void *w_gate_up, const void *w_down,
                        const void *w_sh_gate_up, const void *w_sh_down,
                        const void *sh_gate, const int32_t *topk_idx,
                        const float *topk_w, const float *dout, const void *saved,
                        float aux_coef, float *dx, void *dw_router, void *dw_gate_up,
                        void *dw_down, void *dw_sh_gate_up, void *dw_sh_down, void *dsh_gate,
                        float *aux_loss, void *ws, size_t ws_bytes, void *stream);

/* ---------------------------------------------------------------------------
 * For callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc): moe_forward
 * with the workspace taken from a static device array of the library,
 * MOE_NOALLOC_SCRATCH_BYTES (100 MiB) on each GPU it runs on, held until the
 * process ends.  At the pages' shape (d 2560, 512 experts top-10, width 640,
 * shared 640, bf16) that serves up to 1347 tokens per call.  Arguments,
 * outputs and errors as moe_forward, without ws / ws_bytes; a call whose
 * moe_workspace_size exceeds the array returns MOE_ERR_WORKSPACE (and says
 * so in moe_last_error) before any GPU work.  The call allocates nothing: the
 * first call on a GPU only looks up the array's device address there.  All
 * calls on one GPU share its array, so calls that may overlap on one GPU
 * (different streams, or different threads) race: serialise them.
 * --------------------------------------------------------------------------- */
#define MOE_NOALLOC_SCRATCH_BYTES ((size_t)100 << 20)
moe_status moe_forward_noalloc(const moe_desc *desc, int64_t T, const void *x,
                               const void *w_router, const float *router_bias,
                               const void *w_gate_up, const void *w_down,
                               const void *w_sh_gate_up, const void *w_sh_down,
                               const void *sh_gate, float *out, int32_t *topk_idx,
                               float *topk_w, void *stream);

/* ---------------------------------------------------------------------------
 * Measurement aid (not part of the layer): the practical HBM read ceiling.
 * The expert-weight streams of the layer are HBM reads; this reads `bytes`
 * bytes of device memory at `buf` once, with the whole chip, in coalesced
 * 16-byte loads, so its rate is the read bandwidth those streams can reach.
 * sink (device, MOE_READ_PROBE_SINK_WORDS uint32 words, 4-byte aligned) is
 * overwritten with per-wave XOR folds: the XOR of all sink words equals the
 * XOR of every 32-bit word of the buffer (a check that every byte was read).
 * MOE_ERR_INVALID_ARG for NULL pointers, buf not 16-byte aligned or bytes not
 * a multiple of 16; MOE_ERR_HIP if the launch fails.  Enqueued on `stream`.
 * --------------------------------------------------------------------------- */
#define MOE_READ_PROBE_SINK_WORDS 8192
moe_status moe_read_probe(const void *buf, size_t bytes, uint32_t *sink, void *stream);

/* Static, human-readable name of a status code. */
const char *moe_status_string(moe_status status);

/* Text of the last HIP error seen by this thread ("" if none). */
const char *moe_last_error(void);

/* Stage timing for benchmarks and profilers.  The NEXT moe_forward,
 * moe_experts or moe_backward call on this thread records events[i]
 * (hipEvent_t, created by the caller) on its stream at stage boundaries,
 * then forgets the array.  Forward:
 *   0 start; 1 after routing (moe_experts: after the shared gate);
 *   2 after the histogram/permutation; 3 after the gate/up GEMM;
 *   4 after the down GEMM; 5 after the combine.
 * Backward: 0 start; 1 after the permutation and router logits; 2 after the
 *   gate/up recompute and W_dn^T dout; 3 after the SwiGLU and router
 *   backward; 4 after dx of the rows; 5 after dW_gate_up; 6 after dW_down;
 *   7 after the router GEMMs, the dx combine and the loss.
 * n (<= 8) is the number of entries; entries may be NULL.  The events only
 * observe the stream, they change nothing the call computes. */
moe_status moe_stage_events(void *const *events, int n);

#ifdef __cplusplus
}
#endif

#endif /* SPARSE_MOE_FEED_AMD_MOE_H */
