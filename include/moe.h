/*
 * moe.h -- C ABI of a single-GPU (MI355X, gfx950) Mixture-of-Experts layer
 * forward pass: gate -> top-k -> dispatch -> grouped SwiGLU expert FFN ->
 * combine, on one GPU's share of the tokens with every expert local.
 *
 * Sources for what each call computes (the pages the method comes from):
 *  [wmrh]  "DeepSeek 中 MoE 的同步税" (wmrh.cn/news/47329), section 4.1: the
 *          routing code (gate, softmax, top-k, renormalise by the selected
 *          sum); section 4.3: gate/softmax/top-k fused into one kernel that
 *          writes indices and weights; section 5.1: keep the router in
 *          float32; section 2.1: fine-grained routed experts plus shared
 *          experts every token passes through.
 *  [lpnh]  the DeepSeek MoE routing deep dive (lpnh.cn/news/699721), section
 *          2.2: per-token top-k gating kernel over an [N, E] score matrix.
 *  [gsyq]  "Deepseek-MoE同步税本质与四层实战优化指南" (gsyq.cn), section 2.3:
 *          each token's output is the gate-weighted sum of its experts'
 *          outputs; section 3.1: per-token min/max affine FP8 quantiser at the
 *          dispatch entry; section 5.2: that quantiser's per-token,
 *          per-expert and global modes.
 *  [deepep] "MoE数据特征、训练和推理的通信特点 ... DeepEP ... All-to-All"
 *          (zzszmyf.github.io), section 7: dispatch reorders tokens by target
 *          expert and packs them contiguously ([Local_Batch, Hidden] ->
 *          [Num_Experts * Tokens_Per_Expert, Hidden]); the expert stage is a
 *          local FFN; combine restores the original token order from the
 *          metadata saved at dispatch (7.5(2): indices and locations), with no
 *          padding (7.5(4)) and with sizes known before the payload moves.
 *          Its part on DeepSeek-V3's auxiliary-loss-free load balancing
 *          ("A", hard constraint and capacity): a strict per-expert token
 *          cap; once an expert is full, later tokens that picked it are
 *          turned away (reassigned or dropped).
 *
 * Conventions (all entry points):
 *  - Every pointer argument except the moe_shape is a DEVICE pointer unless
 *    stated; the caller allocates and owns every buffer, including the
 *    workspace. The library never allocates, frees or synchronises inside a
 *    compute call; all work is enqueued on `stream` (a hipStream_t; NULL is
 *    the null stream) and the call returns before it runs.
 *  - Arrays are dense row-major. Device pointers must be 16-byte aligned and
 *    the workspace 256-byte aligned.
 *  - Expert weight groups are ordered routed 0..E-1, then shared E..E+S-1.
 *    W1, W3 are [E+S, h, d] and W2 is [E+S, d, h] (each row is one output
 *    feature, nn.Linear layout). The gate weight is [E, d].
 *  - Arguments are validated on the host before anything is enqueued; a bad
 *    argument returns a negative moe_status and leaves the stream untouched.
 *    T = 0 is valid, needs no buffers (they may be NULL) and enqueues nothing.
 *    No C++ exception crosses the ABI.
 *  - Expert ids in topk_idx outside [0, E), or an expert listed twice for one
 *    token, are detected on the device: the offending slots are skipped
 *    (dest_row = -1), no memory outside the buffers is touched, and a sticky
 *    flag in the workspace is set; moe_get_device_error reports it.
 *
 * Shape limits: 1 <= E <= 256, 1 <= k <= min(E, 8), 0 <= S <= 8, T >= 0,
 * T*k < 2^31 and T*S < 2^31, d and h at most 2^20. act = MOE_F32: d % 4 ==
 * 0. act = MOE_BF16: d % 8 == 0 (d % 16 with fp8 rows), so that every row
 * moves as 16-byte pieces; any h >= 1. dispatch must equal act, or be
 * MOE_FP8_E4M3 with act = MOE_BF16. (Shapes with d % 256 == 0 and h % 128
 * == 0 take the persistent large-tile expert GEMMs; the others a 128 x 128
 * tile kernel.)
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
    MOE_ERR_INVALID_ARG = -1, /* null pointer, bad size, misaligned pointer */
    MOE_ERR_UNSUPPORTED = -2, /* a shape or dtype combination outside the limits */
    MOE_ERR_WORKSPACE = -3,   /* workspace missing or smaller than required */
    MOE_ERR_HIP = -4,         /* a HIP runtime call or kernel launch failed */
    MOE_ERR_BAD_INDEX = -5    /* (device flag) bad or repeated expert id seen */
} moe_status;

typedef enum { MOE_F32 = 0, MOE_BF16 = 1, MOE_FP8_E4M3 = 2 } moe_dtype;

/* what happens to an assignment beyond an expert's capacity */
typedef enum { MOE_OVERFLOW_DROP = 0, MOE_OVERFLOW_REASSIGN = 1 } moe_overflow;

/* the rows whose min/max range an fp8 row is mapped from ([gsyq] 5.2: the
 * quantiser's per-token, per-expert and global modes), or the per-token
 * symmetric absmax map: the same affine map over [-max|x|, max|x|], whose
 * centre is 0 */
typedef enum {
    MOE_QUANT_TOKEN = 0,
    MOE_QUANT_EXPERT = 1,
    MOE_QUANT_GLOBAL = 2,
    MOE_QUANT_TOKEN_ABSMAX = 3
} moe_quant;

/* which entry point a workspace is sized for */
typedef enum {
    MOE_STAGE_GATE = 0,
    MOE_STAGE_DISPATCH = 1,
    MOE_STAGE_FFN = 2,
    MOE_STAGE_COMBINE = 3,
    MOE_STAGE_FORWARD = 4,
    MOE_STAGE_GATE_BACKWARD = 5,
    MOE_STAGE_FFN_BACKWARD = 6,
    MOE_STAGE_FORWARD_FP8W = 7
} moe_stage;

typedef struct {
    int64_t T;        /* tokens on this GPU */
    int32_t d;        /* model (hidden) width */
    int32_t E;        /* routed experts */
    int32_t k;        /* routed experts per token */
    int32_t S;        /* shared experts (every token passes through them) */
    int32_t h;        /* expert SwiGLU hidden width */
    int32_t act;      /* moe_dtype of x, all weights, expert outputs and y */
    int32_t dispatch; /* moe_dtype of the dispatched rows x_perm */
    int32_t capacity; /* rows each routed expert may hold ([deepep] V3 "A"):
                         0 = no limit (every assignment dispatched); C > 0 =
                         assignments beyond an expert's first C, in token
                         order, overflow (see moe_dispatch). Negative is
                         invalid. */
    int32_t overflow; /* moe_overflow: overflowing assignments are dropped or
                         reassigned to the least-loaded expert */
    int32_t quant;    /* moe_quant, with dispatch = MOE_FP8_E4M3 only (else it
                         must be MOE_QUANT_TOKEN) */
} moe_shape;

/* Host only. Bytes of workspace that `stage` needs for shape *s (0 when the
 * stage needs none), or 0 for an invalid shape. */
size_t moe_workspace_bytes(const moe_shape *s, int32_t stage);

/* Clear the workspace header (the error flag and internal counters). Call once
 * after allocating a workspace and before its first use; every call leaves the
 * header in a valid state afterwards. Enqueued on stream. */
int32_t moe_workspace_init(void *ws, size_t ws_bytes, void *stream);

/* Host only. Static text for a moe_status value. */
const char *moe_status_string(int32_t status);

/*
 * Gate + top-k + renormalised weights ([wmrh] 4.1 and 4.3, [lpnh] 2.2).
 *  x [T,d] (act), w_gate [E,d] (act), bias [E] float32 or NULL.
 *  logit[t,e] = sum_i x[t,i]*w_gate[e,i] (+ bias[e]) in float32, summed as one
 *  fused multiply-add chain over i = 0..d-1 from +0.0 ([wmrh] 5.1: float32
 *  router); topk_idx[t,:] (int32 [T,k]) = the k largest logits in descending
 *  order, ties to the lower expert id; topk_w[t,j] (float32 [T,k]) =
 *  softmax over all E renormalised over the selected k (= softmax of the k
 *  selected logits). logits_dbg [T,E] float32 receives the logits if not NULL.
 */
int32_t moe_gate_topk(const moe_shape *s, const void *x, const void *w_gate,
                      const float *bias, int32_t *topk_idx, float *topk_w,
                      float *logits_dbg, void *stream);

/*
 * Dispatch ([deepep] 7 "Dispatch" and 7.5(2)/(4), [gsyq] 3.1 for FP8).
 *  counts[e] (int32 [E]) = number of (t,j) with topk_idx[t,j] == e;
 *  offsets (int32 [E+1]) = exclusive prefix sum (offsets[E] = T*k with no
 *  capacity limit);
 *  dest_row[t,j] (int32 [T,k]) = offsets[e] + number of tokens t' < t that
 *  picked e (stable, expert-major, token order kept, no padding);
 *  src_token[dest_row[t,j]] = t (int32 [T*k]);
 *  With s->capacity = C > 0 ([deepep] V3 "A"): an assignment (t,j) to
 *  expert e keeps its expert iff fewer than C tokens t' < t picked e, and
 *  otherwise overflows. MOE_OVERFLOW_DROP: an overflowing slot gets
 *  dest_row = -1 and no row, and contributes nothing in moe_combine (its
 *  weight is not handed to the other slots); counts[e] = min(C, number
 *  picking e). MOE_OVERFLOW_REASSIGN: after that first pass the overflowing
 *  slots, in token order (t, then j), go one at a time to the expert with
 *  the fewest rows at that moment (ties to the lower id), as its next row,
 *  while some expert holds fewer than C rows; the rest are dropped. A
 *  reassigned slot keeps its gate weight and may land on an expert the
 *  token already picked. An expert's rows are its first-pass rows in token
 *  order, then its reassigned rows in that order; counts are the final rows
 *  per expert. topk_idx is not changed: the expert of a slot's row is the e
 *  with offsets[e] <= dest_row < offsets[e+1]. Only src_token[0 ..
 *  offsets[E]) is written.
 *  x_perm[dest_row[t,j]] = x[t] (rows of act), or, with dispatch =
 *  MOE_FP8_E4M3, the token's per-row affine e4m3 codes (uint8 [T*k, d]) with
 *  qparams[dest_row[t,j]] = (scale, centre) (float32 [T*k, 2]): centre =
 *  (max+min)/2, scale = (max-min)/2/448, code = e4m3 round-to-nearest-even of
 *  clamp((x - centre) * (448 / ((max-min)/2)), +-448), all in float32; a
 *  constant row gets codes 0 and scale 0. With s->quant = MOE_QUANT_EXPERT
 *  ([gsyq] 5.2) max and min are taken over every row dispatched to the
 *  row's expert (its final rows, after any capacity limit), and with
 *  MOE_QUANT_GLOBAL over all T rows of x, and with MOE_QUANT_TOKEN_ABSMAX
 *  they are -max|x[t]| and max|x[t]| (centre 0); the map is otherwise the same, so
 *  each dispatched row still carries its own (scale, centre).
 *  qparams may be NULL otherwise.
 *  ws: MOE_STAGE_DISPATCH bytes.
 */
int32_t moe_dispatch(const moe_shape *s, const void *x, const int32_t *topk_idx,
                     int32_t *counts, int32_t *offsets, int32_t *dest_row,
                     int32_t *src_token, void *x_perm, float *qparams, void *ws,
                     size_t ws_bytes, void *stream);

/*
 * moe_dispatch without a workspace argument, for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc). Same arguments, kernels and results as
 * moe_dispatch; the working arrays live in a 16 MiB device array owned by
 * the library (one per GPU, held until the process ends). The call itself
 * allocates nothing. Limit: the shape's MOE_STAGE_DISPATCH workspace
 * (moe_workspace_bytes) must fit in 16 MiB -- about 4*T*k + 8*E*T/256 bytes,
 * e.g. 2.3 MiB for T = 65536, k = 8, E = 256 -- else MOE_ERR_UNSUPPORTED
 * before anything is enqueued. Every call on a GPU uses that GPU's one array: calls that
 * overlap on one GPU (two streams, or host threads without ordering) race
 * and give undefined results. The array is cleared where the kernels need
 * it on every call; a bad or repeated expert id still gives dest_row = -1
 * and no row, but no error flag is kept for moe_get_device_error. The
 * current device must be the stream's.
 */
int32_t moe_dispatch_noalloc(const moe_shape *s, const void *x, const int32_t *topk_idx,
                             int32_t *counts, int32_t *offsets, int32_t *dest_row,
                             int32_t *src_token, void *x_perm, float *qparams, void *stream);

/*
 * Grouped SwiGLU expert FFN ([deepep] 7 "expert stage", [wmrh] 2.1).
 *  For routed expert e, the rows offsets[e]..offsets[e+1]-1 of x_perm (fp8
 *  rows are first dequantised to code*scale + centre): y_perm[r] =
 *  W2_e (silu(W1_e v) * (W3_e v)), silu(a) = a / (1 + exp(-a)).
 *  For the shared experts (S > 0), every token of x [T,d]:
 *  y_shared[t] = sum_s W2_{E+s} (silu(W1_{E+s} x[t]) * (W3_{E+s} x[t])).
 *  bf16: products in bf16 on the matrix cores with float32 accumulation; the
 *  SwiGLU hidden vector is rounded to bf16 once, each output once.
 *  y_perm [T*k, d] (act), y_shared [T,d] (act; NULL iff S == 0); x may be
 *  NULL iff S == 0; qparams required iff dispatch is fp8.
 *  ws: MOE_STAGE_FFN bytes.
 */
int32_t moe_grouped_ffn(const moe_shape *s, const void *x_perm, const float *qparams,
                        const int32_t *offsets, const void *x, const void *w1,
                        const void *w3, const void *w2, void *y_perm, void *y_shared,
                        void *ws, size_t ws_bytes, void *stream);

/*
 * Combine ([gsyq] 2.3, [deepep] 7 "Combine"): un-permute and weighted sum,
 *  y[t] = y_shared[t] + sum_j topk_w[t,j] * y_perm[dest_row[t,j]], accumulated
 *  in float32 and rounded once to act. y_shared may be NULL (then 0); slots
 *  with dest_row < 0 are skipped.
 */
int32_t moe_combine(const moe_shape *s, const void *y_perm, const void *y_shared,
                    const int32_t *dest_row, const float *topk_w, void *y,
                    void *stream);

/*
 * Backward of combine (the gradients returning along the routing path,
 *  [gsyq] 2.4; [deepep] 7 "Combine", whose transpose this is): for every
 *  slot (t,j) with p = dest_row[t,j] >= 0,
 *    dy_perm[p]    = act(topk_w[t,j] * dy[t])          (rounded once)
 *    dtopk_w[t,j]  = sum_c dy[t,c] * y_perm[p,c]       (float32 accumulation)
 *  and dtopk_w[t,j] = 0 for a dropped slot (no row written).
 *  dy [T,d] (act) is the gradient of the layer output, y_perm [>= max p + 1, d]
 *  (act) the routed experts' forward output rows, dest_row [T,k] and topk_w
 *  [T,k] as from the forward; dy_perm [T*k,d] (act) and dtopk_w [T,k] (f32)
 *  are written. All device pointers, owned by the caller; rows of dy_perm no
 *  slot maps to are left untouched. Errors: MOE_ERR_INVALID_ARG for a bad
 *  shape or a NULL pointer (T = 0 is a no-op), MOE_ERR_HIP for a launch error.
 *  dy_perm must not overlap dy or y_perm.
 */
int32_t moe_combine_backward(const moe_shape *s, const void *dy, const void *y_perm,
                             const int32_t *dest_row, const float *topk_w, void *dy_perm,
                             float *dtopk_w, void *stream);

/*
 * Backward of dispatch ([gsyq] 2.4; [deepep] 7 "Dispatch", whose transpose
 *  this is): dispatch copies token t to its k rows, so its gradient sums them,
 *    dx[t] = dx_shared[t] + sum_{j : dest_row[t,j] >= 0} dx_perm[dest_row[t,j]]
 *  accumulated in float32 in slot order and rounded once to act. dx_perm
 *  [rows,d] (act) holds the routed rows' input gradients, dx_shared [T,d] (act)
 *  the shared experts' (NULL: zero), dest_row [T,k] as from the forward; dx
 *  [T,d] (act) is written. Device pointers owned by the caller; errors as for
 *  moe_combine_backward. The gradient with respect to the gate input is not
 *  part of this call (it is a plain GEMM with the gate weights).
 */
int32_t moe_dispatch_backward(const moe_shape *s, const void *dx_perm, const void *dx_shared,
                              const int32_t *dest_row, void *dx, void *stream);

/*
 * Backward of the gate ([wmrh] 4.1 and [gsyq] 2.1 gate, [gsyq] 2.4 backward)
 *  with each token's top-k choice held fixed. The renormalised weights are a
 *  softmax over the k chosen logits, so for slot j of token t
 *    dlogits_topk[t,j] = w[t,j] (dw[t,j] - sum_l w[t,l] dw[t,l])   (float32)
 *  is the gradient of the logit of expert topk_idx[t,j] (all other logits:
 *  zero; a bias shifts logits by a constant and changes nothing here), with
 *  w = topk_w, dw = dtopk_w (as from moe_combine_backward; 0 on dropped
 *  slots). Through z = x w_gate^T:
 *    dx[t]     = act(dx[t] + sum_j dlogits_topk[t,j] w_gate[topk_idx[t,j]])
 *                (read, float32 sum in slot order, rounded once; NULL: skipped)
 *    dw_gate[e] = sum over slots with topk_idx = e of dlogits_topk[t,j] x[t]
 *                (float32 [E,d], overwritten: summed per range of tokens in
 *                token order, then over the ranges in order; no atomics, so
 *                every call gives the same bits).
 *  ws: MOE_STAGE_GATE_BACKWARD bytes (the per-range partials).
 *  x [T,d] and w_gate [E,d] (act), topk_idx/topk_w/dtopk_w/dlogits_topk
 *  [T,k]; all device pointers owned by the caller, 16-byte aligned. Ids
 *  outside [0,E) contribute nothing. T = 0 only clears dw_gate. Errors:
 *  MOE_ERR_INVALID_ARG (bad shape, NULL or misaligned pointer), MOE_ERR_HIP.
 */
int32_t moe_gate_backward(const moe_shape *s, const void *x, const void *w_gate,
                          const int32_t *topk_idx, const float *topk_w, const float *dtopk_w,
                          float *dlogits_topk, void *dx, float *dw_gate, void *ws,
                          size_t ws_bytes, void *stream);

/*
 * Backward of the grouped SwiGLU expert FFN ([gsyq] 2.4: the gradients go
 *  back along the forward's routing, through the experts' own computation
 *  between the transposes of combine and dispatch). For routed expert e and
 *  each row r of offsets[e]..offsets[e+1]-1 with input v = x_perm[r] (fp8
 *  rows dequantised as in moe_grouped_ffn; the quantiser passes the gradient
 *  straight through) and output gradient g = dy_perm[r] (as written by
 *  moe_combine_backward):
 *    a = W1_e v, b = W3_e v, u = silu(a), hid = u * b  (recomputed, bf16)
 *    dhid = W2_e^T g;  da = dhid * b * s (1 + a (1 - s)), s = sigmoid(a);
 *    db = dhid * u;  dx_perm[r] = W1_e^T da + W3_e^T db     (bf16 [T*k, d])
 *    dW2_e = sum_r g hid^T, dW1_e = sum_r da v^T, dW3_e = sum_r db v^T
 *  The shared experts (S > 0) do the same for every token t with input
 *  x[t] and output gradient dy_shared[t] (the layer output's gradient);
 *  dx_shared[t] (bf16 [T, d]) is the sum over the shared experts.
 *  dw1, dw3 [E+S, h, d] and dw2 [E+S, d, h] are float32 and overwritten
 *  (zero for an expert with no rows); each element is summed over the
 *  group's rows in order by one work-group (no atomics: every call gives
 *  the same bits). moe_dispatch_backward then sums dx_perm and dx_shared
 *  back per token. act must be MOE_BF16 (MOE_ERR_UNSUPPORTED otherwise);
 *  x, dy_shared and dx_shared are required iff S > 0 (else NULL); qparams
 *  iff the rows are fp8. ws: MOE_STAGE_FFN_BACKWARD bytes (the recomputed
 *  a, b, hid and the gradients da, db of every row). T = 0 only zeroes the
 *  weight gradients. Errors as for moe_grouped_ffn.
 */
int32_t moe_grouped_ffn_backward(const moe_shape *s, const void *x_perm, const float *qparams,
                                 const int32_t *offsets, const void *x, const void *w1,
                                 const void *w3, const void *w2, const void *dy_perm,
                                 const void *dy_shared, void *dx_perm, void *dx_shared,
                                 float *dw1, float *dw3, float *dw2, void *ws, size_t ws_bytes,
                                 void *stream);

/*
 * Saving the expert activations for the backward instead of recomputing
 * them (the same quantities as moe_grouped_ffn_backward's recomputation,
 * [gsyq] 2.4; a training caller trades T*(k+S)*3*h*2 bytes of memory for
 * the backward's recomputed up-projection).
 *
 * moe_ffn_saved_bytes: bytes of the buffer that holds them -- a, b and hid,
 *  bf16, for the routed rows [T*k, h] and then the shared experts' token rows
 *  [T, S*h], each section 256-byte aligned -- or 0 when the shape is not
 *  supported: act must be MOE_BF16 and the shape on the persistent tiles
 *  (d % 256 == 0, h % 128 == 0).
 * moe_grouped_ffn_save: moe_grouped_ffn (same arguments, same results, bit
 *  for bit) that also writes a, b and hid of every row into `saved`
 *  (caller-owned, 256-byte aligned, saved_bytes >= moe_ffn_saved_bytes).
 *  MOE_ERR_UNSUPPORTED for shapes moe_ffn_saved_bytes rejects;
 *  MOE_ERR_INVALID_ARG for a missing, misaligned or short `saved`.
 * moe_grouped_ffn_backward_saved: moe_grouped_ffn_backward (same arguments
 *  and results) that reads a, b and hid from `saved`, as written by
 *  moe_grouped_ffn_save on the same rows and weights, instead of recomputing
 *  them; the results are the same bits. Same errors as the two above.
 */
size_t moe_ffn_saved_bytes(const moe_shape *s);
int32_t moe_grouped_ffn_save(const moe_shape *s, const void *x_perm, const float *qparams,
                             const int32_t *offsets, const void *x, const void *w1, const void *w3,
                             const void *w2, void *y_perm, void *y_shared, void *saved,
                             size_t saved_bytes, void *ws, size_t ws_bytes, void *stream);
int32_t moe_grouped_ffn_backward_saved(const moe_shape *s, const void *x_perm,
                                       const float *qparams, const int32_t *offsets,
                                       const void *x, const void *w1, const void *w3,
                                       const void *w2, const void *saved, size_t saved_bytes,
                                       const void *dy_perm, const void *dy_shared, void *dx_perm,
                                       void *dx_shared, float *dw1, float *dw3, float *dw2,
                                       void *ws, size_t ws_bytes, void *stream);

/*
 * The whole layer: moe_gate_topk -> moe_dispatch -> moe_grouped_ffn ->
 * moe_combine with intermediates in the workspace (MOE_STAGE_FORWARD bytes).
 * y [T,d] (act) is the layer output; topk_idx, topk_w, counts, offsets,
 * dest_row and src_token are written as by the stage calls. With bf16 rows
 * on the 256 x 256 tiles (d % 256 == 0, h % 128 == 0) the permuted rows are
 * not written: the up-projection reads routed row r from x[src_token[r]]
 * (same results), and the workspace holds no x_perm.
 */
int32_t moe_forward(const moe_shape *s, const void *x, const void *w_gate,
                    const float *bias, const void *w1, const void *w3, const void *w2,
                    void *y, int32_t *topk_idx, float *topk_w, int32_t *counts,
                    int32_t *offsets, int32_t *dest_row, int32_t *src_token, void *ws,
                    size_t ws_bytes, void *stream);

/*
 * fp8 expert weights ([gsyq] 3.1 and 5.2 quantise the dispatched activations
 * to FP8; the pages leave weight quantisation open). Reading: every weight
 * row -- one output feature of W1, W3 or W2 -- is quantised to e4m3 with the
 * activations' affine map over the symmetric range [-max|w|, max|w|]:
 * centre 0, scale max|w| / 448, code = e4m3 round-to-nearest-even of
 * clamp(w * (448 / max|w|), +-448) in float32 (codes 0 and scale 0 for a zero
 * row). The shared experts' W2 rows are quantised jointly over their S
 * concatenated hidden blocks (one scale per output feature, so that their
 * down-projections still sum in one accumulator).
 *
 * Host only: the float32 count of the scale array wscale for shape *s:
 *   s1 [E+S, h] | qsum1 [E+S, h] | s3 [E+S, h] | qsum3 [E+S, h] | s2 [E+S, d]
 * (s: a row's scale; qsum: the sum of a W1 / W3 row's code values, for the
 * activations' centre term; s2 of the shared experts repeated per expert).
 * 0 for an invalid shape.
 */
size_t moe_fp8_weight_scale_floats(const moe_shape *s);

/*
 * Quantise bf16 expert weights w1, w3 [E+S, h, d] and w2 [E+S, d, h] (act =
 * MOE_BF16, d % 8 == 0, h % 8 == 0) to e4m3 codes w1q, w3q, w2q (uint8, same
 * shapes) and the scales wscale (moe_fp8_weight_scale_floats). Device
 * pointers owned by the caller; errors as for the other calls.
 */
int32_t moe_quantize_weights(const moe_shape *s, const void *w1, const void *w3, const void *w2,
                             uint8_t *w1q, uint8_t *w3q, uint8_t *w2q, float *wscale,
                             void *stream);

/*
 * The whole layer with fp8 expert weights on the fp8 matrix cores: gate and
 * dispatch as in moe_forward (s->dispatch must be MOE_FP8_E4M3, quant
 * MOE_QUANT_TOKEN or MOE_QUANT_TOKEN_ABSMAX, act MOE_BF16); then every
 * expert, routed and shared, computes on the token's fp8 row (so here the
 * shared experts read the quantised rows too):
 *   a = W1q v, b = W3q v (e4m3 x e4m3 products, float32 sums, row and
 *   weight scales and the row's centre applied after the sum),
 *   H = bf16(silu(a) * b), quantised per row with a symmetric absmax e4m3
 *   scale (the shared experts' S blocks of a token together),
 *   Y = W2q H (e4m3 x e4m3, scales after the sum), rounded to bf16,
 * and combine as in moe_forward. w1q, w3q, w2q, wscale from
 * moe_quantize_weights. Shapes: d % 256 == 0 and h % 256 == 0, else
 * MOE_ERR_UNSUPPORTED. ws: MOE_STAGE_FORWARD_FP8W bytes. events (NULL: not
 * traced) as for moe_forward_traced with at least 10 entries, recorded before
 * the first kernel and after gate_topk, dispatch_rank, dispatch_scan,
 * dispatch_permute_fp8, ffn_plan (no kernel when the permute writes the
 * plan), ffn_up, ffn_hidden_quant, ffn_down and combine.
 */
int32_t moe_forward_fp8w(const moe_shape *s, const void *x, const void *w_gate,
                         const float *bias, const uint8_t *w1q, const uint8_t *w3q,
                         const uint8_t *w2q, const float *wscale, void *y, int32_t *topk_idx,
                         float *topk_w, int32_t *counts, int32_t *offsets, int32_t *dest_row,
                         int32_t *src_token, void *ws, size_t ws_bytes, void *stream,
                         void *const *events, int32_t n_events);

/*
 * moe_forward that also records events[i] (hipEvent_t, created by the caller)
 * on the stream before the first kernel and after each kernel, for per-kernel
 * timing. n_events must be at least moe_forward_kernel_count(s) + 1; the
 * kernel names are given by moe_forward_kernel_name. A NULL entry is not
 * recorded (each recorded event adds a few microseconds to the pass, so a
 * caller timing one kernel records only the two events around it). Some
 * options run an extra kernel whose time falls in the next named interval:
 * capacity reassignment (the overflow kernel, in the permute's) and the fp8
 * per-expert / global modes (the range kernel, in the permute's); in a
 * forward with the persistent GEMMs the FFN tile plan is written by the
 * permute kernel, so the "ffn_plan" interval holds no kernel.
 */
int32_t moe_forward_traced(const moe_shape *s, const void *x, const void *w_gate,
                           const float *bias, const void *w1, const void *w3,
                           const void *w2, void *y, int32_t *topk_idx, float *topk_w,
                           int32_t *counts, int32_t *offsets, int32_t *dest_row,
                           int32_t *src_token, void *ws, size_t ws_bytes, void *stream,
                           void *const *events, int32_t n_events);

/* Host only: number of kernels moe_forward launches for *s, and the name of
 * the i-th ("gate_topk", "dispatch_rank", ...); NULL if out of range. The
 * gate's name is "gate_two_phase" when *s takes the two-phase gate. */
int32_t moe_forward_kernel_count(const moe_shape *s);
const char *moe_forward_kernel_name(const moe_shape *s, int32_t i);

/* Reads and clears the workspace's sticky device error flag. This call
 * synchronises `stream`. Returns MOE_OK or MOE_ERR_BAD_INDEX (or an error). */
int32_t moe_get_device_error(void *ws, size_t ws_bytes, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* MOE_MI355X_H */
