/*
 * ttt.h -- C ABI of the MI355X (gfx950) TTT-layer forward library
 *          (libttt_mi355x.so).
 *
 * The library computes the forward pass of a test-time-training layer with
 * KV binding, entered after the slow projections: per (batch, head) it takes
 * queries, keys, values, a per-token learning rate eta and an initial fast
 * weight, runs chunked ("mini-batch") gradient descent on the fast weight and
 * returns the outputs and the final fast weight.
 *
 * Sources (web pages; sections as titled on the pages):
 *   [TTT]  "Test-Time Training (TTT)" summary of *Learning to (Learn at Test
 *          Time)*: "TTT definition" (fast weight W_t, W_t = W_{t-1} -
 *          eta_t grad L, y_t = f(q_t, W_t)); example 1 (inner-product loss
 *          -(kW).v, the linear-attention update); example 2 (MSE loss
 *          1/2||kW - v||^2, the delta rule); "TTT-Linear" (f(x, W) = x W);
 *          "Mini-batch gradient descent" (within a chunk every gradient is
 *          taken at the chunk-start state and the chunk's gradients summed).
 *   [KVB]  "Test-Time Training with KV Binding Is Secretly Linear Attention",
 *          abstract: the layer is a learned linear-attention operator with a
 *          fully parallel formulation.
 *   [LaCT] "LaCT: Test-Time Training Done Right": section 3.2 (SwiGLU fast
 *          weight with three matrices, negative inner-product loss, per-token
 *          learning rate, chunk gradient summed), section 3.3 (update, then L2
 *          normalisation of the fast weights), section 4 (causal
 *          apply-then-update order; update-all-then-apply order).
 *
 * Conventions shared by every entry point
 *   - All tensor pointers are HIP device pointers owned by the caller.  The
 *     library never allocates device memory; scratch space is the caller's
 *     `workspace` (size from the matching *_workspace_bytes query).  It keeps
 *     no state between calls.  Calls on different streams with distinct
 *     workspaces and outputs may run concurrently.
 *   - Work is enqueued on `stream` (a hipStream_t; NULL = the default stream)
 *     and the call returns without synchronising.  Buffers must stay alive
 *     until the stream has passed the call.
 *   - Every argument is validated on the host before anything is enqueued.
 *     On any error nothing is written and the status says why.
 *   - Layouts are dense, row-major (C order), no strides:
 *       q [B][H][Tq][d], k and v [B][H][Tkv][d] in `dtype`;
 *       eta [B][H][Tkv] fp32; out [B][H][Tq][d] in `dtype`.
 *   - Chunk c covers key tokens [c*chunk, min((c+1)*chunk, Tkv)); the last
 *     chunk may be short.
 *   - Rounding: bf16 inputs are used as given; products run on bf16 matrix
 *     cores with fp32 accumulation; the state is kept in fp32 and rounded to
 *     bf16 only as a matrix-core operand.  fp32 inputs run on fp32 matrix
 *     cores end to end.  Outputs are rounded to `dtype` (nearest even).
 */
#ifndef TTT_MI355X_H
#define TTT_MI355X_H

#include <stddef.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    TTT_OK = 0,
    TTT_EINVAL = -1,        /* null pointer, misaligned pointer, bad size or enum   */
    TTT_EUNSUPPORTED = -2,  /* valid arguments for which no kernel is built         */
    TTT_EWORKSPACE = -3,    /* workspace smaller than the *_workspace_bytes answer  */
    TTT_EHIP = -4           /* a HIP launch or query failed                          */
} ttt_status;

typedef enum { TTT_F32 = 0, TTT_BF16 = 1 } ttt_dtype;

/* Inner-product loss L_t = -f(k_t) . v_t ([TTT] example 1; [LaCT] 3.2), or
 * MSE loss L_t = 1/2 ||f(k_t) - v_t||^2 ([TTT] example 2). */
typedef enum { TTT_LOSS_DOT = 0, TTT_LOSS_MSE = 1 } ttt_loss;

/* TTT_CAUSAL: Tq == Tkv.  TTT-Linear: y_t = q_t W_t where W_t already holds
 * the summed gradients of tokens chunk_start..t (inclusive), each taken at the
 * chunk-start state ([TTT] "TTT definition" and "Mini-batch gradient
 * descent").  LaCT: the chunk's queries read the chunk-start weights, then
 * the chunk updates them ([LaCT] section 4).
 * TTT_NONCAUSAL: all Tkv key/value tokens update the state chunk by chunk,
 * then every one of the Tq queries reads the final state ([LaCT] section 4,
 * the view-synthesis order). */
typedef enum { TTT_CAUSAL = 0, TTT_NONCAUSAL = 1 } ttt_order;

/* Human-readable name of a status code (static storage). */
const char *ttt_status_string(int status);

/* Version of this ABI (bumped on any incompatible change). */
int ttt_abi_version(void);

/* ------------------------------------------------------------------------
 * TTT-Linear ([TTT] "TTT-Linear"): f(x, W) = x W with a d x d fp32 fast
 * weight per (batch, head), row-vector convention.  Per chunk c with
 * chunk-start state W_c, H_c = diag(eta over the chunk) and M the inclusive
 * lower-triangular mask (i <= t):
 *   U_c     = V_c - K_c W_c     (MSE)   or   V_c   (DOT)
 *   O_c     = Q_c W_c + ((Q_c K_c^T) * M * eta^T) U_c       (causal)
 *   W_{c+1} = W_c + K_c^T H_c U_c
 * which is the token-by-token rule with y_t read after token t's update.
 * Non-causal: the same updates over all key chunks, then O = Q W_final.
 *
 * w_init  [B][H][d][d] fp32 (w[in][out]); read only.
 * w_final [B][H][d][d] fp32; written; may alias w_init exactly (in-place
 *         state carry), any other overlap with an input is an error of the
 *         caller's.
 * Supported: d in {64, 128}; chunk a positive multiple of 16 (any Tkv,
 * ragged tails included); dtype TTT_F32 or TTT_BF16.  Tkv == 0 copies
 * w_init to w_final; Tq == 0 writes no output.  16-byte aligned pointers.
 * Returns TTT_EUNSUPPORTED for other d or chunk values.
 * ------------------------------------------------------------------------ */
size_t ttt_linear_workspace_bytes(int B, int H, int Tq, int Tkv, int d, int chunk, int loss,
                                  int order, int dtype);

ttt_status ttt_linear_fwd(const void *q, const void *k, const void *v, int dtype,
                          const float *eta, const float *w_init, void *out, float *w_final,
                          int B, int H, int Tq, int Tkv, int d, int chunk, int loss, int order,
                          void *workspace, size_t workspace_bytes, void *stream);

/* ttt_linear_fwd with the segment length chosen by the caller.  The chunk
 * update is affine in the state, so the library cuts the key/value sequence
 * into segments of whole chunks, summarises each as one affine map and chains
 * the maps ([TTT] "Mini-batch gradient descent": the per-chunk rule
 * W <- W + K^T H (V - K W) is affine in W).  ttt_linear_fwd picks the length
 * itself (about one workgroup per compute unit); here seg_tokens > 0 is the
 * requested number of key tokens per segment, rounded up to whole chunks and
 * whole 64-token blocks, and 0 means the library's own choice.  The result is
 * the same for every length up to rounding.  seg_tokens < 0: TTT_EINVAL.  The
 * workspace comes from ttt_linear_workspace_bytes_seg with the same
 * seg_tokens. */
size_t ttt_linear_workspace_bytes_seg(int B, int H, int Tq, int Tkv, int d, int chunk, int loss,
                                      int order, int dtype, int seg_tokens);

ttt_status ttt_linear_fwd_seg(const void *q, const void *k, const void *v, int dtype,
                              const float *eta, const float *w_init, void *out, float *w_final,
                              int B, int H, int Tq, int Tkv, int d, int chunk, int loss, int order,
                              int seg_tokens, void *workspace, size_t workspace_bytes,
                              void *stream);

/* ------------------------------------------------------------------------
 * LaCT SwiGLU ([LaCT] section 3.2): f(x) = W2 (silu(W1 x) * (W3 x)) per
 * (batch, head), column convention, silu(z) = z * sigmoid(z).
 *   w1, w3 [B][H][hidden][d] fp32 (out x in); w2 [B][H][d][hidden] fp32.
 * Per chunk, with the chunk-start weights:
 *   causal: O_c = f(Q_c) first, then the update;
 *   update: W <- W - grad_W sum_{t in chunk} eta_t L_t  (plain GD), then,
 *           when rownorm != 0, every row of W1, W3 (length d) and of W2
 *           (length hidden) is rescaled to its L2 norm before the update
 *           ([LaCT] section 3.3); a row whose new norm is 0 is left as is.
 *   non-causal: all updates, then O = f(Q) with the final weights.
 * There is no intra-chunk term (causality inside a chunk belongs to the
 * window attention beside the layer, [LaCT] section 4).
 * Finals may alias the matching inits exactly.
 * aux_stream (may be NULL): a second stream of the caller's on the same
 * device.  In the causal order with the inner-product loss the apply of each
 * chunk's queries does not lie on the chain of chunk updates, so when
 * aux_stream is given (and differs from `stream`) those applies run on it,
 * each after an event recorded on `stream` once its chunk's weights are
 * written, and `stream` waits for the last of them before the call returns:
 * on `stream` the call is still ordered as a whole.  The two events are made
 * for the call and released at its end.  With NULL, for other orders or
 * losses, or while `stream` is being captured into a graph, every launch stays
 * on `stream`.  Work already queued on aux_stream runs before the applies.
 * Supported: dtype TTT_BF16; d and hidden multiples of 128, each <= 1024;
 * chunk a positive multiple of 128, or >= Tkv (one chunk of any length);
 * any loss and order.  Other shapes return TTT_EUNSUPPORTED.
 * ------------------------------------------------------------------------ */
size_t lact_swiglu_workspace_bytes(int B, int H, int Tq, int Tkv, int d, int hidden, int chunk,
                                   int loss, int order, int dtype);

ttt_status lact_swiglu_fwd(const void *q, const void *k, const void *v, int dtype,
                           const float *eta, const float *w1_init, const float *w2_init,
                           const float *w3_init, void *out, float *w1_final, float *w2_final,
                           float *w3_final, int B, int H, int Tq, int Tkv, int d, int hidden,
                           int chunk, int loss, int order, int rownorm, void *workspace,
                           size_t workspace_bytes, void *stream, void *aux_stream);

/* ------------------------------------------------------------------------
 * LaCT update rules ([LaCT] section 3.3 compares gradient descent, momentum
 * and Muon, which maps the matrix-shaped gradient through a Newton-Schulz
 * iteration; the pages give no coefficients).  With G the chunk's summed
 * gradient of each matrix:
 *   TTT_RULE_GD:       W <- W - G                         (lact_swiglu_fwd)
 *   TTT_RULE_MOMENTUM: M <- beta M + G;  W <- W - M
 *   TTT_RULE_MUON:     M <- beta M + G (M = G when beta == 0);
 *                      W <- W - muon_lr * NS_k(M), where NS_k is k steps of the
 *                      cubic Newton-Schulz iteration for the orthogonal polar
 *                      factor, X_0 = M / ||M||_F, X <- 1.5 X - 0.5 X (X^T X),
 *                      and the zero matrix maps to zero
 * each followed by the row rescale when rownorm != 0.
 * m1, m2, m3: momentum buffers shaped like w1, w2, w3 (fp32), read and
 * updated in place across the call's chunks (pass zeros to start; carry them
 * between calls like the weights).  Required by TTT_RULE_MOMENTUM and by
 * TTT_RULE_MUON with beta != 0; ignored (may be NULL) otherwise.  They must
 * not overlap any other argument.
 * Limits: 0 <= beta <= 1; TTT_RULE_MUON takes 1 <= ns_steps <= 16 and a
 * finite muon_lr >= 0; otherwise TTT_EINVAL.  The Newton-Schulz products run
 * on bf16 matrix cores with fp32 accumulation and an fp32 iterate.  Everything
 * else (aux_stream included) is as for lact_swiglu_fwd, whose workspace
 * query this one extends.
 * ------------------------------------------------------------------------ */
typedef enum { TTT_RULE_GD = 0, TTT_RULE_MOMENTUM = 1, TTT_RULE_MUON = 2 } ttt_rule;

size_t lact_swiglu_rule_workspace_bytes(int B, int H, int Tq, int Tkv, int d, int hidden,
                                        int chunk, int loss, int order, int dtype, int rule);

ttt_status lact_swiglu_fwd_rule(const void *q, const void *k, const void *v, int dtype,
                                const float *eta, const float *w1_init, const float *w2_init,
                                const float *w3_init, void *out, float *w1_final, float *w2_final,
                                float *w3_final, int B, int H, int Tq, int Tkv, int d, int hidden,
                                int chunk, int loss, int order, int rownorm, int rule, float beta,
                                int ns_steps, float muon_lr, float *m1, float *m2, float *m3,
                                void *workspace, size_t workspace_bytes, void *stream,
                                void *aux_stream);

/* ------------------------------------------------------------------------
 * Decode steps: one token per (batch, head) on a carried state.
 *
 * TTT-Linear ([TTT] "TTT definition": one gradient step per token on the
 * state carried from the previous token, the output read after the step;
 * examples 1 and 2 for the gradients; "Mini-batch gradient descent" for the
 * chunk-start anchor).  Per (batch, head), with A the state the gradient is
 * taken at:
 *   u = v - k A   (MSE)   or   v   (DOT)
 *   W <- W + eta k^T u
 *   y = q W       (after the step)
 * q, k, v [B][H][d] in `dtype`; eta [B][H] fp32; out [B][H][d] in `dtype`.
 * w [B][H][d][d] fp32: the carried state, read and rewritten in place.
 * w_anchor == NULL: A = W (the recurrent rule, chunk size 1).
 * w_anchor != NULL: [B][H][d][d] fp32, the state at the start of the current
 *   chunk (A = w_anchor); anchor_update = 1 (the token closes its chunk) also
 *   writes the new W to w_anchor, anchor_update = 0 leaves it as it is.  It
 *   must not overlap w.  The inner-product loss never reads it.
 * Stepping a sequence through this call, with the anchor moved at the last
 * token of every chunk, gives the causal ttt_linear_fwd result for that chunk
 * size.  Arithmetic: fp32 FMA (the state is read once per token; the step is
 * bound by memory bandwidth).  No workspace.
 * Supported: d in {64, 128}; dtype TTT_F32 or TTT_BF16; 16-byte aligned
 * pointers.  Other d: TTT_EUNSUPPORTED.  anchor_update other than 0 or 1, or 1
 * without an anchor: TTT_EINVAL.
 * ------------------------------------------------------------------------ */
ttt_status ttt_linear_decode(const void *q, const void *k, const void *v, int dtype,
                             const float *eta, float *w, float *w_anchor, int anchor_update,
                             void *out, int B, int H, int d, int loss, void *stream);

/* ------------------------------------------------------------------------
 * TTT-Linear backward: the gradients of a scalar loss through ttt_linear_fwd
 * with the same arguments, given its upstream gradients.  Reverse-mode
 * differentiation of the per-chunk rule documented above (the token-by-token
 * definition).  Causal order, per chunk in reverse with G = dL/dW_{c+1}:
 *   dU = S^T dO + H K G,  dS = (dO U^T) * M,  dA = dS H,
 *   d_eta = rowsum_t(dS * A) + rowsum(K G * U),  dQ = dO W_c^T + dA K,
 *   dK = dA^T Q + H U G^T [- dU W_c^T],  dV = dU,  G <- G + Q^T dO [- K^T dU]
 * (A = (Q K^T) * M, S = A H; bracketed terms for the MSE loss only).
 * Non-causal order: dQ = dO W_final^T, G starts at d_w_final + Q^T dO, and the
 * same sweep runs over the key/value chunks without the output terms.
 * Inputs: q, k, v, eta, w_init as given to the forward; d_out [B][H][Tq][d]
 * in `dtype`; d_w_final [B][H][d][d] fp32 or NULL (zero).
 * Outputs: d_q [B][H][Tq][d] and d_k, d_v [B][H][Tkv][d] in `dtype`; d_eta
 * [B][H][Tkv] fp32; d_w_init [B][H][d][d] fp32.  Arithmetic: fp32 throughout
 * (the chunk-start states are recomputed by a forward pass into the
 * workspace).  Tq == Tkv for TTT_CAUSAL; Tkv >= 1; Tq may be 0 (q, d_out and
 * d_q are then not read and may be NULL) in the non-causal order.
 * Supported: the forward's shapes, d = 64 or 128 with chunk a multiple of 16
 * (ragged tails included); dtype TTT_F32 or TTT_BF16.  Others:
 * TTT_EUNSUPPORTED.  Outputs must not overlap the inputs.
 * ------------------------------------------------------------------------ */
size_t ttt_linear_bwd_workspace_bytes(int B, int H, int Tq, int Tkv, int d, int chunk, int loss,
                                      int order, int dtype);

ttt_status ttt_linear_bwd(const void *q, const void *k, const void *v, int dtype, const float *eta,
                          const float *w_init, const void *d_out, const float *d_w_final,
                          void *d_q, void *d_k, void *d_v, float *d_eta, float *d_w_init, int B,
                          int H, int Tq, int Tkv, int d, int chunk, int loss, int order,
                          void *workspace, size_t workspace_bytes, void *stream);

/* ------------------------------------------------------------------------
 * LaCT SwiGLU backward: the gradients of a scalar loss through
 * lact_swiglu_fwd with the same arguments (inner-product loss, gradient
 * descent), given the upstream gradients of the outputs and of the final
 * weights.  The pages train the layer end to end ([LaCT] section 6, Table 3:
 * training throughputs) but give no backward; this is reverse-mode
 * differentiation of the forward's steps ([LaCT] 3.2-3.3, 4): per chunk in
 * reverse, the row rescale's adjoint (with n = |W_c[r]|, m = |U[r]|,
 * U = W_c - D_c: bar_U = (n/m) Lam - (U . Lam) n U / m^3 and
 * bar_W_c = bar_U + (U . Lam) W_c[r] / (m n)), the adjoint of the chunk
 * gradient D_c (second derivatives of the SwiGLU: silu'' included) with
 * respect to the weights, keys, values and learning rates, and, for the
 * chunk's queries, the apply's adjoint at W_c (causal) or at the final
 * weights (non-causal).
 * Inputs as lact_swiglu_fwd, plus d_out [B][H][Tq][d] in `dtype` and
 * d_w1_final, d_w3_final [B][H][hid][d], d_w2_final [B][H][d][hid] fp32 (all
 * three, or all NULL for zero).  Outputs: d_q [B][H][Tq][d], d_k, d_v
 * [B][H][Tkv][d] in `dtype`; d_eta [B][H][Tkv] fp32; d_w1_init, d_w3_init
 * [B][H][hid][d], d_w2_init [B][H][d][hid] fp32.  Outputs must not overlap
 * the inputs or each other (TTT_EINVAL).
 * Arithmetic: a replay of the forward (into the workspace) recovers every
 * chunk's start weights and step; products run on bf16 matrix cores with fp32
 * accumulation, the weight adjoints accumulate in fp32.
 * Supported: dtype TTT_BF16, loss TTT_LOSS_DOT, the forward's shapes (d and
 * hidden multiples of 128 up to 1024, chunk a multiple of 128 or >= Tkv),
 * Tkv >= 1; Tq may be 0 in the non-causal order (q, d_out, d_q unused then).
 * The MSE loss returns TTT_EUNSUPPORTED.
 * ------------------------------------------------------------------------ */
size_t lact_swiglu_bwd_workspace_bytes(int B, int H, int Tq, int Tkv, int d, int hidden,
                                       int chunk, int loss, int order, int dtype);

ttt_status lact_swiglu_bwd(const void *q, const void *k, const void *v, int dtype,
                           const float *eta, const float *w1_init, const float *w2_init,
                           const float *w3_init, const void *d_out, const float *d_w1_final,
                           const float *d_w2_final, const float *d_w3_final, void *d_q, void *d_k,
                           void *d_v, float *d_eta, float *d_w1_init, float *d_w2_init,
                           float *d_w3_init, int B, int H, int Tq, int Tkv, int d, int hidden,
                           int chunk, int loss, int order, int rownorm, void *workspace,
                           size_t workspace_bytes, void *stream);

/* LaCT decode apply ([LaCT] sections 3.2 and 4): out = W2 (silu(W1 q) * (W3 q))
 * for one query per (batch, head), with the weights as they stand (in the
 * causal order, the start-of-chunk weights of the chunk being decoded).  The
 * chunk's keys, values and learning rates are kept by the caller; once the
 * chunk is complete, lact_swiglu_fwd with TTT_NONCAUSAL and Tq = 0 applies
 * its update.  Stepping a sequence this way gives the causal lact_swiglu_fwd
 * result.
 * q [B][H][d] in `dtype`; w1, w3 [B][H][hidden][d], w2 [B][H][d][hidden]
 * fp32, read only; out [B][H][d] in `dtype`.  Arithmetic: fp32 FMA.
 * workspace: at least lact_swiglu_decode_workspace_bytes (it holds the hidden
 * activations between the two launches).
 * Supported: dtype TTT_F32 or TTT_BF16; d and hidden multiples of 64, each
 * <= 1024; 16-byte aligned pointers.  The workspace query returns 0 for
 * anything unsupported. */
size_t lact_swiglu_decode_workspace_bytes(int B, int H, int d, int hidden, int dtype);

ttt_status lact_swiglu_decode(const void *q, int dtype, const float *w1, const float *w2,
                              const float *w3, void *out, int B, int H, int d, int hidden,
                              void *workspace, size_t workspace_bytes, void *stream);

/* ------------------------------------------------------------------------
 * Sliding-window attention beside LaCT ([LaCT] section 3.1: a window attention
 * reads the relations of nearby tokens; section 4: it shares Q, K, V with the
 * fast weight, the two outputs are combined, and its causal sliding window
 * supplies causality inside a chunk).  Per (batch, head) and query t:
 *   out_t (+)= sum_{t - window < s <= t} softmax_s(scale * q_t . k_s) v_s
 * q, k, v, out [B][H][T][d] in `dtype` (the same tensors the fast weight
 * reads).  accumulate = 1 adds the attention to what out holds (out may then
 * be the output of lact_swiglu_fwd), in fp32 with one rounding; 0 overwrites.
 * out must not overlap q, k or v.  scale: a finite value > 0 (1/sqrt(d) is
 * the usual choice).  Scores, the softmax and the output accumulate in fp32;
 * Q K^T and P V run on bf16 matrix cores.  No workspace.
 * Supported: dtype TTT_BF16; d in {64, 128, 256}; any T >= 0 and window >= 1.
 * ------------------------------------------------------------------------ */
ttt_status window_attention_fwd(const void *q, const void *k, const void *v, int dtype, void *out,
                                int B, int H, int T, int d, int window, float scale,
                                int accumulate, void *stream);

/* ------------------------------------------------------------------------
 * ttt_linear_fwd for callers that cannot allocate device memory: code being
 * captured into a HIP graph, tight serving loops, harnesses that forbid
 * allocation.  Same arguments, kernels and results as ttt_linear_fwd, minus
 * the workspace: the scratch the state scan needs (segment summaries, and a
 * copy of w_init for in-place calls) lives in one static device array per
 * GPU of ttt_linear_noalloc_max_scratch_bytes() bytes (64 MiB), held from the
 * first call on that GPU until the process ends.  No allocation is made by
 * the call.  A problem whose scratch (ttt_linear_workspace_bytes) exceeds the
 * array returns TTT_EWORKSPACE before anything is enqueued; with the
 * library's own segment length every causal call fits, and an
 * update-then-apply call fits while heads * d * d * (2 or 4 + 4) bytes does.
 * Every call on a GPU shares that GPU's array: calls that overlap on one GPU
 * (on different streams, not ordered with each other) race on it and must not
 * be issued.  Nothing needs clearing between calls (each call writes all the
 * scratch it reads).
 * ------------------------------------------------------------------------ */
size_t ttt_linear_noalloc_max_scratch_bytes(void);

ttt_status ttt_linear_fwd_noalloc(const void *q, const void *k, const void *v, int dtype,
                                  const float *eta, const float *w_init, void *out,
                                  float *w_final, int B, int H, int Tq, int Tkv, int d, int chunk,
                                  int loss, int order, void *stream);

/* ------------------------------------------------------------------------
 * Measurement helper (not part of the layer): `blocks` workgroups of four
 * waves, each wave running `iters` rounds of four independent bf16 32x32x16
 * matrix-core products (32768 flops each), so the dense bf16 rate this part
 * reaches is blocks * 4 * iters * 4 * 32768 flops over the launch's duration.
 * out: device buffer of blocks * 256 floats (written with the accumulators'
 * sums).  blocks in [1, 2^20], iters >= 1, else TTT_EINVAL.
 * ------------------------------------------------------------------------ */
ttt_status ttt_probe_mfma_bf16(float *out, int blocks, int iters, void *stream);

/* ------------------------------------------------------------------------
 * Measurement helper (not part of the layer): the bf16 GEMM tile the LaCT
 * kernels share, on a plain product, so its rate can be measured:
 * C[m][n] = sum_k A[m][k] B[n][k], fp32 accumulation and output, one
 * workgroup per block_rows x 128 tile of C (block_rows 128: four 64 x 64 wave
 * tiles; 256: four 128 x 64 wave tiles; 64: four 32 x 64 wave tiles).  wave_groups 2 (block_rows 128 only)
 * runs each tile with eight waves, the second four taking the second half of
 * the k steps.  A is [M][K] bf16 (a_kmajor = 0) or [K][M] (a_kmajor = 1,
 * read as its transpose); B likewise [N][K] or [K][N]; C [M][N] fp32, all
 * row-major, device memory, 16-byte aligned.  M a multiple of block_rows, N
 * of 128, K of 64, block_rows 64, 128 or 256, wave_groups 1 or 2, else
 * TTT_EINVAL.
 * ------------------------------------------------------------------------ */
ttt_status ttt_probe_gemm_bf16(const void *a, const void *b, float *c, int M, int N, int K, int a_kmajor,
                               int b_kmajor, int block_rows, int wave_groups, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* TTT_MI355X_H */
