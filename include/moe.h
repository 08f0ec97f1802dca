/*
 * moe.h -- C ABI of the routed mixture-of-experts layer forward pass for
 * AMD Instinct MI355X (gfx950).
 *
 * The layer, on one GPU's share of T tokens:
 *   1. gate logits   l = X Wg (+ gate_bias)                        moe_route
 *   2. affinity a = score(l); selection I_t = TopK(a + beta);
 *      weights G = alpha * a / sum_{I_t} a (or alpha * a)          moe_route
 *   3. dispatch: per-expert counts, row map, permuted copy Xp      moe_permute
 *   4. per-expert Linear1 -> SwiGLU -> Linear2 (grouped GEMM),
 *      plus the shared expert on every token                       moe_expert_ffn
 *   5. y_t = sum_j G[t,j] Yp[row(t,j)] + Ys[t]                     moe_combine
 * and all five in order:                                           moe_forward
 *
 * Sources (page title, section):
 *   - CANN operator page "mega_moe", §计算公式 and §计算过程: the inputs
 *     X[T,hidden], E[T,topk] (expert ids), G[T,topk] (gate weights),
 *     W1[experts, hidden, 2*inter], W2[experts, inter, hidden], the output
 *     Y[T,hidden]; EP Dispatch (rows of X stacked per expert in a fixed order,
 *     row(i,k) unique), Expert Compute (Linear1, SwiGLU with the first half
 *     of the Linear1 columns as gate, Linear2), Token Combine, and the A8W8
 *     block (per-token activation scale, per-output-channel weight scales,
 *     per-row requantisation of the SwiGLU output before Linear2).
 *   - "Megatron-LM 的 MoE 并行：以 DeepSeek-V4 为例": §模型与入口 (layer
 *     equation with the shared expert F_s at weight 1), §路由张量 (affinity,
 *     selection by a + beta, mixing weight from the unbiased affinity, alpha),
 *     §Hash 路由 (token-id table replaces the selection only), §计数与重排
 *     (counts and the duplicating permute).
 *   - "Megatron 分布式训练全维度并行技术文档" §4.1-§4.2 (router weight
 *     W_gate in [H, E]; softmax top-k router with raw top-k probabilities).
 *
 * Conventions for every entry point:
 *   - All tensors are device memory, row major, densely packed, allocated
 *     and owned by the caller.  The library never allocates or frees memory
 *     and keeps no pointer after a call returns.
 *   - Calls are asynchronous on `stream` (0 = the null stream).  None of them
 *     reads device memory from the host, except moe_check_device_error.
 *   - Arguments are validated on the host before any launch; a failed check
 *     returns a negative moe_status and launches nothing.  A launch failure
 *     returns MOE_ERR_HIP.
 *   - Results are deterministic: no atomics decide an order or a sum, so two
 *     calls with the same inputs give bit-identical outputs.
 *   - Element types by precision:
 *       MOE_PREC_F32:  X, Wg, W*, Xp, Yp, Ys, Y fp32.
 *       MOE_PREC_BF16: X, Wg, W*, Xp, Yp, Ys, Y bf16.
 *       MOE_PREC_FP8:  X, Wg, Yp, Ys, Y bf16; W1/W2/Ws1/Ws2 OCP e4m3fn codes
 *                      with fp32 per-output-channel scales; Xp, Xq e4m3fn
 *                      codes with fp32 per-row scales.
 *       MOE_PREC_INT8: the mega_moe page's A8W8 block as printed: as FP8
 *                      with int8 codes in [-127, 127] and the constant 127
 *                      (scale = max|row| / 127, codes rounded half away from
 *                      zero); the products are exact int32 sums.
 *       MOE_PREC_MXFP8: the mega_moe page's MXFP mode (MX block quantisation,
 *                      groups of 32 along the contraction dimension, one
 *                      E8M0 scale byte per group, value = e4m3fn(code) *
 *                      2^(scale - 127)).  X, Wg, Yp, Ys, Y bf16; W* e4m3fn
 *                      codes with E8M0 scales [.., K/32, N]; Xp, Xq e4m3fn
 *                      codes with E8M0 scales [rows, hidden/32].  A group's
 *                      scale exponent is floor(log2(max|v|)) - 8 (0 for an
 *                      all-zero group) and its elements v / 2^exponent
 *                      rounded to nearest even, saturating at 448 (the OCP
 *                      MX rule; the page names the group size and types).
 *       MOE_PREC_MXFP4: the same MX mode with OCP e2m1 (FP4) elements, the
 *                      page's A4W4 scenario: two codes per byte, element 2i
 *                      in the low nibble; exponent floor(log2(max|v|)) - 2,
 *                      saturating at 6.  Weights are K-contiguous as the page
 *                      stores them: W1 [E, 2*inter, hidden/2], W2 [E, hidden,
 *                      inter/2], Ws1 [2*inter, hidden/2], Ws2 [hidden,
 *                      inter/2]; Xp [rows, hidden/2], Xq [T, hidden/2].
 *   - Alignment: X, Wg, the weights and scales, Xp, Xq and their scales, Yp,
 *     Ys and Y are read or written with 16-byte vector accesses and must be
 *     16-byte aligned (MOE_ERR_INVALID_ARG otherwise; allocations are).
 *   - Shape limits: 1 <= T; 1 <= topk <= min(16, experts) (the mega_moe
 *     constraint on top-k); experts <= 512; hidden a multiple of 128 and
 *     inter a multiple of 64 (the kernels' tile granularity); for FP8,
 *     INT8, MXFP8 and MXFP4 hidden a multiple of 256 and inter a multiple of
 *     128.
 */
#ifndef MOE_H
#define MOE_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  MOE_OK = 0,
  MOE_ERR_INVALID_ARG = -1, /* a pointer, size or option is out of contract */
  MOE_ERR_UNSUPPORTED = -2, /* valid, but outside what the kernels implement */
  MOE_ERR_WORKSPACE = -3,   /* workspace NULL, misaligned or too small */
  MOE_ERR_HIP = -4,         /* a HIP launch or runtime call failed */
  MOE_ERR_DEVICE_DATA = -5, /* device data broke the contract (bad expert id) */
  MOE_ERR_SCRATCH = -6      /* larger than the static scratch of moe_permute_no_alloc */
} moe_status;

typedef enum {
  MOE_PREC_F32 = 0,
  MOE_PREC_BF16 = 1,
  MOE_PREC_FP8 = 2,
  MOE_PREC_MXFP8 = 3,
  MOE_PREC_MXFP4 = 4,
  MOE_PREC_INT8 = 5
} moe_precision;

typedef enum {
  MOE_SCORE_SIGMOID = 0,      /* a = 1 / (1 + exp(-l)) */
  MOE_SCORE_SOFTMAX = 1,      /* a = softmax over the experts of l */
  MOE_SCORE_SQRT_SOFTPLUS = 2 /* a = sqrt(log(1 + exp(l))) */
} moe_score_fn;

/* Sizes of one layer invocation. */
typedef struct {
  int32_t tokens;     /* T: rows of X */
  int32_t hidden;     /* h */
  int32_t experts;    /* E: routed experts */
  int32_t topk;       /* k: experts per token */
  int32_t inter;      /* f: SwiGLU width; W1 has 2f columns */
  int32_t has_shared; /* 1: add the shared expert F_s (weight 1) */
  int32_t precision;  /* moe_precision */
} moe_shape;

/* Router options.  Score routing: ids = TopK(a + expert_bias), ordered by
 * key descending, equal keys by ascending expert id.  Hash routing (both
 * token_ids and tid2eid non-NULL): ids[t,:] = tid2eid[token_ids[t], :] and
 * expert_bias is not used.  In both, G[t,j] = alpha * a[ids[t,j]] /
 * sum_j a[ids[t,j]] when renorm, else alpha * a[ids[t,j]]. */
typedef struct {
  int32_t score_fn;          /* moe_score_fn */
  int32_t renorm;            /* 1: divide by the sum over the selected experts */
  float alpha;               /* routing scale */
  const float* expert_bias;  /* [E] fp32 beta, selection only; NULL = 0 */
  const float* gate_bias;    /* [E] fp32 bias of the gating linear; NULL = 0 */
  const int32_t* token_ids;  /* [T] token ids in [0, vocab) (hash routing) */
  const int32_t* tid2eid;    /* [vocab, topk] expert ids (hash routing) */
  int32_t vocab;             /* rows of tid2eid */
} moe_route_opts;

/* Expert weights.  W1 [E, hidden, 2*inter], W2 [E, inter, hidden]; shared
 * Ws1 [hidden, 2*inter], Ws2 [inter, hidden] (NULL without a shared expert).
 * Scales, ignored for F32 and BF16:
 *   MOE_PREC_FP8, MOE_PREC_INT8: fp32 per output channel: w1_scale [E,
 *     2*inter], w2_scale [E, hidden], ws1_scale [2*inter], ws2_scale
 *     [hidden].
 *   MOE_PREC_MXFP8: E8M0 bytes per group of 32 rows (K) and column:
 *     w1_scale [E, hidden/32, 2*inter], w2_scale [E, inter/32, hidden],
 *     ws1_scale [hidden/32, 2*inter], ws2_scale [inter/32, hidden]; the
 *     scale of W1[e, k, n] is w1_scale[e, k/32, n].
 *   MOE_PREC_MXFP4: E8M0 bytes per row of the K-contiguous weights and group
 *     of 32 along K: w1_scale [E, 2*inter, hidden/32], w2_scale [E, hidden,
 *     inter/32], ws1_scale [2*inter, hidden/32], ws2_scale [hidden,
 *     inter/32]. */
typedef struct {
  const void* W1;
  const void* w1_scale;
  const void* W2;
  const void* w2_scale;
  const void* Ws1;
  const void* ws1_scale;
  const void* Ws2;
  const void* ws2_scale;
} moe_expert_weights;

/* Bytes of device workspace that moe_forward needs for this shape (every
 * other entry point needs at most as much).  0 if the shape is invalid.  The
 * workspace must be 256-byte aligned; its contents need no initialisation
 * and are not meaningful between calls. */
size_t moe_workspace_size(const moe_shape* shape);

/* Steps 1-2: gating linear, affinity, bias-for-selection top-k, weights.
 * Source: "Megatron-LM 的 MoE 并行：以 DeepSeek-V4 为例" §路由张量 and §Hash 路由;
 * "Megatron 分布式训练全维度并行技术文档" §4.1-§4.2 (softmax top-k router).
 *   X [T, hidden] (fp32 for F32, else bf16), Wg [hidden, E] same type.
 *   expert_ids [T, topk] int32 out, gate_weights [T, topk] fp32 out.
 *   keys_out [T, E] fp32 out or NULL: the selection keys a + beta as the
 *   kernel compared them (for checking near ties).
 * Hash routing flags token ids outside [0, vocab) in the workspace (see
 * moe_check_device_error); such tokens get expert id -1 and weight 0. */
int moe_route(const moe_shape* shape, const moe_route_opts* opts, const void* X, const void* Wg,
              int32_t* expert_ids, float* gate_weights, float* keys_out, void* workspace,
              size_t workspace_bytes, hipStream_t stream);

/* Step 3: dispatch (a permutation with duplication).
 * Source: CANN "mega_moe" page §计算过程, EP Dispatch (and its A8W8 and MXFP
 * blocks for the quantised X); "Megatron-LM 的 MoE 并行" §计数与重排.
 *   counts [E] out: assignments per expert; offsets [E+1] out: exclusive
 *   prefix sum; dst_row [T*topk] out: destination row of assignment t*k+j
 *   (rows of one expert are contiguous and ordered by ascending t*k+j);
 *   src_tok [T*topk] out: token of each destination row; Xp [T*topk, hidden]
 *   out: Xp[dst_row[i]] = X[i / topk].
 *   MOE_PREC_FP8: X is bf16 and is quantised per token first (scale =
 *   max|x| / 448, codes = round-to-nearest-even of x / scale, saturating);
 *   Xq [T, hidden] e4m3 and x_scale [T] fp32 receive that, Xp holds codes
 *   and xp_scale [T*topk] fp32 the scale of each row.
 *   MOE_PREC_INT8: the same with scale = max|x| / 127 and int8 codes =
 *   x / scale (fp32 quotient) rounded half away from zero.
 *   MOE_PREC_MXFP8: X is bf16 and is MX-quantised per token (groups of 32
 *   along hidden); Xq [T, hidden] e4m3 and x_scale [T, hidden/32] E8M0 bytes
 *   receive that, Xp holds codes and xp_scale [T*topk, hidden/32] the scales
 *   of each row.
 *   MOE_PREC_MXFP4: the same with e2m1 codes, two per byte: Xq [T,
 *   hidden/2], Xp [T*topk, hidden/2], scales as for MXFP8.
 *   Otherwise xp_scale, Xq and x_scale are ignored.
 * Expert ids outside [0, E) are skipped (dst_row = -1) and flagged. */
int moe_permute(const moe_shape* shape, const int32_t* expert_ids, const void* X,
                int32_t* counts, int32_t* offsets, int32_t* dst_row, int32_t* src_tok, void* Xp,
                void* xp_scale, void* Xq, void* x_scale, void* workspace,
                size_t workspace_bytes, hipStream_t stream);

/* moe_permute without a workspace, for callers that cannot allocate device
 * memory: code under HIP graph capture, tight serving loops, harnesses that
 * forbid hipMalloc.  The same dispatch and the same outputs as moe_permute;
 * its scratch (an error flag, the per-block expert counts and the in-block
 * ranks) is a static device array of the library, about 1.3 MiB on each GPU
 * the library runs on, held until the process ends.  At most
 * MOE_NO_ALLOC_MAX_ASSIGNMENTS assignments (tokens * topk); a larger call
 * returns MOE_ERR_SCRATCH and launches nothing.  Every call on one GPU uses
 * that GPU's single array, which keeps the last call's contents: calls that
 * overlap in time on one GPU (other streams, other host threads) race and
 * give wrong results; calls ordered on one stream are safe.  Expert ids
 * outside [0, E) are skipped (dst_row = -1, not counted) as in moe_permute,
 * but with no workspace moe_check_device_error cannot report them.  Nothing
 * is allocated, on the host or on the device. */
#define MOE_NO_ALLOC_MAX_ASSIGNMENTS 262144
int moe_permute_no_alloc(const moe_shape* shape, const int32_t* expert_ids, const void* X,
                         int32_t* counts, int32_t* offsets, int32_t* dst_row, int32_t* src_tok,
                         void* Xp, void* xp_scale, void* Xq, void* x_scale, hipStream_t stream);

/* Step 4: grouped Linear1 -> SwiGLU -> Linear2 over the expert blocks given
 * [source: CANN "mega_moe" page §计算过程, Expert Compute and its A8W8 / MXFP
 * blocks; "Megatron-LM 的 MoE 并行" §ETP 里的矩阵 and §模型与入口 (shared expert)]
 * by offsets [E+1] (rows offsets[e] .. offsets[e+1]-1 of Xp belong to expert
 * e), fp32 accumulation.  Yp [T*topk, hidden] out (fp32 for F32, else bf16).
 * With a shared expert: Xs [T, hidden] is its input (X, or Xq with
 * xs_scale for the quantised precisions) and Ys [T, hidden] its output; else both may
 * be NULL.  Scales have the types moe_permute gives them.  The SwiGLU output
 * is held in the workspace: bf16 (BF16), fp32 before its per-row e4m3 or
 * int8 requantisation (FP8, INT8), or MX-quantised in groups of 32 along inter as it
 * is produced (MXFP8, MXFP4). */
int moe_expert_ffn(const moe_shape* shape, const void* Xp, const void* xp_scale,
                   const int32_t* offsets, const void* Xs, const void* xs_scale,
                   const moe_expert_weights* weights, void* Yp, void* Ys, void* workspace,
                   size_t workspace_bytes, hipStream_t stream);

/* Step 5: Y[t] = sum_{j ascending} G[t,j] * Yp[dst_row[t*k+j]] (+ Ys[t]),
 * [source: CANN "mega_moe" page §计算过程, Token Combine; "Megatron-LM 的 MoE
 * 并行" §模型与入口 (the layer equation, shared expert at weight 1)]
 * fp32 accumulation, rounded once to the output type.  Rows with dst_row < 0
 * are skipped.  Ys may be NULL. */
int moe_combine(const moe_shape* shape, const void* Yp, const int32_t* dst_row,
                const float* gate_weights, const void* Ys, void* Y, hipStream_t stream);

/* Steps 1-5.  With opts != NULL the router runs and writes expert_ids and
 * [source: the layer equation of "Megatron-LM 的 MoE 并行" §模型与入口, computed by
 * the four steps above]
 * gate_weights; with opts == NULL they are inputs (the mega_moe form, which
 * takes the routing as given) and Wg is not read.  Y [T, hidden] out, the
 * same bits as the four entry points chained.  For BF16 with hidden and
 * 2*inter multiples of 256 (and, unless both are multiples of 512, at least
 * 16 rows per expert on average) and T*hidden*2 <= 2^32 - 1, step 3 writes
 * only the row maps: Linear1 reads each routed row as its token's row of X
 * (through the row -> token map) instead of from a permuted copy. */
int moe_forward(const moe_shape* shape, const moe_route_opts* opts, const void* X,
                const void* Wg, const moe_expert_weights* weights, int32_t* expert_ids,
                float* gate_weights, void* Y, void* workspace, size_t workspace_bytes,
                hipStream_t stream);

/* Gradients written by moe_backward (device memory, bf16 unless noted). */
typedef struct {
  void* dX;           /* [T, hidden] out: gradient of X (experts, and router if opts) */
  void* dW1;          /* [E, hidden, 2*inter] out (zeros for an expert without rows) */
  void* dW2;          /* [E, inter, hidden] out */
  void* dWs1;         /* [hidden, 2*inter] out, shared expert (NULL without one) */
  void* dWs2;         /* [inter, hidden] out */
  void* dWg;          /* [hidden, E] out, or NULL (router only) */
  float* dgate_bias;  /* [E] fp32 out, or NULL (router only) */
  float* dG;          /* [T, topk] fp32 out: gradient of gate_weights, or NULL */
} moe_grads;

/* Bytes of device workspace that moe_backward needs (0 if the shape is
 * invalid); 256-byte aligned, no initialisation. */
size_t moe_backward_workspace_size(const moe_shape* shape);

/* The layer's local backward (the blog "Megatron-LM 的 MoE 并行", 反向的
 * 通信, without its collectives): given the forward's inputs and routing
 * (expert_ids, gate_weights as moe_route wrote them, or as the caller gave
 * them) and the upstream gradient dY [T, hidden], writes the gradients in
 * `grads`.  It recomputes the dispatch and the expert activations (Linear1
 * pre-activations H1 and the SwiGLU output A) in the workspace, then:
 * unpermute backward (dY[t] to each of the token's rows), Linear2 dgrad of
 * those rows U = dY[t] W2ᵀ with, in its epilogue, dA = G[t,j] U, the SwiGLU
 * backward of "Megatron 分布式训练全维度并行技术文档" §1.8 and dG[t,j] = U . A
 * (which equals dY[t] . Yp[row], Yp being A W2, so the expert outputs are
 * not recomputed), dW2 = (G A)ᵀ dY, Linear1 dgrad, dW1 = Xpᵀ dH1 (per
 * expert; the shared expert with upstream dY), permute backward (dX[t] = sum
 * of its k rows' gradients + the shared expert's).  With opts (the options of
 * the forward's router) the router is differentiated too: only the chosen
 * experts' continuous affinities carry gradient (the selection is discrete,
 * beta gets none); dWg = Xᵀ dl, dgate_bias = column sums of dl and dl Wgᵀ is
 * added to dX.  With opts == NULL, gate_weights are treated as inputs and dG is their
 * gradient.  Weight gradients are fp32 sums rounded once to bf16; dX sums
 * its parts in fp32.  BF16 layers only (MOE_ERR_UNSUPPORTED otherwise); hidden
 * a multiple of 256, inter of 128, and with opts experts a multiple of 64. */
int moe_backward(const moe_shape* shape, const moe_route_opts* opts, const void* X,
                 const void* Wg, const moe_expert_weights* weights, const int32_t* expert_ids,
                 const float* gate_weights, const void* dY, const moe_grads* grads,
                 void* workspace, size_t workspace_bytes, hipStream_t stream);

/* Training forward: steps 1-5 as moe_forward, for the layers and shapes
 * that moe_backward takes, on a backward workspace (moe_backward_workspace_size
 * bytes), keeping there what the backward reads: the dispatch, the gate
 * weight of each dispatched row, Linear1's pre-activations H1 (gate, up) and
 * the SwiGLU output A of every routed and shared row times its gate weight
 * and, with opts, the router's keys.  H1 is written out in bf16 and SwiGLU
 * applied to it (the values the backward differentiates), not fused into
 * Linear1's epilogue as in moe_forward, so Y agrees with moe_forward to bf16
 * rounding of H1.
 * Arguments and errors as moe_forward, plus those of moe_backward's shape
 * limits. */
int moe_forward_train(const moe_shape* shape, const moe_route_opts* opts, const void* X,
                      const void* Wg, const moe_expert_weights* weights, int32_t* expert_ids,
                      float* gate_weights, void* Y, void* workspace, size_t workspace_bytes,
                      hipStream_t stream);

/* moe_backward on saved activations: the same gradients, without the
 * recompute (dispatch, router keys, Linear1, SwiGLU).  The
 * workspace must hold the moe_forward_train of the same shape, X, weights,
 * routing and opts, unchanged since (the library cannot check this; anything
 * else gives wrong gradients, not an error).  Arguments and errors as
 * moe_backward. */
int moe_backward_saved(const moe_shape* shape, const moe_route_opts* opts, const void* X,
                       const void* Wg, const moe_expert_weights* weights,
                       const int32_t* expert_ids, const float* gate_weights, const void* dY,
                       const moe_grads* grads, void* workspace, size_t workspace_bytes,
                       hipStream_t stream);

/* Synchronises `stream`, then reports (and clears) the device-side error
 * flag in the workspace: MOE_ERR_DEVICE_DATA if the most recent moe_route,
 * moe_permute, moe_forward, moe_forward_train or moe_backward on this
 * workspace saw an expert id outside [0, E) or a token id outside
 * [0, vocab); MOE_OK otherwise.  Each of those calls clears the flag when it
 * starts (the workspace needs no initialisation) and covers all of its own
 * steps, so a caller that runs moe_route and then moe_permute on one
 * workspace checks after moe_route to see the router's errors. */
int moe_check_device_error(void* workspace, size_t workspace_bytes, hipStream_t stream);

/* Static text for a moe_status value. */
const char* moe_status_string(int status);

#ifdef __cplusplus
}
#endif

#endif /* MOE_H */
