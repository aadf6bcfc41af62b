/*
 * moe.h -- C ABI of the DeepSeekMoE layer (forward and backward) on one AMD
 * MI355X (gfx950).
 *
 * The layer (DeepSeekMoE explainer, deepforge.srivtx.xyz "DeepSeekMoE",
 * sections "Routing in a classic MoE layer", "Expert-level balance loss" and
 * "What the 16B configuration looks like"):
 *
 *   s_i = softmax_i(u^T e_i)   over the n = m*N routed (fine-grained) experts
 *   g_i = s_i if s_i is among the k = m*K - K_s largest, else 0
 *         (no renormalisation: the kept gates do not sum to one)
 *   h   = sum_i g_i FFN_i(u) + sum_{q < K_s} FFN^shared_q(u) + u
 *
 * with FFN(x) = W2 (SiLU(W1 x) * (W3 x)) (SwiGLU, no biases), K_s shared
 * experts that every token uses with weight one, and the expert-level
 * balance statistics f_i = n/(k T) * count_i and P_i = (1/T) sum_t s_{t,i}.
 *
 * Conventions for every entry point:
 *   - Buffers are DEVICE pointers owned by the caller; the library never
 *     allocates.  Scratch space comes from the caller's workspace `ws` of
 *     `ws_bytes` bytes (see moe_workspace_bytes; moe_bwd_workspace_bytes for
 *     the backward pass).
 *   - Every pointer must be 16-byte aligned; tensors are dense row-major.
 *   - `stream` is a hipStream_t (NULL = the default stream).  Work is
 *     enqueued asynchronously; no call synchronises the device or copies
 *     data to the host.
 *   - Arguments are validated on the host before anything is enqueued.  On
 *     any error nothing is launched and the status says why.  Errors raised
 *     by the HIP runtime at launch map to MOE_ERR_HIP.
 *   - Element type: MOE_BF16 (bf16 storage, fp32 accumulation) or MOE_F32.
 *     u, h, centroids, weights, x_perm and y use the problem's dtype; gates,
 *     f and P are fp32; indices and counts are int32.
 *   - Inputs must be finite; results are unspecified otherwise.
 *   - Calls on different streams that share a workspace race.
 */
#ifndef MOE_H
#define MOE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum moe_status {
  MOE_OK = 0,
  MOE_ERR_NULL = 1,        /* a required pointer is NULL */
  MOE_ERR_SHAPE = 2,       /* sizes out of range (see moe_problem) */
  MOE_ERR_DTYPE = 3,       /* unknown element type */
  MOE_ERR_ALIGN = 4,       /* a pointer is not 16-byte aligned */
  MOE_ERR_WORKSPACE = 5,   /* ws is NULL or ws_bytes is too small */
  MOE_ERR_UNSUPPORTED = 6, /* valid request this build does not handle */
  MOE_ERR_HIP = 7          /* the HIP runtime reported an error */
} moe_status;

typedef enum moe_dtype { MOE_F32 = 0, MOE_BF16 = 1 } moe_dtype;

#define MOE_MAX_EXPERTS 256 /* n = m*N */
#define MOE_MAX_TOPK 64     /* k = m*K - K_s */

/*
 * The pages' statement of the problem.  Valid when
 *   T >= 1;  T*k*d, T*k*d_ff, T*K_s*d_ff, d*d_ff and K_s*d_ff*d < 2^31;
 *   d, d_ff >= 32 and multiples of 32;
 *   N, m, K >= 1;  K_s >= 0;  n = m*N <= MOE_MAX_EXPERTS;
 *   1 <= k = m*K - K_s <= min(n, MOE_MAX_TOPK).
 * Only the products m*N and m*K enter the result.
 */
typedef struct moe_problem {
  int64_t T;     /* tokens */
  int32_t d;     /* hidden size */
  int32_t N;     /* experts before fine-grained segmentation */
  int32_t m;     /* segmentation factor */
  int32_t K;     /* activated experts before segmentation */
  int32_t K_s;   /* shared (always-on) experts */
  int32_t d_ff;  /* SwiGLU intermediate size of one fine-grained expert */
  int32_t dtype; /* moe_dtype */
} moe_problem;

/* Flags.  MOE_NO_RESIDUAL / MOE_NO_SHARED (moe_layer_fwd, moe_layer_bwd) drop
 * a term for component checks.  MOE_PACKED_WEIGHTS (moe_layer_fwd, moe_grouped_ffn):
 * every expert weight tensor is in the packed layout of moe_pack_weights
 * instead of row-major; bf16 only. */
enum { MOE_NO_RESIDUAL = 1, MOE_NO_SHARED = 2, MOE_PACKED_WEIGHTS = 4, MOE_SAVE_FOR_BACKWARD = 8 };

/* Bytes of workspace that suffice for every entry point on this problem;
 * 0 when the problem is invalid. */
size_t moe_workspace_bytes(const moe_problem *p);

/* Bytes of workspace for moe_layer_fwd with MOE_SAVE_FOR_BACKWARD: the above
 * plus the kept pre-activations, (T*k + T*K_s) * 2 * d_ff bf16 values, and
 * the router's fp32 logits; 0 when the problem is invalid or not bf16. */
size_t moe_train_workspace_bytes(const moe_problem *p);

/*
 * Router: the affinities and the TopK gate of the equation in "Routing in a
 * classic MoE layer" (the selection as in "Top-k routing, from affinities to
 * gates"); the statistics f_i and P_i of "Expert-level balance loss".
 *   u [T][d], centroids [n][d]                        in
 *   topk_idx [T][k]   kept experts, descending logit u^T e_i; equal logits
 *                     keep the lower expert index first (this library's tie
 *                     rule: the equation's set form leaves ties open)
 *   topk_gate [T][k]  s of the kept experts (fp32)
 *   counts [n]        tokens that kept expert i
 *   f [n]             (float)(count_i * n) / (float)(k * T)
 *   P [n]             mean over tokens of s_i (fp32)
 * Logits are accumulated in fp32; selection is made on the fp32 logits.
 */
moe_status moe_route(const moe_problem *p, const void *u, const void *centroids,
                     int32_t *topk_idx, float *topk_gate, int32_t *counts, float *f, float *P,
                     void *ws, size_t ws_bytes, void *stream);

/*
 * Grouping of the T*k (token, slot) pairs by expert, after the note closing
 * "Top-k routing, from affinities to gates" that a production layer groups
 * tokens per expert; expert-major with ascending token inside each expert
 * (a stable counting sort).
 *   u [T][d], topk_idx [T][k]                         in
 *   offsets [n+1]     first grouped row of each expert, offsets[n] = T*k
 *   perm_token [T*k]  token of each grouped row
 *   slot_of [T][k]    grouped row of (t, j)
 *   x_perm [T*k][d]   row r = u[perm_token[r]]; may be NULL (indices only)
 */
moe_status moe_permute(const moe_problem *p, const void *u, const int32_t *topk_idx,
                       int32_t *offsets, int32_t *perm_token, int32_t *slot_of, void *x_perm,
                       void *ws, size_t ws_bytes, void *stream);

/*
 * Grouped SwiGLU FFN, the experts FFN_i of the equation in "Routing in a
 * classic MoE layer" run the way the note closing "Top-k routing, from
 * affinities to gates" describes a production layer: tokens grouped per
 * expert, each expert's weight matrices applied to its group at once (and the
 * always-on shared experts of "What the 16B configuration looks like" as one
 * dense group).  Rows offsets[g] .. offsets[g+1]-1 of x go through
 * expert g: y = W2_g (SiLU(W1_g x) * (W3_g x)).  The intermediate is rounded
 * to the dtype (bf16) between the two products; accumulation is fp32.
 *   n_groups          1 .. MOE_MAX_EXPERTS
 *   rows              total rows (= offsets[n_groups] - offsets[0]); offsets
 *                     must be non-decreasing with offsets[0] = 0
 *   offsets [n_groups+1] (device)
 *   x [rows][d]; w1, w3 [n_groups][d_ff_group][d]; w2 [n_groups][d][d_ff_group]
 *   y [rows][d]       out
 * Routed experts: n_groups = n, rows = T*k, d_ff_group = d_ff.  Shared
 * experts as one dense SwiGLU (their sum): n_groups = 1, rows = T,
 * d_ff_group = K_s*d_ff, offsets = {0, T}.
 * d_ff_group must be a multiple of 32 with d_ff_group*d < 2^31 and
 * rows*d_ff_group fitting the workspace of moe_workspace_bytes(p).  flags: 0 or MOE_PACKED_WEIGHTS.
 */
moe_status moe_grouped_ffn(const moe_problem *p, int32_t n_groups, int64_t rows,
                           const int32_t *offsets, const void *x, const void *w1,
                           const void *w3, const void *w2, int32_t d_ff_group, int flags,
                           void *y, void *ws, size_t ws_bytes, void *stream);

/*
 * Gate-weighted combine with residual ("Routing in a classic MoE layer"):
 *   h[t] = residual[t] + shared_out[t] + sum_j topk_gate[t][j] * y_perm[slot_of[t][j]]
 * summed in fp32 (j ascending, then shared, then residual), rounded once.
 * residual and shared_out may be NULL (term omitted).
 *   y_perm [T*k][d], slot_of [T][k], topk_gate [T][k], h [T][d]
 */
moe_status moe_combine(const moe_problem *p, const void *residual, const void *shared_out,
                       const void *y_perm, const int32_t *slot_of, const float *topk_gate,
                       void *h, void *stream);

/*
 * The expert-level balance loss of "Expert-level balance loss":
 *   loss[0] = alpha * sum_i f_i * P_i      over the n = m*N routed experts,
 * from the statistics f [n] and P [n] that moe_route / moe_layer_fwd write
 * (device pointers).  fp32: each product rounded, then added in ascending i
 * starting from 0, then the product with alpha rounded (no fused
 * multiply-add), so the value does not depend on any reduction tree.
 * Asynchronous on `stream`; errors as for the other entry points.
 */
moe_status moe_balance_loss(const moe_problem *p, const float *f, const float *P, float alpha,
                            float *loss, void *stream);

/*
 * The whole layer: the equation of "Routing in a classic MoE layer"
 * (affinities, TopK gates, h = sum_i g_i FFN_i(u) + u) with the fine-grained
 * experts and the always-on shared experts of "What the 16B configuration
 * looks like", and the statistics of "Expert-level balance loss": route,
 * group, routed experts, shared experts, combine.
 *   u [T][d], centroids [n][d]
 *   w1, w3 [n][d_ff][d], w2 [n][d][d_ff]              routed experts
 *   ws1, ws3 [K_s*d_ff][d], ws2 [d][K_s*d_ff]         shared experts (expert q
 *                     owns rows / columns q*d_ff .. q*d_ff + d_ff - 1); NULL
 *                     allowed when K_s = 0 or flags has MOE_NO_SHARED
 *   h [T][d]          out
 *   topk_idx, topk_gate, counts, f, P                 out, as moe_route
 *   flags             MOE_NO_RESIDUAL drops +u, MOE_NO_SHARED drops the shared
 *                     experts (component checks only); MOE_PACKED_WEIGHTS: all
 *                     six weight tensors come from moe_pack_weights;
 *                     MOE_SAVE_FOR_BACKWARD (bf16): the workspace, of
 *                     moe_train_workspace_bytes(p) bytes, also keeps the
 *                     up projection's pre-activations W1 x and W3 x, the
 *                     router's logits and the grouping, for moe_layer_bwd
 *                     (which then skips computing them again); h is the
 *                     same either way
 */
moe_status moe_layer_fwd(const moe_problem *p, const void *u, const void *centroids,
                         const void *w1, const void *w3, const void *w2, const void *ws1,
                         const void *ws3, const void *ws2, void *h, int32_t *topk_idx,
                         float *topk_gate, int32_t *counts, float *f, float *P, int flags,
                         void *ws, size_t ws_bytes, void *stream);

/*
 * moe_layer_fwd for callers that cannot allocate device memory (code under
 * HIP graph capture, tight serving loops, harnesses that forbid hipMalloc):
 * no workspace argument; the scratch is a fixed array of
 * MOE_NOALLOC_SCRATCH_BYTES bytes that the library holds on every device it
 * runs on until the process ends.  No call allocates; the first call on a
 * device looks the array's address up there once.  Arguments and results are
 * those of moe_layer_fwd (the same kernels).
 *   - MOE_ERR_WORKSPACE: moe_workspace_bytes(p) exceeds the array (at the
 *     16B shape, T = 64 needs 3.3 MB and about 600 tokens fill it);
 *   - MOE_ERR_UNSUPPORTED: flags with MOE_SAVE_FOR_BACKWARD (the backward
 *     could not name the kept workspace), or a stream that belongs to another
 *     device than the calling thread's current one.
 * Every call on one device shares that device's array and leaves its
 * contents there: calls that overlap in time on one device (several streams
 * or host threads) race; calls ordered on one stream do not.
 */
#define MOE_NOALLOC_SCRATCH_BYTES (32u << 20)
moe_status moe_layer_fwd_noalloc(const moe_problem *p, const void *u, const void *centroids,
                                 const void *w1, const void *w3, const void *w2,
                                 const void *ws1, const void *ws3, const void *ws2, void *h,
                                 int32_t *topk_idx, float *topk_gate, int32_t *counts, float *f,
                                 float *P, int flags, void *stream);

/*
 * Weight layout for the grouped FFN's fast path (an implementation choice,
 * made once when weights are loaded; the layer's result does not depend on
 * it).  src is a bf16 matrix [rows][K] row-major; dst (same size, must not
 * overlap src) receives it as 32-row bands, each band a run of K/16 blocks
 * of 32 rows x 16 columns, and each block stored in MFMA operand order:
 * element (r, k) of block sits at ((r % 32) + 32 * ((k % 16) / 8)) * 8 + k % 8.
 * Stacked expert tensors pack as one matrix: w1, w3 with rows = n*d_ff,
 * K = d; w2 with rows = n*d, K = d_ff; ws1, ws3 with rows = K_s*d_ff, K = d;
 * ws2 with rows = d, K = K_s*d_ff.  Requires p->dtype == MOE_BF16,
 * rows % 32 == 0, K % 32 == 0.  Asynchronous on stream.
 */
moe_status moe_pack_weights(const moe_problem *p, int64_t rows, int32_t K, const void *src,
                            void *dst, void *stream);

/*
 * moe_layer_fwd with measurement marks, for callers that time the layer's
 * kernels on the stream they run on.  `marks` holds hipEvent_t handles created
 * by the caller, at least moe_layer_kernels(p, flags, NULL, 0) + 1 of them:
 * marks[0] is recorded before the first kernel and marks[i] right after the
 * i-th kernel launch, all on `stream`.  marks = NULL behaves as moe_layer_fwd.
 */
moe_status moe_layer_fwd_marked(const moe_problem *p, const void *u, const void *centroids,
                                const void *w1, const void *w3, const void *w2,
                                const void *ws1, const void *ws3, const void *ws2, void *h,
                                int32_t *topk_idx, float *topk_gate, int32_t *counts, float *f,
                                float *P, int flags, void *ws, size_t ws_bytes, void *stream,
                                void *const *marks);

/*
 * Number of kernels moe_layer_fwd launches for (p, flags); when names is not
 * NULL, up to max_names static kernel labels are stored.  Returns -1 for an
 * invalid problem.
 */
int moe_layer_kernels(const moe_problem *p, int flags, const char **names, int max_names);

/*
 * Backward pass of the layer.  The gradients are those of
 *   L = sum_t <dh_t, h_t> + alpha * sum_i f_i P_i
 * (the layer's output against an upstream gradient dh, plus the
 * expert-level balance loss of "Expert-level balance loss" with coefficient
 * alpha), with the routing of the forward held fixed: the kept sets and the
 * counts behind f_i are piecewise constant and carry no gradient, the gates
 * and P_i carry it through the softmax.  Chain rule per expert on x with gate
 * g: dhid = W2^T dh, dg = <dhid, SiLU(a) * b>, da = g dhid * b * SiLU'(a),
 * db = g dhid * SiLU(a), dx = W1^T da + W3^T db, dW1 = da x^T,
 * dW3 = db x^T, dW2 = g dh (SiLU(a) * b)^T; router: ds_i = dg (kept i) +
 * alpha f_i / T, dl = s * (ds - <s, ds>), du += E^T dl, dE_i = sum_t dl_{t,i} u_t.
 *   u, centroids, w1, w3, w2, ws1, ws3, ws2   as moe_layer_fwd (bf16; row-major, or
 *                     all six in the layout of moe_pack_weights with
 *                     MOE_PACKED_WEIGHTS, the same copies the forward reads)
 *   topk_idx [T][k], topk_gate [T][k], f [n]  the forward's routing outputs
 *                     (an expert id outside [0, n) breaks the contract; such a
 *                     slot is skipped, as moe_permute leaves it out)
 *   fwd_ws            the workspace of the forward call that produced them, if
 *                     that call had MOE_SAVE_FOR_BACKWARD (with nothing run on
 *                     that workspace since); flags must then include
 *                     MOE_SAVE_FOR_BACKWARD too; the same weights and u must
 *                     be passed.  NULL otherwise: a and b, the router's logits
 *                     and the grouping are computed again.  Status codes:
 *                     MOE_ERR_NULL for the flag without fwd_ws, MOE_ERR_SHAPE
 *                     for fwd_ws without the flag, MOE_ERR_ALIGN if misaligned
 *   dh [T][d]         upstream gradient (bf16)
 *   alpha             balance-loss coefficient (0: no balance term)
 *   du [T][d], dcentroids [n][d]              out, fp32
 *   dw1, dw3 [n][d_ff][d], dw2 [n][d][d_ff]   out, fp32 (zero for experts no
 *                     token kept)
 *   dws1, dws3 [K_s*d_ff][d], dws2 [d][K_s*d_ff]   out, fp32; NULL allowed
 *                     when K_s = 0 or flags has MOE_NO_SHARED
 *   flags             MOE_NO_RESIDUAL / MOE_NO_SHARED as moe_layer_fwd (the
 *                     forward must have used the same flags); MOE_PACKED_WEIGHTS;
 *                     MOE_SAVE_FOR_BACKWARD exactly when fwd_ws is given
 *   ws                workspace of at least moe_bwd_workspace_bytes(p) bytes
 * Intermediates (the SwiGLU gradients, q = W2^T dh, the experts' input
 * gradients, the router's softmax gradient) are rounded to bf16; every
 * product accumulates in fp32; the result does not depend on the weight
 * layout.  Requires p->dtype == MOE_BF16, and beyond the limits of
 * moe_problem: T * (n rounded up to 8) < 2^31, and d_ff*d, K_s*d_ff*d and
 * n*d below 2^29 - 4 (each gradient output of one expert, of the shared
 * experts, of the centroids, in fp32 bytes, stays below 2^31 - 16);
 * MOE_ERR_SHAPE otherwise, before anything is enqueued.
 */
moe_status moe_layer_bwd(const moe_problem *p, const void *u, const void *centroids,
                         const void *w1, const void *w3, const void *w2, const void *ws1,
                         const void *ws3, const void *ws2, const int32_t *topk_idx,
                         const float *topk_gate, const float *f, const void *fwd_ws,
                         const void *dh, float alpha,
                         float *du, float *dcentroids, float *dw1, float *dw3, float *dw2,
                         float *dws1, float *dws3, float *dws2, int flags, void *ws,
                         size_t ws_bytes, void *stream);

/* Workspace bytes moe_layer_bwd needs on this problem; 0 when the problem
 * is invalid or not bf16. */
size_t moe_bwd_workspace_bytes(const moe_problem *p);

/* moe_layer_bwd with measurement marks (as moe_layer_fwd_marked), and the
 * number and labels of the kernels it launches. */
moe_status moe_layer_bwd_marked(const moe_problem *p, const void *u, const void *centroids,
                                const void *w1, const void *w3, const void *w2,
                                const void *ws1, const void *ws3, const void *ws2,
                                const int32_t *topk_idx, const float *topk_gate, const float *f,
                                const void *fwd_ws, const void *dh, float alpha, float *du,
                                float *dcentroids,
                                float *dw1, float *dw3, float *dw2, float *dws1, float *dws3,
                                float *dws2, int flags, void *ws, size_t ws_bytes, void *stream,
                                void *const *marks);
int moe_layer_bwd_kernels(const moe_problem *p, int flags, const char **names, int max_names);

/* Static description of a status code. */
const char *moe_status_str(moe_status s);

/* The hipError_t behind the most recent MOE_ERR_HIP returned on the calling
 * host thread (0 if none yet).  If text is not NULL, *text receives the HIP
 * runtime's static description of it.  Diagnostic only; never fails. */
int moe_last_hip_error(const char **text);

#ifdef __cplusplus
}
#endif

#endif /* MOE_H */
