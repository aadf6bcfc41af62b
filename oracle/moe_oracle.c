/*
 * moe_oracle.c -- plain, slow CPU oracle of the DeepSeekMoE layer forward.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the
 * benchmark's CPU-baseline leg may load this library.  It shares no code,
 * header or constant with the GPU path.
 *
 * Arithmetic is IEEE fp32 with a fixed, ascending summation order and no
 * fused multiply-add; OpenMP splits only independent tokens, so results are
 * identical at any thread count.  bf16 inputs are widened to fp32 exactly.
 *
 * What it computes (DeepSeekMoE pages, deepforge.srivtx.xyz "DeepSeekMoE"):
 *   - fine-grained segmentation: n = m*N routed experts, mK activated, of
 *     which K_s are shared, so k = m*K - K_s routed experts are kept
 *     (sections "What it is" and "The idea in two moves");
 *   - routing of section "Routing in a classic MoE layer":
 *       s_i = softmax_i(u^T e_i) over all n routed experts,
 *       g_i = s_i if s_i is among the k largest, else 0 (no renormalisation,
 *       as the note under "Top-k routing, from affinities to gates" states),
 *       h   = sum_i g_i FFN_i(u) + [shared experts] + u;
 *   - the k kept experts in descending order of their logit (selection on
 *     the logits equals selection on s, the softmax being monotone); equal
 *     logits keep the lower expert index first (this project's tie rule);
 *   - balance statistics of section "Expert-level balance loss": f_i from the
 *     share of tokens that picked expert i, P_i the mean affinity s_i;
 *   - expert FFN = SwiGLU ("GLU Variants Improve Transformer", cited on the
 *     observer.broadside.tech card): FFN(x) = W2 (SiLU(W1 x) * (W3 x)),
 *     SiLU(z) = z / (1 + exp(-z)), no biases.
 * Readings where the pages are silent: softmax over the routed experts only
 * (shared experts have no centroid and weight one); f_i = n/(k T) * count_i so
 * that sum_i f_i = n; the layer is dropless (no capacity limit).
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define ORC_F32 0
#define ORC_BF16 1

#define ORC_OK 0
#define ORC_ERR_ARG 1
#define ORC_ERR_MEM 2

/* Element i of a stored tensor as fp32 (bf16 widening is exact). */
static float orc_get(const void *p, size_t i, int dtype) {
  if (dtype == ORC_BF16) {
    uint32_t b = (uint32_t)((const uint16_t *)p)[i] << 16;
    float f;
    memcpy(&f, &b, sizeof f);
    return f;
  }
  return ((const float *)p)[i];
}

/* Step 1: routed experts n = m N, kept experts k = m K - K_s. */
int oracle_sizes(int N, int m, int K, int K_s, int *n, int *k) {
  if (N < 1 || m < 1 || K < 1 || K_s < 0) return ORC_ERR_ARG;
  *n = m * N;
  *k = m * K - K_s;
  if (*k < 1 || *k > *n) return ORC_ERR_ARG;
  return ORC_OK;
}

/* Affinity logit u^T e_i, summed over j ascending. */
static float orc_logit(const void *u, const void *cent, int64_t t, int i, int d, int dtype) {
  float acc = 0.0f;
  for (int j = 0; j < d; ++j)
    acc += orc_get(u, (size_t)t * d + j, dtype) * orc_get(cent, (size_t)i * d + j, dtype);
  return acc;
}

/*
 * Routing of one token (section "Routing in a classic MoE layer": s_i =
 * softmax_i(u^T e_i) over all n routed experts, g_i = s_i for the k largest
 * s_i, 0 otherwise).  logit[n] in.  s[n] = the softmax, formed with the
 * largest logit subtracted from every logit (the same quotient, no
 * overflow).  sel[k] = the kept experts, chosen in k rounds: each round keeps
 * the largest logit not kept yet.  The softmax is monotone, so these are the
 * k largest s_i, in descending order.  Equal logits: the lower expert index
 * is kept first (this project's tie rule; the pages' set form leaves ties
 * open, the rule makes the set and its order unique).  taken[n] is scratch.
 */
static void orc_route_token(const float *logit, int n, int k, float *s, int *sel, char *taken) {
  float mx = logit[0];
  for (int i = 1; i < n; ++i)
    if (logit[i] > mx) mx = logit[i];
  float z = 0.0f;
  for (int i = 0; i < n; ++i) {
    s[i] = expf(logit[i] - mx);
    z += s[i];
  }
  for (int i = 0; i < n; ++i) s[i] = s[i] / z;
  for (int i = 0; i < n; ++i) taken[i] = 0;
  for (int j = 0; j < k; ++j) {
    int best = -1;
    for (int i = 0; i < n; ++i)
      if (!taken[i] && (best < 0 || logit[i] > logit[best])) best = i;
    taken[best] = 1;
    sel[j] = best;
  }
}

/*
 * Steps 2-6 over all T tokens.
 *   u [T][d], cent [n][d]                    (dtype storage)
 *   topk_idx [T][k], topk_gate [T][k]        kept experts in selection order
 *   logits, scores [T][n]                    optional (NULL to skip)
 *   counts [n]; f [n] = (count_i * n) / (k * T); P [n] = (sum_t s_ti) / T
 */
int oracle_route(int64_t T, int d, int n, int k, int dtype, const void *u, const void *cent,
                 int32_t *topk_idx, float *topk_gate, float *logits, float *scores,
                 int32_t *counts, float *f, float *P) {
  if (T < 1 || d < 1 || n < 1 || k < 1 || k > n) return ORC_ERR_ARG;
  float *s_all = scores;
  float *own = NULL;
  if (!s_all) {
    own = (float *)malloc(sizeof(float) * (size_t)T * n);
    if (!own) return ORC_ERR_MEM;
    s_all = own;
  }
  int fail = 0;
#pragma omp parallel
  {
    float *lg = (float *)malloc(sizeof(float) * n);
    int *sel = (int *)malloc(sizeof(int) * k);
    char *taken = (char *)malloc((size_t)n);
#pragma omp for schedule(static)
    for (int64_t t = 0; t < T; ++t) {
      if (!lg || !sel || !taken) {
#pragma omp atomic write
        fail = 1;
        continue;
      }
      {
        for (int i = 0; i < n; ++i) lg[i] = orc_logit(u, cent, t, i, d, dtype);
        float *s = s_all + (size_t)t * n;
        orc_route_token(lg, n, k, s, sel, taken);
        for (int j = 0; j < k; ++j) {
          topk_idx[(size_t)t * k + j] = sel[j];
          topk_gate[(size_t)t * k + j] = s[sel[j]];
        }
        if (logits) memcpy(logits + (size_t)t * n, lg, sizeof(float) * n);
      }
    }
    free(lg);
    free(sel);
    free(taken);
  }
  if (fail) {
    free(own);
    return ORC_ERR_MEM;
  }
  for (int i = 0; i < n; ++i) counts[i] = 0;
  for (int64_t t = 0; t < T; ++t)
    for (int j = 0; j < k; ++j) counts[topk_idx[(size_t)t * k + j]] += 1;
  for (int i = 0; i < n; ++i) {
    f[i] = (float)((int64_t)counts[i] * n) / (float)((int64_t)k * T);
    float acc = 0.0f;
    for (int64_t t = 0; t < T; ++t) acc += s_all[(size_t)t * n + i];
    P[i] = acc / (float)T;
  }
  free(own);
  return ORC_OK;
}

/* L_ExpBal = alpha * sum_i f_i P_i (section "Expert-level balance loss"). */
float oracle_balance_loss(int n, const float *f, const float *P, float alpha) {
  float acc = 0.0f;
  for (int i = 0; i < n; ++i) acc += f[i] * P[i];
  return alpha * acc;
}

/*
 * Grouping of (token, slot) pairs by expert: a stable counting sort, expert
 * major and token ascending.  offsets [n+1]; perm_token [T*k] = token of each
 * grouped row; slot_of [T][k] = grouped row of (t, j).
 */
int oracle_permute(int64_t T, int n, int k, const int32_t *topk_idx, int32_t *offsets,
                   int32_t *perm_token, int32_t *slot_of) {
  int32_t *cursor = (int32_t *)calloc((size_t)n + 1, sizeof(int32_t));
  if (!cursor) return ORC_ERR_MEM;
  for (int64_t r = 0; r < T * k; ++r) {
    int e = topk_idx[r];
    if (e < 0 || e >= n) {
      free(cursor);
      return ORC_ERR_ARG;
    }
    cursor[e + 1] += 1;
  }
  for (int e = 0; e < n; ++e) cursor[e + 1] += cursor[e];
  memcpy(offsets, cursor, sizeof(int32_t) * ((size_t)n + 1));
  for (int64_t t = 0; t < T; ++t)
    for (int j = 0; j < k; ++j) {
      int e = topk_idx[(size_t)t * k + j];
      int32_t pos = cursor[e]++;
      perm_token[pos] = (int32_t)t;
      slot_of[(size_t)t * k + j] = pos;
    }
  free(cursor);
  return ORC_OK;
}

static float orc_silu(float z) { return z / (1.0f + expf(-z)); }

/*
 * One SwiGLU expert on one fp32 vector x [d]:
 *   a = W1 x, b = W3 x (W1, W3 rows of length d, row stride ldw13),
 *   hid = SiLU(a) * b,
 *   y = W2 hid (W2 rows of length d_ff, row stride ldw2).
 * Weights are read from dtype storage starting at element offsets o13 / o2.
 * hid is scratch of d_ff floats; y [d] is overwritten.
 */
static void orc_swiglu(int d, int d_ff, const float *x, const void *w1, const void *w3,
                       size_t o13, size_t ldw13, const void *w2, size_t o2, size_t ldw2,
                       int dtype, float *hid, float *y) {
  for (int c = 0; c < d_ff; ++c) {
    float a = 0.0f, b = 0.0f;
    for (int j = 0; j < d; ++j) {
      a += orc_get(w1, o13 + (size_t)c * ldw13 + j, dtype) * x[j];
      b += orc_get(w3, o13 + (size_t)c * ldw13 + j, dtype) * x[j];
    }
    hid[c] = orc_silu(a) * b;
  }
  for (int i = 0; i < d; ++i) {
    float acc = 0.0f;
    for (int c = 0; c < d_ff; ++c) acc += orc_get(w2, o2 + (size_t)i * ldw2 + c, dtype) * hid[c];
    y[i] = acc;
  }
}

/*
 * Routed expert e on x: w1, w3 [n][d_ff][d], w2 [n][d][d_ff].
 */
int oracle_expert(int d, int d_ff, int e, int dtype, const float *x, const void *w1,
                  const void *w3, const void *w2, float *y) {
  float *hid = (float *)malloc(sizeof(float) * (size_t)d_ff);
  if (!hid) return ORC_ERR_MEM;
  orc_swiglu(d, d_ff, x, w1, w3, (size_t)e * d_ff * d, (size_t)d, w2, (size_t)e * d * d_ff,
             (size_t)d_ff, dtype, hid, y);
  free(hid);
  return ORC_OK;
}

/*
 * Whole layer for a list of tokens (all T tokens are routed, since counts and
 * P need the full batch; the expert sums are formed only for the listed ones).
 *
 * Inputs (dtype storage): u [T][d], cent [n][d], routed w1, w3 [n][d_ff][d],
 * w2 [n][d][d_ff]; shared ws1, ws3 [K_s*d_ff][d], ws2 [d][K_s*d_ff] where
 * shared expert q owns rows (resp. columns) q*d_ff .. q*d_ff + d_ff - 1; the
 * shared expert sum is formed expert by expert.
 * toks [nt]: token indices (NULL: all T tokens in order, nt = T).
 * Outputs (all fp32, rows in toks order; any may be NULL except the routing
 * ones): topk_idx, topk_gate [T][k], counts, f, P [n];
 *   Y [nt][k][d]  ungated routed expert outputs per slot,
 *   S [nt][d]     shared expert sum,
 *   ysum [nt][d]  sum_j g_j Y_j + S,
 *   h [nt][d]     ysum + u.
 */
int oracle_layer(int64_t T, int d, int N, int m, int K, int K_s, int d_ff, int dtype,
                 const void *u, const void *cent, const void *w1, const void *w3,
                 const void *w2, const void *ws1, const void *ws3, const void *ws2,
                 const int64_t *toks, int64_t nt, int32_t *topk_idx, float *topk_gate,
                 int32_t *counts, float *f, float *P, float *Y, float *S, float *ysum,
                 float *h) {
  int n, k;
  if (oracle_sizes(N, m, K, K_s, &n, &k) != ORC_OK) return ORC_ERR_ARG;
  if (d < 1 || d_ff < 1 || (K_s > 0 && (!ws1 || !ws3 || !ws2))) return ORC_ERR_ARG;
  if (!toks) nt = T;
  int rc = oracle_route(T, d, n, k, dtype, u, cent, topk_idx, topk_gate, NULL, NULL, counts,
                        f, P);
  if (rc != ORC_OK) return rc;
  const size_t ldws2 = (size_t)K_s * d_ff;
  int fail = 0;
#pragma omp parallel
  {
    float *x = (float *)malloc(sizeof(float) * (size_t)d);
    float *hid = (float *)malloc(sizeof(float) * (size_t)d_ff);
    float *yk = (float *)malloc(sizeof(float) * (size_t)k * d);
    float *sh = (float *)malloc(sizeof(float) * (size_t)d);
    float *tmp = (float *)malloc(sizeof(float) * (size_t)d);
#pragma omp for schedule(dynamic, 1)
    for (int64_t r = 0; r < nt; ++r) {
      if (!x || !hid || !yk || !sh || !tmp) {
#pragma omp atomic write
        fail = 1;
        continue;
      }
      {
        int64_t t = toks ? toks[r] : r;
        for (int j = 0; j < d; ++j) x[j] = orc_get(u, (size_t)t * d + j, dtype);
        /* routed experts, ungated, in selection order */
        for (int j = 0; j < k; ++j) {
          int e = topk_idx[(size_t)t * k + j];
          orc_swiglu(d, d_ff, x, w1, w3, (size_t)e * d_ff * d, (size_t)d, w2,
                     (size_t)e * d * d_ff, (size_t)d_ff, dtype, hid, yk + (size_t)j * d);
        }
        /* shared experts, always on, weight one */
        for (int i = 0; i < d; ++i) sh[i] = 0.0f;
        for (int q = 0; q < K_s; ++q) {
          orc_swiglu(d, d_ff, x, ws1, ws3, (size_t)q * d_ff * d, (size_t)d, ws2,
                     (size_t)q * d_ff, ldws2, dtype, hid, tmp);
          for (int i = 0; i < d; ++i) sh[i] += tmp[i];
        }
        /* h = sum_j g_j FFN_j(u) + shared + u */
        for (int i = 0; i < d; ++i) {
          float acc = 0.0f;
          for (int j = 0; j < k; ++j) acc += topk_gate[(size_t)t * k + j] * yk[(size_t)j * d + i];
          acc += sh[i];
          if (ysum) ysum[(size_t)r * d + i] = acc;
          if (h) h[(size_t)r * d + i] = acc + x[i];
          if (S) S[(size_t)r * d + i] = sh[i];
        }
        if (Y) memcpy(Y + (size_t)r * k * d, yk, sizeof(float) * (size_t)k * d);
      }
    }
    free(x);
    free(hid);
    free(yk);
    free(sh);
    free(tmp);
  }
  return fail ? ORC_ERR_MEM : ORC_OK;
}

/*
 * Combine alone (section "Routing in a classic MoE layer"):
 *   h[t] = sum_j gate[t][j] * y_perm[slot_of[t][j]] + shared[t] + residual[t]
 * summed in fp32 (j ascending, then shared, then residual).  residual and
 * shared may be NULL.  y_perm [T*k][d] and the others in dtype storage; h fp32.
 */
int oracle_combine(int64_t T, int d, int k, int dtype, const void *residual, const void *shared,
                   const void *y_perm, const int32_t *slot_of, const float *gate, float *h) {
  if (T < 1 || d < 1 || k < 1) return ORC_ERR_ARG;
#pragma omp parallel for schedule(static)
  for (int64_t t = 0; t < T; ++t)
    for (int i = 0; i < d; ++i) {
      float acc = 0.0f;
      for (int j = 0; j < k; ++j)
        acc += gate[(size_t)t * k + j] *
               orc_get(y_perm, (size_t)slot_of[(size_t)t * k + j] * d + i, dtype);
      if (shared) acc += orc_get(shared, (size_t)t * d + i, dtype);
      if (residual) acc += orc_get(residual, (size_t)t * d + i, dtype);
      h[(size_t)t * d + i] = acc;
    }
  return ORC_OK;
}

/* ------------------------------------------------------------------------
 * Backward pass (fp64 arithmetic; inputs widened exactly).
 *
 * The quantity differentiated is the layer's output contracted with an
 * upstream gradient dh, plus the expert-level balance loss of section
 * "Expert-level balance loss" with coefficient alpha:
 *   L = sum_t <dh_t, h_t> + alpha * sum_i f_i P_i.
 * The kept set of every token and the counts behind f_i are piecewise
 * constant in the inputs, so they carry no gradient; the gates and P_i
 * carry it through the softmax.  Chain rule, written out:
 *   expert on x with gate g (g = 1 for a shared expert), upstream dh:
 *     a = W1 x, b = W3 x, hid = SiLU(a) * b,
 *     dhid = W2^T dh                 (ungated),
 *     dg   = <dhid, hid>             (= <dh, W2 hid>, the gate's gradient),
 *     da   = g dhid * b * SiLU'(a),  db = g dhid * SiLU(a),
 *     dx  += W1^T da + W3^T db,
 *     dW1 += da x^T, dW3 += db x^T, dW2 += (g dh) hid^T,
 *   SiLU'(z) = sigma(z) (1 + z (1 - sigma(z))), sigma the logistic function;
 *   ds_i = dg of the slot that kept i (0 if none) + alpha f_i / T,
 *   dl_i = s_i (ds_i - sum_j s_j ds_j)        (softmax),
 *   du  += dl^T E (router), de_i = sum_t dl_{t,i} u_t,
 *   du  += dh (residual) + dx of the kept and the shared experts.
 * ------------------------------------------------------------------------ */

#define ORC_BWD_NO_RESIDUAL 1
#define ORC_BWD_NO_SHARED 2

static double orc_sigmoid(double z) { return 1.0 / (1.0 + exp(-z)); }

/* Affinities of token t in fp64: l [n] logits, s [n] softmax. */
static void orc_scores64(const void *u, const void *cent, int64_t t, int d, int n, int dtype,
                         double *l, double *s) {
  double mx = 0.0, z = 0.0;
  for (int i = 0; i < n; ++i) {
    double acc = 0.0;
    for (int j = 0; j < d; ++j)
      acc += (double)orc_get(u, (size_t)t * d + j, dtype) *
             (double)orc_get(cent, (size_t)i * d + j, dtype);
    l[i] = acc;
    if (i == 0 || acc > mx) mx = acc;
  }
  for (int i = 0; i < n; ++i) {
    s[i] = exp(l[i] - mx);
    z += s[i];
  }
  for (int i = 0; i < n; ++i) s[i] /= z;
}

/*
 * One expert's forward pieces on x [d] and the gradient of its hidden layer:
 * a, b [d_ff]; hid [d_ff]; dhid = W2^T dy [d_ff] (dy [d], ungated).
 * Weights: W1/W3 rows of length d at o13 + c*ldw13; W2 row i at o2 + i*ldw2.
 */
static void orc_expert_fwd64(int d, int d_ff, const double *x, const void *w1, const void *w3,
                             size_t o13, size_t ldw13, const void *w2, size_t o2, size_t ldw2,
                             int dtype, const double *dy, double *a, double *b, double *hid,
                             double *dhid) {
  for (int c = 0; c < d_ff; ++c) {
    double sa = 0.0, sb = 0.0;
    for (int j = 0; j < d; ++j) {
      sa += (double)orc_get(w1, o13 + (size_t)c * ldw13 + j, dtype) * x[j];
      sb += (double)orc_get(w3, o13 + (size_t)c * ldw13 + j, dtype) * x[j];
    }
    a[c] = sa;
    b[c] = sb;
    hid[c] = sa * orc_sigmoid(sa) * sb;
  }
  /* dhid[c] = sum_i W2[i][c] dy[i], i ascending for every c (rows of W2 are
   * walked in storage order) */
  for (int c = 0; c < d_ff; ++c) dhid[c] = 0.0;
  for (int i = 0; i < d; ++i) {
    const double yi = dy[i];
    for (int c = 0; c < d_ff; ++c)
      dhid[c] += (double)orc_get(w2, o2 + (size_t)c + (size_t)i * ldw2, dtype) * yi;
  }
}

/* da, db of the SwiGLU from a, b, dhid and the gate g. */
static void orc_swiglu_bwd64(int d_ff, double g, const double *a, const double *b,
                             const double *dhid, double *da, double *db) {
  for (int c = 0; c < d_ff; ++c) {
    const double sg = orc_sigmoid(a[c]);
    const double silu = a[c] * sg;
    const double dsilu = sg * (1.0 + a[c] * (1.0 - sg));
    da[c] = g * dhid[c] * b[c] * dsilu;
    db[c] = g * dhid[c] * silu;
  }
}

/* dx += W1^T da + W3^T db: for every j the sum over c runs ascending into
 * acc [d] (scratch), which is then added to dx; rows of W1 and W3 are walked
 * in storage order. */
static void orc_dx64(int d, int d_ff, const void *w1, const void *w3, size_t o13, size_t ldw13,
                     int dtype, const double *da, const double *db, double *acc, double *dx) {
  for (int j = 0; j < d; ++j) acc[j] = 0.0;
  for (int c = 0; c < d_ff; ++c) {
    const double ac = da[c], bc = db[c];
    for (int j = 0; j < d; ++j)
      acc[j] += (double)orc_get(w1, o13 + (size_t)c * ldw13 + j, dtype) * ac +
                (double)orc_get(w3, o13 + (size_t)c * ldw13 + j, dtype) * bc;
  }
  for (int j = 0; j < d; ++j) dx[j] += acc[j];
}

/*
 * Weight gradients of one expert over its rows (ascending token order):
 * row r has input token tok[r], gate g[r] and upstream dh[tok[r]].
 * dw1, dw3 [d_ff][d] and dw2 [d][ldw2o] (columns 0 .. d_ff-1 written).
 */
static int orc_expert_wgrad64(int d, int d_ff, int64_t nr, const int64_t *tok, const double *g,
                              const void *u, const float *dh, const void *w1, const void *w3,
                              size_t o13, size_t ldw13, const void *w2, size_t o2, size_t ldw2,
                              int dtype, double *dw1, double *dw3, double *dw2, size_t ldw2o) {
  const size_t R = nr > 0 ? (size_t)nr : 1;
  double *X = (double *)malloc(sizeof(double) * R * d);
  double *DY = (double *)malloc(sizeof(double) * R * d);
  double *HID = (double *)malloc(sizeof(double) * R * d_ff);
  double *DA = (double *)malloc(sizeof(double) * R * d_ff);
  double *DB = (double *)malloc(sizeof(double) * R * d_ff);
  int fail = !X || !DY || !HID || !DA || !DB;
  if (!fail) {
#pragma omp parallel
    {
      double *a = (double *)malloc(sizeof(double) * (size_t)d_ff);
      double *b = (double *)malloc(sizeof(double) * (size_t)d_ff);
      double *dhid = (double *)malloc(sizeof(double) * (size_t)d_ff);
#pragma omp for schedule(dynamic, 4)
      for (int64_t r = 0; r < nr; ++r) {
        if (!a || !b || !dhid) {
#pragma omp atomic write
          fail = 1;
          continue;
        }
        double *x = X + (size_t)r * d, *dy = DY + (size_t)r * d;
        for (int j = 0; j < d; ++j) {
          x[j] = (double)orc_get(u, (size_t)tok[r] * d + j, dtype);
          dy[j] = g[r] * (double)dh[(size_t)tok[r] * d + j];
        }
        orc_expert_fwd64(d, d_ff, x, w1, w3, o13, ldw13, w2, o2, ldw2, dtype, dy, a, b,
                         HID + (size_t)r * d_ff, dhid);
        /* dy is gated already, so the SwiGLU backward takes gate one */
        orc_swiglu_bwd64(d_ff, 1.0, a, b, dhid, DA + (size_t)r * d_ff, DB + (size_t)r * d_ff);
      }
      free(a);
      free(b);
      free(dhid);
    }
  }
  if (!fail) {
    /* every output element sums its rows r in ascending order; the loops
     * over r run outside the contiguous column loops */
#pragma omp parallel for schedule(static)
    for (int c = 0; c < d_ff; ++c) {
      double *o1 = dw1 + (size_t)c * d, *o3 = dw3 + (size_t)c * d;
      for (int j = 0; j < d; ++j) o1[j] = o3[j] = 0.0;
      for (int64_t r = 0; r < nr; ++r) {
        const double a = DA[(size_t)r * d_ff + c], b = DB[(size_t)r * d_ff + c];
        const double *xr = X + (size_t)r * d;
        for (int j = 0; j < d; ++j) {
          o1[j] += a * xr[j];
          o3[j] += b * xr[j];
        }
      }
    }
#pragma omp parallel for schedule(static)
    for (int i = 0; i < d; ++i) {
      double *o2 = dw2 + (size_t)i * ldw2o;
      for (int c = 0; c < d_ff; ++c) o2[c] = 0.0;
      for (int64_t r = 0; r < nr; ++r) {
        const double y = DY[(size_t)r * d + i];
        const double *hr = HID + (size_t)r * d_ff;
        for (int c = 0; c < d_ff; ++c) o2[c] += y * hr[c];
      }
    }
  }
  free(X);
  free(DY);
  free(HID);
  free(DA);
  free(DB);
  return fail ? ORC_ERR_MEM : ORC_OK;
}

/*
 * Gradients of L.  Inputs as oracle_layer (dtype storage), plus the routing
 * the forward made (topk_idx [T][k] and f [n], as oracle_route returns them),
 * dh [T][d] fp32 and alpha.  flags: ORC_BWD_NO_RESIDUAL drops the residual
 * term of h, ORC_BWD_NO_SHARED the shared experts.  Outputs (fp64, each may
 * be NULL to skip it):
 *   du [nt][d]        rows of the tokens toks[0..nt) (all tokens if toks NULL)
 *   dcent [n][d]      needs every token's softmax gradient
 *   dw1, dw3 [ne][d_ff][d], dw2 [ne][d][d_ff]   experts[0..ne)
 *   dws1, dws3 [K_s*d_ff][d], dws2 [d][K_s*d_ff] shared experts
 */
int oracle_layer_bwd(int64_t T, int d, int N, int m, int K, int K_s, int d_ff, int dtype,
                     const void *u, const void *cent, const void *w1, const void *w3,
                     const void *w2, const void *ws1, const void *ws3, const void *ws2,
                     const int32_t *topk_idx, const float *f, const float *dh, double alpha,
                     int flags, const int64_t *toks, int64_t nt, double *du, double *dcent,
                     const int32_t *experts, int ne, double *dw1, double *dw3, double *dw2,
                     double *dws1, double *dws3, double *dws2) {
  int n, k;
  if (oracle_sizes(N, m, K, K_s, &n, &k) != ORC_OK) return ORC_ERR_ARG;
  const int shared = K_s > 0 && !(flags & ORC_BWD_NO_SHARED);
  if (T < 1 || d < 1 || d_ff < 1 || (shared && (!ws1 || !ws3 || !ws2))) return ORC_ERR_ARG;
  if (!toks) nt = T;
  const size_t ldws2 = (size_t)K_s * d_ff;
  int fail = 0;

  /* Per-token part: softmax gradient (all tokens when dcent is wanted) and du. */
  double *DL = NULL;
  if (dcent) {
    DL = (double *)malloc(sizeof(double) * (size_t)T * n);
    if (!DL) return ORC_ERR_MEM;
  }
  const int64_t nrow = dcent ? T : (du ? nt : 0);
#pragma omp parallel
  {
    double *x = (double *)malloc(sizeof(double) * (size_t)d);
    double *dy = (double *)malloc(sizeof(double) * (size_t)d);
    double *dx = (double *)malloc(sizeof(double) * (size_t)d);
    double *l = (double *)malloc(sizeof(double) * (size_t)n);
    double *s = (double *)malloc(sizeof(double) * (size_t)n);
    double *ds = (double *)malloc(sizeof(double) * (size_t)n);
    double *a = (double *)malloc(sizeof(double) * (size_t)d_ff);
    double *b = (double *)malloc(sizeof(double) * (size_t)d_ff);
    double *hid = (double *)malloc(sizeof(double) * (size_t)d_ff);
    double *dhid = (double *)malloc(sizeof(double) * (size_t)d_ff);
    double *da = (double *)malloc(sizeof(double) * (size_t)d_ff);
    double *db = (double *)malloc(sizeof(double) * (size_t)d_ff);
    double *dxe = (double *)malloc(sizeof(double) * (size_t)d);
#pragma omp for schedule(dynamic, 1)
    for (int64_t r = 0; r < nrow; ++r) {
      if (!x || !dy || !dx || !l || !s || !ds || !a || !b || !hid || !dhid || !da || !db ||
          !dxe) {
#pragma omp atomic write
        fail = 1;
        continue;
      }
      /* token of this row; when every token is visited, du rows are looked up later */
      const int64_t t = dcent ? r : (toks ? toks[r] : r);
      for (int j = 0; j < d; ++j) {
        x[j] = (double)orc_get(u, (size_t)t * d + j, dtype);
        dy[j] = (double)dh[(size_t)t * d + j];
        dx[j] = (flags & ORC_BWD_NO_RESIDUAL) ? 0.0 : dy[j];
      }
      orc_scores64(u, cent, t, d, n, dtype, l, s);
      for (int i = 0; i < n; ++i) ds[i] = alpha * (double)f[i] / (double)T;
      /* kept experts: gate gradient and input gradient */
      for (int j = 0; j < k; ++j) {
        const int e = topk_idx[(size_t)t * k + j];
        const double g = s[e];
        orc_expert_fwd64(d, d_ff, x, w1, w3, (size_t)e * d_ff * d, (size_t)d, w2,
                         (size_t)e * d * d_ff, (size_t)d_ff, dtype, dy, a, b, hid, dhid);
        double dg = 0.0;
        for (int c = 0; c < d_ff; ++c) dg += dhid[c] * hid[c];
        ds[e] += dg;
        orc_swiglu_bwd64(d_ff, g, a, b, dhid, da, db);
        orc_dx64(d, d_ff, w1, w3, (size_t)e * d_ff * d, (size_t)d, dtype, da, db, dxe, dx);
      }
      /* shared experts, weight one */
      for (int q = 0; shared && q < K_s; ++q) {
        orc_expert_fwd64(d, d_ff, x, ws1, ws3, (size_t)q * d_ff * d, (size_t)d, ws2,
                         (size_t)q * d_ff, ldws2, dtype, dy, a, b, hid, dhid);
        orc_swiglu_bwd64(d_ff, 1.0, a, b, dhid, da, db);
        orc_dx64(d, d_ff, ws1, ws3, (size_t)q * d_ff * d, (size_t)d, dtype, da, db, dxe, dx);
      }
      /* softmax backward, then the router's share of du */
      double sds = 0.0;
      for (int i = 0; i < n; ++i) sds += s[i] * ds[i];
      for (int i = 0; i < n; ++i) {
        const double dl = s[i] * (ds[i] - sds);
        if (DL) DL[(size_t)t * n + i] = dl;
        for (int j = 0; j < d; ++j) dx[j] += dl * (double)orc_get(cent, (size_t)i * d + j, dtype);
      }
      if (du && !dcent) memcpy(du + (size_t)r * d, dx, sizeof(double) * (size_t)d);
      if (du && dcent) {
        /* every token visited: keep the rows the caller listed */
        if (!toks) {
          memcpy(du + (size_t)t * d, dx, sizeof(double) * (size_t)d);
        } else {
          for (int64_t q = 0; q < nt; ++q)
            if (toks[q] == t) memcpy(du + (size_t)q * d, dx, sizeof(double) * (size_t)d);
        }
      }
    }
    free(x);
    free(dy);
    free(dx);
    free(l);
    free(s);
    free(ds);
    free(a);
    free(b);
    free(hid);
    free(dhid);
    free(da);
    free(db);
    free(dxe);
  }
  if (fail) {
    free(DL);
    return ORC_ERR_MEM;
  }
  if (dcent) {
    /* dcent[i][j] sums over t ascending */
#pragma omp parallel for schedule(static)
    for (int i = 0; i < n; ++i) {
      double *o = dcent + (size_t)i * d;
      for (int j = 0; j < d; ++j) o[j] = 0.0;
      for (int64_t t = 0; t < T; ++t) {
        const double dl = DL[(size_t)t * n + i];
        for (int j = 0; j < d; ++j) o[j] += dl * (double)orc_get(u, (size_t)t * d + j, dtype);
      }
    }
    free(DL);
  }

  /* Routed experts' weight gradients: rows = tokens that kept the expert. */
  if (ne > 0 && (dw1 || dw3 || dw2)) {
    if (!dw1 || !dw3 || !dw2 || !experts) return ORC_ERR_ARG;
    int64_t *tok = (int64_t *)malloc(sizeof(int64_t) * (size_t)T);
    double *g = (double *)malloc(sizeof(double) * (size_t)T);
    double *l = (double *)malloc(sizeof(double) * (size_t)n);
    double *s = (double *)malloc(sizeof(double) * (size_t)n);
    if (!tok || !g || !l || !s) fail = 1;
    for (int q = 0; !fail && q < ne; ++q) {
      const int e = experts[q];
      if (e < 0 || e >= n) {
        fail = 2;
        break;
      }
      int64_t nr = 0;
      for (int64_t t = 0; t < T; ++t)
        for (int j = 0; j < k; ++j)
          if (topk_idx[(size_t)t * k + j] == e) {
            orc_scores64(u, cent, t, d, n, dtype, l, s);
            tok[nr] = t;
            g[nr] = s[e];
            ++nr;
          }
      int rc = orc_expert_wgrad64(d, d_ff, nr, tok, g, u, dh, w1, w3, (size_t)e * d_ff * d,
                                  (size_t)d, w2, (size_t)e * d * d_ff, (size_t)d_ff, dtype,
                                  dw1 + (size_t)q * d_ff * d, dw3 + (size_t)q * d_ff * d,
                                  dw2 + (size_t)q * d * d_ff, (size_t)d_ff);
      if (rc != ORC_OK) fail = 1;
    }
    free(tok);
    free(g);
    free(l);
    free(s);
    if (fail) return fail == 2 ? ORC_ERR_ARG : ORC_ERR_MEM;
  }

  /* Shared experts: every token, gate one, expert by expert. */
  if (shared && (dws1 || dws3 || dws2)) {
    if (!dws1 || !dws3 || !dws2) return ORC_ERR_ARG;
    int64_t *tok = (int64_t *)malloc(sizeof(int64_t) * (size_t)T);
    double *g = (double *)malloc(sizeof(double) * (size_t)T);
    if (!tok || !g) fail = 1;
    for (int64_t t = 0; !fail && t < T; ++t) {
      tok[t] = t;
      g[t] = 1.0;
    }
    for (int q = 0; !fail && q < K_s; ++q) {
      int rc = orc_expert_wgrad64(d, d_ff, T, tok, g, u, dh, ws1, ws3, (size_t)q * d_ff * d,
                                  (size_t)d, ws2, (size_t)q * d_ff, ldws2, dtype,
                                  dws1 + (size_t)q * d_ff * d, dws3 + (size_t)q * d_ff * d,
                                  dws2 + (size_t)q * d_ff, ldws2);
      if (rc != ORC_OK) fail = 1;
    }
    free(tok);
    free(g);
    if (fail) return ORC_ERR_MEM;
  }
  return ORC_OK;
}

#ifdef _OPENMP
#include <omp.h>
#endif
/* Threads the oracle's parallel loops use. */
int oracle_threads(void) {
#ifdef _OPENMP
  return omp_get_max_threads();
#else
  return 1;
#endif
}
