/*
 * hsa_oracle.c -- plain fp64 CPU oracle for the Hierarchical Sparse Attention
 * (HSA) forward step.
 *
 * TEST INFRASTRUCTURE ONLY.  This file is the reference the HIP library is
 * checked against.  Only the tests, the smoke check and the benchmark's CPU
 * baseline leg may load it; the library never calls it and shares no code,
 * header, table or helper with it.
 *
 * Source: "Every Token Counts: Generalizing 16M Ultra-Long Context in LLMs",
 * agent-atlas explainer page, section "How It Works (Technically)":
 *   Step 1  chunks of S = 64 tokens, one landmark per chunk;
 *   Step 2  retrieval score  s[t,i] = (Q_slc[t] . K_slc[i]) / sqrt(d) for chunks
 *           before t, -inf for the rest; keep the K best chunks (I_t);
 *   Step 3  attend inside each selected chunk separately:
 *           O[t,i] = softmax(norm(Q_attn[t]) . norm(K[i])^T / sqrt(d_h)) V[i],
 *           norm = L2 normalisation (query-key normalisation);
 *   Step 4  w[t,i] = softmax of s over the selected chunks,
 *           O_t = sum_i w[t,i] O[t,i];
 * and section "The algorithm, simplified" (the hsa_step sketch): a stable
 * descending sort picks the chunks, so equal scores keep chunk order, and an
 * empty selection sums to zero.
 *
 * Readings taken where the page leaves a step open (each one is listed in the
 * design notes of the repository):
 *   - a chunk is eligible for the token at absolute position p only if it lies
 *     entirely before p's own chunk: chunks 0 .. min(p/64, Nc)-1;
 *   - fewer eligible chunks than K: all eligible chunks are used; unused
 *     output slots hold index -1 and score -inf;
 *   - no eligible chunk: the output is 0 (the empty sum);
 *   - ranking uses the unscaled dot product (raw); ties go to the lower chunk
 *     index, i.e. the order is (raw descending, index ascending);
 *   - GQA: one retrieval query and one landmark set per kv head; scores,
 *     selection and blend weights are shared by the q heads of that group;
 *   - query-key normalisation x / max(||x||_2, 1e-6), applied to the attention
 *     query and to every key when qk_norm is set, never on the retrieval path;
 *   - ret_scale and attn_scale are explicit arguments (1/sqrt(d) by default in
 *     the caller).
 *
 * Arithmetic: every value is the exact stored fp32/bf16 value widened to fp64;
 * every reduction runs in plain index order, so results do not depend on the
 * number of threads.  OpenMP only splits independent query rows.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

#define ORC_CHUNK 64
#define ORC_NORM_EPS 1e-6

enum { ORC_OK = 0, ORC_BAD_ARGS = 1, ORC_NO_MEMORY = 2 };

typedef struct {
  int64_t B, Lq, q_pos0, Lkv, Hq, Hkv, d, K, Nc;
  double ret_scale, attn_scale;
  int qk_norm, is_bf16;
  const void *q_ret, *landmarks, *q_attn, *k, *v;
} orc_problem;

/* Exact widening of one stored element. */
static double elem(const void* base, int64_t i, int is_bf16) {
  if (is_bf16) {
    uint32_t u = ((uint32_t)((const uint16_t*)base)[i]) << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return (double)f;
  }
  return (double)((const float*)base)[i];
}

typedef struct {
  double raw;
  int64_t idx;
} orc_cand;

/* Total order of the selection: raw descending, then chunk index ascending. */
static int cand_order(const void* a, const void* b) {
  const orc_cand* x = (const orc_cand*)a;
  const orc_cand* y = (const orc_cand*)b;
  if (x->raw > y->raw) return -1;
  if (x->raw < y->raw) return 1;
  if (x->idx < y->idx) return -1;
  if (x->idx > y->idx) return 1;
  return 0;
}

static int64_t eligible_chunks(const orc_problem* P, int64_t r) {
  int64_t pos = P->q_pos0 + r;
  int64_t n = pos / ORC_CHUNK;
  return n < P->Nc ? n : P->Nc;
}

/* Step 2: raw retrieval score of chunk c for (b, r, g). */
static double raw_score(const orc_problem* P, int64_t b, int64_t r, int64_t g, int64_t c) {
  const int64_t d = P->d;
  const int64_t qo = ((b * P->Lq + r) * P->Hkv + g) * d;
  const int64_t lo = ((b * P->Hkv + g) * P->Nc + c) * d;
  double acc = 0.0;
  for (int64_t x = 0; x < d; ++x)
    acc += elem(P->q_ret, qo + x, P->is_bf16) * elem(P->landmarks, lo + x, P->is_bf16);
  return acc;
}

/* Step 3: softmax attention of one q head inside one chunk c (kv head g).
 * qhat holds the (optionally normalised) attention query; result in o[d]. */
static void chunk_attention(const orc_problem* P, int64_t b, int64_t g, int64_t c,
                            const double* qhat, double* o) {
  const int64_t d = P->d;
  double logit[ORC_CHUNK];
  for (int64_t t = 0; t < ORC_CHUNK; ++t) {
    const int64_t ko = ((b * P->Hkv + g) * P->Lkv + c * ORC_CHUNK + t) * d;
    double kn = 1.0;
    if (P->qk_norm) {
      double ss = 0.0;
      for (int64_t x = 0; x < d; ++x) {
        double kv = elem(P->k, ko + x, P->is_bf16);
        ss += kv * kv;
      }
      kn = sqrt(ss);
      if (kn < ORC_NORM_EPS) kn = ORC_NORM_EPS;
    }
    double dot = 0.0;
    for (int64_t x = 0; x < d; ++x) dot += qhat[x] * (elem(P->k, ko + x, P->is_bf16) / kn);
    logit[t] = dot * P->attn_scale;
  }
  double mu = logit[0];
  for (int64_t t = 1; t < ORC_CHUNK; ++t)
    if (logit[t] > mu) mu = logit[t];
  double denom = 0.0, p[ORC_CHUNK];
  for (int64_t t = 0; t < ORC_CHUNK; ++t) {
    p[t] = exp(logit[t] - mu);
    denom += p[t];
  }
  for (int64_t x = 0; x < d; ++x) o[x] = 0.0;
  for (int64_t t = 0; t < ORC_CHUNK; ++t) {
    const double pt = p[t] / denom;
    const int64_t vo = ((b * P->Hkv + g) * P->Lkv + c * ORC_CHUNK + t) * d;
    for (int64_t x = 0; x < d; ++x) o[x] += pt * elem(P->v, vo + x, P->is_bf16);
  }
}

/* Step 4, weights: w_k = exp(s_k - max s) / sum_j exp(s_j - max s) over the
 * used slots (index in [0, Nc)); unused slots get 0.  Returns 0 when no slot
 * is used (the empty selection). */
static int blend_weights(const orc_problem* P, const int32_t* idx, const double* score,
                         double* w) {
  const int64_t K = P->K;
  int any = 0;
  double m = 0.0;
  for (int64_t k = 0; k < K; ++k) {
    w[k] = 0.0;
    if (idx[k] < 0 || idx[k] >= P->Nc) continue;
    if (!any || score[k] > m) m = score[k];
    any = 1;
  }
  if (!any) return 0;
  double denom = 0.0;
  for (int64_t k = 0; k < K; ++k) {
    if (idx[k] < 0 || idx[k] >= P->Nc) continue;
    w[k] = exp(score[k] - m);
    denom += w[k];
  }
  for (int64_t k = 0; k < K; ++k) w[k] /= denom;
  return 1;
}

/* Step 4, output: for each q head of group g, the weighted sum of its
 * per-chunk attentions.  out_row points at out[row, g*G, 0]. */
static void blend_group(const orc_problem* P, int64_t b, int64_t r, int64_t g,
                        const int32_t* idx, const double* w, int any, double* out_row,
                        double* qhat, double* obar) {
  const int64_t d = P->d, K = P->K, G = P->Hq / P->Hkv;
  for (int64_t j = 0; j < G * d; ++j) out_row[j] = 0.0;
  if (!any) return; /* the empty sum */
  for (int64_t j = 0; j < G; ++j) {
    const int64_t h = g * G + j;
    const int64_t qo = ((b * P->Lq + r) * P->Hq + h) * d;
    double qn = 1.0;
    if (P->qk_norm) {
      double ss = 0.0;
      for (int64_t x = 0; x < d; ++x) {
        double qv = elem(P->q_attn, qo + x, P->is_bf16);
        ss += qv * qv;
      }
      qn = sqrt(ss);
      if (qn < ORC_NORM_EPS) qn = ORC_NORM_EPS;
    }
    for (int64_t x = 0; x < d; ++x) qhat[x] = elem(P->q_attn, qo + x, P->is_bf16) / qn;
    for (int64_t k = 0; k < K; ++k) {
      if (idx[k] < 0 || idx[k] >= P->Nc) continue;
      chunk_attention(P, b, g, idx[k], qhat, obar);
      for (int64_t x = 0; x < d; ++x) out_row[j * d + x] += w[k] * obar[x];
    }
  }
}

/* Steps 2 and the selection for one (b, r, g): fills idx/score (length K). */
static int select_group(const orc_problem* P, int64_t b, int64_t r, int64_t g,
                        orc_cand* cand, int32_t* idx, double* score) {
  const int64_t n = eligible_chunks(P, r);
  for (int64_t c = 0; c < n; ++c) {
    cand[c].raw = raw_score(P, b, r, g, c);
    cand[c].idx = c;
  }
  qsort(cand, (size_t)n, sizeof(orc_cand), cand_order);
  const int64_t keff = n < P->K ? n : P->K;
  for (int64_t k = 0; k < P->K; ++k) {
    if (k < keff) {
      idx[k] = (int32_t)cand[k].idx;
      score[k] = cand[k].raw * P->ret_scale;
    } else {
      idx[k] = -1;
      score[k] = -INFINITY;
    }
  }
  return ORC_OK;
}

static int check(const orc_problem* P) {
  if (P->B < 1 || P->Lq < 1 || P->Hq < 1 || P->Hkv < 1 || P->d < 1 || P->K < 1) return ORC_BAD_ARGS;
  if (P->Hq % P->Hkv) return ORC_BAD_ARGS;
  if (P->q_pos0 < 0 || P->Lkv < 0 || P->Nc != P->Lkv / ORC_CHUNK) return ORC_BAD_ARGS;
  return ORC_OK;
}

static orc_problem make_problem(int64_t B, int64_t Lq, int64_t q_pos0, int64_t Lkv, int64_t Hq,
                                int64_t Hkv, int64_t d, int64_t K, double ret_scale,
                                double attn_scale, int qk_norm, int is_bf16, const void* q_ret,
                                const void* landmarks, const void* q_attn, const void* k,
                                const void* v) {
  orc_problem P;
  P.B = B; P.Lq = Lq; P.q_pos0 = q_pos0; P.Lkv = Lkv; P.Hq = Hq; P.Hkv = Hkv;
  P.d = d; P.K = K; P.Nc = Lkv / ORC_CHUNK;
  P.ret_scale = ret_scale; P.attn_scale = attn_scale;
  P.qk_norm = qk_norm; P.is_bf16 = is_bf16;
  P.q_ret = q_ret; P.landmarks = landmarks; P.q_attn = q_attn; P.k = k; P.v = v;
  return P;
}

/*
 * Full forward for a list of query rows.  rows[i] = b*Lq + r (flat row id);
 * rows == NULL means every row in order.  Outputs are packed per listed row:
 *   topk_idx   [n_rows, Hkv, K] int32
 *   topk_score [n_rows, Hkv, K] fp64   (s = raw * ret_scale)
 *   weights    [n_rows, Hkv, K] fp64   (may be NULL)
 *   out        [n_rows, Hq, d]  fp64   (may be NULL: selection only)
 */
int hsa_oracle_forward(int64_t B, int64_t Lq, int64_t q_pos0, int64_t Lkv, int64_t Hq,
                       int64_t Hkv, int64_t d, int64_t K, double ret_scale, double attn_scale,
                       int qk_norm, int is_bf16, const void* q_ret, const void* landmarks,
                       const void* q_attn, const void* k, const void* v, const int64_t* rows,
                       int64_t n_rows, int32_t* topk_idx, double* topk_score, double* weights,
                       double* out) {
  orc_problem P = make_problem(B, Lq, q_pos0, Lkv, Hq, Hkv, d, K, ret_scale, attn_scale, qk_norm,
                               is_bf16, q_ret, landmarks, q_attn, k, v);
  if (check(&P)) return ORC_BAD_ARGS;
  if (!rows) n_rows = B * Lq;
  int status = ORC_OK;
#pragma omp parallel
  {
    orc_cand* cand = (orc_cand*)malloc(sizeof(orc_cand) * (size_t)(P.Nc > 0 ? P.Nc : 1));
    double* qhat = (double*)malloc(sizeof(double) * (size_t)d);
    double* obar = (double*)malloc(sizeof(double) * (size_t)d);
    double* wtmp = (double*)malloc(sizeof(double) * (size_t)K);
    if (!cand || !qhat || !obar || !wtmp) {
#pragma omp atomic write
      status = ORC_NO_MEMORY;
    } else {
#pragma omp for schedule(dynamic, 1)
      for (int64_t i = 0; i < n_rows; ++i) {
        const int64_t flat = rows ? rows[i] : i;
        const int64_t b = flat / Lq, r = flat % Lq;
        for (int64_t g = 0; g < Hkv; ++g) {
          int32_t* ix = topk_idx + (i * Hkv + g) * K;
          double* sc = topk_score + (i * Hkv + g) * K;
          select_group(&P, b, r, g, cand, ix, sc);
          double* w = weights ? weights + (i * Hkv + g) * K : wtmp;
          const int any = blend_weights(&P, ix, sc, w);
          if (out)
            blend_group(&P, b, r, g, ix, w, any, out + (i * Hq + g * (Hq / Hkv)) * d, qhat, obar);
        }
      }
    }
    free(cand);
    free(qhat);
    free(obar);
    free(wtmp);
  }
  return status;
}

/*
 * Steps 3-4 only, for a caller-given selection (same packing as above):
 *   topk_idx, topk_score [n_rows, Hkv, K]; slots whose index is outside
 *   [0, Nc) are unused.  Writes weights (may be NULL) and out [n_rows, Hq, d].
 */
int hsa_oracle_attend_blend(int64_t B, int64_t Lq, int64_t Lkv, int64_t Hq, int64_t Hkv,
                            int64_t d, int64_t K, double attn_scale, int qk_norm, int is_bf16,
                            const void* q_attn, const void* k, const void* v,
                            const int32_t* topk_idx, const double* topk_score,
                            const int64_t* rows, int64_t n_rows, double* weights, double* out) {
  orc_problem P = make_problem(B, Lq, 0, Lkv, Hq, Hkv, d, K, 1.0, attn_scale, qk_norm, is_bf16,
                               NULL, NULL, q_attn, k, v);
  if (check(&P)) return ORC_BAD_ARGS;
  if (!rows) n_rows = B * Lq;
  int status = ORC_OK;
#pragma omp parallel
  {
    double* qhat = (double*)malloc(sizeof(double) * (size_t)d);
    double* obar = (double*)malloc(sizeof(double) * (size_t)d);
    double* wtmp = (double*)malloc(sizeof(double) * (size_t)K);
    if (!qhat || !obar || !wtmp) {
#pragma omp atomic write
      status = ORC_NO_MEMORY;
    } else {
#pragma omp for schedule(dynamic, 1)
      for (int64_t i = 0; i < n_rows; ++i) {
        const int64_t flat = rows ? rows[i] : i;
        const int64_t b = flat / Lq, r = flat % Lq;
        for (int64_t g = 0; g < Hkv; ++g) {
          const int32_t* ix = topk_idx + (i * Hkv + g) * K;
          const double* sc = topk_score + (i * Hkv + g) * K;
          double* w = weights ? weights + (i * Hkv + g) * K : wtmp;
          const int any = blend_weights(&P, ix, sc, w);
          blend_group(&P, b, r, g, ix, w, any, out + (i * Hq + g * (Hq / Hkv)) * d, qhat, obar);
        }
      }
    }
    free(qhat);
    free(obar);
    free(wtmp);
  }
  return status;
}

/* Raw scores of every chunk for one (row, kv head): raw[c] for c < n(p),
 * NaN for chunks that are not eligible.  Returns n(p), or -1 on bad args. */
int64_t hsa_oracle_raw_scores(int64_t B, int64_t Lq, int64_t q_pos0, int64_t Lkv, int64_t Hkv,
                              int64_t d, int is_bf16, const void* q_ret, const void* landmarks,
                              int64_t flat_row, int64_t g, double* raw) {
  orc_problem P = make_problem(B, Lq, q_pos0, Lkv, Hkv, Hkv, d, 1, 1.0, 1.0, 0, is_bf16, q_ret,
                               landmarks, NULL, NULL, NULL);
  if (check(&P) || flat_row < 0 || flat_row >= B * Lq || g < 0 || g >= Hkv) return -1;
  const int64_t b = flat_row / Lq, r = flat_row % Lq;
  const int64_t n = eligible_chunks(&P, r);
  for (int64_t c = 0; c < P.Nc; ++c) raw[c] = c < n ? raw_score(&P, b, r, g, c) : NAN;
  return n;
}

/* Gradient of x_hat = x / max(||x||, eps) (the query-key normalisation):
 * with n = ||x|| > eps, dx = (dxh - xh (xh . dxh)) / n; below eps the divisor
 * is the constant eps and dx = dxh / eps. */
static void norm_backward(const double* x, int64_t d, const double* dxh, double* dx) {
  double ss = 0.0;
  for (int64_t i = 0; i < d; ++i) ss += x[i] * x[i];
  const double n = sqrt(ss);
  if (n <= ORC_NORM_EPS) {
    for (int64_t i = 0; i < d; ++i) dx[i] = dxh[i] / ORC_NORM_EPS;
    return;
  }
  double dot = 0.0;
  for (int64_t i = 0; i < d; ++i) dot += (x[i] / n) * dxh[i];
  for (int64_t i = 0; i < d; ++i) dx[i] = (dxh[i] - (x[i] / n) * dot) / n;
}

/*
 * HSA backward for a given selection: the gradients of sum(out * dout) with
 * respect to every input of Steps 2-4.  The selection itself is discrete and
 * carries no gradient; the gradient reaches the retrieval path through the
 * blend weights w = softmax(s) (Step 4) and s = ret_scale * (q_ret . landmark)
 * (Step 2), and the attention path through each chunk's softmax attention
 * with the query-key normalisation (Step 3).  For one (b, r, g):
 *   dw_k  = sum_h dout_h . O_k[h]          ds_k = w_k (dw_k - sum_j w_j dw_j)
 *   dq_ret += ret_scale ds_k landmark[c_k]  dlandmark[c_k] += ret_scale ds_k q_ret
 * and per head h and slot k, with P the in-chunk softmax and dO_k = w_k dout_h:
 *   dv_t += P_t dO_k    dP_t = dO_k . v_t    dz_t = P_t (dP_t - sum_u P_u dP_u)
 *   dqhat += attn_scale sum_t dz_t khat_t    dkhat_t += attn_scale dz_t qhat
 * followed by the normalisation's gradient (norm_backward).  score is the
 * given s of each slot (as hsa_oracle_attend_blend); idx as there.
 * Outputs (fp64, overwritten): dq_ret [B,Lq,Hkv,d], dlm [B,Hkv,Nc,d],
 * dq_attn [B,Lq,Hq,d], dk and dv [B,Hkv,Lkv,d].  Accumulation runs over rows
 * in index order inside each (b, g), so results do not depend on threads.
 */
int hsa_oracle_backward(int64_t B, int64_t Lq, int64_t Lkv, int64_t Hq, int64_t Hkv, int64_t d,
                        int64_t K, double ret_scale, double attn_scale, int qk_norm, int is_bf16,
                        const void* q_ret, const void* landmarks, const void* q_attn, const void* k,
                        const void* v, const void* dout, const int32_t* idx, const double* score,
                        double* dq_ret, double* dlm, double* dq_attn, double* dk, double* dv) {
  orc_problem P = make_problem(B, Lq, 0, Lkv, Hq, Hkv, d, K, ret_scale, attn_scale, qk_norm, is_bf16,
                               q_ret, landmarks, q_attn, k, v);
  if (check(&P) != ORC_OK || !dout || !idx || !score || !dq_ret || !dlm || !dq_attn || !dk || !dv)
    return ORC_BAD_ARGS;
  const int64_t G = Hq / Hkv, Nc = P.Nc;
  int status = ORC_OK;
#pragma omp parallel for schedule(dynamic)
  for (int64_t bg = 0; bg < B * Hkv; ++bg) {
    const int64_t b = bg / Hkv, g = bg % Hkv;
    double* dkh = calloc((size_t)(Lkv * d + 1), sizeof(double));      /* d khat, before the norm */
    double* w = malloc(sizeof(double) * (size_t)K);
    double* wdw = malloc(sizeof(double) * (size_t)K);
    double* buf = malloc(sizeof(double) * (size_t)(8 * d + 4 * ORC_CHUNK));
    if (!dkh || !w || !wdw || !buf) {
#pragma omp critical
      status = ORC_NO_MEMORY;
      free(dkh); free(w); free(wdw); free(buf);
      continue;
    }
    double *q = buf, *qh = buf + d, *dqh = buf + 2 * d, *dq = buf + 3 * d, *dob = buf + 4 * d;
    double *kh = buf + 5 * d, *vt = buf + 6 * d, *tmp = buf + 7 * d;
    double *pr = buf + 8 * d, *dp = pr + ORC_CHUNK, *kn = dp + ORC_CHUNK;
    double* dv_bg = dv + bg * Lkv * d;
    double* dlm_bg = dlm + bg * Nc * d;
    for (int64_t i = 0; i < Lkv * d; ++i) dv_bg[i] = 0.0;
    for (int64_t i = 0; i < Nc * d; ++i) dlm_bg[i] = 0.0;
    for (int64_t r = 0; r < Lq; ++r) {
      const int64_t srow = (b * Lq + r) * Hkv + g;
      const int32_t* ix = idx + srow * K;
      const int any = blend_weights(&P, ix, score + srow * K, w);
      double* dqr = dq_ret + srow * d;
      for (int64_t x = 0; x < d; ++x) dqr[x] = 0.0;
      for (int64_t kk = 0; kk < K; ++kk) wdw[kk] = 0.0;
      for (int64_t j = 0; j < G; ++j) {
        const int64_t h = g * G + j;
        const int64_t qo = ((b * Lq + r) * Hq + h) * d;
        double ss = 0.0;
        for (int64_t x = 0; x < d; ++x) {
          q[x] = elem(q_attn, qo + x, is_bf16);
          ss += q[x] * q[x];
        }
        double qn = 1.0;
        if (qk_norm) {
          qn = sqrt(ss);
          if (qn < ORC_NORM_EPS) qn = ORC_NORM_EPS;
        }
        for (int64_t x = 0; x < d; ++x) {
          qh[x] = q[x] / qn;
          dqh[x] = 0.0;
        }
        for (int64_t kk = 0; kk < K && any; ++kk) {
          const int64_t c = ix[kk];
          if (c < 0 || c >= Nc) continue;
          /* in-chunk softmax (Step 3), recomputed */
          double mu = -INFINITY;
          for (int64_t t = 0; t < ORC_CHUNK; ++t) {
            const int64_t ko = (bg * Lkv + c * ORC_CHUNK + t) * d;
            double kss = 0.0;
            for (int64_t x = 0; x < d; ++x) {
              const double kv = elem(k, ko + x, is_bf16);
              kss += kv * kv;
            }
            kn[t] = 1.0;
            if (qk_norm) {
              kn[t] = sqrt(kss);
              if (kn[t] < ORC_NORM_EPS) kn[t] = ORC_NORM_EPS;
            }
            double dot = 0.0;
            for (int64_t x = 0; x < d; ++x) dot += qh[x] * (elem(k, ko + x, is_bf16) / kn[t]);
            pr[t] = dot * attn_scale;
            if (pr[t] > mu) mu = pr[t];
          }
          double den = 0.0;
          for (int64_t t = 0; t < ORC_CHUNK; ++t) {
            pr[t] = exp(pr[t] - mu);
            den += pr[t];
          }
          for (int64_t t = 0; t < ORC_CHUNK; ++t) pr[t] /= den;
          /* dO_k = w_k dout_h */
          const int64_t oo = ((b * Lq + r) * Hq + h) * d;
          for (int64_t x = 0; x < d; ++x) dob[x] = w[kk] * elem(dout, oo + x, is_bf16);
          double pdp = 0.0;
          for (int64_t t = 0; t < ORC_CHUNK; ++t) {
            const int64_t vo = (bg * Lkv + c * ORC_CHUNK + t) * d;
            double acc = 0.0;
            for (int64_t x = 0; x < d; ++x) {
              vt[x] = elem(v, vo + x, is_bf16);
              acc += dob[x] * vt[x];
              dv_bg[(c * ORC_CHUNK + t) * d + x] += pr[t] * dob[x];
            }
            dp[t] = acc;
            pdp += pr[t] * acc;
          }
          wdw[kk] += pdp;                    /* w_k (dout_h . O_k[h]) */
          for (int64_t t = 0; t < ORC_CHUNK; ++t) {
            const double dz = pr[t] * (dp[t] - pdp) * attn_scale;
            const int64_t ko = (bg * Lkv + c * ORC_CHUNK + t) * d;
            for (int64_t x = 0; x < d; ++x) {
              kh[x] = elem(k, ko + x, is_bf16) / kn[t];
              dqh[x] += dz * kh[x];
              dkh[(c * ORC_CHUNK + t) * d + x] += dz * qh[x];
            }
          }
        }
        if (qk_norm) norm_backward(q, d, dqh, dq);
        else
          for (int64_t x = 0; x < d; ++x) dq[x] = dqh[x];
        for (int64_t x = 0; x < d; ++x) dq_attn[qo + x] = any ? dq[x] : 0.0;
      }
      if (!any) continue;
      double swdw = 0.0;
      for (int64_t kk = 0; kk < K; ++kk) swdw += wdw[kk];
      const int64_t qro = srow * d;
      for (int64_t kk = 0; kk < K; ++kk) {
        const int64_t c = ix[kk];
        if (c < 0 || c >= Nc) continue;
        const double dr = ret_scale * (wdw[kk] - w[kk] * swdw);   /* ret_scale * ds_k */
        const int64_t lo = (bg * Nc + c) * d;
        for (int64_t x = 0; x < d; ++x) {
          dqr[x] += dr * elem(landmarks, lo + x, is_bf16);
          dlm_bg[c * d + x] += dr * elem(q_ret, qro + x, is_bf16);
        }
      }
    }
    /* keys: the normalisation's gradient after all rows */
    for (int64_t t = 0; t < Lkv; ++t) {
      const int64_t ko = (bg * Lkv + t) * d;
      for (int64_t x = 0; x < d; ++x) tmp[x] = elem(k, ko + x, is_bf16);
      if (qk_norm && t < Nc * ORC_CHUNK) norm_backward(tmp, d, dkh + t * d, dk + ko);
      else
        for (int64_t x = 0; x < d; ++x) dk[ko + x] = dkh[t * d + x];
    }
    free(dkh); free(w); free(wdw); free(buf);
  }
  return status;
}

/*
 * Landmark of chunk c of one (batch, kv head): the mean of the chunk's 64
 * stored keys.  Step 1 of the page gives every chunk one landmark from a learned
 * encoder, which needs trained weights; the workloads' stand-in (the chunk mean
 * of the keys) is what this computes, in fp64, summing in key order.
 * out [B, Hkv, c_end - c_begin, d] receives the landmarks of chunks
 * [c_begin, c_end).
 */
int hsa_oracle_chunk_landmarks(int64_t B, int64_t Hkv, int64_t Lkv, int64_t d, int is_bf16,
                               const void* k, int64_t c_begin, int64_t c_end, double* out) {
  const int64_t Nc = Lkv / ORC_CHUNK;
  if (B < 1 || Hkv < 1 || d < 1 || Lkv < 0 || !k || !out || c_begin < 0 || c_end < c_begin || c_end > Nc)
    return ORC_BAD_ARGS;
  const int64_t nc = c_end - c_begin;
#pragma omp parallel for schedule(static)
  for (int64_t bg = 0; bg < B * Hkv; ++bg) {
    for (int64_t c = 0; c < nc; ++c) {
      const int64_t row0 = bg * Lkv + (c_begin + c) * ORC_CHUNK;
      double* o = out + (bg * nc + c) * d;
      for (int64_t x = 0; x < d; ++x) {
        double s = 0.0;
        for (int64_t j = 0; j < ORC_CHUNK; ++j) s += elem(k, (row0 + j) * d + x, is_bf16);
        o[x] = s / ORC_CHUNK;
      }
    }
  }
  return ORC_OK;
}

int hsa_oracle_max_threads(void) {
#ifdef _OPENMP
  return omp_get_max_threads();
#else
  return 1;
#endif
}

void hsa_oracle_set_threads(int n) {
#ifdef _OPENMP
  if (n > 0) omp_set_num_threads(n);
#else
  (void)n;
#endif
}
