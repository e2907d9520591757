/*
 * hs_oracle.c -- plain, slow, obviously-correct CPU reference (IEEE double).
 *
 * TEST INFRASTRUCTURE ONLY: used by the tests, the smoke check and the benchmark's CPU-baseline
 * leg; never by the product library.  Page keys [P1] [P2] [P4] [P5] are listed in hs_oracle.h.
 *
 * Readings taken where the pages are silent (each also listed in the design notes):
 *   - token score = max over the GQA group's query heads of the normalized probability p;
 *     no aggregation across query positions (every query row gets its own set);
 *   - the k_global best keys are taken among positions 0..t-w only ("outside the window"), so the
 *     set is a disjoint union and |I_t| = min(t+1, k_global + w);
 *   - ties are broken by the lower position (blocks: the lower block id);
 *   - 0-based positions, the window includes the query's own position t;
 *   - blocks are 0-based and truncated at t; only causal blocks r <= floor(t/B) are candidates.
 */
#include "hs_oracle.h"

#include <math.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

static int g_threads = 0;

int orc_set_threads(int n) {
  g_threads = n > 0 ? n : 0;
  return orc_threads();
}

int orc_threads(void) {
#ifdef _OPENMP
  return g_threads > 0 ? g_threads : omp_get_max_threads();
#else
  return 1;
#endif
}

/* ------------------------------------------------------------------------------------------ */
/* shape helpers                                                                               */
/* ------------------------------------------------------------------------------------------ */

static int shape_ok(const orc_shape* s) {
  if (!s) return 0;
  if (s->batch < 1 || s->q_len < 1 || s->kv_len < 1 || s->n_q_heads < 1 || s->n_kv_heads < 1 ||
      s->head_dim < 1)
    return 0;
  if (s->n_q_heads % s->n_kv_heads) return 0;
  if (s->q_offset < 0 || s->q_offset + s->q_len > s->kv_len) return 0;
  if (!(s->scale >= 0.0)) return 0;
  return 1;
}

static int rows_ok(const orc_shape* s, const int32_t* rows, int n_rows) {
  if (!rows) return 1;
  if (n_rows < 0) return 0;
  for (int r = 0; r < n_rows; r++)
    if (rows[r] < 0 || rows[r] >= s->q_len) return 0;
  return 1;
}

static int64_t q_at(const orc_shape* s, int b, int j, int h) {
  return (((int64_t)b * s->q_len + j) * s->n_q_heads + h) * s->head_dim;
}
static int64_t kv_at(const orc_shape* s, int b, int64_t i, int u) {
  return (((int64_t)b * s->kv_len + i) * s->n_kv_heads + u) * s->head_dim;
}
static int64_t lse_at(const orc_shape* s, int b, int h, int j) {
  return ((int64_t)b * s->n_q_heads + h) * s->q_len + j;
}
static int64_t set_at(const orc_shape* s, int b, int j, int u) {
  return ((int64_t)b * s->q_len + j) * s->n_kv_heads + u;
}

/* Logits of one (b, j, h) against keys 0..t:  a_{t,i} = tau q_t . k_i with tau = 1/sqrt(d)
 * [P2 "Extracting block scores from exact attention", scaled dot-product equation], or the
 * caller's scale when one is given (a model may fold another constant into tau). */
static void logits_row(const orc_shape* s, const float* q, const float* k, int b, int j, int h,
                       double* a) {
  const int d = s->head_dim;
  const int u = h / (s->n_q_heads / s->n_kv_heads);
  const int64_t t = s->q_offset + j;
  const double tau = s->scale > 0.0 ? s->scale : 1.0 / sqrt((double)d);
  const float* qr = q + q_at(s, b, j, h);
  for (int64_t i = 0; i <= t; i++) {
    const float* kr = k + kv_at(s, b, i, u);
    double acc = 0.0;
    for (int c = 0; c < d; c++) acc += (double)qr[c] * (double)kr[c];
    a[i] = acc * tau;
  }
}

/* LSE of a row of logits restricted to keys with keep[i] != 0 (keep == NULL: all keys).
 * The max is subtracted before exponentiating so that exp never overflows. */
static double lse_of(const double* a, const unsigned char* keep, int64_t n) {
  double m = -INFINITY;
  for (int64_t i = 0; i < n; i++)
    if (!keep || keep[i]) m = a[i] > m ? a[i] : m;
  if (m == -INFINITY) return -INFINITY;
  double l = 0.0;
  for (int64_t i = 0; i < n; i++)
    if (!keep || keep[i]) l += exp(a[i] - m);
  return m + log(l);
}

/* o = sum_i exp(a_i - lse) v_i over kept keys; v rows of the KV head u. */
static void weighted_sum(const orc_shape* s, const float* v, int b, int u, const double* a,
                         const unsigned char* keep, int64_t n, double lse, double* o) {
  const int d = s->head_dim;
  for (int c = 0; c < d; c++) o[c] = 0.0;
  if (lse == -INFINITY) return;
  for (int64_t i = 0; i < n; i++) {
    if (keep && !keep[i]) continue;
    const double p = exp(a[i] - lse);
    const float* vr = v + kv_at(s, b, i, u);
    for (int c = 0; c < d; c++) o[c] += p * (double)vr[c];
  }
}

/* The (b, j, h) work items of a row subset, flattened for one parallel loop. */
typedef struct {
  int64_t n;
  int nb, nr, nh;
  const int32_t* rows;
} work_list;

static work_list make_work(const orc_shape* s, const int32_t* rows, int n_rows, int heads) {
  work_list w;
  w.nb = s->batch;
  w.nr = rows ? n_rows : s->q_len;
  w.nh = heads;
  w.rows = rows;
  w.n = (int64_t)w.nb * w.nr * w.nh;
  return w;
}
static void work_item(const work_list* w, int64_t it, int* b, int* j, int* h) {
  *h = (int)(it % w->nh);
  int64_t r = it / w->nh;
  int jr = (int)(r % w->nr);
  *b = (int)(r / w->nr);
  *j = w->rows ? w->rows[jr] : jr;
}

/* Logits a_{t,i}, i = 0..t, of one (b, j, h): the first step above, exported so that stored
 * attention logits can be checked against it. */
int orc_logit_row(const orc_shape* s, const float* q, const float* k, int b, int j, int h,
                  double* a) {
  if (!shape_ok(s) || !q || !k || !a) return ORC_EINVAL;
  if (b < 0 || b >= s->batch || j < 0 || j >= s->q_len || h < 0 || h >= s->n_q_heads)
    return ORC_EINVAL;
  logits_row(s, q, k, b, j, h, a);
  return ORC_OK;
}

/* ------------------------------------------------------------------------------------------ */
/* per-head probabilities                                                                      */
/* ------------------------------------------------------------------------------------------ */

/* p_{t,i} = exp(a_{t,i}) / sum_{j<=t} exp(a_{t,j}) = exp(a_{t,i} - LSE_t)
 * [P2 "Extracting block scores from exact attention", softmax equation]. */
int orc_prob_row(const orc_shape* s, const float* q, const float* k, const double* lse, int b,
                 int j, int h, double* p) {
  if (!shape_ok(s) || !q || !k || !p) return ORC_EINVAL;
  if (b < 0 || b >= s->batch || j < 0 || j >= s->q_len || h < 0 || h >= s->n_q_heads)
    return ORC_EINVAL;
  const int64_t n = s->q_offset + j + 1;
  logits_row(s, q, k, b, j, h, p);
  const double L = lse ? lse[lse_at(s, b, h, j)] : lse_of(p, NULL, n);
  for (int64_t i = 0; i < n; i++) p[i] = exp(p[i] - L);
  return ORC_OK;
}

/* ------------------------------------------------------------------------------------------ */
/* full attention                                                                              */
/* ------------------------------------------------------------------------------------------ */

/* Exact causal attention o_t = sum_{i<=t} p_{t,i} v_i and LSE_t = ln sum_{i<=t} exp(a_{t,i})
 * [P2 "Extracting block scores from exact attention", attention equations; P4 section 3.2]. */
int orc_full_attention(const orc_shape* s, const float* q, const float* k, const float* v,
                       double* o, double* lse, const int32_t* rows, int n_rows) {
  if (!shape_ok(s) || !q || !k || !v || !o || !rows_ok(s, rows, n_rows)) return ORC_EINVAL;
  const work_list w = make_work(s, rows, n_rows, s->n_q_heads);
  const int g = s->n_q_heads / s->n_kv_heads;
#pragma omp parallel num_threads(orc_threads())
  {
    double* a = (double*)malloc(sizeof(double) * (size_t)s->kv_len);
#pragma omp for schedule(dynamic, 4)
    for (int64_t it = 0; it < w.n; it++) {
      int b, j, h;
      work_item(&w, it, &b, &j, &h);
      const int64_t n = s->q_offset + j + 1;
      logits_row(s, q, k, b, j, h, a);
      const double L = lse_of(a, NULL, n);
      weighted_sum(s, v, b, h / g, a, NULL, n, L, o + q_at(s, b, j, h));
      if (lse) lse[lse_at(s, b, h, j)] = L;
    }
    free(a);
  }
  return ORC_OK;
}

/* ------------------------------------------------------------------------------------------ */
/* token scores and token top-k                                                                */
/* ------------------------------------------------------------------------------------------ */

/* Token score s_{t,i} = max over the group's heads h of p^h_{t,i}.  The group maximum follows the
 * GQA rule for block scores [P2 "GQA: the group shares one index set"; P4 section 3.2]; applying
 * it to single tokens is the token-level selection of HySparse2 [P1 section 4.2 change 1;
 * P5 "KV Reuse (Inner Level)"].  The aggregation itself is not disclosed by the pages [P1
 * "undisclosed points"]; this is the reading adopted.  lse == NULL recomputes each head's LSE. */
static void score_row(const orc_shape* s, const float* q, const float* k, const double* lse,
                      int b, int j, int u, double* score, double* tmp) {
  const int g = s->n_q_heads / s->n_kv_heads;
  const int64_t n = s->q_offset + j + 1;
  for (int64_t i = 0; i < n; i++) score[i] = -INFINITY;
  for (int h = u * g; h < (u + 1) * g; h++) {
    logits_row(s, q, k, b, j, h, tmp);
    const double L = lse ? lse[lse_at(s, b, h, j)] : lse_of(tmp, NULL, n);
    for (int64_t i = 0; i < n; i++) {
      const double p = exp(tmp[i] - L);
      if (p > score[i]) score[i] = p;
    }
  }
}

int orc_token_score_row(const orc_shape* s, const float* q, const float* k, const double* lse,
                        int b, int j, int u, double* score) {
  if (!shape_ok(s) || !q || !k || !score) return ORC_EINVAL;
  if (b < 0 || b >= s->batch || j < 0 || j >= s->q_len || u < 0 || u >= s->n_kv_heads)
    return ORC_EINVAL;
  double* tmp = (double*)malloc(sizeof(double) * (size_t)(s->q_offset + j + 1));
  score_row(s, q, k, lse, b, j, u, score, tmp);
  free(tmp);
  return ORC_OK;
}

typedef struct {
  double s;
  int64_t i;
} scored;

/* Order: higher score first; equal scores -> lower position (or block id) first. */
static int by_score_desc(const void* x, const void* y) {
  const scored* a = (const scored*)x;
  const scored* b = (const scored*)y;
  if (a->s > b->s) return -1;
  if (a->s < b->s) return 1;
  return (a->i > b->i) - (a->i < b->i);
}

/* Index set of query t: the most recent w positions are always taken, then the k_global
 * highest-scoring positions outside that window [P1 section 4.2 change 2; P5 "KV Reuse (Inner
 * Level)": 128 local + 1024 global].  Selection is a full sort of the candidates. */
int orc_token_topk(const orc_shape* s, const float* q, const float* k, const double* lse,
                   int k_global, int window, int cap, int32_t* idx, int32_t* count,
                   const int32_t* rows, int n_rows) {
  if (!shape_ok(s) || !q || !k || !idx || !count || !rows_ok(s, rows, n_rows)) return ORC_EINVAL;
  if (k_global < 0 || window < 0 || cap < k_global + window || cap < 1) return ORC_EINVAL;
  const work_list w = make_work(s, rows, n_rows, s->n_kv_heads);
#pragma omp parallel num_threads(orc_threads())
  {
    double* score = (double*)malloc(sizeof(double) * (size_t)s->kv_len);
    double* tmp = (double*)malloc(sizeof(double) * (size_t)s->kv_len);
    scored* cand = (scored*)malloc(sizeof(scored) * (size_t)s->kv_len);
    unsigned char* take = (unsigned char*)malloc((size_t)s->kv_len);
#pragma omp for schedule(dynamic, 1)
    for (int64_t it = 0; it < w.n; it++) {
      int b, j, u;
      work_item(&w, it, &b, &j, &u);
      const int64_t t = s->q_offset + j;
      score_row(s, q, k, lse, b, j, u, score, tmp);
      memset(take, 0, (size_t)(t + 1));
      /* candidates: positions 0 .. t-w (outside the window) */
      const int64_t n_cand = t - window + 1 > 0 ? t - window + 1 : 0;
      for (int64_t i = 0; i < n_cand; i++) {
        cand[i].s = score[i];
        cand[i].i = i;
      }
      qsort(cand, (size_t)n_cand, sizeof(scored), by_score_desc);
      const int64_t n_top = n_cand < k_global ? n_cand : k_global;
      for (int64_t r = 0; r < n_top; r++) take[cand[r].i] = 1;
      /* window: positions max(0, t-w+1) .. t */
      for (int64_t i = (t - window + 1 > 0 ? t - window + 1 : 0); i <= t; i++) take[i] = 1;
      int32_t* out = idx + set_at(s, b, j, u) * cap;
      int n_out = 0;
      for (int64_t i = 0; i <= t; i++)
        if (take[i]) out[n_out++] = (int32_t)i;
      count[set_at(s, b, j, u)] = n_out;
      for (int e = n_out; e < cap; e++) out[e] = -1;
    }
    free(score);
    free(tmp);
    free(cand);
    free(take);
  }
  return ORC_OK;
}

/* ------------------------------------------------------------------------------------------ */
/* sparse layer over a token index set                                                         */
/* ------------------------------------------------------------------------------------------ */

/* A sparse layer attends with its own query over the full layer's K, V restricted to the shared
 * index set [P2 "Cross-layer KV cache reuse" gather equations; P2 "Same query, two memories",
 * global-branch equation; P4 section 3.3].  Written as a dense masked softmax over all keys
 * 0..t (non-members at -inf), so no gather loop is involved. */
/* ln(e^L + e^s): the denominator of a softmax whose keys give LSE L, with one more logit s
 * that carries no value (the per-head sink).  sink == NULL: L unchanged. */
static double with_sink(double L, const float* sink, int h) {
  if (!sink) return L;
  const double sv = (double)sink[h];
  if (L == -INFINITY) return sv;
  const double m = L > sv ? L : sv;
  return m + log(exp(L - m) + exp(sv - m));
}

static double sigmoid(double z);

int orc_masked_attention(const orc_shape* s, const float* q, const float* k, const float* v,
                         const int32_t* idx, const int32_t* count, int cap, double* o,
                         double* lse, const int32_t* rows, int n_rows) {
  return orc_masked_attention_ex(s, q, k, v, idx, count, cap, NULL, NULL, o, lse, rows, n_rows);
}

/* Sparse layer with the options of the pages' sparse layers [P1 section 6.1: every sparse and
 * SWA layer has a sigmoid output gate and a learnable per-head sink bias; P4 experimental setup:
 * per-head sink bias in the manner of gpt-oss]: LSE' = ln(e^{s_h} + sum_{i in I} e^{a_i}),
 * o = sigmoid(g) sum_{i in I} e^{a_i - LSE'} v_i. */
/* Output gate of the sparse and sliding-window layers: one logit per (query, head) (out_gate,
 * [B, Tq, Hq]) or one per channel (out_gate_ch, [B, Tq, Hq, d]) [P1 section 6.1 (gated
 * attention); P2 "Two sigmoid gates, not one of two": a gate may act per head or per channel].
 * Returns the factor of channel c; 1 without a gate. */
static double out_gate_factor(const orc_shape* s, const float* out_gate, const float* out_gate_ch,
                              int b, int j, int h, int c) {
  const int64_t row = ((int64_t)b * s->q_len + j) * s->n_q_heads + h;
  if (out_gate_ch) return sigmoid((double)out_gate_ch[row * s->head_dim + c]);
  if (out_gate) return sigmoid((double)out_gate[row]);
  return 1.0;
}

static int masked_attention(const orc_shape* s, const float* q, const float* k, const float* v,
                            const int32_t* idx, const int32_t* count, int cap, const float* sink,
                            const float* out_gate, const float* out_gate_ch, double* o,
                            double* lse, const int32_t* rows, int n_rows);

int orc_masked_attention_ex(const orc_shape* s, const float* q, const float* k, const float* v,
                            const int32_t* idx, const int32_t* count, int cap, const float* sink,
                            const float* out_gate, double* o, double* lse, const int32_t* rows,
                            int n_rows) {
  return masked_attention(s, q, k, v, idx, count, cap, sink, out_gate, NULL, o, lse, rows,
                          n_rows);
}

int orc_masked_attention_ch(const orc_shape* s, const float* q, const float* k, const float* v,
                            const int32_t* idx, const int32_t* count, int cap, const float* sink,
                            const float* out_gate_ch, double* o, double* lse,
                            const int32_t* rows, int n_rows) {
  if (!out_gate_ch) return ORC_EINVAL;
  return masked_attention(s, q, k, v, idx, count, cap, sink, NULL, out_gate_ch, o, lse, rows,
                          n_rows);
}

static int masked_attention(const orc_shape* s, const float* q, const float* k, const float* v,
                            const int32_t* idx, const int32_t* count, int cap, const float* sink,
                            const float* out_gate, const float* out_gate_ch, double* o,
                            double* lse, const int32_t* rows, int n_rows) {
  if (!shape_ok(s) || !q || !k || !v || !idx || !count || !o || cap < 1 ||
      !rows_ok(s, rows, n_rows))
    return ORC_EINVAL;
  const work_list w = make_work(s, rows, n_rows, s->n_q_heads);
  const int g = s->n_q_heads / s->n_kv_heads;
  int status = ORC_OK;
#pragma omp parallel num_threads(orc_threads())
  {
    double* a = (double*)malloc(sizeof(double) * (size_t)s->kv_len);
    unsigned char* keep = (unsigned char*)malloc((size_t)s->kv_len);
#pragma omp for schedule(dynamic, 4)
    for (int64_t it = 0; it < w.n; it++) {
      int b, j, h;
      work_item(&w, it, &b, &j, &h);
      const int u = h / g;
      const int64_t t = s->q_offset + j;
      const int32_t* set = idx + set_at(s, b, j, u) * cap;
      const int32_t n_set = count[set_at(s, b, j, u)];
      memset(keep, 0, (size_t)(t + 1));
      int bad = n_set < 0 || n_set > cap;
      for (int e = 0; !bad && e < n_set; e++) {
        if (set[e] < 0 || set[e] > t) bad = 1;
        else keep[set[e]] = 1;
      }
      if (bad) {
#pragma omp atomic write
        status = ORC_EINDEX;
        continue;
      }
      logits_row(s, q, k, b, j, h, a);
      const double L = with_sink(lse_of(a, keep, t + 1), sink, h);
      double* out = o + q_at(s, b, j, h);
      weighted_sum(s, v, b, u, a, keep, t + 1, L, out);
      if (out_gate || out_gate_ch)
        for (int c = 0; c < s->head_dim; c++)
          out[c] *= out_gate_factor(s, out_gate, out_gate_ch, b, j, h, c);
      if (lse) lse[lse_at(s, b, h, j)] = L;
    }
    free(a);
    free(keep);
  }
  return status;
}

/* ------------------------------------------------------------------------------------------ */
/* block scores and block top-k (HySparse)                                                     */
/* ------------------------------------------------------------------------------------------ */

/* S_{t,r} = max_{i in B_r} p_{t,i} with B_r = {rB, .., min((r+1)B-1, t)}
 * [P2 "Extracting block scores from exact attention", block-score equation; P4 section 3.2],
 * then the group maximum over the heads of the GQA group [P2 "GQA: the group shares one index
 * set"].  Blocks are 0-based and causally truncated at t (P2's form). */
static void block_row(const orc_shape* s, const float* q, const float* k, const double* lse,
                      int b, int j, int u, int block, double* bs, double* tmp) {
  const int g = s->n_q_heads / s->n_kv_heads;
  const int64_t t = s->q_offset + j;
  const int64_t nb = t / block + 1;
  for (int64_t r = 0; r < nb; r++) bs[r] = -INFINITY;
  for (int h = u * g; h < (u + 1) * g; h++) {
    logits_row(s, q, k, b, j, h, tmp);
    const double L = lse ? lse[lse_at(s, b, h, j)] : lse_of(tmp, NULL, t + 1);
    for (int64_t i = 0; i <= t; i++) {
      const double p = exp(tmp[i] - L);
      if (p > bs[i / block]) bs[i / block] = p;
    }
  }
}

int orc_block_score_row(const orc_shape* s, const float* q, const float* k, const double* lse,
                        int b, int j, int u, int block, double* score) {
  if (!shape_ok(s) || !q || !k || !score || block < 1) return ORC_EINVAL;
  if (b < 0 || b >= s->batch || j < 0 || j >= s->q_len || u < 0 || u >= s->n_kv_heads)
    return ORC_EINVAL;
  double* tmp = (double*)malloc(sizeof(double) * (size_t)(s->q_offset + j + 1));
  block_row(s, q, k, lse, b, j, u, block, score, tmp);
  free(tmp);
  return ORC_OK;
}

/* I_t = TopKBlocks(S_{t,:}, k/B) [P2 "Extracting block scores from exact attention", TopK
 * equation; P4 section 3.2]: the n_blocks best causal blocks by (score desc, block id asc). */
int orc_block_topk(const orc_shape* s, const float* q, const float* k, const double* lse,
                   int block, int n_blocks, int32_t* blk_idx, int32_t* count,
                   const int32_t* rows, int n_rows) {
  if (!shape_ok(s) || !q || !k || !blk_idx || !count || block < 1 || n_blocks < 1 ||
      !rows_ok(s, rows, n_rows))
    return ORC_EINVAL;
  const work_list w = make_work(s, rows, n_rows, s->n_kv_heads);
#pragma omp parallel num_threads(orc_threads())
  {
    double* bs = (double*)malloc(sizeof(double) * (size_t)(s->kv_len / block + 1));
    double* tmp = (double*)malloc(sizeof(double) * (size_t)s->kv_len);
    scored* cand = (scored*)malloc(sizeof(scored) * (size_t)(s->kv_len / block + 1));
    unsigned char* take = (unsigned char*)malloc((size_t)(s->kv_len / block + 1));
#pragma omp for schedule(dynamic, 1)
    for (int64_t it = 0; it < w.n; it++) {
      int b, j, u;
      work_item(&w, it, &b, &j, &u);
      const int64_t t = s->q_offset + j;
      const int64_t nb = t / block + 1;
      block_row(s, q, k, lse, b, j, u, block, bs, tmp);
      for (int64_t r = 0; r < nb; r++) {
        cand[r].s = bs[r];
        cand[r].i = r;
      }
      qsort(cand, (size_t)nb, sizeof(scored), by_score_desc);
      const int64_t n_top = nb < n_blocks ? nb : n_blocks;
      memset(take, 0, (size_t)nb);
      for (int64_t r = 0; r < n_top; r++) take[cand[r].i] = 1;
      int32_t* out = blk_idx + set_at(s, b, j, u) * n_blocks;
      int n_out = 0;
      for (int64_t r = 0; r < nb; r++)
        if (take[r]) out[n_out++] = (int32_t)r;
      count[set_at(s, b, j, u)] = n_out;
      for (int e = n_out; e < n_blocks; e++) out[e] = -1;
    }
    free(bs);
    free(tmp);
    free(cand);
    free(take);
  }
  return ORC_OK;
}

/* ------------------------------------------------------------------------------------------ */
/* HySparse sparse layer: block-sparse branch + own sliding window + sigmoid gates             */
/* ------------------------------------------------------------------------------------------ */

static double sigmoid(double z) { return 1.0 / (1.0 + exp(-z)); }

/* o_glob: softmax over the keys of the selected blocks of the shared K, V, masked causally inside
 * a block that crosses t [P2 "Same query, two memories", global-branch equation; P2 engineering
 * constraint 4 (causal mask inside the block)].
 * o_loc: softmax over positions max(0,t-w+1)..t of the layer's own K', V' [P2 "Same query, two
 * memories", SWA equation, written 1-based there].
 * o = sigmoid(zG) * o_glob + sigmoid(zL) * o_loc with per-head scalar gate logits
 * [P2 "Two sigmoid gates, not a choice"; P4 section 3.3]. */
int orc_gated_block_swa(const orc_shape* s, const float* q, const float* k, const float* v,
                        const int32_t* blk_idx, const int32_t* count, int n_blocks, int block,
                        const float* k_loc, const float* v_loc, int window, const float* gate,
                        double* o, double* o_glob, double* o_loc, const int32_t* rows,
                        int n_rows) {
  return orc_gated_block_swa_ex(s, q, k, v, blk_idx, count, n_blocks, block, k_loc, v_loc, window,
                                gate, NULL, NULL, NULL, o, o_glob, o_loc, rows, n_rows);
}

static int gated_block_swa(const orc_shape* s, const float* q, const float* k, const float* v,
                           const int32_t* blk_idx, const int32_t* count, int n_blocks, int block,
                           const float* k_loc, const float* v_loc, int window, const float* gate,
                           const float* gate_ch, const float* sink, const float* sink_loc,
                           const float* out_gate, const float* out_gate_ch, double* o,
                           double* o_glob, double* o_loc, const int32_t* rows, int n_rows);

/* The gated layer with a per-head sink in each branch and an output gate applied to the sum
 * (same sources as orc_masked_attention_ex). */
int orc_gated_block_swa_ex(const orc_shape* s, const float* q, const float* k, const float* v,
                           const int32_t* blk_idx, const int32_t* count, int n_blocks, int block,
                           const float* k_loc, const float* v_loc, int window, const float* gate,
                           const float* sink, const float* sink_loc, const float* out_gate,
                           double* o, double* o_glob, double* o_loc, const int32_t* rows,
                           int n_rows) {
  if (!gate) return ORC_EINVAL;
  return gated_block_swa(s, q, k, v, blk_idx, count, n_blocks, block, k_loc, v_loc, window, gate,
                         NULL, sink, sink_loc, out_gate, NULL, o, o_glob, o_loc, rows, n_rows);
}

/* The gated layer with per-channel gates [P2 "Two sigmoid gates, not one of two": each gate may
 * act per head or per channel]: o_c = sigmoid(zG_c) o_glob,c + sigmoid(zL_c) o_loc,c with
 * gate_ch [B, Tq, Hq, 2, d] (the d logits of zG, then the d of zL), and an optional per-channel
 * output gate out_gate_ch [B, Tq, Hq, d] on the sum. */
int orc_gated_block_swa_ch(const orc_shape* s, const float* q, const float* k, const float* v,
                           const int32_t* blk_idx, const int32_t* count, int n_blocks, int block,
                           const float* k_loc, const float* v_loc, int window,
                           const float* gate_ch, const float* sink, const float* sink_loc,
                           const float* out_gate_ch, double* o, double* o_glob, double* o_loc,
                           const int32_t* rows, int n_rows) {
  if (!gate_ch) return ORC_EINVAL;
  return gated_block_swa(s, q, k, v, blk_idx, count, n_blocks, block, k_loc, v_loc, window, NULL,
                         gate_ch, sink, sink_loc, NULL, out_gate_ch, o, o_glob, o_loc, rows,
                         n_rows);
}

static int gated_block_swa(const orc_shape* s, const float* q, const float* k, const float* v,
                           const int32_t* blk_idx, const int32_t* count, int n_blocks, int block,
                           const float* k_loc, const float* v_loc, int window, const float* gate,
                           const float* gate_ch, const float* sink, const float* sink_loc,
                           const float* out_gate, const float* out_gate_ch, double* o,
                           double* o_glob, double* o_loc, const int32_t* rows, int n_rows) {
  if (!shape_ok(s) || !q || !k || !v || !blk_idx || !count || !k_loc || !v_loc ||
      (!gate && !gate_ch) || !o || n_blocks < 1 || block < 1 || window < 1 ||
      !rows_ok(s, rows, n_rows))
    return ORC_EINVAL;
  const work_list w = make_work(s, rows, n_rows, s->n_q_heads);
  const int g = s->n_q_heads / s->n_kv_heads;
  const int d = s->head_dim;
  int status = ORC_OK;
#pragma omp parallel num_threads(orc_threads())
  {
    double* a = (double*)malloc(sizeof(double) * (size_t)s->kv_len);
    unsigned char* keep = (unsigned char*)malloc((size_t)s->kv_len);
    double* og = (double*)malloc(sizeof(double) * (size_t)d);
    double* ol = (double*)malloc(sizeof(double) * (size_t)d);
#pragma omp for schedule(dynamic, 4)
    for (int64_t it = 0; it < w.n; it++) {
      int b, j, h;
      work_item(&w, it, &b, &j, &h);
      const int u = h / g;
      const int64_t t = s->q_offset + j;
      const int64_t nb = t / block + 1;
      const int32_t* set = blk_idx + set_at(s, b, j, u) * n_blocks;
      const int32_t n_set = count[set_at(s, b, j, u)];
      int bad = n_set < 0 || n_set > n_blocks;
      memset(keep, 0, (size_t)(t + 1));
      for (int e = 0; !bad && e < n_set; e++) {
        if (set[e] < 0 || set[e] >= nb) {
          bad = 1;
          break;
        }
        for (int64_t i = (int64_t)set[e] * block; i < (int64_t)(set[e] + 1) * block && i <= t;
             i++)
          keep[i] = 1;
      }
      if (bad) {
#pragma omp atomic write
        status = ORC_EINDEX;
        continue;
      }
      /* global branch over the shared K, V */
      logits_row(s, q, k, b, j, h, a);
      double L = with_sink(lse_of(a, keep, t + 1), sink, h);
      weighted_sum(s, v, b, u, a, keep, t + 1, L, og);
      /* local branch over the layer's own K', V' */
      memset(keep, 0, (size_t)(t + 1));
      for (int64_t i = (t - window + 1 > 0 ? t - window + 1 : 0); i <= t; i++) keep[i] = 1;
      logits_row(s, q, k_loc, b, j, h, a);
      L = with_sink(lse_of(a, keep, t + 1), sink_loc, h);
      weighted_sum(s, v_loc, b, u, a, keep, t + 1, L, ol);
      const int64_t row = ((int64_t)b * s->q_len + j) * s->n_q_heads + h;
      double* out = o + q_at(s, b, j, h);
      for (int c = 0; c < d; c++) {
        const double zG = gate_ch ? gate_ch[(row * 2 + 0) * d + c] : gate[row * 2 + 0];
        const double zL = gate_ch ? gate_ch[(row * 2 + 1) * d + c] : gate[row * 2 + 1];
        const double gO = out_gate_factor(s, out_gate, out_gate_ch, b, j, h, c);
        out[c] = gO * (sigmoid(zG) * og[c] + sigmoid(zL) * ol[c]);
      }
      if (o_glob)
        for (int c = 0; c < d; c++) o_glob[q_at(s, b, j, h) + c] = og[c];
      if (o_loc)
        for (int c = 0; c < d; c++) o_loc[q_at(s, b, j, h) + c] = ol[c];
    }
    free(a);
    free(keep);
    free(og);
    free(ol);
  }
  return status;
}
