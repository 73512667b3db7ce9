/*
 * tsel_oracle.c -- plain, slow CPU oracle for batched token selection and
 * greedy draft verification.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing on the product path may include, link,
 * load or call this file: only the test suite, the smoke check and the CPU
 * baseline leg of the benchmark use it.  It shares no header, table or helper
 * with the HIP library; it is written straight from the definitions on the
 * pages, one processor at a time, over whole rows, with no fusion.
 *
 * Sources (page title -- section):
 *   [T] "Transmuter.Generation (transmuter v2.0.0)": module doc, the paragraph
 *       on token selection (processor order); "Lengths"; "Processors";
 *       "Log-probabilities"; "Batches"; function doc of generate/5.
 *   [A] "Assisted Generation: a new direction toward low-latency text
 *       generation": "Greedy decoding with assisted generation" (the six-step
 *       loop); "Sample with assisted generation".
 *   [M] mlxcel "추론 파이프라인" (inference pipeline): "3단계: 디코드 루프"
 *       (fused draw, EOS set).
 *
 * Arithmetic: every elementwise processor is one IEEE-754 binary32 operation
 * rounded to nearest even (compiled with -ffp-contract=off, no fast-math);
 * softmax masses, their sums and cumulative sums are binary64.  bf16 logits
 * are widened exactly (the 16 bits become the high half of a binary32).
 *
 * Readings taken where the pages are silent (each is repeated in the design
 * notes): removed scores are -inf; the penalty acts once per distinct id; a
 * forced token gets score 0 and every other id -inf; ties in top-p order and
 * in the sampling CDF go to the lower index; the sample is the inverse CDF of
 * a caller uniform u in [0,1) over the kept ids in (score desc, index asc)
 * order; greedy ties go to the lowest index; an all-removed row selects id 0;
 * the next draft count is floored at 1.
 */
#include <float.h>
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define ORACLE_MAX_ADMISSIBLE 64

typedef struct {
  int32_t vocab;
  int32_t dtype;                 /* 0 = binary32 logits, 1 = bf16 logits */
  float repetition_penalty;      /* 1.0 = off */
  int32_t no_repeat_ngram_size;  /* 0 = off */
  const int32_t *bad_ids;        /* single-token bad words */
  int32_t n_bad;
  int32_t min_length;            /* 0 = off */
  int32_t min_new_tokens;        /* 0 = off; when > 0 it replaces min_length */
  const int32_t *eos_ids;
  int32_t n_eos;
  int32_t forced_bos;            /* < 0 = off */
  int32_t forced_eos;            /* < 0 = off */
  const int32_t *suppress_ids;
  int32_t n_suppress;
  const int32_t *begin_ids;      /* begin_suppress_tokens */
  int32_t n_begin;
  int32_t do_sample;             /* 0 = greedy */
  float temperature;             /* 1.0 = identity */
  int32_t top_k;                 /* 0 = off */
  float top_p;                   /* >= 1.0 = off */
  int32_t renormalize_logits;    /* 0 = off */
} oracle_cfg;

typedef struct {
  int32_t token;
  int32_t n_finite;              /* ids with a finite final score */
  float topk_threshold;          /* k-th largest score (or -inf / NaN if off) */
  double margin;                 /* sampling decision margin, normalized mass */
  double greedy_margin;          /* (x1 - x2) / max(1, |x1|) */
  int32_t n_admissible;
  int32_t admissible[ORACLE_MAX_ADMISSIBLE];
  int32_t keep_min, keep_max;    /* ids top_p keeps for sure / may keep when
                                    each normalized mass before an id moves
                                    by at most eps (sampling; else n_finite) */
  float logprob;                 /* log-softmax of the final scores at the token
                                    (quiet NaN for a row with no token) */
} oracle_row_result;

/* ------------------------------------------------------------------ */
/* Exact widening of one logit to binary32.                            */
static float load_logit(const void *row, int32_t dtype, int32_t v) {
  if (dtype == 0) return ((const float *)row)[v];
  uint32_t bits = ((uint32_t)((const uint16_t *)row)[v]) << 16;
  float f;
  memcpy(&f, &bits, sizeof f);
  return f;
}

static int in_vocab(int32_t id, int32_t V) { return id >= 0 && id < V; }

/* [T] module doc (processor order, first entry) + the Python transformers
 * penalty rule: a seen id with a negative score is multiplied by the
 * penalty, any other seen id is divided by it.  Each distinct id once. */
static void repetition_penalty(float *x, int32_t V, const int32_t *h, int32_t L,
                               float p) {
  unsigned char *seen = (unsigned char *)calloc((size_t)V, 1);
  for (int32_t i = 0; i < L; ++i) {
    int32_t v = h[i];
    if (!in_vocab(v, V) || seen[v]) continue;
    seen[v] = 1;
    x[v] = (x[v] < 0.0f) ? x[v] * p : x[v] / p;
  }
  free(seen);
}

/* [T] "Lengths", no_repeat_ngram_size: an n-gram of prompt + new tokens may
 * occur only once.  The next id t is banned when the last n-1 ids followed
 * by t form an n-gram that already occurs in the history. */
static void no_repeat_ngram(float *x, int32_t V, const int32_t *h, int32_t L,
                            int32_t n, float removed) {
  if (n <= 0 || L < n) return;
  const int32_t *tail = h + (L - n + 1); /* the last n-1 ids */
  for (int32_t i = 0; i + n <= L; ++i) {
    int match = 1;
    for (int32_t j = 0; j < n - 1; ++j)
      if (h[i + j] != tail[j]) { match = 0; break; }
    if (match && in_vocab(h[i + n - 1], V)) x[h[i + n - 1]] = removed;
  }
}

/* Removed ids take `removed`: -inf for selection; the smallest finite
 * value in beam search ([T], the beam paragraph under "Log-probabilities"). */
static void ban_ids(float *x, int32_t V, const int32_t *ids, int32_t n, float removed) {
  for (int32_t i = 0; i < n; ++i)
    if (in_vocab(ids[i], V)) x[ids[i]] = removed;
}

/* [T] "Lengths", forced_bos_token_id / forced_eos_token_id. */
static void force_token(float *x, int32_t V, int32_t id, float removed) {
  for (int32_t v = 0; v < V; ++v) x[v] = removed;
  if (in_vocab(id, V)) x[id] = 0.0f;
}

/* Greedy choice: the largest score, lowest index among equals. */
static int32_t argmax_lowest(const float *x, int32_t V) {
  int32_t best = 0;
  for (int32_t v = 1; v < V; ++v)
    if (x[v] > x[best]) best = v;
  return best;
}

/* log(sum over the finite scores of exp(x - m)), m the largest finite
 * score, in binary64; returns -inf (and m = -inf) when none is finite. */
static double log_sum_exp_shifted(const float *x, int32_t V, double *m_out) {
  double m = -INFINITY;
  for (int32_t v = 0; v < V; ++v)
    if ((double)x[v] > m) m = (double)x[v];
  *m_out = m;
  if (m == -INFINITY) return -INFINITY;
  double sum = 0.0;
  for (int32_t v = 0; v < V; ++v)
    if (x[v] > -INFINITY) sum += exp((double)x[v] - m);
  return log(sum);
}

/* [T] module doc, renormalize_logits (after the processors of the task,
 * before temperature): the log-softmax of the row.  Reading: the largest
 * score m and ls = log(sum exp(x - m)) rounded once to binary32, then two
 * binary32 subtractions, (x - m) - ls; -inf stays -inf; a row with no finite
 * score is left as it is. */
static void renormalize(float *x, int32_t V) {
  double m;
  const double ls = log_sum_exp_shifted(x, V, &m);
  if (m == -INFINITY) return;
  const float mf = (float)m, lsf = (float)ls;
  for (int32_t v = 0; v < V; ++v)
    if (x[v] > -INFINITY) x[v] = (x[v] - mf) - lsf;
}

/* [T] "Log-probabilities": the log-softmax of the scores the step selects
 * from, at the token: x[t] - m - log(sum exp(x - m)) in binary64, rounded
 * once to binary32 (all scores -inf: NaN, as the arithmetic gives). */
static float token_logprob(const float *x, int32_t V, int32_t t) {
  double m;
  const double ls = log_sum_exp_shifted(x, V, &m);
  if (m == -INFINITY) return NAN;
  return (float)(((double)x[t] - m) - ls);
}

static int cmp_float_desc(const void *a, const void *b) {
  float fa = *(const float *)a, fb = *(const float *)b;
  return (fa < fb) - (fa > fb);
}

/* Sort order of the sampling warpers: score descending, index ascending. */
static _Thread_local const float *g_sort_scores;
static int cmp_idx_by_score(const void *a, const void *b) {
  int32_t ia = *(const int32_t *)a, ib = *(const int32_t *)b;
  float fa = g_sort_scores[ia], fb = g_sort_scores[ib];
  if (fa > fb) return -1;
  if (fa < fb) return 1;
  return (ia > ib) - (ia < ib);
}

/* Indices of finite scores in (score desc, index asc) order. */
static int32_t sorted_finite(const float *x, int32_t V, int32_t *order) {
  int32_t n = 0;
  for (int32_t v = 0; v < V; ++v)
    if (x[v] > -INFINITY) order[n++] = v;
  g_sort_scores = x;
  qsort(order, (size_t)n, sizeof(int32_t), cmp_idx_by_score);
  return n;
}

/* [T] module doc, top_k: keep every score >= the k-th largest score
 * (multiset order statistic); all others become -inf. */
static float top_k_filter(float *x, int32_t V, int32_t k) {
  int32_t keff = k < V ? k : V;
  float *copy = (float *)malloc(sizeof(float) * (size_t)V);
  memcpy(copy, x, sizeof(float) * (size_t)V);
  qsort(copy, (size_t)V, sizeof(float), cmp_float_desc);
  float t = copy[keff - 1];
  free(copy);
  for (int32_t v = 0; v < V; ++v)
    if (x[v] < t) x[v] = -INFINITY;
  return t;
}

/* [T] module doc, top_p: over the finite scores in (score desc, index asc)
 * order, with softmax masses q, the id at position j stays iff the mass of
 * the ids before it is < p; the first id always stays. */
typedef struct {
  int32_t n;        /* finite ids before the filter */
  int32_t kept;     /* ids kept */
  double a_last;    /* A of the last kept id */
  double a_next;    /* A of the first removed id (or 2.0 if none) */
} top_p_info;

static top_p_info top_p_filter(float *x, int32_t V, float p, int32_t *order,
                               double *w) {
  top_p_info info = {0, 0, 0.0, 2.0};
  int32_t n = sorted_finite(x, V, order);
  info.n = n;
  if (n == 0) return info;
  double m = (double)x[order[0]];
  double W = 0.0;
  for (int32_t j = 0; j < n; ++j) {
    w[j] = exp((double)x[order[j]] - m);
    W += w[j];
  }
  double run = 0.0; /* unnormalized mass of the positions before j */
  for (int32_t j = 0; j < n; ++j) {
    double A = run / W;
    if (A < (double)p) {
      info.kept = j + 1;
      info.a_last = A;
    } else {
      if (info.a_next > 1.5) info.a_next = A;
      x[order[j]] = -INFINITY;
    }
    run += w[j];
  }
  return info;
}

/* Inverse-CDF sample over the finite scores, in the same order as top_p,
 * from the caller uniform u in [0,1); also the decision margin and the set of
 * ids reachable when each cumulative sum moves by at most eps * W'. */
static int32_t sample_inverse_cdf(const float *x, int32_t V, float u,
                                  int32_t *order, double *w, double *margin_u) {
  int32_t n = sorted_finite(x, V, order);
  if (n == 0) return -1;
  double m = (double)x[order[0]];
  double Wp = 0.0;
  for (int32_t j = 0; j < n; ++j) {
    w[j] = exp((double)x[order[j]] - m);
    Wp += w[j];
  }
  double target = (double)u * Wp;
  double C = 0.0;
  int32_t pick = n - 1;
  double lo = 0.0, hi = Wp;
  for (int32_t j = 0; j < n; ++j) {
    double prev = C;
    C += w[j];
    if (C > target) {
      pick = j;
      lo = prev;
      hi = C;
      break;
    }
  }
  double mu = target - lo < hi - target ? target - lo : hi - target;
  *margin_u = mu / Wp;
  return order[pick];
}

/* The processors of [T] module doc, in its order, over one row of scores
 * (from the repetition penalty to begin_suppress_tokens); removed ids take
 * `removed`. */
static void apply_processors(float *x, int32_t V, const int32_t *h, int32_t L, int32_t P,
                             int32_t M, const oracle_cfg *cfg, float removed) {
  const int32_t new_tokens = L - P;
  if (cfg->repetition_penalty != 1.0f)
    repetition_penalty(x, V, h, L, cfg->repetition_penalty);
  if (cfg->no_repeat_ngram_size > 0)
    no_repeat_ngram(x, V, h, L, cfg->no_repeat_ngram_size, removed);
  ban_ids(x, V, cfg->bad_ids, cfg->n_bad, removed);
  {
    /* [T] "Lengths": min_new_tokens replaces min_length when both are set. */
    int active = 0;
    if (cfg->min_new_tokens > 0) active = new_tokens < cfg->min_new_tokens;
    else if (cfg->min_length > 0) active = L < cfg->min_length;
    if (active) ban_ids(x, V, cfg->eos_ids, cfg->n_eos, removed);
  }
  if (cfg->forced_bos >= 0 && L == 1) force_token(x, V, cfg->forced_bos, removed);
  if (cfg->forced_eos >= 0 && L == M - 1) force_token(x, V, cfg->forced_eos, removed);
  ban_ids(x, V, cfg->suppress_ids, cfg->n_suppress, removed);
  {
    /* [T] "Lengths", begin_suppress_tokens: at the first new token, or at
     * the second when a forced bos followed a one-token prompt. */
    int32_t begin = (cfg->forced_bos >= 0 && P == 1) ? 1 : 0;
    if (new_tokens == begin) ban_ids(x, V, cfg->begin_ids, cfg->n_begin, removed);
  }
}

/* ------------------------------------------------------------------ */
/* The whole selection for one row.  logits_row: V logits of dtype;
 * h: L history ids (prompt then new tokens, chronological); P: prompt
 * length; M: max_length = P + max_new_tokens; u: the row's uniform.
 * x_out (may be NULL) receives the final scores the token is chosen from.
 * Returns 0, or -1 on allocation failure. */
int oracle_select_row(const void *logits_row, const int32_t *h, int32_t L,
                      int32_t P, int32_t M, const oracle_cfg *cfg, float u,
                      float *x_out, oracle_row_result *res) {
  const int32_t V = cfg->vocab;
  memset(res, 0, sizeof *res);
  res->topk_threshold = NAN;
  res->margin = INFINITY;
  res->greedy_margin = INFINITY;
  /* [T] "Batches" and generate/5: an empty row is a padding row with no
   * token, reported as -1. */
  if (L == 0) {
    res->token = -1;
    res->logprob = NAN;
    if (x_out)
      for (int32_t v = 0; v < V; ++v) x_out[v] = -INFINITY;
    return 0;
  }
  float *x = (float *)malloc(sizeof(float) * (size_t)V);
  int32_t *order = (int32_t *)malloc(sizeof(int32_t) * (size_t)V);
  double *buf = (double *)malloc(sizeof(double) * (size_t)V);
  if (!x || !order || !buf) { free(x); free(order); free(buf); return -1; }
  for (int32_t v = 0; v < V; ++v) x[v] = load_logit(logits_row, cfg->dtype, v);

  apply_processors(x, V, h, L, P, M, cfg, -INFINITY);
  if (cfg->renormalize_logits) renormalize(x, V);

  if (!cfg->do_sample) {
    int32_t t = argmax_lowest(x, V);
    res->token = t;
    float x1 = x[t], x2 = -INFINITY;
    for (int32_t v = 0; v < V; ++v)
      if (v != t && x[v] > x2) x2 = x[v];
    float den = fabsf(x1) > 1.0f ? fabsf(x1) : 1.0f;
    res->greedy_margin = (x1 > -INFINITY) ? ((double)x1 - (double)x2) / den : 0.0;
    for (int32_t v = 0; v < V; ++v) res->n_finite += x[v] > -INFINITY;
    res->keep_min = res->keep_max = res->n_finite;
    res->logprob = token_logprob(x, V, t);
    if (x_out) memcpy(x_out, x, sizeof(float) * (size_t)V);
    free(x); free(order); free(buf);
    return 0;
  }

  /* Warpers of sampling, in order: temperature, top_k, top_p. */
  if (cfg->temperature != 1.0f)
    for (int32_t v = 0; v < V; ++v) x[v] = x[v] / cfg->temperature;
  if (cfg->top_k > 0) res->topk_threshold = top_k_filter(x, V, cfg->top_k);

  double margin_p = INFINITY;
  /* Keep a copy of the pre-top_p scores for the admissible-set search. */
  float *pre = (float *)malloc(sizeof(float) * (size_t)V);
  memcpy(pre, x, sizeof(float) * (size_t)V);
  if (cfg->top_p < 1.0f) {
    top_p_info info = top_p_filter(x, V, cfg->top_p, order, buf);
    if (info.n > 0) {
      double a = (double)cfg->top_p - info.a_last;
      double b = info.a_next - (double)cfg->top_p;
      margin_p = a < b ? a : b;
    }
  }

  double margin_u = INFINITY;
  int32_t t = sample_inverse_cdf(x, V, u, order, buf, &margin_u);
  if (t < 0) { /* every score removed: same as greedy */
    t = argmax_lowest(x, V);
    margin_u = INFINITY;
  }
  res->token = t;
  res->margin = margin_p < margin_u ? margin_p : margin_u;
  for (int32_t v = 0; v < V; ++v) res->n_finite += x[v] > -INFINITY;

  /* Admissible ids: every token that some perturbation of the cumulative
   * sums by at most eps (normalized) for the top_p decisions and eps * W'
   * for the sample could select. */
  {
    const double eps = 1e-6;
    int32_t n = sorted_finite(pre, V, order);
    int32_t na = 0;
    if (n == 0) {
      res->admissible[na++] = t;
      res->keep_min = res->keep_max = 0;
    } else {
      double m = (double)pre[order[0]];
      double W = 0.0;
      for (int32_t j = 0; j < n; ++j) {
        buf[j] = exp((double)pre[order[j]] - m);
        W += buf[j];
      }
      int32_t kmin = n, kmax = n;
      if (cfg->top_p < 1.0f) {
        double run = 0.0;
        int32_t must = 0, may = 0;
        for (int32_t j = 0; j < n; ++j) {
          double A = run / W;
          if (A + eps < (double)cfg->top_p) must = j + 1;
          if (A - eps < (double)cfg->top_p) may = j + 1;
          run += buf[j];
        }
        kmin = must < 1 ? 1 : must;
        kmax = may < 1 ? 1 : may;
      }
      res->keep_min = kmin;
      res->keep_max = kmax;
      if (kmax - kmin > 4 * ORACLE_MAX_ADMISSIBLE) kmax = kmin + 4 * ORACLE_MAX_ADMISSIBLE;
      for (int32_t K = kmin; K <= kmax; ++K) {
        double Wp = 0.0;
        for (int32_t j = 0; j < K; ++j) Wp += buf[j];
        double target = (double)u * Wp, tol = eps * Wp, C = 0.0;
        for (int32_t j = 0; j < K; ++j) {
          double lo = C;
          C += buf[j];
          int hit = (C > target - tol) && (lo <= target + tol);
          if (j == K - 1 && C <= target + tol) hit = 1;
          if (hit) {
            int dup = 0;
            for (int32_t q = 0; q < na; ++q) dup |= res->admissible[q] == order[j];
            if (!dup && na < ORACLE_MAX_ADMISSIBLE) res->admissible[na++] = order[j];
          }
          if (lo > target + tol) break;
        }
      }
    }
    res->n_admissible = na;
  }
  free(pre);
  res->logprob = token_logprob(x, V, t);
  if (x_out) memcpy(x_out, x, sizeof(float) * (size_t)V);
  free(x); free(order); free(buf);
  return 0;
}

/* ------------------------------------------------------------------ */
/* [A] "Greedy decoding with assisted generation", steps 4-6: the selected
 * tokens sel[0..k] against the k drafts. */
static void match_drafts(int32_t k, const int32_t *cand, const int32_t *sel, int32_t *n_match,
                         int32_t *tokens, int32_t *next, int32_t *k_next) {
  /* step 4: left to right, stop at the first mismatch */
  int32_t n = 0;
  while (n < k && cand[n] == sel[n]) ++n;
  /* step 5: keep the matches plus the first divergent token */
  for (int32_t j = 0; j <= k; ++j) tokens[j] = j <= n ? sel[j] : -1;
  *n_match = n;
  *next = sel[n];
  /* step 6: +2 when every candidate matched, else -1 (floor 1) */
  *k_next = (n == k) ? k + 2 : (k - 1 > 1 ? k - 1 : 1);
}

/* [A] "Greedy decoding with assisted generation", steps 3-6, for one
 * batch row.  logits: (k+1) rows of V logits, row stride `stride` elements;
 * cand: the k draft ids.  Outputs: the match count, the kept tokens
 * (n_match + 1 of them, then -1), the first divergent (or bonus) token and
 * the next draft count. */
void oracle_verify_row(const void *logits, int32_t dtype, int32_t k, int32_t V,
                       int64_t stride, const int32_t *cand, int32_t *n_match,
                       int32_t *tokens, int32_t *next, int32_t *k_next) {
  const size_t esize = dtype == 0 ? 4 : 2;
  float *x = (float *)malloc(sizeof(float) * (size_t)V);
  int32_t *sel = (int32_t *)calloc((size_t)(k + 1), sizeof(int32_t));
  if (!x || !sel) { free(x); free(sel); *n_match = -1; return; }
  for (int32_t j = 0; j <= k; ++j) {
    const char *row = (const char *)logits + (size_t)j * (size_t)stride * esize;
    for (int32_t v = 0; v < V; ++v) x[v] = load_logit(row, dtype, v);
    sel[j] = argmax_lowest(x, V); /* step 3: .argmax() per position */
  }
  match_drafts(k, cand, sel, n_match, tokens, next, k_next);
  free(x);
  free(sel);
}

/* [A] steps 3-6 with the token selection method of the step (the
 * processors, and for sampling the warpers and a draw: ".multinomial() for
 * sampling"; "Sample with assisted generation").  Position j was computed
 * by the model after the history h[0..L) and the drafts cand[0..j), so its
 * selection sees that extended history and the length L + j (the length
 * rules of [T] "Lengths" move with it); its draw takes the uniform u[j].  A
 * padding row (L == 0) stays one at every position.  Returns 0, or -1 on
 * allocation failure. */
int oracle_verify_select_row(const void *logits, int32_t k, int64_t stride, const int32_t *h,
                             int32_t L, int32_t P, int32_t M, const oracle_cfg *cfg,
                             const float *u, const int32_t *cand, int32_t *n_match,
                             int32_t *tokens, int32_t *next, int32_t *k_next) {
  const size_t esize = cfg->dtype == 0 ? 4 : 2;
  int32_t *hx = (int32_t *)malloc(sizeof(int32_t) * (size_t)(L + k + 1));
  int32_t *sel = (int32_t *)calloc((size_t)(k + 1), sizeof(int32_t));
  if (!hx || !sel) { free(hx); free(sel); return -1; }
  for (int32_t i = 0; i < L; ++i) hx[i] = h[i];
  for (int32_t i = 0; i < k; ++i) hx[L + i] = cand[i];
  for (int32_t j = 0; j <= k; ++j) {
    const char *row = (const char *)logits + (size_t)j * (size_t)stride * esize;
    oracle_row_result r;
    if (oracle_select_row(row, hx, L == 0 ? 0 : L + j, P, M, cfg, u ? u[j] : 0.0f, NULL, &r) != 0) {
      free(hx);
      free(sel);
      return -1;
    }
    sel[j] = r.token;
  }
  match_drafts(k, cand, sel, n_match, tokens, next, k_next);
  free(hx);
  free(sel);
  return 0;
}

/* ------------------------------------------------------------------ */
/* [T] the beam paragraph under "Log-probabilities": one step of beam
 * search for one prompt of nb beams.  Each beam row takes the log-softmax
 * of its logits (read as renormalize_logits above: (x - m) - ls in binary32
 * with ls from binary64), then the processors with removed ids at the
 * smallest finite value, then adds the beam's score; a score never goes
 * below the smallest finite value.  Of the nb * V candidates (beam j, id v)
 * at flattened index j * V + v, the best K are kept, by score descending
 * and, among equal scores, by flattened index ascending.  On the first step
 * only beam 0 counts (all beams of a prompt are equal); a padding beam row
 * (L == 0) gives no candidates.  Slots past the candidates there are take
 * score -inf, beam -1 and id -1.
 *
 * logits: nb rows of V logits at `stride` elements; h: nb histories at
 * `hstride`; L, P, M: per beam.  Returns 0, or -1 on allocation failure. */
typedef struct {
  float score;
  int64_t flat;
} beam_cand;

static int cmp_beam_cand(const void *a, const void *b) {
  const beam_cand *x = (const beam_cand *)a, *y = (const beam_cand *)b;
  if (x->score > y->score) return -1;
  if (x->score < y->score) return 1;
  return (x->flat > y->flat) - (x->flat < y->flat);
}

int oracle_beam_step(const void *logits, int64_t stride, int32_t nb, const int32_t *h,
                     int64_t hstride, const int32_t *L, const int32_t *P, const int32_t *M,
                     const oracle_cfg *cfg, const float *beam_scores, int32_t first_step,
                     int32_t K, float *out_scores, int32_t *out_beams, int32_t *out_tokens) {
  const int32_t V = cfg->vocab;
  const size_t esize = cfg->dtype == 0 ? 4 : 2;
  float *x = (float *)malloc(sizeof(float) * (size_t)V);
  beam_cand *c = (beam_cand *)malloc(sizeof(beam_cand) * (size_t)nb * (size_t)V);
  if (!x || !c) { free(x); free(c); return -1; }
  int64_t n = 0;
  for (int32_t j = 0; j < nb; ++j) {
    if ((first_step && j > 0) || L[j] == 0) continue;
    const char *row = (const char *)logits + (size_t)j * (size_t)stride * esize;
    for (int32_t v = 0; v < V; ++v) x[v] = load_logit(row, cfg->dtype, v);
    renormalize(x, V);  /* the log-softmax of the logits */
    apply_processors(x, V, h + (size_t)j * (size_t)hstride, L[j], P[j], M[j], cfg, -FLT_MAX);
    for (int32_t v = 0; v < V; ++v) {
      float sc = x[v] + beam_scores[j];
      if (!(sc >= -FLT_MAX)) sc = -FLT_MAX;  /* never below the smallest finite value */
      c[n].score = sc;
      c[n].flat = (int64_t)j * V + v;
      ++n;
    }
  }
  qsort(c, (size_t)n, sizeof(beam_cand), cmp_beam_cand);
  for (int32_t q = 0; q < K; ++q) {
    if (q < n) {
      out_scores[q] = c[q].score;
      out_beams[q] = (int32_t)(c[q].flat / V);
      out_tokens[q] = (int32_t)(c[q].flat % V);
    } else {
      out_scores[q] = -INFINITY;
      out_beams[q] = -1;
      out_tokens[q] = -1;
    }
  }
  free(x);
  free(c);
  return 0;
}

/* Bitmask of an id list (ids outside [0, V) are ignored): bit v of word
 * v / 32 is set iff v is listed. */
void oracle_mask_build(int32_t V, const int32_t *ids, int32_t n, uint32_t *mask) {
  int32_t words = (V + 31) / 32;
  for (int32_t w = 0; w < words; ++w) mask[w] = 0u;
  for (int32_t i = 0; i < n; ++i)
    if (in_vocab(ids[i], V)) mask[ids[i] >> 5] |= 1u << (ids[i] & 31);
}

/* The end of one decode step for one row ("Transmuter.Generation
 * (transmuter v2.0.0)", function doc of generate/5, the on_token callback
 * and the return value: a row with no new token reports -1, a finished row
 * has no more tokens, the eos token is not returned; mlxcel inference
 * pipeline, decode loop, "EOS 감지와 정지": a sampled id in the merged stop
 * set ends the row and is not emitted, and the loop also ends at the
 * maximum length).  t: the step's selected token (-1: none); L: the row's
 * length before it; M: its maximum length; *fin: 0 or 1, updated. */
int32_t oracle_finish_row(int32_t t, int32_t L, int32_t M, const int32_t *eos, int32_t n_eos,
                          uint8_t *fin) {
  if (*fin || t < 0) { /* no new token: nothing more from this row */
    *fin = 1;
    return -1;
  }
  for (int32_t i = 0; i < n_eos; ++i) {
    if (eos[i] == t) { /* a stop id: the row ends, the id is not emitted */
      *fin = 1;
      return -1;
    }
  }
  /* the token is emitted; the row is then L + 1 long */
  *fin = (int64_t)L + 1 >= (int64_t)M ? 1 : 0;
  return t;
}
