/*
 * oracle.c -- plain, slow, single-threaded fp64 CPU oracle for the
 * speculative-decoding verify step.
 *
 * TEST INFRASTRUCTURE ONLY: the test suite, the package smoke check and the
 * benchmark's CPU-baseline leg are the only code allowed to load it.  It shares
 * nothing with the GPU library.
 *
 * Source of the method: the encyclopedia entry "Speculative decoding"
 * (glopedia, 推测解码), section "Basic steps of proposal and verification"
 * (提议与核验的基本步骤):
 *   - the draft token x at position i is accepted with probability
 *     min(1, p(x)/q(x)), p and q being the target's and the proposer's
 *     conditional probabilities under the sampling settings actually in force;
 *   - after the first rejection no later candidate is accepted, and the
 *     rejected position is redrawn from the normalised positive residual
 *     max(0, p - q);
 *   - if every candidate passes, one extra token is drawn from the target;
 *   - in greedy decoding the draft is compared with the target's most
 *     probable token and the first mismatch is replaced by that token;
 *   - temperature, top-k and nucleus (top-p) rules must be applied in the same
 *     way to p and q.
 *
 * Where the entry is silent this file takes these readings (the GPU library
 * takes the same ones):
 *   R1 target rows are k+1 per sequence, row k is the bonus distribution;
 *   R2 uniforms are [B][k+1]: column j is the accept draw of position j,
 *      column k the single draw for whichever token is sampled;
 *   R3 accept iff u < alpha (strict), so P(accept) = alpha for u in [0,1);
 *   R4 q(x) = 0 gives alpha = 1 if p(x) > 0, else 0;
 *   R5 sampling is an inverse CDF in ascending vocabulary order: the first
 *      index whose running sum exceeds u * S; if rounding leaves none, the
 *      last index with positive mass;
 *   R6 a residual with zero total mass falls back to p at that position;
 *   R7 temperature T > 0 divides (logit - max logit);
 *   R8 top-k keeps every logit >= the k-th largest (duplicates counted);
 *   R9 order is temperature -> top-k -> top-p; top-p uses probabilities
 *      renormalised over the top-k set, keeps the shortest descending prefix
 *      whose mass reaches top_p, ties at the cut kept;
 *   R12 -inf logits have probability 0; NaN, +inf or a row without a finite
 *      logit make the row invalid, and a position is ill-formed when one of
 *      its rows (target and, stochastic, draft) is invalid or its draft token
 *      lies outside [0, V).  Positions are examined in order and the first
 *      rejection ends the walk, so a sequence is invalid (accepted length -1)
 *      only when an ill-formed position comes before any rejection, or every
 *      candidate passes and the bonus row is invalid; rows past the stop are
 *      never consulted;
 *   R13 everything is computed in double precision on exactly decoded inputs;
 *   R14 alpha is reported for every position, past the stop too, and is NaN
 *      at an ill-formed position.
 */
#include "oracle.h"

#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

/* ---- exact decoding of one logit ---------------------------------------- */

static double decode_logit(const void* base, int dtype, long long idx) {
  if (dtype == ORC_BF16) {
    uint16_t half = ((const uint16_t*)base)[idx];
    uint32_t word = ((uint32_t)half) << 16; /* bf16 is the top half of f32 */
    float f;
    memcpy(&f, &word, sizeof f);
    return (double)f;
  }
  return (double)((const float*)base)[idx];
}

static void decode_row(const void* base, int dtype, long long offset, int V,
                       double* out) {
  for (int i = 0; i < V; i++) out[i] = decode_logit(base, dtype, offset + i);
}

/* ---- logits processing --------------------------------------------------- */

typedef struct {
  int valid;
  double max_logit;
  double threshold;
  double log_norm;
  double mass_above_cut; /* top-p mass strictly above the cut value (or NaN) */
  double mass_at_cut;    /* top-p mass at or above the cut value (or NaN)    */
} row_result;

static int by_value_descending(const void* a, const void* b) {
  double x = *(const double*)a, y = *(const double*)b;
  if (x > y) return -1;
  if (x < y) return 1;
  return 0;
}

/* Temperature, then top-k, then top-p, then normalisation (R7-R9).  prob gets
 * p for every index; scratch must hold V doubles. */
static row_result process_logits(const double* l, int V, double T, int top_k,
                                 double top_p, double* prob, double* scratch) {
  row_result res;
  res.valid = 0;
  res.max_logit = res.threshold = res.log_norm = NAN;
  res.mass_above_cut = res.mass_at_cut = NAN;

  double m = -INFINITY;
  for (int i = 0; i < V; i++) {
    if (isnan(l[i]) || l[i] == INFINITY) return res; /* R12 */
    if (l[i] > m) m = l[i];
  }
  if (m == -INFINITY) return res; /* R12: no finite logit */

  /* top-k: the top_k-th largest logit, duplicates counted (R8). */
  double t_k = -INFINITY;
  if (top_k > 0 && top_k < V) {
    memcpy(scratch, l, (size_t)V * sizeof(double));
    qsort(scratch, (size_t)V, sizeof(double), by_value_descending);
    t_k = scratch[top_k - 1];
  }

  /* top-p over the top-k set, probabilities renormalised over that set (R9). */
  double t_p = -INFINITY;
  if (top_p < 1.0) {
    int n_kept = 0;
    for (int i = 0; i < V; i++)
      if (l[i] >= t_k) scratch[n_kept++] = l[i];
    qsort(scratch, (size_t)n_kept, sizeof(double), by_value_descending);
    double z_k = 0.0;
    for (int j = 0; j < n_kept; j++) z_k += exp((scratch[j] - m) / T);
    double cum = 0.0;
    int cut = n_kept - 1; /* if rounding never reaches top_p, keep all */
    for (int j = 0; j < n_kept; j++) {
      cum += exp((scratch[j] - m) / T) / z_k;
      if (cum >= top_p) {
        cut = j;
        break;
      }
    }
    t_p = scratch[cut];
    double above = 0.0, at = 0.0;
    for (int j = 0; j < n_kept; j++) {
      double pi = exp((scratch[j] - m) / T) / z_k;
      if (scratch[j] > t_p) above += pi;
      if (scratch[j] >= t_p) at += pi;
    }
    res.mass_above_cut = above;
    res.mass_at_cut = at;
  }

  double thr = t_k > t_p ? t_k : t_p;
  double z = 0.0;
  for (int i = 0; i < V; i++)
    if (l[i] >= thr) z += exp((l[i] - m) / T);
  for (int i = 0; i < V; i++)
    prob[i] = (l[i] >= thr) ? exp((l[i] - m) / T) / z : 0.0;

  res.valid = 1;
  res.max_logit = m;
  res.threshold = thr;
  res.log_norm = log(z);
  return res;
}

/* R5: first index whose running sum exceeds u * S; else last positive index. */
static int inverse_cdf(const double* r, int V, double u, double* total_out,
                       double* before_out, double* at_out) {
  double S = 0.0;
  for (int i = 0; i < V; i++) S += r[i];
  double target = u * S;
  double run = 0.0;
  int pick = -1;
  double before = 0.0;
  for (int i = 0; i < V; i++) {
    before = run;
    run += r[i];
    if (run > target) {
      pick = i;
      break;
    }
  }
  if (pick < 0) {
    for (int i = V - 1; i >= 0; i--)
      if (r[i] > 0.0) {
        pick = i;
        break;
      }
    before = 0.0;
    for (int i = 0; i < pick; i++) before += r[i];
    run = before + (pick >= 0 ? r[pick] : 0.0);
  }
  if (total_out) *total_out = S;
  if (before_out) *before_out = before;
  if (at_out) *at_out = run;
  return pick;
}

/* R3, R4: the ratio test's acceptance probability. */
static double acceptance_probability(double p, double q) {
  if (q > 0.0) {
    double a = p / q;
    return a < 1.0 ? a : 1.0;
  }
  return p > 0.0 ? 1.0 : 0.0;
}

/* ---- public entry points -------------------------------------------------- */

int orc_process_row(const void* row, int dtype, int V, double temperature,
                    int top_k, double top_p, double* prob, double* stats) {
  double* l = (double*)malloc((size_t)V * sizeof(double));
  double* scratch = (double*)malloc((size_t)V * sizeof(double));
  double* p = prob ? prob : (double*)malloc((size_t)V * sizeof(double));
  if (!l || !scratch || !p) {
    free(l);
    free(scratch);
    if (!prob) free(p);
    return -1;
  }
  decode_row(row, dtype, 0, V, l);
  row_result r = process_logits(l, V, temperature, top_k, top_p, p, scratch);
  if (stats) {
    stats[0] = r.max_logit;
    stats[1] = r.threshold;
    stats[2] = r.log_norm;
    stats[3] = r.mass_above_cut;
    stats[4] = r.mass_at_cut;
  }
  free(l);
  free(scratch);
  if (!prob) free(p);
  return r.valid;
}

int orc_sample_row(const void* row, int dtype, int V, double temperature,
                   int top_k, double top_p, double u) {
  double* l = (double*)malloc((size_t)V * sizeof(double));
  double* scratch = (double*)malloc((size_t)V * sizeof(double));
  double* p = (double*)malloc((size_t)V * sizeof(double));
  int pick = -1;
  if (l && scratch && p) {
    decode_row(row, dtype, 0, V, l);
    row_result r = process_logits(l, V, temperature, top_k, top_p, p, scratch);
    if (r.valid) pick = inverse_cdf(p, V, u, NULL, NULL, NULL);
  }
  free(l);
  free(scratch);
  free(p);
  return pick;
}

/* First maximum; -1 when the row holds NaN/+inf or no finite logit (R12). */
static int first_argmax(const double* l, int V) {
  int best = -1;
  for (int i = 0; i < V; i++) {
    if (isnan(l[i]) || l[i] == INFINITY) return -1;
    if (l[i] == -INFINITY) continue;
    if (best < 0 || l[i] > l[best]) best = i;
  }
  return best;
}

int orc_argmax_row(const void* row, int dtype, int V) {
  double* l = (double*)malloc((size_t)V * sizeof(double));
  if (!l) return -1;
  decode_row(row, dtype, 0, V, l);
  int a = first_argmax(l, V);
  free(l);
  return a;
}

static int near(double a, double b) { return fabs(a - b) <= 1e-6; }

int orc_verify_stochastic(const void* target, long long t_seq, long long t_pos,
                          const void* draft, long long d_seq, long long d_pos,
                          int dtype, const int* tokens, const float* u, int B,
                          int k, int V, double temperature, int top_k,
                          double top_p, int* accepted_len, int* out_tokens,
                          double* accept_prob, int* flags) {
  double* P = (double*)malloc((size_t)(k + 1) * V * sizeof(double));
  double* Q = (double*)malloc((size_t)k * V * sizeof(double));
  double* l = (double*)malloc((size_t)V * sizeof(double));
  double* scratch = (double*)malloc((size_t)V * sizeof(double));
  double* r = (double*)malloc((size_t)V * sizeof(double));
  row_result* pres = (row_result*)malloc((size_t)(k + 1) * sizeof(row_result));
  row_result* qres = (row_result*)malloc((size_t)k * sizeof(row_result));
  double* alpha = (double*)malloc((size_t)k * sizeof(double));
  if (!P || !Q || !l || !scratch || !r || !pres || !qres || !alpha) {
    free(P), free(Q), free(l), free(scratch), free(r), free(pres), free(qres);
    free(alpha);
    return -1;
  }

  for (int b = 0; b < B; b++) {
    for (int j = 0; j <= k; j++) {
      decode_row(target, dtype, b * t_seq + j * t_pos, V, l);
      pres[j] = process_logits(l, V, temperature, top_k, top_p,
                               P + (size_t)j * V, scratch);
    }
    for (int j = 0; j < k; j++) {
      decode_row(draft, dtype, b * d_seq + j * d_pos, V, l);
      qres[j] = process_logits(l, V, temperature, top_k, top_p,
                               Q + (size_t)j * V, scratch);
    }
    /* R14: the ratio test's alpha at every well-formed position. */
    for (int j = 0; j < k; j++) {
      int x = tokens[(size_t)b * k + j];
      int formed = pres[j].valid && qres[j].valid && x >= 0 && x < V;
      alpha[j] = formed ? acceptance_probability(P[(size_t)j * V + x],
                                                 Q[(size_t)j * V + x])
                        : NAN;
      if (accept_prob) accept_prob[(size_t)b * k + j] = alpha[j];
    }
    /* Positions in order; the first rejection stops the walk (R12). */
    const float* ub = u + (size_t)b * (k + 1);
    int n = k, valid = 1;
    for (int j = 0; j < k; j++) {
      if (isnan(alpha[j])) {
        valid = 0;
        break;
      }
      if (!((double)ub[j] < alpha[j])) {
        n = j;
        break;
      }
    }
    if (valid && n == k && !pres[k].valid) valid = 0;
    int* out = out_tokens + (size_t)b * (k + 1);
    if (!valid) {
      accepted_len[b] = -1;
      for (int j = 0; j <= k; j++) out[j] = -1;
      if (flags) flags[b] = 0;
      continue;
    }

    /* Correction: residual max(0, p - q) at the rejected position, or the
     * bonus distribution p_k when every candidate passed (R6 fallback). */
    const double* pn = P + (size_t)n * V;
    if (n < k) {
      const double* qn = Q + (size_t)n * V;
      double S = 0.0;
      for (int i = 0; i < V; i++) {
        double d = pn[i] - qn[i];
        r[i] = d > 0.0 ? d : 0.0;
        S += r[i];
      }
      if (S == 0.0)
        for (int i = 0; i < V; i++) r[i] = pn[i];
    } else {
      for (int i = 0; i < V; i++) r[i] = pn[i];
    }
    double S, before, at;
    int emitted = inverse_cdf(r, V, (double)ub[k], &S, &before, &at);

    accepted_len[b] = n;
    for (int j = 0; j < n; j++) out[j] = tokens[(size_t)b * k + j];
    out[n] = emitted;
    for (int j = n + 1; j <= k; j++) out[j] = -1;

    if (flags) {
      int f = 0;
      int last = n < k ? n : k - 1;
      for (int j = 0; j <= last; j++)
        if (near((double)ub[j], alpha[j])) f |= ORC_NEAR_ACCEPT;
      if (S > 0.0 && (near((double)ub[k], before / S) || near((double)ub[k], at / S)))
        f |= ORC_NEAR_SAMPLE;
      if (top_p < 1.0) {
        for (int j = 0; j <= n; j++)
          if (near(pres[j].mass_above_cut, top_p) || near(pres[j].mass_at_cut, top_p))
            f |= ORC_NEAR_TOPP;
        for (int j = 0; j <= last; j++)
          if (near(qres[j].mass_above_cut, top_p) || near(qres[j].mass_at_cut, top_p))
            f |= ORC_NEAR_TOPP;
      }
      flags[b] = f;
    }
  }

  free(P), free(Q), free(l), free(scratch), free(r), free(pres), free(qres);
  free(alpha);
  return 0;
}

int orc_verify_greedy(const void* target, long long t_seq, long long t_pos,
                      int dtype, const int* tokens, int B, int k, int V,
                      int* accepted_len, int* out_tokens) {
  double* l = (double*)malloc((size_t)V * sizeof(double));
  int* best = (int*)malloc((size_t)(k + 1) * sizeof(int));
  if (!l || !best) {
    free(l), free(best);
    return -1;
  }
  for (int b = 0; b < B; b++) {
    for (int j = 0; j <= k; j++) {
      decode_row(target, dtype, b * t_seq + j * t_pos, V, l);
      best[j] = first_argmax(l, V);
    }
    /* Positions in order up to the first mismatch (R12). */
    int n = k, valid = 1;
    for (int j = 0; j < k; j++) {
      int x = tokens[(size_t)b * k + j];
      if (best[j] < 0 || x < 0 || x >= V) {
        valid = 0;
        break;
      }
      if (x != best[j]) {
        n = j;
        break;
      }
    }
    if (valid && n == k && best[k] < 0) valid = 0;
    int* out = out_tokens + (size_t)b * (k + 1);
    if (!valid) {
      accepted_len[b] = -1;
      for (int j = 0; j <= k; j++) out[j] = -1;
      continue;
    }
    accepted_len[b] = n;
    for (int j = 0; j < n; j++) out[j] = tokens[(size_t)b * k + j];
    out[n] = best[n];
    for (int j = n + 1; j <= k; j++) out[j] = -1;
  }
  free(l), free(best);
  return 0;
}
