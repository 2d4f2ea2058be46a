/*
 * attn_oracle.c -- fp64 CPU oracle for softmax attention.
 *
 * TEST INFRASTRUCTURE ONLY (see attn_oracle.h for the definition it follows,
 * with the page citations).  Plain loops, one output row at a time: the full
 * row of logits z_i. is materialised, then the max, the denominator and the
 * weighted sum of values are taken exactly as the definition states.  No
 * tiling, no online rescaling, no folding of the RBF distance.
 */
#include "attn_oracle.h"

#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

static double load_elem(int dtype, const void* p, size_t idx) {
  if (dtype == ORACLE_BF16) {
    uint32_t bits = ((uint32_t)((const uint16_t*)p)[idx]) << 16;
    float f;
    memcpy(&f, &bits, sizeof f);
    return (double)f;
  }
  if (dtype == ORACLE_F32) return (double)((const float*)p)[idx];
  return ((const double*)p)[idx];
}

int oracle_visible(int L, int S, int causal, int window, int n_reg, int i, int j) {
  if (j < n_reg) return 1;                 /* register tokens: always visible */
  long long r = (long long)j - n_reg;      /* position among the real keys */
  long long ip = (long long)i + ((long long)S - n_reg - L);  /* bottom-right */
  if (causal && r > ip) return 0;
  if (window > 0 && ip - r >= window) return 0;
  return 1;
}

int oracle_num_threads(int threads) {
#ifdef _OPENMP
  return threads > 0 ? threads : omp_get_max_threads();
#else
  (void)threads;
  return 1;
#endif
}

/* logit of query row qoff against key row koff, definition form */
static double logit(int dtype, const void* q, size_t qoff, const void* k, size_t koff, int E,
                    int mode, double scale, double gamma) {
  double acc = 0.0;
  if (mode == ORACLE_DOT) {
    for (int e = 0; e < E; ++e) acc += load_elem(dtype, q, qoff + e) * load_elem(dtype, k, koff + e);
    return scale * acc;
  }
  for (int e = 0; e < E; ++e) {
    double d = load_elem(dtype, q, qoff + e) - load_elem(dtype, k, koff + e);
    acc += d * d;
  }
  return -gamma * acc;
}

int oracle_attn_rows(int dtype, int N, int Hq, int Hkv, int L, int S, int E,
                     const void* q, const void* k, const void* v,
                     int mode, double scale, double gamma,
                     int causal, int window, int n_reg, const double* sink,
                     long long nrows, const long long* rows,
                     double* o, double* lse, double* p, int threads) {
  return oracle_attn_rows_ex(dtype, N, Hq, Hkv, L, S, E, q, k, v, mode, scale, gamma, causal, window, n_reg,
                             sink, ORACLE_BIAS_NONE, NULL, 0, 0, NULL, nrows, rows, o, lse, p, threads);
}

/* user bias of pair (n, h, i, j): 0 when absent; -inf for a masked-out pair */
static double user_bias(int kind, const void* bias, long long sn, long long sh, int S, int n, int h, int i,
                        int j) {
  if (kind == ORACLE_BIAS_NONE) return 0.0;
  const long long idx = (long long)n * sn + (long long)h * sh + (long long)i * S + j;
  if (kind == ORACLE_BIAS_F32) return (double)((const float*)bias)[idx];
  return ((const unsigned char*)bias)[idx] ? 0.0 : -INFINITY;
}

int oracle_attn_rows_ex(int dtype, int N, int Hq, int Hkv, int L, int S, int E,
                        const void* q, const void* k, const void* v,
                        int mode, double scale, double gamma,
                        int causal, int window, int n_reg, const double* sink,
                        int bias_kind, const void* bias, long long bias_sn, long long bias_sh,
                        const int* key_len,
                        long long nrows, const long long* rows,
                        double* o, double* lse, double* p, int threads) {
  if (dtype < ORACLE_BF16 || dtype > ORACLE_F64) return -1;
  if (bias_kind < ORACLE_BIAS_NONE || bias_kind > ORACLE_BIAS_BOOL) return -1;
  if (bias_kind != ORACLE_BIAS_NONE && (!bias || bias_sn < 0 || bias_sh < 0)) return -3;
  if (mode != ORACLE_DOT && mode != ORACLE_RBF) return -1;
  if (N <= 0 || Hq <= 0 || Hkv <= 0 || L <= 0 || S < 0 || E <= 0) return -2;
  if (Hq % Hkv != 0) return -2;
  if (n_reg < 0 || n_reg > S) return -2;
  if (!q || !k || !v || !o || !lse) return -3;
  const long long total = (long long)N * Hq * L;
  if (!rows && nrows != total) return -2;
  for (long long r = 0; rows && r < nrows; ++r)
    if (rows[r] < 0 || rows[r] >= total) return -2;

  const int G = Hq / Hkv;
  const int nt = oracle_num_threads(threads);
  int failed = 0;

#pragma omp parallel num_threads(nt)
  {
    double* z = (double*)malloc(sizeof(double) * (size_t)(S > 0 ? S : 1));
    if (!z) {
#pragma omp atomic write
      failed = 1;
    }
#pragma omp for schedule(dynamic, 4)
    for (long long r = 0; r < nrows; ++r) {
      if (!z) continue;
      const long long flat = rows ? rows[r] : r;
      const int i = (int)(flat % L);
      const long long nh = flat / L;
      const int h = (int)(nh % Hq);
      const int n = (int)(nh / Hq);
      const int kh = h / G;
      const size_t qoff = (size_t)flat * E;
      const size_t kvrow0 = ((size_t)n * Hkv + kh) * (size_t)S;
      double* orow = o + (size_t)r * E;
      double* prow = p ? p + (size_t)r * S : NULL;

      /* z_ij = l_ij + B_ij: B_ij = -inf for a pair the rule hides or a padding
         key, else the user bias (0 without one); M_i = row max (with sink) */
      double M = -INFINITY;
      for (int j = 0; j < S; ++j) {
        const int padded = key_len && j >= n_reg && (j - n_reg) >= key_len[n];
        const double b = user_bias(bias_kind, bias, bias_sn, bias_sh, S, n, h, i, j);
        if (oracle_visible(L, S, causal, window, n_reg, i, j) && !padded && b != -INFINITY)
          z[j] = logit(dtype, q, qoff, k, (kvrow0 + j) * E, E, mode, scale, gamma) + b;
        else
          z[j] = -INFINITY;
        if (z[j] > M) M = z[j];
      }
      if (sink && sink[h] > M) M = sink[h];

      if (M == -INFINITY) { /* nothing visible and no sink: O = 0, LSE = -inf */
        for (int e = 0; e < E; ++e) orow[e] = 0.0;
        lse[r] = -INFINITY;
        if (prow) for (int j = 0; j < S; ++j) prow[j] = 0.0;
        continue;
      }

      double D = 0.0;
      for (int j = 0; j < S; ++j) D += exp(z[j] - M);
      if (sink) D += exp(sink[h] - M);

      for (int e = 0; e < E; ++e) orow[e] = 0.0;
      for (int j = 0; j < S; ++j) {
        const double pij = exp(z[j] - M) / D;
        if (prow) prow[j] = pij;
        const size_t voff = (kvrow0 + j) * E;
        for (int e = 0; e < E; ++e) orow[e] += pij * load_elem(dtype, v, voff + e);
      }
      lse[r] = M + log(D);
    }
    free(z);
  }
  return failed ? -4 : 0;
}

/* ------------------------------------------------------------------------ backward */

/* d z_ij / d q_i (into g[E], scaled by w): dot: scale*k_j; rbf: -2*gamma*(q_i - k_j) */
static void dlogit_dq(int dtype, const void* q, size_t qoff, const void* k, size_t koff, int E, int mode,
                      double scale, double gamma, double w, double* g) {
  for (int e = 0; e < E; ++e) {
    const double ke = load_elem(dtype, k, koff + e);
    if (mode == ORACLE_DOT)
      g[e] += w * scale * ke;
    else
      g[e] += w * (-2.0 * gamma) * (load_elem(dtype, q, qoff + e) - ke);
  }
}

/* d z_ij / d k_j (into g[E], scaled by w): dot: scale*q_i; rbf: 2*gamma*(q_i - k_j) */
static void dlogit_dk(int dtype, const void* q, size_t qoff, const void* k, size_t koff, int E, int mode,
                      double scale, double gamma, double w, double* g) {
  for (int e = 0; e < E; ++e) {
    const double qe = load_elem(dtype, q, qoff + e);
    if (mode == ORACLE_DOT)
      g[e] += w * scale * qe;
    else
      g[e] += w * (2.0 * gamma) * (qe - load_elem(dtype, k, koff + e));
  }
}

int oracle_attn_bwd(int dtype, int N, int Hq, int Hkv, int L, int S, int E,
                    const void* q, const void* k, const void* v, const void* dout,
                    int mode, double scale, double gamma,
                    int causal, int window, int n_reg, const double* sink,
                    long long nq, const long long* qrows, double* dq,
                    long long nk, const long long* krows, double* dk, double* dv,
                    double* dsink, double* lse_out, double* delta_out, int threads) {
  if (dtype < ORACLE_BF16 || dtype > ORACLE_F64) return -1;
  if (mode != ORACLE_DOT && mode != ORACLE_RBF) return -1;
  if (N <= 0 || Hq <= 0 || Hkv <= 0 || L <= 0 || S < 0 || E <= 0) return -2;
  if (Hq % Hkv != 0) return -2;
  if (n_reg < 0 || n_reg > S) return -2;
  if (!q || !k || !v || !dout) return -3;
  const long long total_q = (long long)N * Hq * L;
  const long long total_k = (long long)N * Hkv * S;
  if (!qrows && dq && nq != total_q) return -2;
  if (!krows && (dk || dv) && nk != total_k) return -2;
  for (long long r = 0; qrows && r < nq; ++r)
    if (qrows[r] < 0 || qrows[r] >= total_q) return -2;
  for (long long r = 0; krows && r < nk; ++r)
    if (krows[r] < 0 || krows[r] >= total_k) return -2;
  const int G = Hq / Hkv;
  const int nt = oracle_num_threads(threads);

  /* Phase 1, every row: LSE_i of the forward (definition form, sink included)
     and D_i = dO_i . O_i with O_i the exact forward output. */
  double* LSE = (double*)malloc(sizeof(double) * (size_t)total_q);
  double* DEL = (double*)malloc(sizeof(double) * (size_t)total_q);
  if (!LSE || !DEL) {
    free(LSE);
    free(DEL);
    return -4;
  }
  int failed = 0;
#pragma omp parallel num_threads(nt)
  {
    double* z = (double*)malloc(sizeof(double) * (size_t)(S > 0 ? S : 1));
    double* o = (double*)malloc(sizeof(double) * (size_t)E);
    if (!z || !o) {
#pragma omp atomic write
      failed = 1;
    }
#pragma omp for schedule(dynamic, 4)
    for (long long flat = 0; flat < total_q; ++flat) {
      if (!z || !o) continue;
      const int i = (int)(flat % L);
      const long long nh = flat / L;
      const int h = (int)(nh % Hq), n = (int)(nh / Hq);
      const size_t kvrow0 = ((size_t)n * Hkv + h / G) * (size_t)S;
      double M = -INFINITY;
      for (int j = 0; j < S; ++j) {
        z[j] = oracle_visible(L, S, causal, window, n_reg, i, j)
                   ? logit(dtype, q, (size_t)flat * E, k, (kvrow0 + j) * E, E, mode, scale, gamma)
                   : -INFINITY;
        if (z[j] > M) M = z[j];
      }
      if (sink && sink[h] > M) M = sink[h];
      if (M == -INFINITY) { /* empty row: O = 0, no gradient flows */
        LSE[flat] = -INFINITY;
        DEL[flat] = 0.0;
        continue;
      }
      double Dn = 0.0;
      for (int j = 0; j < S; ++j) Dn += exp(z[j] - M);
      if (sink) Dn += exp(sink[h] - M);
      for (int e = 0; e < E; ++e) o[e] = 0.0;
      for (int j = 0; j < S; ++j) {
        const double p = exp(z[j] - M) / Dn;
        if (p == 0.0) continue;
        for (int e = 0; e < E; ++e) o[e] += p * load_elem(dtype, v, (kvrow0 + j) * E + e);
      }
      double d = 0.0;
      for (int e = 0; e < E; ++e) d += load_elem(dtype, dout, (size_t)flat * E + e) * o[e];
      LSE[flat] = M + log(Dn);
      DEL[flat] = d;
    }
    free(z);
    free(o);
  }
  if (failed) {
    free(LSE);
    free(DEL);
    return -4;
  }

  /* dsink_h = -sum over (n, i) of p_sink * D_i, p_sink = exp(s_h - LSE_i) */
  if (dsink) {
    for (int h = 0; h < Hq; ++h) dsink[h] = 0.0;
    if (sink)
      for (long long flat = 0; flat < total_q; ++flat) {
        const int h = (int)((flat / L) % Hq);
        if (LSE[flat] != -INFINITY) dsink[h] -= exp(sink[h] - LSE[flat]) * DEL[flat];
      }
  }

  /* Phase 2a, requested query rows: dq_i = sum_j dZ_ij dz_ij/dq_i,
     dZ_ij = p_ij (dP_ij - D_i), dP_ij = dO_i . v_j */
  if (dq) {
#pragma omp parallel for schedule(dynamic, 4) num_threads(nt)
    for (long long r = 0; r < nq; ++r) {
      const long long flat = qrows ? qrows[r] : r;
      const int i = (int)(flat % L);
      const long long nh = flat / L;
      const int h = (int)(nh % Hq), n = (int)(nh / Hq);
      const size_t kvrow0 = ((size_t)n * Hkv + h / G) * (size_t)S;
      double* g = dq + (size_t)r * E;
      for (int e = 0; e < E; ++e) g[e] = 0.0;
      if (LSE[flat] == -INFINITY) continue;
      for (int j = 0; j < S; ++j) {
        if (!oracle_visible(L, S, causal, window, n_reg, i, j)) continue;
        const size_t koff = (kvrow0 + j) * E;
        const double p = exp(logit(dtype, q, (size_t)flat * E, k, koff, E, mode, scale, gamma) - LSE[flat]);
        double dp = 0.0;
        for (int e = 0; e < E; ++e) dp += load_elem(dtype, dout, (size_t)flat * E + e) * load_elem(dtype, v, koff + e);
        dlogit_dq(dtype, q, (size_t)flat * E, k, koff, E, mode, scale, gamma, p * (dp - DEL[flat]), g);
      }
    }
  }

  /* Phase 2b, requested key rows (n, kv head, j): sums over the G query heads
     of the group and every query row that sees key j */
  if (dk || dv) {
#pragma omp parallel for schedule(dynamic, 4) num_threads(nt)
    for (long long r = 0; r < nk; ++r) {
      const long long kflat = krows ? krows[r] : r;
      const int j = (int)(kflat % S);
      const long long nkh = kflat / S;
      const int kh = (int)(nkh % Hkv), n = (int)(nkh / Hkv);
      const size_t koff = (size_t)kflat * E;
      double* gk = dk ? dk + (size_t)r * E : NULL;
      double* gv = dv ? dv + (size_t)r * E : NULL;
      for (int e = 0; e < E; ++e) {
        if (gk) gk[e] = 0.0;
        if (gv) gv[e] = 0.0;
      }
      for (int h = kh * G; h < (kh + 1) * G; ++h)
        for (int i = 0; i < L; ++i) {
          if (!oracle_visible(L, S, causal, window, n_reg, i, j)) continue;
          const long long flat = ((long long)n * Hq + h) * L + i;
          if (LSE[flat] == -INFINITY) continue;
          const size_t qoff = (size_t)flat * E;
          const double p = exp(logit(dtype, q, qoff, k, koff, E, mode, scale, gamma) - LSE[flat]);
          if (gv)
            for (int e = 0; e < E; ++e) gv[e] += p * load_elem(dtype, dout, qoff + e);
          if (gk) {
            double dp = 0.0;
            for (int e = 0; e < E; ++e) dp += load_elem(dtype, dout, qoff + e) * load_elem(dtype, v, koff + e);
            dlogit_dk(dtype, q, qoff, k, koff, E, mode, scale, gamma, p * (dp - DEL[flat]), gk);
          }
        }
    }
  }
  if (lse_out) memcpy(lse_out, LSE, sizeof(double) * (size_t)total_q);
  if (delta_out) memcpy(delta_out, DEL, sizeof(double) * (size_t)total_q);
  free(LSE);
  free(DEL);
  return 0;
}

/* ------------------------------------------------------------------------ SOCKET soft-LSH scoring */

int oracle_socket_hash(int dtype, long long nkeys, int E, int tables, int bits, const void* k, const void* v,
                       const float* proj, unsigned char* buckets, double* vnorm) {
  if (dtype < ORACLE_BF16 || dtype > ORACLE_F64) return -1;
  if (nkeys < 0 || E <= 0 || tables <= 0 || bits <= 0 || bits > 8) return -2;
#pragma omp parallel for schedule(static)
  for (long long j = 0; j < nkeys; ++j) {
    for (int t = 0; t < tables; ++t) {
      unsigned code = 0;
      for (int b = 0; b < bits; ++b) {
        /* fp32 projection, one fused multiply-add per element in element order */
        const float* w = proj + ((size_t)t * bits + b) * E;
        float x = 0.0f;
        for (int e = 0; e < E; ++e) x = fmaf((float)load_elem(dtype, k, (size_t)j * E + e), w[e], x);
        if (x > 0.0f) code |= 1u << b;
      }
      buckets[(size_t)j * tables + t] = (unsigned char)code;
    }
    if (vnorm) {
      double ss = 0.0;
      for (int e = 0; e < E; ++e) {
        const double x = load_elem(dtype, v, (size_t)j * E + e);
        ss += x * x;
      }
      vnorm[j] = sqrt(ss);
    }
  }
  return 0;
}

int oracle_socket_scores(int dtype, int E, int tables, int bits, double tau, const void* q, const float* proj,
                         long long nkeys, const unsigned char* buckets, const double* vnorm, double* scores) {
  if (dtype < ORACLE_BF16 || dtype > ORACLE_F64) return -1;
  if (E <= 0 || tables <= 0 || bits <= 0 || bits > 8 || !(tau > 0.0)) return -2;
  const int nb = 1 << bits;
  double* prob = (double*)malloc(sizeof(double) * (size_t)tables * nb);
  if (!prob) return -4;
  for (int t = 0; t < tables; ++t) {
    /* query projections y_b and the softmax over the 2^bits buckets of
       sum_b s_b(bucket) y_b / tau, s_b = +1 if bit b of the bucket is set else -1 */
    double y[8];
    for (int b = 0; b < bits; ++b) {
      const float* w = proj + ((size_t)t * bits + b) * E;
      double acc = 0.0;
      for (int e = 0; e < E; ++e) acc += load_elem(dtype, q, (size_t)e) * (double)w[e];
      y[b] = acc;
    }
    double mx = -INFINITY;
    for (int c = 0; c < nb; ++c) {
      double a = 0.0;
      for (int b = 0; b < bits; ++b) a += ((c >> b) & 1 ? 1.0 : -1.0) * y[b] / tau;
      prob[(size_t)t * nb + c] = a;
      if (a > mx) mx = a;
    }
    double den = 0.0;
    for (int c = 0; c < nb; ++c) den += exp(prob[(size_t)t * nb + c] - mx);
    for (int c = 0; c < nb; ++c) prob[(size_t)t * nb + c] = exp(prob[(size_t)t * nb + c] - mx) / den;
  }
  /* score_j = |v_j| * sum_t prob_t(bucket of key j in table t) */
  for (long long j = 0; j < nkeys; ++j) {
    double sum = 0.0;
    for (int t = 0; t < tables; ++t) sum += prob[(size_t)t * nb + buckets[(size_t)j * tables + t]];
    scores[j] = vnorm[j] * sum;
  }
  free(prob);
  return 0;
}

/* ------------------------------------------------------------------------ SOCKET top-k selection */

typedef struct {
  double score;
  long long idx;
} scored_key;

/* Order for the deterministic top-k: higher score first, and among equal
   scores the lower key index first. */
static int by_score_then_index(const void* a, const void* b) {
  const scored_key* x = (const scored_key*)a;
  const scored_key* y = (const scored_key*)b;
  if (x->score > y->score) return -1;
  if (x->score < y->score) return 1;
  return (x->idx < y->idx) ? -1 : 1;
}

static int by_index(const void* a, const void* b) {
  const long long x = *(const long long*)a, y = *(const long long*)b;
  return (x > y) - (x < y);
}

int oracle_socket_select(long long nkeys, const double* scores, long long top_k, long long* selected) {
  if (nkeys < 0 || top_k < 0 || top_k > nkeys) return -2;
  for (long long j = 0; j < nkeys; ++j)
    if (isnan(scores[j])) return -3;
  scored_key* all = (scored_key*)malloc(sizeof(scored_key) * (size_t)(nkeys > 0 ? nkeys : 1));
  if (!all) return -4;
  for (long long j = 0; j < nkeys; ++j) {
    all[j].score = scores[j];
    all[j].idx = j;
  }
  qsort(all, (size_t)nkeys, sizeof(scored_key), by_score_then_index);
  for (long long r = 0; r < top_k; ++r) selected[r] = all[r].idx;
  free(all);
  qsort(selected, (size_t)top_k, sizeof(long long), by_index);
  return 0;
}
