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
