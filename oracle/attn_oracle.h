/*
 * attn_oracle.h -- fp64 CPU oracle for softmax attention.
 *
 * TEST INFRASTRUCTURE ONLY.  This is the slow, plain reference that the GPU
 * library is checked against.  Only the test suite, the smoke check and the
 * benchmark's CPU-baseline leg may load it; the GPU library never includes,
 * links or calls anything here, and nothing here includes the GPU library.
 *
 * What it computes (per output row, all in double precision):
 *
 *   logits   dot: l_ij = scale * sum_e q_ie k_je
 *                 ("SDPA란 무엇인가?" section 1, the Attention equation with
 *                 scale in place of 1/sqrt(E); "어텐션 메커니즘" section 2)
 *            rbf: l_ij = -gamma * sum_e (q_ie - k_je)^2
 *                 (RBF-attention digest, section details paragraph 2: the
 *                 Euclidean distance form, written out before any folding)
 *   bias     z_ij = l_ij if the pair is visible, else -inf
 *                 (SDPA page section 1: B holds 0 or -inf; "어텐션 메커니즘"
 *                 section 5: causal masking adds -inf above the diagonal)
 *   softmax  M_i = max(max_j z_ij, s_h if a sink is given)
 *            D_i = sum_j exp(z_ij - M_i) + [sink] exp(s_h - M_i)
 *            p_ij = exp(z_ij - M_i) / D_i,  O_i = sum_j p_ij v_j,
 *            LSE_i = M_i + ln D_i
 *                 ("어텐션 메커니즘" section 2: row-wise softmax, outputs are
 *                 convex combinations of V; "Attention Sink" section 4.2: the
 *                 per-head sink logit sits in the denominator and its mass
 *                 takes no part in the value sum)
 *   empty    a row with no visible key and no sink gives O_i = 0 and
 *            LSE_i = -inf (SDPA page section 4: the math backend returns 0,
 *            not NaN, for a fully masked row)
 *
 * Visibility of key j for query i, with off = S - n_reg - L:
 *   j < n_reg (register token, RBF digest paragraph 4)      -> visible
 *   otherwise r = j - n_reg, i' = i + off (bottom-right alignment, SDPA page
 *   section 4 pitfall 3), visible iff (!causal || r <= i') and
 *   (window <= 0 || i' - r < window).
 *
 * GQA: query head h reads key/value head h / (Hq / Hkv) (SDPA page section 5:
 * several query heads share one key/value head, in contiguous groups).
 *
 * Layouts: q (N,Hq,L,E), k and v (N,Hkv,S,E), row-major, E innermost.
 * Element type given by `dtype`: bf16 bit patterns (uint16), float32 or
 * float64; every element is widened exactly to double before use.
 */
#ifndef ATTN_ORACLE_H
#define ATTN_ORACLE_H

#ifdef __cplusplus
extern "C" {
#endif

enum { ORACLE_BF16 = 0, ORACLE_F32 = 1, ORACLE_F64 = 2 };
enum { ORACLE_DOT = 0, ORACLE_RBF = 1 };

/* Returns 1 if key j is visible to query i under the rule above, else 0. */
int oracle_visible(int L, int S, int causal, int window, int n_reg, int i, int j);

/*
 * Computes `nrows` output rows.  rows[r] is the flat row index
 * (n*Hq + h)*L + i; rows == NULL means every row, in order (nrows must then
 * equal N*Hq*L).  Outputs: o[r*E + e], lse[r]; p (may be NULL) receives the
 * attention weights p[r*S + j].  sink (may be NULL) holds Hq logits.
 * threads <= 0 uses the OpenMP default.  Returns 0, or a negative value for
 * an invalid argument (nothing is written then).
 */
int oracle_attn_rows(int dtype, int N, int Hq, int Hkv, int L, int S, int E,
                     const void* q, const void* k, const void* v,
                     int mode, double scale, double gamma,
                     int causal, int window, int n_reg, const double* sink,
                     long long nrows, const long long* rows,
                     double* o, double* lse, double* p, int threads);

/*
 * Same, with a general bias B on top of the rule above ("SDPA란 무엇인가?"
 * section 1: B is an L x S matrix added to the logits before the softmax;
 * section 4: a boolean attn_mask is True where a pair is used, the opposite of
 * a key-padding mask, and masks are combined with AND):
 *   bias_kind ORACLE_BIAS_F32:  float32 b[n*bias_sn + h*bias_sh + i*S + j] is
 *                               added to the logit of a visible pair (natural-
 *                               log units; -inf hides the pair)
 *   bias_kind ORACLE_BIAS_BOOL: uint8 m[...] at the same index; 0 hides the pair
 *   key_len (may be NULL):      key_len[n] real keys are valid in sequence n;
 *                               real keys r >= key_len[n] are padding (hidden)
 * Strides are in elements; 0 broadcasts over that dimension.  The causal and
 * window rule keeps its bottom-right alignment over all S keys.
 */
enum { ORACLE_BIAS_NONE = 0, ORACLE_BIAS_F32 = 1, ORACLE_BIAS_BOOL = 2 };
int oracle_attn_rows_ex(int dtype, int N, int Hq, int Hkv, int L, int S, int E,
                        const void* q, const void* k, const void* v,
                        int mode, double scale, double gamma,
                        int causal, int window, int n_reg, const double* sink,
                        int bias_kind, const void* bias, long long bias_sn, long long bias_sh,
                        const int* key_len,
                        long long nrows, const long long* rows,
                        double* o, double* lse, double* p, int threads);

/*
 * Gradients of the forward above (no user bias) for an upstream gradient dO
 * of O (LSE is an auxiliary output: no gradient flows into it).  With
 * P_ij the attention weights, D_i = dO_i . O_i (the exact forward O),
 * dP_ij = dO_i . v_j and dZ_ij = P_ij (dP_ij - D_i) (the softmax Jacobian;
 * "어텐션 메커니즘" section 2 defines the row softmax it differentiates):
 *   dv_j = sum_i P_ij dO_i
 *   dq_i = sum_j dZ_ij dz_ij/dq_i,  dk_j = sum_i dZ_ij dz_ij/dk_j
 *          dot: dz/dq = scale k_j, dz/dk = scale q_i
 *          rbf: dz/dq = -2 gamma (q_i - k_j), dz/dk = 2 gamma (q_i - k_j)
 *               (the definition form -gamma |q - k|^2 of the RBF digest, paragraph 2)
 *   dsink_h = -sum_i p_sink_i D_i,  p_sink_i = exp(s_h - LSE_i)
 *            (the sink only enters the denominator: "Attention Sink" section 4.2)
 * Sums for dk / dv run over the G query heads sharing the key/value head.
 * Rows of dq: qrows (flat (n*Hq+h)*L+i) or all (qrows NULL, nq = N*Hq*L);
 * rows of dk and dv: krows (flat (n*Hkv+kh)*S+j) or all.  Any of dq, dk, dv,
 * dsink, lse_out, delta_out may be NULL.  Every row's LSE and D are computed
 * first (the gradients of any row need them).  Returns 0 or a negative value.
 */
int oracle_attn_bwd(int dtype, int N, int Hq, int Hkv, int L, int S, int E,
                    const void* q, const void* k, const void* v, const void* dout,
                    int mode, double scale, double gamma,
                    int causal, int window, int n_reg, const double* sink,
                    long long nq, const long long* qrows, double* dq,
                    long long nk, const long long* krows, double* dk, double* dv,
                    double* dsink, double* lse_out, double* delta_out, int threads);

/*
 * SOCKET soft-LSH scoring ("기술 요약: SOCKET" page, method: soft LSH steps 1-4).
 *   oracle_socket_hash: for nkeys rows of k (E elements each) and table t,
 *     bit b: x = proj[(t*bits + b)*E + .] . k_j in float32, one fused
 *     multiply-add per element in element order (so the sign decision is the
 *     same one a float32 kernel makes); bit set iff x > 0.  buckets[j*tables + t]
 *     holds the bits of table t; vnorm[j] = |v_j| (fp64, may be NULL).
 *   oracle_socket_scores: for one query q: y_tb = proj_tb . q (fp64), for each
 *     table the softmax over its 2^bits buckets of sum_b s_b y_tb / tau
 *     (s_b = +1 if bit b of the bucket is set, -1 otherwise: the query's soft
 *     assignment from its hyperplane projections, temperature tau), and
 *     scores[j] = vnorm[j] * sum_t prob_t(buckets[j*tables + t]).
 * bits <= 8.  Return 0 or a negative value.
 */
int oracle_socket_hash(int dtype, long long nkeys, int E, int tables, int bits, const void* k, const void* v,
                       const float* proj, unsigned char* buckets, double* vnorm);
int oracle_socket_scores(int dtype, int E, int tables, int bits, double tau, const void* q, const float* proj,
                         long long nkeys, const unsigned char* buckets, const double* vnorm, double* scores);

/*
 * SOCKET selection (same page, method step 4: a deterministic top-k).
 *   oracle_socket_select: the top_k of nkeys scores, higher score first and,
 *     among equal scores, the lower key index first; selected[0..top_k) gets
 *     the chosen key indices in ascending order.  A NaN score returns -3.
 */
int oracle_socket_select(long long nkeys, const double* scores, long long top_k, long long* selected);

/* Number of OpenMP threads oracle_attn_rows uses for a given `threads`. */
int oracle_num_threads(int threads);

#ifdef __cplusplus
}
#endif
#endif
