/*
 * attn.h -- C ABI of the MI355X (gfx950) fused softmax-attention library.
 *
 * One operation, computed by attn_fwd (prefill), attn_fwd_biased (prefill
 * with a general bias), attn_decode (split-K decode) and attn_stream_decode
 * (decode over a rolling cache) and attn_socket_decode (decode over the keys a
 * soft-LSH score selects), with its gradients from attn_bwd:
 *
 *   O = softmax(Z) V,  Z_ij = logit(q_i, k_j) + B_ij,  B_ij in {0, -inf}
 *
 * computed with a streaming (online) softmax so that the L x S matrix of
 * logits never exists in memory.  The problem statement, argument names and
 * tensor shapes follow "SDPA란 무엇인가?" (molayo1419.me) section 1: Q is
 * (N, Hq, L, E), K and V are (N, H, S, E), B is an L x S matrix of 0 / -inf,
 * and the scale is an explicit argument.  Variants:
 *
 *  - logits.  DOT: l_ij = scale * q_i . k_j ("어텐션 메커니즘", section 2).
 *    RBF: l_ij = -gamma * |q_i - k_j|^2 (RBF-attention digest, section
 *    details paragraph 2); the kernels evaluate it as gamma*(2 q.k - |k|^2),
 *    dropping -gamma*|q_i|^2 by softmax shift invariance, with |k_j|^2 formed
 *    on chip for each staged key tile (same digest, paragraph 3).  LSE is
 *    still reported for the definition logits -gamma*|q-k|^2.
 *  - visibility.  Keys j < n_reg are register tokens (RBF digest, paragraph
 *    4): always visible.  Real key r = j - n_reg is visible to query i, with
 *    i' = i + (S - n_reg - L) (bottom-right alignment, SDPA page section 4,
 *    pitfall 3), iff (!causal || r <= i') and (window <= 0 || i' - r < window)
 *    (sliding window, "어텐션 메커니즘" section 6 and "Attention Sink"
 *    section 1).
 *  - sink.  sink[h] (one logit per query head, "Attention Sink" section 4.2)
 *    is added to the softmax denominator and contributes no value:
 *    O_i = sum_j e^{Z_ij} v_j / (e^{s_h} + sum_j e^{Z_ij}); LSE includes it.
 *  - GQA.  Query head h reads key/value head h / (Hq / Hkv) (SDPA page
 *    section 5).
 *  - empty rows.  A row with no visible key and no sink gives O = 0 and
 *    LSE = -inf (SDPA page section 4: 0, never NaN).
 *
 * Conventions for every entry point:
 *  - All tensor pointers are DEVICE pointers owned by the caller; the library
 *    never allocates, frees or synchronises.  Work is enqueued on `stream`
 *    (a hipStream_t; NULL = the default stream) and the call returns at once.
 *  - Layouts are contiguous row-major with E innermost: q and o (N,Hq,L,E),
 *    k and v (N,Hkv,S,E), lse (N,Hq,L) float32, sink (Hq) float32.
 *  - q, k, v, o must be 16-byte aligned; lse and sink 4-byte aligned.
 *  - Arguments are checked completely before any HIP call; on error nothing
 *    is enqueued or written and a negative attn_status is returned.  The
 *    library never substitutes a slower path for an unsupported case.
 *  - attn_last_error() gives a message for the last failing call on the
 *    calling thread.
 */
#ifndef ATTN_H
#define ATTN_H

#include <stddef.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  ATTN_OK = 0,
  ATTN_ERR_NULL = -1,        /* a required pointer is NULL */
  ATTN_ERR_SHAPE = -2,       /* sizes inconsistent (Hq % Hkv, n_reg > S, decode with L != 1, ...) */
  ATTN_ERR_DTYPE = -3,       /* unknown element type */
  ATTN_ERR_UNSUPPORTED = -4, /* valid request outside what the kernels implement (E, window w/o causal, ...) */
  ATTN_ERR_ALIGN = -5,       /* pointer misaligned */
  ATTN_ERR_WORKSPACE = -6,   /* decode workspace NULL or too small */
  ATTN_ERR_HIP = -7,         /* the HIP runtime reported an error at launch */
  ATTN_ERR_ARG = -8          /* bad scalar argument (mode, non-finite scale/gamma, negative window, splits) */
} attn_status;

typedef enum { ATTN_BF16 = 0, ATTN_F32 = 1 } attn_dtype;
typedef enum { ATTN_MODE_DOT = 0, ATTN_MODE_RBF = 1 } attn_mode;
typedef enum { ATTN_BIAS_NONE = 0, ATTN_BIAS_F32 = 1, ATTN_BIAS_BOOL = 2 } attn_bias_kind;

/*
 * attn_fwd -- prefill / general forward.
 *   dt      element type of q, k, v, o (bf16: fp32 accumulation, P rounded to
 *           bf16 for the PV product; f32: fp32 throughout)
 *   N,Hq,Hkv,L,S,E  sizes; S counts the n_reg register rows; E in {64, 128}
 *   scale   DOT logit scale (ignored for RBF); gamma  RBF width (ignored for DOT)
 *   causal, window, n_reg  visibility as described above; window > 0 needs causal
 *   sink    Hq logits (natural-log units, like the logits) or NULL
 *   o, lse  outputs; o has element type dt, lse float32 (natural log)
 * Sizes with N*Hq*L == 0 succeed without launching anything.
 */
int attn_fwd(attn_dtype dt, int N, int Hq, int Hkv, int L, int S, int E,
             const void* q, const void* k, const void* v,
             attn_mode mode, float scale, float gamma,
             int causal, int window, int n_reg, const float* sink,
             void* o, float* lse, void* stream);

/*
 * attn_fwd_biased -- attn_fwd with a general bias B on top of the visibility
 * rule ("SDPA란 무엇인가?" section 1: B is an L x S matrix added to the logits;
 * section 4: a boolean attn_mask is True where a pair is used -- the opposite
 * of a key-padding mask -- and padding and causal masks combine with AND).
 * Same arguments as attn_fwd, plus:
 *   bias_kind  ATTN_BIAS_NONE: no bias (bias is ignored)
 *              ATTN_BIAS_F32:  bias is float32, added to the logit of every
 *                              visible pair, in natural-log units like the
 *                              logits; -inf hides the pair; +inf and NaN are
 *                              not allowed (the result is then undefined)
 *              ATTN_BIAS_BOOL: bias is uint8; 0 hides the pair, any other
 *                              value keeps it
 *   bias       device pointer; the entry of pair (n, h, i, j) is
 *              bias[n*bias_stride_n + h*bias_stride_h + i*S + j] (strides in
 *              elements; 0 broadcasts, e.g. one (L, S) matrix for every
 *              batch and head); float32 bias 4-byte aligned
 *   key_len    NULL, or N int32 device values: in sequence n the real keys
 *              r >= key_len[n] are padding (hidden); registers are unaffected
 *              and the causal / window alignment is unchanged
 * A row with no visible pair left gives O = 0, LSE = -inf (LSE = s_h with a
 * sink).  Errors as attn_fwd, plus ATTN_ERR_ARG for an unknown bias kind or a
 * negative stride and ATTN_ERR_NULL for a missing bias.
 */
int attn_fwd_biased(attn_dtype dt, int N, int Hq, int Hkv, int L, int S, int E,
                    const void* q, const void* k, const void* v,
                    attn_mode mode, float scale, float gamma,
                    int causal, int window, int n_reg, const float* sink,
                    attn_bias_kind bias_kind, const void* bias, long long bias_stride_n, long long bias_stride_h,
                    const int* key_len,
                    void* o, float* lse, void* stream);

/*
 * attn_bwd -- gradients of attn_fwd's O for an upstream gradient dout (LSE is
 * an auxiliary output; no gradient flows into it).  With P recomputed from the
 * saved LSE (the flash-attention recomputation: the L x S matrices never exist
 * in memory, "어텐션 메커니즘" section 6), D_i = dout_i . o_i and
 * dS_ij = P_ij (dout_i . v_j - D_i):
 *   dv_j = sum_i P_ij dout_i;  dq_i = sum_j dS_ij dz_ij/dq_i;  dk_j = sum_i dS_ij dz_ij/dk_j
 *   (DOT: dz/dq = scale k_j, dz/dk = scale q_i; RBF: dz/dq = 2 gamma (k_j - q_i),
 *   dz/dk = 2 gamma (q_i - k_j), the derivative of -gamma |q - k|^2 that also
 *   covers the |k|^2 term formed on chip);
 *   dsink_h = -sum over rows of exp(s_h - LSE_i) D_i  ("Attention Sink" section 4.2:
 *   the sink only enters the denominator).
 * dk and dv of a key/value head sum over the query heads of its group.
 *   q, k, v, sink, sizes, mode, scale, gamma, causal, window, n_reg: exactly as
 *             passed to attn_fwd
 *   o, lse    attn_fwd's outputs for those inputs
 *   dout      (N,Hq,L,E) upstream gradient, element type dt
 *   dq        (N,Hq,L,E); dk, dv (N,Hkv,S,E); element type dt; written whole
 *   dsink     Hq float32 values, or NULL; 0 when sink is NULL
 *   workspace device scratch of attn_bwd_workspace_bytes(N, Hq, L) bytes,
 *             16-byte aligned, caller-owned; contents on entry do not matter
 * bf16 (P and dS rounded to bf16 as MFMA operands, as P in attn_fwd) or f32
 * (fp32 throughout, on the vector ALUs).  Results are deterministic (no
 * atomics).  The general bias of attn_fwd_biased has no backward here.
 */
int attn_bwd(attn_dtype dt, int N, int Hq, int Hkv, int L, int S, int E,
             const void* q, const void* k, const void* v, const void* o, const float* lse, const void* dout,
             attn_mode mode, float scale, float gamma,
             int causal, int window, int n_reg, const float* sink,
             void* dq, void* dk, void* dv, float* dsink,
             void* workspace, size_t workspace_bytes, void* stream);

/* Workspace bytes attn_bwd needs (0 for invalid sizes). */
size_t attn_bwd_workspace_bytes(int N, int Hq, int L);

/*
 * attn_decode -- one query token per sequence (L must be 1) against a long
 * key/value cache, split along the keys (flash-decode, named in the SOCKET
 * summary, contributions 2): each split writes a partial (running max,
 * running sum, unnormalised output) to `workspace`, and a second kernel merges
 * the partials with log-sum-exp weights and the sink.  Same arguments and
 * semantics as attn_fwd with L = 1 (so causal only matters for the window),
 * plus:
 *   num_splits       0 = choose from the sizes; otherwise the exact count
 *                    (results are identical up to rounding for any count)
 *   workspace, workspace_bytes  device scratch of at least
 *                    attn_decode_workspace_bytes(...) bytes, 16-byte aligned,
 *                    owned by the caller; its contents on entry do not matter.
 * bf16 runs the split products on MFMA (P rounded to bf16, as in attn_fwd);
 * f32 runs them on the vector ALUs in fp32 throughout.
 */
int attn_decode(attn_dtype dt, int N, int Hq, int Hkv, int L, int S, int E,
                const void* q, const void* k, const void* v,
                attn_mode mode, float scale, float gamma,
                int causal, int window, int n_reg, const float* sink,
                void* o, float* lse,
                int num_splits, void* workspace, size_t workspace_bytes, void* stream);

/* Split count attn_decode uses for these sizes when num_splits == 0
 * (a pure function of its arguments); negative attn_status on bad sizes. */
int attn_decode_num_splits(int N, int Hq, int Hkv, int S, int E, int causal, int window, int n_reg);

/* Workspace bytes attn_decode needs for these sizes and num_splits
 * (0 = the automatic count); 0 if the sizes are invalid. */
size_t attn_decode_workspace_bytes(int N, int Hq, int Hkv, int S, int E, int causal, int window,
                                   int n_reg, int num_splits);

/*
 * attn_decode_noalloc -- attn_decode for callers that cannot allocate device
 * memory: code under HIP graph capture, tight serving loops, harnesses that
 * forbid hipMalloc.  Same arguments, semantics, kernels and results as
 * attn_decode with the same split count, but no workspace: the split partials
 * go to a static device array of ATTN_DECODE_NOALLOC_SCRATCH_BYTES (8 MiB) that
 * the library holds on every GPU it runs on until the process ends.  Sizes
 * whose partials (attn_decode_workspace_bytes(...) for the same arguments)
 * exceed it return ATTN_ERR_WORKSPACE before any HIP call: 8 MiB holds, e.g.,
 * 8 sequences x 32 query heads x 64 splits at E = 128.  Calls no allocator.
 * Every call on one GPU shares that GPU's array and overwrites what the last
 * call left there (nothing is read before it is written, so no clearing is
 * needed); calls that may overlap on one GPU (different streams, or host
 * threads) race and must be serialised by the caller.  The first call on a
 * device looks the array's address up (hipGetSymbolAddress) and caches it.
 */
#define ATTN_DECODE_NOALLOC_SCRATCH_BYTES ((size_t)8 << 20)
int attn_decode_noalloc(attn_dtype dt, int N, int Hq, int Hkv, int L, int S, int E,
                        const void* q, const void* k, const void* v,
                        attn_mode mode, float scale, float gamma,
                        int causal, int window, int n_reg, const float* sink,
                        void* o, float* lse, int num_splits, void* stream);

/*
 * Rolling key/value cache for streaming decode ("Attention Sink LLM..." page,
 * section 3.2, StreamingLLM): the key/value rows of the first n_sink tokens
 * stay in the cache for good, and only the `window` most recent tokens after
 * them are kept, in a ring.  A cache holds C = n_sink + window rows per
 * (batch, kv head): k_cache and v_cache are (N, Hkv, C, E).  The token at
 * absolute position p (0-based) lives in row
 *     slot(p) = p                                 if p < n_sink,
 *     slot(p) = n_sink + (p - n_sink) % window    otherwise.
 * Once the tokens up to position `pos` have been appended, rows
 * [0, min(pos + 1, C)) hold exactly the kept tokens
 *     { p < n_sink }  U  { pos - window < p <= pos }
 * (positions are whatever the caller's keys encode; the kernels never look
 * at them, and attention over a set of keys does not depend on their order).
 * Requirements for both calls: n_sink >= 0, window >= 1, pos >= 0
 * (ATTN_ERR_ARG otherwise); k_cache / v_cache 16-byte aligned.
 */

/*
 * attn_stream_append -- write the T tokens at positions pos .. pos+T-1 into the
 * cache.  k_new, v_new: (N, Hkv, T, E) of element type dt (bf16 or f32), 16-byte
 * aligned.  Only tokens still kept after the whole append are written, so a
 * block longer than the window is fine and rows of evicted tokens are
 * overwritten in place.  Rows of tokens at positions below pos are left as they
 * are: the caller appends positions in order (the library keeps no position
 * state).  N*T == 0 succeeds without launching anything.
 */
int attn_stream_append(attn_dtype dt, int N, int Hkv, int E, int n_sink, int window, long long pos, int T,
                       const void* k_new, const void* v_new, void* k_cache, void* v_cache, void* stream);

/*
 * attn_stream_decode -- the query of the token at position `pos` (whose key and
 * value are already in the cache) against every kept token: q (N, Hq, 1, E),
 * o (N, Hq, 1, E), lse (N, Hq, 1).  The result equals attn_decode over the full
 * history of pos + 1 keys with n_reg = n_sink, window = window, causal = 1.
 * mode, scale, gamma, sink, num_splits, workspace: as for attn_decode, with
 * workspace size from attn_stream_decode_workspace_bytes.  bf16 or f32 (the
 * cache rows and q of element type dt, as written by attn_stream_append).
 */
int attn_stream_decode(attn_dtype dt, int N, int Hq, int Hkv, int E, int n_sink, int window, long long pos,
                       const void* q, const void* k_cache, const void* v_cache,
                       attn_mode mode, float scale, float gamma, const float* sink,
                       void* o, float* lse,
                       int num_splits, void* workspace, size_t workspace_bytes, void* stream);

/* Workspace bytes attn_stream_decode needs (0 if the sizes are invalid). */
size_t attn_stream_decode_workspace_bytes(int N, int Hq, int Hkv, int E, int n_sink, int window, long long pos,
                                          int num_splits);

/*
 * SOCKET soft-LSH sparse decode ("기술 요약: SOCKET" page, method: soft LSH
 * steps 1-4).  proj: (tables*bits, E) float32 random hyperplanes, drawn by the
 * caller (the method is data-independent: any fixed random draw).
 *
 * attn_socket_hash -- prefill step: for every key row of k (N, Hkv, S, E; bf16
 * or f32 as dt says, v likewise) and table t, bit b of the code of (key j, table t) is set iff the float32
 * projection proj[t*bits + b] . k_j (fused multiply-adds in element order) is
 * > 0.  buckets: (N, Hkv, S, C) bytes with C = attn_socket_code_bytes(tables,
 * bits): with bits <= 4 two codes share a byte (table t in the low nibble of
 * byte t/2 when t is even, in the high nibble when t is odd, an unused high
 * nibble 0), else byte t holds table t.  vnorm (N, Hkv, S) float32 receives
 * |v_j| (may be NULL, then v may be NULL).  1 <= tables <= 64, 1 <= bits <= 8.
 */
int attn_socket_hash(attn_dtype dt, int N, int Hkv, int S, int E, int tables, int bits,
                     const void* k, const void* v, const float* proj,
                     unsigned char* buckets, float* vnorm, void* stream);

/* Bytes of bucket codes per key for these sizes (ATTN_ERR_ARG if tables or
 * bits is out of range). */
int attn_socket_code_bytes(int tables, int bits);

/*
 * attn_socket_decode -- decode step for q (N, Hq, 1, E): per query head, the
 * soft assignment of the query to each table's buckets, p_t(c) = softmax over
 * the 2^bits sign patterns c of sum_b s_b(c) (proj[t*bits+b] . q) / tau
 * (s_b(c) = +1 if bit b of c is set, else -1); key scores
 * score_j = vnorm_j * sum_t p_t(bucket of key j in table t); the top_k keys by
 * score (ties to the lower index) are attended to exactly, with the logits,
 * sink and LSE conventions of attn_decode (no mask: every key precedes the
 * query).  o (N, Hq, 1, E), lse (N, Hq, 1).  selected: NULL, or (N, Hq, top_k)
 * int32 receiving the chosen key rows in ascending order.  1 <= top_k <= S;
 * tau > 0; Hq/Hkv <= 16 and (Hq/Hkv) * tables * 2^bits * 4 bytes <= 64 KB.
 * num_splits: 0 = choose; a split takes at most 4096 selected keys, so a count
 * below ceil(top_k / 4096) is raised to it.
 * workspace: attn_socket_decode_workspace_bytes(...) bytes, 256-byte aligned.
 * bf16 or f32 (q, k, v and o of element type dt; the exact attention over the
 * chosen keys runs as attn_decode does for that type).
 */
int attn_socket_decode(attn_dtype dt, int N, int Hq, int Hkv, int S, int E, int tables, int bits, float tau,
                       int top_k, const void* q, const void* k, const void* v, const float* proj,
                       const unsigned char* buckets, const float* vnorm,
                       attn_mode mode, float scale, float gamma, const float* sink,
                       void* o, float* lse, int* selected,
                       int num_splits, void* workspace, size_t workspace_bytes, void* stream);

/* Workspace bytes attn_socket_decode needs (0 for invalid sizes). */
size_t attn_socket_decode_workspace_bytes(int N, int Hq, int Hkv, int S, int E, int tables, int bits, int top_k,
                                          int num_splits);

/* Static text for a status code. */
const char* attn_status_string(int status);

/* Message describing the last failing call on this thread ("" if none). */
const char* attn_last_error(void);

#ifdef __cplusplus
}
#endif
#endif /* ATTN_H */
