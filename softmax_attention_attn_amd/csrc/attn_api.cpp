// attn_api.cpp -- the C ABI declared in include/attn.h.
//
// Every argument is checked before the first HIP call, so that misuse returns
// a status (and a message) without touching the GPU; the error lessons follow
// the SDPA page's table of errors (loud failure for head-count mismatches,
// unsupported requests and bad arguments, never a silent fallback).
#include "attn.h"

#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdarg>
#include <cstdint>
#include <cstdio>

#include "kernels.h"

namespace {

thread_local char g_last_error[512] = "";

int fail(int code, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  std::vsnprintf(g_last_error, sizeof g_last_error, fmt, ap);
  va_end(ap);
  return code;
}

int ok() {
  g_last_error[0] = '\0';
  return ATTN_OK;
}

bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

constexpr long long kMaxElems = 1LL << 40;  // per tensor; keeps every offset in int64 comfortably
constexpr long long kMaxGrid = 0x7fffffffLL;

// Checks shared by attn_fwd and attn_decode.  Returns ATTN_OK or an error.
int check_args(attn_dtype dt, int N, int Hq, int Hkv, int L, int S, int E, const void* q, const void* k,
               const void* v, attn_mode mode, float scale, float gamma, int causal, int window, int n_reg,
               const float* sink, const void* o, const float* lse) {
  (void)causal;
  if (dt != ATTN_BF16 && dt != ATTN_F32) return fail(ATTN_ERR_DTYPE, "unknown dtype %d", (int)dt);
  if (mode != ATTN_MODE_DOT && mode != ATTN_MODE_RBF) return fail(ATTN_ERR_ARG, "unknown mode %d", (int)mode);
  if (N < 0 || L < 0 || S < 0) return fail(ATTN_ERR_SHAPE, "negative size (N=%d L=%d S=%d)", N, L, S);
  if (Hq <= 0 || Hkv <= 0) return fail(ATTN_ERR_SHAPE, "head counts must be positive (Hq=%d Hkv=%d)", Hq, Hkv);
  if (Hq % Hkv != 0)
    return fail(ATTN_ERR_SHAPE, "query heads (%d) must be a multiple of key/value heads (%d)", Hq, Hkv);
  if (n_reg < 0 || n_reg > S) return fail(ATTN_ERR_SHAPE, "n_reg=%d outside [0, S=%d]", n_reg, S);
  if (window < 0) return fail(ATTN_ERR_ARG, "window=%d must be >= 0", window);
  if (window > 0 && !causal) return fail(ATTN_ERR_UNSUPPORTED, "a sliding window needs causal=1");
  if (E != 64 && E != 128) return fail(ATTN_ERR_UNSUPPORTED, "head dimension E=%d (supported: 64, 128)", E);
  if (mode == ATTN_MODE_DOT && !std::isfinite(scale)) return fail(ATTN_ERR_ARG, "scale must be finite");
  if (mode == ATTN_MODE_RBF && !(std::isfinite(gamma) && gamma >= 0.f))
    return fail(ATTN_ERR_ARG, "gamma must be finite and >= 0");
  if ((long long)N * Hq * L * E > kMaxElems || (long long)N * Hkv * S * E > kMaxElems)
    return fail(ATTN_ERR_SHAPE, "tensor too large");
  if ((long long)N * Hq * L == 0) return ATTN_OK;  // nothing to compute; pointers unused
  if (!q || !o || !lse) return fail(ATTN_ERR_NULL, "q, o and lse must not be NULL");
  if (S > 0 && (!k || !v)) return fail(ATTN_ERR_NULL, "k and v must not be NULL when S > 0");
  if (!aligned(q, 16) || !aligned(o, 16) || (S > 0 && (!aligned(k, 16) || !aligned(v, 16))))
    return fail(ATTN_ERR_ALIGN, "q, k, v and o must be 16-byte aligned");
  if (!aligned(lse, 4) || (sink && !aligned(sink, 4))) return fail(ATTN_ERR_ALIGN, "lse and sink must be 4-byte aligned");
  return ATTN_OK;
}

attn_impl::FwdArgs make_args(int N, int Hq, int Hkv, int L, int S, int E, const void* q, const void* k,
                             const void* v, attn_mode mode, float scale, float gamma, int causal, int window,
                             int n_reg, const float* sink, void* o, float* lse) {
  attn_impl::FwdArgs a;
  a.q = q;
  a.k = k;
  a.v = v;
  a.o = o;
  a.lse = lse;
  a.sink = sink;
  a.N = N;
  a.Hq = Hq;
  a.Hkv = Hkv;
  a.L = L;
  a.S = S;
  a.E = E;
  a.kv_rows = S;
  a.key_len = nullptr;
  a.bias = nullptr;
  a.bias_kind = 0;
  a.bias_sn = 0;
  a.bias_sh = 0;
  a.n_reg = n_reg;
  a.causal = causal ? 1 : 0;
  a.window = window;
  a.rbf = (mode == ATTN_MODE_RBF) ? 1 : 0;
  a.scale = scale;
  a.gamma = gamma;
  return a;
}

// bf16 forward kernel choice: narrow causal windows at E = 64 take the key-band
// kernel, everything else the tiled kernel.
hipError_t launch_bf16_forward(const attn_impl::FwdArgs& a, hipStream_t st) {
  if (attn_impl::prefill_band_fits(a)) return attn_impl::launch_prefill_bf16_band(a, st);
  return attn_impl::launch_prefill_bf16(a, st);
}

int hip_status(hipError_t e, const char* what) {
  if (e == hipSuccess) return ok();
  return fail(ATTN_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

// Split count for decode (pure function of the sizes): enough workgroups to
// cover the chip several times over, but at least 512 keys per split (on the
// 4096-row rolling-cache decode 256 keys per split were 0-2 % and 128 keys
// 11 % slower).
int resolve_splits(int N, int Hq, int Hkv, int S, int causal, int window, int n_reg, int num_splits) {
  if (num_splits > 0) return num_splits;
  const attn_impl::DecodeKeys dk = attn_impl::decode_keys(S, n_reg, causal ? 1 : 0, window);
  const long long units = (long long)N * Hkv * ((Hq / Hkv + 15) / 16);
  const long long want = units > 0 ? (2048 + units - 1) / units : 1;
  const long long cap = dk.count > 512 ? (dk.count + 511) / 512 : 1;
  long long s = want < cap ? want : cap;
  if (s < 1) s = 1;
  if (s > 65535) s = 65535;
  return (int)s;
}

size_t workspace_for(int N, int Hq, int E, int splits) {
  const size_t parts = (size_t)N * Hq * splits;
  return parts * E * sizeof(float) + parts * 2 * sizeof(float);
}

// Rows of the rolling cache that hold kept tokens once position `pos` has been
// appended (they are rows [0, n) of every slice); -1 for invalid arguments.
long long stream_rows(int n_sink, int window, long long pos) {
  if (n_sink < 0 || window < 1 || pos < 0) return -1;
  const long long cap = (long long)n_sink + window;
  return pos + 1 < cap ? pos + 1 : cap;
}

// Split-K decode of either element type (bf16: MFMA kernel, f32: vector-ALU kernel).
hipError_t launch_decode(attn_dtype dt, const attn_impl::DecodeArgs& d, hipStream_t stream) {
  return dt == ATTN_BF16 ? attn_impl::launch_decode_bf16(d, stream) : attn_impl::launch_decode_f32(d, stream);
}

// Validation and launch set-up shared by attn_decode and attn_decode_noalloc:
// everything but the partial-result buffers.  *need = their size in bytes.
// Returns ATTN_OK (with *empty set when there is nothing to compute) or an error.
int decode_setup(attn_dtype dt, int N, int Hq, int Hkv, int L, int S, int E, const void* q, const void* k,
                 const void* v, attn_mode mode, float scale, float gamma, int causal, int window, int n_reg,
                 const float* sink, void* o, float* lse, int num_splits, attn_impl::DecodeArgs* d, size_t* need,
                 bool* empty) {
  *empty = false;
  if (L != 1) return fail(ATTN_ERR_SHAPE, "decode takes exactly one query per sequence (L=%d)", L);
  int rc = check_args(dt, N, Hq, Hkv, L, S, E, q, k, v, mode, scale, gamma, causal, window, n_reg, sink, o, lse);
  if (rc != ATTN_OK) return rc;
  if (num_splits < 0) return fail(ATTN_ERR_ARG, "num_splits=%d must be >= 0", num_splits);
  if (N == 0) {
    *empty = true;
    return ATTN_OK;
  }
  const int splits = resolve_splits(N, Hq, Hkv, S, causal, window, n_reg, num_splits);
  *need = workspace_for(N, Hq, E, splits);
  if ((long long)N * Hkv * ((Hq / Hkv + 15) / 16) > 65535LL || (long long)N * Hq > kMaxGrid)
    return fail(ATTN_ERR_SHAPE, "grid too large");
  d->f = make_args(N, Hq, Hkv, L, S, E, q, k, v, mode, scale, gamma, causal, window, n_reg, sink, o, lse);
  d->num_splits = splits;
  return ATTN_OK;
}

}  // namespace

#pragma GCC visibility push(default)
extern "C" {

int attn_fwd(attn_dtype dt, int N, int Hq, int Hkv, int L, int S, int E, const void* q, const void* k,
             const void* v, attn_mode mode, float scale, float gamma, int causal, int window, int n_reg,
             const float* sink, void* o, float* lse, void* stream) {
  int rc = check_args(dt, N, Hq, Hkv, L, S, E, q, k, v, mode, scale, gamma, causal, window, n_reg, sink, o, lse);
  if (rc != ATTN_OK) return rc;
  if ((long long)N * Hq * L == 0) return ok();
  // bf16 tiles are addressed with 32-bit byte offsets into one (batch, kv head)
  // slice, including one tile of rows past its end.
  if (dt == ATTN_BF16 && ((long long)S + 64) * E * 2 > 0x7fffffffLL)
    return fail(ATTN_ERR_UNSUPPORTED, "a (batch, kv head) slice of K/V near or above 2 GiB (S=%d, E=%d)", S, E);
  const int tile = 64;  // smallest query tile of any kernel
  if ((long long)((L + tile - 1) / tile) * N * Hq > kMaxGrid) return fail(ATTN_ERR_SHAPE, "grid too large");
  const attn_impl::FwdArgs a =
      make_args(N, Hq, Hkv, L, S, E, q, k, v, mode, scale, gamma, causal, window, n_reg, sink, o, lse);
  hipStream_t st = static_cast<hipStream_t>(stream);
  const hipError_t e = dt == ATTN_BF16 ? launch_bf16_forward(a, st) : attn_impl::launch_prefill_f32(a, st);
  return hip_status(e, "attn_fwd launch");
}

int attn_fwd_biased(attn_dtype dt, int N, int Hq, int Hkv, int L, int S, int E, const void* q, const void* k,
                    const void* v, attn_mode mode, float scale, float gamma, int causal, int window, int n_reg,
                    const float* sink, attn_bias_kind bias_kind, const void* bias, long long bias_stride_n,
                    long long bias_stride_h, const int* key_len, void* o, float* lse, void* stream) {
  int rc = check_args(dt, N, Hq, Hkv, L, S, E, q, k, v, mode, scale, gamma, causal, window, n_reg, sink, o, lse);
  if (rc != ATTN_OK) return rc;
  if (bias_kind != ATTN_BIAS_NONE && bias_kind != ATTN_BIAS_F32 && bias_kind != ATTN_BIAS_BOOL)
    return fail(ATTN_ERR_ARG, "unknown bias kind %d", (int)bias_kind);
  if (bias_kind != ATTN_BIAS_NONE && (bias_stride_n < 0 || bias_stride_h < 0))
    return fail(ATTN_ERR_ARG, "bias strides must be >= 0 (got %lld, %lld)", bias_stride_n, bias_stride_h);
  if ((long long)N * Hq * L == 0) return ok();
  if (bias_kind != ATTN_BIAS_NONE) {
    if (!bias) return fail(ATTN_ERR_NULL, "bias must not be NULL for bias kind %d", (int)bias_kind);
    if (bias_kind == ATTN_BIAS_F32 && !aligned(bias, 4)) return fail(ATTN_ERR_ALIGN, "a float32 bias must be 4-byte aligned");
    // the last element addressed must stay within an int64 element index
    const long long last = (long long)(N - 1) * bias_stride_n + (long long)(Hq - 1) * bias_stride_h +
                           (long long)L * S;
    if (bias_stride_n > kMaxElems || bias_stride_h > kMaxElems || last > (1LL << 50))
      return fail(ATTN_ERR_SHAPE, "bias strides too large");
  }
  if (key_len && !aligned(key_len, 4)) return fail(ATTN_ERR_ALIGN, "key_len must be 4-byte aligned");
  if (dt == ATTN_BF16 && ((long long)S + 64) * E * 2 > 0x7fffffffLL)
    return fail(ATTN_ERR_UNSUPPORTED, "a (batch, kv head) slice of K/V near or above 2 GiB (S=%d, E=%d)", S, E);
  if ((long long)((L + 63) / 64) * N * Hq > kMaxGrid) return fail(ATTN_ERR_SHAPE, "grid too large");
  attn_impl::FwdArgs a =
      make_args(N, Hq, Hkv, L, S, E, q, k, v, mode, scale, gamma, causal, window, n_reg, sink, o, lse);
  a.key_len = key_len;
  if (bias_kind != ATTN_BIAS_NONE) {
    a.bias = bias;
    a.bias_kind = (int)bias_kind;
    a.bias_sn = bias_stride_n;
    a.bias_sh = bias_stride_h;
  }
  hipStream_t st = static_cast<hipStream_t>(stream);
  const hipError_t e = dt == ATTN_BF16 ? launch_bf16_forward(a, st) : attn_impl::launch_prefill_f32(a, st);
  return hip_status(e, "attn_fwd_biased launch");
}

size_t attn_bwd_workspace_bytes(int N, int Hq, int L) {
  if (N < 0 || Hq <= 0 || L < 0) return 0;
  return attn_impl::backward_workspace_bytes(N, Hq, L);
}

int attn_bwd(attn_dtype dt, int N, int Hq, int Hkv, int L, int S, int E, const void* q, const void* k, const void* v,
             const void* o, const float* lse, const void* dout, attn_mode mode, float scale, float gamma, int causal,
             int window, int n_reg, const float* sink, void* dq, void* dk, void* dv, float* dsink, void* workspace,
             size_t workspace_bytes, void* stream) {
  int rc = check_args(dt, N, Hq, Hkv, L, S, E, q, k, v, mode, scale, gamma, causal, window, n_reg, sink, o, lse);
  if (rc != ATTN_OK) return rc;
  if ((long long)N * Hq * L == 0 && (long long)N * Hkv * S == 0) return ok();
  if ((long long)N * Hq * L == 0 || (long long)N * Hkv * S == 0)
    return fail(ATTN_ERR_UNSUPPORTED, "backward with an empty query or key side (L=%d, S=%d)", L, S);
  if (!dout || !dq || !dk || !dv) return fail(ATTN_ERR_NULL, "dout, dq, dk and dv must not be NULL");
  if (!aligned(dout, 16) || !aligned(dq, 16) || !aligned(dk, 16) || !aligned(dv, 16))
    return fail(ATTN_ERR_ALIGN, "dout, dq, dk and dv must be 16-byte aligned");
  if (dsink && !aligned(dsink, 4)) return fail(ATTN_ERR_ALIGN, "dsink must be 4-byte aligned");
  const size_t need = attn_impl::backward_workspace_bytes(N, Hq, L);
  if (!workspace) return fail(ATTN_ERR_WORKSPACE, "workspace is NULL (need %zu bytes)", need);
  if (workspace_bytes < need) return fail(ATTN_ERR_WORKSPACE, "workspace has %zu bytes, need %zu", workspace_bytes, need);
  if (!aligned(workspace, 16)) return fail(ATTN_ERR_ALIGN, "workspace must be 16-byte aligned");
  if (dt == ATTN_BF16 && (((long long)S + 64) * E * 2 > 0x7fffffffLL || ((long long)L + 64) * E * 2 > 0x7fffffffLL))
    return fail(ATTN_ERR_UNSUPPORTED, "a (batch, head) slice near or above 2 GiB (L=%d, S=%d, E=%d)", L, S, E);
  if ((long long)((L + 127) / 128) * N * Hq > kMaxGrid || (long long)((S + 127) / 128) * N * Hkv > kMaxGrid ||
      (long long)N * Hq > 65535LL)
    return fail(ATTN_ERR_SHAPE, "grid too large");
  attn_impl::BwdArgs a;
  a.f = make_args(N, Hq, Hkv, L, S, E, q, k, v, mode, scale, gamma, causal, window, n_reg, sink, nullptr, nullptr);
  a.o = o;
  a.lse = lse;
  a.dout = dout;
  a.dq = dq;
  a.dk = dk;
  a.dv = dv;
  a.dsink = dsink;
  a.workspace = static_cast<float*>(workspace);
  hipStream_t st = static_cast<hipStream_t>(stream);
  return hip_status(dt == ATTN_BF16 ? attn_impl::launch_backward_bf16(a, st) : attn_impl::launch_backward_f32(a, st),
                    "attn_bwd launch");
}

// ----------------------------------------------------------------------------- SOCKET

int socket_check(int N, int Hq, int Hkv, int S, int E, int tables, int bits) {
  if (N < 0 || Hq <= 0 || Hkv <= 0 || S < 0 || Hq % Hkv != 0) return fail(ATTN_ERR_SHAPE, "invalid sizes");
  if (E != 64 && E != 128) return fail(ATTN_ERR_UNSUPPORTED, "head dimension E=%d (supported: 64, 128)", E);
  if (tables < 1 || tables > 64 || bits < 1 || bits > 8)
    return fail(ATTN_ERR_ARG, "need 1 <= tables <= 64 and 1 <= bits <= 8 (tables=%d bits=%d)", tables, bits);
  if ((long long)N * Hkv * S * E > kMaxElems) return fail(ATTN_ERR_SHAPE, "tensor too large");
  return ATTN_OK;
}

int attn_socket_code_bytes(int tables, int bits) {
  if (tables < 1 || tables > 64 || bits < 1 || bits > 8)
    return fail(ATTN_ERR_ARG, "tables=%d (1..64) or bits=%d (1..8) out of range", tables, bits);
  return attn_impl::socket_code_bytes(tables, bits);
}

int attn_socket_hash(attn_dtype dt, int N, int Hkv, int S, int E, int tables, int bits, const void* k, const void* v,
                     const float* proj, unsigned char* buckets, float* vnorm, void* stream) {
  if (dt != ATTN_BF16 && dt != ATTN_F32) return fail(ATTN_ERR_DTYPE, "unknown dtype %d", (int)dt);
  int rc = socket_check(N, Hkv, Hkv, S, E, tables, bits);
  if (rc != ATTN_OK) return rc;
  if ((long long)N * S == 0) return ok();
  if (!k || !proj || !buckets || (vnorm && !v)) return fail(ATTN_ERR_NULL, "k, proj and buckets (and v with vnorm) must not be NULL");
  if (!aligned(k, 16) || (v && !aligned(v, 16)) || !aligned(proj, 4) || (vnorm && !aligned(vnorm, 4)))
    return fail(ATTN_ERR_ALIGN, "k and v must be 16-byte aligned, proj and vnorm 4-byte aligned");
  if (((long long)N * Hkv * S + 255) / 256 > kMaxGrid) return fail(ATTN_ERR_SHAPE, "grid too large");
  attn_impl::SocketHashArgs a{k, v, proj, buckets, vnorm, N, Hkv, S, E, tables, bits, dt == ATTN_F32};
  return hip_status(attn_impl::launch_socket_hash(a, static_cast<hipStream_t>(stream)), "attn_socket_hash launch");
}

// Workspace layout: bucket probabilities, scores, selected rows, decode partials.
struct SocketLayout {
  size_t probs, scores, sel, parts, total;
  int splits;
};

SocketLayout socket_layout(int N, int Hq, int S, int E, int tables, int bits, int top_k, int num_splits) {
  SocketLayout l;
  const size_t heads = (size_t)N * Hq;
  auto up = [](size_t x) { return (x + 255) & ~(size_t)255; };
  l.splits = num_splits > 0 ? num_splits : (int)std::min<long long>(std::max<long long>(1, (top_k + 255) / 256),
                                                                     std::max<long long>(1, (2048 + (long long)heads - 1) / std::max<long long>(1, (long long)heads)));
  // A split's key list is staged in LDS: at most kDecodeIndexMax keys per split.
  l.splits = std::max(l.splits, (top_k + attn_impl::kDecodeIndexMax - 1) / attn_impl::kDecodeIndexMax);
  l.probs = 0;
  l.scores = up(l.probs + heads * tables * ((size_t)1 << bits) * sizeof(float));
  l.sel = up(l.scores + heads * (size_t)S * sizeof(float));
  l.parts = up(l.sel + heads * (size_t)top_k * sizeof(int));
  l.total = l.parts + workspace_for(N, Hq, E, l.splits);
  return l;
}

size_t attn_socket_decode_workspace_bytes(int N, int Hq, int Hkv, int S, int E, int tables, int bits, int top_k,
                                          int num_splits) {
  if (N < 0 || Hq <= 0 || Hkv <= 0 || S < 0 || Hq % Hkv != 0 || (E != 64 && E != 128) || tables < 1 ||
      tables > 64 || bits < 1 || bits > 8 || top_k < 1 || top_k > S || num_splits < 0)
    return 0;
  return socket_layout(N, Hq, S, E, tables, bits, top_k, num_splits).total;
}

int attn_socket_decode(attn_dtype dt, int N, int Hq, int Hkv, int S, int E, int tables, int bits, float tau, int top_k,
                       const void* q, const void* k, const void* v, const float* proj, const unsigned char* buckets,
                       const float* vnorm, attn_mode mode, float scale, float gamma, const float* sink, void* o,
                       float* lse, int* selected, int num_splits, void* workspace, size_t workspace_bytes,
                       void* stream) {
  int rc = check_args(dt, N, Hq, Hkv, 1, S, E, q, k, v, mode, scale, gamma, 1, 0, 0, sink, o, lse);
  if (rc != ATTN_OK) return rc;
  rc = socket_check(N, Hq, Hkv, S, E, tables, bits);
  if (rc != ATTN_OK) return rc;
  if (!(std::isfinite(tau) && tau > 0.f)) return fail(ATTN_ERR_ARG, "tau must be finite and > 0");
  if (top_k < 1 || top_k > S) return fail(ATTN_ERR_ARG, "top_k=%d outside [1, S=%d]", top_k, S);
  if (num_splits < 0) return fail(ATTN_ERR_ARG, "num_splits=%d must be >= 0", num_splits);
  const int G = Hq / Hkv;
  if (G > 16) return fail(ATTN_ERR_UNSUPPORTED, "SOCKET scoring handles up to 16 query heads per key/value head");
  if (attn_impl::socket_lds_bytes(G, tables, bits) > 64 * 1024)
    return fail(ATTN_ERR_UNSUPPORTED, "(Hq/Hkv) * tables * 2^bits probabilities exceed 64 KB of LDS");
  if (N == 0) return ok();
  if (!proj || !buckets || !vnorm) return fail(ATTN_ERR_NULL, "proj, buckets and vnorm must not be NULL");
  if (!aligned(proj, 4) || !aligned(vnorm, 4) || (selected && !aligned(selected, 4)))
    return fail(ATTN_ERR_ALIGN, "proj, vnorm and selected must be 4-byte aligned");
  const SocketLayout l = socket_layout(N, Hq, S, E, tables, bits, top_k, num_splits);
  if (!workspace) return fail(ATTN_ERR_WORKSPACE, "workspace is NULL (need %zu bytes)", l.total);
  if (workspace_bytes < l.total) return fail(ATTN_ERR_WORKSPACE, "workspace has %zu bytes, need %zu", workspace_bytes, l.total);
  if (!aligned(workspace, 256)) return fail(ATTN_ERR_ALIGN, "workspace must be 256-byte aligned");
  if ((long long)N * Hq > 65535LL) return fail(ATTN_ERR_SHAPE, "grid too large");
  uint8_t* ws = static_cast<uint8_t*>(workspace);
  attn_impl::SocketSelectArgs s;
  s.q = q;
  s.proj = proj;
  s.buckets = buckets;
  s.vnorm = vnorm;
  s.probs = reinterpret_cast<float*>(ws + l.probs);
  s.scores = reinterpret_cast<float*>(ws + l.scores);
  s.selected = selected ? selected : reinterpret_cast<int*>(ws + l.sel);
  s.N = N;
  s.Hq = Hq;
  s.Hkv = Hkv;
  s.S = S;
  s.E = E;
  s.tables = tables;
  s.bits = bits;
  s.top_k = top_k;
  s.tau = tau;
  s.f32 = dt == ATTN_F32;
  hipStream_t st = static_cast<hipStream_t>(stream);
  rc = hip_status(attn_impl::launch_socket_select(s, st), "attn_socket_decode select launch");
  if (rc != ATTN_OK) return rc;
  attn_impl::DecodeArgs d;
  d.f = make_args(N, Hq, Hkv, 1, S, E, q, k, v, mode, scale, gamma, 1, 0, 0, sink, o, lse);
  d.num_splits = l.splits;
  d.part_o = reinterpret_cast<float*>(ws + l.parts);
  d.part_ml = d.part_o + (size_t)N * Hq * l.splits * E;
  d.key_index = s.selected;
  d.index_count = top_k;
  return hip_status(launch_decode(dt, d, st), "attn_socket_decode launch");
}

int attn_decode_num_splits(int N, int Hq, int Hkv, int S, int E, int causal, int window, int n_reg) {
  if (N < 0 || Hq <= 0 || Hkv <= 0 || S < 0 || Hq % Hkv != 0 || n_reg < 0 || n_reg > S || window < 0)
    return fail(ATTN_ERR_SHAPE, "invalid decode sizes");
  if (E != 64 && E != 128) return fail(ATTN_ERR_UNSUPPORTED, "head dimension E=%d (supported: 64, 128)", E);
  return resolve_splits(N, Hq, Hkv, S, causal, window, n_reg, 0);
}

size_t attn_decode_workspace_bytes(int N, int Hq, int Hkv, int S, int E, int causal, int window, int n_reg,
                                   int num_splits) {
  if (N < 0 || Hq <= 0 || Hkv <= 0 || S < 0 || Hq % Hkv != 0 || n_reg < 0 || n_reg > S || window < 0 ||
      num_splits < 0 || (E != 64 && E != 128))
    return 0;
  const int splits = resolve_splits(N, Hq, Hkv, S, causal, window, n_reg, num_splits);
  return workspace_for(N, Hq, E, splits);
}

int attn_decode(attn_dtype dt, int N, int Hq, int Hkv, int L, int S, int E, const void* q, const void* k,
                const void* v, attn_mode mode, float scale, float gamma, int causal, int window, int n_reg,
                const float* sink, void* o, float* lse, int num_splits, void* workspace, size_t workspace_bytes,
                void* stream) {
  attn_impl::DecodeArgs d;
  size_t need = 0;
  bool empty = false;
  const int rc = decode_setup(dt, N, Hq, Hkv, L, S, E, q, k, v, mode, scale, gamma, causal, window, n_reg, sink, o,
                              lse, num_splits, &d, &need, &empty);
  if (rc != ATTN_OK) return rc;
  if (empty) return ok();
  if (!workspace) return fail(ATTN_ERR_WORKSPACE, "workspace is NULL (need %zu bytes)", need);
  if (workspace_bytes < need)
    return fail(ATTN_ERR_WORKSPACE, "workspace has %zu bytes, need %zu", workspace_bytes, need);
  if (!aligned(workspace, 16)) return fail(ATTN_ERR_ALIGN, "workspace must be 16-byte aligned");
  d.part_o = static_cast<float*>(workspace);
  d.part_ml = d.part_o + (size_t)N * Hq * d.num_splits * E;
  return hip_status(launch_decode(dt, d, static_cast<hipStream_t>(stream)), "attn_decode launch");
}

int attn_decode_noalloc(attn_dtype dt, int N, int Hq, int Hkv, int L, int S, int E, const void* q, const void* k,
                        const void* v, attn_mode mode, float scale, float gamma, int causal, int window, int n_reg,
                        const float* sink, void* o, float* lse, int num_splits, void* stream) {
  attn_impl::DecodeArgs d;
  size_t need = 0;
  bool empty = false;
  const int rc = decode_setup(dt, N, Hq, Hkv, L, S, E, q, k, v, mode, scale, gamma, causal, window, n_reg, sink, o,
                              lse, num_splits, &d, &need, &empty);
  if (rc != ATTN_OK) return rc;
  if (empty) return ok();
  if (need > attn_impl::kDecodeScratchBytes)
    return fail(ATTN_ERR_WORKSPACE,
                "these sizes need %zu bytes of split partials; the library's static scratch holds %zu "
                "(use fewer splits, or attn_decode with a workspace)", need, attn_impl::kDecodeScratchBytes);
  float* scratch = nullptr;
  const hipError_t e = attn_impl::decode_scratch(&scratch);
  if (e != hipSuccess) return hip_status(e, "attn_decode_noalloc scratch lookup");
  // Every split writes all of its partials (an empty split writes max -inf, sum 0),
  // so nothing left by an earlier call is read: no clearing is needed.
  d.part_o = scratch;
  d.part_ml = scratch + (size_t)N * Hq * d.num_splits * E;
  return hip_status(launch_decode(dt, d, static_cast<hipStream_t>(stream)), "attn_decode_noalloc launch");
}

// ----------------------------------------------------------------------------- rolling cache

int attn_stream_append(attn_dtype dt, int N, int Hkv, int E, int n_sink, int window, long long pos, int T,
                       const void* k_new, const void* v_new, void* k_cache, void* v_cache, void* stream) {
  if (dt != ATTN_BF16 && dt != ATTN_F32) return fail(ATTN_ERR_DTYPE, "unknown dtype %d", (int)dt);
  if (N < 0 || Hkv <= 0 || T < 0) return fail(ATTN_ERR_SHAPE, "invalid sizes (N=%d Hkv=%d T=%d)", N, Hkv, T);
  if (E != 64 && E != 128) return fail(ATTN_ERR_UNSUPPORTED, "head dimension E=%d (supported: 64, 128)", E);
  if (n_sink < 0 || window < 1) return fail(ATTN_ERR_ARG, "need n_sink >= 0 and window >= 1 (n_sink=%d window=%d)", n_sink, window);
  if (pos < 0) return fail(ATTN_ERR_ARG, "pos=%lld must be >= 0", pos);
  const long long cap = (long long)n_sink + window;
  if ((long long)N * Hkv * cap * E > kMaxElems || (long long)N * Hkv * T * E > kMaxElems)
    return fail(ATTN_ERR_SHAPE, "tensor too large");
  if ((long long)N * T == 0) return ok();
  if (!k_new || !v_new || !k_cache || !v_cache) return fail(ATTN_ERR_NULL, "k_new, v_new, k_cache and v_cache must not be NULL");
  if (!aligned(k_new, 16) || !aligned(v_new, 16) || !aligned(k_cache, 16) || !aligned(v_cache, 16))
    return fail(ATTN_ERR_ALIGN, "k_new, v_new, k_cache and v_cache must be 16-byte aligned");
  const int eb = dt == ATTN_BF16 ? 2 : 4;
  if ((long long)N * Hkv * T * (E * eb / 16) / 256 + 1 > kMaxGrid) return fail(ATTN_ERR_SHAPE, "grid too large");
  attn_impl::StreamAppendArgs a;
  a.k_new = k_new;
  a.v_new = v_new;
  a.k_cache = k_cache;
  a.v_cache = v_cache;
  a.N = N;
  a.Hkv = Hkv;
  a.E = E;
  a.elem_bytes = eb;
  a.n_sink = n_sink;
  a.window = window;
  a.T = T;
  a.pos = pos;
  return hip_status(attn_impl::launch_stream_append(a, static_cast<hipStream_t>(stream)), "attn_stream_append launch");
}

size_t attn_stream_decode_workspace_bytes(int N, int Hq, int Hkv, int E, int n_sink, int window, long long pos,
                                          int num_splits) {
  const long long rows = stream_rows(n_sink, window, pos);
  if (rows < 0 || rows > 0x7fffffffLL) return 0;
  return attn_decode_workspace_bytes(N, Hq, Hkv, (int)rows, E, 1, 0, 0, num_splits);
}

int attn_stream_decode(attn_dtype dt, int N, int Hq, int Hkv, int E, int n_sink, int window, long long pos,
                       const void* q, const void* k_cache, const void* v_cache, attn_mode mode, float scale,
                       float gamma, const float* sink, void* o, float* lse, int num_splits, void* workspace,
                       size_t workspace_bytes, void* stream) {
  if (n_sink < 0 || window < 1) return fail(ATTN_ERR_ARG, "need n_sink >= 0 and window >= 1 (n_sink=%d window=%d)", n_sink, window);
  if (pos < 0) return fail(ATTN_ERR_ARG, "pos=%lld must be >= 0", pos);
  const long long cap = (long long)n_sink + window;
  if (cap > 0x7fffffffLL - 64) return fail(ATTN_ERR_SHAPE, "n_sink + window too large");
  const int S = (int)stream_rows(n_sink, window, pos);
  // Every kept row is visible to the newest token (its own row included), in
  // any order: plain decode over rows [0, S) of slices that are `cap` rows apart.
  int rc = check_args(dt, N, Hq, Hkv, 1, (int)cap, E, q, k_cache, v_cache, mode, scale, gamma, 1, 0, 0, sink, o, lse);
  if (rc != ATTN_OK) return rc;
  if (num_splits < 0) return fail(ATTN_ERR_ARG, "num_splits=%d must be >= 0", num_splits);
  if (N == 0) return ok();
  const int splits = resolve_splits(N, Hq, Hkv, S, 1, 0, 0, num_splits);
  const size_t need = workspace_for(N, Hq, E, splits);
  if (!workspace) return fail(ATTN_ERR_WORKSPACE, "workspace is NULL (need %zu bytes)", need);
  if (workspace_bytes < need) return fail(ATTN_ERR_WORKSPACE, "workspace has %zu bytes, need %zu", workspace_bytes, need);
  if (!aligned(workspace, 16)) return fail(ATTN_ERR_ALIGN, "workspace must be 16-byte aligned");
  if ((long long)N * Hkv * ((Hq / Hkv + 15) / 16) > 65535LL || (long long)N * Hq > kMaxGrid)
    return fail(ATTN_ERR_SHAPE, "grid too large");
  attn_impl::DecodeArgs d;
  d.f = make_args(N, Hq, Hkv, 1, S, E, q, k_cache, v_cache, mode, scale, gamma, 1, 0, 0, sink, o, lse);
  d.f.kv_rows = (int)cap;
  d.num_splits = splits;
  d.part_o = static_cast<float*>(workspace);
  d.part_ml = d.part_o + (size_t)N * Hq * splits * E;
  return hip_status(launch_decode(dt, d, static_cast<hipStream_t>(stream)), "attn_stream_decode launch");
}

const char* attn_status_string(int status) {
  switch (status) {
    case ATTN_OK: return "ok";
    case ATTN_ERR_NULL: return "null pointer";
    case ATTN_ERR_SHAPE: return "inconsistent sizes";
    case ATTN_ERR_DTYPE: return "unknown element type";
    case ATTN_ERR_UNSUPPORTED: return "unsupported configuration";
    case ATTN_ERR_ALIGN: return "misaligned pointer";
    case ATTN_ERR_WORKSPACE: return "workspace missing or too small";
    case ATTN_ERR_HIP: return "HIP runtime error";
    case ATTN_ERR_ARG: return "invalid argument";
    default: return "unknown status";
  }
}

const char* attn_last_error(void) { return g_last_error; }

}  // extern "C"
#pragma GCC visibility pop
