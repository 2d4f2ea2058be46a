// kernels.h -- launch-side description of the gfx950 kernels (internal to libattn).
//
// The host API (attn_api.cpp) validates arguments, fills these parameter blocks
// and calls the launchers; each launcher enqueues its kernel(s) on the given
// stream and returns the hipError_t of the launch.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "attn.h"

namespace attn_impl {

// Everything a forward kernel needs; element pointers are raw bit storage
// (uint16_t for bf16, float for f32).  Layouts: q,o (N,Hq,L,E); k,v (N,Hkv,S,E).
struct FwdArgs {
  const void* q;
  const void* k;
  const void* v;
  void* o;
  float* lse;
  const float* sink;  // Hq logits or nullptr
  int N, Hq, Hkv, L, S, E;
  int kv_rows;        // rows between consecutive (batch, kv head) slices of k/v (>= S)
  int n_reg;          // register rows at the start of K/V
  int causal;
  int window;         // 0 = none
  int rbf;            // 0 = dot, 1 = rbf
  float scale;        // dot logit scale
  float gamma;        // rbf width
  // General bias (prefill only): key_len (N ints) marks real keys r >= key_len[n]
  // as padding; bias is a float32 addend (bias_kind 1, natural-log units) or a
  // uint8 mask (bias_kind 2, 0 hides the pair) at bias[n*bias_sn + h*bias_sh +
  // i*S + j].  nullptr = none.
  const int* key_len;
  const void* bias;
  int bias_kind;
  long long bias_sn, bias_sh;
};

// Split-K decode: workspace holds the per-split partial results.
struct DecodeArgs {
  FwdArgs f;          // f.L == 1
  int num_splits;
  float* part_o;      // [N][Hq][num_splits][E]   unnormalised outputs
  float* part_ml;     // [N][Hq][num_splits][2]   running max (log2 units), running sum
  const int* key_index = nullptr;  // optional: per query head, index_count key rows to attend to
  int index_count = 0;
};

hipError_t launch_prefill_bf16(const FwdArgs& a, hipStream_t stream);
// Sliding-window variant: one key band in LDS per (kv head, query block), shared by
// the GQA group; prefill_band_fits() tells whether a call is in its scope.
bool prefill_band_fits(const FwdArgs& a);
hipError_t launch_prefill_bf16_band(const FwdArgs& a, hipStream_t stream);
hipError_t launch_prefill_f32(const FwdArgs& a, hipStream_t stream);
hipError_t launch_decode_bf16(const DecodeArgs& a, hipStream_t stream);
// fp32 inputs: the same split-K scheme, partials and indexed mode on the vector ALUs.
hipError_t launch_decode_f32(const DecodeArgs& a, hipStream_t stream);

// Device scratch for the no-allocation decode (decode_bf16.hip): a static
// device array of kDecodeScratchBytes per GPU.  decode_scratch() returns its
// address on the current device (looked up once per device, then cached).
constexpr size_t kDecodeScratchBytes = ATTN_DECODE_NOALLOC_SCRATCH_BYTES;
hipError_t decode_scratch(float** out);

// Backward: gradients of O for the upstream gradient dout (bf16, no user bias).
// workspace: backward_workspace_bytes(N, Hq, L) bytes (D_i, reference max per
// row, sink partial sums).
struct BwdArgs {
  FwdArgs f;          // q, k, v, sizes, mode, flags, sink (o / lse of f unused)
  const void* o;      // forward output (N,Hq,L,E)
  const float* lse;   // forward LSE (N,Hq,L)
  const void* dout;   // upstream gradient (N,Hq,L,E)
  void* dq;           // (N,Hq,L,E)
  void* dk;           // (N,Hkv,S,E)
  void* dv;           // (N,Hkv,S,E)
  float* dsink;       // Hq values or nullptr
  float* workspace;
};
hipError_t launch_backward_bf16(const BwdArgs& a, hipStream_t stream);
// fp32 inputs: the same gradients, workspace layout and conventions on the vector ALUs.
hipError_t launch_backward_f32(const BwdArgs& a, hipStream_t stream);
size_t backward_workspace_bytes(int N, int Hq, int L);

// SOCKET soft-LSH sparse decode (socket_bf16.hip).
// Longest key list one split of an indexed decode takes (it is staged in LDS).
constexpr int kDecodeIndexMax = 4096;

// Bytes of bucket codes per key: codes of at most 4 bits are packed two per
// byte (table t in the low nibble of byte t/2 when t is even, else the high
// nibble); wider codes take one byte per table.
__host__ __device__ inline int socket_code_bytes(int tables, int bits) { return bits <= 4 ? (tables + 1) / 2 : tables; }

struct SocketHashArgs {
  const void* k;
  const void* v;
  const float* proj;       // (tables*bits, E)
  uint8_t* buckets;        // (N, Hkv, S, socket_code_bytes(tables, bits))
  float* vnorm;            // (N, Hkv, S)
  int N, Hkv, S, E, tables, bits;
  bool f32 = false;        // k and v are float32 (else bf16)
};
hipError_t launch_socket_hash(const SocketHashArgs& a, hipStream_t stream);

struct SocketSelectArgs {
  const void* q;           // (N, Hq, 1, E)
  const float* proj;
  const uint8_t* buckets;
  const float* vnorm;
  float* probs;            // workspace [N*Hq][tables][2^bits]
  float* scores;           // workspace [N*Hq][S]
  int* selected;           // [N*Hq][top_k] ascending key rows
  int N, Hq, Hkv, S, E, tables, bits, top_k;
  float tau;
  bool f32 = false;        // q is float32 (else bf16)
};
hipError_t launch_socket_select(const SocketSelectArgs& a, hipStream_t stream);
size_t socket_lds_bytes(int G, int tables, int bits);

// Rolling key/value cache append: tokens at positions pos .. pos+T-1 from
// k_new / v_new (N, Hkv, T, E) into k_cache / v_cache (N, Hkv, n_sink+window, E);
// only the tokens still kept after the append are written (see slot rule in attn.h).
struct StreamAppendArgs {
  const void* k_new;
  const void* v_new;
  void* k_cache;
  void* v_cache;
  int N, Hkv, E, elem_bytes;
  int n_sink, window, T;
  long long pos;
};
hipError_t launch_stream_append(const StreamAppendArgs& a, hipStream_t stream);

// Key range attn_decode streams: registers [0, n_reg) followed by the visible
// real keys [n_reg + first_real, S); `count` = number of keys in that list.
struct DecodeKeys {
  int first_real;
  int count;
};
DecodeKeys decode_keys(int S, int n_reg, int causal, int window);

}  // namespace attn_impl
