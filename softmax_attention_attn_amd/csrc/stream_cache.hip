// stream_cache.hip -- rolling key/value cache append for streaming decode.
//
// The StreamingLLM recipe ("Attention Sink LLM..." page, section 3.2) keeps the
// key/value rows of the first n_sink tokens for good and only the `window`
// most recent tokens after them, in a ring.  Per (batch, kv head) the cache has
// C = n_sink + window rows; the token at absolute position p lives in row
//   p                               (p < n_sink)
//   n_sink + (p - n_sink) % window  (otherwise).
// Appending T tokens at positions pos .. pos+T-1 writes only those that are
// still kept once the append is complete (p < n_sink, or p > pos+T-1-window),
// so no two threads write one row and the result does not depend on order.
//
// The copy is HBM-bound and has no arithmetic: one thread moves one 16-byte
// chunk of a K row and the same chunk of the V row; consecutive threads cover
// consecutive chunks of a row, then consecutive rows, so both the reads and
// the writes of a wave are whole contiguous rows.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "kernels.h"

namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

struct AppendParams {
  const uint8_t* k_new;
  const uint8_t* v_new;
  uint8_t* k_cache;
  uint8_t* v_cache;
  long long pos;
  int Hkv, T, n_sink, window;
  int row_chunks;  // 16-byte chunks per row
  int A;           // written tokens t in [0, A) (the sink part) ...
  int B;           // ... and t in [B, T) (the window part), B >= A
  int per_slice;   // A + (T - B): written tokens per (batch, kv head)
  long long total; // chunks to move
};

__global__ __launch_bounds__(256) void stream_append_kernel(AppendParams p) {
  const long long id = (long long)blockIdx.x * blockDim.x + threadIdx.x;
  if (id >= p.total) return;
  const int c = (int)(id % p.row_chunks);
  const long long row = id / p.row_chunks;           // written-row index over all slices
  const int i = (int)(row % p.per_slice);             // written token within the slice
  const long long slice = row / p.per_slice;          // n * Hkv + kv head
  const int t = i < p.A ? i : p.B + (i - p.A);        // token index within the new block
  const long long pabs = p.pos + t;
  const long long slot = pabs < p.n_sink ? pabs : p.n_sink + (pabs - p.n_sink) % p.window;
  const long long cap = (long long)p.n_sink + p.window;
  const size_t rb = (size_t)p.row_chunks * 16;
  const size_t src = ((size_t)slice * p.T + t) * rb + (size_t)c * 16;
  const size_t dst = ((size_t)slice * cap + slot) * rb + (size_t)c * 16;
  *reinterpret_cast<u32x4*>(p.k_cache + dst) = *reinterpret_cast<const u32x4*>(p.k_new + src);
  *reinterpret_cast<u32x4*>(p.v_cache + dst) = *reinterpret_cast<const u32x4*>(p.v_new + src);
}

}  // namespace

namespace attn_impl {

hipError_t launch_stream_append(const StreamAppendArgs& a, hipStream_t stream) {
  AppendParams p;
  p.k_new = static_cast<const uint8_t*>(a.k_new);
  p.v_new = static_cast<const uint8_t*>(a.v_new);
  p.k_cache = static_cast<uint8_t*>(a.k_cache);
  p.v_cache = static_cast<uint8_t*>(a.v_cache);
  p.pos = a.pos;
  p.Hkv = a.Hkv;
  p.T = a.T;
  p.n_sink = a.n_sink;
  p.window = a.window;
  p.row_chunks = a.E * a.elem_bytes / 16;
  // Sink part: positions below n_sink; window part: the last `window` tokens.
  const long long sink_left = (long long)a.n_sink - a.pos;
  p.A = (int)(sink_left <= 0 ? 0 : (sink_left < a.T ? sink_left : a.T));
  const int wstart = a.T > a.window ? a.T - a.window : 0;
  p.B = wstart > p.A ? wstart : p.A;
  p.per_slice = p.A + (a.T - p.B);
  p.total = (long long)a.N * a.Hkv * p.per_slice * p.row_chunks;
  if (p.total == 0) return hipSuccess;
  const long long blocks = (p.total + 255) / 256;
  hipLaunchKernelGGL(stream_append_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, p);
  return hipGetLastError();
}

}  // namespace attn_impl
