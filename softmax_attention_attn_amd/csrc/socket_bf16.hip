// socket_bf16.hip -- SOCKET soft-LSH key selection for sparse decode, gfx950.
//
// Follows the method of the "기술 요약: SOCKET" page (method, soft LSH steps
// 1-4): at prefill every key is hashed by random hyperplanes into `tables`
// tables of 2^bits buckets and the norm of its value vector is cached; at
// decode the query gets a temperature-controlled soft assignment over each
// table's buckets, every key is scored by the probability mass of its own
// buckets summed over the tables times its value norm, and the top_k keys by
// score are attended to exactly (by the split-K decode in indexed mode).
//
// Kernels (all HBM / latency bound; the scores read tables + 4 bytes per key
// where dense decode reads 4E bytes of K and V):
//  - socket_hash_kernel: one thread per (key, table); the `bits` projections
//    are float32 fused multiply-add chains over the key's elements in element
//    order (the same float32 decision an fp32 reference makes), bit set iff > 0.
//    Threads of table 0 also write |v|.
//  - socket_prob_kernel: per query head, y = W q and, per table, the
//    probability of every bucket: the softmax over the 2^bits sign patterns of
//    sum_b s_b y_b / tau factorises into prod_b sigmoid(2 s_b y_b / tau).
//  - socket_score_kernel: one thread per key of a (batch, kv head); the bucket
//    probabilities of the group's query heads sit in LDS, so the key's codes
//    are read once for all of them.
//  - socket_select_kernel: one workgroup per query head; exact top_k by a
//    3-pass radix select on the float bits (scores are >= 0, so their bit
//    patterns order like the values), then an ordered compaction: every key
//    above the threshold and the lowest-index keys equal to it, ascending.
#include "device_common.h"
#include "kernels.h"

using namespace attn_dev;

namespace {

constexpr int kMaxProj = 512;  // tables * bits
constexpr int SEL_T = 1024;    // threads of the selection workgroup

template <int E>
__global__ __launch_bounds__(256) void socket_hash_kernel(attn_impl::SocketHashArgs a) {
  const long long gid = (long long)blockIdx.x * 256 + threadIdx.x;
  const long long nkeys = (long long)a.N * a.Hkv * a.S;
  if (gid >= nkeys * a.tables) return;
  const long long j = gid / a.tables;
  const int t = (int)(gid % a.tables);
  const uint16_t* krow = static_cast<const uint16_t*>(a.k) + (size_t)j * E;
  uint32_t kw[E / 2];
#pragma unroll
  for (int c = 0; c < E / 8; ++c) {
    const u32x4 x = *reinterpret_cast<const u32x4*>(krow + 8 * c);
#pragma unroll
    for (int w = 0; w < 4; ++w) kw[4 * c + w] = x[w];
  }
  float x[8];
#pragma unroll
  for (int b = 0; b < 8; ++b) x[b] = 0.f;
  const float* w0 = a.proj + (size_t)t * a.bits * E;  // this table's hyperplanes (cached)
  for (int e2 = 0; e2 < E / 2; ++e2) {
    const float k0 = bf16_lo(kw[e2]), k1 = bf16_hi(kw[e2]);
#pragma unroll
    for (int b = 0; b < 8; ++b) {
      if (b < a.bits) {
        x[b] = __builtin_fmaf(k0, w0[b * E + 2 * e2], x[b]);
        x[b] = __builtin_fmaf(k1, w0[b * E + 2 * e2 + 1], x[b]);
      }
    }
  }
  uint32_t code = 0;
#pragma unroll
  for (int b = 0; b < 8; ++b)
    if (b < a.bits && x[b] > 0.f) code |= 1u << b;
  a.buckets[gid] = (uint8_t)code;
  if (t == 0 && a.vnorm) {
    const uint16_t* vrow = static_cast<const uint16_t*>(a.v) + (size_t)j * E;
    float ss = 0.f;
#pragma unroll
    for (int c = 0; c < E / 8; ++c) ss += sumsq8(*reinterpret_cast<const u32x4*>(vrow + 8 * c));
    a.vnorm[j] = sqrtf(ss);
  }
}

template <int E>
__global__ __launch_bounds__(256) void socket_prob_kernel(attn_impl::SocketSelectArgs a) {
  __shared__ float sY[kMaxProj];
  const int nh = blockIdx.x;
  const int tid = threadIdx.x;
  const int nproj = a.tables * a.bits;
  const uint16_t* qrow = static_cast<const uint16_t*>(a.q) + (size_t)nh * E;
  for (int i = tid; i < nproj; i += 256) {
    const float* w = a.proj + (size_t)i * E;
    float y = 0.f;
    for (int e2 = 0; e2 < E / 2; ++e2) {
      const uint32_t qq = *reinterpret_cast<const uint32_t*>(qrow + 2 * e2);
      y = __builtin_fmaf(bf16_lo(qq), w[2 * e2], y);
      y = __builtin_fmaf(bf16_hi(qq), w[2 * e2 + 1], y);
    }
    sY[i] = y;
  }
  __syncthreads();
  const int nb = 1 << a.bits;
  const float c = 2.f * kLog2e / a.tau;
  float* out = a.probs + (size_t)nh * a.tables * nb;
  for (int i = tid; i < a.tables * nb; i += 256) {
    const int t = i / nb, code = i % nb;
    float pr = 1.f;
    for (int b = 0; b < a.bits; ++b) {
      const float sy = ((code >> b) & 1) ? sY[t * a.bits + b] : -sY[t * a.bits + b];
      pr *= 1.f / (1.f + exp2f(-c * sy));  // sigmoid(2 s y / tau)
    }
    out[i] = pr;
  }
}

__global__ __launch_bounds__(256) void socket_score_kernel(attn_impl::SocketSelectArgs a) {
  extern __shared__ float sP[];  // [G][tables][2^bits]
  const int G = a.Hq / a.Hkv;
  const int nk = blockIdx.y;     // n * Hkv + kv head
  const int n = nk / a.Hkv, kh = nk % a.Hkv;
  const int nb = 1 << a.bits;
  const int per = a.tables * nb;
  const float* src = a.probs + ((size_t)n * a.Hq + (size_t)kh * G) * per;
  for (int i = threadIdx.x; i < G * per; i += 256) sP[i] = src[i];
  __syncthreads();
  const int j = blockIdx.x * 256 + threadIdx.x;
  if (j >= a.S) return;
  const size_t key = (size_t)nk * a.S + j;
  const uint8_t* code = a.buckets + key * a.tables;
  const float nv = a.vnorm[key];
  float acc[16];
#pragma unroll
  for (int g = 0; g < 16; ++g) acc[g] = 0.f;
  for (int t = 0; t < a.tables; ++t) {
    const int c = code[t];
#pragma unroll
    for (int g = 0; g < 16; ++g)
      if (g < G) acc[g] += sP[(g * a.tables + t) * nb + c];
  }
#pragma unroll
  for (int g = 0; g < 16; ++g)
    if (g < G) a.scores[((size_t)n * a.Hq + (size_t)kh * G + g) * a.S + j] = nv * acc[g];
}

// Exclusive prefix sum over the workgroup of one int per thread (LDS
// Hillis-Steele scan); every thread must call it.
__device__ __forceinline__ int block_exclusive_scan(int* buf, int v) {
  const int tid = threadIdx.x;
  buf[tid] = v;
  __syncthreads();
  for (int off = 1; off < SEL_T; off <<= 1) {
    const int add = tid >= off ? buf[tid - off] : 0;
    __syncthreads();
    buf[tid] += add;
    __syncthreads();
  }
  const int excl = buf[tid] - v;
  __syncthreads();  // buf is reused by the next call
  return excl;
}

__global__ __launch_bounds__(SEL_T) void socket_select_kernel(attn_impl::SocketSelectArgs a) {
  __shared__ int hist[2048];
  __shared__ int scan[SEL_T];
  __shared__ uint32_t sPrefix, sMask;
  __shared__ int sRemain;
  const int nh = blockIdx.x;
  const int tid = threadIdx.x;
  const uint32_t* sc = reinterpret_cast<const uint32_t*>(a.scores) + (size_t)nh * a.S;
  int* out = a.selected + (size_t)nh * a.top_k;

  // Radix select of the top_k-th largest bit pattern: 11 + 11 + 10 bits.
  if (tid == 0) {
    sPrefix = 0;
    sMask = 0;
    sRemain = a.top_k;
  }
#pragma unroll
  for (int pass = 0; pass < 3; ++pass) {
    const int sh = pass == 0 ? 21 : (pass == 1 ? 10 : 0);
    const int nbins = pass == 2 ? 1024 : 2048;
    for (int i = tid; i < nbins; i += SEL_T) hist[i] = 0;
    __syncthreads();
    const uint32_t prefix = sPrefix, mask = sMask;
    for (int j = tid; j < a.S; j += SEL_T) {
      const uint32_t v = sc[j];
      if ((v & mask) == prefix) atomicAdd(&hist[(v >> sh) & (nbins - 1)], 1);
    }
    __syncthreads();
    if (tid == 0) {  // walk the bins from the top until `remain` keys are covered
      int remain = sRemain, bin = nbins - 1;
      for (; bin > 0; --bin) {
        if (hist[bin] >= remain) break;
        remain -= hist[bin];
      }
      sPrefix = prefix | ((uint32_t)bin << sh);
      sMask = mask | ((uint32_t)(nbins - 1) << sh);
      sRemain = remain;
    }
    __syncthreads();
  }
  const uint32_t thr = sPrefix;  // the top_k-th largest value
  const int need_eq = sRemain;   // keys equal to it that are taken (lowest indices)

  // Ordered compaction over contiguous chunks of keys.
  const int chunk = (a.S + SEL_T - 1) / SEL_T;
  const int j0 = min(a.S, tid * chunk), j1 = min(a.S, j0 + chunk);
  int gt = 0, eq = 0;
  for (int j = j0; j < j1; ++j) {
    const uint32_t v = sc[j];
    gt += v > thr;
    eq += v == thr;
  }
  const int eq_before = block_exclusive_scan(scan, eq);
  const int take_eq = max(0, min(eq, need_eq - eq_before));
  int pos = block_exclusive_scan(scan, gt + take_eq);
  int eq_seen = 0;
  for (int j = j0; j < j1; ++j) {
    const uint32_t v = sc[j];
    if (v > thr) {
      out[pos++] = j;
    } else if (v == thr) {
      if (eq_seen < take_eq) out[pos++] = j;
      ++eq_seen;
    }
  }
}

}  // namespace

namespace attn_impl {

hipError_t launch_socket_hash_bf16(const SocketHashArgs& a, hipStream_t stream) {
  const long long total = (long long)a.N * a.Hkv * a.S * a.tables;
  if (total == 0) return hipSuccess;
  const unsigned blocks = (unsigned)((total + 255) / 256);
  if (a.E == 128)
    hipLaunchKernelGGL((socket_hash_kernel<128>), dim3(blocks), dim3(256), 0, stream, a);
  else
    hipLaunchKernelGGL((socket_hash_kernel<64>), dim3(blocks), dim3(256), 0, stream, a);
  return hipGetLastError();
}

hipError_t launch_socket_select_bf16(const SocketSelectArgs& a, hipStream_t stream) {
  if (a.E == 128)
    hipLaunchKernelGGL((socket_prob_kernel<128>), dim3((unsigned)(a.N * a.Hq)), dim3(256), 0, stream, a);
  else
    hipLaunchKernelGGL((socket_prob_kernel<64>), dim3((unsigned)(a.N * a.Hq)), dim3(256), 0, stream, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int G = a.Hq / a.Hkv;
  const size_t lds = (size_t)G * a.tables * (1u << a.bits) * sizeof(float);
  hipLaunchKernelGGL(socket_score_kernel, dim3((unsigned)((a.S + 255) / 256), (unsigned)(a.N * a.Hkv)), dim3(256),
                     lds, stream, a);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(socket_select_kernel, dim3((unsigned)(a.N * a.Hq)), dim3(SEL_T), 0, stream, a);
  return hipGetLastError();
}

size_t socket_lds_bytes(int G, int tables, int bits) { return (size_t)G * tables * (1u << bits) * sizeof(float); }

}  // namespace attn_impl
