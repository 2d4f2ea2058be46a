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
//  - socket_hash_kernel: one thread per key; the `bits` projections of each
//    table are float32 fused multiply-add chains over the key's elements in
//    element order (the same float32 decision an fp32 reference makes), bit
//    set iff > 0; hyperplanes staged in LDS.  Also writes |v|.  Keys and
//    values are bf16 or float32 (the key row is held as 32-bit words either
//    way: two bf16 elements or one float32 element per word).
//  - socket_prob_kernel: per query head, y = W q and, per table, the
//    probability of every bucket: the softmax over the 2^bits sign patterns of
//    sum_b s_b y_b / tau factorises into prod_b sigmoid(2 s_b y_b / tau).
//  - socket_score_fast / socket_score_kernel: threads own keys of a (batch,
//    kv head); the bucket probabilities of the group's query heads sit in LDS,
//    packed per (table, code), so the key's codes are read once for all of
//    them (the fast kernel for group sizes 1/2/4/8/16 and tables a multiple of
//    16, the other for any shape).
//  - socket_select_kernel: one workgroup per query head; exact top_k on the
//    float bits (scores are >= 0, so their bit patterns order like the
//    values): a sampled bracket narrows the threshold to a few thousand
//    candidates in one read of the scores (else a 3-pass radix select), then
//    an ordered compaction writes every key above the threshold and the
//    lowest-index keys equal to it, ascending.
#include "device_common.h"
#include "kernels.h"

using namespace attn_dev;

namespace {

constexpr int kMaxProj = 512;  // tables * bits
constexpr int SEL_T = 1024;    // threads of the selection workgroup

// Hashing: one thread per key, its row in registers.  The hyperplanes of the
// TG tables that fit in HASH_LDS bytes sit in LDS as [table][element][BP]
// (BP = bits padded to 4 or 8, padding weights zero), so every element's weights of all the table's
// hyperplanes are one broadcast LDS read.  Each projection is a float32 fused
// multiply-add chain over the elements in order, starting from zero.
constexpr int HASH_LDS = 32 * 1024;

template <int E, int BP, bool F32>
__global__ __launch_bounds__(256) void socket_hash_kernel(attn_impl::SocketHashArgs a) {
  extern __shared__ float sW[];
  constexpr int TG = HASH_LDS / (E * BP * 4);  // tables per LDS stage
  constexpr int KW = F32 ? E : E / 2;          // 32-bit words of one key row
  typedef float wvec __attribute__((ext_vector_type(BP)));
  const long long nkeys = (long long)a.N * a.Hkv * a.S;
  const long long j = (long long)blockIdx.x * 256 + threadIdx.x;
  const bool ok = j < nkeys;
  uint32_t kw[KW];
  {
    const uint32_t* krow = static_cast<const uint32_t*>(a.k) + (size_t)(ok ? j : 0) * KW;
#pragma unroll
    for (int c = 0; c < KW / 4; ++c) {
      const u32x4 x = *reinterpret_cast<const u32x4*>(krow + 4 * c);
#pragma unroll
      for (int w = 0; w < 4; ++w) kw[4 * c + w] = x[w];
    }
  }
  if (ok && a.vnorm) {
    const uint32_t* vrow = static_cast<const uint32_t*>(a.v) + (size_t)j * KW;
    float ss = 0.f;
#pragma unroll
    for (int c = 0; c < KW / 4; ++c) {
      const u32x4 x = *reinterpret_cast<const u32x4*>(vrow + 4 * c);
      if (F32) {
#pragma unroll
        for (int w = 0; w < 4; ++w) ss = __builtin_fmaf(__uint_as_float(x[w]), __uint_as_float(x[w]), ss);
      } else {
        ss += sumsq8(x);
      }
    }
    a.vnorm[j] = sqrtf(ss);
  }
  // Codes are gathered into 32-bit words (8 four-bit or 4 eight-bit codes),
  // stored whole when every key's code bytes are whole aligned words.
  const int cw = a.bits <= 4 ? 4 : 8;  // bits per stored code
  const int per = 32 / cw;              // codes per word
  const int cbytes = attn_impl::socket_code_bytes(a.tables, a.bits);
  const bool words = (cbytes & 3) == 0 && (reinterpret_cast<uintptr_t>(a.buckets) & 3) == 0;
  uint8_t* dst = a.buckets + (size_t)(ok ? j : 0) * cbytes;
  uint32_t word = 0;
  for (int t0 = 0; t0 < a.tables; t0 += TG) {
    const int tn = min(TG, a.tables - t0);
    __syncthreads();  // the previous stage's weights are no longer read
    for (int i = threadIdx.x; i < tn * E * BP; i += 256) {
      const int tt = i / (E * BP), r = i % (E * BP), e = r / BP, b = r % BP;
      sW[i] = b < a.bits ? a.proj[((size_t)(t0 + tt) * a.bits + b) * E + e] : 0.f;
    }
    __syncthreads();
    for (int tt = 0; tt < tn; ++tt) {
      const float* w = sW + tt * E * BP;
      float x[BP];
#pragma unroll
      for (int b = 0; b < BP; ++b) x[b] = 0.f;
#pragma unroll
      for (int e2 = 0; e2 < E / 2; ++e2) {
        const float k0 = F32 ? __uint_as_float(kw[2 * e2]) : bf16_lo(kw[e2]);
        const float k1 = F32 ? __uint_as_float(kw[2 * e2 + 1]) : bf16_hi(kw[e2]);
        const wvec w0 = *reinterpret_cast<const wvec*>(w + (2 * e2) * BP);
        const wvec w1 = *reinterpret_cast<const wvec*>(w + (2 * e2 + 1) * BP);
#pragma unroll
        for (int b = 0; b < BP; ++b) {
          x[b] = __builtin_fmaf(k0, w0[b], x[b]);
          x[b] = __builtin_fmaf(k1, w1[b], x[b]);
        }
      }
      uint32_t code = 0;
#pragma unroll
      for (int b = 0; b < BP; ++b)
        if (b < a.bits && x[b] > 0.f) code |= 1u << b;
      const int t = t0 + tt;
      word |= code << (cw * (t % per));
      if (t % per == per - 1 || t == a.tables - 1) {  // a word is complete
        const int wi = t / per;
        if (ok) {
          if (words) {
            *reinterpret_cast<uint32_t*>(dst + 4 * wi) = word;
          } else {
            const int nb = min(4, cbytes - 4 * wi);
            for (int b = 0; b < nb; ++b) dst[4 * wi + b] = (uint8_t)(word >> (8 * b));
          }
        }
        word = 0;
      }
    }
  }
}

template <int E, bool F32>
__global__ __launch_bounds__(256) void socket_prob_kernel(attn_impl::SocketSelectArgs a) {
  __shared__ float sY[kMaxProj];
  const int nh = blockIdx.x;
  const int tid = threadIdx.x;
  const int nproj = a.tables * a.bits;
  constexpr int QW = F32 ? E : E / 2;  // 32-bit words of the query row
  const uint32_t* qrow = static_cast<const uint32_t*>(a.q) + (size_t)nh * QW;
  for (int i = tid; i < nproj; i += 256) {
    const float* w = a.proj + (size_t)i * E;
    float y = 0.f;
    for (int e2 = 0; e2 < E / 2; ++e2) {
      float q0, q1;
      if (F32) {
        q0 = __uint_as_float(qrow[2 * e2]);
        q1 = __uint_as_float(qrow[2 * e2 + 1]);
      } else {
        q0 = bf16_lo(qrow[e2]);
        q1 = bf16_hi(qrow[e2]);
      }
      y = __builtin_fmaf(q0, w[2 * e2], y);
      y = __builtin_fmaf(q1, w[2 * e2 + 1], y);
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

// Per (key, table) the bucket probabilities of the P query heads packed
// together (P = 4, 2 or 1, a divisor of the group size) are one LDS read.
template <int P>
__device__ __forceinline__ void score_lookup(const float* __restrict__ sP, int row, int ngrp, int stride,
                                             float (&acc)[16]) {
#pragma unroll
  for (int g = 0; g < 16 / P; ++g) {
    if (g < ngrp) {
      const float* e = sP + (size_t)(g * stride + row) * P;
      if constexpr (P == 4) {
        const f32x4 x = *reinterpret_cast<const f32x4*>(e);
        acc[4 * g] += x[0];
        acc[4 * g + 1] += x[1];
        acc[4 * g + 2] += x[2];
        acc[4 * g + 3] += x[3];
      } else if constexpr (P == 2) {
        const float2 x = *reinterpret_cast<const float2*>(e);
        acc[2 * g] += x.x;
        acc[2 * g + 1] += x.y;
      } else {
        acc[g] += e[0];
      }
    }
  }
}

constexpr int SCORE_KPT = 4;  // keys per thread of the score kernel

// Generic scoring (any group size, table count and alignment; codes read a
// byte at a time): one workgroup scores 256 * SCORE_KPT keys of one (batch, kv
// head) for all G query heads of its group.  LDS holds the group's bucket
// probabilities as [G/P][tables][2^bits][P].
template <int P>
__global__ __launch_bounds__(256) void socket_score_kernel(attn_impl::SocketSelectArgs a) {
  extern __shared__ float sP[];
  const int G = a.Hq / a.Hkv;
  const int ngrp = G / P;
  const int nk = blockIdx.y;  // n * Hkv + kv head
  const int n = nk / a.Hkv, kh = nk % a.Hkv;
  const int nb = 1 << a.bits;
  const int per = a.tables * nb;
  const float* src = a.probs + ((size_t)n * a.Hq + (size_t)kh * G) * per;
  for (int i = threadIdx.x; i < G * per; i += 256) {
    const int g = i / per, r = i % per;  // source head g, row (table, code)
    sP[((g / P) * per + r) * P + g % P] = src[i];
  }
  __syncthreads();
  const int cbytes = attn_impl::socket_code_bytes(a.tables, a.bits);
  const bool packed = a.bits <= 4;
  const size_t row0 = (size_t)n * a.Hq + (size_t)kh * G;
  for (int kk = 0; kk < SCORE_KPT; ++kk) {
    const int j = (blockIdx.x * SCORE_KPT + kk) * 256 + threadIdx.x;
    if (j >= a.S) break;
    const size_t key = (size_t)nk * a.S + j;
    const uint8_t* code = a.buckets + key * cbytes;
    float acc[16];
#pragma unroll
    for (int g = 0; g < 16; ++g) acc[g] = 0.f;
    for (int t = 0; t < a.tables; ++t) {
      const int c = packed ? (code[t >> 1] >> (4 * (t & 1))) & 15 : code[t];
      score_lookup<P>(sP, t * nb + c, ngrp, per, acc);
    }
    const float nv = a.vnorm[key];
#pragma unroll
    for (int g = 0; g < 16; ++g)
      if (g < G) a.scores[(row0 + g) * a.S + j] = nv * acc[g];
  }
}

// Ordering key of a score: its bit pattern without the sign bit (scores are
// >= 0, so this orders like the values; a NaN orders above every number).
__device__ __forceinline__ uint32_t score_key(uint32_t bits) { return bits & 0x7fffffffu; }

template <int P>
__device__ __forceinline__ void lookup_load(const float* e, float (&x)[P]) {
  if constexpr (P == 4) {
    const f32x4 v = *reinterpret_cast<const f32x4*>(e);
    x[0] = v[0];
    x[1] = v[1];
    x[2] = v[2];
    x[3] = v[3];
  } else if constexpr (P == 2) {
    const float2 v = *reinterpret_cast<const float2*>(e);
    x[0] = v.x;
    x[1] = v.y;
  } else {
    x[0] = e[0];
  }
}

// Scoring for the common shapes: group size GT in {1, 2, 4, 8, 16}, code
// bytes per key a multiple of 16 (at most 64 tables: 16-byte chunks of 16 byte
// codes, or of 32 packed 4-bit codes when PK), 16-byte aligned codes; NB =
// 2^bits when fixed at build time (constant LDS offsets), else 0.  A workgroup stages the
// group's probabilities once and scores FAST_ROUNDS * 256 * FAST_KPT keys; in
// each round every code and norm of the thread's keys is loaded first, then per
// 16-table chunk, key and packed head group 16 independent LDS reads are
// issued before they are summed.
constexpr int FAST_KPT = 2;   // keys per thread per round
constexpr int FAST_ROUNDS = 4;  // rounds per workgroup (amortise the LDS staging)

template <int GT, int NB, bool PK>
__global__ __launch_bounds__(256) void socket_score_fast(attn_impl::SocketSelectArgs a) {
  constexpr int P = GT % 4 == 0 ? 4 : (GT % 2 == 0 ? 2 : 1);
  constexpr int NG = GT / P;
  constexpr int KPT = FAST_KPT;
  extern __shared__ float sP[];
  const int nk = blockIdx.y;  // n * Hkv + kv head
  const int n = nk / a.Hkv, kh = nk % a.Hkv;
  const int nb = NB ? NB : (1 << a.bits);
  const int per = a.tables * nb;
  const float* src = a.probs + ((size_t)n * a.Hq + (size_t)kh * GT) * per;
  for (int i = threadIdx.x; i < GT * per; i += 256) {
    const int g = i / per, r = i % per;
    sP[((g / P) * per + r) * P + g % P] = src[i];
  }
  __syncthreads();
  constexpr int CPC = PK ? 32 : 16;  // codes per 16-byte chunk
  constexpr int MAXCH = 64 / CPC;    // chunks for 64 tables
  const int nch = a.tables / CPC;
  const size_t row0 = (size_t)n * a.Hq + (size_t)kh * GT;  // first query head of the group
  for (int it = 0; it < FAST_ROUNDS; ++it) {
    const int blk = blockIdx.x * FAST_ROUNDS + it;
    if (blk * KPT * 256 >= a.S) break;
    u32x4 w[KPT][MAXCH];
    float nv[KPT];
#pragma unroll
    for (int kk = 0; kk < KPT; ++kk) {
      const int j = (blk * KPT + kk) * 256 + threadIdx.x;
      const bool ok = j < a.S;
      const size_t key = (size_t)nk * a.S + (ok ? j : 0);
      const u32x4* c16 = reinterpret_cast<const u32x4*>(a.buckets + key * (a.tables * 16 / CPC));
#pragma unroll
      for (int c = 0; c < MAXCH; ++c) w[kk][c] = (ok && c < nch) ? c16[c] : u32x4{0u, 0u, 0u, 0u};
      nv[kk] = ok ? a.vnorm[key] : 0.f;
    }
    float acc[KPT][GT];
#pragma unroll
    for (int kk = 0; kk < KPT; ++kk)
#pragma unroll
      for (int g = 0; g < GT; ++g) acc[kk][g] = 0.f;
#pragma unroll
    for (int c = 0; c < MAXCH; ++c) {
      if (c < nch) {
#pragma unroll
        for (int kk = 0; kk < KPT; ++kk) {
#pragma unroll
          for (int g = 0; g < NG; ++g) {
#pragma unroll
            for (int h16 = 0; h16 < CPC / 16; ++h16) {
              // 16 tables of this chunk: codes are bytes, or nibbles of 2 words.
              float x[16][P];
#pragma unroll
              for (int b = 0; b < 16; ++b) {
                const int tb = 16 * h16 + b;  // table within the chunk
                const int code = PK ? (int)((w[kk][c][tb / 8] >> (4 * (tb % 8))) & 0xfu)
                                    : (int)((w[kk][c][tb / 4] >> (8 * (tb % 4))) & 0xffu);
                lookup_load<P>(sP + ((size_t)g * per + (CPC * c + tb) * nb + code) * P, x[b]);
              }
#pragma unroll
              for (int b = 0; b < 16; ++b)
#pragma unroll
                for (int q = 0; q < P; ++q) acc[kk][g * P + q] += x[b][q];
            }
          }
        }
      }
    }
#pragma unroll
    for (int kk = 0; kk < KPT; ++kk) {
      const int j = (blk * KPT + kk) * 256 + threadIdx.x;
      if (j < a.S) {
#pragma unroll
        for (int g = 0; g < GT; ++g) a.scores[(row0 + g) * a.S + j] = nv[kk] * acc[kk][g];
      }
    }
  }
}

template <int GT>
hipError_t launch_score_fast(const attn_impl::SocketSelectArgs& a, size_t lds, hipStream_t stream) {
  constexpr int KPT = FAST_KPT * FAST_ROUNDS;
  const dim3 grid((unsigned)((a.S + 256 * KPT - 1) / (256 * KPT)), (unsigned)(a.N * a.Hkv));
  if (a.bits == 4)
    hipLaunchKernelGGL((socket_score_fast<GT, 16, true>), grid, dim3(256), lds, stream, a);
  else if (a.bits < 4)
    hipLaunchKernelGGL((socket_score_fast<GT, 0, true>), grid, dim3(256), lds, stream, a);
  else
    hipLaunchKernelGGL((socket_score_fast<GT, 0, false>), grid, dim3(256), lds, stream, a);
  return hipGetLastError();
}

// ---- exact top-k selection -------------------------------------------------
//
// Score bit patterns without the sign bit order like the scores (they are
// >= 0), so the selection works on those integer keys: the bracket path or
// the radix path finds the top_k-th largest key, the write pass emits the
// chosen keys in ascending order (socket_select_kernel below).

constexpr int SEL_WAVES = SEL_T / 64;
static_assert(SEL_WAVES * 256 >= 4096, "pass-3 histograms must cover the pass-1 bins' storage");
constexpr int SEL_U = 8;  // loads in flight per lane

__device__ __forceinline__ int lanes_below(uint64_t m) {
  return (int)__builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0u));
}

__device__ __forceinline__ int wave_sum_int(int v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}

// Exclusive prefix sum over the workgroup of one int per thread: a shuffle
// scan inside each wave, then the wave totals through LDS (two barriers);
// every thread must call it.  buf holds at least SEL_WAVES ints.
__device__ __forceinline__ int block_exclusive_scan(int* buf, int v) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  int x = v;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int y = __shfl_up(x, o, 64);
    if (lane >= o) x += y;
  }
  if (lane == 63) buf[wave] = x;
  __syncthreads();
  int base = 0;
  for (int w = 0; w < wave; ++w) base += buf[w];
  __syncthreads();  // buf is reused by the next call
  return base + x - v;
}

// Finds, among `nbins` bins whose counts are in hist, the bin holding the
// `remain`-th largest key counting down from the top bin; sets *bin_out and
// *remain_out (the rank inside that bin).  All threads call it.
__device__ __forceinline__ void find_bin(const int* hist, int nbins, int remain, int* scan, int* bin_out,
                                         int* remain_out) {
  const int tid = threadIdx.x;
  const int bpt = (nbins + SEL_T - 1) / SEL_T;  // bins per thread, highest bins to thread 0
  const int hi = nbins - 1 - tid * bpt;
  int local = 0;
  for (int i = 0; i < bpt; ++i)
    if (hi - i >= 0) local += hist[hi - i];
  const int above = block_exclusive_scan(scan, local);
  if (above < remain && above + local >= remain) {
    int r = remain - above, b = hi;
    for (int i = 0; i < bpt; ++i, --b) {
      if (hist[b] >= r) break;
      r -= hist[b];
    }
    *bin_out = b;
    *remain_out = r;
  }
  __syncthreads();
}

// Four consecutive scores from key j on (zero past s1); 16-byte loads where
// the row allows them.
__device__ __forceinline__ u32x4 load_scores4(const uint32_t* sc, int j, int s1, bool vec) {
  u32x4 r;
  if (vec && j + 3 < s1) {
    r = *reinterpret_cast<const u32x4*>(sc + j);
  } else {
#pragma unroll
    for (int e = 0; e < 4; ++e) r[e] = j + e < s1 ? sc[j + e] : 0u;
  }
#pragma unroll
  for (int e = 0; e < 4; ++e) r[e] = score_key(r[e]);
  return r;
}

// Exclusive prefix over the wave's lanes of x in [0, 7], and the wave total.
__device__ __forceinline__ int wave_prefix3(int x, int* total) {
  int pre = 0, tot = 0;
#pragma unroll
  for (int b = 0; b < 3; ++b) {
    const uint64_t m = __ballot((x >> b) & 1);
    pre += lanes_below(m) << b;
    tot += __popcll(m) << b;
  }
  *total = tot;
  return pre;
}

constexpr int CAP = 512;          // per-wave capacity of the one-read path's two key lists
constexpr int SAMPLE_MAX = 8192;  // sample size of the one-read path
constexpr int SEL_SMEM = 4096 + 3 * SEL_WAVES * CAP;
static_assert(SEL_WAVES * CAP >= SAMPLE_MAX, "the sample lives in the first list area");
static_assert(SEL_SMEM >= SEL_WAVES * 256 + 256, "the radix path's histograms share the same LDS");

// Radix select over `n` keys (read through key(i)) whose bits under `mask`
// equal `prefix`: the `remain`-th largest, 11 bits per pass down to bit 0,
// starting below the bits already fixed (bit `top` is the highest unfixed
// bit).  Returns the key; *remain_out = its rank among the keys equal to it.
template <typename KeyAt>
__device__ __forceinline__ uint32_t select_small(KeyAt key, int n, uint32_t prefix, uint32_t mask, int top,
                                                 int remain, int* hist, int* scan, int* sv, int* remain_out) {
  const int tid = threadIdx.x;
  for (int hi = top; hi >= 0; hi -= 11) {
    const int width = hi + 1 < 11 ? hi + 1 : 11;
    const int sh = hi + 1 - width;
    const int nbins = 1 << width;
    for (int i = tid; i < nbins; i += SEL_T) hist[i] = 0;
    __syncthreads();
    for (int i = tid; i < n; i += SEL_T) {
      const uint32_t u = key(i);
      if ((u & mask) == prefix) atomicAdd(&hist[(u >> sh) & (nbins - 1)], 1);
    }
    __syncthreads();
    find_bin(hist, nbins, remain, scan, &sv[0], &sv[1]);
    prefix |= (uint32_t)sv[0] << sh;
    mask |= (uint32_t)(nbins - 1) << sh;
    remain = sv[1];
  }
  *remain_out = remain;
  return prefix;
}

// Number of entries of the ascending list d[0, n) below x.
__device__ __forceinline__ int count_below(const int* d, int n, int x) {
  int lo = 0, hi = n;
  while (lo < hi) {
    const int mid = (lo + hi) >> 1;
    if (d[mid] < x) lo = mid + 1;
    else hi = mid;
  }
  return lo;
}

// One-read path.  A sample of the scores (runs of 64 keys every Z keys, at
// most SAMPLE_MAX of them; every key when S is small) gives, by two radix
// passes over its top 22 key bits, scores L <= U around ranks top_k*f -/+ a
// 4-sigma margin (f the sample fraction; the exact rank when the sample is
// every key), so that the threshold lies in [L, U].  One pass over the scores
// by wave segments appends, in key order, each wave's keys above U (all
// chosen) and its candidates in [L, U] (index and score) to per-wave LDS
// lists.  A radix select over the candidates alone gives the exact threshold;
// each wave keeps the candidates above it and the first equal ones within the
// tie budget (lowest indices first, over the waves in order) and merges them
// with its keys above U into the output, ascending.  The bracket only decides
// speed: when it misses (more than top_k keys above U, fewer than top_k at or
// above L, or a wave list over CAP) this returns false having written
// nothing, and the radix path runs.
__device__ bool select_one_read(const attn_impl::SocketSelectArgs& a, const uint32_t* sc, bool vec, int seg,
                                int* out, int* smem, int* scan, int* sv, int* sA, int* sC, int* sPos,
                                int* sTake) {
  const int tid = threadIdx.x, wave = tid / 64, lane = tid % 64;
  const int S = a.S, K = a.top_k;
  int* hist = smem;                          // 2 x 2048 bins
  int* A = smem + 4096;                      // [SEL_WAVES][CAP] keys above U
  int* Ci = A + SEL_WAVES * CAP;             // [SEL_WAVES][CAP] candidate keys
  uint32_t* Cv = reinterpret_cast<uint32_t*>(Ci + SEL_WAVES * CAP);  // their score keys
  int* samp = A;

  // Sample: key j with (j % Z) < 64.
  int Z = 64;
  while ((long long)((S + Z - 1) / Z) * 64 > SAMPLE_MAX) Z <<= 1;
  const int nfull = S / Z, tail = S - nfull * Z;
  const int ns = nfull * 64 + (tail < 64 ? tail : 64);
  int rhi = K, rlo = K;
  if (ns < S) {
    const double f = (double)ns / S, mean = K * f;
    const int m = (int)ceil(4.0 * sqrt(mean * (1.0 - f))) + 8;
    rhi = (int)floor(mean) - m;
    rlo = (int)ceil(mean) + m;
  }
  const bool do_hi = rhi >= 1, do_lo = rlo <= ns;
  for (int i = tid; i < 2048; i += SEL_T) hist[i] = 0;
  for (int i = tid; i < ns; i += SEL_T) samp[i] = (int)score_key(sc[(i / 64) * Z + (i % 64)]);
  __syncthreads();
  for (int i = tid; i < ns; i += SEL_T) atomicAdd(&hist[samp[i] >> 20], 1);
  __syncthreads();
  uint32_t phi = 0, plo = 0;
  if (do_hi) {
    find_bin(hist, 2048, rhi, scan, &sv[0], &sv[1]);
    phi = (uint32_t)sv[0] << 20;
    rhi = sv[1];
  }
  if (do_lo) {
    find_bin(hist, 2048, rlo, scan, &sv[0], &sv[1]);
    plo = (uint32_t)sv[0] << 20;
    rlo = sv[1];
  }
  for (int i = tid; i < 4096; i += SEL_T) hist[i] = 0;
  __syncthreads();
  for (int i = tid; i < ns; i += SEL_T) {
    const uint32_t v = (uint32_t)samp[i];
    if (do_hi && (v & 0x7ff00000u) == phi) atomicAdd(&hist[(v >> 9) & 2047], 1);
    if (do_lo && (v & 0x7ff00000u) == plo) atomicAdd(&hist[2048 + ((v >> 9) & 2047)], 1);
  }
  __syncthreads();
  if (do_hi) {
    find_bin(hist, 2048, rhi, scan, &sv[0], &sv[1]);
    phi |= (uint32_t)sv[0] << 9;
  }
  if (do_lo) {
    find_bin(hist + 2048, 2048, rlo, scan, &sv[0], &sv[1]);
    plo |= (uint32_t)sv[0] << 9;
  }
  const uint32_t U = do_hi ? (phi | 0x1ffu) : 0xffffffffu;  // top of the sample's 22-bit bin
  const uint32_t L = do_lo ? plo : 0u;                       // bottom of its 22-bit bin
  __syncthreads();  // the sample (in A) is dead from here

  // Gather by wave segments, in key order.
  const int s0 = min(S, wave * seg), s1 = min(S, s0 + seg);
  int* myA = A + wave * CAP;
  int* myCi = Ci + wave * CAP;
  uint32_t* myCv = Cv + wave * CAP;
  int na = 0, nc = 0;  // wave-uniform
  for (int j0 = s0; j0 < s1; j0 += 256 * SEL_U) {
    u32x4 v[SEL_U];
#pragma unroll
    for (int u = 0; u < SEL_U; ++u) v[u] = load_scores4(sc, j0 + u * 256 + lane * 4, s1, vec);
#pragma unroll
    for (int u = 0; u < SEL_U; ++u) {
      const int jb = j0 + u * 256 + lane * 4;
      int ma = 0, mc = 0;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const bool in = jb + e < s1;
        ma |= (int)(in && v[u][e] > U) << e;
        mc |= (int)(in && v[u][e] >= L && v[u][e] <= U) << e;
      }
      int ta, tc;
      int pa = na + wave_prefix3(__builtin_popcount(ma), &ta);
      int pc = nc + wave_prefix3(__builtin_popcount(mc), &tc);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        if ((ma >> e) & 1) {
          if (pa < CAP) myA[pa] = jb + e;
          ++pa;
        }
        if ((mc >> e) & 1) {
          if (pc < CAP) {
            myCi[pc] = jb + e;
            myCv[pc] = v[u][e];
          }
          ++pc;
        }
      }
      na += ta;
      nc += tc;
    }
  }
  if (lane == 0) {
    sA[wave] = na;
    sC[wave] = nc;
  }
  __syncthreads();
  int nA = 0, nC = 0;
  bool fits = true;
  for (int w = 0; w < SEL_WAVES; ++w) {
    nA += sA[w];
    nC += sC[w];
    fits = fits && sA[w] <= CAP && sC[w] <= CAP;
  }
  if (!fits || nA > K || nA + nC < K) {  // same decision in every thread
    __syncthreads();  // everyone has read the counts before LDS is reused
    return false;
  }

  // Exact threshold among the candidates (nA == K: exactly the keys above U).
  uint32_t thr = U;
  int need_eq = 0;
  if (nA < K)
    thr = select_small(
        [&](int i) { return (i % CAP) < sC[i / CAP] ? Cv[i] : 0xffffffffu; }, SEL_WAVES * CAP, 0u, 0x80000000u, 30,
        K - nA, hist, scan, sv, &need_eq);

  // Per wave: candidates above thr and equal to it.
  int gt = 0, eq = 0;
  if (nA < K)
    for (int r = lane; r < sC[wave]; r += 64) {
      gt += myCv[r] > thr;
      eq += myCv[r] == thr;
    }
  gt = wave_sum_int(gt);
  eq = wave_sum_int(eq);
  if (lane == 0) {
    sTake[wave] = eq;  // equal-key counts for now
    sPos[wave] = gt;
  }
  __syncthreads();
  if (tid == 0) {
    int eq_before = 0, pos = 0;
    for (int w = 0; w < SEL_WAVES; ++w) {
      const int e = sTake[w], g = sPos[w];
      const int take = max(0, min(e, need_eq - eq_before));
      eq_before += e;
      sTake[w] = take;
      sPos[w] = pos;
      pos += sA[w] + g + take;
    }
  }
  __syncthreads();

  // Keep the chosen candidates, in order, at the front of the wave's list.
  const int take_eq = sTake[wave];
  int kept = 0, eq_seen = 0;
  if (nA < K)
    for (int r0 = 0; r0 < sC[wave]; r0 += 64) {
      const int r = r0 + lane;
      const bool in = r < sC[wave];
      const uint32_t x = in ? myCv[r] : 0u;
      const int idx = in ? myCi[r] : 0;
      const bool is_eq = in && x == thr;
      const uint64_t em = __ballot(is_eq);
      const bool take = in && (x > thr || (is_eq && eq_seen + lanes_below(em) < take_eq));
      const uint64_t tm = __ballot(take);
      if (take) myCi[kept + lanes_below(tm)] = idx;
      kept += __popcll(tm);
      eq_seen += __popcll(em);
    }

  // Merge the wave's keys above U with its kept candidates (both ascending).
  const int na_w = sA[wave];
  int* o = out + sPos[wave];
  for (int i = lane; i < na_w; i += 64) o[i + count_below(myCi, kept, myA[i])] = myA[i];
  for (int i = lane; i < kept; i += 64) o[i + count_below(myA, na_w, myCi[i])] = myCi[i];
  return true;
}

// One workgroup of SEL_T threads per query head.  Wave w owns the contiguous
// key segment [w * seg, (w + 1) * seg) and walks it in steps of 256 keys (64
// lanes x 4 consecutive keys), so (wave, step, lane, element) is ascending key
// order.  The threshold and the per-wave counts come from the bracket path
// (one read of the scores) or, when its bracket misses, from three radix
// passes (12 + 12 + 8 bits; the last keeps one histogram per wave, which gives
// every wave its counts without another read).  The write pass then places
// the keys above the threshold and the lowest-index keys equal to it in
// ascending order using ballots.
__global__ __launch_bounds__(SEL_T) void socket_select_kernel(attn_impl::SocketSelectArgs a) {
  __shared__ int smem[SEL_SMEM];
  __shared__ int scan[SEL_T];
  __shared__ int sv[8];
  __shared__ int sGt[SEL_WAVES], sEq[SEL_WAVES], sPos[SEL_WAVES], sTake[SEL_WAVES];
  const int nh = blockIdx.x;
  const int tid = threadIdx.x, wave = tid / 64, lane = tid % 64;
  const uint32_t* sc = reinterpret_cast<const uint32_t*>(a.scores) + (size_t)nh * a.S;
  const bool vec = (a.S & 3) == 0;  // rows start 16-byte aligned
  int* out = a.selected + (size_t)nh * a.top_k;
  const int seg = (a.S + SEL_WAVES * 256 - 1) / (SEL_WAVES * 256) * 256;
  const int s0 = min(a.S, wave * seg), s1 = min(a.S, s0 + seg);
  if (select_one_read(a, sc, vec, seg, out, smem, scan, sv, sGt, sEq, sPos, sTake)) return;

  uint32_t thr;
  int need_eq;
  {
    int* hist = smem;  // passes 1-2: 4096 bins; pass 3: [SEL_WAVES][256] + their sum
    uint32_t prefix = 0, mask = 0;
    int remain = a.top_k;
    int above = 0;  // this lane's keys whose top 24 bits exceed the pass-3 prefix
#pragma unroll
    for (int pass = 0; pass < 3; ++pass) {
      const int sh = pass == 0 ? 20 : (pass == 1 ? 8 : 0);
      const int nbins = pass == 2 ? 256 : 4096;
      const int hsize = pass == 2 ? SEL_WAVES * 256 : 4096;
      int* h = pass == 2 ? hist + wave * 256 : hist;
      for (int i = tid; i < hsize; i += SEL_T) hist[i] = 0;
      __syncthreads();
      for (int j0 = s0; j0 < s1; j0 += 256 * SEL_U) {
        u32x4 v[SEL_U];
#pragma unroll
        for (int u = 0; u < SEL_U; ++u) v[u] = load_scores4(sc, j0 + u * 256 + lane * 4, s1, vec);
#pragma unroll
        for (int u = 0; u < SEL_U; ++u) {
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            if (j0 + u * 256 + lane * 4 + e < s1) {
              const uint32_t x = v[u][e];
              if ((x & mask) == prefix) atomicAdd(&h[(x >> sh) & (nbins - 1)], 1);
              if (pass == 2) above += (x >> 8) > (prefix >> 8);
            }
          }
        }
      }
      __syncthreads();
      if (pass == 2) {  // fold the per-wave histograms into hist[SEL_WAVES * 256 ...]
        if (tid < 256) {
          int t = 0;
          for (int w = 0; w < SEL_WAVES; ++w) t += hist[w * 256 + tid];
          hist[SEL_WAVES * 256 + tid] = t;
        }
        __syncthreads();
      }
      find_bin(pass == 2 ? hist + SEL_WAVES * 256 : hist, nbins, remain, scan, &sv[0], &sv[1]);
      prefix |= (uint32_t)sv[0] << sh;
      mask |= (uint32_t)(nbins - 1) << sh;
      remain = sv[1];
    }
    thr = prefix;
    need_eq = remain;
    // Per-wave counts: above the 24-bit prefix, plus the wave's own last-pass bins.
    const int bin = (int)(thr & 0xffu);
    int gt = above;
    for (int b = lane; b < 256; b += 64) gt += b > bin ? hist[wave * 256 + b] : 0;
    gt = wave_sum_int(gt);
    if (lane == 0) {
      sGt[wave] = gt;
      sEq[wave] = hist[wave * 256 + bin];
    }
    __syncthreads();
  }

  if (tid == 0) {
    int eq_before = 0, pos = 0;
    for (int w = 0; w < SEL_WAVES; ++w) {
      const int take = max(0, min(sEq[w], need_eq - eq_before));
      eq_before += sEq[w];
      sPos[w] = pos;
      sTake[w] = take;
      pos += sGt[w] + take;
    }
  }
  __syncthreads();

  // Ordered write: ascending key index = (wave, step, lane, element).
  const int take_eq = sTake[wave];
  const int quota = sGt[wave] + take_eq;
  int pos = sPos[wave], written = 0, eq_seen = 0;
  for (int j0 = s0; j0 < s1 && written < quota; j0 += 256 * SEL_U) {
    u32x4 v[SEL_U];
#pragma unroll
    for (int u = 0; u < SEL_U; ++u) v[u] = load_scores4(sc, j0 + u * 256 + lane * 4, s1, vec);
#pragma unroll
    for (int u = 0; u < SEL_U; ++u) {
      const int jb = j0 + u * 256 + lane * 4;
      int eqm = 0, neq = 0;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const bool is_eq = jb + e < s1 && v[u][e] == thr;
        eqm |= (int)is_eq << e;
        neq += is_eq;
      }
      int eq_tot;
      const int eq_pre = eq_seen + wave_prefix3(neq, &eq_tot);
      int tkm = 0, ntk = 0, r = 0;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const bool is_eq = (eqm >> e) & 1;
        const bool take = (jb + e < s1 && v[u][e] > thr) || (is_eq && eq_pre + r < take_eq);
        r += is_eq;
        tkm |= (int)take << e;
        ntk += take;
      }
      int tk_tot;
      int p = pos + written + wave_prefix3(ntk, &tk_tot);
#pragma unroll
      for (int e = 0; e < 4; ++e)
        if ((tkm >> e) & 1) out[p++] = jb + e;
      written += tk_tot;
      eq_seen += eq_tot;
    }
  }
}

template <bool F32>
void launch_hash_t(const attn_impl::SocketHashArgs& a, dim3 grid, hipStream_t stream) {
  if (a.E == 128) {
    if (a.bits <= 4)
      hipLaunchKernelGGL((socket_hash_kernel<128, 4, F32>), grid, dim3(256), HASH_LDS, stream, a);
    else
      hipLaunchKernelGGL((socket_hash_kernel<128, 8, F32>), grid, dim3(256), HASH_LDS, stream, a);
  } else {
    if (a.bits <= 4)
      hipLaunchKernelGGL((socket_hash_kernel<64, 4, F32>), grid, dim3(256), HASH_LDS, stream, a);
    else
      hipLaunchKernelGGL((socket_hash_kernel<64, 8, F32>), grid, dim3(256), HASH_LDS, stream, a);
  }
}

template <bool F32>
void launch_prob_t(const attn_impl::SocketSelectArgs& a, hipStream_t stream) {
  if (a.E == 128)
    hipLaunchKernelGGL((socket_prob_kernel<128, F32>), dim3((unsigned)(a.N * a.Hq)), dim3(256), 0, stream, a);
  else
    hipLaunchKernelGGL((socket_prob_kernel<64, F32>), dim3((unsigned)(a.N * a.Hq)), dim3(256), 0, stream, a);
}

}  // namespace

namespace attn_impl {

hipError_t launch_socket_hash(const SocketHashArgs& a, hipStream_t stream) {
  const long long keys = (long long)a.N * a.Hkv * a.S;
  if (keys == 0) return hipSuccess;
  const dim3 grid((unsigned)((keys + 255) / 256));
  if (a.f32)
    launch_hash_t<true>(a, grid, stream);
  else
    launch_hash_t<false>(a, grid, stream);
  return hipGetLastError();
}

hipError_t launch_socket_select(const SocketSelectArgs& a, hipStream_t stream) {
  if (a.f32)
    launch_prob_t<true>(a, stream);
  else
    launch_prob_t<false>(a, stream);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int G = a.Hq / a.Hkv;
  const size_t lds = socket_lds_bytes(G, a.tables, a.bits);
  const bool fast = (a.tables % (a.bits <= 4 ? 32 : 16)) == 0 && a.tables <= 64 &&
                    (reinterpret_cast<uintptr_t>(a.buckets) & 15) == 0;
  if (fast && (G == 1 || G == 2 || G == 4 || G == 8 || G == 16)) {
    e = G == 1 ? launch_score_fast<1>(a, lds, stream)
      : G == 2 ? launch_score_fast<2>(a, lds, stream)
      : G == 4 ? launch_score_fast<4>(a, lds, stream)
      : G == 8 ? launch_score_fast<8>(a, lds, stream)
               : launch_score_fast<16>(a, lds, stream);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(socket_select_kernel, dim3((unsigned)(a.N * a.Hq)), dim3(SEL_T), 0, stream, a);
    return hipGetLastError();
  }
  const dim3 grid((unsigned)((a.S + 256 * SCORE_KPT - 1) / (256 * SCORE_KPT)), (unsigned)(a.N * a.Hkv));
  if (G % 4 == 0)
    hipLaunchKernelGGL(socket_score_kernel<4>, grid, dim3(256), lds, stream, a);
  else if (G % 2 == 0)
    hipLaunchKernelGGL(socket_score_kernel<2>, grid, dim3(256), lds, stream, a);
  else
    hipLaunchKernelGGL(socket_score_kernel<1>, grid, dim3(256), lds, stream, a);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(socket_select_kernel, dim3((unsigned)(a.N * a.Hq)), dim3(SEL_T), 0, stream, a);
  return hipGetLastError();
}

size_t socket_lds_bytes(int G, int tables, int bits) { return (size_t)G * tables * (1u << bits) * sizeof(float); }

}  // namespace attn_impl
