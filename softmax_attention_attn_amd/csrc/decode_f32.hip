// decode_f32.hip -- split-K decode for float32 inputs on gfx950.
//
// The same split-K scheme and partial format as the bf16 decode
// (decode_bf16.hip): workgroup (split, kv head x query group, batch) streams
// the keys of its split once for up to 16 query heads of the GQA group and
// writes, per query head, the running max (log2 units), the running sum and
// the unnormalised output; decode_f32_combine merges the splits with
// log-sum-exp weights and adds the sink logit ("Attention Sink" section 4.2).
// The arithmetic is fp32 throughout (no operand is rounded).  With one or two
// query heads per kv head (and in indexed mode) the products run on the vector
// ALUs: a key row is spread over R = E/4 lanes, 16 bytes each; every lane
// forms the partial dot products of its 4 dims with the group's query heads
// and a butterfly over the R lanes (DPP row operations, then
// v_permlane16_swap at E = 128) completes them.  Each R-lane row group keeps
// its own online-softmax state (running max and sum, 4 output dims per query
// head; "SDPA란 무엇인가?" section 2) over the keys it takes, and the row
// groups of the 4 waves are merged through LDS at the end.  With more heads
// that per-head work would bound the kernel, so the products run on
// v_mfma_f32_16x16x4_f32 instead (decode_split_f32_mfma_kernel).  Decode is
// bound by the K/V bytes (SOCKET summary, problem statement), which are read
// once, with the non-temporal hint.
#include "device_common.h"
#include "kernels.h"

using namespace attn_dev;

namespace {

constexpr int NT = 256;  // threads per workgroup
constexpr int NWAVE = 4;

struct DecodeF32Params {
  const float* q;
  const float* k;
  const float* v;
  float* part_o;
  float* part_ml;
  int N, Hq, Hkv, kv_rows, n_reg;
  int first_real;  // keys n_reg .. n_reg+first_real-1 are outside the window
  int nkeys;       // n_reg + visible real keys
  int chunk;       // keys per split
  int num_splits;
  int qgroups;     // ceil(G / 16)
  float c_logit, c_bias;
  // Indexed mode: every query head has its own list of nkeys key rows at
  // key_index[(n*Hq + h)*nkeys ..]; one query head per workgroup.
  const int* key_index;
};

constexpr int kIdxMax = attn_impl::kDecodeIndexMax;  // indexed mode: longest key list of one split

// Sum over the R lanes of a row group (R = 16: one DPP row; R = 32: two rows).
template <int R>
__device__ __forceinline__ float row_group_sum(float v) {
  v = group_sum<16>(v);
  if (R == 32) v = pair16_sum(v);
  return v;
}

// NS: query slots per workgroup (a power of two, at least the group size when
// G <= 16, else 16 per query group; 1 in indexed mode).  PF: key steps whose
// loads are in flight.  IDX: indexed mode.
template <int E, bool RBF, int NS, int PF, bool IDX>
__global__ __launch_bounds__(NT, 2) void decode_split_f32_kernel(DecodeF32Params p) {
  static_assert(!IDX || NS == 1, "indexed mode takes one query head per workgroup");
  constexpr int R = E / 4;         // lanes per key row
  constexpr int RG = 64 / R;       // row groups per wave
  constexpr int KPS = NWAVE * RG;  // keys per workgroup step
  __shared__ float sM[NWAVE * RG][NS];
  __shared__ float sL[NWAVE * RG][NS];
  __shared__ __attribute__((aligned(16))) float sO[NWAVE * RG][NS][E];
  __shared__ int sIdx[IDX ? kIdxMax : 1];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int rg = lane / R, rl = lane % R;
  const int grp = wave * RG + rg;  // this lane's row group in the workgroup
  const int split = blockIdx.x;
  const int n = blockIdx.z;
  const int G = p.Hq / p.Hkv;
  // The workgroup's query heads are hbase .. hbase + nslots - 1.
  const int kvh = IDX ? (int)blockIdx.y / G : (int)blockIdx.y / p.qgroups;
  const int hbase = IDX ? (int)blockIdx.y : kvh * G + ((int)blockIdx.y % p.qgroups) * 16;
  const int nslots = IDX ? 1 : min(NS, kvh * G + G - hbase);

  // The query heads' 4 dims of this lane (zeros for slots past the group).
  f32x4 qv[NS];
#pragma unroll
  for (int s = 0; s < NS; ++s) {
    const int h = hbase + min(s, nslots - 1);
    const f32x4 x = *reinterpret_cast<const f32x4*>(p.q + ((size_t)n * p.Hq + h) * E + 4 * rl);
    qv[s] = s < nslots ? x : f32x4{0.f, 0.f, 0.f, 0.f};
  }

  const size_t kvoff = ((size_t)n * p.Hkv + kvh) * (size_t)p.kv_rows * E;
  const float* kbase = p.k + kvoff;
  const float* vbase = p.v + kvoff;
  const int v0 = split * p.chunk;
  const int v1 = min(v0 + p.chunk, p.nkeys);
  const int steps = v1 > v0 ? (v1 - v0 + KPS - 1) / KPS : 0;
  if (IDX) {  // the split's key rows, read once (chunk <= kIdxMax)
    const int* kidx = p.key_index + ((size_t)n * p.Hq + hbase) * p.nkeys;
    for (int i = tid; i < v1 - v0; i += NT) sIdx[i] = kidx[v0 + i];
    __syncthreads();
  }
  // Key index -> key row: the split's list in indexed mode; else registers
  // first, then the visible real keys.
  auto key_row = [&](int vidx) {
    if (IDX) return sIdx[vidx - v0];
    return vidx < p.n_reg ? vidx : vidx + p.first_real;
  };

  float m[NS], l[NS];
  f32x4 acc[NS];
#pragma unroll
  for (int s = 0; s < NS; ++s) {
    m[s] = kNegInf;
    l[s] = 0.f;
    acc[s] = f32x4{0.f, 0.f, 0.f, 0.f};
  }

  // Step st: this row group's key is v0 + st*KPS + grp; past v1 it reads row
  // v0 (every lane stays in bounds) and is masked.
  auto load = [&](int st, f32x4& kr, f32x4& vr) {
    const int vk = v0 + st * KPS + grp;
    const size_t row = (size_t)key_row(vk < v1 ? vk : v0);
    kr = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(kbase + row * E + 4 * rl));
    vr = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(vbase + row * E + 4 * rl));
  };
  auto compute = [&](int st, const f32x4& kr, const f32x4& vr) {
    const bool live = v0 + st * KPS + grp < v1;
    float nk = 0.f;
    if (RBF) nk = row_group_sum<R>(kr[0] * kr[0] + kr[1] * kr[1] + kr[2] * kr[2] + kr[3] * kr[3]);
#pragma unroll
    for (int s = 0; s < NS; ++s) {
      float d = qv[s][0] * kr[0];
      d = __builtin_fmaf(qv[s][1], kr[1], d);
      d = __builtin_fmaf(qv[s][2], kr[2], d);
      d = __builtin_fmaf(qv[s][3], kr[3], d);
      d = row_group_sum<R>(d);
      float x = d * p.c_logit;
      if (RBF) x = __builtin_fmaf(p.c_bias, nk, x);
      if (!live) x = kNegInf;
      const float m_new = fmaxf(m[s], x);
      const float m_use = (m_new == kNegInf) ? 0.f : m_new;
      const float alpha = exp2f(m[s] - m_use);
      const float w = exp2f(x - m_use);
      m[s] = m_new;
      l[s] = __builtin_fmaf(l[s], alpha, w);
#pragma unroll
      for (int e = 0; e < 4; ++e) acc[s][e] = __builtin_fmaf(acc[s][e], alpha, w * vr[e]);
    }
  };

  // A ring of PF steps in flight: once step st is computed, its registers take
  // the request for step st + PF (unconditional requests: a step past the end
  // reads row v0, masked).  The ring index is a compile-time constant.
  if (steps > 0) {
    f32x4 kb[PF], vb[PF];
#pragma unroll
    for (int i = 0; i < PF; ++i) load(i, kb[i], vb[i]);
    for (int st = 0; st < steps; st += PF) {
#pragma unroll
      for (int i = 0; i < PF; ++i) {
        if (st + i < steps) {
          compute(st + i, kb[i], vb[i]);
          load(st + i + PF, kb[i], vb[i]);
        }
      }
    }
  }

  // Merge the row groups: max, sum and output dims of every (row group, slot).
#pragma unroll
  for (int s = 0; s < NS; ++s) {
    if (rl == 0) {
      sM[grp][s] = m[s];
      sL[grp][s] = l[s];
    }
    *reinterpret_cast<f32x4*>(&sO[grp][s][4 * rl]) = acc[s];
  }
  __syncthreads();
  const size_t part_base = ((size_t)n * p.Hq + hbase) * p.num_splits + split;
  for (int idx = tid; idx < nslots * E; idx += NT) {
    const int sl = idx / E, e = idx % E;
    float M = kNegInf;
#pragma unroll
    for (int r = 0; r < NWAVE * RG; ++r) M = fmaxf(M, sM[r][sl]);
    const float Mu = (M == kNegInf) ? 0.f : M;
    float o = 0.f;
#pragma unroll
    for (int r = 0; r < NWAVE * RG; ++r) o += exp2f(sM[r][sl] - Mu) * sO[r][sl][e];
    const size_t pi = part_base + (size_t)sl * p.num_splits;
    p.part_o[pi * E + e] = o;
    if (e == 0) {
      float lt = 0.f;
#pragma unroll
      for (int r = 0; r < NWAVE * RG; ++r) lt += exp2f(sM[r][sl] - Mu) * sL[r][sl];
      p.part_ml[pi * 2 + 0] = M;
      p.part_ml[pi * 2 + 1] = lt;
    }
  }
}

// GQA groups of more than two query heads: the same split, partials and merge
// with the products on v_mfma_f32_16x16x4_f32 (fp32 operands, fp32
// accumulation), so the per-head cross-lane sums of the kernel above go away.
// A wave step is 16 keys x 16 query slots (the group's heads, padded):
//   S^T = K Q^T: E/4 MFMAs; lane (l16, g) holds, for every 16-dim chunk c of a
//     row, dims 16c + 4g .. +3 of key l16 (A) and of query slot l16 (B), so one
//     load takes 64 contiguous bytes of each of 16 key rows;
//   O^T += V^T P^T: 4 x E/16 MFMAs; lane (l16, g) holds dims 64u + 4 l16 .. +3
//     (u < E/64) of keys 4g .. 4g+3 (A: 256 contiguous bytes of each of 4 rows
//     per load) and the weights of those keys for slot l16 (B: its own scores).
// Accumulator element r of the scores is key 4g + r for slot l16; element r of
// output block b = 4u + i is dim 64u + 4(4g + r) + i of slot l16.  The 4 waves take
// every 4th step, step st + 4 requested while step st is computed.
template <int E, bool RBF>
__global__ __launch_bounds__(NT, 2) void decode_split_f32_mfma_kernel(DecodeF32Params p) {
  constexpr int QC = E / 16;  // 16-dim chunks of a row
  constexpr int VB = E / 16;  // value dims per lane per key, and output blocks
  constexpr int KST = 16;     // keys per wave step
  __shared__ float sM[NWAVE][16];
  __shared__ float sL[NWAVE][64];
  __shared__ __attribute__((aligned(16))) float sO[NWAVE][16][E];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l16 = lane & 15, g = lane >> 4;
  const int split = blockIdx.x;
  const int n = blockIdx.z;
  const int G = p.Hq / p.Hkv;
  const int kvh = blockIdx.y / p.qgroups;
  const int qg = blockIdx.y % p.qgroups;
  const int hbase = kvh * G + qg * 16;
  const int nslots = min(16, G - qg * 16);
  const bool qvalid = l16 < nslots;

  f32x4 qf[QC];
  {
    const float* qrow = p.q + ((size_t)n * p.Hq + hbase + (qvalid ? l16 : 0)) * E;
#pragma unroll
    for (int c = 0; c < QC; ++c) {
      const f32x4 x = *reinterpret_cast<const f32x4*>(qrow + 16 * c + 4 * g);
      qf[c] = qvalid ? x : f32x4{0.f, 0.f, 0.f, 0.f};
    }
  }

  const size_t kvoff = ((size_t)n * p.Hkv + kvh) * (size_t)p.kv_rows * E;
  const float* kbase = p.k + kvoff;
  const float* vbase = p.v + kvoff;
  const int v0 = split * p.chunk;
  const int v1 = min(v0 + p.chunk, p.nkeys);
  const int steps = v1 > v0 ? (v1 - v0 + KST - 1) / KST : 0;
  auto key_row = [&](int vidx) { return vidx < p.n_reg ? vidx : vidx + p.first_real; };

  float m = kNegInf, lsum = 0.f;
  f32x4 acc[VB];
#pragma unroll
  for (int b = 0; b < VB; ++b) acc[b] = f32x4{0.f, 0.f, 0.f, 0.f};

  // Keys past v1 read row v0 (in bounds) and are masked.
  auto load = [&](int st, f32x4 (&kr)[QC], f32x4 (&vr)[4][VB / 4]) {
    const int vb = v0 + st * KST;
    {
      const int vk = vb + l16;
      const float* row = kbase + (size_t)key_row(vk < v1 ? vk : v0) * E;
#pragma unroll
      for (int c = 0; c < QC; ++c)
        kr[c] = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(row + 16 * c + 4 * g));
    }
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int vk = vb + 4 * g + r;
      const float* row = vbase + (size_t)key_row(vk < v1 ? vk : v0) * E + 4 * l16;
#pragma unroll
      for (int u = 0; u < VB / 4; ++u) vr[r][u] = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(row + 64 * u));
    }
  };

  auto compute = [&](int st, const f32x4 (&kr)[QC], const f32x4 (&vr)[4][VB / 4]) {
    const int vb = v0 + st * KST;
    f32x4 sc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int c = 0; c < QC; ++c)
#pragma unroll
      for (int i = 0; i < 4; ++i) sc = __builtin_amdgcn_mfma_f32_16x16x4f32(kr[c][i], qf[c][i], sc, 0, 0, 0);
    float nk = 0.f;
    if (RBF) {  // |k|^2 of key l16 (its four quarters sit in lanes l16 + 16g), then of keys 4g + r
#pragma unroll
      for (int c = 0; c < QC; ++c)
#pragma unroll
        for (int i = 0; i < 4; ++i) nk = __builtin_fmaf(kr[c][i], kr[c][i], nk);
      nk = pair32_sum(pair16_sum(nk));
    }
    float x[4];
    float mx = kNegInf;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      float xv = sc[r] * p.c_logit;
      if (RBF) xv = __builtin_fmaf(p.c_bias, __shfl(nk, 4 * g + r, 64), xv);
      if (vb + 4 * g + r >= v1) xv = kNegInf;
      x[r] = xv;
      mx = fmaxf(mx, xv);
    }
    mx = pair32_max(pair16_max(mx));  // over the step's 16 keys, for slot l16
    const float m_new = fmaxf(m, mx);
    const float m_use = (m_new == kNegInf) ? 0.f : m_new;
    if (__any(m_new > m)) {  // the running max moved for some slot: rescale
      const float alpha = exp2f(m - m_use);
      lsum *= alpha;
#pragma unroll
      for (int b = 0; b < VB; ++b) acc[b] *= alpha;
    }
    m = m_new;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      x[r] = exp2f(x[r] - m_use);
      lsum += x[r];
    }
#pragma unroll
    for (int r = 0; r < 4; ++r)
#pragma unroll
      for (int b = 0; b < VB; ++b)
        acc[b] = __builtin_amdgcn_mfma_f32_16x16x4f32(vr[r][b >> 2][b & 3], x[r], acc[b], 0, 0, 0);
  };

  if (steps > 0) {
    f32x4 kA[QC], vA[4][VB / 4];
    int st = wave;
    load(st, kA, vA);
    for (; st < steps; st += NWAVE) {
      f32x4 kB[QC], vB[4][VB / 4];
      load(st + NWAVE, kB, vB);
      compute(st, kA, vA);
#pragma unroll
      for (int c = 0; c < QC; ++c) kA[c] = kB[c];
#pragma unroll
      for (int r = 0; r < 4; ++r)
#pragma unroll
        for (int u = 0; u < VB / 4; ++u) vA[r][u] = vB[r][u];
    }
  }

  // Merge the 4 waves: running max per slot, sums per lane, outputs per (slot, dim).
  if (g == 0) sM[wave][l16] = m;
  sL[wave][lane] = lsum;
#pragma unroll
  for (int b = 0; b < VB; ++b)
#pragma unroll
    for (int r = 0; r < 4; ++r) sO[wave][l16][64 * (b >> 2) + 4 * (4 * g + r) + (b & 3)] = acc[b][r];
  __syncthreads();
  const size_t part_base = ((size_t)n * p.Hq + hbase) * p.num_splits + split;
  for (int idx = tid; idx < nslots * E; idx += NT) {
    const int sl = idx / E, e = idx % E;
    float M = kNegInf;
#pragma unroll
    for (int w = 0; w < NWAVE; ++w) M = fmaxf(M, sM[w][sl]);
    const float Mu = (M == kNegInf) ? 0.f : M;
    float o = 0.f;
#pragma unroll
    for (int w = 0; w < NWAVE; ++w) o += exp2f(sM[w][sl] - Mu) * sO[w][sl][e];
    const size_t pi = part_base + (size_t)sl * p.num_splits;
    p.part_o[pi * E + e] = o;
    if (e == 0) {
      float lt = 0.f;
#pragma unroll
      for (int w = 0; w < NWAVE; ++w) {
        const float lw = (sL[w][sl] + sL[w][sl + 16]) + (sL[w][sl + 32] + sL[w][sl + 48]);
        lt += exp2f(sM[w][sl] - Mu) * lw;
      }
      p.part_ml[pi * 2 + 0] = M;
      p.part_ml[pi * 2 + 1] = lt;
    }
  }
}

struct CombineF32Params {
  const float* q;
  const float* part_o;
  const float* part_ml;
  const float* sink;
  float* o;
  float* lse;
  int Hq, num_splits, rbf;
  float gamma;
};

template <int E>
__device__ __forceinline__ float block_reduce(float v, float* red, bool is_max) {
  const int e = threadIdx.x;
  red[e] = v;
  __syncthreads();
#pragma unroll
  for (int s = E / 2; s > 0; s >>= 1) {
    if (e < s) red[e] = is_max ? fmaxf(red[e], red[e + s]) : red[e] + red[e + s];
    __syncthreads();
  }
  const float r = red[0];
  __syncthreads();
  return r;
}

// One workgroup per (batch, query head), one thread per output dim: the split
// maxima are reduced first, then the weighted partial outputs summed in chunks
// of splits whose weights sit in LDS (as in the bf16 combine).
constexpr int kCombineChunk = 1024;

template <int E>
__global__ __launch_bounds__(E) void decode_f32_combine(CombineF32Params p) {
  __shared__ float sRed[E];
  __shared__ float sW[kCombineChunk];
  const int nh = blockIdx.x;
  const int h = nh % p.Hq;
  const int e = threadIdx.x;

  float qn2 = 0.f;
  if (p.rbf) {
    const float qe = p.q[(size_t)nh * E + e];
    qn2 = block_reduce<E>(qe * qe, sRed, false);
  }
  const size_t base = (size_t)nh * p.num_splits;
  float sink2 = kNegInf;
  if (p.sink) sink2 = (p.sink[h] + (p.rbf ? p.gamma * qn2 : 0.f)) * kLog2e;
  float mloc = kNegInf;
  for (int s = e; s < p.num_splits; s += E) mloc = fmaxf(mloc, p.part_ml[(base + s) * 2]);
  const float M = fmaxf(sink2, block_reduce<E>(mloc, sRed, true));
  const float Mu = (M == kNegInf) ? 0.f : M;

  float lloc = 0.f, acc = 0.f;
  for (int c0 = 0; c0 < p.num_splits; c0 += kCombineChunk) {
    const int cn = min(kCombineChunk, p.num_splits - c0);
    for (int s = e; s < cn; s += E) {
      const float w = exp2f(p.part_ml[(base + c0 + s) * 2] - Mu);
      sW[s] = w;
      lloc += w * p.part_ml[(base + c0 + s) * 2 + 1];
    }
    __syncthreads();
    const float* po = p.part_o + (base + c0) * E + e;
    for (int s = 0; s < cn; ++s) acc += sW[s] * po[(size_t)s * E];
    __syncthreads();
  }
  float l = block_reduce<E>(lloc, sRed, false);
  if (p.sink) l += exp2f(sink2 - Mu);
  p.o[(size_t)nh * E + e] = l > 0.f ? acc / l : 0.f;
  if (e == 0) {
    float lv = kNegInf;
    if (l > 0.f) {
      lv = (M + log2f(l)) * kLn2;
      if (p.rbf) lv -= p.gamma * qn2;
    }
    p.lse[nh] = lv;
  }
}

template <int E, bool RBF, int NS, bool IDX = false>
hipError_t launch_t(const DecodeF32Params& p, const CombineF32Params& c, int N, hipStream_t stream) {
  dim3 grid((unsigned)p.num_splits, (unsigned)(IDX ? p.Hq : p.Hkv * p.qgroups), (unsigned)N);
  constexpr int PF = NS >= 16 ? 2 : 4;
  hipLaunchKernelGGL((decode_split_f32_kernel<E, RBF, NS, PF, IDX>), grid, dim3(NT), 0, stream, p);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  hipLaunchKernelGGL((decode_f32_combine<E>), dim3((unsigned)(N * p.Hq)), dim3(E), 0, stream, c);
  return hipGetLastError();
}

template <int E, bool RBF>
hipError_t launch_mfma(const DecodeF32Params& p, const CombineF32Params& c, int N, hipStream_t stream) {
  dim3 grid((unsigned)p.num_splits, (unsigned)(p.Hkv * p.qgroups), (unsigned)N);
  hipLaunchKernelGGL((decode_split_f32_mfma_kernel<E, RBF>), grid, dim3(NT), 0, stream, p);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  hipLaunchKernelGGL((decode_f32_combine<E>), dim3((unsigned)(N * p.Hq)), dim3(E), 0, stream, c);
  return hipGetLastError();
}

// One or two heads per kv head: the vector-ALU kernel streams at the HBM rate;
// more: the MFMA kernel (the vector one becomes bound by its per-head work).
template <int E, bool RBF>
hipError_t launch_ns(const DecodeF32Params& p, const CombineF32Params& c, int N, int G, hipStream_t stream) {
  if (p.key_index) return launch_t<E, RBF, 1, true>(p, c, N, stream);
  if (G <= 1) return launch_t<E, RBF, 1>(p, c, N, stream);
  if (G <= 2) return launch_t<E, RBF, 2>(p, c, N, stream);
  return launch_mfma<E, RBF>(p, c, N, stream);
}

}  // namespace

namespace attn_impl {

hipError_t launch_decode_f32(const DecodeArgs& a, hipStream_t stream) {
  const FwdArgs& f = a.f;
  const DecodeKeys dk = decode_keys(f.S, f.n_reg, f.causal, f.window);
  DecodeF32Params p;
  p.q = static_cast<const float*>(f.q);
  p.k = static_cast<const float*>(f.k);
  p.v = static_cast<const float*>(f.v);
  p.part_o = a.part_o;
  p.part_ml = a.part_ml;
  p.N = f.N;
  p.Hq = f.Hq;
  p.Hkv = f.Hkv;
  p.kv_rows = f.kv_rows;
  p.n_reg = f.n_reg;
  p.first_real = dk.first_real;
  p.nkeys = a.key_index ? a.index_count : dk.count;
  p.key_index = a.key_index;
  p.num_splits = a.num_splits;
  p.chunk = (p.nkeys + a.num_splits - 1) / a.num_splits;
  if (p.chunk == 0) p.chunk = 1;
  if (p.key_index && p.chunk > kIdxMax) return hipErrorInvalidValue;
  const int G = f.Hq / f.Hkv;
  p.qgroups = (G + 15) / 16;
  if (f.rbf) {
    p.c_logit = 2.f * f.gamma * 1.4426950408889634f;
    p.c_bias = -f.gamma * 1.4426950408889634f;
  } else {
    p.c_logit = f.scale * 1.4426950408889634f;
    p.c_bias = 0.f;
  }
  CombineF32Params c;
  c.q = p.q;
  c.part_o = a.part_o;
  c.part_ml = a.part_ml;
  c.sink = f.sink;
  c.o = static_cast<float*>(f.o);
  c.lse = f.lse;
  c.Hq = f.Hq;
  c.num_splits = a.num_splits;
  c.rbf = f.rbf;
  c.gamma = f.gamma;
  if (f.E == 128)
    return f.rbf ? launch_ns<128, true>(p, c, f.N, G, stream) : launch_ns<128, false>(p, c, f.N, G, stream);
  return f.rbf ? launch_ns<64, true>(p, c, f.N, G, stream) : launch_ns<64, false>(p, c, f.N, G, stream);
}

}  // namespace attn_impl
