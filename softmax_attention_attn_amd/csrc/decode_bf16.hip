// decode_bf16.hip -- split-K ("flash-decode") attention for one query token per
// sequence against a long bf16 key/value cache, on gfx950.
//
// Decode reads every cached key and value once and does little arithmetic per
// byte, so it is bound by HBM bandwidth (SOCKET summary, problem statement:
// decoding is a memory bottleneck).  The keys are split into `num_splits`
// ranges; workgroup (split, kv head, batch) streams its range once for all
// the query heads that share this kv head (GQA, "SDPA란 무엇인가?" section 5),
// so K/V bytes are read exactly once in total.  Each workgroup writes a
// partial (running max in log2 units, running sum, unnormalised output) per
// query head; decode_combine merges the partials with log-sum-exp weights and
// adds the sink logit ("Attention Sink" section 4.2) once.
//
// Inside a workgroup each of the 4 waves takes every 4th step of 32 keys.  A
// step is two v_mfma_f32_16x16x32_bf16 products S^T = K * Q^T (16 keys x 16
// query slots; only the group's G heads are real) followed by O^T += V^T * P^T.
// K rows are loaded straight into the MFMA A operand (64 contiguous bytes per
// row per load).  K and V are read once, so their loads carry the
// non-temporal hint.  V is loaded as whole 256-byte rows -- lane (m, g) takes dims
// 8m..8m+7 of 8 keys -- and transposed in registers, so the 8 PV products of a
// step each produce the 16 dims {8m + j}.
//
// Indexed mode (SOCKET sparse decode): every query head attends to its own
// list of key rows, so a workgroup serves one query head (MFMA column 0) and
// first copies its split's part of the list (at most kDecodeIndexMax rows)
// into LDS, where the row addresses of every step are then read without a
// global-memory round trip.
#include <mutex>

#include "device_common.h"
#include "kernels.h"

using namespace attn_dev;

namespace {

// Scratch for attn_decode_noalloc: the split partials of one call live in this
// file-scope device array instead of a caller workspace.  Each GPU the library
// runs on holds its own copy (at its own address) until the process ends; the
// host reaches it only through the address hipGetSymbolAddress returns for the
// current device, never through the array's name.
static __device__ __align__(256) unsigned char scratch[attn_impl::kDecodeScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mutex;
void* g_scratch_ptr[kMaxDevices] = {};

constexpr int NT = 256;   // threads per workgroup
constexpr int NWAVE = 4;
constexpr int KSTEP = 32; // keys per wave step
constexpr int kIdxMax = attn_impl::kDecodeIndexMax;  // indexed mode: longest key list of one split

struct DecodeParams {
  const uint16_t* q;
  const uint16_t* k;
  const uint16_t* v;
  float* part_o;
  float* part_ml;
  int N, Hq, Hkv, kv_rows, n_reg;
  int first_real;  // keys n_reg .. n_reg+first_real-1 are outside the window
  int nkeys;       // n_reg + visible real keys (indexed: keys per query head)
  int chunk;       // keys per split (multiple of KSTEP)
  int num_splits;
  int qgroups;     // ceil(G / 16)
  float c_logit, c_bias;
  // Indexed mode (key_index != nullptr): every query head has its own list of
  // nkeys key rows at key_index[(n*Hq + h)*nkeys ..]; one query head per
  // workgroup (grid y = Hq), its key/value head h / (Hq/Hkv).
  const int* key_index;
};

// Virtual key index -> key row: registers first, then the visible real keys;
// in indexed mode the split's list, staged in LDS from key v0 on.
__device__ __forceinline__ int key_row(int vidx, const DecodeParams& p, const int* sidx, int v0) {
  if (sidx) return sidx[vidx - v0];
  return vidx < p.n_reg ? vidx : vidx + p.first_real;
}

template <int E, bool RBF>
__global__ __launch_bounds__(NT, 2) void decode_split_kernel(DecodeParams p) {
  constexpr int QS = E / 32;   // K-dim steps of the 16x16x32 product
  constexpr int ECH = E / 8;   // 16-byte chunks of a row (V^T rows m < ECH are real)
  constexpr int OSTR = E + 4;  // LDS row stride of the per-wave output

  __shared__ float sM[NWAVE][16];
  __shared__ float sL[NWAVE][64];
  // The per-wave outputs of the epilogue share LDS with the indexed mode's key list.
  constexpr int SO_FLOATS = NWAVE * 16 * OSTR;
  static_assert(SO_FLOATS >= kIdxMax, "key list must fit in the output staging area");
  __shared__ __attribute__((aligned(16))) float sOraw[SO_FLOATS];
  float(*sO)[16][OSTR] = reinterpret_cast<float(*)[16][OSTR]>(sOraw);

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform per wave
  const int l16 = lane & 15, g = lane >> 4;
  const int split = blockIdx.x;
  const int n = blockIdx.z;
  const int G = p.Hq / p.Hkv;
  const bool indexed = p.key_index != nullptr;
  int kvh, qg, slot, h;
  bool qvalid;
  if (indexed) {  // one query head per workgroup, in MFMA column 0
    h = blockIdx.y;
    kvh = h / G;
    qg = 0;
    slot = l16;
    qvalid = l16 == 0;
  } else {
    kvh = blockIdx.y / p.qgroups;
    qg = blockIdx.y % p.qgroups;
    slot = qg * 16 + l16;
    qvalid = slot < G;
    h = kvh * G + (qvalid ? slot : 0);
  }
  const int* kidx = indexed ? p.key_index + ((size_t)n * p.Hq + h) * p.nkeys : nullptr;

  // Q^T fragments (B operand): lane (l16, g) holds Q[h][32s + 8g .. +8].
  const uint16_t* qrow = p.q + ((size_t)n * p.Hq + h) * E;
  bf16x8 qf[QS];
#pragma unroll
  for (int s = 0; s < QS; ++s) qf[s] = as_bf16x8(load16_or_zero(qrow + 32 * s + 8 * g, qvalid));

  const size_t kvoff = ((size_t)n * p.Hkv + kvh) * (size_t)p.kv_rows * E;
  const uint16_t* kbase = p.k + kvoff;
  const uint16_t* vbase = p.v + kvoff;

  const int v0 = split * p.chunk;
  const int v1 = min(v0 + p.chunk, p.nkeys);
  const int steps = v1 > v0 ? (v1 - v0 + KSTEP - 1) / KSTEP : 0;
  int* sidx = nullptr;
  if (indexed) {  // the split's key rows, read once (chunk <= kIdxMax)
    sidx = reinterpret_cast<int*>(sOraw);
    for (int i = tid; i < v1 - v0; i += NT) sidx[i] = kidx[v0 + i];
    __syncthreads();
  }

  float m = kNegInf, lsum = 0.f;
  f32x4 acc[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) acc[j] = f32x4{0.f, 0.f, 0.f, 0.f};

  // Key of element i of lane-half g in a step's PV operand:
  // i < 4 -> 4g + i (first 16-key block), i >= 4 -> 16 + 4g + i - 4 (second).
  auto load_step = [&](int st, u32x4 (&kr)[2][QS], u32x4 (&vr)[8]) {
    const int vb = v0 + st * KSTEP;
#pragma unroll
    for (int b = 0; b < 2; ++b) {
      const int vk = vb + 16 * b + l16;
      const bool ok = vk < v1;
      const uint16_t* row = kbase + (size_t)key_row(ok ? vk : v0, p, sidx, v0) * E;
#pragma unroll
      for (int s = 0; s < QS; ++s)
        kr[b][s] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(row + 32 * s + 8 * g));
    }
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int vk = vb + (i < 4 ? 4 * g + i : 16 + 4 * g + (i - 4));
      const bool ok = vk < v1;
      vr[i] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(
          vbase + (size_t)key_row(ok ? vk : v0, p, sidx, v0) * E + 8 * min(l16, ECH - 1)));
    }
  };

  auto compute_step = [&](int st, const u32x4 (&kr)[2][QS], const u32x4 (&vr)[8]) {
    const int vb = v0 + st * KSTEP;
    f32x4 sc[2];
#pragma unroll
    for (int b = 0; b < 2; ++b) {
      sc[b] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int s = 0; s < QS; ++s)
        sc[b] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(kr[b][s]), qf[s], sc[b], 0, 0, 0);
    }
    // Accumulator element r of block b is key vb + 16b + 4g + r for query slot l16.
    float x[2][4];
    float mx = kNegInf;
#pragma unroll
    for (int b = 0; b < 2; ++b) {
      float nk = 0.f;
      if (RBF) {
        // |k|^2 of key vb + 16b + l16, then fetched for keys 4g + r.
#pragma unroll
        for (int s = 0; s < QS; ++s) nk += sumsq8(kr[b][s]);
        nk = pair32_sum(pair16_sum(nk));
      }
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        float xv = sc[b][r] * p.c_logit;
        if (RBF) xv += p.c_bias * __shfl(nk, 4 * g + r, 64);
        if (vb + 16 * b + 4 * g + r >= v1) xv = kNegInf;
        x[b][r] = xv;
        mx = fmaxf(mx, xv);
      }
    }
    mx = pair32_max(pair16_max(mx));
    const float m_new = fmaxf(m, mx);
    const float m_use = (m_new == kNegInf) ? 0.f : m_new;
    const float alpha = fast_exp2(m - m_use);
    m = m_new;
    lsum *= alpha;
#pragma unroll
    for (int j = 0; j < 8; ++j) acc[j] *= alpha;
    float ps = 0.f;
#pragma unroll
    for (int b = 0; b < 2; ++b)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        x[b][r] = fast_exp2(x[b][r] - m_use);
        ps += x[b][r];
      }
    lsum += ps;
    const bf16x8 pf = pack_bf16x8(x[0][0], x[0][1], x[0][2], x[0][3], x[1][0], x[1][1], x[1][2], x[1][3]);
    // V^T operand j: element i = V[key of element i][8*l16 + j].
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int w = j >> 1, sh = (j & 1) * 16;
      u32x4 t;
#pragma unroll
      for (int d = 0; d < 4; ++d) {
        const uint32_t a = (vr[2 * d][w] >> sh) & 0xffffu;
        const uint32_t b = (vr[2 * d + 1][w] >> sh) & 0xffffu;
        t[d] = a | (b << 16);
      }
      acc[j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(t), pf, acc[j], 0, 0, 0);
    }
  };

  // Step st + 4 is requested while step st is computed.  The requests are
  // unconditional (a step past the end reads row v0 for every key, all masked):
  // a conditional one leaves the compiler unable to count the loads in flight,
  // and it then waits for all of them -- the prefetch included -- before each step.
  if (steps > 0) {
    u32x4 kA[2][QS], vA[8];
    int st = wave;
    load_step(st, kA, vA);
    for (; st < steps; st += NWAVE) {
      u32x4 kB[2][QS], vB[8];
      load_step(st + NWAVE, kB, vB);
      compute_step(st, kA, vA);
#pragma unroll
      for (int b = 0; b < 2; ++b)
#pragma unroll
        for (int s = 0; s < QS; ++s) kA[b][s] = kB[b][s];
#pragma unroll
      for (int i = 0; i < 8; ++i) vA[i] = vB[i];
    }
  }

  if (indexed) __syncthreads();  // every wave is done with the key list before sO overwrites it

  // Merge the 4 waves.  Lane (l16, g): acc[j][r] is dim 8(4g + r) + j of slot l16.
  if (g == 0) sM[wave][l16] = m;
  sL[wave][lane] = lsum;
#pragma unroll
  for (int j = 0; j < 8; ++j)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int e = 8 * (4 * g + r) + j;
      if (e < E) sO[wave][l16][e] = acc[j][r];
    }
  __syncthreads();

  const size_t part_base = ((size_t)n * p.Hq + (indexed ? (size_t)h : (size_t)kvh * G)) * p.num_splits + split;
  const int nslots = indexed ? 1 : G;
  for (int idx = tid; idx < 16 * E; idx += NT) {
    const int sl = idx / E, e = idx % E;
    const int gs = qg * 16 + sl;
    if (gs >= nslots) continue;
    float M = kNegInf;
#pragma unroll
    for (int w = 0; w < NWAVE; ++w) M = fmaxf(M, sM[w][sl]);
    const float Mu = (M == kNegInf) ? 0.f : M;
    float o = 0.f;
#pragma unroll
    for (int w = 0; w < NWAVE; ++w) o += fast_exp2(sM[w][sl] - Mu) * sO[w][sl][e];
    const size_t pi = part_base + (size_t)gs * p.num_splits;
    p.part_o[pi * E + e] = o;
    if (e == 0) {
      float l = 0.f;
#pragma unroll
      for (int w = 0; w < NWAVE; ++w) {
        const float lw = sL[w][sl] + sL[w][sl + 16] + sL[w][sl + 32] + sL[w][sl + 48];
        l += fast_exp2(sM[w][sl] - Mu) * lw;
      }
      p.part_ml[pi * 2 + 0] = M;
      p.part_ml[pi * 2 + 1] = l;
    }
  }
}

struct CombineParams {
  const uint16_t* q;
  const float* part_o;
  const float* part_ml;
  const float* sink;
  uint16_t* o;
  float* lse;
  int Hq, num_splits, rbf;
  float gamma;
};

// One workgroup per (batch, query head), one thread per output dim.  The
// partial maxima are reduced first (all splits read at once, strided over the
// threads); then, in chunks of kCombineChunk splits, the split weights
// 2^(m_s - M) go to LDS and every thread sums its output column over the chunk
// with independent loads, so the merge costs a few memory round trips rather
// than one per split.
constexpr int kCombineChunk = 1024;

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

template <int E>
__global__ __launch_bounds__(E) void decode_combine_kernel(CombineParams p) {
  __shared__ float sRed[E];
  __shared__ float sW[kCombineChunk];
  const int nh = blockIdx.x;
  const int h = nh % p.Hq;
  const int e = threadIdx.x;

  float qn2 = 0.f;
  if (p.rbf) {
    const float qe = bf16_lo(p.q[(size_t)nh * E + e]);
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
    const int n = min(kCombineChunk, p.num_splits - c0);
    for (int s = e; s < n; s += E) {
      const float w = exp2f(p.part_ml[(base + c0 + s) * 2] - Mu);
      sW[s] = w;
      lloc += w * p.part_ml[(base + c0 + s) * 2 + 1];
    }
    __syncthreads();
    const float* po = p.part_o + (base + c0) * E + e;
#pragma unroll 8
    for (int s = 0; s < n; ++s) acc += sW[s] * po[(size_t)s * E];
    __syncthreads();
  }
  float l = block_reduce<E>(lloc, sRed, false);
  if (p.sink) l += exp2f(sink2 - Mu);
  const float ov = l > 0.f ? acc / l : 0.f;
  p.o[(size_t)nh * E + e] = __builtin_bit_cast(uint16_t, (__bf16)ov);
  if (e == 0) {
    float lv = kNegInf;
    if (l > 0.f) {
      lv = (M + log2f(l)) * kLn2;
      if (p.rbf) lv -= p.gamma * qn2;
    }
    p.lse[nh] = lv;
  }
}

template <int E, bool RBF>
hipError_t launch_t(const DecodeParams& p, const CombineParams& c, int N, hipStream_t stream) {
  dim3 grid((unsigned)p.num_splits, (unsigned)(p.key_index ? p.Hq : p.Hkv * p.qgroups), (unsigned)N);
  hipLaunchKernelGGL((decode_split_kernel<E, RBF>), grid, dim3(NT), 0, stream, p);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  hipLaunchKernelGGL((decode_combine_kernel<E>), dim3((unsigned)(N * p.Hq)), dim3(E), 0, stream, c);
  return hipGetLastError();
}

}  // namespace

namespace attn_impl {

DecodeKeys decode_keys(int S, int n_reg, int causal, int window) {
  const int S_real = S - n_reg;
  DecodeKeys dk;
  // The single query sits at real position S_real - 1 (bottom-right), so the
  // causal rule admits every real key and the window admits the last `window`.
  dk.first_real = (causal && window > 0) ? (S_real > window ? S_real - window : 0) : 0;
  dk.count = n_reg + (S_real - dk.first_real);
  return dk;
}

hipError_t decode_scratch(float** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mutex);
  if (!g_scratch_ptr[dev]) {
    void* ptr = nullptr;
    e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (!ptr) return hipErrorInvalidSymbol;
    g_scratch_ptr[dev] = ptr;
  }
  *out = static_cast<float*>(g_scratch_ptr[dev]);
  return hipSuccess;
}

hipError_t launch_decode_bf16(const DecodeArgs& a, hipStream_t stream) {
  const FwdArgs& f = a.f;
  const DecodeKeys dk = decode_keys(f.S, f.n_reg, f.causal, f.window);
  DecodeParams p;
  p.q = static_cast<const uint16_t*>(f.q);
  p.k = static_cast<const uint16_t*>(f.k);
  p.v = static_cast<const uint16_t*>(f.v);
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
  const int per = (p.nkeys + a.num_splits - 1) / a.num_splits;
  p.chunk = ((per + KSTEP - 1) / KSTEP) * KSTEP;
  if (p.chunk == 0) p.chunk = KSTEP;
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
  CombineParams c;
  c.q = p.q;
  c.part_o = a.part_o;
  c.part_ml = a.part_ml;
  c.sink = f.sink;
  c.o = static_cast<uint16_t*>(f.o);
  c.lse = f.lse;
  c.Hq = f.Hq;
  c.num_splits = a.num_splits;
  c.rbf = f.rbf;
  c.gamma = f.gamma;
  if (f.E == 128) return f.rbf ? launch_t<128, true>(p, c, f.N, stream) : launch_t<128, false>(p, c, f.N, stream);
  return f.rbf ? launch_t<64, true>(p, c, f.N, stream) : launch_t<64, false>(p, c, f.N, stream);
}

}  // namespace attn_impl
