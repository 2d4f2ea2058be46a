// prefill_f32.hip -- fused tiled attention forward for float32 inputs on gfx950.
//
// Full fp32 arithmetic (no bf16 rounding of P).  A workgroup owns 64 query
// rows, one per lane, and runs W waves over them (4 at E = 128, 8 at E = 64): keys stream through LDS
// in tiles of 32 (staged by all W waves), and wave w takes the keys w, w + W,
// ... of every tile, keeping its own online-softmax state (running max,
// running sum, accumulator: "SDPA란 무엇인가?" section 2).  At the end the W
// partial states of each row are merged through LDS with log-sum-exp weights,
// the split-K combine of the decode path.  Same logit frame, visibility rule,
// sink and LSE conventions as the bf16 kernel: x = c_logit*(q.k) +
// c_bias*|k|^2 in log2 units, with |k|^2 summed over a key row's staged
// pieces (consecutive lanes) on their way to LDS; tile t+1 is fetched into
// registers while tile t is consumed.  Within a wave keys are taken one at a
// time: the running max only moves (and the accumulator is only rescaled) when
// a larger logit arrives.
#include "device_common.h"
#include "kernels.h"

using namespace attn_dev;

namespace {

constexpr int BQ = 64;  // query rows per workgroup (one per lane)
constexpr int BK = 32;  // keys per staged tile
// Waves per workgroup, each taking every W-th key: E = 128 needs ~400 VGPRs
// (one wave per SIMD, 4 waves); E = 64 fits in 256 (two per SIMD, 8 waves).
template <int E>
struct F32Waves {
  static constexpr int W = E == 128 ? 4 : 8;
};

struct PrefillF32Params {
  const float* q;
  const float* k;
  const float* v;
  float* o;
  float* lse;
  const float* sink;
  int N, Hq, Hkv, L, S, n_reg, S_real, off, causal, window;
  float c_logit, c_bias, gamma;
  const int* key_len;     // N valid real-key counts, or nullptr
  const void* ubias;      // user bias (float32 addend or uint8 mask), or nullptr
  int ub_kind;            // 1 = float32, 2 = uint8 mask
  long long ub_sn, ub_sh; // element strides over batch and head (0 = broadcast); rows are S apart
  int num_q_tiles;
};

template <int E, bool RBF>
__global__ __launch_bounds__(BQ * F32Waves<E>::W) __attribute__((amdgpu_waves_per_eu(F32Waves<E>::W / 4,
                                                                                    F32Waves<E>::W / 4)))
void prefill_f32_kernel(PrefillF32Params p) {
  constexpr int W = F32Waves<E>::W;
  __shared__ __attribute__((aligned(16))) float sK[BK * E];
  __shared__ __attribute__((aligned(16))) float sV[BK * E];
  __shared__ float sBias[BK];
  // Partial states of waves 1 .. W-1: per row max, sum and E accumulator values.
  __shared__ float sM[W - 1][BQ], sL[W - 1][BQ];
  __shared__ __attribute__((aligned(16))) float sAcc[W - 1][E][BQ];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int qt = blockIdx.x % p.num_q_tiles;
  const int nh = blockIdx.x / p.num_q_tiles;
  const int h = nh % p.Hq, n = nh / p.Hq;
  const int kh = h / (p.Hq / p.Hkv);
  const int i0 = qt * BQ;
  const int qi = i0 + lane;
  const bool qvalid = qi < p.L;

  float q[E], acc[E];
  const float* qrow = p.q + (((size_t)n * p.Hq + h) * p.L + (qvalid ? qi : 0)) * E;
  float qn2 = 0.f;
#pragma unroll
  for (int e = 0; e < E; ++e) {
    q[e] = qvalid ? qrow[e] : 0.f;
    qn2 = __builtin_fmaf(q[e], q[e], qn2);
    acc[e] = 0.f;
  }
  // The sink seeds wave 0's state only (it enters the denominator once).
  float m = kNegInf, lsum = 0.f;
  if (p.sink && wave == 0) {
    float s0 = p.sink[h];
    if (RBF) s0 += p.gamma * qn2;
    m = s0 * kLog2e;
    lsum = 1.f;
  }

  // Real keys at or past kl are padding of this sequence (no key lengths: none).
  const int kl = p.key_len ? max(0, min(p.S_real, p.key_len[n])) : p.S_real;
  const long long ub_row = (long long)n * p.ub_sn + (long long)h * p.ub_sh + (long long)(qvalid ? qi : 0) * p.S;
  const int i_last = min(i0 + BQ, p.L) - 1;
  const int r_hi = p.causal ? min(kl - 1, i_last + p.off) : kl - 1;
  const int r_lo = p.window > 0 ? max(0, i0 + p.off - p.window + 1) : 0;
  const int n_real_tiles = r_hi >= r_lo ? (r_hi - r_lo + BK) / BK : 0;
  const int n_reg_tiles = (p.n_reg + BK - 1) / BK;
  const int T = n_reg_tiles + n_real_tiles;
  const size_t kvoff = ((size_t)n * p.Hkv + kh) * (size_t)p.S * E;

  // Tile t+1 is fetched into registers while tile t is consumed from LDS.
  // Thread tid stages 16-byte pieces tid, tid + BQ*W, ... of a tile; the E/4
  // pieces of one key row sit in consecutive lanes, where |k|^2 is summed on
  // the way to LDS.
  constexpr int NPT = BK * E / 4 / (BQ * W);
  static_assert(NPT * BQ * W * 4 == BK * E, "tile must split evenly over the threads");
  auto tile_keys = [&](int t, int& j0, int& kc) {
    if (t < n_reg_tiles) {
      j0 = t * BK;
      kc = min(BK, p.n_reg - j0);
    } else {
      j0 = p.n_reg + r_lo + (t - n_reg_tiles) * BK;
      kc = min(BK, p.S - j0);
    }
  };
  f32x4 kr[NPT], vr[NPT];
  auto fetch_tile = [&](int t) {
    int j0, kc;
    tile_keys(t, j0, kc);
#pragma unroll
    for (int i = 0; i < NPT; ++i) {
      const int idx = tid + i * BQ * W;
      const int row = (idx * 4) / E, col = (idx * 4) % E;
      kr[i] = f32x4{0.f, 0.f, 0.f, 0.f};
      vr[i] = f32x4{0.f, 0.f, 0.f, 0.f};
      if (row < kc) {
        kr[i] = *reinterpret_cast<const f32x4*>(p.k + kvoff + (size_t)(j0 + row) * E + col);
        vr[i] = *reinterpret_cast<const f32x4*>(p.v + kvoff + (size_t)(j0 + row) * E + col);
      }
    }
  };
  if (T > 0) fetch_tile(0);

  for (int t = 0; t < T; ++t) {
    int j0, kc;
    tile_keys(t, j0, kc);
    const bool is_reg = t < n_reg_tiles;
    __syncthreads();  // every wave is done with the previous tile
#pragma unroll
    for (int i = 0; i < NPT; ++i) {
      const int idx = tid + i * BQ * W;
      const int row = (idx * 4) / E, col = (idx * 4) % E;
      *reinterpret_cast<f32x4*>(&sK[row * E + col]) = kr[i];
      *reinterpret_cast<f32x4*>(&sV[row * E + col]) = vr[i];
      if (RBF) {
        float ss = kr[i][0] * kr[i][0];
        ss = __builtin_fmaf(kr[i][1], kr[i][1], ss);
        ss = __builtin_fmaf(kr[i][2], kr[i][2], ss);
        ss = __builtin_fmaf(kr[i][3], kr[i][3], ss);
        ss = group_sum<16>(ss);
        if (E / 4 == 32) ss += __shfl_xor(ss, 16, 64);
        if (col == 0) sBias[row] = p.c_bias * ss;
      }
    }
    __syncthreads();
    if (t + 1 < T) fetch_tile(t + 1);

#pragma unroll 1
    for (int kt = wave; kt < BK; kt += W) {
      // q.k as four interleaved partial sums (a quarter of the dependent chain).
      float d4[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int e = 0; e < E; ++e) d4[e & 3] = __builtin_fmaf(q[e], sK[kt * E + e], d4[e & 3]);
      const float d = (d4[0] + d4[1]) + (d4[2] + d4[3]);
      float x = d * p.c_logit;
      if (RBF) x += sBias[kt];
      bool vis;
      if (is_reg) {
        vis = kt < kc;
      } else {
        const int rr = j0 - p.n_reg + kt;
        vis = rr < kl && (!p.causal || rr <= qi + p.off) &&
              (p.window <= 0 || qi + p.off - rr < p.window);
      }
      if (vis && p.ubias) {  // user bias: natural-log addend, or a mask where 0 hides the pair
        if (p.ub_kind == 1) {
          const float b = static_cast<const float*>(p.ubias)[ub_row + j0 + kt];
          vis = b != kNegInf;
          x = __builtin_fmaf(b, kLog2e, x);
        } else {
          vis = static_cast<const uint8_t*>(p.ubias)[ub_row + j0 + kt] != 0;
        }
      }
      if (!vis) continue;  // weight exactly zero
      if (x > m) {         // new running max: rescale what was accumulated
        const float alpha = exp2f(m - x);
        lsum *= alpha;
#pragma unroll
        for (int e = 0; e < E; ++e) acc[e] *= alpha;
        m = x;
      }
      const float pv = exp2f(x - m);
      lsum += pv;
#pragma unroll
      for (int e = 0; e < E; ++e) acc[e] = __builtin_fmaf(pv, sV[kt * E + e], acc[e]);
    }
  }

  // Merge: waves 1 .. W-1 publish their states, wave 0 combines them.
  if (wave > 0) {
    sM[wave - 1][lane] = m;
    sL[wave - 1][lane] = lsum;
#pragma unroll
    for (int e = 0; e < E; ++e) sAcc[wave - 1][e][lane] = acc[e];
  }
  __syncthreads();
  if (wave != 0) return;
  float mt = m;
#pragma unroll
  for (int w = 0; w < W - 1; ++w) mt = fmaxf(mt, sM[w][lane]);
  const float mu = mt == kNegInf ? 0.f : mt;
  const float a0 = exp2f(m - mu);
  lsum *= a0;
#pragma unroll
  for (int e = 0; e < E; ++e) acc[e] *= a0;
#pragma unroll
  for (int w = 0; w < W - 1; ++w) {
    const float aw = exp2f(sM[w][lane] - mu);
    lsum = __builtin_fmaf(sL[w][lane], aw, lsum);
#pragma unroll
    for (int e = 0; e < E; ++e) acc[e] = __builtin_fmaf(sAcc[w][e][lane], aw, acc[e]);
  }
  m = mt;

  if (qvalid) {
    const float inv = lsum > 0.f ? 1.f / lsum : 0.f;
    float* orow = p.o + (((size_t)n * p.Hq + h) * p.L + qi) * E;
#pragma unroll
    for (int e = 0; e < E; e += 4) {
      f32x4 ov = {acc[e] * inv, acc[e + 1] * inv, acc[e + 2] * inv, acc[e + 3] * inv};
      *reinterpret_cast<f32x4*>(orow + e) = ov;
    }
    float l = kNegInf;
    if (lsum > 0.f) {
      l = (m + log2f(lsum)) * kLn2;
      if (RBF) l -= p.gamma * qn2;
    }
    p.lse[((size_t)n * p.Hq + h) * p.L + qi] = l;
  }
}

// Small problems (a few row tiles, e.g. one head of 256 rows) leave the tiled
// kernel above on a handful of CUs, where each lane walks its row's keys one
// after another.  This kernel spreads them instead: one workgroup (256 threads)
// per query row.  The row's visible keys (registers, then the real keys of its
// causal / window interval: a contiguous run) are taken in chunks of 256, one key
// per thread: every thread loads its key row and forms its logit, so all the
// loads of a chunk are in flight together; the chunk's max and sum are reduced
// across the workgroup (shuffles, then LDS) and fold into the running state,
// the weights go to LDS, and the threads then take (4 output dims, every KG-th
// key of the chunk) for the weighted value sum, requesting all their value rows
// before using any.  The KG partial outputs are summed through LDS at the end.
// Same logit frame, sink, bias and LSE conventions as the tiled kernel.
constexpr int RT = 256;   // threads per workgroup = keys per chunk

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int s = 32; s > 0; s >>= 1) v = fmaxf(v, __shfl_xor(v, s, 64));
  return v;
}
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int s = 32; s > 0; s >>= 1) v += __shfl_xor(v, s, 64);
  return v;
}

template <int E, bool RBF>
__global__ __launch_bounds__(RT) void prefill_f32_rows_kernel(PrefillF32Params p) {
  constexpr int NQ = E / 4;        // float4 quads of a row
  constexpr int KG = RT / NQ;      // key groups in the value sum (16 at E = 64, 8 at E = 128)
  constexpr int PER = RT / KG;     // value rows per thread per chunk (16 or 32)
  __shared__ float sP[RT];
  __shared__ float sRed[2][4];
  __shared__ __attribute__((aligned(16))) f32x4 sAcc[KG][NQ];
  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const long long row = blockIdx.x;  // flat (n, h, i)
  const int i = (int)(row % p.L);
  const int nh = (int)(row / p.L);
  const int h = nh % p.Hq, n = nh / p.Hq;
  const int kh = h / (p.Hq / p.Hkv);

  // The query row, whole in every thread (one address for all: broadcast loads).
  const float* qrow = p.q + (size_t)row * E;
  float q[E];
  float qn2 = 0.f;
#pragma unroll
  for (int e = 0; e < E; e += 4) {
    const f32x4 c = *reinterpret_cast<const f32x4*>(qrow + e);
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      q[e + u] = c[u];
      qn2 = __builtin_fmaf(c[u], c[u], qn2);
    }
  }

  // Visible keys: registers [0, n_reg), then real keys [lo, hi] (virtual index v -> row).
  const int kl = p.key_len ? max(0, min(p.S_real, p.key_len[n])) : p.S_real;
  const int ip = i + p.off;
  const int hi = p.causal ? min(kl - 1, ip) : kl - 1;
  const int lo = p.window > 0 ? max(0, ip - p.window + 1) : 0;
  const int cnt = p.n_reg + max(0, hi - lo + 1);
  auto key_of = [&](int v) { return v < p.n_reg ? v : p.n_reg + lo + (v - p.n_reg); };
  const size_t kvoff = ((size_t)n * p.Hkv + kh) * (size_t)p.S * E;
  const long long ub_row = (long long)n * p.ub_sn + (long long)h * p.ub_sh + (long long)i * p.S;

  float m = kNegInf, l = 0.f;
  if (p.sink) {
    float s0 = p.sink[h];
    if (RBF) s0 += p.gamma * qn2;
    m = s0 * kLog2e;
    l = 1.f;
  }
  const int quad = tid % NQ, grp = tid / NQ;
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};

  for (int c0 = 0; c0 < cnt; c0 += RT) {
    // this thread's key: its logit (keys past the list take the list's first key,
    // so that every thread loads, and are masked)
    const int v = c0 + tid;
    const bool ok = v < cnt;
    float x;
    {
      const int j = key_of(ok ? v : 0);
      const float* krow = p.k + kvoff + (size_t)j * E;
      float d4[4] = {0.f, 0.f, 0.f, 0.f};
      float k2 = 0.f;
#pragma unroll
      for (int e = 0; e < E; e += 4) {
        const f32x4 kc = *reinterpret_cast<const f32x4*>(krow + e);
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          d4[u] = __builtin_fmaf(q[e + u], kc[u], d4[u]);
          if (RBF) k2 = __builtin_fmaf(kc[u], kc[u], k2);
        }
      }
      x = ((d4[0] + d4[1]) + (d4[2] + d4[3])) * p.c_logit;
      if (RBF) x = __builtin_fmaf(p.c_bias, k2, x);
      if (p.ubias) {  // user bias: natural-log addend, or a mask where 0 hides the pair
        if (p.ub_kind == 1) {
          const float b = static_cast<const float*>(p.ubias)[ub_row + j];
          x = (b == kNegInf) ? kNegInf : __builtin_fmaf(b, kLog2e, x);
        } else if (!static_cast<const uint8_t*>(p.ubias)[ub_row + j]) {
          x = kNegInf;
        }
      }
      if (!ok) x = kNegInf;
    }
    // chunk max across the workgroup
    float cm = wave_max(x);
    if (lane == 0) sRed[0][wave] = cm;
    __syncthreads();
    cm = fmaxf(fmaxf(sRed[0][0], sRed[0][1]), fmaxf(sRed[0][2], sRed[0][3]));
    const float m_new = fmaxf(m, cm);
    const float m_use = (m_new == kNegInf) ? 0.f : m_new;
    const float alpha = exp2f(m - m_use);
    const float pv = exp2f(x - m_use);
    sP[tid] = pv;
    const float ws = wave_sum(pv);
    if (lane == 0) sRed[1][wave] = ws;
    __syncthreads();  // weights and partial sums visible
    l = __builtin_fmaf(l, alpha, (sRed[1][0] + sRed[1][1]) + (sRed[1][2] + sRed[1][3]));
    m = m_new;
#pragma unroll
    for (int u = 0; u < 4; ++u) acc[u] *= alpha;
    // value rows: keys grp, grp + KG, ... of the chunk, all requested first
    const int n_here = min(RT, cnt - c0);
    f32x4 vr[PER];
    float pw[PER];
#pragma unroll
    for (int t = 0; t < PER; ++t) {
      const int vi = grp + t * KG;
      const bool okv = vi < n_here;
      pw[t] = okv ? sP[vi] : 0.f;
      vr[t] = *reinterpret_cast<const f32x4*>(p.v + kvoff + (size_t)key_of(c0 + (okv ? vi : 0)) * E + 4 * quad);
    }
    f32x4 a2 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int t = 0; t < PER; ++t)
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        if (t & 1)
          a2[u] = __builtin_fmaf(pw[t], vr[t][u], a2[u]);
        else
          acc[u] = __builtin_fmaf(pw[t], vr[t][u], acc[u]);
      }
#pragma unroll
    for (int u = 0; u < 4; ++u) acc[u] += a2[u];
    __syncthreads();  // every thread is done with sP and sRed before the next chunk
  }
  // Sum the key groups' partial outputs through LDS.
  sAcc[grp][quad] = acc;
  __syncthreads();
  if (tid < NQ) {
    f32x4 o = sAcc[0][tid];
#pragma unroll
    for (int gi = 1; gi < KG; ++gi)
#pragma unroll
      for (int u = 0; u < 4; ++u) o[u] += sAcc[gi][tid][u];
    const float inv = l > 0.f ? 1.f / l : 0.f;
#pragma unroll
    for (int u = 0; u < 4; ++u) o[u] *= inv;
    *reinterpret_cast<f32x4*>(p.o + (size_t)row * E + 4 * tid) = o;
  }
  if (tid == 0) {
    float lv = kNegInf;
    if (l > 0.f) {
      lv = (m + log2f(l)) * kLn2;
      if (RBF) lv -= p.gamma * qn2;
    }
    p.lse[row] = lv;
  }
}

template <int E, bool RBF>
hipError_t launch_rows_t(const PrefillF32Params& p, hipStream_t stream) {
  const long long rows = (long long)p.N * p.Hq * p.L;
  hipLaunchKernelGGL((prefill_f32_rows_kernel<E, RBF>), dim3((unsigned)rows), dim3(RT), 0, stream, p);
  return hipGetLastError();
}

// Below this many row tiles the tiled kernel would leave most of the chip idle.
constexpr long long kRowsKernelTiles = 64;

template <int E, bool RBF>
hipError_t launch_t(const PrefillF32Params& p, hipStream_t stream) {
  const long long blocks = (long long)p.num_q_tiles * p.N * p.Hq;
  if (blocks < kRowsKernelTiles) return launch_rows_t<E, RBF>(p, stream);
  hipLaunchKernelGGL((prefill_f32_kernel<E, RBF>), dim3((unsigned)blocks), dim3(BQ * F32Waves<E>::W), 0, stream, p);
  return hipGetLastError();
}

}  // namespace

namespace attn_impl {

hipError_t launch_prefill_f32(const FwdArgs& a, hipStream_t stream) {
  PrefillF32Params p;
  p.q = static_cast<const float*>(a.q);
  p.k = static_cast<const float*>(a.k);
  p.v = static_cast<const float*>(a.v);
  p.o = static_cast<float*>(a.o);
  p.lse = a.lse;
  p.sink = a.sink;
  p.N = a.N;
  p.Hq = a.Hq;
  p.Hkv = a.Hkv;
  p.L = a.L;
  p.S = a.S;
  p.n_reg = a.n_reg;
  p.S_real = a.S - a.n_reg;
  p.off = a.S - a.n_reg - a.L;
  p.causal = a.causal ? 1 : 0;
  p.key_len = a.key_len;
  p.ubias = a.bias;
  p.ub_kind = a.bias_kind;
  p.ub_sn = a.bias_sn;
  p.ub_sh = a.bias_sh;
  p.window = a.window;
  p.gamma = a.gamma;
  if (a.rbf) {
    p.c_logit = 2.f * a.gamma * 1.4426950408889634f;
    p.c_bias = -a.gamma * 1.4426950408889634f;
  } else {
    p.c_logit = a.scale * 1.4426950408889634f;
    p.c_bias = 0.f;
  }
  p.num_q_tiles = (a.L + BQ - 1) / BQ;
  if (a.E == 128) return a.rbf ? launch_t<128, true>(p, stream) : launch_t<128, false>(p, stream);
  return a.rbf ? launch_t<64, true>(p, stream) : launch_t<64, false>(p, stream);
}

}  // namespace attn_impl
