// backward_f32.hip -- gradients of the fused attention forward for float32
// inputs, gfx950.
//
// The same gradients as the bf16 backward (backward_bf16.hip), in fp32
// throughout (no operand is rounded), so the products run on the vector ALUs.
// For an upstream gradient dO of O, with P_ij = exp(z_ij - LSE_i) recomputed
// from the saved LSE, D_i = dO_i . O_i, dP_ij = dO_i . v_j and
// dS_ij = P_ij (dP_ij - D_i) (the Jacobian of the row softmax, "어텐션 메커니즘"
// section 2):
//   dV_j = sum_i P_ij dO_i
//   dQ_i = c sum_j dS_ij k_j            (dot, c = scale)
//        = c (sum_j dS_ij k_j - q_i sum_j dS_ij)   (rbf, c = 2 gamma)
//   dK_j = c sum_i dS_ij q_i            (dot)
//        = c (sum_i dS_ij q_i - k_j sum_i dS_ij)   (rbf)
//   dsink_h = -sum_i exp(s_h - LSE_i) D_i ("Attention Sink" section 4.2: the
//        sink sits only in the denominator)
// dK and dV of a key/value head sum over the query heads of its GQA group.
//
// Four launches, no atomics (results are deterministic):
//  1. bwd_f32_pre_kernel: one thread per query row: D_i, the reference
//     mref_i = (LSE_i [+ gamma |q_i|^2]) log2 e the weights are taken against
//     (+inf for a row with nothing visible), and one partial sum of the sink
//     gradient per 64 rows.
//  2. bwd_f32_dq_kernel: a query row is spread over E/64 lanes (64 dims each,
//     q, dO and the dQ accumulator in registers); every wave owns its own rows
//     and takes every key of the tiles staged in LDS (a key row is one
//     broadcast read per 16 bytes for all the lanes of a half), so the dot
//     products need no reduction beyond the E/64 lanes of a row.
//  3. bwd_f32_dkdv_kernel: the transposed layout: a key row is spread over
//     E/32 lanes (32 dims each; k, v and the dK, dV accumulators in
//     registers), query tiles of every head of the group staged in LDS.
//  4. bwd_f32_sink_kernel (with a sink): the partials summed in a fixed order.
// Keys and queries of a tile are taken in order, and tile t+1 is fetched into
// registers while tile t is consumed.  Visibility rule, logit frame and sink
// conventions are the forward's.
#include "device_common.h"
#include "kernels.h"

using namespace attn_dev;

namespace {

constexpr int NT = 256;  // threads per workgroup
constexpr int NW = 4;    // waves per workgroup
constexpr int BT = 32;   // rows per staged LDS tile (keys in dQ, queries in dK/dV)
constexpr int PRE = 64;  // query rows per workgroup of the first kernel

struct BwdF32Params {
  const float* q;
  const float* k;
  const float* v;
  const float* o;
  const float* dout;
  const float* lse;
  const float* sink;
  float* dq;
  float* dk;
  float* dv;
  float* dsink;
  float* delta;      // [N*Hq*L] D_i
  float* mref;       // [N*Hq*L] reference (log2 units); +inf for empty rows
  float* sink_part;  // [N*Hq*pre_blocks] partial sink gradients
  int N, Hq, Hkv, L, S, n_reg, S_real, off, causal, window;
  float c_logit, c_bias, gamma, dz;  // dz: scale (dot) or 2 gamma (rbf)
  int pre_blocks;
};

__device__ __forceinline__ float wave_sum64(float v) {
#pragma unroll
  for (int s = 32; s > 0; s >>= 1) v += __shfl_xor(v, s, 64);
  return v;
}

// Does query row i see key row j?  Register rows always; real key r = j - n_reg
// when r <= i + off (causal) and i + off - r < window (window > 0).
__device__ __forceinline__ bool visible(const BwdF32Params& p, int i, int j) {
  if (j < p.n_reg) return true;
  const int r = j - p.n_reg, ip = i + p.off;
  return (!p.causal || r <= ip) && (p.window <= 0 || ip - r < p.window);
}

template <int E, bool RBF>
__global__ __launch_bounds__(PRE) void bwd_f32_pre_kernel(BwdF32Params p) {
  const int nh = blockIdx.y, h = nh % p.Hq;
  const int i = blockIdx.x * PRE + threadIdx.x;
  float part = 0.f;
  if (i < p.L) {
    const size_t row = (size_t)nh * p.L + i;
    float d = 0.f, qn2 = 0.f;
#pragma unroll
    for (int e = 0; e < E; e += 4) {
      const f32x4 a = *reinterpret_cast<const f32x4*>(p.o + row * E + e);
      const f32x4 g = *reinterpret_cast<const f32x4*>(p.dout + row * E + e);
#pragma unroll
      for (int u = 0; u < 4; ++u) d = __builtin_fmaf(a[u], g[u], d);
      if (RBF) {
        const f32x4 x = *reinterpret_cast<const f32x4*>(p.q + row * E + e);
#pragma unroll
        for (int u = 0; u < 4; ++u) qn2 = __builtin_fmaf(x[u], x[u], qn2);
      }
    }
    const float lse = p.lse[row];
    p.delta[row] = d;
    p.mref[row] = lse == kNegInf ? __builtin_huge_valf() : (RBF ? lse + p.gamma * qn2 : lse) * kLog2e;
    if (p.sink && lse != kNegInf) part = -exp2f((p.sink[h] - lse) * kLog2e) * d;
  }
  if (p.dsink) {
    part = wave_sum64(part);
    if (threadIdx.x == 0) p.sink_part[(size_t)nh * p.pre_blocks + blockIdx.x] = part;
  }
}

// One workgroup per query head: the partials of every batch entry and block,
// summed in a fixed order.
__global__ __launch_bounds__(64) void bwd_f32_sink_kernel(BwdF32Params p) {
  const int h = blockIdx.x;
  float s = 0.f;
  for (int n = 0; n < p.N; ++n)
    for (int b = threadIdx.x; b < p.pre_blocks; b += 64) s += p.sink_part[((size_t)n * p.Hq + h) * p.pre_blocks + b];
  s = wave_sum64(s);
  if (threadIdx.x == 0) p.dsink[h] = s;
}

// Rows of E floats staged in LDS as H chunks of E/H floats, each chunk padded
// by 4 floats so that the H addresses one read serves fall in distinct banks.
template <int E, int H>
struct Staged {
  static constexpr int ED = E / H;      // dims per chunk (per lane)
  static constexpr int CS = ED + 4;     // chunk stride
  static constexpr int RS = H * CS;     // row stride
  static constexpr int NPT = BT * E / 4 / NT;  // 16-byte pieces per thread per tile
  static_assert(NPT * NT * 4 == BT * E, "tile must split evenly over the threads");
  // Piece idx of a tile: its row and the LDS offset it goes to.
  __device__ static int row_of(int idx) { return (idx * 4) / E; }
  __device__ static int lds_of(int idx) {
    const int row = (idx * 4) / E, col = (idx * 4) % E;
    return row * RS + (col / ED) * CS + col % ED;
  }
};

template <int E, bool RBF>
__global__ __launch_bounds__(NT, 1) void bwd_f32_dq_kernel(BwdF32Params p) {
  constexpr int HP = E / 64;       // lanes per query row
  constexpr int ED = E / HP;       // dims per lane
  constexpr int RW = 64 / HP;      // query rows per wave
  constexpr int BQ = NW * RW;      // query rows per workgroup
  using ST = Staged<E, HP>;
  constexpr int NPT = ST::NPT;
  __shared__ __attribute__((aligned(16))) float sK[BT * ST::RS];
  __shared__ __attribute__((aligned(16))) float sV[BT * ST::RS];
  __shared__ float sKb[BT];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int hh = lane % HP;
  const int nh = blockIdx.y, n = nh / p.Hq, h = nh % p.Hq;
  const int kh = h / (p.Hq / p.Hkv);
  const int i0 = blockIdx.x * BQ;
  const int qi = i0 + wave * RW + lane / HP;
  const bool qvalid = qi < p.L;
  const size_t row = (size_t)nh * p.L + (qvalid ? qi : 0);

  float q[ED], g[ED], acc[ED];
#pragma unroll
  for (int e = 0; e < ED; e += 4) {
    const f32x4 a = *reinterpret_cast<const f32x4*>(p.q + row * E + hh * ED + e);
    const f32x4 b = *reinterpret_cast<const f32x4*>(p.dout + row * E + hh * ED + e);
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      q[e + u] = a[u];
      g[e + u] = b[u];
      acc[e + u] = 0.f;
    }
  }
  const float D = qvalid ? p.delta[row] : 0.f;
  const float mr = qvalid ? p.mref[row] : __builtin_huge_valf();
  float dsum = 0.f;

  // Key tiles: register rows first, then the real keys any row of the
  // workgroup sees (its causal / window interval).
  const int i_last = min(i0 + BQ, p.L) - 1;
  const int r_hi = p.causal ? min(p.S_real - 1, i_last + p.off) : p.S_real - 1;
  const int r_lo = p.window > 0 ? max(0, i0 + p.off - p.window + 1) : 0;
  const int n_real_tiles = r_hi >= r_lo ? (r_hi - r_lo + BT) / BT : 0;
  const int n_reg_tiles = (p.n_reg + BT - 1) / BT;
  const int T = n_reg_tiles + n_real_tiles;
  const size_t kvoff = ((size_t)n * p.Hkv + kh) * (size_t)p.S * E;
  auto tile_keys = [&](int t, int& j0, int& kc) {
    if (t < n_reg_tiles) {
      j0 = t * BT;
      kc = min(BT, p.n_reg - j0);
    } else {
      j0 = p.n_reg + r_lo + (t - n_reg_tiles) * BT;
      kc = min(BT, p.S - j0);
    }
  };
  f32x4 kr[NPT], vr[NPT];
  auto fetch = [&](int t) {
    int j0, kc;
    tile_keys(t, j0, kc);
#pragma unroll
    for (int u = 0; u < NPT; ++u) {
      const int idx = tid + u * NT;
      const int r = ST::row_of(idx), col = (idx * 4) % E;
      kr[u] = f32x4{0.f, 0.f, 0.f, 0.f};
      vr[u] = f32x4{0.f, 0.f, 0.f, 0.f};
      if (r < kc) {
        kr[u] = *reinterpret_cast<const f32x4*>(p.k + kvoff + (size_t)(j0 + r) * E + col);
        vr[u] = *reinterpret_cast<const f32x4*>(p.v + kvoff + (size_t)(j0 + r) * E + col);
      }
    }
  };
  if (T > 0) fetch(0);

  for (int t = 0; t < T; ++t) {
    int j0, kc;
    tile_keys(t, j0, kc);
    __syncthreads();  // every wave is done with the previous tile
#pragma unroll
    for (int u = 0; u < NPT; ++u) {
      const int idx = tid + u * NT;
      *reinterpret_cast<f32x4*>(&sK[ST::lds_of(idx)]) = kr[u];
      *reinterpret_cast<f32x4*>(&sV[ST::lds_of(idx)]) = vr[u];
      if (RBF) {  // |k|^2: the E/4 pieces of a key row sit in consecutive lanes
        float ss = kr[u][0] * kr[u][0];
        ss = __builtin_fmaf(kr[u][1], kr[u][1], ss);
        ss = __builtin_fmaf(kr[u][2], kr[u][2], ss);
        ss = __builtin_fmaf(kr[u][3], kr[u][3], ss);
        ss = group_sum<16>(ss);
        if (E / 4 == 32) ss += __shfl_xor(ss, 16, 64);
        if ((idx * 4) % E == 0) sKb[ST::row_of(idx)] = p.c_bias * ss;
      }
    }
    __syncthreads();
    if (t + 1 < T) fetch(t + 1);

#pragma unroll 1
    for (int kt = 0; kt < kc; ++kt) {
      const float* kp = sK + kt * ST::RS + hh * ST::CS;
      const float* vp = sV + kt * ST::RS + hh * ST::CS;
      float s4[4] = {0.f, 0.f, 0.f, 0.f}, d4[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int e = 0; e < ED; ++e) {
        s4[e & 3] = __builtin_fmaf(q[e], kp[e], s4[e & 3]);
        d4[e & 3] = __builtin_fmaf(g[e], vp[e], d4[e & 3]);
      }
      float s = (s4[0] + s4[1]) + (s4[2] + s4[3]);
      float dp = (d4[0] + d4[1]) + (d4[2] + d4[3]);
      if (HP == 2) {
        s += dpp_mov<0xB1>(s);  // the other half of the row (lane ^ 1)
        dp += dpp_mov<0xB1>(dp);
      }
      float x = s * p.c_logit;
      if (RBF) x += sKb[kt];
      const float pe = visible(p, qi, j0 + kt) ? exp2f(x - mr) : 0.f;
      const float ds = pe * (dp - D);
      dsum += ds;
      // The key row is read again from LDS rather than kept in registers.
      asm volatile("" ::: "memory");
#pragma unroll
      for (int e = 0; e < ED; ++e) acc[e] = __builtin_fmaf(ds, kp[e], acc[e]);
    }
  }

  if (qvalid) {
    float* out = p.dq + row * E + hh * ED;
#pragma unroll
    for (int e = 0; e < ED; e += 4) {
      f32x4 r;
#pragma unroll
      for (int u = 0; u < 4; ++u) r[u] = p.dz * (RBF ? __builtin_fmaf(-q[e + u], dsum, acc[e + u]) : acc[e + u]);
      *reinterpret_cast<f32x4*>(out + e) = r;
    }
  }
}

template <int E, bool RBF>
__global__ __launch_bounds__(NT, 2) void bwd_f32_dkdv_kernel(BwdF32Params p) {
  constexpr int HK = E / 32;       // lanes per key row
  constexpr int ED = 32;           // dims per lane
  constexpr int KW = 64 / HK;      // key rows per wave
  constexpr int BK = NW * KW;      // key rows per workgroup
  using ST = Staged<E, HK>;
  constexpr int NPT = ST::NPT;
  __shared__ __attribute__((aligned(16))) float sQ[BT * ST::RS];
  __shared__ __attribute__((aligned(16))) float sG[BT * ST::RS];
  __shared__ float sD[BT], sM[BT];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int c = lane % HK;
  const int nk = blockIdx.y, n = nk / p.Hkv, kh = nk % p.Hkv;
  const int G = p.Hq / p.Hkv;
  const int j0 = blockIdx.x * BK;
  const int j = j0 + wave * KW + lane / HK;
  const bool kvalid = j < p.S;
  const size_t krow = (size_t)nk * p.S + (kvalid ? j : 0);

  float k[ED], v[ED], dk[ED], dv[ED];
  float kn2 = 0.f;
#pragma unroll
  for (int e = 0; e < ED; e += 4) {
    const f32x4 a = *reinterpret_cast<const f32x4*>(p.k + krow * E + c * ED + e);
    const f32x4 b = *reinterpret_cast<const f32x4*>(p.v + krow * E + c * ED + e);
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      k[e + u] = a[u];
      v[e + u] = b[u];
      dk[e + u] = 0.f;
      dv[e + u] = 0.f;
      kn2 = __builtin_fmaf(a[u], a[u], kn2);
    }
  }
  kn2 += dpp_mov<0xB1>(kn2);
  if (HK == 4) kn2 += dpp_mov<0x4E>(kn2);
  const float kb = RBF ? p.c_bias * kn2 : 0.f;
  float dsum = 0.f;

  // Query rows any key of the workgroup is seen by: all of them when the
  // workgroup holds a register row, else the causal / window interval of its
  // real keys.
  int lo = 0, hi = p.L - 1;
  if (j0 >= p.n_reg) {
    const int r_min = j0 - p.n_reg, r_max = min(j0 + BK, p.S) - 1 - p.n_reg;
    if (p.causal) lo = max(0, r_min - p.off);
    if (p.window > 0) hi = min(p.L - 1, r_max - p.off + p.window - 1);
  }
  const int ntiles = hi >= lo ? (hi - lo + BT) / BT : 0;
  const int T = G * ntiles;
  auto tile_rows = [&](int t, size_t& base, int& i0, int& qc) {
    const int hq = t / ntiles, tt = t % ntiles;
    base = ((size_t)n * p.Hq + (size_t)kh * G + hq) * p.L;
    i0 = lo + tt * BT;
    qc = min(BT, hi + 1 - i0);
  };
  f32x4 qr[NPT], gr[NPT];
  auto fetch = [&](int t) {
    size_t base;
    int i0, qc;
    tile_rows(t, base, i0, qc);
#pragma unroll
    for (int u = 0; u < NPT; ++u) {
      const int idx = tid + u * NT;
      const int r = ST::row_of(idx), col = (idx * 4) % E;
      qr[u] = f32x4{0.f, 0.f, 0.f, 0.f};
      gr[u] = f32x4{0.f, 0.f, 0.f, 0.f};
      if (r < qc) {
        qr[u] = *reinterpret_cast<const f32x4*>(p.q + (base + i0 + r) * E + col);
        gr[u] = *reinterpret_cast<const f32x4*>(p.dout + (base + i0 + r) * E + col);
      }
    }
  };
  if (T > 0) fetch(0);

  for (int t = 0; t < T; ++t) {
    size_t base;
    int i0, qc;
    tile_rows(t, base, i0, qc);
    __syncthreads();  // every wave is done with the previous tile
#pragma unroll
    for (int u = 0; u < NPT; ++u) {
      const int idx = tid + u * NT;
      *reinterpret_cast<f32x4*>(&sQ[ST::lds_of(idx)]) = qr[u];
      *reinterpret_cast<f32x4*>(&sG[ST::lds_of(idx)]) = gr[u];
    }
    if (tid < BT) {
      const bool ok = tid < qc;
      sD[tid] = ok ? p.delta[base + i0 + tid] : 0.f;
      sM[tid] = ok ? p.mref[base + i0 + tid] : __builtin_huge_valf();
    }
    __syncthreads();
    if (t + 1 < T) fetch(t + 1);

#pragma unroll 1
    for (int qt = 0; qt < qc; ++qt) {
      const float* qp = sQ + qt * ST::RS + c * ST::CS;
      const float* gp = sG + qt * ST::RS + c * ST::CS;
      float s4[4] = {0.f, 0.f, 0.f, 0.f}, d4[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int e = 0; e < ED; ++e) {
        s4[e & 3] = __builtin_fmaf(k[e], qp[e], s4[e & 3]);
        d4[e & 3] = __builtin_fmaf(v[e], gp[e], d4[e & 3]);
      }
      float s = (s4[0] + s4[1]) + (s4[2] + s4[3]);
      float dp = (d4[0] + d4[1]) + (d4[2] + d4[3]);
      s += dpp_mov<0xB1>(s);  // the other pieces of the key row (lane ^ 1, lane ^ 2)
      dp += dpp_mov<0xB1>(dp);
      if (HK == 4) {
        s += dpp_mov<0x4E>(s);
        dp += dpp_mov<0x4E>(dp);
      }
      const float x = __builtin_fmaf(s, p.c_logit, kb);
      const float pe = (kvalid && visible(p, i0 + qt, j)) ? exp2f(x - sM[qt]) : 0.f;
      const float ds = pe * (dp - sD[qt]);
      dsum += ds;
      asm volatile("" ::: "memory");
#pragma unroll
      for (int e = 0; e < ED; ++e) {
        dv[e] = __builtin_fmaf(pe, gp[e], dv[e]);
        dk[e] = __builtin_fmaf(ds, qp[e], dk[e]);
      }
    }
  }

  if (kvalid) {
    float* ok_ = p.dk + krow * E + c * ED;
    float* ov_ = p.dv + krow * E + c * ED;
#pragma unroll
    for (int e = 0; e < ED; e += 4) {
      f32x4 a, b;
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        a[u] = p.dz * (RBF ? __builtin_fmaf(-k[e + u], dsum, dk[e + u]) : dk[e + u]);
        b[u] = dv[e + u];
      }
      *reinterpret_cast<f32x4*>(ok_ + e) = a;
      *reinterpret_cast<f32x4*>(ov_ + e) = b;
    }
  }
}

template <int E, bool RBF>
hipError_t launch_t(const BwdF32Params& p, hipStream_t stream) {
  hipLaunchKernelGGL((bwd_f32_pre_kernel<E, RBF>), dim3((unsigned)p.pre_blocks, (unsigned)(p.N * p.Hq)),
                     dim3(PRE), 0, stream, p);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  constexpr int BQ = NW * (64 / (E / 64));
  hipLaunchKernelGGL((bwd_f32_dq_kernel<E, RBF>), dim3((unsigned)((p.L + BQ - 1) / BQ), (unsigned)(p.N * p.Hq)),
                     dim3(NT), 0, stream, p);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  constexpr int BK = NW * (64 / (E / 32));
  hipLaunchKernelGGL((bwd_f32_dkdv_kernel<E, RBF>), dim3((unsigned)((p.S + BK - 1) / BK), (unsigned)(p.N * p.Hkv)),
                     dim3(NT), 0, stream, p);
  e = hipGetLastError();
  if (e != hipSuccess || !p.dsink) return e;
  hipLaunchKernelGGL(bwd_f32_sink_kernel, dim3((unsigned)p.Hq), dim3(64), 0, stream, p);
  return hipGetLastError();
}

}  // namespace

namespace attn_impl {

hipError_t launch_backward_f32(const BwdArgs& a, hipStream_t stream) {
  const FwdArgs& f = a.f;
  BwdF32Params p;
  p.q = static_cast<const float*>(f.q);
  p.k = static_cast<const float*>(f.k);
  p.v = static_cast<const float*>(f.v);
  p.o = static_cast<const float*>(a.o);
  p.dout = static_cast<const float*>(a.dout);
  p.lse = a.lse;
  p.sink = f.sink;
  p.dq = static_cast<float*>(a.dq);
  p.dk = static_cast<float*>(a.dk);
  p.dv = static_cast<float*>(a.dv);
  p.dsink = a.dsink;
  p.N = f.N;
  p.Hq = f.Hq;
  p.Hkv = f.Hkv;
  p.L = f.L;
  p.S = f.S;
  p.n_reg = f.n_reg;
  p.S_real = f.S - f.n_reg;
  p.off = f.S - f.n_reg - f.L;
  p.causal = f.causal ? 1 : 0;
  p.window = f.window;
  p.gamma = f.gamma;
  if (f.rbf) {
    p.c_logit = 2.f * f.gamma * 1.4426950408889634f;
    p.c_bias = -f.gamma * 1.4426950408889634f;
    p.dz = 2.f * f.gamma;
  } else {
    p.c_logit = f.scale * 1.4426950408889634f;
    p.c_bias = 0.f;
    p.dz = f.scale;
  }
  // One sink-gradient partial per PRE rows: within the partial area the
  // workspace provides (backward_workspace_bytes).
  p.pre_blocks = (f.L + PRE - 1) / PRE;
  p.delta = a.workspace;
  p.mref = p.delta + (size_t)f.N * f.Hq * f.L;
  p.sink_part = p.mref + (size_t)f.N * f.Hq * f.L;
  if (f.E == 128) return f.rbf ? launch_t<128, true>(p, stream) : launch_t<128, false>(p, stream);
  return f.rbf ? launch_t<64, true>(p, stream) : launch_t<64, false>(p, stream);
}

}  // namespace attn_impl
