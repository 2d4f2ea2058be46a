// backward_bf16.hip -- gradients of the fused attention forward, bf16, gfx950.
//
// For an upstream gradient dO of O (LSE is an auxiliary output, no gradient
// flows into it), with P_ij = exp(z_ij - LSE_i) recomputed from the saved LSE,
// D_i = dO_i . O_i, dP_ij = dO_i . v_j and dS_ij = P_ij (dP_ij - D_i) (the
// Jacobian of the row softmax of "어텐션 메커니즘" section 2):
//   dV_j = sum_i P_ij dO_i
//   dQ_i = sum_j dS_ij dz_ij/dq_i,   dK_j = sum_i dS_ij dz_ij/dk_j
//     dot: dz/dq = scale k_j,                dz/dk = scale q_i
//     rbf: dz/dq = 2 gamma (k_j - q_i),      dz/dk = 2 gamma (q_i - k_j)
//          (the RBF digest's -gamma |q - k|^2, section details paragraph 2;
//          the |q|^2 and |k|^2 terms of the fold give the -2 gamma q_i sum_j dS_ij
//          and -2 gamma k_j sum_i dS_ij parts)
//   dsink_h = -sum_i exp(s_h - LSE_i) D_i   (the sink sits only in the
//          denominator, "Attention Sink" section 4.2)
// dK and dV of a key/value head sum over the query heads of its GQA group.
//
// Up to three launches, no atomics (results are deterministic):
//  1. bwd_dq_kernel: the forward's layout (128 query rows per workgroup, each
//     wave 32 rows, keys streamed through LDS in tiles of 64): S^T = K Q^T and
//     dP^T = V dO^T on v_mfma_f32_32x32x16_bf16, dS^T in registers, then
//     dQ^T += K^T dS^T with K^T read by the transposing LDS read.  Before its
//     key loop it forms, per row, D_i and the reference the weights are taken
//     against in the kernels' log2 frame, mref_i = (LSE_i [+ gamma |q_i|^2])
//     log2 e (+inf for a row with nothing visible, whose weights are all 0),
//     stores both for the dK/dV kernel, and writes one partial sum of the sink
//     gradient per wave.
//  2. bwd_dkdv_kernel: the transposed layout (128 keys per workgroup, each wave
//     32 keys held in VGPRs as K^T and V^T operands), streaming the query tiles
//     of every head of the group through LDS: S = Q K^T, dP = dO V^T, then
//     dV^T += dO^T P and dK^T += Q^T dS with dO^T and Q^T read transposed.
//  3. bwd_sink_kernel (with a sink): the partials summed in a fixed order.
// P and dS are rounded to bf16 as MFMA operands (fp32 accumulation), like P in
// the forward; outputs are bf16.
#include <type_traits>

#include "device_common.h"
#include "kernels.h"
#include "tile_common.h"

using namespace attn_dev;

namespace {

constexpr int NT = 256;   // threads per workgroup (4 waves)
constexpr int BT = 64;    // rows per staged LDS tile (keys in dQ, queries in dK/dV)
constexpr int BR = 128;   // rows owned per workgroup (queries in dQ, keys in dK/dV)

struct BwdParams {
  const uint16_t* q;
  const uint16_t* k;
  const uint16_t* v;
  const uint16_t* o;
  const uint16_t* dout;
  const float* lse;
  const float* sink;
  uint16_t* dq;
  uint16_t* dk;
  uint16_t* dv;
  float* dsink;
  float* delta;      // [N*Hq*L] D_i
  float* mref;       // [N*Hq*L] reference (log2 units); +inf for empty rows
  float* sink_part;  // [N*Hq*pre_blocks] partial sink gradients (one per dQ wave)
  int N, Hq, Hkv, L, S, n_reg, S_real, off, causal, window, rbf;
  float c_logit, c_bias, gamma, scale;
  int pre_blocks;
};

// One workgroup per query head: the partial sums in a fixed order.
__global__ __launch_bounds__(64) void bwd_sink_kernel(BwdParams p) {
  __shared__ float red[64];
  const int h = blockIdx.x;
  const int tid = threadIdx.x;
  float s = 0.f;
  for (int n = 0; n < p.N; ++n)
    for (int b = tid; b < p.pre_blocks; b += 64) s += p.sink_part[((size_t)n * p.Hq + h) * p.pre_blocks + b];
  red[tid] = s;
  __syncthreads();
  for (int w = 32; w > 0; w >>= 1) {
    if (tid < w) red[tid] += red[tid + w];
    __syncthreads();
  }
  if (tid == 0) p.dsink[h] = red[0];
}

// ---------------------------------------------------------------------------- shared pieces

// Logit frames (log2 units), as in the forward: dot x = c_logit*s; rbf
// x = c_logit*s + c_bias*|k|^2 = c_logit*(s - |k|^2/2) (c_bias = -c_logit/2; the
// -gamma|q|^2 part is folded into mref).  In RBF mode both kernels add -|k|^2/2
// to the scores inside the matrix product, as the forward does: one 32x32x8
// MFMA per 32x32 block whose key-side operand holds -|k|^2/2 as three bf16
// parts in K-dims 0..2 (lanes 0..31) against ones on the query side, so that a
// logit costs one multiply by c_logit.
enum { kDot = 0, kRbf = 1 };

typedef short short4v __attribute__((ext_vector_type(4)));

// v as hi + mid + lo, each rounded to bf16 (nearest even) in turn (about 24
// significant bits; the residuals are exact in fp32), packed as K-dims 0..3 of
// a 32x32x8 bf16 operand: {hi | mid << 16, lo}.
__device__ __forceinline__ u32x2 split3_bf16(float v) {
  const __bf16 hi = (__bf16)v;
  const float r1 = v - (float)hi;
  const __bf16 mid = (__bf16)r1;
  const __bf16 lo = (__bf16)(r1 - (float)mid);
  const uint32_t h = __builtin_bit_cast(uint16_t, hi), m = __builtin_bit_cast(uint16_t, mid),
                 l = __builtin_bit_cast(uint16_t, lo);
  return u32x2{h | (m << 16), l};
}

// bf16 ones in K-dims 0..2 of a 32x32x8 operand (lanes 0..31; zero elsewhere).
__device__ __forceinline__ u32x2 ones3_bf16(int g) {
  return g == 0 ? u32x2{0x3f803f80u, 0x00003f80u} : u32x2{0u, 0u};
}

template <int E, int R = BT>
struct TileGeom {
  static constexpr int QS = E / 16;         // MFMA steps over the head dimension
  static constexpr int EB = E / 32;         // 32-row blocks of a transposed E x 32 accumulator
  static constexpr int ECH = E / 8;         // 16-byte chunks per row
  static constexpr int ROWB = E * 2;        // bytes per row
  static constexpr int TILEB = R * ROWB;    // bytes per staged tile of R rows
  static constexpr int RPI = 1024 / ROWB;   // rows per 1 KB wave-wide LDS-direct load
  static constexpr int IPW = R / RPI / 4;   // such loads per wave per tile
  static constexpr int KCH = R * ECH / NT;  // 16-byte chunks per thread (register staging)
};

// Row-operand read offsets (A operand: row l32 of a 32-row block, chunk 2s+g)
// and transposing-read offsets (A operand built from 16 rows x 32 columns
// with the key/query order the accumulator hands out), as in the forward.
template <int E>
__device__ __forceinline__ void tile_offsets(int lane, uint32_t* rd, uint32_t (*trd)[2]) {
  using T = TileGeom<E>;
  const int l32 = lane & 31, g = lane >> 5;
#pragma unroll
  for (int s = 0; s < T::QS; ++s) rd[s] = (uint32_t)(l32 * T::ROWB + (((2 * s + g) ^ tile_swz<E>(l32)) * 16));
  const int q16 = lane >> 4, m16 = lane & 15;
#pragma unroll
  for (int c = 0; c < T::EB; ++c)
#pragma unroll
    for (int hh = 0; hh < 2; ++hh) {
      const int row = 4 * (q16 >> 1) + (m16 >> 2) + 8 * hh;
      const int d = 32 * c + 16 * (q16 & 1) + 4 * (m16 & 3);
      trd[c][hh] = (uint32_t)(row * T::ROWB + (((d >> 3) ^ tile_swz<E>(row)) * 16) + (d & 7) * 2);
    }
}

// Transposed A operand for 16 rows starting at row 16*u of a tile.
template <int E>
__device__ __forceinline__ bf16x8 read_tr_operand(const uint8_t* tile, const uint32_t (*trd)[2], int c, int u) {
  using T = TileGeom<E>;
  const shortx4 lo = lds_read_tr(tile + trd[c][0] + 16 * u * T::ROWB);
  const shortx4 hi = lds_read_tr(tile + trd[c][1] + 16 * u * T::ROWB);
  return __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
}

// Stage an E x 32 transposed accumulator block (acc[c][r] = X^T[dim 32c +
// 8(r/4) + 4g + r%4][row l32]) through this wave's LDS region and store whole
// bf16 rows row0 .. row0+31 (rows >= nrows are skipped); `ext` adds a
// per-element term from global memory (RBF corrections), scaled by the lane's
// `ext_scale`.  Called by every wave of the workgroup (it contains a barrier).
template <int E, int EB>
__device__ __forceinline__ void store_rows(const f32x16 (&acc)[EB], float mul, const uint16_t* ext, float ext_scale,
                                           uint16_t* sO, int lane, int row0, int nrows, uint16_t* dst) {
  constexpr int OSTR = E + 8;
  constexpr int ECH = E / 8;
  const int l32 = lane & 31, g = lane >> 5;
  const bool ok = row0 + l32 < nrows;
#pragma unroll
  for (int c = 0; c < EB; ++c)
#pragma unroll
    for (int rq = 0; rq < 4; ++rq) {
      float x[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) x[e] = acc[c][4 * rq + e] * mul;
      if (ext && ok) {
        const u32x2 w = *reinterpret_cast<const u32x2*>(ext + (size_t)l32 * E + 32 * c + 8 * rq + 4 * g);
        x[0] = __builtin_fmaf(ext_scale, bf16_lo(w[0]), x[0]);
        x[1] = __builtin_fmaf(ext_scale, bf16_hi(w[0]), x[1]);
        x[2] = __builtin_fmaf(ext_scale, bf16_lo(w[1]), x[2]);
        x[3] = __builtin_fmaf(ext_scale, bf16_hi(w[1]), x[3]);
      }
      *reinterpret_cast<bf16x4*>(&sO[l32 * OSTR + 32 * c + 8 * rq + 4 * g]) = pack_bf16x4(x[0], x[1], x[2], x[3]);
    }
  __syncthreads();
#pragma unroll
  for (int it = 0; it < (32 * ECH) / 64; ++it) {
    const int id = lane + 64 * it;
    const int rloc = id / ECH, c = id % ECH;
    if (row0 + rloc < nrows)
      __builtin_nontemporal_store(*reinterpret_cast<const u32x4*>(&sO[rloc * OSTR + 8 * c]),
                                  reinterpret_cast<u32x4*>(dst + (size_t)rloc * E + 8 * c));  // written once
  }
}

// Waves per SIMD: the dQ kernel holds Q^T and dO^T fragments, S^T and dP^T,
// and the dQ^T accumulator (E = 128: ~230 VGPRs); the dK/dV kernel holds K^T
// and two E x 32 accumulators, plus V^T at E = 64 (at E = 128 V^T is read
// from LDS, which keeps it within 256 registers: 2 waves).  In RBF mode the dQ
// kernel keeps a second E x 32 accumulator (see there).
template <int E, int MODE>
struct BwdOcc {
  static constexpr int kDq = E == 64 ? (MODE == 1 ? 2 : 3) : (MODE == 1 ? 1 : 2);
  static constexpr int kDkdv = 2;
};

// ---------------------------------------------------------------------------- 2. dQ

template <int E, int MODE>
__global__ __launch_bounds__(NT) __attribute__((amdgpu_waves_per_eu(BwdOcc<E, MODE>::kDq, BwdOcc<E, MODE>::kDq)))
void bwd_dq_kernel(BwdParams p, int num_q_tiles) {
  using T = TileGeom<E>;
  constexpr bool RBF = MODE == kRbf;
  constexpr int NB = BT / 32;
  constexpr int QS = T::QS, EB = T::EB, ECH = T::ECH, ROWB = T::ROWB, TILEB = T::TILEB;
  static_assert(2 * 32 * (E + 8) * 2 <= 2 * TILEB, "epilogue staging of two waves must fit one tile buffer");

  // Two separate LDS objects for the two [K | V] buffers: with the buffer index
  // a compile-time constant (tiles are taken in pairs) the compiler can tell
  // the reads of one buffer from the LDS-direct loads in flight into the other.
  __shared__ __attribute__((aligned(16))) uint8_t sKV0[2 * TILEB];
  __shared__ __attribute__((aligned(16))) uint8_t sKV1[2 * TILEB];
  __shared__ __attribute__((aligned(16))) u32x2 sKn[RBF ? 2 : 1][RBF ? BT : 1];  // RBF: -|k|^2/2 as 3 bf16
  auto k_tile = [&](int buf) { return buf ? sKV1 : sKV0; };
  auto v_tile = [&](int buf) { return (buf ? sKV1 : sKV0) + TILEB; };

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l32 = lane & 31, g = lane >> 5;
  // Query tiles in descending order when causal (the last tiles see the most
  // keys: heaviest first); consecutive blocks are different heads, so every
  // tile of a head lands on the same XCD (its K/V stays in that L2).
  const int nhs = gridDim.x / num_q_tiles;
  const int qt = p.causal ? num_q_tiles - 1 - (int)blockIdx.x / nhs : (int)blockIdx.x / nhs;
  const int nh = blockIdx.x % nhs;
  const int h = nh % p.Hq, n = nh / p.Hq;
  const int kh = h / (p.Hq / p.Hkv);
  const int i0 = qt * BR;
  const int qa = i0 + wave * 32;
  const int qi = qa + l32;
  const u32x2 qone = ones3_bf16(RBF ? g : 1);  // RBF: query side of the -|k|^2/2 fold
  const int qb = min(qa + 31, p.L - 1);
  const size_t row = (size_t)nh * p.L + min(qi, p.L - 1);

  // Q^T and dO^T fragments, and this workgroup's share of the row
  // preliminaries: D_i = dO_i . O_i, the reference the weights are taken
  // against in the log2 frame, mref_i = (LSE_i [+ gamma |q_i|^2]) log2 e (+inf
  // for a row with nothing visible, whose weights are all 0), both stored for
  // the dK/dV kernel, and one partial sum of the sink gradient per wave.
  bf16x8 qf[QS], gf[QS];
  float dd = 0.f, qn2 = 0.f;
#pragma unroll
  for (int s = 0; s < QS; ++s) {
    const u32x4 qc = *reinterpret_cast<const u32x4*>(p.q + row * E + 16 * s + 8 * g);
    const u32x4 gc = *reinterpret_cast<const u32x4*>(p.dout + row * E + 16 * s + 8 * g);
    const u32x4 oc = *reinterpret_cast<const u32x4*>(p.o + row * E + 16 * s + 8 * g);
    qf[s] = as_bf16x8(qc);
    gf[s] = as_bf16x8(gc);
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      dd = __builtin_fmaf(bf16_lo(oc[w]), bf16_lo(gc[w]), dd);
      dd = __builtin_fmaf(bf16_hi(oc[w]), bf16_hi(gc[w]), dd);
    }
    if (RBF) qn2 += sumsq8(qc);
  }
  dd = pair32_sum(dd);
  if (RBF) qn2 = pair32_sum(qn2);
  const float lse = qi < p.L ? p.lse[row] : kNegInf;
  float mr = __builtin_huge_valf(), dl = 0.f;
  if (lse != kNegInf) {
    mr = (lse + (RBF ? p.gamma * qn2 : 0.f)) * kLog2e;
    dl = dd;
  }
  if (g == 0 && qi < p.L) {
    p.delta[row] = dl;
    p.mref[row] = mr;
  }
  if (p.dsink) {
    float part = (g == 0 && lse != kNegInf && p.sink) ? -exp2f((p.sink[h] - lse) * kLog2e) * dl : 0.f;
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) part += xor_lane(part, o);
    if (lane == 0) p.sink_part[(size_t)nh * p.pre_blocks + qt * 4 + wave] = part;
  }
  // Dot mode: acc = K^T dS^T.  RBF mode: dQ_i/2gamma = sum_j dS_ij (k_j - q_i)
  // would difference two large terms (|q| >> |k - q| is common), and D_i from
  // the bf16 O would be amplified by |q_i|; instead acc = K^T (P o dP)^T and
  // acc2 = K^T P^T are kept apart, D_i = sum_j P_ij dP_ij is summed here in fp32
  // from the same P and dP, and dQ_i/2gamma = acc - D acc2 - q_i D (1 - sum_j P_ij).
  float rsa = 0.f, rsb = 0.f;  // RBF: this lane's share of sum_j P dP and sum_j P
  f32x16 acc[EB], acc2[RBF ? EB : 1];
#pragma unroll
  for (int c = 0; c < EB; ++c)
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      acc[c][r] = 0.f;
      if (RBF) acc2[c][r] = 0.f;
    }

  const int i_last = min(i0 + BR, p.L) - 1;
  const int r_hi = p.causal ? min(p.S_real - 1, i_last + p.off) : p.S_real - 1;
  const int r_lo = p.window > 0 ? max(0, i0 + p.off - p.window + 1) : 0;
  const int n_real_tiles = r_hi >= r_lo ? (r_hi - r_lo + BT) / BT : 0;
  const int n_reg_tiles = (p.n_reg + BT - 1) / BT;
  const int TT = n_reg_tiles + n_real_tiles;

  const size_t kvoff = ((size_t)n * p.Hkv + kh) * (size_t)p.S * E;
  const __amdgpu_buffer_rsrc_t krs = make_rsrc(p.k + kvoff, (uint32_t)p.S * ROWB);
  const __amdgpu_buffer_rsrc_t vrs = make_rsrc(p.v + kvoff, (uint32_t)p.S * ROWB);
  uint32_t ld_off[T::IPW];
#pragma unroll
  for (int b = 0; b < T::IPW; ++b) {
    const int rr = T::RPI * (T::IPW * wave + b) + lane / ECH;
    ld_off[b] = (uint32_t)(rr * ROWB + (((lane % ECH) ^ tile_swz<E>(rr)) * 16));
  }
  uint32_t rd[QS], trd[EB][2];
  tile_offsets<E>(lane, rd, trd);
  u32x4 kreg[T::KCH];

  auto tile_keys = [&](int t, int& j0, int& kc) __attribute__((always_inline)) {
    if (t < n_reg_tiles) {
      j0 = t * BT;
      kc = min(BT, p.n_reg - j0);
    } else {
      j0 = p.n_reg + r_lo + (t - n_reg_tiles) * BT;
      kc = min(BT, p.S - j0);
    }
  };
  auto issue_tile = [&](int t, int buf) __attribute__((always_inline)) {
    int j0, kc;
    tile_keys(t, j0, kc);
    const uint32_t tb = (uint32_t)j0 * ROWB;
#pragma unroll
    for (int b = 0; b < T::IPW; ++b) {
      const int blk = T::IPW * wave + b;
      buffer_load16_to_lds(vrs, v_tile(buf) + blk * 1024, tb + ld_off[b]);
      if (!RBF) buffer_load16_to_lds(krs, k_tile(buf) + blk * 1024, tb + ld_off[b]);
    }
    if (RBF) {
#pragma unroll
      for (int i = 0; i < T::KCH; ++i) {
        const int id = tid + NT * i;
        kreg[i] = buffer_load16(krs, tb + (uint32_t)((id / ECH) * ROWB + (id % ECH) * 16));
      }
    }
  };
  auto finish_tile = [&](int buf) __attribute__((always_inline)) {
    if (RBF) {
#pragma unroll
      for (int i = 0; i < T::KCH; ++i) {
        const int id = tid + NT * i;
        const int rr = id / ECH, c = id % ECH;
        *reinterpret_cast<u32x4*>(k_tile(buf) + rr * ROWB + ((c ^ tile_swz<E>(rr)) * 16)) = kreg[i];
        const float ss = group_sum<ECH>(sumsq8(kreg[i]));
        if (c == 0) sKn[buf][rr] = split3_bf16(-0.5f * ss);
      }
    }
    __builtin_amdgcn_s_waitcnt(0x0f70);  // vmcnt(0)
  };

  // MASKED: a tile not every row of the workgroup sees whole (visibility
  // tested per element); otherwise no visibility code.
  auto compute_tile = [&](int t, int buf, auto masked_tag) __attribute__((always_inline)) {
    constexpr bool MASKED = decltype(masked_tag)::value;
    int j0, kc;
    tile_keys(t, j0, kc);
    const bool is_reg = t < n_reg_tiles;
    if (qb < qa) return;
    if (MASKED && !is_reg) {
      const int ra = j0 - p.n_reg, rb = ra + BT - 1;
      const bool any = !((ra >= p.S_real) || (p.causal && ra > qb + p.off) ||
                         (p.window > 0 && qa + p.off - rb >= p.window));
      if (!any) return;
    }
    const uint8_t* k_s = k_tile(buf);
    const uint8_t* v_s = v_tile(buf);
    f32x16 st[NB], dp[NB];
#pragma unroll
    for (int b = 0; b < NB; ++b)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        st[b][r] = 0.f;
        dp[b][r] = 0.f;
      }
#pragma unroll
    for (int s = 0; s < QS; ++s) {
      bf16x8 a[NB], bv[NB];
#pragma unroll
      for (int b = 0; b < NB; ++b) {
        a[b] = *reinterpret_cast<const bf16x8*>(k_s + rd[s] + 32 * b * ROWB);
        bv[b] = *reinterpret_cast<const bf16x8*>(v_s + rd[s] + 32 * b * ROWB);
      }
#pragma unroll
      for (int b = 0; b < NB; ++b) {
        st[b] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[b], qf[s], st[b], 0, 0, 0);
        dp[b] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(bv[b], gf[s], dp[b], 0, 0, 0);
      }
    }
    if (RBF) {
      // -|k|^2/2 of key row l32 of block b (lanes g = 0) against ones.
#pragma unroll
      for (int b = 0; b < NB; ++b) {
        const u32x2 kn = g == 0 ? sKn[buf][32 * b + l32] : u32x2{0u, 0u};
        st[b] = __builtin_amdgcn_mfma_f32_32x32x8bf16_1k(__builtin_bit_cast(short4v, kn),
                                                          __builtin_bit_cast(short4v, qone), st[b], 0, 0, 0);
      }
    }
    // Visible keys of this lane's row: one interval [lo, hi] of tile offsets.
    int lo = 0, hi = BT - 1;
    if (MASKED) {
      if (is_reg) {
        lo = 0;
        hi = kc - 1;
      } else {
        const int base = j0 - p.n_reg;
        const int ip = qi + p.off;
        hi = min(p.S_real - 1, p.causal ? ip : p.S_real - 1) - base;
        lo = (p.window > 0 ? ip - p.window + 1 : 0) - base;
      }
      lo -= 4 * g;
      hi -= 4 * g;
    }
#pragma unroll
    for (int b = 0; b < NB; ++b)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int ko = 32 * b + 8 * (r >> 2) + (r & 3);
        const float x = st[b][r] * p.c_logit;
        const float pw = (!MASKED || ((ko >= lo) & (ko <= hi))) ? fast_exp2(x - mr) : 0.f;
        if (RBF) {
          const float pd = pw * dp[b][r];
          rsa += pd;
          rsb += pw;
          st[b][r] = pd;
          dp[b][r] = pw;
        } else {
          st[b][r] = pw * (dp[b][r] - dl);
        }
      }
    // dQ^T += K^T dS^T (RBF: K^T (P o dP)^T and K^T P^T), 16 keys per MFMA step.
#pragma unroll
    for (int b = 0; b < NB; ++b)
#pragma unroll
      for (int s2 = 0; s2 < 2; ++s2) {
        const int r0 = 8 * s2;
        const bf16x8 sf = pack_bf16x8(st[b][r0 + 0], st[b][r0 + 1], st[b][r0 + 2], st[b][r0 + 3],
                                      st[b][r0 + 4], st[b][r0 + 5], st[b][r0 + 6], st[b][r0 + 7]);
        bf16x8 pf;
        if (RBF)
          pf = pack_bf16x8(dp[b][r0 + 0], dp[b][r0 + 1], dp[b][r0 + 2], dp[b][r0 + 3], dp[b][r0 + 4],
                           dp[b][r0 + 5], dp[b][r0 + 6], dp[b][r0 + 7]);
#pragma unroll
        for (int c = 0; c < EB; ++c) {
          const bf16x8 kt = read_tr_operand<E>(k_s, trd, c, 2 * b + s2);
          acc[c] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kt, sf, acc[c], 0, 0, 0);
          if (RBF) acc2[c] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kt, pf, acc2[c], 0, 0, 0);
        }
      }
  };

  if (TT > 0) {
    issue_tile(0, 0);
    finish_tile(0);
  }
  __syncthreads();
  auto step = [&](int t, int buf, auto masked_tag) __attribute__((always_inline)) {
    if (t + 1 < TT) issue_tile(t + 1, buf ^ 1);
    compute_tile(t, buf, masked_tag);
    if (t + 1 < TT) finish_tile(buf ^ 1);
    __syncthreads();
  };
  // Tiles t in [ta, tb), of one class, in pairs (compile-time buffer index).
  auto run = [&](int ta, int tb, auto masked_tag) __attribute__((always_inline)) {
    int t = ta;
    if (t < tb && (t & 1)) step(t++, 1, masked_tag);
    for (; t + 1 < tb; t += 2) {
      step(t, 0, masked_tag);
      step(t + 1, 1, masked_tag);
    }
    if (t < tb) step(t, 0, masked_tag);
  };
  // Real tiles [k_full0, k_full1] are seen whole by every row of the
  // workgroup; register tiles and the real tiles before and after them are
  // of the masked class.
  int k_full0 = 0, k_full1 = -1;
  {
    const int lim = min(p.S_real - 1, p.causal ? i0 + p.off : p.S_real - 1);
    k_full1 = (lim - r_lo - (BT - 1)) >= 0 ? (lim - r_lo - (BT - 1)) / BT : -1;
    if (p.window > 0) {
      const int need = i_last + p.off - p.window + 1 - r_lo;  // first tile start allowed
      k_full0 = need > 0 ? (need + BT - 1) / BT : 0;
    }
    k_full1 = min(k_full1, n_real_tiles - 1);
    if (k_full0 > k_full1) {
      k_full0 = 0;
      k_full1 = -1;
    }
  }
  const int t_full0 = n_reg_tiles + k_full0, t_full1 = n_reg_tiles + k_full1 + 1;
  const int head_end = (t_full1 > t_full0) ? t_full0 : TT;
  run(0, head_end, std::true_type{});
  run(head_end, t_full1, std::false_type{});
  run(max(head_end, t_full1), TT, std::true_type{});

  // dQ = scale K^T dS^T (dot) or 2 gamma (acc - D acc2 - q_i D (1 - sum_j P_ij)) (rbf).
  float ext = 0.f;
  const size_t obase = (size_t)nh * p.L;
  if (RBF) {
    const float d = pair32_sum(rsa), sp = pair32_sum(rsb);
#pragma unroll
    for (int c = 0; c < EB; ++c)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[c][r] = __builtin_fmaf(-d, acc2[c][r], acc[c][r]);
    ext = -2.f * p.gamma * d * (1.f - sp);
    if (g == 0 && qi < p.L) p.delta[obase + qi] = d;  // the dK/dV kernel uses the same D
  }
  const float mul = RBF ? 2.f * p.gamma : p.scale;
  uint16_t* sO = reinterpret_cast<uint16_t*>(wave < 2 ? sKV0 : sKV1) + (wave & 1) * 32 * (E + 8);
  store_rows<E, EB>(acc, mul, RBF ? p.q + (obase + qa) * E : nullptr, ext, sO, lane, qa, p.L,
                    p.dq + (obase + qa) * E);
}

// ---------------------------------------------------------------------------- 3. dK, dV

template <int E, int MODE>
__global__ __launch_bounds__(NT) __attribute__((amdgpu_waves_per_eu(BwdOcc<E, MODE>::kDkdv, BwdOcc<E, MODE>::kDkdv)))
void bwd_dkdv_kernel(BwdParams p, int num_k_tiles) {
  // E = 128: the V^T operands live in LDS (the workgroup's 128 value rows)
  // instead of registers, and query tiles are 32 rows, so that the kernel fits
  // 256 registers and runs 2 waves per SIMD; E = 64 keeps them in registers.
  constexpr bool VL = E == 128;
  constexpr int QT = VL ? 32 : BT;  // query rows per staged tile
  using T = TileGeom<E, QT>;
  constexpr bool RBF = MODE == kRbf;
  constexpr int QS = T::QS, EB = T::EB, ECH = T::ECH, ROWB = T::ROWB, TILEB = T::TILEB;
  constexpr int VB = VL ? BR * ROWB : 0;  // bytes of the staged value rows

  // [buf][Q tile | dO tile] then (VL) the value rows; per buf the tile rows'
  // reference and D values.  The epilogue reuses the same bytes.
  // The two [Q | dO] buffers and the value rows are separate LDS objects (see
  // the dQ kernel); the epilogue stages each wave's rows in one of them.
  constexpr int EPW = 32 * (E + 8) * 2;   // epilogue staging per wave
  constexpr int SQB = (2 * TILEB) > EPW ? (2 * TILEB) : EPW;
  constexpr int SVB = VB > 2 * EPW ? VB : 2 * EPW;
  __shared__ __attribute__((aligned(16))) uint8_t sQG0[SQB];
  __shared__ __attribute__((aligned(16))) uint8_t sQG1[SQB];
  __shared__ __attribute__((aligned(16))) uint8_t sVR[SVB];
  __shared__ __attribute__((aligned(16))) float sMR[2][QT];
  __shared__ __attribute__((aligned(16))) float sDL[2][QT];
  auto q_tile = [&](int buf) { return buf ? sQG1 : sQG0; };
  auto g_tile = [&](int buf) { return (buf ? sQG1 : sQG0) + TILEB; };
  uint8_t* sV = sVR;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l32 = lane & 31, g = lane >> 5;
  // Key tiles in ascending order (with a causal mask the first tiles are seen
  // by the most queries: heaviest first); consecutive blocks are different kv
  // heads, so every tile of a kv head lands on the same XCD.
  const int nks = gridDim.x / num_k_tiles;
  const int kt = blockIdx.x / nks;
  const int nk = blockIdx.x % nks;
  const int kh = nk % p.Hkv, n = nk / p.Hkv;
  const int G = p.Hq / p.Hkv;
  const int j0 = kt * BR;                 // first key (flat, registers included) of the workgroup
  const int ja = j0 + wave * 32;          // first key of this wave
  const int kj = ja + l32;                // this lane's key
  const size_t kvbase = ((size_t)n * p.Hkv + kh) * (size_t)p.S;

  // K^T and V^T fragments: lane holds row kj, dims 16s + 8g .. +8 (zeros past S).
  // VL: the workgroup's value rows go to LDS instead (row r, 16-byte chunk c at
  // chunk slot c ^ swz(r): the fragment reads of a 32-row block are then
  // conflict-free, as for the forward's K tile); a barrier precedes their use.
  bf16x8 kf[QS], vf[VL ? 1 : QS];
  float nk2 = 0.f;
#pragma unroll
  for (int s = 0; s < QS; ++s) {
    const bool ok = kj < p.S;
    const u32x4 kc = load16_or_zero(p.k + (kvbase + min(kj, p.S - 1)) * E + 16 * s + 8 * g, ok);
    kf[s] = as_bf16x8(kc);
    if (!VL) vf[s] = as_bf16x8(load16_or_zero(p.v + (kvbase + min(kj, p.S - 1)) * E + 16 * s + 8 * g, ok));
    if (RBF) nk2 += sumsq8(kc);
  }
  if (VL) {
#pragma unroll
    for (int i = 0; i < BR * ECH / NT; ++i) {
      const int id = tid + NT * i;
      const int r = id / ECH, c = id % ECH;
      const int row = j0 + r;
      const u32x4 x = load16_or_zero(p.v + (kvbase + min(row, p.S - 1)) * E + 8 * c, row < p.S);
      *reinterpret_cast<u32x4*>(sV + r * ROWB + ((c ^ tile_swz<E>(r)) * 16)) = x;
    }
  }
  // RBF: this lane's key's -|k|^2/2 as the key-side operand of the fold (lanes g = 0).
  // The halves' sum is a cross-lane exchange: every lane takes part, the lane
  // test comes after it.
  const u32x2 ksplit = split3_bf16(-0.5f * (RBF ? pair32_sum(nk2) : 0.f));
  const u32x2 kfold = (RBF && g == 0) ? ksplit : u32x2{0u, 0u};
  const u32x2 qone = ones3_bf16(RBF ? g : 1);
  float csum = 0.f;  // RBF: this lane's share of sum_i dS_ij
  f32x16 accv[EB], acck[EB];
#pragma unroll
  for (int c = 0; c < EB; ++c)
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      accv[c][r] = 0.f;
      acck[c][r] = 0.f;
    }

  // Query rows that see this lane's key: [qlo, qhi] (empty for keys past S).
  int qlo, qhi;
  if (kj >= p.S) {
    qlo = 1;
    qhi = 0;
  } else if (kj < p.n_reg) {
    qlo = 0;
    qhi = p.L - 1;
  } else {
    const int r = kj - p.n_reg;
    qlo = p.causal ? max(0, r - p.off) : 0;
    qhi = p.window > 0 ? min(p.L - 1, r - p.off + p.window - 1) : p.L - 1;
  }
  // Query tiles some key of the workgroup sees.
  int i_lo = 0, i_hi = p.L - 1;
  {
    const int jb = min(j0 + BR, p.S) - 1;
    if (j0 >= p.n_reg) {
      const int ra = j0 - p.n_reg, rb = jb - p.n_reg;
      if (p.causal) i_lo = max(0, ra - p.off);
      if (p.window > 0) i_hi = min(p.L - 1, rb - p.off + p.window - 1);
    }
  }
  const int t_lo = i_lo / QT;
  const int ntq = i_hi >= i_lo ? i_hi / QT - t_lo + 1 : 0;
  const int steps = G * ntq;

  uint32_t ld_off[T::IPW];
#pragma unroll
  for (int b = 0; b < T::IPW; ++b) {
    const int rr = T::RPI * (T::IPW * wave + b) + lane / ECH;
    ld_off[b] = (uint32_t)(rr * ROWB + (((lane % ECH) ^ tile_swz<E>(rr)) * 16));
  }
  uint32_t rd[QS], trd[EB][2];
  tile_offsets<E>(lane, rd, trd);
  float mrv = 0.f, dlv = 0.f;  // staged per-row values (threads < QT)

  auto step_rows = [&](int st_i, int& h, int& i0) __attribute__((always_inline)) {
    h = kh * G + st_i / ntq;
    i0 = (t_lo + st_i % ntq) * QT;
  };
  auto issue_step = [&](int st_i, int buf) __attribute__((always_inline)) {
    int h, i0;
    step_rows(st_i, h, i0);
    const size_t qoff = ((size_t)n * p.Hq + h) * p.L;
    const __amdgpu_buffer_rsrc_t qrs = make_rsrc(p.q + qoff * E, (uint32_t)p.L * ROWB);
    const __amdgpu_buffer_rsrc_t grs = make_rsrc(p.dout + qoff * E, (uint32_t)p.L * ROWB);
    const uint32_t tb = (uint32_t)i0 * ROWB;
#pragma unroll
    for (int b = 0; b < T::IPW; ++b) {
      const int blk = T::IPW * wave + b;
      buffer_load16_to_lds(qrs, q_tile(buf) + blk * 1024, tb + ld_off[b]);
      buffer_load16_to_lds(grs, g_tile(buf) + blk * 1024, tb + ld_off[b]);
    }
    if (tid < QT) {
      const int i = i0 + tid;
      mrv = i < p.L ? p.mref[qoff + i] : __builtin_huge_valf();
      dlv = i < p.L ? p.delta[qoff + i] : 0.f;
    }
  };
  auto finish_step = [&](int buf) __attribute__((always_inline)) {
    if (tid < QT) {
      sMR[buf][tid] = mrv;
      sDL[buf][tid] = dlv;
    }
    __builtin_amdgcn_s_waitcnt(0x0f70);  // vmcnt(0)
  };

  // MASKED: a query tile not every key of the workgroup sees whole (tested per
  // element); otherwise no visibility code (rows past L have weight 0 anyway:
  // their reference is +inf).
  auto compute_step = [&](int st_i, int buf, auto masked_tag) __attribute__((always_inline)) {
    constexpr bool MASKED = decltype(masked_tag)::value;
    int h, i0;
    step_rows(st_i, h, i0);
    (void)h;
    const uint8_t* q_s = q_tile(buf);
    const uint8_t* g_s = g_tile(buf);
#pragma unroll
    for (int b = 0; b < QT / 32; ++b) {
      const int ib = i0 + 32 * b;  // first query row of this block
      f32x16 s_acc, d_acc;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        s_acc[r] = 0.f;
        d_acc[r] = 0.f;
      }
#pragma unroll
      for (int s = 0; s < QS; ++s) {
        const bf16x8 a = *reinterpret_cast<const bf16x8*>(q_s + rd[s] + 32 * b * ROWB);
        const bf16x8 ga = *reinterpret_cast<const bf16x8*>(g_s + rd[s] + 32 * b * ROWB);
        // V^T fragment of this wave's 32 value rows (same offsets as the tile reads).
        const bf16x8 vs = VL ? *reinterpret_cast<const bf16x8*>(sV + wave * 32 * ROWB + rd[s]) : vf[VL ? 0 : s];
        s_acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, kf[s], s_acc, 0, 0, 0);
        d_acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ga, vs, d_acc, 0, 0, 0);
      }
      if (RBF)
        s_acc = __builtin_amdgcn_mfma_f32_32x32x8bf16_1k(__builtin_bit_cast(short4v, qone),
                                                          __builtin_bit_cast(short4v, kfold), s_acc, 0, 0, 0);
      // Register r holds query row ib + 8(r/4) + 4g + r%4 for this lane's key.
      const int lo = qlo - ib - 4 * g, hi = qhi - ib - 4 * g;
      f32x16 pw, ds;
#pragma unroll
      for (int rq = 0; rq < 4; ++rq) {
        const f32x4 m4 = *reinterpret_cast<const f32x4*>(&sMR[buf][32 * b + 8 * rq + 4 * g]);
        const f32x4 d4 = *reinterpret_cast<const f32x4*>(&sDL[buf][32 * b + 8 * rq + 4 * g]);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int r = 4 * rq + e;
          const int ro = 8 * rq + e;
          const float x = s_acc[r] * p.c_logit;
          const float w = (!MASKED || ((ro >= lo) & (ro <= hi))) ? fast_exp2(x - m4[e]) : 0.f;
          pw[r] = w;
          ds[r] = w * (d_acc[r] - d4[e]);
          if (RBF) csum += ds[r];
        }
      }
      // dV^T += dO^T P and dK^T += Q^T dS, 16 query rows per MFMA step.
#pragma unroll
      for (int s2 = 0; s2 < 2; ++s2) {
        const int r0 = 8 * s2;
        const bf16x8 pf = pack_bf16x8(pw[r0 + 0], pw[r0 + 1], pw[r0 + 2], pw[r0 + 3], pw[r0 + 4], pw[r0 + 5],
                                      pw[r0 + 6], pw[r0 + 7]);
        const bf16x8 sf = pack_bf16x8(ds[r0 + 0], ds[r0 + 1], ds[r0 + 2], ds[r0 + 3], ds[r0 + 4], ds[r0 + 5],
                                      ds[r0 + 6], ds[r0 + 7]);
#pragma unroll
        for (int c = 0; c < EB; ++c) {
          accv[c] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(read_tr_operand<E>(g_s, trd, c, 2 * b + s2), pf, accv[c],
                                                            0, 0, 0);
          acck[c] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(read_tr_operand<E>(q_s, trd, c, 2 * b + s2), sf, acck[c],
                                                            0, 0, 0);
        }
      }
    }
  };

  if (steps > 0) {
    issue_step(0, 0);
    finish_step(0);
  }
  __syncthreads();
  auto step = [&](int st_i, int buf, auto masked_tag) __attribute__((always_inline)) {
    if (st_i + 1 < steps) issue_step(st_i + 1, buf ^ 1);
    compute_step(st_i, buf, masked_tag);
    if (st_i + 1 < steps) finish_step(buf ^ 1);
    __syncthreads();
  };
  // Steps [ta, tb), of one class, in pairs (compile-time buffer index).
  auto run = [&](int ta, int tb, auto masked_tag) __attribute__((always_inline)) {
    int t = ta;
    if (t < tb && (t & 1)) step(t++, 1, masked_tag);
    for (; t + 1 < tb; t += 2) {
      step(t, 0, masked_tag);
      step(t + 1, 1, masked_tag);
    }
    if (t < tb) step(t, 0, masked_tag);
  };
  // Query tiles j (of each head's ntq) in [jf0, jf1] are seen whole by every
  // key of the workgroup: causal needs i0 + off >= the last real key, the
  // window needs the last row i0 + QT - 1 within window - 1 of the first real
  // key.  Workgroups holding keys past S keep every tile masked.
  int jf0 = 0, jf1 = ntq - 1;
  {
    const int jb = j0 + BR - 1;
    if (jb >= p.S) {
      jf0 = 0;
      jf1 = -1;
    } else if (jb >= p.n_reg) {
      const int ra = max(j0, p.n_reg) - p.n_reg, rb = jb - p.n_reg;
      auto fdiv = [](int a, int b) { return a >= 0 ? a / b : -((-a + b - 1) / b); };
      if (p.causal) jf0 = max(jf0, -fdiv(-(rb - p.off), QT) - t_lo);  // ceil((rb - off) / QT)
      if (p.window > 0) jf1 = min(jf1, fdiv(ra - p.off + p.window - QT, QT) - t_lo);
    }
    if (jf0 > jf1) {
      jf0 = 0;
      jf1 = -1;
    }
  }
  const int nm0 = jf1 >= jf0 ? jf0 : ntq;   // leading masked tiles per head
  const int nfl = jf1 >= jf0 ? jf1 - jf0 + 1 : 0;
  for (int hh = 0; hh < G; ++hh) {
    const int base = hh * ntq;
    run(base, base + nm0, std::true_type{});
    run(base + nm0, base + nm0 + nfl, std::false_type{});
    run(base + nm0 + nfl, base + ntq, std::true_type{});
  }

  // dV = P^T dO; dK = scale Q^T dS (dot) or 2 gamma (Q^T dS - k_j sum_i dS_ij) (rbf).
  const float cs = RBF ? pair32_sum(csum) : 0.f;
  uint16_t* sO = reinterpret_cast<uint16_t*>(wave < 2 ? sVR + wave * EPW : wave == 2 ? sQG0 : sQG1);
  store_rows<E, EB>(accv, 1.f, nullptr, 0.f, sO, lane, ja, p.S, p.dv + (kvbase + ja) * E);
  __syncthreads();
  store_rows<E, EB>(acck, RBF ? 2.f * p.gamma : p.scale, RBF ? p.k + (kvbase + ja) * E : nullptr,
                    -2.f * p.gamma * cs, sO, lane, ja, p.S, p.dk + (kvbase + ja) * E);
}

template <int E, int MODE>
hipError_t launch_main(const BwdParams& p, hipStream_t stream) {
  const int qtiles = (p.L + BR - 1) / BR;
  hipLaunchKernelGGL((bwd_dq_kernel<E, MODE>), dim3((unsigned)(qtiles * p.N * p.Hq)), dim3(NT), 0, stream, p, qtiles);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int ktiles = (p.S + BR - 1) / BR;
  hipLaunchKernelGGL((bwd_dkdv_kernel<E, MODE>), dim3((unsigned)(ktiles * p.N * p.Hkv)), dim3(NT), 0, stream, p,
                     ktiles);
  return hipGetLastError();
}

}  // namespace

namespace attn_impl {

hipError_t launch_backward_bf16(const BwdArgs& a, hipStream_t stream) {
  const FwdArgs& f = a.f;
  BwdParams p;
  p.q = static_cast<const uint16_t*>(f.q);
  p.k = static_cast<const uint16_t*>(f.k);
  p.v = static_cast<const uint16_t*>(f.v);
  p.o = static_cast<const uint16_t*>(a.o);
  p.dout = static_cast<const uint16_t*>(a.dout);
  p.lse = a.lse;
  p.sink = f.sink;
  p.dq = static_cast<uint16_t*>(a.dq);
  p.dk = static_cast<uint16_t*>(a.dk);
  p.dv = static_cast<uint16_t*>(a.dv);
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
  p.rbf = f.rbf;
  p.gamma = f.gamma;
  p.scale = f.scale;
  if (f.rbf) {
    p.c_logit = 2.f * f.gamma * kLog2e;
    p.c_bias = -f.gamma * kLog2e;
  } else {
    p.c_logit = f.scale * kLog2e;
    p.c_bias = 0.f;
  }
  p.pre_blocks = 4 * ((f.L + BR - 1) / BR);  // one sink-gradient partial per wave of the dQ kernel
  p.delta = a.workspace;
  p.mref = p.delta + (size_t)f.N * f.Hq * f.L;
  p.sink_part = p.mref + (size_t)f.N * f.Hq * f.L;

  hipError_t e;
  if (f.E == 128)
    e = f.rbf ? launch_main<128, kRbf>(p, stream) : launch_main<128, kDot>(p, stream);
  else
    e = f.rbf ? launch_main<64, kRbf>(p, stream) : launch_main<64, kDot>(p, stream);
  if (e != hipSuccess || !p.dsink) return e;
  hipLaunchKernelGGL(bwd_sink_kernel, dim3((unsigned)f.Hq), dim3(64), 0, stream, p);
  return hipGetLastError();
}

size_t backward_workspace_bytes(int N, int Hq, int L) {
  const size_t rows = (size_t)N * Hq * L;
  const size_t partials = 4 * (size_t)((L + BR - 1) / BR);
  return (2 * rows + (size_t)N * Hq * partials) * sizeof(float);
}

}  // namespace attn_impl
