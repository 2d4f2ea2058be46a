// prefill_bf16.hip -- fused tiled attention forward for bf16 inputs on gfx950.
//
// One workgroup = 4 waves = 128 query rows of one (batch, query head); each
// wave owns 32 rows.  Keys are streamed in tiles of 64 through LDS; the score
// tile is never written to memory (the tiling + online softmax of the
// FlashAttention row in "어텐션 메커니즘" section 6, and the running max /
// running sum described in "SDPA란 무엇인가?" section 2).
//
// Orientation.  Each wave computes S^T = K * Q^T with v_mfma_f32_32x32x16_bf16
// (A = 32 keys x 16 head-dims from LDS, B = the wave's Q^T held in VGPRs), so in
// the accumulator layout every lane holds ONE query (column) and 16 keys.  The
// row max and the rescale factor are then per-lane scalars; only one exchange
// with lane^32 (the other half of the same query's keys) is needed per tile.
// The output is accumulated the same way, O^T = V^T * P^T: P^T comes straight
// from the S^T registers (rounded to bf16), V^T is read from an LDS copy of the
// V tile that was transposed while staging, with its keys permuted into the
// order in which the S^T accumulator hands them to each lane.
//
// Logits are kept in log2 units: x = c_logit * (q.k) + c_bias * |k|^2 with
//   dot: c_logit = scale*log2(e),     c_bias = 0
//   rbf: c_logit = 2*gamma*log2(e),   c_bias = -gamma*log2(e)
// i.e. the RBF logit -gamma|q-k|^2 with -gamma|q|^2 dropped by shift invariance
// (RBF-attention digest, section details paragraph 2); |k|^2 is formed from the
// staged key tile on chip (same digest, paragraph 3).  The sink logit seeds the
// running state (m = s_h, l = 1: "Attention Sink" section 4.2 -- in the
// denominator, no value), shifted by gamma|q|^2 in RBF mode so that it competes
// in the same frame; the LSE is reported for the unfolded logits.
//
// Pipeline.  K and V^T tiles are double-buffered in LDS: while tile t is
// consumed from one buffer, tile t+1 (loaded into registers one tile earlier)
// is written to the other, so one barrier per tile suffices.  Two workgroups
// share a CU (2 waves per SIMD), so one wave's softmax overlaps the other's
// MFMAs.  The running max moves lazily: the accumulator is rescaled only when
// a row max grows by more than 2^8 over the reference (O = acc / l does not
// depend on the reference; it only bounds p by 256).  With a positive scale the
// dot-mode max is taken on the raw scores and each weight costs one fma + exp2.
// The epilogue transposes O through LDS so that stores are whole rows.
#include <type_traits>

#include "device_common.h"
#include "kernels.h"

using namespace attn_dev;

namespace {

constexpr int BM = 128;  // query rows per workgroup
constexpr int BN = 64;   // keys per staged tile
constexpr int NT = 256;  // threads per workgroup
constexpr float kLazy = 8.f;  // rescale when a row max grows by more than this (log2 units)

struct PrefillParams {
  const uint16_t* q;
  const uint16_t* k;
  const uint16_t* v;
  uint16_t* o;
  float* lse;
  const float* sink;
  int N, Hq, Hkv, L, S, n_reg, S_real, off, causal, window;
  float c_logit, c_bias, gamma;
  int num_q_tiles;
  int xcd_groups;   // 1: the 8 XCDs each take whole K/V heads (needs N*Hkv % 8 == 0)
  int heavy_first;  // 1: causal, dispatch the query tiles with the most keys first
};

// Workgroup id -> (query tile, batch, head).  Workgroups are handed to the 8
// XCDs round-robin (id % 8), and each XCD has its own L2: with xcd_groups all
// query heads that read one K/V head land on the same XCD.
__device__ __forceinline__ void map_block(int bid, const PrefillParams& p, int& qt, int& n, int& h) {
  const int G = p.Hq / p.Hkv;
  int qt_rev;
  if (p.xcd_groups) {
    const int U = p.N * p.Hkv;
    const int x = bid & 7, y = bid >> 3;
    const int per = (U >> 3) * G;
    qt_rev = y / per;
    const int rest = y - qt_rev * per;
    const int ul = rest / G;
    const int u = ul * 8 + x;
    n = u / p.Hkv;
    h = (u - n * p.Hkv) * G + (rest - ul * G);
  } else {
    const int per = p.N * p.Hq;
    qt_rev = bid / per;
    const int nh = bid - qt_rev * per;
    n = nh / p.Hq;
    h = nh - n * p.Hq;
  }
  qt = p.heavy_first ? (p.num_q_tiles - 1 - qt_rev) : qt_rev;
}

// Softmax front end, fixed per launch:
//   kDotPos: dot mode, scale > 0 -- max over raw scores, weight = exp2(fma(s, c, -m));
//   kDotAny: dot mode, any finite scale -- x = c*s first;
//   kRbf:    x = c*s + bias_k with bias_k = -gamma*log2(e)*|k|^2 from the staged tile.
enum { kDotPos = 0, kDotAny = 1, kRbf = 2 };

// Waves per SIMD the register budget allows: E = 128 needs ~230 VGPRs (2 waves),
// E = 64 fits under 168 (3 waves, i.e. 3 workgroups per CU).
template <int E>
struct Occupancy {
  static constexpr int kWaves = E == 64 ? 3 : 2;
};

template <int E, int MODE>
__global__ __launch_bounds__(NT) __attribute__((amdgpu_waves_per_eu(Occupancy<E>::kWaves, Occupancy<E>::kWaves)))
void prefill_bf16_kernel(PrefillParams p) {
  constexpr bool RBF = MODE == kRbf;
  constexpr bool FAST = MODE == kDotPos;
  constexpr int KSTR = E + 8;   // K tile row stride (elements): +16 B against bank conflicts
  constexpr int VSTR = BN + 8;  // V^T tile row stride (elements)
  constexpr int OSTR = E + 8;   // epilogue O row stride (elements)
  constexpr int QS = E / 16;    // MFMA steps over the head dimension
  constexpr int EB = E / 32;    // 32-row blocks of O^T
  constexpr int NB = BN / 32;   // 32-key blocks of S^T per tile
  constexpr int ECH = E / 8;    // 16-byte chunks per row
  constexpr int KCH = BN * ECH / NT;          // K chunks staged per thread
  constexpr int VTHREADS = (BN / 4) * ECH;    // threads staging a 4-key x 8-dim block of V
  constexpr int KTILE = BN * KSTR;
  constexpr int VTILE = E * VSTR;
  static_assert(KCH * NT == BN * ECH, "K staging must tile evenly");
  static_assert(VTHREADS <= NT, "V staging needs at most one block per thread");
  static_assert(BM * OSTR <= 2 * (KTILE + VTILE), "epilogue staging must fit the tile buffers");

  __shared__ __attribute__((aligned(16))) uint16_t sKV[2 * (KTILE + VTILE)];
  __shared__ __attribute__((aligned(16))) float sBias[2][BN];
  uint16_t* const sK = sKV;                // [2][KTILE]
  uint16_t* const sVT = sKV + 2 * KTILE;   // [2][VTILE]

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform per wave
  const int l32 = lane & 31, g = lane >> 5;

  int qt, n, h;
  map_block(blockIdx.x, p, qt, n, h);
  const int G = p.Hq / p.Hkv;
  const int kh = h / G;
  const int i0 = qt * BM;
  const int qa = i0 + wave * 32;          // first query row of this wave
  const int qi = qa + l32;                // this lane's query row
  const bool qvalid = qi < p.L;
  const int qb = min(qa + 31, p.L - 1);   // last valid row of this wave (qb < qa: none)

  // Q^T fragments: lane holds Q[qi][16s + 8g .. +8] for every step s.  Rows past
  // the end read the last row instead (their results are never stored).
  const uint16_t* qrow = p.q + (((size_t)n * p.Hq + h) * p.L + min(qi, p.L - 1)) * E;
  bf16x8 qf[QS];
  float qn2 = 0.f;
#pragma unroll
  for (int s = 0; s < QS; ++s) {
    const u32x4 c = *reinterpret_cast<const u32x4*>(qrow + 16 * s + 8 * g);
    qf[s] = as_bf16x8(c);
    if (RBF) qn2 += sumsq8(c);
  }
  if (RBF) qn2 = pair32_sum(qn2);

  // Running state in log2 units: m is the reference max, lsum this lane's share
  // of the row sum (its 16 keys per block); the halves are added at the end.
  float m = kNegInf, lsum = 0.f;
  if (p.sink) {
    float s0 = p.sink[h];
    if (RBF) s0 += p.gamma * qn2;
    m = s0 * kLog2e;
    lsum = (g == 0) ? 1.f : 0.f;
  }
  f32x16 acc[EB];
#pragma unroll
  for (int c = 0; c < EB; ++c)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[c][r] = 0.f;

  // Tiles: register rows first, then the real keys some row of this workgroup sees.
  const int i_last = min(i0 + BM, p.L) - 1;
  const int r_hi = p.causal ? min(p.S_real - 1, i_last + p.off) : p.S_real - 1;
  const int r_lo = p.window > 0 ? max(0, i0 + p.off - p.window + 1) : 0;
  const int n_real_tiles = r_hi >= r_lo ? (r_hi - r_lo + BN) / BN : 0;
  const int n_reg_tiles = (p.n_reg + BN - 1) / BN;
  const int T = n_reg_tiles + n_real_tiles;

  // K and V of this (batch, kv head): one buffer resource each over exactly the
  // S rows of the slice, so rows past the end load as zeros.
  const size_t kvoff = ((size_t)n * p.Hkv + kh) * (size_t)p.S * E;
  const __amdgpu_buffer_rsrc_t krs = make_rsrc(p.k + kvoff, (uint32_t)p.S * E * 2);
  const __amdgpu_buffer_rsrc_t vrs = make_rsrc(p.v + kvoff, (uint32_t)p.S * E * 2);

  // Staging roles.  K: chunk id = tid + NT*i is row id/ECH, dims 8*(id%ECH)..+8.
  // V: thread (va, vc) stages rows 4va..4va+3, dims 8vc..8vc+7, transposed.
  const int va = tid % (BN / 4), vc = tid / (BN / 4);
  const bool vrole = tid < VTHREADS;
  // Position of key quad va in the permuted V^T row: within each 16-key group the
  // order is keys {0-3, 8-11, 4-7, 12-15}, i.e. lane half g of the PV operand
  // reads keys {4g..4g+3, 8+4g..8+4g+3} as 8 consecutive elements.
  const int vpos = 16 * (va >> 2) + ((va & 1) ? 8 : 0) + ((va & 2) ? 4 : 0);

  u32x4 kreg[KCH], vreg[4];

  auto tile_keys = [&](int t, int& j0, int& kc) {
    if (t < n_reg_tiles) {
      j0 = t * BN;
      kc = min(BN, p.n_reg - j0);
    } else {
      j0 = p.n_reg + r_lo + (t - n_reg_tiles) * BN;
      kc = min(BN, p.S - j0);
    }
  };

  // Byte offsets within a tile of this thread's K chunks and V rows.  Rows past
  // the tile's last key are loaded anyway (they are real keys of the slice, or
  // zeros past its end) and masked in the softmax.
  uint32_t koff[KCH], voff[4];
#pragma unroll
  for (int i = 0; i < KCH; ++i) {
    const int id = tid + NT * i;
    koff[i] = (uint32_t)((id / ECH) * E * 2 + 16 * (id % ECH));
  }
#pragma unroll
  for (int ii = 0; ii < 4; ++ii) voff[ii] = (uint32_t)((4 * va + ii) * E * 2 + 16 * vc);

  auto load_tile = [&](int t) {
    int j0, kc;
    tile_keys(t, j0, kc);
    const uint32_t tb = (uint32_t)j0 * E * 2;
#pragma unroll
    for (int i = 0; i < KCH; ++i) kreg[i] = buffer_load16(krs, tb + koff[i]);
    if (vrole) {
#pragma unroll
      for (int ii = 0; ii < 4; ++ii) vreg[ii] = buffer_load16(vrs, tb + voff[ii]);
    }
  };

  auto store_tile = [&](int buf) {
    uint16_t* k_s = sK + buf * KTILE;
    uint16_t* v_s = sVT + buf * VTILE;
#pragma unroll
    for (int i = 0; i < KCH; ++i) {
      const int id = tid + NT * i;
      const int row = id / ECH, c = id % ECH;
      *reinterpret_cast<u32x4*>(&k_s[row * KSTR + 8 * c]) = kreg[i];
      if (RBF) {
        // |k|^2 of this key row: its ECH chunks sit in ECH consecutive lanes.
        const float ss = group_sum<ECH>(sumsq8(kreg[i]));
        if (c == 0) sBias[buf][row] = p.c_bias * ss;
      }
    }
    if (vrole) {
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const int w = j >> 1;
        const bool hi = j & 1;
        u32x2 d = {pack_halves(vreg[0][w], vreg[1][w], hi), pack_halves(vreg[2][w], vreg[3][w], hi)};
        *reinterpret_cast<u32x2*>(&v_s[(8 * vc + j) * VSTR + vpos]) = d;
      }
    }
  };

  // MASKED is a compile-time flag: false only for tiles every row of the
  // workgroup sees completely, whose code then carries no visibility test.
  auto compute_tile = [&](int t, int buf, auto masked_tag) {
    constexpr bool MASKED = decltype(masked_tag)::value;
    int j0, kc;
    tile_keys(t, j0, kc);
    const bool is_reg = t < n_reg_tiles;
    bool any, full;
    if (!MASKED) {
      any = qb >= qa;
      full = true;
    } else if (qb < qa) {
      any = false;
      full = false;
    } else if (is_reg) {
      any = true;
      full = (kc == BN);
    } else {
      const int ra = j0 - p.n_reg, rb = ra + BN - 1;
      any = !((ra >= p.S_real) || (p.causal && ra > qb + p.off) ||
              (p.window > 0 && qa + p.off - rb >= p.window));
      full = rb < p.S_real && (!p.causal || rb <= qa + p.off) &&
             (p.window <= 0 || qb + p.off - ra < p.window);
    }
    if (!any) return;
    const uint16_t* k_s = sK + buf * KTILE;
    const uint16_t* v_s = sVT + buf * VTILE;

    // S^T = K * Q^T for NB blocks of 32 keys; the NB accumulation chains are
    // interleaved so that consecutive MFMAs never depend on each other.
    f32x16 st[NB];
#pragma unroll
    for (int b = 0; b < NB; ++b)
#pragma unroll
      for (int r = 0; r < 16; ++r) st[b][r] = 0.f;
#pragma unroll
    for (int s = 0; s < QS; ++s) {
      bf16x8 a[NB];
#pragma unroll
      for (int b = 0; b < NB; ++b)
        a[b] = *reinterpret_cast<const bf16x8*>(&k_s[(32 * b + l32) * KSTR + 16 * s + 8 * g]);
#pragma unroll
      for (int b = 0; b < NB; ++b) st[b] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[b], qf[s], st[b], 0, 0, 0);
    }

    // Accumulator row of register r in block b = key 32b + 8(r/4) + 4g + r%4 of
    // the tile.  FAST keeps raw scores (the scale goes into the exponent);
    // otherwise the scores become log2-unit logits here.
    if (!FAST) {
#pragma unroll
      for (int b = 0; b < NB; ++b)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          float x = st[b][r] * p.c_logit;
          if (RBF) x += sBias[buf][32 * b + 8 * (r >> 2) + 4 * g + (r & 3)];
          st[b][r] = x;
        }
    }
    if (MASKED && !full) {
      // Visible keys of this lane's row form one interval [lo, hi] of tile
      // offsets; the offset of register r is its compile-time key minus 4g.
      int lo, hi;
      if (is_reg) {
        lo = 0;
        hi = kc - 1;
      } else {
        const int base = j0 - p.n_reg;  // real position of tile key 0
        const int ip = qi + p.off;      // this row's aligned position
        hi = min(p.S_real - 1, p.causal ? ip : p.S_real - 1) - base;
        lo = (p.window > 0 ? ip - p.window + 1 : 0) - base;
      }
      lo -= 4 * g;
      hi -= 4 * g;
#pragma unroll
      for (int b = 0; b < NB; ++b)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int ko = 32 * b + 8 * (r >> 2) + (r & 3);
          const bool vis = (ko >= lo) & (ko <= hi);
          st[b][r] = vis ? st[b][r] : kNegInf;
        }
    }
    float mx = kNegInf;
#pragma unroll
    for (int b = 0; b < NB; ++b)
#pragma unroll
      for (int r = 0; r < 16; r += 2) mx = fmaxf(mx, fmaxf(st[b][r], st[b][r + 1]));
    mx = pair32_max(mx);
    if (FAST) mx = (mx == kNegInf) ? kNegInf : mx * p.c_logit;

    // Lazy reference max: move it (and rescale) only when a row max would grow
    // by more than kLazy; otherwise weights stay below 2^kLazy.
    if (__any(mx > m + kLazy)) {
      const float m_new = fmaxf(m, mx);
      const float alpha = (m_new == kNegInf) ? 1.f : fast_exp2(m - m_new);
      m = m_new;
      lsum *= alpha;
#pragma unroll
      for (int c = 0; c < EB; ++c)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[c][r] *= alpha;
    }
    const float m_use = (m == kNegInf) ? 0.f : m;

    float ps = 0.f;
#pragma unroll
    for (int b = 0; b < NB; ++b)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const float pv = FAST ? fast_exp2(__builtin_fmaf(st[b][r], p.c_logit, -m_use))
                              : fast_exp2(st[b][r] - m_use);
        st[b][r] = pv;
        ps += pv;
      }
    lsum += ps;

    // O^T += V^T * P^T, 16 keys per MFMA step.
#pragma unroll
    for (int b = 0; b < NB; ++b) {
#pragma unroll
      for (int s2 = 0; s2 < 2; ++s2) {
        const int r0 = 8 * s2;
        const bf16x8 pf = pack_bf16x8(st[b][r0 + 0], st[b][r0 + 1], st[b][r0 + 2], st[b][r0 + 3],
                                      st[b][r0 + 4], st[b][r0 + 5], st[b][r0 + 6], st[b][r0 + 7]);
        const int u = 2 * b + s2;
#pragma unroll
        for (int c = 0; c < EB; ++c) {
          const bf16x8 vt = *reinterpret_cast<const bf16x8*>(&v_s[(32 * c + l32) * VSTR + 16 * u + 8 * g]);
          acc[c] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vt, pf, acc[c], 0, 0, 0);
        }
      }
    }
  };

  // Tile t lives in buffer t % 2.  Iteration t computes it while tile t+1
  // (already in registers) goes to the other buffer and tile t+2 is loaded.
  // Real tiles k in [k_full0, k_full1] are seen completely by every row of the
  // workgroup and run without visibility code; the tiles before and after them
  // (and the register tiles) run with it.
  int k_full0 = 0, k_full1 = -1;
  {
    const int lim = min(p.S_real - 1, p.causal ? i0 + p.off : p.S_real - 1);
    k_full1 = (lim - r_lo - (BN - 1)) >= 0 ? (lim - r_lo - (BN - 1)) / BN : -1;
    if (p.window > 0) {
      const int need = i_last + p.off - p.window + 1 - r_lo;  // first ra allowed
      k_full0 = need > 0 ? (need + BN - 1) / BN : 0;
    }
    k_full1 = min(k_full1, n_real_tiles - 1);
    if (k_full0 > k_full1) {
      k_full0 = 0;
      k_full1 = -1;
    }
  }
  const int t_full0 = n_reg_tiles + k_full0, t_full1 = n_reg_tiles + k_full1 + 1;  // [t_full0, t_full1)

  auto step = [&](int t, auto masked_tag) {
    compute_tile(t, t & 1, masked_tag);
    if (t + 1 < T) {
      store_tile((t + 1) & 1);
      if (t + 2 < T) load_tile(t + 2);
    }
    __syncthreads();
  };

  if (T > 0) {
    load_tile(0);
    store_tile(0);
  }
  // Q and tile 0 have landed (the stores above consumed tile 0; loads return in
  // order).  Say so explicitly, so that no wait on the Q registers is left
  // inside the loop, where it would also wait for the prefetch of later tiles.
  __builtin_amdgcn_s_waitcnt(0x0f70);  // vmcnt(0); expcnt and lgkmcnt untouched
  if (T > 1) load_tile(1);
  __syncthreads();
  const int head_end = (t_full1 > t_full0) ? t_full0 : T;
  for (int t = 0; t < head_end; ++t) step(t, std::true_type{});
  for (int t = head_end; t < t_full1; ++t) step(t, std::false_type{});
  for (int t = max(head_end, t_full1); t < T; ++t) step(t, std::true_type{});

  // Epilogue: O = acc / l (0 for an empty row) staged through LDS (free after
  // the last barrier) so that global stores are whole rows; LSE in natural log.
  const float ltot = pair32_sum(lsum);
  const float inv = ltot > 0.f ? 1.f / ltot : 0.f;
  uint16_t* sO = sKV + wave * 32 * OSTR;
#pragma unroll
  for (int c = 0; c < EB; ++c)
#pragma unroll
    for (int rq = 0; rq < 4; ++rq) {
      const bf16x4 pk = pack_bf16x4(acc[c][4 * rq + 0] * inv, acc[c][4 * rq + 1] * inv,
                                    acc[c][4 * rq + 2] * inv, acc[c][4 * rq + 3] * inv);
      *reinterpret_cast<bf16x4*>(&sO[l32 * OSTR + 32 * c + 8 * rq + 4 * g]) = pk;
    }
  if (g == 0 && qvalid) {
    float l = kNegInf;
    if (ltot > 0.f) {
      l = (m + log2f(ltot)) * kLn2;
      if (RBF) l -= p.gamma * qn2;
    }
    p.lse[((size_t)n * p.Hq + h) * p.L + qi] = l;
  }
  __syncthreads();
  const size_t obase = ((size_t)n * p.Hq + h) * p.L;
#pragma unroll
  for (int it = 0; it < (32 * ECH) / 64; ++it) {
    const int id = lane + 64 * it;
    const int rloc = id / ECH, c = id % ECH;
    const int row = qa + rloc;
    if (row < p.L) {
      const u32x4 val = *reinterpret_cast<const u32x4*>(&sO[rloc * OSTR + 8 * c]);
      *reinterpret_cast<u32x4*>(p.o + (obase + row) * E + 8 * c) = val;
    }
  }
}

template <int E, int MODE>
hipError_t launch_t(const PrefillParams& p, hipStream_t stream) {
  const long long blocks = (long long)p.num_q_tiles * p.N * p.Hq;
  hipLaunchKernelGGL((prefill_bf16_kernel<E, MODE>), dim3((unsigned)blocks), dim3(NT), 0, stream, p);
  return hipGetLastError();
}

template <int E>
hipError_t launch_e(const PrefillParams& p, bool rbf, hipStream_t stream) {
  if (rbf) return launch_t<E, kRbf>(p, stream);
  if (p.c_logit > 0.f) return launch_t<E, kDotPos>(p, stream);
  return launch_t<E, kDotAny>(p, stream);
}

}  // namespace

namespace attn_impl {

hipError_t launch_prefill_bf16(const FwdArgs& a, hipStream_t stream) {
  PrefillParams p;
  p.q = static_cast<const uint16_t*>(a.q);
  p.k = static_cast<const uint16_t*>(a.k);
  p.v = static_cast<const uint16_t*>(a.v);
  p.o = static_cast<uint16_t*>(a.o);
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
  p.window = a.window;
  p.gamma = a.gamma;
  if (a.rbf) {
    p.c_logit = 2.f * a.gamma * 1.4426950408889634f;
    p.c_bias = -a.gamma * 1.4426950408889634f;
  } else {
    p.c_logit = a.scale * 1.4426950408889634f;
    p.c_bias = 0.f;
  }
  p.num_q_tiles = (a.L + BM - 1) / BM;
  p.xcd_groups = ((a.N * a.Hkv) % 8 == 0) ? 1 : 0;
  p.heavy_first = p.causal;
  if (a.E == 128) return launch_e<128>(p, a.rbf != 0, stream);
  return launch_e<64>(p, a.rbf != 0, stream);
}

}  // namespace attn_impl
