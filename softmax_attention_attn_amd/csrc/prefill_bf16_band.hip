// prefill_bf16_band.hip -- sliding-window attention forward for bf16 on gfx950:
// one key band in LDS per workgroup, every query head of a GQA group served from it.
//
// With a causal window of W keys (the StreamingLLM-style local attention of
// "Attention Sink LLM..." section 1) a block of 32 consecutive query positions
// sees at most W + 31 keys, the same band for all Hq/Hkv query heads that share
// a key/value head ("SDPA란 무엇인가?" section 5).  A workgroup takes one kv head
// and a run of QPW consecutive 32-position query blocks; its four waves split the
// group's query heads.  The keys live in a ring of 32-row blocks in LDS (K and V,
// LDS-direct buffer loads, rows past the slice end read as zeros): the first
// block's band is loaded once, and while the waves compute block b the 32 keys
// block b+1 adds and its Q rows are already on their way (one barrier per
// block), so HBM latency is exposed once per workgroup.  Per (head, block) a wave
// forms S^T = K * Q^T for every 32-key block of its part of the band
// (v_mfma_f32_32x32x16_bf16, one query per lane as in prefill_bf16.hip), so the
// whole row of logits is in registers: one max (with the sink logit of
// "Attention Sink" section 4.2), one pass of exp2 and sums, bf16 weights
// straight into O^T = V^T * P^T -- no running rescale and no per-tile loop.
// Only the key blocks on the band's two edges (window start, causal diagonal)
// carry the visibility mask.
//
// Scope (the caller checks it): bf16, dot logits, causal, 0 < W <= 128, E = 64,
// Hq/Hkv = 4 or 8, no register tokens, no key lengths, no user bias.
#include "device_common.h"
#include "kernels.h"
#include "tile_common.h"

using namespace attn_dev;

namespace {

constexpr int E = 64;
constexpr int NT = 256;             // four waves
constexpr int QB = 32;              // query positions per block (one MFMA column block)
constexpr int KB = 32;              // keys per key block
constexpr int WMAX = 128;           // longest window this kernel takes
constexpr int NKB = (WMAX + QB - 1 + KB - 1) / KB + 1;  // key blocks one query block can touch: 6
constexpr int NRING = NKB + 1;      // ring slots: the blocks in use plus the one being loaded
constexpr int QPW = 2;              // query blocks per workgroup
constexpr int ROWB = E * 2;
constexpr int BLKB = KB * ROWB;     // bytes of one 32-row block of K (or V)
constexpr int ECH = E / 8;
constexpr int OSTR = E + 8;

struct BandParams {
  const uint16_t* q;
  const uint16_t* k;
  const uint16_t* v;
  uint16_t* o;
  float* lse;
  const float* sink;
  int N, Hq, Hkv, L, S, off, window;
  float c_logit;
  int num_groups;   // workgroups per (batch, kv head): ceil(L / (32 * QPW))
  int xcd_groups;   // 1: each XCD takes whole kv heads
};

// PPW: query heads per wave (Hq/Hkv / 4).
template <int PPW, bool FAST>
__global__ __launch_bounds__(NT) __attribute__((amdgpu_waves_per_eu(2, 2)))
void prefill_band_kernel(BandParams p) {
  __shared__ __attribute__((aligned(16))) uint8_t sK[NRING * BLKB];
  __shared__ __attribute__((aligned(16))) uint8_t sV[NRING * BLKB];
  __shared__ __attribute__((aligned(16))) uint16_t sO[4][QB * OSTR];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l32 = lane & 31, g = lane >> 5;

  // Workgroup -> (batch n, kv head kh, first query block).  With xcd_groups the
  // workgroups of one kv head all run on one XCD (ids congruent mod 8), in order
  // of position, so neighbouring bands meet in its L2.
  const int U = p.N * p.Hkv;
  int u, grp;
  if (p.xcd_groups) {
    const int x = blockIdx.x & 7, y = blockIdx.x >> 3;
    const int per = U >> 3;
    grp = y / per;
    u = (y - grp * per) * 8 + x;
  } else {
    u = blockIdx.x % U;
    grp = blockIdx.x / U;
  }
  const int n = u / p.Hkv, kh = u - n * p.Hkv;
  const int G = p.Hq / p.Hkv;

  const size_t kvoff = ((size_t)n * p.Hkv + kh) * (size_t)p.S * E;
  const __amdgpu_buffer_rsrc_t krs = make_rsrc(p.k + kvoff, (uint32_t)p.S * ROWB);
  const __amdgpu_buffer_rsrc_t vrs = make_rsrc(p.v + kvoff, (uint32_t)p.S * ROWB);

  // Key block kb (keys 32 kb ..) lives in ring slot kb % NRING.  Each wave moves
  // 8 of its 32 rows per tensor: lane l takes row 8 wave + l/8, logical chunk
  // (l % 8) ^ swz(row), landing at physical chunk l % 8 (conflict-free reads).
  auto load_block = [&](int kb) __attribute__((always_inline)) {
    const int slot = kb % NRING;
    const int row = 8 * wave + lane / ECH;
    const uint32_t soff = (uint32_t)((kb * KB + row) * ROWB + (((lane % ECH) ^ tile_swz<E>(row)) * 16));
    buffer_load16_to_lds(krs, sK + slot * BLKB + 8 * wave * ROWB, soff);
    buffer_load16_to_lds(vrs, sV + slot * BLKB + 8 * wave * ROWB, soff);
  };
  // Keys query block qb sees: real positions [lo_b, hi_b]; blocks lo_b/32 .. hi_b/32.
  auto key_range = [&](int qb, int& lo_b, int& hi_b) __attribute__((always_inline)) {
    const int qa = qb * QB;
    const int qlast = min(qa + QB - 1, p.L - 1);
    hi_b = min(p.S - 1, qlast + p.off);
    lo_b = max(0, qa + p.off - p.window + 1);
  };
  // Q rows of query block qb for this wave's pp-th query head.
  auto load_q = [&](int qb, int pp, bf16x8 (&qf)[4]) __attribute__((always_inline)) {
    const int qi = min(qb * QB + l32, p.L - 1);
    const int h = kh * G + wave + 4 * pp;
    const uint16_t* qrow = p.q + (((size_t)n * p.Hq + h) * p.L + qi) * E;
#pragma unroll
    for (int s = 0; s < 4; ++s) qf[s] = as_bf16x8(*reinterpret_cast<const u32x4*>(qrow + 16 * s + 8 * g));
  };

  const uint32_t krd[4] = {
      (uint32_t)(l32 * ROWB + (((0 + g) ^ tile_swz<E>(l32)) * 16)),
      (uint32_t)(l32 * ROWB + (((2 + g) ^ tile_swz<E>(l32)) * 16)),
      (uint32_t)(l32 * ROWB + (((4 + g) ^ tile_swz<E>(l32)) * 16)),
      (uint32_t)(l32 * ROWB + (((6 + g) ^ tile_swz<E>(l32)) * 16))};
  uint32_t vrd[2][2];
  {
    const int q16 = lane >> 4, m16 = lane & 15;
#pragma unroll
    for (int c = 0; c < 2; ++c)
#pragma unroll
      for (int hh = 0; hh < 2; ++hh) {
        const int row = 4 * (q16 >> 1) + (m16 >> 2) + 8 * hh;
        const int d = 32 * c + 16 * (q16 & 1) + 4 * (m16 & 3);
        vrd[c][hh] = (uint32_t)(row * ROWB + (((d >> 3) ^ tile_swz<E>(row)) * 16) + (d & 7) * 2);
      }
  }

  // One (query head h, query block at row qa) on this wave: all its logits, one
  // softmax, PV, and the stores.
  auto compute_pair = [&](int h, int qa, int lo_b, int hi_b, const bf16x8 (&qf)[4]) __attribute__((always_inline)) {
    const int qi = qa + l32;
    const bool qvalid = qi < p.L;
    const int qlast = min(qa + QB - 1, p.L - 1);
    const int kb_lo = lo_b / KB;
    const int nj = hi_b >= lo_b ? min(NKB, hi_b / KB - kb_lo + 1) : 0;
    const int ip = qi + p.off;
    const int lo = ip - p.window + 1, hi = min(ip, p.S - 1);

    f32x16 st[NKB];
#pragma unroll
    for (int j = 0; j < NKB; ++j) {
#pragma unroll
      for (int r = 0; r < 16; ++r) st[j][r] = 0.f;
      if (j < nj) {
        const uint8_t* kt = sK + ((kb_lo + j) % NRING) * BLKB;
        __builtin_amdgcn_s_setprio(1);
#pragma unroll
        for (int s = 0; s < 4; ++s) {
          const bf16x8 a = *reinterpret_cast<const bf16x8*>(kt + krd[s]);
          st[j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qf[s], st[j], 0, 0, 0);
        }
        __builtin_amdgcn_s_setprio(0);
      }
    }

    // Logits (FAST keeps raw scores), the edge masks, one row max.
    float mx = kNegInf;
#pragma unroll
    for (int j = 0; j < NKB; ++j) {
      if (j < nj) {
        const int base = (kb_lo + j) * KB;  // real position of the block's key 0
        // whole for every row of the block when its keys lie in [qlast + off - W + 1, qa + off]
        const bool whole = base >= qlast + p.off - p.window + 1 && base + KB - 1 <= qa + p.off;
        if (whole) {
          if (!FAST) {
#pragma unroll
            for (int r = 0; r < 16; ++r) st[j][r] *= p.c_logit;
          }
        } else {
          // this lane's visible offsets within the block; the empty asm keeps the
          // comparisons here (hoisted, the 16 x NKB lane masks would not fit the
          // scalar registers)
          int lo_r = lo - base - 4 * g, hi_r = hi - base - 4 * g;
          asm volatile("" : "+v"(lo_r), "+v"(hi_r));
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int ko = 8 * (r >> 2) + (r & 3);
            const float x = FAST ? st[j][r] : st[j][r] * p.c_logit;
            st[j][r] = (ko >= lo_r && ko <= hi_r) ? x : kNegInf;
          }
        }
#pragma unroll
        for (int r = 0; r < 16; r += 2) mx = fmaxf(fmaxf(mx, st[j][r]), st[j][r + 1]);
      }
    }
    mx = pair32_max(mx);
    if (FAST) mx = (mx == kNegInf) ? kNegInf : mx * p.c_logit;
    float sink2 = kNegInf;
    if (p.sink) sink2 = p.sink[h] * kLog2e;
    const float M = fmaxf(mx, sink2);
    const float Mu = (M == kNegInf) ? 0.f : M;

    f32x16 acc[2];
#pragma unroll
    for (int c = 0; c < 2; ++c)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[c][r] = 0.f;
    float lsum = (p.sink && g == 0) ? fast_exp2(sink2 - Mu) : 0.f;
#pragma unroll
    for (int j = 0; j < NKB; ++j) {
      if (j < nj) {
        const uint8_t* vt_s = sV + ((kb_lo + j) % NRING) * BLKB;
        float ps = 0.f;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const float w = FAST ? fast_exp2(__builtin_fmaf(st[j][r], p.c_logit, -Mu)) : fast_exp2(st[j][r] - Mu);
          st[j][r] = w;
          ps += w;
        }
        lsum += ps;
        __builtin_amdgcn_s_setprio(1);
#pragma unroll
        for (int s2 = 0; s2 < 2; ++s2) {
          const bf16x8 pf = pack_bf16x8(st[j][8 * s2 + 0], st[j][8 * s2 + 1], st[j][8 * s2 + 2], st[j][8 * s2 + 3],
                                        st[j][8 * s2 + 4], st[j][8 * s2 + 5], st[j][8 * s2 + 6], st[j][8 * s2 + 7]);
#pragma unroll
          for (int c = 0; c < 2; ++c) {
            const shortx4 lo4 = lds_read_tr(vt_s + vrd[c][0] + 16 * s2 * ROWB);
            const shortx4 hi4 = lds_read_tr(vt_s + vrd[c][1] + 16 * s2 * ROWB);
            const bf16x8 vt = __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo4, hi4, 0, 1, 2, 3, 4, 5, 6, 7));
            acc[c] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vt, pf, acc[c], 0, 0, 0);
          }
        }
        __builtin_amdgcn_s_setprio(0);
      }
    }

    // Epilogue: O = acc / l through this wave's LDS rows (whole-row stores), LSE.
    const float ltot = pair32_sum(lsum);
    const float inv = ltot > 0.f ? 1.f / ltot : 0.f;
    uint16_t* so = sO[wave];
#pragma unroll
    for (int c = 0; c < 2; ++c)
#pragma unroll
      for (int rq = 0; rq < 4; ++rq) {
        const bf16x4 pk = pack_bf16x4(acc[c][4 * rq + 0] * inv, acc[c][4 * rq + 1] * inv, acc[c][4 * rq + 2] * inv,
                                      acc[c][4 * rq + 3] * inv);
        *reinterpret_cast<bf16x4*>(&so[l32 * OSTR + 32 * c + 8 * rq + 4 * g]) = pk;
      }
    const size_t obase = ((size_t)n * p.Hq + h) * p.L;
    if (g == 0 && qvalid) p.lse[obase + qi] = ltot > 0.f ? (M + log2f(ltot)) * kLn2 : kNegInf;
    // the staging rows are this wave's own: wait for its LDS writes, then read them back
    __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0)
    __builtin_amdgcn_wave_barrier();
#pragma unroll
    for (int it = 0; it < (QB * ECH) / 64; ++it) {
      const int id = lane + 64 * it;
      const int rloc = id / ECH, c = id % ECH;
      const int row = qa + rloc;
      if (row < p.L) {
        const u32x4 val = *reinterpret_cast<const u32x4*>(&so[rloc * OSTR + 8 * c]);
        *reinterpret_cast<u32x4*>(p.o + (obase + row) * E + 8 * c) = val;
      }
    }
    __builtin_amdgcn_s_waitcnt(0xc07f);  // reads done before the next pair overwrites the rows
    __builtin_amdgcn_wave_barrier();
  };

  // First block: its whole band, and the Q rows of this wave's first head.
  const int qb0 = grp * QPW;
  const int nqb = min(QPW, (p.L + QB - 1) / QB - qb0);  // query blocks of this workgroup (>= 1)
  int lo_b, hi_b;
  key_range(qb0, lo_b, hi_b);
  int loaded_hi = -1;  // highest key block loaded so far (the bands only move forward)
  if (hi_b >= lo_b) {
    for (int kb = lo_b / KB; kb <= hi_b / KB; ++kb) load_block(kb);
    loaded_hi = hi_b / KB;
  }
  bf16x8 qcur[4], qnext[4];
  load_q(qb0, 0, qcur);
  __builtin_amdgcn_s_waitcnt(0x0f70);  // vmcnt(0)
  __syncthreads();

  for (int b = 0; b < nqb; ++b) {
    // Block b+1: the keys it adds, loaded while block b is computed.
    int lo_n = 0, hi_n = -1;
    if (b + 1 < nqb) {
      key_range(qb0 + b + 1, lo_n, hi_n);
      if (hi_n >= lo_n) {
        for (int kb = max(loaded_hi + 1, lo_n / KB); kb <= hi_n / KB; ++kb) load_block(kb);
        loaded_hi = max(loaded_hi, hi_n / KB);
      }
    }
#pragma unroll 1
    for (int pp = 0; pp < PPW; ++pp) {
      // the next (head, block) pair's Q rows, one pair ahead
      if (pp + 1 < PPW)
        load_q(qb0 + b, pp + 1, qnext);
      else if (b + 1 < nqb)
        load_q(qb0 + b + 1, 0, qnext);
      compute_pair(kh * G + wave + 4 * pp, (qb0 + b) * QB, lo_b, hi_b, qcur);
#pragma unroll
      for (int s = 0; s < 4; ++s) qcur[s] = qnext[s];
    }
    lo_b = lo_n;
    hi_b = hi_n;
    __builtin_amdgcn_s_waitcnt(0x0f70);  // vmcnt(0): this wave's part of block b+1 landed
    __syncthreads();
  }
}

template <int PPW>
hipError_t launch_band(const BandParams& p, bool fast, hipStream_t stream) {
  const long long blocks = (long long)p.num_groups * p.N * p.Hkv;
  if (fast)
    hipLaunchKernelGGL((prefill_band_kernel<PPW, true>), dim3((unsigned)blocks), dim3(NT), 0, stream, p);
  else
    hipLaunchKernelGGL((prefill_band_kernel<PPW, false>), dim3((unsigned)blocks), dim3(NT), 0, stream, p);
  return hipGetLastError();
}

}  // namespace

namespace attn_impl {

bool prefill_band_fits(const FwdArgs& a) {
  const int G = a.Hq / a.Hkv;
  return a.E == E && !a.rbf && a.causal && a.window > 0 && a.window <= WMAX && a.n_reg == 0 && !a.key_len &&
         !a.bias && a.L > 0 && (G == 4 || G == 8);
}

hipError_t launch_prefill_bf16_band(const FwdArgs& a, hipStream_t stream) {
  BandParams p;
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
  p.off = a.S - a.L;
  p.window = a.window;
  p.c_logit = a.scale * 1.4426950408889634f;
  p.num_groups = (a.L + QB * QPW - 1) / (QB * QPW);
  p.xcd_groups = ((a.N * a.Hkv) % 8 == 0) ? 1 : 0;
  const bool fast = p.c_logit > 0.f;
  if (a.Hq / a.Hkv == 8) return launch_band<2>(p, fast, stream);
  return launch_band<1>(p, fast, stream);
}

}  // namespace attn_impl
