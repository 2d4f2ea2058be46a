// prefill_bf16_band.hip -- sliding-window attention forward for bf16 on gfx950:
// one key band in LDS per workgroup, every query head of a GQA group served from it.
//
// With a causal window of W keys (the StreamingLLM-style local attention of
// "Attention Sink LLM..." section 1) a block of 32 consecutive query positions
// sees at most W + 31 keys, the same band for all Hq/Hkv query heads that share
// a key/value head ("SDPA란 무엇인가?" section 5).  A workgroup takes one kv head
// and two consecutive 32-position query blocks; its four waves split the
// group's query heads.  The keys live in LDS as 32-row blocks of K and V
// (LDS-direct buffer loads, rows past the slice end read as zeros): the first
// query block's band in one pair of arrays, and the one block the second query
// block adds in another pair, loaded while the waves compute the first (the Q
// rows of the next (head, block) pair are requested ahead too), so HBM latency
// is exposed once per workgroup.  The reads of the first block's compute never
// touch the array the loads in flight write, which lets them go without
// waiting for those loads.  Per (head, block) a wave forms S^T = K * Q^T for the
// 32-key blocks of the band (v_mfma_f32_32x32x16_bf16, one query per lane as in
// prefill_bf16.hip), the row max with the sink logit of "Attention Sink"
// section 4.2, exp2 and sums, and bf16 weights straight into O^T = V^T * P^T.
// Only the key blocks on the band's two edges (window start, causal diagonal)
// carry the visibility mask.
//
// With eight query heads per kv head each wave takes two heads of a block at
// once: every K and V^T fragment read from LDS feeds both heads' MFMAs and the
// two heads' instruction streams interleave (the kernel is bound by the
// latency of each head's chain of steps, not by any one unit); the band then
// goes in chunks of two key blocks with an online softmax across chunks.  With
// four heads per kv head a wave takes one head and the whole band at once
// (all its logits in registers, one max, no rescale).
//
// Scope (the caller checks it): bf16, dot logits, causal, 0 < W <= 128, E = 64,
// Hq/Hkv = 4 or 8, no register tokens, no key lengths, no user bias.
#include <type_traits>

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
constexpr int QPW = 2;              // query blocks per workgroup (the layout below is for two)
constexpr int ROWB = E * 2;
constexpr int BLKB = KB * ROWB;     // bytes of one 32-row block of K (or V)
constexpr int ECH = E / 8;
constexpr float kLazyBand = 8.f;     // rescale when a chunk's row max exceeds the reference by more (log2)
constexpr int OSTR = E;             // O staging row stride (elements); 16-byte chunks XOR-swizzled by row

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
  __shared__ __attribute__((aligned(16))) uint8_t sK[NKB * BLKB];   // band of the first query block
  __shared__ __attribute__((aligned(16))) uint8_t sV[NKB * BLKB];
  __shared__ __attribute__((aligned(16))) uint8_t sKn[BLKB];        // the block the second one adds
  __shared__ __attribute__((aligned(16))) uint8_t sVn[BLKB];
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

  // Key block kb (keys 32 kb ..) into the 32-row LDS blocks dk, dv.  Each wave
  // moves 8 of the 32 rows per tensor: lane l takes row 8 wave + l/8, logical
  // chunk (l % 8) ^ swz(row), landing at physical chunk l % 8 (conflict-free reads).
  auto load_block = [&](int kb, uint8_t* dk, uint8_t* dv) __attribute__((always_inline)) {
    const int row = 8 * wave + lane / ECH;
    const uint32_t soff = (uint32_t)((kb * KB + row) * ROWB + (((lane % ECH) ^ tile_swz<E>(row)) * 16));
    buffer_load16_to_lds(krs, dk + 8 * wave * ROWB, soff);
    buffer_load16_to_lds(vrs, dv + 8 * wave * ROWB, soff);
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
  // softmax, PV, and the stores.  Key block kb sits in slot kb - kb0 of sK/sV
  // when that is below n0, else (second query block only) in sKn/sVn.
  auto compute_pair = [&](auto second, int h, int qa, int lo_b, int hi_b, const bf16x8 (&qf)[4], float sink2,
                          int kb0, int n0) __attribute__((always_inline)) {
    constexpr bool SECOND = decltype(second)::value;
    auto slot_k = [&](int kb) __attribute__((always_inline)) -> const uint8_t* {
      if (!SECOND) return sK + (kb - kb0) * BLKB;
      const int sl = kb - kb0;
      return (sl >= 0 && sl < n0) ? sK + sl * BLKB : sKn;
    };
    auto slot_v = [&](int kb) __attribute__((always_inline)) -> const uint8_t* {
      if (!SECOND) return sV + (kb - kb0) * BLKB;
      const int sl = kb - kb0;
      return (sl >= 0 && sl < n0) ? sV + sl * BLKB : sVn;
    };
    const int qi = qa + l32;
    const int qlast = min(qa + QB - 1, p.L - 1);
    const int kb_lo = lo_b / KB;
    const int nj = hi_b >= lo_b ? min(NKB, hi_b / KB - kb_lo + 1) : 0;
    const int ip = qi + p.off;
    const int lo = ip - p.window + 1, hi = min(ip, p.S - 1);

    // Blocks j >= nj are never read (every later loop stops at nj).
    f32x16 st[NKB];
#pragma unroll
    for (int j = 0; j < NKB; ++j) {
      if (j < nj) {
        const uint8_t* kt = slot_k(kb_lo + j);
        const f32x16 zero = {};
        __builtin_amdgcn_s_setprio(1);
#pragma unroll
        for (int s = 0; s < 4; ++s) {
          const bf16x8 a = *reinterpret_cast<const bf16x8*>(kt + krd[s]);
          st[j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qf[s], s == 0 ? zero : st[j], 0, 0, 0);
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
          // A block cut only by the window start (or only by the diagonal or
          // the slice end) tests one bound.
          int lo_r = lo - base - 4 * g, hi_r = hi - base - 4 * g;
          asm volatile("" : "+v"(lo_r), "+v"(hi_r));
          const bool cut_lo = base < qlast + p.off - p.window + 1;
          const bool cut_hi = base + KB - 1 > qa + p.off;
          if (cut_lo && cut_hi) {
#pragma unroll
            for (int r = 0; r < 16; ++r) {
              const int ko = 8 * (r >> 2) + (r & 3);
              const float x = FAST ? st[j][r] : st[j][r] * p.c_logit;
              st[j][r] = (ko >= lo_r && ko <= hi_r) ? x : kNegInf;
            }
          } else if (cut_lo) {
#pragma unroll
            for (int r = 0; r < 16; ++r) {
              const int ko = 8 * (r >> 2) + (r & 3);
              const float x = FAST ? st[j][r] : st[j][r] * p.c_logit;
              st[j][r] = ko >= lo_r ? x : kNegInf;
            }
          } else {
#pragma unroll
            for (int r = 0; r < 16; ++r) {
              const int ko = 8 * (r >> 2) + (r & 3);
              const float x = FAST ? st[j][r] : st[j][r] * p.c_logit;
              st[j][r] = ko <= hi_r ? x : kNegInf;
            }
          }
        }
#pragma unroll
        for (int r = 0; r < 16; r += 2) mx = fmaxf(fmaxf(mx, st[j][r]), st[j][r + 1]);
      }
    }
    mx = pair32_max(mx);
    if (FAST) mx = (mx == kNegInf) ? kNegInf : mx * p.c_logit;
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
        const uint8_t* vt_s = slot_v(kb_lo + j);
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
    const float inv = ltot > 0.f ? __builtin_amdgcn_rcpf(ltot) : 0.f;
    uint16_t* so = sO[wave];
#pragma unroll
    for (int c = 0; c < 2; ++c)
#pragma unroll
      for (int rq = 0; rq < 4; ++rq) {
        const bf16x4 pk = pack_bf16x4(acc[c][4 * rq + 0] * inv, acc[c][4 * rq + 1] * inv, acc[c][4 * rq + 2] * inv,
                                      acc[c][4 * rq + 3] * inv);
        *reinterpret_cast<bf16x4*>(&so[l32 * OSTR + 8 * ((4 * c + rq) ^ (l32 & 7)) + 4 * g]) = pk;
      }
    // Stores go through resources over this head's L rows: rows at or past L
    // are dropped by the range check, so no store sits behind a branch (a
    // skipped store would make the wait for the next pair's Q rows, issued
    // before these stores, wait for them as well).  Both halves of the wave
    // write the same LSE value.  O goes out with the non-temporal hint: it is
    // written once, and kept out of the caches it leaves them to the K/V bands
    // that neighbouring workgroups read again (measured 14 % faster on the
    // window-128 GQA shape).
    const size_t obase = ((size_t)n * p.Hq + h) * p.L;
    const __amdgpu_buffer_rsrc_t lrs = make_rsrc(p.lse + obase, (uint32_t)p.L * 4u);
    const __amdgpu_buffer_rsrc_t ors = make_rsrc(p.o + obase * E, (uint32_t)p.L * ROWB);
    buffer_store4(lrs, (uint32_t)qi * 4u, ltot > 0.f ? (M + __builtin_amdgcn_logf(ltot)) * kLn2 : kNegInf);
    // the staging rows are this wave's own: wait for its LDS writes, then read them back
    __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0)
    __builtin_amdgcn_wave_barrier();
#pragma unroll
    for (int it = 0; it < (QB * ECH) / 64; ++it) {
      const int id = lane + 64 * it;
      const int rloc = id / ECH, c = id % ECH;
      const u32x4 val = *reinterpret_cast<const u32x4*>(&so[rloc * OSTR + 8 * (c ^ (rloc & 7))]);
      buffer_store16_nt(ors, (uint32_t)((qa + rloc) * ROWB + 16 * c), val);
    }
    __builtin_amdgcn_s_waitcnt(0xc07f);  // reads done before the next pair overwrites the rows
    __builtin_amdgcn_wave_barrier();
  };

  // Both query heads of this wave (kh*G + wave and + 4) on one query block at
  // once: each K and V^T fragment read from LDS feeds both heads' MFMAs, and
  // the two heads' chains interleave.  The band goes in chunks of up to two
  // key blocks with an online softmax across chunks (running reference max,
  // lazy rescale as in the tiled kernel).  After the last chunk's QK^T the Q
  // registers are refilled with the next pair's rows (nq >= 0).
  auto compute_pair2 = [&](auto second, int qa, int lo_b, int hi_b, bf16x8 (&qA)[4], bf16x8 (&qB)[4],
                           float sinkA, float sinkB, int kb0, int n0, int nq) __attribute__((always_inline)) {
    constexpr bool SECOND = decltype(second)::value;
    auto slot_k = [&](int kb) __attribute__((always_inline)) -> const uint8_t* {
      if (!SECOND) return sK + (kb - kb0) * BLKB;
      const int sl = kb - kb0;
      return (sl >= 0 && sl < n0) ? sK + sl * BLKB : sKn;
    };
    auto slot_v = [&](int kb) __attribute__((always_inline)) -> const uint8_t* {
      if (!SECOND) return sV + (kb - kb0) * BLKB;
      const int sl = kb - kb0;
      return (sl >= 0 && sl < n0) ? sV + sl * BLKB : sVn;
    };
    const int hA = kh * G + wave, hB = hA + 4;
    const int qi = qa + l32;
    const int qlast = min(qa + QB - 1, p.L - 1);
    const int kb_lo = lo_b / KB;
    const int nj = hi_b >= lo_b ? min(NKB, hi_b / KB - kb_lo + 1) : 0;
    const int ip = qi + p.off;
    const int lo = ip - p.window + 1, hi = min(ip, p.S - 1);
    constexpr int CH = 2;  // key blocks per chunk
    // running state (log2 units), seeded with the sink as in the tiled kernel
    float mA = p.sink ? sinkA : kNegInf, mB = p.sink ? sinkB : kNegInf;
    float lA = (p.sink && g == 0) ? 1.f : 0.f, lB = lA;
    // Derived from the references, updated only where they move: the value a
    // half-row max (raw scores when FAST) must pass to grow the row max by more
    // than kLazyBand, and -m (0 while the row has seen nothing).
    const float inv_c = FAST ? 1.f / p.c_logit : 1.f;
    auto lazy_thr = [&](float mref) { return FAST ? (mref + kLazyBand) * inv_c : mref + kLazyBand; };
    float tA = lazy_thr(mA), tB = lazy_thr(mB);
    float nA = (mA == kNegInf) ? 0.f : -mA, nB = (mB == kNegInf) ? 0.f : -mB;
    f32x16 aA[2], aB[2];
#pragma unroll
    for (int c = 0; c < 2; ++c)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        aA[c][r] = 0.f;
        aB[c][r] = 0.f;
      }
#pragma unroll
    for (int ck = 0; ck < (NKB + CH - 1) / CH; ++ck) {
      if (ck * CH < nj) {
        f32x16 sA[CH], sB[CH];
#pragma unroll
        for (int jj = 0; jj < CH; ++jj) {
          const int j = ck * CH + jj;
          if (j < nj) {
            const uint8_t* kt = slot_k(kb_lo + j);
            const f32x16 zero = {};
            __builtin_amdgcn_s_setprio(1);
#pragma unroll
            for (int s4 = 0; s4 < 4; ++s4) {
              const bf16x8 a = *reinterpret_cast<const bf16x8*>(kt + krd[s4]);
              sA[jj] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qA[s4], s4 == 0 ? zero : sA[jj], 0, 0, 0);
              sB[jj] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qB[s4], s4 == 0 ? zero : sB[jj], 0, 0, 0);
            }
            __builtin_amdgcn_s_setprio(0);
          }
        }
        if (nq >= 0 && (ck + 1) * CH >= nj) {  // last chunk: Q no longer needed
          load_q(nq, 0, qA);
          load_q(nq, 1, qB);
        }
        // edge masks (the same for both heads) and the chunk's row maxima
        float xA = kNegInf, xB = kNegInf;
#pragma unroll
        for (int jj = 0; jj < CH; ++jj) {
          const int j = ck * CH + jj;
          if (j < nj) {
            const int base = (kb_lo + j) * KB;
            const bool whole = base >= qlast + p.off - p.window + 1 && base + KB - 1 <= qa + p.off;
            if (!FAST) {
#pragma unroll
              for (int r = 0; r < 16; ++r) {
                sA[jj][r] *= p.c_logit;
                sB[jj][r] *= p.c_logit;
              }
            }
            if (!whole) {
              int lo_r = lo - base - 4 * g, hi_r = hi - base - 4 * g;
              asm volatile("" : "+v"(lo_r), "+v"(hi_r));
#pragma unroll
              for (int r = 0; r < 16; ++r) {
                const int ko = 8 * (r >> 2) + (r & 3);
                const bool vis = (ko >= lo_r) & (ko <= hi_r);
                sA[jj][r] = vis ? sA[jj][r] : kNegInf;
                sB[jj][r] = vis ? sB[jj][r] : kNegInf;
              }
            }
#pragma unroll
            for (int r = 0; r < 16; r += 2) {
              xA = fmaxf(fmaxf(xA, sA[jj][r]), sA[jj][r + 1]);
              xB = fmaxf(fmaxf(xB, sB[jj][r]), sB[jj][r + 1]);
            }
          }
        }
        // xA, xB: this lane's half of the chunk's row max (the other half sits
        // in lane ^ 32); the whole-row max is formed only when a reference moves.
        if (__any(xA > tA)) {
          xA = pair32_max(xA);
          if (FAST) xA = (xA == kNegInf) ? kNegInf : xA * p.c_logit;
          const float mn = fmaxf(mA, xA);
          const float al = (mn == kNegInf) ? 1.f : fast_exp2(mA - mn);
          mA = mn;
          tA = lazy_thr(mA);
          nA = (mA == kNegInf) ? 0.f : -mA;
          lA *= al;
#pragma unroll
          for (int c = 0; c < 2; ++c)
#pragma unroll
            for (int r = 0; r < 16; ++r) aA[c][r] *= al;
        }
        if (__any(xB > tB)) {
          xB = pair32_max(xB);
          if (FAST) xB = (xB == kNegInf) ? kNegInf : xB * p.c_logit;
          const float mn = fmaxf(mB, xB);
          const float al = (mn == kNegInf) ? 1.f : fast_exp2(mB - mn);
          mB = mn;
          tB = lazy_thr(mB);
          nB = (mB == kNegInf) ? 0.f : -mB;
          lB *= al;
#pragma unroll
          for (int c = 0; c < 2; ++c)
#pragma unroll
            for (int r = 0; r < 16; ++r) aB[c][r] *= al;
        }
#pragma unroll
        for (int jj = 0; jj < CH; ++jj) {
          const int j = ck * CH + jj;
          if (j < nj) {
            const uint8_t* vt_s = slot_v(kb_lo + j);
            float pa = -0.f, pb = -0.f;  // (-0 + x == x: the first additions fold away)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
              const float wa = FAST ? fast_exp2(__builtin_fmaf(sA[jj][r], p.c_logit, nA)) : fast_exp2(sA[jj][r] + nA);
              const float wb = FAST ? fast_exp2(__builtin_fmaf(sB[jj][r], p.c_logit, nB)) : fast_exp2(sB[jj][r] + nB);
              sA[jj][r] = wa;
              sB[jj][r] = wb;
              pa += wa;
              pb += wb;
            }
            lA += pa;
            lB += pb;
            __builtin_amdgcn_s_setprio(1);
#pragma unroll
            for (int s2 = 0; s2 < 2; ++s2) {
              const bf16x8 fa = pack_bf16x8(sA[jj][8 * s2 + 0], sA[jj][8 * s2 + 1], sA[jj][8 * s2 + 2], sA[jj][8 * s2 + 3],
                                            sA[jj][8 * s2 + 4], sA[jj][8 * s2 + 5], sA[jj][8 * s2 + 6], sA[jj][8 * s2 + 7]);
              const bf16x8 fb = pack_bf16x8(sB[jj][8 * s2 + 0], sB[jj][8 * s2 + 1], sB[jj][8 * s2 + 2], sB[jj][8 * s2 + 3],
                                            sB[jj][8 * s2 + 4], sB[jj][8 * s2 + 5], sB[jj][8 * s2 + 6], sB[jj][8 * s2 + 7]);
#pragma unroll
              for (int c = 0; c < 2; ++c) {
                const shortx4 lo4 = lds_read_tr(vt_s + vrd[c][0] + 16 * s2 * ROWB);
                const shortx4 hi4 = lds_read_tr(vt_s + vrd[c][1] + 16 * s2 * ROWB);
                const bf16x8 vt = __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo4, hi4, 0, 1, 2, 3, 4, 5, 6, 7));
                aA[c] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vt, fa, aA[c], 0, 0, 0);
                aB[c] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vt, fb, aB[c], 0, 0, 0);
              }
            }
            __builtin_amdgcn_s_setprio(0);
          }
        }
      }
    }
    if (nq >= 0 && nj == 0) {  // nothing visible: the rows are still needed next
      load_q(nq, 0, qA);
      load_q(nq, 1, qB);
    }
    // Epilogue, one head after the other through this wave's staging rows.
    auto out = [&](int h, const f32x16 (&ac)[2], float lsum, float M) __attribute__((always_inline)) {
      const float ltot = pair32_sum(lsum);
      const float inv = ltot > 0.f ? __builtin_amdgcn_rcpf(ltot) : 0.f;
      uint16_t* so = sO[wave];
#pragma unroll
      for (int c = 0; c < 2; ++c)
#pragma unroll
        for (int rq = 0; rq < 4; ++rq) {
          const bf16x4 pk = pack_bf16x4(ac[c][4 * rq + 0] * inv, ac[c][4 * rq + 1] * inv, ac[c][4 * rq + 2] * inv,
                                        ac[c][4 * rq + 3] * inv);
          *reinterpret_cast<bf16x4*>(&so[l32 * OSTR + 8 * ((4 * c + rq) ^ (l32 & 7)) + 4 * g]) = pk;
        }
      const size_t obase = ((size_t)n * p.Hq + h) * p.L;
      const __amdgpu_buffer_rsrc_t lrs = make_rsrc(p.lse + obase, (uint32_t)p.L * 4u);
      const __amdgpu_buffer_rsrc_t ors = make_rsrc(p.o + obase * E, (uint32_t)p.L * ROWB);
      buffer_store4(lrs, (uint32_t)qi * 4u, ltot > 0.f ? (M + __builtin_amdgcn_logf(ltot)) * kLn2 : kNegInf);
      __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0)
      __builtin_amdgcn_wave_barrier();
#pragma unroll
      for (int it = 0; it < (QB * ECH) / 64; ++it) {
        const int id = lane + 64 * it;
        const int rloc = id / ECH, c = id % ECH;
        const u32x4 val = *reinterpret_cast<const u32x4*>(&so[rloc * OSTR + 8 * (c ^ (rloc & 7))]);
        buffer_store16_nt(ors, (uint32_t)((qa + rloc) * ROWB + 16 * c), val);
      }
      __builtin_amdgcn_s_waitcnt(0xc07f);  // reads done before the rows are written again
      __builtin_amdgcn_wave_barrier();
    };
    out(hA, aA, lA, mA);
    out(hB, aB, lB, mB);
  };

  // First query block: its whole band into sK/sV, and the Q rows of this wave's
  // first head.
  const int qb0 = grp * QPW;
  const int nqb = min(QPW, (p.L + QB - 1) / QB - qb0);  // query blocks of this workgroup (1 or 2)
  int lo0, hi0;
  key_range(qb0, lo0, hi0);
  const int n0 = hi0 >= lo0 ? hi0 / KB - lo0 / KB + 1 : 0;  // at most NKB (window <= WMAX)
  const int kb0 = hi0 >= lo0 ? lo0 / KB : 0;
  for (int sl = 0; sl < n0; ++sl) load_block(kb0 + sl, sK + sl * BLKB, sV + sl * BLKB);
  // Sink logits (log2 units) of this wave's heads, read once here: a load in
  // the pair loop would wait for every memory operation in flight before it.
  float sink_l2[2] = {kNegInf, kNegInf};
  if (p.sink) {
#pragma unroll
    for (int pp = 0; pp < PPW; ++pp) sink_l2[pp] = p.sink[kh * G + wave + 4 * pp] * kLog2e;
  }
  bf16x8 qcur[4], qnext[4];
  load_q(qb0, 0, qcur);
  // (the empty asm keeps these loads above the barrier, in flight with the band's)
#pragma unroll
  for (int s4 = 0; s4 < 4; ++s4) asm volatile("" : "+v"(qcur[s4]));
  __builtin_amdgcn_s_waitcnt(0x0f70);  // vmcnt(0)
  __syncthreads();

  // Second query block: its band ends at most one block past the first one's
  // (both ends move by 32 positions); that block goes to sKn/sVn now.
  int lo1 = 0, hi1 = -1;
  if (nqb > 1) {
    key_range(qb0 + 1, lo1, hi1);
    if (hi1 >= lo1 && (n0 == 0 || hi1 / KB > kb0 + n0 - 1)) load_block(hi1 / KB, sKn, sVn);
  }

  if constexpr (PPW == 2) {
    load_q(qb0, 1, qnext);  // the second head's rows
    compute_pair2(std::false_type{}, qb0 * QB, lo0, hi0, qcur, qnext, sink_l2[0], sink_l2[1], kb0, n0,
                  nqb > 1 ? qb0 + 1 : -1);
    if (nqb < 2) return;
    __builtin_amdgcn_s_waitcnt(0x0f70);  // vmcnt(0): this wave's part of the added block landed
    __syncthreads();
    compute_pair2(std::true_type{}, (qb0 + 1) * QB, lo1, hi1, qcur, qnext, sink_l2[0], sink_l2[1], kb0, n0, -1);
    return;
  }
#pragma unroll 1
  for (int pp = 0; pp < PPW; ++pp) {
    // the next (head, block) pair's Q rows, one pair ahead
    if (pp + 1 < PPW)
      load_q(qb0, pp + 1, qnext);
    else if (nqb > 1)
      load_q(qb0 + 1, 0, qnext);
    compute_pair(std::false_type{}, kh * G + wave + 4 * pp, qb0 * QB, lo0, hi0, qcur,
                 pp == 0 ? sink_l2[0] : sink_l2[1], kb0, n0);
#pragma unroll
    for (int s4 = 0; s4 < 4; ++s4) qcur[s4] = qnext[s4];
  }
  if (nqb < 2) return;
  __builtin_amdgcn_s_waitcnt(0x0f70);  // vmcnt(0): this wave's part of the added block landed
  __syncthreads();
#pragma unroll 1
  for (int pp = 0; pp < PPW; ++pp) {
    if (pp + 1 < PPW) load_q(qb0 + 1, pp + 1, qnext);
    compute_pair(std::true_type{}, kh * G + wave + 4 * pp, (qb0 + 1) * QB, lo1, hi1, qcur,
                 pp == 0 ? sink_l2[0] : sink_l2[1], kb0, n0);
#pragma unroll
    for (int s4 = 0; s4 < 4; ++s4) qcur[s4] = qnext[s4];
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
         !a.bias && a.L > 0 && (long long)a.L * ROWB < (1LL << 31) && (long long)a.S * ROWB < (1LL << 31) &&
         (G == 4 || G == 8);
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
