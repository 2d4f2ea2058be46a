// prefill_bf16.hip -- fused tiled attention forward for bf16 inputs on gfx950.
//
// One workgroup = 4 waves = 128 query rows of one (batch, query head); each
// wave owns 32 rows.  Keys are streamed in tiles of 64 (32 in dot mode at
// E = 128, see TileShape) through LDS; the score tile is never written to memory (the tiling + online softmax of the
// FlashAttention row in "어텐션 메커니즘" section 6, and the running max /
// running sum described in "SDPA란 무엇인가?" section 2).
//
// Orientation.  Each wave computes S^T = K * Q^T with v_mfma_f32_32x32x16_bf16
// (A = 32 keys x 16 head-dims from LDS, B = the wave's Q^T held in VGPRs), so in
// the accumulator layout every lane holds ONE query (column) and 16 keys.  The
// row max and the rescale factor are then per-lane scalars; only one exchange
// with lane^32 (the other half of the same query's keys) is needed per tile.
// The output is accumulated the same way, O^T = V^T * P^T: P^T comes straight
// from the S^T registers (rounded to bf16), and the V^T operand is gathered
// from the row-major V tile by ds_read_b64_tr_b16 (transposing LDS read: in
// each 16-lane group, lane j's element e is element j%4 of the 8-byte row piece
// addressed by lane 4e + j/4), pointed at the keys in the order in which the
// S^T accumulator hands them to each lane.
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
// Pipeline.  K and V tiles are double-buffered in LDS and filled by
// LDS-direct buffer loads (no register round trip, rows past the end of the
// slice arrive as zeros): right after the barrier that frees buffer (t+1)%2,
// tile t+1 is requested; tile t is consumed meanwhile; each wave waits for its
// own requests before the next barrier, so one barrier per tile suffices.  In
// RBF mode K still goes through registers, where |k|^2 is formed on its way to
// LDS.  Tiles are stored row-major with the 16-byte chunks of row r permuted by
// an XOR with swz(r), which keeps both the K reads (16 rows, one chunk) and the
// transposing V reads (4 rows, two chunks) free of bank conflicts.  The two
// buffers are separate LDS objects and tiles are taken in pairs, so every LDS
// address is a base register plus an immediate offset.  Several workgroups
// share a CU, so one wave's softmax overlaps another's MFMAs.  The running max
// moves lazily: the accumulator is rescaled only when a row max grows by more
// than 2^8 over the reference (O = acc / l does not depend on the reference;
// it only bounds p by 256).  With a positive scale the dot-mode max is taken on
// the raw scores and each weight costs one fma + exp2; the tile max itself is
// skipped when each lane's sum of weights formed against the current reference
// shows that no weight exceeds 256.  In folded RBF mode no
// logit of a row exceeds c|q|^2/2, and the tile max is skipped once the
// reference is within 2^16 of that bound.  Row sums are compensated (Kahan)
// where a register allows it.
// The epilogue transposes O through LDS so that stores are whole rows.
#include <type_traits>

#include "device_common.h"
#include "kernels.h"
#include "tile_common.h"

using namespace attn_dev;

namespace {

constexpr int BM = 128;  // query rows per workgroup
constexpr int NT = 256;  // threads per workgroup
constexpr float kLazy = 8.f;  // rescale when a row max grows by more than this (log2 units)
constexpr float kSumCap = 256.f;  // 2^kLazy: bound on a lane's weight sum that needs no tile max
constexpr float kLazyBound = 16.f;  // RBF: skip the tile max once the reference is this close to the bound

struct PrefillParams {
  const uint16_t* q;
  const uint16_t* k;
  const uint16_t* v;
  uint16_t* o;
  float* lse;
  const float* sink;
  int N, Hq, Hkv, L, S, n_reg, S_real, off, causal, window;
  float c_logit, c_bias, gamma;
  const int* key_len;     // N valid real-key counts, or nullptr
  const void* ubias;      // user bias: float32 (log2 units after scaling) or uint8 mask, or nullptr
  long long ub_sn, ub_sh; // its element strides over batch and head (0 = broadcast); rows are S apart
  int num_q_tiles;
  int xcd_groups;   // 1: the 8 XCDs each take whole K/V heads (needs N*Hkv % 8 == 0)
  int xcd_contig;   // with xcd_groups: XCD x takes consecutive (batch, kv head) units instead of every 8th
  int heavy_first;  // 1: causal, dispatch the query tiles with the most keys first
};

// Workgroup id -> (query tile, batch, head).  Workgroups are handed to the 8
// XCDs round-robin (id % 8), and each XCD has its own L2: with xcd_groups all
// query heads that read one K/V head land on the same XCD.  With xcd_contig an
// XCD's (batch, kv head) units are consecutive, so that the heads of one batch
// share XCDs: for a user bias broadcast over heads, each bias tile is then
// read by 2 XCDs instead of all 8 (3 % faster on the biased 4x16x2048x128
// prefill; neutral to 1 % slower without such a bias, where it stays off).
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
    const int u = p.xcd_contig ? x * (U >> 3) + ul : ul * 8 + x;
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
//   kDotPos:  dot mode, scale > 0 -- max over raw scores, weight = exp2(fma(s, c, -m));
//   kDotAny:  dot mode, any finite scale -- x = c*s first;
//   kRbf:     x = c*s + bias_k with bias_k = -gamma*log2(e)*|k|^2 from the staged tile;
//   kRbfFold: RBF with gamma > 0 -- the key term goes into the matrix product instead:
//             one more K step (a 32x32x8 MFMA, half the K width of the others: the
//             three terms fit one 4-wide K group) whose A operand holds -|k|^2/2 split into three
//             bf16 parts (hi + mid + lo, ~24 significant bits, summed exactly in the
//             fp32 accumulator) against ones in Q^T, so s' = q.k - |k|^2/2 and the
//             weights are formed as in kDotPos: exp2(fma(s', c, -m)), c = 2*gamma*log2(e).
enum { kDotPos = 0, kDotAny = 1, kRbf = 2, kRbfFold = 3 };

// User bias kinds (a compile-time parameter): none, float32 added to the
// logits, uint8 mask (0 hides the pair).
enum { kBiasNone = 0, kBiasF32 = 1, kBiasBool = 2 };

// Keys per staged tile, and waves per SIMD the register budget allows.  64-key
// tiles: E = 128 needs ~230 VGPRs (2 waves); E = 64 fits in 128 VGPRs in dot
// mode (4 waves = 4 workgroups per CU, 128 KB of LDS) and under 168 in RBF mode
// (3 waves), where 128 would spill; with a user bias it needs up to ~210 (2
// waves).  Dot mode at E = 128 without a user bias takes 32-key tiles instead:
// S^T then holds 16 registers instead of 32 and the kernel fits 160 VGPRs, so
// three waves per SIMD (three workgroups of 32 KB LDS per CU) -- 2.7 % faster on
// the causal 4x16x2048x128 prefill than 64-key tiles at two waves (32-key tiles
// at two waves: 5 % slower; 64-key tiles at three waves spill).
template <int E, int MODE, int UB>
struct TileShape {
  static constexpr bool kNarrow = E == 128 && UB == 0 && (MODE == kDotPos || MODE == kDotAny);
  static constexpr int kKeys = kNarrow ? 32 : 64;
  static constexpr int kWaves = kNarrow ? 3 : (E == 128 || UB != 0) ? 2 : ((MODE == kRbf || MODE == kRbfFold) ? 3 : 4);
};

template <int E, int MODE, int UB>
__global__ __launch_bounds__(NT) __attribute__((amdgpu_waves_per_eu(TileShape<E, MODE, UB>::kWaves, TileShape<E, MODE, UB>::kWaves)))
void prefill_bf16_kernel(PrefillParams p) {
  constexpr bool RBF = MODE == kRbf || MODE == kRbfFold;  // K staged through registers, |k|^2 on chip
  constexpr bool FOLD = MODE == kRbfFold;
  constexpr bool FAST = MODE == kDotPos || FOLD;
  // Dot mode with a positive scale: weights against the current reference first,
  // the tile max only when their sums say the reference must move.
  constexpr bool SUMCHK = MODE == kDotPos;
  static_assert(UB == kBiasNone || !FAST, "a user bias needs the logits formed before the max");
  constexpr int BN = TileShape<E, MODE, UB>::kKeys;  // keys per staged tile
  // Epilogue O staging: padded rows, or (32-key tiles, where padded rows of two
  // waves would not fit one tile buffer) unpadded rows with XOR-swizzled chunks.
  constexpr bool OSWZ = BN == 32;
  constexpr int OSTR = OSWZ ? E : E + 8;  // O row stride (elements)
  constexpr int QS = E / 16;    // MFMA steps over the head dimension
  constexpr int EB = E / 32;    // 32-row blocks of O^T
  constexpr int NB = BN / 32;   // 32-key blocks of S^T per tile
  constexpr int ECH = E / 8;    // 16-byte chunks per row
  constexpr int ROWB = E * 2;   // bytes per K/V row
  constexpr int TILEB = BN * ROWB;         // bytes per K (or V) tile
  constexpr int RPI = 1024 / ROWB;         // rows per 1 KB wave-wide LDS-direct load
  constexpr int IPW = BN / RPI / 4;        // such loads per wave per tile (4 waves)
  constexpr int KCH = BN * ECH / NT;       // K chunks per thread (RBF register staging)
  static_assert(IPW * RPI * 4 == BN, "tile must split into whole 1 KB loads per wave");
  static_assert(KCH * NT == BN * ECH, "K staging must tile evenly");
  static_assert(!FOLD || KCH % 2 == 0, "the norm split converts two rows at a time");
  static_assert(2 * 32 * OSTR * 2 <= 2 * TILEB, "epilogue staging of two waves must fit one tile buffer");

  // [buf][K tile | V tile], each tile row-major with swizzled 16-byte chunks.
  // The two buffers are separate LDS objects: where the buffer index is a
  // compile-time constant, the compiler can then tell a read of one buffer from
  // the LDS-direct loads in flight into the other and does not make the
  // transposing V reads wait for them.
  __shared__ __attribute__((aligned(16))) uint8_t sKV0[2 * TILEB];
  __shared__ __attribute__((aligned(16))) uint8_t sKV1[2 * TILEB];
  __shared__ __attribute__((aligned(16))) float sBias[2][BN];
  __shared__ __attribute__((aligned(16))) u32x2 sKn[FOLD ? 2 : 1][FOLD ? BN : 1];  // kRbfFold: -|k|^2/2 as 3 bf16
  auto k_tile = [&](int buf) { return buf ? sKV1 : sKV0; };
  auto v_tile = [&](int buf) { return (buf ? sKV1 : sKV0) + TILEB; };

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
  // kRbfFold: Q^T fragment of the extra K step (a 32x32x8 operand), bf16 ones in
  // K-dims 0..2 (lanes g = 0).
  const u32x2 qone = (FOLD && g == 0) ? u32x2{0x3f803f80u, 0x00003f80u} : u32x2{0u, 0u};

  // Running state in log2 units: m is the reference max, lsum this lane's share
  // of the row sum (its 16 keys per block); the halves are added at the end.
  float m = kNegInf, lsum = 0.f;
  // lsum is a compensated (Kahan) sum: lcomp carries the low-order part lost by
  // each tile's addition.  With every tile adding nearly the same amount (long
  // rows of near-equal logits) the plain fp32 sum's rounding is systematic: over
  // 8M keys in 32-key tiles it drifted by 2.4e-3 relative (1.7e-4 in 64-key
  // tiles).  The four-wave kernels (E = 64 dot, 128 VGPRs) keep the plain sum:
  // the extra register spills there.
  constexpr bool KSUM = TileShape<E, MODE, UB>::kWaves < 4;
  float lcomp = 0.f;
  // RBF (folded): the largest logit a key can give this row, c * |q|^2 / 2.
  const float qbound = FOLD ? 0.5f * p.c_logit * qn2 : 0.f;
  if (p.sink) {
    float s0 = p.sink[h];
    if (RBF) s0 += p.gamma * qn2;
    m = s0 * kLog2e;
    lsum = (g == 0) ? 1.f : 0.f;
  }
  // Derived from m, updated only where m moves: thr, the value a raw score (FAST)
  // or logit must pass to grow the row max by more than kLazy, and -m (0 while
  // the row has seen nothing).
  const float inv_c = FAST ? 1.f / p.c_logit : 1.f;
  auto lazy_thr = [&](float mref) { return FAST ? (mref + kLazy) * inv_c : mref + kLazy; };
  float thr = lazy_thr(m);
  float negm = (m == kNegInf) ? 0.f : -m;
  f32x16 acc[EB];
#pragma unroll
  for (int c = 0; c < EB; ++c)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[c][r] = 0.f;

  // Tiles: register rows first, then the real keys some row of this workgroup sees.
  // Real keys at or past kl are padding of this sequence (no key lengths: none).
  const int kl = p.key_len ? max(0, min(p.S_real, p.key_len[n])) : p.S_real;
  const int i_last = min(i0 + BM, p.L) - 1;
  const int r_hi = p.causal ? min(kl - 1, i_last + p.off) : kl - 1;
  const int r_lo = p.window > 0 ? max(0, i0 + p.off - p.window + 1) : 0;
  const int n_real_tiles = r_hi >= r_lo ? (r_hi - r_lo + BN) / BN : 0;
  const int n_reg_tiles = (p.n_reg + BN - 1) / BN;
  const int T = n_reg_tiles + n_real_tiles;

  // K and V of this (batch, kv head): one buffer resource each over exactly the
  // S rows of the slice, so rows past the end load as zeros.
  const size_t kvoff = ((size_t)n * p.Hkv + kh) * (size_t)p.S * E;
  const __amdgpu_buffer_rsrc_t krs = make_rsrc(p.k + kvoff, (uint32_t)p.S * ROWB);
  const __amdgpu_buffer_rsrc_t vrs = make_rsrc(p.v + kvoff, (uint32_t)p.S * ROWB);

  // LDS-direct loads: this wave's block b of a tile is rows RPI*(IPW*wave + b) ..;
  // lane l fills physical chunk l % ECH of row l / ECH, i.e. logical chunk
  // (l % ECH) ^ swz(row) of the global row.
  uint32_t ld_off[IPW];
#pragma unroll
  for (int b = 0; b < IPW; ++b) {
    const int row = RPI * (IPW * wave + b) + lane / ECH;
    ld_off[b] = (uint32_t)(row * ROWB + (((lane % ECH) ^ tile_swz<E>(row)) * 16));
  }
  // K operand reads: row l32 (+32 for block 1), logical chunk 2s + g.
  uint32_t krd[QS];
#pragma unroll
  for (int s = 0; s < QS; ++s) krd[s] = (uint32_t)(l32 * ROWB + (((2 * s + g) ^ tile_swz<E>(l32)) * 16));
  // V^T operand reads (transposing): lane m of 16-lane group q points at key
  // row 4*(q/2) + (m%16)/4 (+8 for the second half of the operand) of the
  // current 16-key group, dims 32c + 16*(q%2) + 4*(m%4) .. +4.
  uint32_t vrd[EB][2];
  {
    const int q16 = lane >> 4, m16 = lane & 15;
#pragma unroll
    for (int c = 0; c < EB; ++c)
#pragma unroll
      for (int hh = 0; hh < 2; ++hh) {
        const int row = 4 * (q16 >> 1) + (m16 >> 2) + 8 * hh;
        const int d = 32 * c + 16 * (q16 & 1) + 4 * (m16 & 3);
        vrd[c][hh] = (uint32_t)(row * ROWB + (((d >> 3) ^ tile_swz<E>(row)) * 16) + (d & 7) * 2);
      }
  }

  u32x4 kreg[KCH];  // RBF only: K chunks on their way to LDS
  // RBF: LDS byte offset of each staged chunk (row (tid + NT*i) / ECH, swizzled),
  // formed once; the empty asm keeps the compiler from recomputing it per tile.
  uint32_t kwo[RBF ? KCH : 1];
  if (RBF) {
#pragma unroll
    for (int i = 0; i < KCH; ++i) {
      const int id = tid + NT * i;
      const int row = id / ECH, c = id % ECH;
      kwo[i] = (uint32_t)(row * ROWB + ((c ^ tile_swz<E>(row)) * 16));
      asm volatile("" : "+v"(kwo[i]));
    }
  }

  auto tile_keys = [&](int t, int& j0, int& kc) __attribute__((always_inline)) {
    if (t < n_reg_tiles) {
      j0 = t * BN;
      kc = min(BN, p.n_reg - j0);
    } else {
      j0 = p.n_reg + r_lo + (t - n_reg_tiles) * BN;
      kc = min(BN, p.S - j0);
    }
  };

  // Request tile t into buffer `buf`.  Rows past the tile's last key are loaded
  // anyway (real keys of the slice, or zeros past its end) and masked later.
  auto issue_tile = [&](int t, int buf) __attribute__((always_inline)) {
    int j0, kc;
    tile_keys(t, j0, kc);
    const uint32_t tb = (uint32_t)j0 * ROWB;
#pragma unroll
    for (int b = 0; b < IPW; ++b) {
      const int blk = IPW * wave + b;
      buffer_load16_to_lds(vrs, v_tile(buf) + blk * 1024, tb + ld_off[b]);
      if (!RBF) buffer_load16_to_lds(krs, k_tile(buf) + blk * 1024, tb + ld_off[b]);
    }
    if (RBF) {
#pragma unroll
      for (int i = 0; i < KCH; ++i) {
        const int id = tid + NT * i;
        kreg[i] = buffer_load16(krs, tb + (uint32_t)((id / ECH) * ROWB + (id % ECH) * 16));
      }
    }
  };

  // Complete the requested tile in `buf`: in RBF mode write the K registers
  // (swizzled) and the per-key bias c_bias * |k|^2; then wait until this wave's
  // LDS-direct requests have landed.
  auto finish_tile = [&](int buf) __attribute__((always_inline)) {
    if (RBF) {
      // |k|^2 of each staged key row: its ECH chunks sit in ECH consecutive lanes.
      float ss[KCH];
#pragma unroll
      for (int i = 0; i < KCH; ++i) {
        *reinterpret_cast<u32x4*>(k_tile(buf) + kwo[i]) = kreg[i];
        ss[i] = group_sum<ECH>(sumsq8(kreg[i]));
      }
      const int c = tid % ECH;  // the same chunk for every i (NT is a multiple of ECH)
      if (c == 0) {
        const int row0 = tid / ECH;
        if (FOLD) {
          // -|k|^2/2 = hi + mid + lo, each rounded to bf16 (nearest even) in
          // turn; two rows per conversion (v_cvt_pk_bf16_f32).
          typedef float f32x2v __attribute__((ext_vector_type(2)));
          typedef __bf16 bf16x2v __attribute__((ext_vector_type(2)));
          auto widen = [](bf16x2v x) {
            const uint32_t w = __builtin_bit_cast(uint32_t, x);
            return f32x2v{bf16_lo(w), bf16_hi(w)};
          };
#pragma unroll
          for (int i = 0; i < KCH; i += 2) {
            const f32x2v v0 = {-0.5f * ss[i], -0.5f * ss[i + 1]};
            const bf16x2v hi = __builtin_convertvector(v0, bf16x2v);
            const f32x2v v1 = v0 - widen(hi);
            const bf16x2v mid = __builtin_convertvector(v1, bf16x2v);
            const bf16x2v lo = __builtin_convertvector(v1 - widen(mid), bf16x2v);
            const uint32_t h = __builtin_bit_cast(uint32_t, hi), md = __builtin_bit_cast(uint32_t, mid),
                           l = __builtin_bit_cast(uint32_t, lo);
            sKn[buf][row0 + (NT / ECH) * i] = u32x2{__builtin_amdgcn_perm(md, h, 0x05040100u), l & 0xffffu};
            sKn[buf][row0 + (NT / ECH) * (i + 1)] = u32x2{__builtin_amdgcn_perm(md, h, 0x07060302u), l >> 16};
          }
        } else {
#pragma unroll
          for (int i = 0; i < KCH; ++i) sBias[buf][row0 + (NT / ECH) * i] = p.c_bias * ss[i];
        }
      }
    }
    __builtin_amdgcn_s_waitcnt(0x0f70);  // vmcnt(0)
  };

  auto compute_tile = [&](int t, int buf, auto masked_tag) __attribute__((always_inline)) {
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
      any = !((ra >= kl) || (p.causal && ra > qb + p.off) ||
              (p.window > 0 && qa + p.off - rb >= p.window));
      full = rb < kl && (!p.causal || rb <= qa + p.off) &&
             (p.window <= 0 || qb + p.off - ra < p.window);
    }
    if (!any) return;
    const uint8_t* k_s = k_tile(buf);
    const uint8_t* v_s = v_tile(buf);

    // User bias of this lane's row for the tile's keys, in log2 units (a masked
    // pair gets -inf), loaded before the MFMAs so that the loads overlap them.
    // Keys past the end of K read the last column; the rule hides those pairs.
    // Each lane's keys come in runs of 4 consecutive columns; when every run is
    // 4-element aligned and inside the row (uniform test), one 16-byte (float)
    // or 4-byte (mask) load fetches a run.
    float ubv[UB != kBiasNone ? NB : 1][16];
    if (UB != kBiasNone) {
      const long long base_nh = (long long)n * p.ub_sn + (long long)h * p.ub_sh;
      const long long rowoff = base_nh + (long long)min(qi, p.L - 1) * p.S;
      const bool vec = (p.S % 4 == 0) && ((base_nh + j0) % 4 == 0) && (j0 + BN <= p.S) &&
                       (reinterpret_cast<uintptr_t>(p.ubias) % (UB == kBiasF32 ? 16 : 4) == 0);
      if (vec) {
#pragma unroll
        for (int b = 0; b < NB; ++b)
#pragma unroll
          for (int rq = 0; rq < 4; ++rq) {
            const long long j = rowoff + j0 + 32 * b + 8 * rq + 4 * g;
            if (UB == kBiasF32) {
              const f32x4 x = *reinterpret_cast<const f32x4*>(static_cast<const float*>(p.ubias) + j);
#pragma unroll
              for (int e = 0; e < 4; ++e) ubv[b][4 * rq + e] = x[e] * kLog2e;
            } else {
              const uint32_t x = *reinterpret_cast<const uint32_t*>(static_cast<const uint8_t*>(p.ubias) + j);
#pragma unroll
              for (int e = 0; e < 4; ++e) ubv[b][4 * rq + e] = ((x >> (8 * e)) & 0xffu) ? 0.f : kNegInf;
            }
          }
      } else {
#pragma unroll
        for (int b = 0; b < NB; ++b)
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const long long j = rowoff + min(j0 + 32 * b + 8 * (r >> 2) + 4 * g + (r & 3), p.S - 1);
            if (UB == kBiasF32)
              ubv[b][r] = static_cast<const float*>(p.ubias)[j] * kLog2e;
            else
              ubv[b][r] = static_cast<const uint8_t*>(p.ubias)[j] ? 0.f : kNegInf;
          }
      }
    }

    // S^T = K * Q^T for NB blocks of 32 keys; the NB accumulation chains are
    // interleaved so that consecutive MFMAs never depend on each other.  The
    // scores are then made logits (unless FAST) and masked; a second pass forms
    // them again, from the same K tile, when the sum-checked weights of SUMCHK
    // fail their check.
    f32x16 st[NB];
    float ps = -0.f;  // (-0 + x == x: the first addition folds away)
    bool general = true;
#pragma unroll
    for (int pass = 0; pass < (SUMCHK ? 2 : 1); ++pass) {
#pragma unroll
    for (int b = 0; b < NB; ++b)
#pragma unroll
      for (int r = 0; r < 16; ++r) st[b][r] = 0.f;
    // Raised wave priority while a wave issues its MFMA chains, so that a wave
    // holding matrix work is picked over one doing softmax arithmetic.
    __builtin_amdgcn_s_setprio(1);
#pragma unroll
    for (int s = 0; s < QS; ++s) {
      bf16x8 a[NB];
#pragma unroll
      for (int b = 0; b < NB; ++b)
        a[b] = *reinterpret_cast<const bf16x8*>(k_s + krd[s] + 32 * b * ROWB);
#pragma unroll
      for (int b = 0; b < NB; ++b) st[b] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[b], qf[s], st[b], 0, 0, 0);
    }
    if (FOLD) {
      // The extra K step: key row l32 of block b contributes its three parts of
      // -|k|^2/2 in K-dims 0..2 (lanes g = 0 hold K-dims 0..3 of the 32x32x8
      // operands, lanes g = 1 K-dims 4..7), the query side ones there.
#pragma unroll
      for (int b = 0; b < NB; ++b) {
        const u32x2 kn = sKn[buf][32 * b + l32];
        typedef short short4v __attribute__((ext_vector_type(4)));
        const u32x2 av = g == 0 ? kn : u32x2{0u, 0u};
        st[b] = __builtin_amdgcn_mfma_f32_32x32x8bf16_1k(__builtin_bit_cast(short4v, av),
                                                          __builtin_bit_cast(short4v, qone), st[b], 0, 0, 0);
      }
    }
    __builtin_amdgcn_s_setprio(0);

    // Accumulator row of register r in block b = key 32b + 8(r/4) + 4g + r%4 of
    // the tile.  FAST keeps raw scores (the scale goes into the exponent);
    // otherwise the scores become log2-unit logits here.
    if (!FAST) {
#pragma unroll
      for (int b = 0; b < NB; ++b)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          float x = st[b][r] * p.c_logit;
          if (RBF && !FOLD) x += sBias[buf][32 * b + 8 * (r >> 2) + 4 * g + (r & 3)];
          if (UB != kBiasNone) x += ubv[b][r];
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
        hi = min(kl - 1, p.causal ? ip : kl - 1) - base;
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

    // SUMCHK: once every row of the wave has a reference, the weights are formed
    // against it without the tile max.  A lane's sum of its 16 (or 32) weights
    // bounds each of them, so a sum at most 2^kLazy shows that no weight passed
    // 2^kLazy: the bound the lazy rule below keeps, met without moving the
    // reference.  Otherwise (rare: the row max jumped, or many weights near the
    // reference) the scores are formed again and go the general way.
    if (SUMCHK && pass == 0 && !__any(m == kNegInf)) {
#pragma unroll
      for (int b = 0; b < NB; ++b)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const float pv = fast_exp2(__builtin_fmaf(st[b][r], p.c_logit, negm));
          st[b][r] = pv;
          ps += pv;
        }
      general = __any(!(ps <= kSumCap));
      if (general) {
        ps = -0.f;
        continue;
      }
    }
    break;
    }  // pass
    if (general) {
    // RBF: no logit of this row exceeds qbound (the logit of a key equal to q),
    // so once every row's reference is within kLazyBound of it no weight can
    // pass 2^kLazyBound and the tile's max is not needed.
    if (!FOLD || __any(qbound - m > kLazyBound)) {
    // This lane's half of its row's max (the other half sits in lane ^ 32).
    float mx = kNegInf;
#pragma unroll
    for (int b = 0; b < NB; ++b)
#pragma unroll
      for (int r = 0; r < 16; r += 2) mx = fmaxf(fmaxf(mx, st[b][r]), st[b][r + 1]);  // v_max3 chain

    // Lazy reference max: move it (and rescale) only when a row max would grow
    // by more than kLazy -- i.e. when some half-row max passes thr; otherwise
    // weights stay below 2^kLazy.  Only then is the whole row's max formed.
    if (__any(mx > thr)) {
      mx = pair32_max(mx);
      if (FAST) mx = (mx == kNegInf) ? kNegInf : mx * p.c_logit;
      const float m_new = fmaxf(m, mx);
      const float alpha = (m_new == kNegInf) ? 1.f : fast_exp2(m - m_new);
      m = m_new;
      thr = lazy_thr(m);
      negm = (m == kNegInf) ? 0.f : -m;
      lsum *= alpha;
      if (KSUM) lcomp *= alpha;
#pragma unroll
      for (int c = 0; c < EB; ++c)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[c][r] *= alpha;
    }
    }

#pragma unroll
    for (int b = 0; b < NB; ++b)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const float pv = FAST ? fast_exp2(__builtin_fmaf(st[b][r], p.c_logit, negm))
                              : fast_exp2(st[b][r] + negm);
        st[b][r] = pv;
        ps += pv;
      }
    }  // general
    if (KSUM) {
      const float y = ps - lcomp;
      const float t = lsum + y;
      lcomp = (t - lsum) - y;
      lsum = t;
    } else {
      lsum += ps;
    }

    // O^T += V^T * P^T, 16 keys per MFMA step.
    __builtin_amdgcn_s_setprio(1);
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
          const shortx4 lo = lds_read_tr(v_s + vrd[c][0] + 16 * u * ROWB);
          const shortx4 hi = lds_read_tr(v_s + vrd[c][1] + 16 * u * ROWB);
          const bf16x8 vt = __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
          acc[c] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vt, pf, acc[c], 0, 0, 0);
        }
      }
    }
    __builtin_amdgcn_s_setprio(0);
  };

  // Real tiles k in [k_full0, k_full1] are seen completely by every row of the
  // workgroup and run without visibility code; the tiles before and after them
  // (and the register tiles) run with it.
  int k_full0 = 0, k_full1 = -1;
  {
    const int lim = min(kl - 1, p.causal ? i0 + p.off : kl - 1);
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

  // Tile t lives in buffer t % 2: right after the barrier that frees the other
  // buffer, tile t+1 is requested into it; tile t is consumed; the wave waits
  // for its own requests; one barrier publishes tile t+1 to every wave.
  // The buffer index is a compile-time constant at each call (the loops below
  // take tiles in pairs), so LDS addresses become base registers plus
  // immediate offsets instead of per-tile address arithmetic.
  // Both buffers are free at the start, so in dot mode (K straight to LDS)
  // tile 1 is requested together with tile 0 and its latency overlaps tile 0's.
  const bool pre1 = !RBF && T > 1;
  auto step = [&](int t, int buf, auto masked_tag) __attribute__((always_inline)) {
    if (t + 1 < T && !(pre1 && t == 0)) issue_tile(t + 1, buf ^ 1);
    compute_tile(t, buf, masked_tag);
    if (t + 1 < T) finish_tile(buf ^ 1);
    __syncthreads();
  };
  auto run = [&](int ta, int tb, auto masked_tag) __attribute__((always_inline)) {
    int t = ta;
    if constexpr (UB != kBiasNone) {  // no registers to spare for the doubled loop body
      for (; t < tb; ++t) step(t, t & 1, masked_tag);
      return;
    }
    if (t < tb && (t & 1)) step(t++, 1, masked_tag);
    for (; t + 1 < tb; t += 2) {
      step(t, 0, masked_tag);
      step(t + 1, 1, masked_tag);
    }
    if (t < tb) step(t, 0, masked_tag);
  };

  if (T > 0) {
    issue_tile(0, 0);
    if (pre1) {
      issue_tile(1, 1);
      static_assert(2 * IPW < 16, "vmcnt field");
      __builtin_amdgcn_s_waitcnt(0x0f70 | (2 * IPW));  // Q and tile 0 landed; tile 1 in flight
    } else {
      finish_tile(0);  // also waits for the Q loads issued above
    }
  }
  __syncthreads();
  const int head_end = (t_full1 > t_full0) ? t_full0 : T;
  run(0, head_end, std::true_type{});
  run(head_end, t_full1, std::false_type{});
  run(max(head_end, t_full1), T, std::true_type{});

  // Epilogue: O = acc / l (0 for an empty row) staged through LDS (free after
  // the last barrier) so that global stores are whole rows; LSE in natural log.
  const float ltot = pair32_sum(lsum);
  const float inv = ltot > 0.f ? 1.f / ltot : 0.f;
  uint16_t* sO = reinterpret_cast<uint16_t*>(wave < 2 ? sKV0 : sKV1) + (wave & 1) * 32 * OSTR;
  auto ochunk = [&](int row, int ch) { return OSWZ ? (ch ^ (row & (ECH - 1))) : ch; };
#pragma unroll
  for (int c = 0; c < EB; ++c)
#pragma unroll
    for (int rq = 0; rq < 4; ++rq) {
      const bf16x4 pk = pack_bf16x4(acc[c][4 * rq + 0] * inv, acc[c][4 * rq + 1] * inv,
                                    acc[c][4 * rq + 2] * inv, acc[c][4 * rq + 3] * inv);
      *reinterpret_cast<bf16x4*>(&sO[l32 * OSTR + 8 * ochunk(l32, 4 * c + rq) + 4 * g]) = pk;
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
      const u32x4 val = *reinterpret_cast<const u32x4*>(&sO[rloc * OSTR + 8 * ochunk(rloc, c)]);
      __builtin_nontemporal_store(val, reinterpret_cast<u32x4*>(p.o + (obase + row) * E + 8 * c));  // written once
    }
  }
}

template <int E, int MODE, int UB>
hipError_t launch_t(const PrefillParams& p, hipStream_t stream) {
  const long long blocks = (long long)p.num_q_tiles * p.N * p.Hq;
  hipLaunchKernelGGL((prefill_bf16_kernel<E, MODE, UB>), dim3((unsigned)blocks), dim3(NT), 0, stream, p);
  return hipGetLastError();
}

template <int E>
hipError_t launch_e(const PrefillParams& p, bool rbf, int ub, hipStream_t stream) {
  if (ub == kBiasF32) return rbf ? launch_t<E, kRbf, kBiasF32>(p, stream) : launch_t<E, kDotAny, kBiasF32>(p, stream);
  if (ub == kBiasBool) return rbf ? launch_t<E, kRbf, kBiasBool>(p, stream) : launch_t<E, kDotAny, kBiasBool>(p, stream);
  if (rbf) return p.c_logit > 0.f ? launch_t<E, kRbfFold, kBiasNone>(p, stream) : launch_t<E, kRbf, kBiasNone>(p, stream);
  if (p.c_logit > 0.f) return launch_t<E, kDotPos, kBiasNone>(p, stream);
  return launch_t<E, kDotAny, kBiasNone>(p, stream);
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
  p.key_len = a.key_len;
  p.ubias = a.bias;
  p.ub_sn = a.bias_sn;
  p.ub_sh = a.bias_sh;
  p.num_q_tiles = (a.L + BM - 1) / BM;
  p.xcd_groups = ((a.N * a.Hkv) % 8 == 0) ? 1 : 0;
  p.xcd_contig = (a.bias && a.bias_sh == 0) ? 1 : 0;
  p.heavy_first = p.causal;
  const int ub = a.bias ? a.bias_kind : kBiasNone;
  if (a.E == 128) return launch_e<128>(p, a.rbf != 0, ub, stream);
  return launch_e<64>(p, a.rbf != 0, ub, stream);
}

}  // namespace attn_impl
