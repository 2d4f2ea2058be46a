// device_common.h -- small device-side helpers shared by the gfx950 kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace attn_dev {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr float kNegInf = -__builtin_huge_valf();

// Exact widening of the low / high bf16 halves of a packed dword.
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// Sum of squares of the 8 bf16 values in a 16-byte chunk, in fp32 (products are
// exact): v_dot2_f32_bf16 of each packed pair with itself, two squares per instruction.
__device__ __forceinline__ float sumsq8(u32x4 c) {
  typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
  float s = 0.f;
  const uint32_t w[4] = {c[0], c[1], c[2], c[3]};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const bf16x2 x = __builtin_bit_cast(bf16x2, w[i]);
    s = __builtin_amdgcn_fdot2_f32_bf16(x, x, s, false);
  }
  return s;
}

// Sum of v over aligned groups of N consecutive lanes (N = 8 or 16), result in
// every lane of the group; DPP row permutes, no LDS traffic.
template <int CTRL>
__device__ __forceinline__ float dpp_mov(float x) {
  return __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, x), CTRL, 0xF, 0xF, true));
}
template <int N>
__device__ __forceinline__ float group_sum(float v) {
  static_assert(N == 8 || N == 16, "group of 8 or 16 lanes");
  v += dpp_mov<0xB1>(v);   // quad_perm [1,0,3,2]: lane ^ 1
  v += dpp_mov<0x4E>(v);   // quad_perm [2,3,0,1]: lane ^ 2
  v += dpp_mov<0x141>(v);  // row_half_mirror: the other quad of the 8
  if (N == 16) v += dpp_mov<0x140>(v);  // row_mirror: the other 8 of the row
  return v;
}

// Round 8 floats to bf16 (nearest-even, v_cvt_pk_bf16_f32) as an MFMA operand.
__device__ __forceinline__ bf16x8 pack_bf16x8(float a0, float a1, float a2, float a3,
                                              float a4, float a5, float a6, float a7) {
  f32x8 f = {a0, a1, a2, a3, a4, a5, a6, a7};
  return __builtin_convertvector(f, bf16x8);
}

__device__ __forceinline__ bf16x4 pack_bf16x4(float a0, float a1, float a2, float a3) {
  f32x4 f = {a0, a1, a2, a3};
  return __builtin_convertvector(f, bf16x4);
}

__device__ __forceinline__ bf16x8 as_bf16x8(u32x4 v) { return __builtin_bit_cast(bf16x8, v); }

// 2^x on the hardware transcendental unit (v_exp_f32); 2^-inf = 0.
__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// Value held by lane (lane ^ mask) of the wave (LDS crossbar; any mask).
__device__ __forceinline__ float xor_lane(float v, int mask) { return __shfl_xor(v, mask, 64); }

// max / sum of v over the lane pair {l, l ^ 32} (v_permlane32_swap, no LDS).
// The swap hands each lane the values of both halves, in some order, which is
// all a symmetric combine needs.
__device__ __forceinline__ float pair32_max(float v) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float pair32_sum(float v) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
// Same for the pair {l, l ^ 16} (v_permlane16_swap).
__device__ __forceinline__ float pair16_max(float v) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float pair16_sum(float v) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// Buffer resource over `bytes` bytes at `base` (raw addressing, gfx9 data format
// word).  Loads through it whose byte offset lies at or past `bytes` return
// zeros without touching memory.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
}
__device__ __forceinline__ u32x4 buffer_load16(__amdgpu_buffer_rsrc_t r, uint32_t byte_off) {
  return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, (int)byte_off, 0, 0));
}

// Stores through a buffer resource: a byte offset at or past the resource's
// size writes nothing (the hardware's range check), so a store of a row that may
// lie past the end of a tensor needs no branch around it.
__device__ __forceinline__ void buffer_store16(__amdgpu_buffer_rsrc_t r, uint32_t byte_off, u32x4 v) {
  __builtin_amdgcn_raw_buffer_store_b128(v, r, (int)byte_off, 0, 0);
}
// The same with the non-temporal hint (cache policy bit 1), for outputs written
// once and not read back by the kernel.
__device__ __forceinline__ void buffer_store16_nt(__amdgpu_buffer_rsrc_t r, uint32_t byte_off, u32x4 v) {
  __builtin_amdgcn_raw_buffer_store_b128(v, r, (int)byte_off, 0, 2);
}
__device__ __forceinline__ void buffer_store4(__amdgpu_buffer_rsrc_t r, uint32_t byte_off, float v) {
  __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(v), r, (int)byte_off, 0, 0);
}

// Two bf16 halves (low halves when hi == false, else high halves) of a and b
// packed as {a_half, b_half} (v_perm_b32).
__device__ __forceinline__ uint32_t pack_halves(uint32_t a, uint32_t b, bool hi) {
  return __builtin_amdgcn_perm(b, a, hi ? 0x07060302u : 0x05040100u);
}

// 16-byte global load that returns zeros when `ok` is false (no access is made then).
__device__ __forceinline__ u32x4 load16_or_zero(const uint16_t* p, bool ok) {
  u32x4 z = {0u, 0u, 0u, 0u};
  return ok ? *reinterpret_cast<const u32x4*>(p) : z;
}

// The same with the non-temporal hint, for data a kernel streams exactly once
// (decode K/V, packed SOCKET codes): such lines are not kept in the caches for
// reuse, which measured 10-13 % more read bandwidth on long streams.
__device__ __forceinline__ u32x4 load16_nt_or_zero(const uint16_t* p, bool ok) {
  u32x4 z = {0u, 0u, 0u, 0u};
  return ok ? __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p)) : z;
}

}  // namespace attn_dev
