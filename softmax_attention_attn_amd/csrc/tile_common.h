// tile_common.h -- LDS tile helpers shared by the bf16 MFMA kernels (forward
// prefill and backward): the XOR swizzle of 16-byte chunks in row-major
// (rows x E) bf16 tiles, the transposing LDS read, and the wave-wide
// LDS-direct buffer load.
#pragma once

#include "device_common.h"

namespace attn_dev {

// XOR permutation of the 16-byte chunks of tile row r (K and V tiles are
// row-major, E*2 bytes per row).  E = 128: 16 consecutive rows map one chunk to
// 16 different chunk slots (conflict-free K reads), and the 4 consecutive rows x
// 4 chunks that a transposing V read touches in each half-wave land in 16
// different slots.  E = 64 (two rows share a 64-bank span): the same two
// properties per bank half.
template <int E>
__device__ __forceinline__ int tile_swz(int r) {
  if (E == 128) return ((r & 3) << 2) | ((r >> 2) & 3);
  return (((r >> 1) & 1) << 2) | ((r >> 2) & 3);
}

typedef short shortx4 __attribute__((ext_vector_type(4)));

// The two helpers below wrap gfx950 builtins that take LDS pointers.  Their
// bodies exist only in the device compilation pass: in the host pass clang
// otherwise drops the launch stubs of the kernel templates that use them
// (the host pass never executes device code; it only needs the declarations).

// Transposing 8-byte LDS read (ds_read_b64_tr_b16) at byte address a.
__device__ __forceinline__ shortx4 lds_read_tr(const uint8_t* a) {
#if defined(__HIP_DEVICE_COMPILE__)
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (__attribute__((address_space(3))) shortx4*)(const_cast<uint8_t*>(a)));
#else
  (void)a;
  return shortx4{0, 0, 0, 0};
#endif
}

// Wave-wide LDS-direct load: lane l's 16 bytes at byte offset `off` of the
// buffer land at lds + 16*l (zeros if `off` is past the buffer's range).
__device__ __forceinline__ void buffer_load16_to_lds(__amdgpu_buffer_rsrc_t r, uint8_t* lds, uint32_t off) {
#if defined(__HIP_DEVICE_COMPILE__)
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, lds, 16, (int)off, 0, 0, 0);
#else
  (void)r;
  (void)lds;
  (void)off;
#endif
}

}  // namespace attn_dev
