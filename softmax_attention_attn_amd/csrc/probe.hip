// probe.hip -- HBM bandwidth probes (include/attn_probe.h): a streaming read
// and a streaming copy with 16-byte non-temporal accesses, each workgroup
// streaming one contiguous chunk (as a decode split streams its keys), a grid
// of up to 16 workgroups per CU.
#include <hip/hip_runtime.h>

#include <cstdint>

#include "attn.h"
#include "attn_probe.h"

namespace {

typedef uint32_t u32x4p __attribute__((ext_vector_type(4)));

constexpr int PT = 256;           // threads per workgroup
constexpr size_t PBLOCKS = 4096;  // workgroups at most (16 per CU)
constexpr int UR = 16;            // 16-byte pieces in flight per lane (read)
constexpr int UC = 8;             // 16-byte pieces in flight per lane (copy)

size_t grid_for(size_t n16) {
  const size_t want = (n16 + PT - 1) / PT;
  return want < PBLOCKS ? want : PBLOCKS;
}

// Workgroup b streams the contiguous chunk [b*chunk, min((b+1)*chunk, n)) of
// 16-byte pieces; each step of a wave covers U whole KB.  (Measured on MI355X
// over 1 GiB: a chunk per workgroup reads at 6.9-7.1 TB/s and copies at
// 5.5-5.6 TB/s, where a grid-stride loop over the whole buffer reaches 5.5-5.9
// and 4.2-4.6.)
__global__ __launch_bounds__(PT) void probe_read_kernel(const u32x4p* __restrict__ src, size_t n, size_t chunk,
                                                        uint32_t* sink) {
  const size_t b0 = (size_t)blockIdx.x * chunk;
  const size_t b1 = b0 + chunk < n ? b0 + chunk : n;
  u32x4p a = {0u, 0u, 0u, 0u};
  size_t i = b0 + threadIdx.x;
  for (; i + (UR - 1) * PT < b1; i += UR * PT) {
    u32x4p x[UR];
#pragma unroll
    for (int u = 0; u < UR; ++u) x[u] = __builtin_nontemporal_load(src + i + u * PT);
#pragma unroll
    for (int u = 0; u < UR; ++u) a ^= x[u];
  }
  for (; i < b1; i += PT) a ^= __builtin_nontemporal_load(src + i);
  uint32_t r = a[0] ^ a[1] ^ a[2] ^ a[3];
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) r ^= (uint32_t)__shfl_xor((int)r, o, 64);
  if ((threadIdx.x & 63) == 0) sink[(size_t)blockIdx.x * (PT / 64) + (threadIdx.x >> 6)] = r;
}

__global__ __launch_bounds__(PT) void probe_copy_kernel(const u32x4p* __restrict__ src, u32x4p* __restrict__ dst,
                                                        size_t n, size_t chunk) {
  const size_t b0 = (size_t)blockIdx.x * chunk;
  const size_t b1 = b0 + chunk < n ? b0 + chunk : n;
  size_t i = b0 + threadIdx.x;
  for (; i + (UC - 1) * PT < b1; i += UC * PT) {
    u32x4p x[UC];
#pragma unroll
    for (int u = 0; u < UC; ++u) x[u] = __builtin_nontemporal_load(src + i + u * PT);
#pragma unroll
    for (int u = 0; u < UC; ++u) __builtin_nontemporal_store(x[u], dst + i + u * PT);
  }
  for (; i < b1; i += PT) __builtin_nontemporal_store(__builtin_nontemporal_load(src + i), dst + i);
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15) == 0; }

}  // namespace

#pragma GCC visibility push(default)
extern "C" {

size_t attn_probe_sink_words(size_t bytes) { return grid_for(bytes / 16) * (PT / 64); }

int attn_probe_read(const void* src, size_t bytes, unsigned int* sink, void* stream) {
  if (bytes == 0) return ATTN_OK;
  if (!src || !sink) return ATTN_ERR_NULL;
  if (!aligned16(src) || (reinterpret_cast<uintptr_t>(sink) & 3)) return ATTN_ERR_ALIGN;
  if (bytes % 16) return ATTN_ERR_SHAPE;
  const size_t n = bytes / 16, grid = grid_for(n), chunk = (n + grid - 1) / grid;
  hipLaunchKernelGGL(probe_read_kernel, dim3((unsigned)grid), dim3(PT), 0, static_cast<hipStream_t>(stream),
                     static_cast<const u32x4p*>(src), n, chunk, sink);
  return hipGetLastError() == hipSuccess ? ATTN_OK : ATTN_ERR_HIP;
}

int attn_probe_copy(const void* src, void* dst, size_t bytes, void* stream) {
  if (bytes == 0) return ATTN_OK;
  if (!src || !dst) return ATTN_ERR_NULL;
  if (!aligned16(src) || !aligned16(dst)) return ATTN_ERR_ALIGN;
  if (bytes % 16) return ATTN_ERR_SHAPE;
  const size_t n = bytes / 16, grid = grid_for(n), chunk = (n + grid - 1) / grid;
  hipLaunchKernelGGL(probe_copy_kernel, dim3((unsigned)grid), dim3(PT), 0, static_cast<hipStream_t>(stream),
                     static_cast<const u32x4p*>(src), static_cast<u32x4p*>(dst), n, chunk);
  return hipGetLastError() == hipSuccess ? ATTN_OK : ATTN_ERR_HIP;
}

}  // extern "C"
#pragma GCC visibility pop
