// rb_bench.hip -- measurement probes, not part of the method: the HBM read rate a plain
// kernel reaches for a given footprint, and the rate of random 4-byte reads from a small
// table; the ceilings against which the product kernels are read.
#include "rb_device.hpp"

namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

__global__ __launch_bounds__(256) void stream_read_kernel(const u32x4* __restrict__ src, int64_t n16,
                                                          uint32_t* __restrict__ sink) {
  // each thread keeps 4 independent 16-byte loads in flight per iteration
  uint32_t acc = 0u;
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  for (; i + 3 * stride < n16; i += 4 * stride) {
    const u32x4 a = __builtin_nontemporal_load(src + i);
    const u32x4 b = __builtin_nontemporal_load(src + i + stride);
    const u32x4 c = __builtin_nontemporal_load(src + i + 2 * stride);
    const u32x4 d = __builtin_nontemporal_load(src + i + 3 * stride);
    acc ^= a.x ^ a.y ^ a.z ^ a.w ^ b.x ^ b.y ^ b.z ^ b.w ^ c.x ^ c.y ^ c.z ^ c.w ^ d.x ^ d.y ^ d.z ^ d.w;
  }
  for (; i < n16; i += stride) {
    const u32x4 v = __builtin_nontemporal_load(src + i);
    acc ^= v.x ^ v.y ^ v.z ^ v.w;
  }
  if (acc == 0x9e3779b9u) sink[0] = acc;  // keeps the loads alive; practically never taken
}

}  // namespace

extern "C" int rb_bench_stream_read(const void* src, int64_t bytes, uint32_t* sink, int32_t blocks,
                                    void* stream) {
  if (!src || !sink || bytes < 16 || blocks < 1) return 1;
  stream_read_kernel<<<blocks, 256, 0, static_cast<hipStream_t>(stream)>>>(
      static_cast<const u32x4*>(src), bytes / 16, sink);
  return hipGetLastError() == hipSuccess ? 0 : 5;
}

namespace {

// Random 4-byte gathers from a table of `mask + 1` dwords (a power of two): each thread
// makes `per_thread` reads at indices from its own linear congruential sequence. With a
// 256 KB table this is the rate of the codeword reads of the codebook product.
__global__ __launch_bounds__(256) void gather_kernel(const uint32_t* __restrict__ table, uint32_t mask,
                                                     int32_t per_thread, uint32_t* __restrict__ sink) {
  uint32_t h = (blockIdx.x * 256u + threadIdx.x) * 2654435761u + 12345u;
  uint32_t acc = 0u;
  for (int32_t g = 0; g < per_thread; g += 8) {
    uint32_t v[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      h = h * 1664525u + 1013904223u;
      v[u] = table[(h >> 7) & mask];
    }
#pragma unroll
    for (int u = 0; u < 8; ++u) acc += v[u];
  }
  if (acc == 0x9e3779b9u) sink[0] = acc;  // keeps the loads alive; practically never taken
}

}  // namespace

extern "C" int rb_bench_gather(const uint32_t* table, uint32_t entries, int32_t per_thread, uint32_t* sink,
                               int32_t blocks, void* stream) {
  if (!table || !sink || entries == 0 || (entries & (entries - 1)) != 0 || per_thread < 8 ||
      per_thread % 8 != 0 || blocks < 1)
    return 1;
  gather_kernel<<<blocks, 256, 0, static_cast<hipStream_t>(stream)>>>(table, entries - 1, per_thread, sink);
  return hipGetLastError() == hipSuccess ? 0 : 5;
}
