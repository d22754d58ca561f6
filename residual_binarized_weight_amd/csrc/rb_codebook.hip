// rb_codebook.hip -- sub-1-bit binary codebook: encode and product (gfx950).
//
// [BTC-LLM page, 2.1.1] The sign matrix is cut into v-column +-1 sub-vectors; each is
// replaced by the index of its nearest codeword in Hamming distance (XOR + popcount).
// [BTC-LLM page, 2.1.2 and 3.2.1] The product runs on the indices with one scale per
// 16 weights, without dequantising the matrix.
#include "rb_device.hpp"
#include "rb_internal.h"

namespace rb {
namespace {

// v bits of row `prow` starting at column c (bit t = column c + t); columns >= K read as 1.
__device__ __forceinline__ uint32_t extract_block(const uint32_t* __restrict__ prow, int64_t K,
                                                  int64_t c, int v) {
  const int64_t Kw = (K + 31) >> 5;
  const int64_t w = c >> 5;
  const int sh = (int)(c & 31);
  const uint32_t lo = w < Kw ? prow[w] : 0u;
  const uint32_t hi = (w + 1) < Kw ? prow[w + 1] : 0u;
  const uint64_t both = ((uint64_t)hi << 32) | lo;
  const uint32_t vmask = v == 32 ? 0xffffffffu : ((1u << v) - 1u);
  uint32_t b = (uint32_t)(both >> sh) & vmask;
  const int64_t real = K - c;  // columns of this block that exist
  if (real < v) b |= vmask & ~((1u << real) - 1u);
  return b;
}

constexpr int kEncodeTile = 8192;  // codewords staged in LDS per round (32 KB)
constexpr int kPatternsPerThread = 4;

// Each thread keeps kPatternsPerThread patterns; the block streams the codebook through
// LDS and every thread scores all staged codewords against its patterns. The running
// best is the packed key (distance << 16 | index), whose unsigned minimum is the nearest
// codeword with ties to the lowest index.
__global__ __launch_bounds__(256) void encode_kernel(const uint32_t* __restrict__ plane, int64_t ldp,
                                                     int64_t N, int64_t K,
                                                     const uint32_t* __restrict__ codebook, int c,
                                                     int v, uint16_t* __restrict__ idx) {
  __shared__ uint32_t cb[kEncodeTile];
  const int64_t nb = (K + v - 1) / v;
  const int64_t total = N * nb;
  const int64_t base = ((int64_t)blockIdx.x * blockDim.x + threadIdx.x) * kPatternsPerThread;
  uint32_t pat[kPatternsPerThread];
  uint32_t best[kPatternsPerThread];
#pragma unroll
  for (int p = 0; p < kPatternsPerThread; ++p) {
    const int64_t e = base + p;
    pat[p] = 0u;
    best[p] = 0xffffffffu;
    if (e < total) {
      const int64_t n = e / nb;
      const int64_t j = e - n * nb;
      pat[p] = extract_block(plane + n * ldp, K, j * v, v);
    }
  }
  for (int t0 = 0; t0 < c; t0 += kEncodeTile) {
    const int cnt = (c - t0) < kEncodeTile ? (c - t0) : kEncodeTile;
    __syncthreads();
    for (int t = threadIdx.x; t < cnt; t += blockDim.x) cb[t] = codebook[t0 + t];
    __syncthreads();
    for (int t = 0; t < cnt; ++t) {
      const uint32_t cw = cb[t];
      const uint32_t id = (uint32_t)(t0 + t);
#pragma unroll
      for (int p = 0; p < kPatternsPerThread; ++p) {
        const uint32_t key = ((uint32_t)__popc(pat[p] ^ cw) << 16) | id;
        best[p] = key < best[p] ? key : best[p];
      }
    }
  }
#pragma unroll
  for (int p = 0; p < kPatternsPerThread; ++p) {
    const int64_t e = base + p;
    if (e < total) idx[e] = (uint16_t)(best[p] & 0xffffu);
  }
}

// Product: one wave per output row and batch row; lane l takes blocks l, l+64, ...
__global__ __launch_bounds__(256) void codebook_gemv_kernel(
    const uint16_t* __restrict__ idx, const uint32_t* __restrict__ codebook, int c, int v,
    const __half* __restrict__ s, int group, int64_t N, int64_t K, const __half* __restrict__ x,
    int64_t M, __half* __restrict__ y) {
  const int lane = threadIdx.x & 63;
  const int64_t n = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  const int64_t m = blockIdx.y;
  if (n >= N) return;
  const int64_t nb = (K + v - 1) / v;
  const int64_t G = (K + group - 1) / group;
  float acc = 0.0f;
  for (int64_t j = lane; j < nb; j += 64) {
    const uint32_t id = idx[n * nb + j];
    const uint32_t cw = codebook[id < (uint32_t)c ? id : (uint32_t)(c - 1)];  // indices must be < c
    for (int t = 0; t < v; ++t) {
      const int64_t col = j * v + t;
      if (col >= K) break;
      const float sx = __half2float(s[n * G + col / group]) * __half2float(x[m * K + col]);
      acc += ((cw >> t) & 1u) ? sx : -sx;
    }
  }
  acc = wave_sum(acc);
  if (lane == 0) y[m * N + n] = __float2half_rn(acc);
}

}  // namespace

hipError_t launch_codebook_encode(const uint32_t* plane, int64_t ldp, int64_t N, int64_t K,
                                  const uint32_t* codebook, int c, int v, uint16_t* idx,
                                  hipStream_t s) {
  const int64_t nb = (K + v - 1) / v;
  const int64_t total = N * nb;
  const int64_t per_block = 256 * kPatternsPerThread;
  const unsigned grid = (unsigned)((total + per_block - 1) / per_block);
  encode_kernel<<<grid, 256, 0, s>>>(plane, ldp, N, K, codebook, c, v, idx);
  return hipGetLastError();
}

size_t codebook_gemv_workspace_bytes(int64_t, int64_t, int64_t) { return 0; }

hipError_t launch_codebook_gemv(const uint16_t* idx, const uint32_t* codebook, int c, int v,
                                const void* s, int group, int64_t N, int64_t K, const void* x,
                                int64_t M, void* y, void*, hipStream_t st) {
  const dim3 grid((unsigned)((N + 3) / 4), (unsigned)M);
  codebook_gemv_kernel<<<grid, 256, 0, st>>>(idx, codebook, c, v, static_cast<const __half*>(s), group,
                                             N, K, static_cast<const __half*>(x), M,
                                             static_cast<__half*>(y));
  return hipGetLastError();
}

}  // namespace rb
