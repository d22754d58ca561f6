// rb_gemv.hip -- matmul-free product on packed sign planes, decode-sized batches (gfx950).
//
// [RaBiT summary page, background "Residual binarization"] Each plane is a +-1 matrix
// with a row scale g_i and a column scale h_i; inference needs additions and element-wise
// scaling only:  y = sum_i g_i (.) (B_i (h_i (.) x)).
//
// Masked-add identity: for a +-1 row b, sum_c b_c x'_c = 2 * sum_{c: bit=1} x'_c - sum_c x'_c,
// so each plane only needs T_i = the sum of x'_i = h_i (.) x over the set bits, plus the
// full sum S_i; y = sum_i g_i (2 T_i - S_i), all in fp32.
//
// Direct kernel (any M <= 16): a block stages x'_i for a 2048-column chunk of an m-block
// in LDS (fp32, 36-float stride per 32 columns so that 16-byte reads by 8 consecutive
// lanes cover all 32 banks); each lane owns one 32-column word of the chunk, keeps the
// 32 x' values of that word in registers and applies them to the words of the wave's
// rows. Row totals come from a wave butterfly.
#include "rb_device.hpp"
#include "rb_internal.h"

namespace rb {
namespace {

constexpr int kChunkCols = 2048;          // 64 lanes x 32 columns
constexpr int kSegStride = 36;            // floats per 32-column segment in LDS
constexpr int kRowsPerWave = 4;
constexpr int kWavesPerBlock = 4;

template <typename T> __device__ __forceinline__ void store_out(T* p, float v);
template <> __device__ __forceinline__ void store_out<float>(float* p, float v) { *p = v; }
template <> __device__ __forceinline__ void store_out<__half>(__half* p, float v) {
  *p = __float2half_rn(v);
}

template <typename TX, typename TS, typename TY, int MB>
__global__ __launch_bounds__(256) void gemv_direct_kernel(
    const uint32_t* __restrict__ planes, int64_t ldp, const TS* __restrict__ g,
    const TS* __restrict__ h, int k, int64_t N, int64_t K, const TX* __restrict__ x, int64_t M,
    TY* __restrict__ y) {
  __shared__ __align__(16) float xs[MB][(kChunkCols / 32) * kSegStride];
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int64_t row0 = ((int64_t)blockIdx.x * kWavesPerBlock + wave) * kRowsPerWave;
  const int64_t m0 = (int64_t)blockIdx.y * MB;
  const int64_t Kw = (K + 31) >> 5;

  float yacc[kRowsPerWave][MB];
#pragma unroll
  for (int r = 0; r < kRowsPerWave; ++r)
#pragma unroll
    for (int m = 0; m < MB; ++m) yacc[r][m] = 0.0f;

  for (int i = 0; i < k; ++i) {
    float Tacc[kRowsPerWave][MB];
    float Sacc[MB];
#pragma unroll
    for (int m = 0; m < MB; ++m) {
      Sacc[m] = 0.0f;
#pragma unroll
      for (int r = 0; r < kRowsPerWave; ++r) Tacc[r][m] = 0.0f;
    }
    for (int64_t c0 = 0; c0 < K; c0 += kChunkCols) {
      __syncthreads();
      for (int idx = threadIdx.x; idx < MB * kChunkCols; idx += blockDim.x) {
        const int m = idx / kChunkCols;
        const int c = idx - m * kChunkCols;
        const int64_t col = c0 + c;
        float v = 0.0f;
        if (m0 + m < M && col < K) {
          v = to_f32(x[(m0 + m) * K + col]);
          if (h) v *= to_f32(h[(int64_t)i * K + col]);  // exact: fp16*fp16 fits fp32
        }
        xs[m][(c >> 5) * kSegStride + (c & 31)] = v;
      }
      __syncthreads();
      const int64_t wi = (c0 >> 5) + lane;
      uint32_t words[kRowsPerWave];
#pragma unroll
      for (int r = 0; r < kRowsPerWave; ++r) {
        const int64_t row = row0 + r;
        words[r] = (row < N && wi < Kw) ? planes[((int64_t)i * N + row) * ldp + wi] : 0u;
      }
#pragma unroll
      for (int m = 0; m < MB; ++m) {
        float xr[32];
        const float4* src = reinterpret_cast<const float4*>(&xs[m][lane * kSegStride]);
#pragma unroll
        for (int q = 0; q < 8; ++q) {
          const float4 t = src[q];
          xr[4 * q + 0] = t.x;
          xr[4 * q + 1] = t.y;
          xr[4 * q + 2] = t.z;
          xr[4 * q + 3] = t.w;
        }
        float s = 0.0f;
#pragma unroll
        for (int j = 0; j < 32; ++j) s += xr[j];
        Sacc[m] += s;
#pragma unroll
        for (int r = 0; r < kRowsPerWave; ++r) {
          float t = 0.0f;
#pragma unroll
          for (int j = 0; j < 32; ++j) t += ((words[r] >> j) & 1u) ? xr[j] : 0.0f;
          Tacc[r][m] += t;
        }
      }
    }
#pragma unroll
    for (int m = 0; m < MB; ++m) {
      const float S = wave_sum(Sacc[m]);
#pragma unroll
      for (int r = 0; r < kRowsPerWave; ++r) {
        const float T = wave_sum(Tacc[r][m]);
        const int64_t row = row0 + r;
        const float gi = row < N ? to_f32(g[(int64_t)i * N + row]) : 0.0f;
        yacc[r][m] += gi * (2.0f * T - S);
      }
    }
  }
#pragma unroll
  for (int r = 0; r < kRowsPerWave; ++r) {
#pragma unroll
    for (int m = 0; m < MB; ++m) {
      const int64_t row = row0 + r;
      if (lane == r * MB + m && row < N && m0 + m < M) store_out<TY>(&y[(m0 + m) * N + row], yacc[r][m]);
    }
  }
}

template <typename TX, typename TS, typename TY>
hipError_t launch_direct(const uint32_t* planes, int64_t ldp, const void* g, const void* h, int k,
                         int64_t N, int64_t K, const void* x, int64_t M, void* y, hipStream_t s) {
  const int64_t rows_per_block = (int64_t)kRowsPerWave * kWavesPerBlock;
  const unsigned gx = (unsigned)((N + rows_per_block - 1) / rows_per_block);
  if (M == 1) {
    gemv_direct_kernel<TX, TS, TY, 1><<<dim3(gx, 1), dim3(256), 0, s>>>(
        planes, ldp, static_cast<const TS*>(g), static_cast<const TS*>(h), k, N, K,
        static_cast<const TX*>(x), M, static_cast<TY*>(y));
  } else {
    gemv_direct_kernel<TX, TS, TY, 4><<<dim3(gx, (unsigned)((M + 3) / 4)), dim3(256), 0, s>>>(
        planes, ldp, static_cast<const TS*>(g), static_cast<const TS*>(h), k, N, K,
        static_cast<const TX*>(x), M, static_cast<TY*>(y));
  }
  return hipGetLastError();
}

template <typename TX, typename TS>
hipError_t launch_y(rb_dtype y_dtype, const uint32_t* planes, int64_t ldp, const void* g,
                    const void* h, int k, int64_t N, int64_t K, const void* x, int64_t M, void* y,
                    hipStream_t s) {
  if (y_dtype == RB_F16) return launch_direct<TX, TS, __half>(planes, ldp, g, h, k, N, K, x, M, y, s);
  return launch_direct<TX, TS, float>(planes, ldp, g, h, k, N, K, x, M, y, s);
}

template <typename TX>
hipError_t launch_s(rb_dtype scale_dtype, rb_dtype y_dtype, const uint32_t* planes, int64_t ldp,
                    const void* g, const void* h, int k, int64_t N, int64_t K, const void* x,
                    int64_t M, void* y, hipStream_t s) {
  if (scale_dtype == RB_F16) return launch_y<TX, __half>(y_dtype, planes, ldp, g, h, k, N, K, x, M, y, s);
  return launch_y<TX, float>(y_dtype, planes, ldp, g, h, k, N, K, x, M, y, s);
}

}  // namespace

size_t gemv_workspace_bytes(int, int64_t, int64_t, int64_t) { return 0; }

hipError_t launch_gemv(const uint32_t* planes, int64_t ldp, const void* g, const void* h,
                       rb_dtype scale_dtype, int k, int64_t N, int64_t K, const void* x,
                       rb_dtype x_dtype, int64_t M, void* y, rb_dtype y_dtype, void*, hipStream_t s) {
  if (x_dtype == RB_F16)
    return launch_s<__half>(scale_dtype, y_dtype, planes, ldp, g, h, k, N, K, x, M, y, s);
  return launch_s<float>(scale_dtype, y_dtype, planes, ldp, g, h, k, N, K, x, M, y, s);
}

}  // namespace rb
