// rb_qat.hip -- the coupled-training layer: paths derived from one shared weight on every
// forward, straight-through backward with scale gradients.
//
// [RaBiT, "Method step details", Algorithm 2]
//   forward:  R_0 = W; for i = 1..k: B_i = sign(R_{i-1}) (0 -> +1), What_i = g_i (.) B_i (.) h_i,
//             R_i = R_{i-1} - What_i; the layer multiplies by What = sum_i What_i: Y = X What^T.
//   backward: dW = dY^T X is the shared weight's gradient (the derivation is not
//             differentiated); dX = dY What; the scales by the chain rule with B_i constant:
//             dg_i[n] = sum_c dW[n,c] B_i[n,c] h_i[c],  dh_i[c] = sum_n dW[n,c] B_i[n,c] g_i[n].
//
// Kernels of this file:
//   qat_derive_kernel      one pass over W: the k sign planes and What (fp16 or bf16). The
//                          residual is fp64 in the order above, so every sign is the one an
//                          fp64 evaluation gives; What is the fp64 sum rounded once.
//   qat_scale_grad_kernel  one pass over dW and the planes: per 256-column strip row partials
//                          of dg and per 256-row tile column partials of dh, fixed order.
//   qat_scale_grad_finish  the partials summed in a fixed order.
// The three dense products (Y, dW, dX) are rocBLAS GEMMs with fp32 accumulation on one handle
// per device; the forward product Y = X What^T also has this library's matrix-core kernel
// (rb_qat_gemm.hip), which rb_qat_forward uses for a shape where rb_qat_autotune timed it at
// least as fast as rocBLAS's best.
#define ROCBLAS_BETA_FEATURES_API  // rocblas_gemm_ex_get_solutions
#include <rocblas/rocblas.h>

#include <algorithm>
#include <array>
#include <cstdio>
#include <cstdlib>
#include <functional>
#include <map>
#include <mutex>
#include <utility>
#include <vector>

#include "rb_device.hpp"
#include "rb_internal.h"

namespace rb {
namespace {

// ---------------------------------------------------------------------------------------------
// derivation
// ---------------------------------------------------------------------------------------------
// round a finite double to the nearest bf16 (ties to even), directly. fp64 -> fp32 is first
// made round-to-odd (the RNE conversion, stepped back toward zero when it went away from it,
// then the last bit forced to 1 if inexact); with fp32's 16 spare bits below bf16's last
// bit, the RNE rounding of that to bf16 equals the direct rounding of the double.
__device__ __forceinline__ uint16_t f64_to_bf16_bits_rne(double d) {
  const float f = (float)d;
  uint32_t u = __float_as_uint(f);
  const double back = (double)f;
  if (back != d) {
    if (fabs(back) > fabs(d)) u -= 1u;  // magnitude one fp32 ulp down (also from inf to FLT_MAX)
    u |= 1u;
  }
  u += 0x7fffu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

constexpr int kDeriveWaves = 4;   // waves per block
constexpr int kDeriveSteps = 8;   // 64-column steps per wave: a chunk of 512 columns
constexpr int kDeriveRows = 4;    // rows per wave, sharing the chunk's h values

// Wave task t: rows 4 (t / nchunk) .. +3, columns 512 (t % nchunk) .. +511, lane l column
// 512 c + 64 j + l of step j. Every load goes through a buffer resource clipped at the row's
// end (columns past K read 0); stores past K are masked.
template <int KP, bool BF16>
__global__ __launch_bounds__(64 * kDeriveWaves) void qat_derive_kernel(
    const float* __restrict__ W, int64_t N, int64_t K, int64_t ldw, const float* __restrict__ g,
    const float* __restrict__ h, uint32_t* __restrict__ planes, int64_t ldp,
    uint16_t* __restrict__ What, int64_t ldwh, int64_t nchunk) {
  const int lane = threadIdx.x & (RB_WAVE - 1);
  const int64_t task = (int64_t)blockIdx.x * kDeriveWaves + (threadIdx.x >> 6);
  const int64_t n0 = (task / nchunk) * kDeriveRows;
  if (n0 >= N) return;  // uniform per wave
  const uint32_t chunk = (uint32_t)(task % nchunk);
  const uint32_t Kc = (uint32_t)K;
  const uint32_t Kw = (Kc + 31u) >> 5;
  const uint32_t c0 = chunk * (64u * kDeriveSteps);

  float hv[KP][kDeriveSteps];
#pragma unroll
  for (int i = 0; i < KP; ++i) {
    const __amdgpu_buffer_rsrc_t rh = buffer_rsrc(h + (int64_t)i * K, Kc * 4u);
#pragma unroll
    for (int j = 0; j < kDeriveSteps; ++j)
      hv[i][j] = __uint_as_float(buf_u32(rh, (c0 + 64u * j + (uint32_t)lane) * 4u, 0u));
  }

  // the next row's loads are issued before the current row is processed; a row past N reads 0
  // through an empty buffer range, so every load is unconditional
  auto load_row = [&](int64_t n, float (&v)[kDeriveSteps]) {
    const bool in = n < N;
    const __amdgpu_buffer_rsrc_t rw = buffer_rsrc(W + (in ? n : 0) * ldw, in ? Kc * 4u : 0u);
#pragma unroll
    for (int j = 0; j < kDeriveSteps; ++j)
      v[j] = __uint_as_float(buf_u32(rw, (c0 + 64u * j + (uint32_t)lane) * 4u, 0u));
  };
  float wv[kDeriveSteps];
  load_row(n0, wv);
#pragma unroll
  for (int r = 0; r < kDeriveRows; ++r) {
    const int64_t n = n0 + r;
    float wn[kDeriveSteps];
    if (r + 1 < kDeriveRows) load_row(n + 1, wn);
    if (n < N) {  // uniform
      double gd[KP];
#pragma unroll
      for (int i = 0; i < KP; ++i) gd[i] = (double)g[(int64_t)i * N + n];

      uint16_t* __restrict__ wrow = What + n * ldwh;
      uint32_t wlo[KP], whi[KP];  // lane j: the two words of step j, per plane
#pragma unroll
      for (int i = 0; i < KP; ++i) wlo[i] = whi[i] = 0u;
#pragma unroll
      for (int j = 0; j < kDeriveSteps; ++j) {
        const uint32_t col = c0 + 64u * j + (uint32_t)lane;
        const bool valid = col < Kc;
        double R = (double)wv[j];
        bool b = nonneg_bits(wv[j]);
        double acc = 0.0;
#pragma unroll
        for (int i = 0; i < KP; ++i) {
          if (i > 0) b = R >= 0.0;  // -0.0 >= 0 holds: sign(0) = +1
          const double gh = gd[i] * (double)hv[i][j];  // exact: <= 48 significant bits
          const double wi = b ? gh : -gh;
          acc += wi;
          if (i + 1 < KP) R -= wi;
          const uint64_t m = __ballot(valid && b);
          wlo[i] = lane == j ? (uint32_t)m : wlo[i];
          whi[i] = lane == j ? (uint32_t)(m >> 32) : whi[i];
        }
        if (valid) wrow[col] = BF16 ? f64_to_bf16_bits_rne(acc) : f64_to_f16_bits_rne(acc);
      }
      // lane j < kDeriveSteps stores words 2 j, 2 j + 1 of the chunk, per plane
      const uint32_t w0 = chunk * (2u * kDeriveSteps) + 2u * (uint32_t)lane;
#pragma unroll
      for (int i = 0; i < KP; ++i) {
        uint32_t* __restrict__ prow = planes + ((int64_t)i * N + n) * ldp;
        if (lane < kDeriveSteps && w0 < Kw) prow[w0] = wlo[i];
        if (lane < kDeriveSteps && w0 + 1u < Kw) prow[w0 + 1u] = whi[i];
      }
    }
    if (r + 1 < kDeriveRows) {
#pragma unroll
      for (int j = 0; j < kDeriveSteps; ++j) wv[j] = wn[j];
    }
  }
}

// ---------------------------------------------------------------------------------------------
// scale gradients
// ---------------------------------------------------------------------------------------------
constexpr int kSgWaves = 4;
constexpr int kSgStrip = 256;     // columns per block: 4 per lane
constexpr int kSgTileRows = 256;  // rows per block: wave w takes rows 4 j + w
constexpr int kSgUnroll = 8;      // rows whose loads are issued together

int64_t sg_strips(int64_t K) { return (K + kSgStrip - 1) / kSgStrip; }
int64_t sg_tiles(int64_t N) { return (N + kSgTileRows - 1) / kSgTileRows; }
size_t align256(size_t b) { return (b + 255) & ~(size_t)255; }

// Block (strip s, tile t). Lane l holds columns 256 s + 4 l .. +3 of each row it visits:
// t_i = dW (.) B_i there (sign applied by the plane bit). Row partial of dg_i: the lane's
// 4 products with h_i, summed over the wave (DPP, total in lane 63) and stored to
// rowpart[s][i][n]. Column partial of dh_i: each lane accumulates t_i g_i[n] over the rows of
// its wave in row order; the 4 waves are then added in wave order through LDS and stored to
// colpart[t][i][c]. Rows past N and columns past K read 0 through the buffer resources.
// vec16: every row of dW starts 16-byte aligned, so a lane's 4 columns are one 16-byte load.
template <int KP>
__global__ __launch_bounds__(64 * kSgWaves) void qat_scale_grad_kernel(
    const float* __restrict__ dW, int64_t N, int64_t K, int64_t lddw,
    const uint32_t* __restrict__ planes, int64_t ldp, const float* __restrict__ g,
    const float* __restrict__ h, float* __restrict__ rowpart, float* __restrict__ colpart, bool vec16) {
  __shared__ float red[kSgWaves][KP][kSgStrip];
  const int lane = threadIdx.x & (RB_WAVE - 1);
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const uint32_t Kc = (uint32_t)K;
  const uint32_t Kw = (Kc + 31u) >> 5;
  const int64_t strip = blockIdx.x;
  const int64_t tile = blockIdx.y;
  const uint32_t c = (uint32_t)strip * kSgStrip + 4u * (uint32_t)lane;  // first of 4 columns
  const uint32_t word = c >> 5;
  const uint32_t shift = c & 31u;

  float hq[KP][4];
#pragma unroll
  for (int i = 0; i < KP; ++i) {
    const __amdgpu_buffer_rsrc_t rh = buffer_rsrc(h + (int64_t)i * K, Kc * 4u);
#pragma unroll
    for (int q = 0; q < 4; ++q) hq[i][q] = __uint_as_float(buf_u32(rh, (c + q) * 4u, 0u));
  }
  float cacc[KP][4];
#pragma unroll
  for (int i = 0; i < KP; ++i)
#pragma unroll
    for (int q = 0; q < 4; ++q) cacc[i][q] = 0.0f;

  const int64_t nbase = tile * kSgTileRows + wave;
  for (int j0 = 0; j0 < kSgTileRows / kSgWaves; j0 += kSgUnroll) {
    if (nbase + (int64_t)kSgWaves * j0 >= N) break;  // uniform
    float4 dv[kSgUnroll];
    uint32_t bits[kSgUnroll][KP];
#pragma unroll
    for (int u = 0; u < kSgUnroll; ++u) {
      const int64_t n = nbase + (int64_t)kSgWaves * (j0 + u);
      const bool in = n < N;
      const int64_t nn = in ? n : 0;
      const __amdgpu_buffer_rsrc_t rd = buffer_rsrc(dW + nn * lddw, in ? Kc * 4u : 0u);
      if (vec16) {
        dv[u] = __builtin_bit_cast(float4, __builtin_amdgcn_raw_buffer_load_b128(rd, (int)(c * 4u), 0, 0));
      } else {
        dv[u] = make_float4(__uint_as_float(buf_u32(rd, c * 4u, 0u)), __uint_as_float(buf_u32(rd, c * 4u + 4u, 0u)),
                            __uint_as_float(buf_u32(rd, c * 4u + 8u, 0u)),
                            __uint_as_float(buf_u32(rd, c * 4u + 12u, 0u)));
      }
#pragma unroll
      for (int i = 0; i < KP; ++i) {
        const __amdgpu_buffer_rsrc_t rp = buffer_rsrc(planes + ((int64_t)i * N + nn) * ldp, in ? Kw * 4u : 0u);
        bits[u][i] = buf_u32(rp, word * 4u, 0u) >> shift;
      }
    }
#pragma unroll
    for (int u = 0; u < kSgUnroll; ++u) {
      const int64_t n = nbase + (int64_t)kSgWaves * (j0 + u);
      const bool in = n < N;  // uniform
      const float d4[4] = {dv[u].x, dv[u].y, dv[u].z, dv[u].w};
#pragma unroll
      for (int i = 0; i < KP; ++i) {
        const float gi = in ? g[(int64_t)i * N + n] : 0.0f;
        float rs = 0.0f;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const float t = ((bits[u][i] >> q) & 1u) ? d4[q] : -d4[q];
          rs = fmaf(t, hq[i][q], rs);
          cacc[i][q] = fmaf(t, gi, cacc[i][q]);
        }
        rs = wave_sum_dpp(rs);
        if (in && lane == 63) rowpart[(strip * KP + i) * N + n] = rs;
      }
    }
  }

#pragma unroll
  for (int i = 0; i < KP; ++i)
#pragma unroll
    for (int q = 0; q < 4; ++q) red[wave][i][4 * lane + q] = cacc[i][q];
  __syncthreads();
  const int t = threadIdx.x;  // one column of the strip per thread
  const uint32_t col = (uint32_t)strip * kSgStrip + (uint32_t)t;
  if (col < Kc) {
#pragma unroll
    for (int i = 0; i < KP; ++i) {
      float s = red[0][i][t];
#pragma unroll
      for (int v = 1; v < kSgWaves; ++v) s += red[v][i][t];
      colpart[(tile * KP + i) * K + col] = s;
    }
  }
}

// dg[i][n] = sum over strips of rowpart[s][i][n]; dh[i][c] = sum over tiles of colpart[t][i][c];
// each in strip / tile order.
__global__ __launch_bounds__(256) void qat_scale_grad_finish(const float* __restrict__ rowpart,
                                                             const float* __restrict__ colpart, int64_t N,
                                                             int64_t K, int kp, int64_t nstrip, int64_t ntile,
                                                             float* __restrict__ dg, float* __restrict__ dh) {
  const int64_t e = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int64_t nrow = (int64_t)kp * N;
  // loads batched 8 at a time (independent), added in index order
  auto ordered_sum = [](const float* __restrict__ p, int64_t stride, int64_t count) {
    float s = 0.0f;
    int64_t i = 0;
    for (; i + 8 <= count; i += 8) {
      float v[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) v[u] = p[(i + u) * stride];
#pragma unroll
      for (int u = 0; u < 8; ++u) s += v[u];
    }
    for (; i < count; ++i) s += p[i * stride];
    return s;
  };
  if (e < nrow) {
    dg[e] = ordered_sum(rowpart + e, nrow, nstrip);
  } else if (e < nrow + (int64_t)kp * K) {
    const int64_t f = e - nrow;
    dh[f] = ordered_sum(colpart + f, (int64_t)kp * K, ntile);
  }
}

// ---------------------------------------------------------------------------------------------
// dense products
// ---------------------------------------------------------------------------------------------
constexpr int kMaxDevices = 64;
std::mutex g_blas_mu;
rocblas_handle g_blas[kMaxDevices] = {};

rocblas_datatype blas_type(rb_dtype d) {
  return d == RB_F32 ? rocblas_datatype_f32_r : d == RB_F16 ? rocblas_datatype_f16_r : rocblas_datatype_bf16_r;
}

hipError_t blas_fail(const char* what, rocblas_status s) {
  if (std::getenv("RB_LOG")) std::fprintf(stderr, "librb: rocBLAS %s failed: %s\n", what, rocblas_status_to_string(s));
  return hipErrorLaunchFailure;
}

// One dense product: C[m][n] (column-major, ldc) = op(A) op(B), fp32 accumulation, alpha 1,
// beta 0; A and B in type `at`, C in `ct`.
struct GemmShape {
  rocblas_operation ta, tb;
  int64_t m, n, kk, lda, ldb, ldc;
  rb_dtype at, ct;
};

// Solutions chosen by rb_qat_autotune, per device and shape; a shape not in the table runs
// rocBLAS's default choice. g_blas_slower holds the forward shapes for which the matrix-core
// kernel of this library was timed at least as fast as rocBLAS's best.
using GemmKey = std::array<int64_t, 11>;
std::map<GemmKey, int32_t> g_tuned;
std::map<GemmKey, bool> g_blas_slower;

GemmKey gemm_key(int dev, const GemmShape& s) {
  return {dev, (int64_t)s.ta, (int64_t)s.tb, s.m, s.n, s.kk, s.lda, s.ldb, s.ldc, (int64_t)s.at, (int64_t)s.ct};
}

bool blas_ok(rocblas_status s) {
  // perf_degraded: computed, with less workspace than the fastest kernel wanted
  return s == rocblas_status_success || s == rocblas_status_perf_degraded;
}

rocblas_status gemm_run(rocblas_handle hd, const GemmShape& s, const void* A, const void* B, void* C, int32_t sol) {
  const float one = 1.0f, zero = 0.0f;
  return rocblas_gemm_ex(hd, s.ta, s.tb, (rocblas_int)s.m, (rocblas_int)s.n, (rocblas_int)s.kk, &one, A,
                         blas_type(s.at), (rocblas_int)s.lda, B, blas_type(s.at), (rocblas_int)s.ldb, &zero, C,
                         blas_type(s.ct), (rocblas_int)s.ldc, C, blas_type(s.ct), (rocblas_int)s.ldc,
                         rocblas_datatype_f32_r,
                         sol > 0 ? rocblas_gemm_algo_solution_index : rocblas_gemm_algo_standard, sol, 0);
}

// Caller holds g_blas_mu; the handle is bound to the stream first.
hipError_t gemm_locked(rocblas_handle hd, int dev, const GemmShape& s, const void* A, const void* B, void* C) {
  const auto it = g_tuned.find(gemm_key(dev, s));
  const rocblas_status st = gemm_run(hd, s, A, B, C, it == g_tuned.end() ? 0 : it->second);
  return blas_ok(st) ? hipSuccess : blas_fail("gemm_ex", st);
}

// Average time of `reps` runs of one solution (after one untimed run), or a negative value if
// the solution rejects the problem.
float time_solution(rocblas_handle hd, const GemmShape& s, const void* A, const void* B, void* C, int32_t sol,
                    int reps, hipStream_t stream, hipEvent_t e0, hipEvent_t e1) {
  if (!blas_ok(gemm_run(hd, s, A, B, C, sol))) return -1.0f;
  if (hipEventRecord(e0, stream) != hipSuccess) return -1.0f;
  for (int r = 0; r < reps; ++r) gemm_run(hd, s, A, B, C, sol);
  if (hipEventRecord(e1, stream) != hipSuccess || hipEventSynchronize(e1) != hipSuccess) return -1.0f;
  float ms = 0.0f;
  if (hipEventElapsedTime(&ms, e0, e1) != hipSuccess) return -1.0f;
  return ms / (float)reps;
}

// Times rocBLAS's default and every solution it lists for the shape (2 runs each), re-times
// the 8 fastest (5 runs each) and records the fastest in g_tuned; with `mine` (the forward
// product on the matrix-core kernel of this library) that kernel is timed as well (5 runs)
// and g_blas_slower records whether it was at least as fast. Caller holds g_blas_mu.
hipError_t autotune_locked(rocblas_handle hd, int dev, const GemmShape& s, const void* A, const void* B, void* C,
                           hipStream_t stream, const std::function<hipError_t()>& mine = nullptr) {
  const float one = 1.0f, zero = 0.0f;
  rocblas_int count = 0;
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Wdeprecated-declarations"
  auto list_solutions = [&](rocblas_int* list) {
    return rocblas_gemm_ex_get_solutions(
        hd, s.ta, s.tb, (rocblas_int)s.m, (rocblas_int)s.n, (rocblas_int)s.kk, &one, A, blas_type(s.at),
        (rocblas_int)s.lda, B, blas_type(s.at), (rocblas_int)s.ldb, &zero, C, blas_type(s.ct), (rocblas_int)s.ldc, C,
        blas_type(s.ct), (rocblas_int)s.ldc, rocblas_datatype_f32_r, rocblas_gemm_algo_solution_index, 0, list,
        &count);
  };
#pragma clang diagnostic pop
  rocblas_status st = list_solutions(nullptr);
  if (!blas_ok(st)) return blas_fail("gemm_ex_get_solutions", st);
  std::vector<rocblas_int> sols((size_t)count);
  if (count > 0) {
    st = list_solutions(sols.data());
    if (!blas_ok(st)) return blas_fail("gemm_ex_get_solutions", st);
  }
  sols.insert(sols.begin(), 0);  // 0: rocBLAS's default choice
  hipEvent_t e0, e1;
  if (hipEventCreate(&e0) != hipSuccess) return hipErrorOutOfMemory;
  if (hipEventCreate(&e1) != hipSuccess) {
    (void)hipEventDestroy(e0);
    return hipErrorOutOfMemory;
  }
  std::vector<std::pair<float, int32_t>> timed;
  for (rocblas_int sol : sols) {
    const float t = time_solution(hd, s, A, B, C, sol, 2, stream, e0, e1);
    if (t > 0.0f) timed.emplace_back(t, sol);
  }
  std::sort(timed.begin(), timed.end());
  if (timed.size() > 8) timed.resize(8);
  for (auto& tv : timed) {
    const float t = time_solution(hd, s, A, B, C, tv.second, 5, stream, e0, e1);
    tv.first = t > 0.0f ? t : 1e30f;
  }
  std::sort(timed.begin(), timed.end());
  float t_mine = -1.0f;
  if (mine && mine() == hipSuccess && hipEventRecord(e0, stream) == hipSuccess) {
    bool ok = true;
    for (int r = 0; r < 5 && ok; ++r) ok = mine() == hipSuccess;
    float ms = 0.0f;
    if (ok && hipEventRecord(e1, stream) == hipSuccess && hipEventSynchronize(e1) == hipSuccess &&
        hipEventElapsedTime(&ms, e0, e1) == hipSuccess)
      t_mine = ms / 5.0f;
  }
  (void)hipEventDestroy(e0);
  (void)hipEventDestroy(e1);
  const GemmKey key = gemm_key(dev, s);
  if (mine) g_blas_slower[key] = t_mine > 0.0f && (timed.empty() || t_mine <= timed.front().first);
  if (timed.empty()) {
    if (mine && g_blas_slower[key]) return hipStreamSynchronize(stream);
    return blas_fail("autotune", rocblas_status_not_implemented);
  }
  g_tuned[key] = timed.front().second;
  return hipStreamSynchronize(stream);
}

// The device's handle (created on first use), bound to `stream`; g_blas_mu must be held.
hipError_t blas_handle_locked(hipStream_t stream, rocblas_handle* out, int* dev_out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  if (!g_blas[dev]) {
    rocblas_status s = rocblas_create_handle(&g_blas[dev]);
    if (s != rocblas_status_success) {
      g_blas[dev] = nullptr;
      return blas_fail("create_handle", s);
    }
  }
  rocblas_status s = rocblas_set_stream(g_blas[dev], stream);
  if (s != rocblas_status_success) return blas_fail("set_stream", s);
  *out = g_blas[dev];
  *dev_out = dev;
  return hipSuccess;
}

template <int KP>
hipError_t derive_kp(const float* W, int64_t N, int64_t K, int64_t ldw, const float* g, const float* h,
                     uint32_t* planes, int64_t ldp, void* What, rb_dtype wt, int64_t ldwh, hipStream_t st) {
  const int64_t nchunk = (K + 64 * kDeriveSteps - 1) / (64 * kDeriveSteps);
  const int64_t tasks = (N + kDeriveRows - 1) / kDeriveRows * nchunk;
  const int64_t blocks = (tasks + kDeriveWaves - 1) / kDeriveWaves;
  if (blocks > 0x7fffffff) return hipErrorInvalidConfiguration;
  if (wt == RB_BF16)
    hipLaunchKernelGGL((qat_derive_kernel<KP, true>), dim3((uint32_t)blocks), dim3(64 * kDeriveWaves), 0, st, W, N,
                       K, ldw, g, h, planes, ldp, static_cast<uint16_t*>(What), ldwh, nchunk);
  else
    hipLaunchKernelGGL((qat_derive_kernel<KP, false>), dim3((uint32_t)blocks), dim3(64 * kDeriveWaves), 0, st, W, N,
                       K, ldw, g, h, planes, ldp, static_cast<uint16_t*>(What), ldwh, nchunk);
  return hipGetLastError();
}

template <int KP>
hipError_t scale_grad_kp(const float* dW, int64_t N, int64_t K, int64_t lddw, const uint32_t* planes, int64_t ldp,
                         const float* g, const float* h, float* dg, float* dh, void* ws, hipStream_t st) {
  const int64_t ns = sg_strips(K), nt = sg_tiles(N);
  if (nt > 65535 || ns > 0x7fffffff) return hipErrorInvalidConfiguration;
  float* rowpart = static_cast<float*>(ws);
  float* colpart = reinterpret_cast<float*>(static_cast<char*>(ws) + align256(sizeof(float) * (size_t)(ns * KP * N)));
  hipLaunchKernelGGL(qat_scale_grad_kernel<KP>, dim3((uint32_t)ns, (uint32_t)nt), dim3(64 * kSgWaves), 0, st, dW, N,
                     K, lddw, planes, ldp, g, h, rowpart, colpart,
                     (reinterpret_cast<uintptr_t>(dW) & 15u) == 0 && (lddw & 3) == 0);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int64_t total = (int64_t)KP * (N + K);
  hipLaunchKernelGGL(qat_scale_grad_finish, dim3((uint32_t)((total + 255) / 256)), dim3(256), 0, st, rowpart, colpart,
                     N, K, KP, ns, nt, dg, dh);
  return hipGetLastError();
}

}  // namespace

size_t qat_backward_workspace_bytes(int k, int64_t N, int64_t K) {
  return align256(sizeof(float) * (size_t)(sg_strips(K) * k * N)) + align256(sizeof(float) * (size_t)(sg_tiles(N) * k * K));
}

hipError_t launch_qat_derive(const float* W, int64_t N, int64_t K, int64_t ldw, int k, const float* g,
                             const float* h, uint32_t* planes, int64_t ldp, void* What, rb_dtype what_dtype,
                             int64_t ldwh, hipStream_t stream) {
  switch (k) {
    case 1: return derive_kp<1>(W, N, K, ldw, g, h, planes, ldp, What, what_dtype, ldwh, stream);
    case 2: return derive_kp<2>(W, N, K, ldw, g, h, planes, ldp, What, what_dtype, ldwh, stream);
    case 3: return derive_kp<3>(W, N, K, ldw, g, h, planes, ldp, What, what_dtype, ldwh, stream);
    default: return derive_kp<4>(W, N, K, ldw, g, h, planes, ldp, What, what_dtype, ldwh, stream);
  }
}

namespace {

// The layer's three products as column-major GEMMs (row-major M x N = column-major N x M):
//   Y [M][ldy] = X What^T    Y^T (N x M) = What^T^T X^T: A = What stored K x N, transposed;
//                            B = X stored K x M
//   dW [N][lddw] = dY^T X    dW^T (K x N) = X^T dY: A = X stored K x M; B = dY stored N x M,
//                            transposed
//   dX [M][lddx] = dY What   dX^T (K x M) = What^T dY^T: A = What stored K x N; B = dY stored
//                            N x M
GemmShape shape_y(rb_dtype at, int64_t M, int64_t ldx, int64_t ldwh, int64_t N, int64_t K, rb_dtype yt, int64_t ldy) {
  return {rocblas_operation_transpose, rocblas_operation_none, N, M, K, ldwh, ldx, ldy, at, yt};
}
GemmShape shape_dw(rb_dtype at, int64_t M, int64_t ldx, int64_t lddy, int64_t N, int64_t K, int64_t lddw) {
  return {rocblas_operation_none, rocblas_operation_transpose, K, N, M, ldx, lddy, lddw, at, RB_F32};
}
GemmShape shape_dx(rb_dtype at, int64_t M, int64_t ldwh, int64_t lddy, int64_t N, int64_t K, rb_dtype xt,
                   int64_t lddx) {
  return {rocblas_operation_none, rocblas_operation_none, K, M, N, ldwh, lddy, lddx, at, xt};
}

}  // namespace

hipError_t launch_qat_forward_gemm(const void* X, rb_dtype a_dtype, int64_t M, int64_t ldx, const void* What,
                                   int64_t ldwh, int64_t N, int64_t K, void* Y, rb_dtype y_dtype, int64_t ldy,
                                   hipStream_t stream, int engine) {
  const bool mine = qat_gemm_tn_supported(X, ldx, What, ldwh, M, N, K);
  if (engine == 1) {
    if (!mine) return hipErrorNotSupported;
    return launch_qat_gemm_tn(X, a_dtype, ldx, What, ldwh, M, N, K, Y, y_dtype, ldy, stream);
  }
  const GemmShape sh = shape_y(a_dtype, M, ldx, ldwh, N, K, y_dtype, ldy);
  if (engine == 0 && mine) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    bool mine_faster = false;
    {
      std::lock_guard<std::mutex> lock(g_blas_mu);
      const auto it = g_blas_slower.find(gemm_key(dev, sh));
      mine_faster = it != g_blas_slower.end() && it->second;
    }
    if (mine_faster) return launch_qat_gemm_tn(X, a_dtype, ldx, What, ldwh, M, N, K, Y, y_dtype, ldy, stream);
  }
  std::lock_guard<std::mutex> lock(g_blas_mu);
  rocblas_handle hd;
  int dev;
  hipError_t e = blas_handle_locked(stream, &hd, &dev);
  if (e != hipSuccess) return e;
  const auto it = g_tuned.find(gemm_key(dev, sh));
  const int32_t sol = it == g_tuned.end() ? 0 : it->second;
  const rocblas_status st = gemm_run(hd, sh, What, X, Y, sol);
  return blas_ok(st) ? hipSuccess : blas_fail("gemm_ex", st);
}

// the two backward products, then the scale gradients from dW and the planes
hipError_t launch_qat_backward(const void* dY, rb_dtype a_dtype, int64_t M, int64_t lddy, const void* X, int64_t ldx,
                               const void* What, int64_t ldwh, const uint32_t* planes, int64_t ldp, const float* g,
                               const float* h, int k, int64_t N, int64_t K, float* dW, int64_t lddw, void* dX,
                               rb_dtype dx_dtype, int64_t lddx, float* dg, float* dh, void* ws, hipStream_t stream) {
  {
    std::lock_guard<std::mutex> lock(g_blas_mu);
    rocblas_handle hd;
    int dev;
    hipError_t e = blas_handle_locked(stream, &hd, &dev);
    if (e != hipSuccess) return e;
    e = gemm_locked(hd, dev, shape_dw(a_dtype, M, ldx, lddy, N, K, lddw), X, dY, dW);
    if (e != hipSuccess) return e;
    e = gemm_locked(hd, dev, shape_dx(a_dtype, M, ldwh, lddy, N, K, dx_dtype, lddx), What, dY, dX);
    if (e != hipSuccess) return e;
  }
  switch (k) {
    case 1: return scale_grad_kp<1>(dW, N, K, lddw, planes, ldp, g, h, dg, dh, ws, stream);
    case 2: return scale_grad_kp<2>(dW, N, K, lddw, planes, ldp, g, h, dg, dh, ws, stream);
    case 3: return scale_grad_kp<3>(dW, N, K, lddw, planes, ldp, g, h, dg, dh, ws, stream);
    default: return scale_grad_kp<4>(dW, N, K, lddw, planes, ldp, g, h, dg, dh, ws, stream);
  }
}

hipError_t launch_qat_autotune(const void* X, const void* dY, rb_dtype a_dtype, int64_t M, int64_t ldx, int64_t lddy,
                               const void* What, int64_t ldwh, int64_t N, int64_t K, void* Y, rb_dtype y_dtype,
                               int64_t ldy, float* dW, int64_t lddw, void* dX, rb_dtype dx_dtype, int64_t lddx,
                               hipStream_t stream) {
  std::lock_guard<std::mutex> lock(g_blas_mu);
  rocblas_handle hd;
  int dev;
  hipError_t e = blas_handle_locked(stream, &hd, &dev);
  if (e != hipSuccess) return e;
  std::function<hipError_t()> mine = nullptr;
  if (qat_gemm_tn_supported(X, ldx, What, ldwh, M, N, K))
    mine = [&]() { return launch_qat_gemm_tn(X, a_dtype, ldx, What, ldwh, M, N, K, Y, y_dtype, ldy, stream); };
  e = autotune_locked(hd, dev, shape_y(a_dtype, M, ldx, ldwh, N, K, y_dtype, ldy), What, X, Y, stream, mine);
  if (e != hipSuccess) return e;
  e = autotune_locked(hd, dev, shape_dw(a_dtype, M, ldx, lddy, N, K, lddw), X, dY, dW, stream);
  if (e != hipSuccess) return e;
  return autotune_locked(hd, dev, shape_dx(a_dtype, M, ldwh, lddy, N, K, dx_dtype, lddx), What, dY, dX, stream);
}

}  // namespace rb
