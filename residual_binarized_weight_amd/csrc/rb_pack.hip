// rb_pack.hip -- derivation of k residual sign bit-planes with dual scales (gfx950).
//
// [RaBiT summary page, "Method step details", Algorithm 2, forward pass]
//   R_0 = W; for each plane i: B_i = sign(R_i), g_i = L2-optimal scale for B_i and h_i,
//   R_{i+1} = R_i - g_i (.) B_i (.) h_i.
// [RaBiT "Technical novelty"] 32 columns per uint32 word.
//
// One wave64 per weight row. Lane l reads column c0 + l of each 64-column step, so
// every load of W is a fully coalesced 64-element run. __ballot of (R >= 0) turns one
// step into two uint32 words; after 16 steps lanes 0..31 hold the words of a 1024-column
// chunk and the wave writes them with one coalesced store.
//
// Row-scale mode (group == 0): the scale of plane i needs the whole row of R_i, so the
// row is traversed once per plane. The residual is never stored: each pass recomputes
// R_i from W with the earlier planes' stored scales (kept in registers) and re-derives
// their signs on the fly. Sums of |R_i| h_i and h_i^2 are fp64 per lane, then a fixed
// butterfly across the wave; the quotient is rounded once to the scale type.
//
// Group mode (group = 2..64, h = 1): a scale covers `group` consecutive columns, all
// inside one 64-column step, so all k planes of a step are derived in registers before
// moving on (one pass over W).
#include "rb_device.hpp"
#include "rb_internal.h"

namespace rb {
namespace {

constexpr int kRowsPerBlock = 4;  // 4 waves of 64
constexpr int kPackSteps = 16;    // 64-column steps per chunk of the row kernel

template <typename TW, typename TS>
__global__ __launch_bounds__(256) void pack_rows_kernel(const TW* __restrict__ W, int64_t N,
                                                        int64_t K, int64_t ldw, int k,
                                                        const TS* __restrict__ h,
                                                        uint32_t* __restrict__ planes, int64_t ldp,
                                                        TS* __restrict__ g,
                                                        int32_t* __restrict__ d_status) {
  const int lane = threadIdx.x & (RB_WAVE - 1);
  const int64_t n = (int64_t)blockIdx.x * kRowsPerBlock + (threadIdx.x >> 6);
  if (n >= N) return;  // uniform per wave
  const TW* __restrict__ Wr = W + n * ldw;
  const int64_t Kw = (K + 31) >> 5;
  double gprev[4] = {0.0, 0.0, 0.0, 0.0};  // stored scales of earlier planes
  bool bad = false;

  for (int i = 0; i < k; ++i) {
    double num = 0.0, den = 0.0;
    uint32_t* __restrict__ prow = planes + ((int64_t)i * N + n) * ldp;
    // 1024-column chunks: the 16 loads of a chunk are issued before any is used (enough
    // requests in flight to stream W); lanes 0..31 collect the chunk's 32 words
    for (int64_t c0 = 0; c0 < K; c0 += 64 * kPackSteps) {
      float wv[kPackSteps];
#pragma unroll
      for (int j = 0; j < kPackSteps; ++j) {
        const int64_t col = c0 + 64 * j + lane;
        wv[j] = col < K ? to_f32(Wr[col]) : 0.0f;
      }
      uint32_t word = 0u;
#pragma unroll
      for (int j = 0; j < kPackSteps; ++j) {
        const int64_t col = c0 + 64 * j + lane;
        const bool valid = col < K;
        const float w = wv[j];
        if (i == 0) bad |= valid && !isfinite(w);
        // R_i at this column, re-derived through the earlier planes
        double R = (double)w;
        bool b = nonneg_bits(w);
        for (int p = 0; p < i; ++p) {
          const double hp = h ? (double)to_f32(h[(int64_t)p * K + (valid ? col : 0)]) : 1.0;
          const double gh = gprev[p] * hp;  // exact: <= 48 significant bits
          R = b ? R - gh : R + gh;
          b = R >= 0.0;  // -0.0 >= 0 holds: sign(0) = +1
        }
        const double hi = h ? (double)to_f32(h[(int64_t)i * K + (valid ? col : 0)]) : 1.0;
        if (valid) {
          num += fabs(R) * hi;
          den += hi * hi;
        }
        const uint64_t m = __ballot(valid && b);
        if (lane == ((2 * j) & 63)) word = (uint32_t)m;
        if (lane == ((2 * j + 1) & 63)) word = (uint32_t)(m >> 32);
      }
      const int64_t w0 = c0 >> 5;
      if (lane < 2 * kPackSteps && w0 + lane < Kw) prow[w0 + lane] = word;
    }
    num = wave_sum(num);
    den = h ? wave_sum(den) : (double)K;
    const double q = den > 0.0 ? num / den : 0.0;
    double stored;
    if (lane == 0) {
      stored = ScaleRound<TS>::store(g + (int64_t)i * N + n, q);
    } else {
      TS tmp;
      stored = ScaleRound<TS>::store(&tmp, q);
    }
    gprev[i] = stored;
  }
  if (d_status) {
    const uint64_t anybad = __ballot(bad);
    if (anybad && lane == 0) atomicOr(d_status, 1);
  }
}

template <typename TW, typename TS>
__global__ __launch_bounds__(256) void pack_groups_kernel(const TW* __restrict__ W, int64_t N,
                                                          int64_t K, int64_t ldw, int k, int group,
                                                          uint32_t* __restrict__ planes,
                                                          int64_t ldp, TS* __restrict__ g,
                                                          int32_t* __restrict__ d_status) {
  const int lane = threadIdx.x & (RB_WAVE - 1);
  const int64_t n = (int64_t)blockIdx.x * kRowsPerBlock + (threadIdx.x >> 6);
  if (n >= N) return;
  const TW* __restrict__ Wr = W + n * ldw;
  const int64_t Kw = (K + 31) >> 5;
  const int64_t G = (K + group - 1) / group;
  bool bad = false;
  for (int64_t c0 = 0; c0 < K; c0 += 64 * 32) {
    uint32_t word[4] = {0u, 0u, 0u, 0u};
    for (int j = 0; j < 32; ++j) {
      const int64_t col = c0 + 64 * j + lane;
      if (c0 + 64 * j >= K) break;  // uniform
      const bool valid = col < K;
      const float w = valid ? to_f32(Wr[col]) : 0.0f;
      bad |= valid && !isfinite(w);
      // columns of this lane's group that exist (the last group of a row may be short)
      const int64_t gq = (valid ? col : K - 1) / group;
      const int64_t gstart = gq * group;
      const int64_t gend = gstart + group < K ? gstart + group : K;
      const double cnt = (double)(gend - gstart);
      double R = (double)w;
      bool b = nonneg_bits(w);
      for (int i = 0; i < k; ++i) {
        const double sum = group_sum(valid ? fabs(R) : 0.0, group);
        const double q = sum / cnt;
        const bool leader = valid && (col == gstart);
        double stored;
        if (leader) {
          stored = ScaleRound<TS>::store(g + ((int64_t)i * N + n) * G + gq, q);
        } else {
          TS tmp;
          stored = ScaleRound<TS>::store(&tmp, q);
        }
        const uint64_t m = __ballot(valid && b);
        if (lane == ((2 * j) & 63)) word[i] = (uint32_t)m;
        if (lane == ((2 * j + 1) & 63)) word[i] = (uint32_t)(m >> 32);
        R = b ? R - stored : R + stored;
        b = R >= 0.0;
      }
    }
    const int64_t w0 = c0 >> 5;
    if (w0 + lane < Kw) {
      for (int i = 0; i < k; ++i) planes[((int64_t)i * N + n) * ldp + w0 + lane] = word[i];
    }
  }
  if (d_status) {
    const uint64_t anybad = __ballot(bad);
    if (anybad && lane == 0) atomicOr(d_status, 1);
  }
}

template <typename TW, typename TS>
hipError_t launch_typed(const void* W, int64_t N, int64_t K, int64_t ldw, int k, int group,
                        const void* h, uint32_t* planes, int64_t ldp, void* g, int32_t* d_status,
                        hipStream_t s) {
  const dim3 grid((unsigned)((N + kRowsPerBlock - 1) / kRowsPerBlock));
  const dim3 block(64 * kRowsPerBlock);
  if (group == 0) {
    pack_rows_kernel<TW, TS><<<grid, block, 0, s>>>(
        static_cast<const TW*>(W), N, K, ldw, k, static_cast<const TS*>(h), planes, ldp,
        static_cast<TS*>(g), d_status);
  } else {
    pack_groups_kernel<TW, TS><<<grid, block, 0, s>>>(static_cast<const TW*>(W), N, K, ldw, k,
                                                      group, planes, ldp, static_cast<TS*>(g),
                                                      d_status);
  }
  return hipGetLastError();
}

template <typename TW>
hipError_t launch_w(rb_dtype scale_dtype, const void* W, int64_t N, int64_t K, int64_t ldw, int k,
                    int group, const void* h, uint32_t* planes, int64_t ldp, void* g,
                    int32_t* d_status, hipStream_t s) {
  if (scale_dtype == RB_F16)
    return launch_typed<TW, __half>(W, N, K, ldw, k, group, h, planes, ldp, g, d_status, s);
  return launch_typed<TW, float>(W, N, K, ldw, k, group, h, planes, ldp, g, d_status, s);
}

}  // namespace

hipError_t launch_pack(const void* W, rb_dtype w_dtype, int64_t N, int64_t K, int64_t ldw, int k,
                       int group, const void* h, rb_dtype scale_dtype, uint32_t* planes, int64_t ldp,
                       void* g, int32_t* d_status, hipStream_t s) {
  switch (w_dtype) {
    case RB_F32:
      return launch_w<float>(scale_dtype, W, N, K, ldw, k, group, h, planes, ldp, g, d_status, s);
    case RB_F16:
      return launch_w<__half>(scale_dtype, W, N, K, ldw, k, group, h, planes, ldp, g, d_status, s);
    default:
      return launch_w<__hip_bfloat16>(scale_dtype, W, N, K, ldw, k, group, h, planes, ldp, g,
                                      d_status, s);
  }
}

}  // namespace rb
