// rb_pack.hip -- derivation of k residual sign bit-planes with dual scales (gfx950).
//
// [RaBiT summary page, "Method step details", Algorithm 2, forward pass]
//   R_0 = W; for each plane i: B_i = sign(R_i), g_i = L2-optimal scale for B_i and h_i,
//   R_{i+1} = R_i - g_i (.) B_i (.) h_i.
// [RaBiT "Technical novelty"] 32 columns per uint32 word.
//
// Row-scale mode (group == 0): the scale of plane i needs the whole row of R_i. Rows of up
// to 16384 columns are held in registers by one block of 4 waves (pack_rows_block_kernel):
// W is read once and each plane is a pass over registers. Longer rows use one wave per row
// (pack_rows_kernel), which traverses the row once per plane. Neither stores the residual:
// each pass re-derives R_i from W with the earlier planes' stored scales and their signs.
// Sums of |R_i| h_i and h_i^2 are fp64 in a fixed order; the quotient is rounded once to
// the scale type. __ballot of (R >= 0) turns each 64-column step into two uint32 words.
//
// Group mode (group = 2..64, h = 1): a scale covers `group` consecutive columns, all
// inside one 64-column step, so all k planes of a step are derived in registers before
// moving on (one pass over W, one wave per row).
#include <type_traits>

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

// Row-scale mode with the row held in registers: one block of 4 waves per row, W read once.
// Wave w owns the 64-column steps s = 4 j + w (j < J), lane l column 64 s + l, so each load
// of a wave is a coalesced 256-byte run and the 4 waves' runs are adjacent. Each plane is a
// pass over registers; R_i is re-derived in fp64 from w and the earlier planes' stored
// scales exactly as in pack_rows_kernel, so the signs are the same. Sums of |R_i| h_i (and
// h_i^2) are fp64: a butterfly per wave, then the 4 wave totals added in a fixed order
// through LDS, so every wave holds the same quotient (deterministic).
constexpr int kRowBlockWaves = 4;

template <typename TW> struct RowLoad;
template <> struct RowLoad<float> {
  __device__ static __forceinline__ float get(__amdgpu_buffer_rsrc_t r, uint32_t off) {
    return __uint_as_float(buf_u32(r, off, 0u));
  }
};
template <> struct RowLoad<__half> {
  __device__ static __forceinline__ float get(__amdgpu_buffer_rsrc_t r, uint32_t off) {
    return __half2float(__ushort_as_half((uint16_t)buf_u16(r, off, 0u)));
  }
};
template <> struct RowLoad<__hip_bfloat16> {
  __device__ static __forceinline__ float get(__amdgpu_buffer_rsrc_t r, uint32_t off) {
    return __uint_as_float(buf_u16(r, off, 0u) << 16);
  }
};

template <typename TW, typename TS, int J, bool HAS_H>
__global__ __launch_bounds__(64 * kRowBlockWaves) void pack_rows_block_kernel(
    const TW* __restrict__ W, int64_t N, int64_t K, int64_t ldw, int k, const TS* __restrict__ h,
    uint32_t* __restrict__ planes, int64_t ldp, TS* __restrict__ g, int32_t* __restrict__ d_status) {
  __shared__ double part[2][kRowBlockWaves][2];  // [pass parity][wave][num, den]
  const int lane = threadIdx.x & (RB_WAVE - 1);
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int64_t n = blockIdx.x;
  const TW* __restrict__ Wr = W + n * ldw;
  const uint32_t Kc = (uint32_t)K;
  const uint32_t Kw = (Kc + 31u) >> 5;
  // steps wholly inside the row, and the columns of the one partial step (if any): a step is
  // skipped or not by a wave-uniform test, and one lane mask serves the partial step
  const int full = (int)(Kc >> 6);
  const bool in_tail = (uint32_t)lane < (Kc & 63u);
  auto step_of = [&](int j) { return kRowBlockWaves * j + wave; };

  // the row through a buffer resource: every load is issued unconditionally (a column past
  // K reads 0), so all J loads of a wave are in flight together
  const __amdgpu_buffer_rsrc_t rw = buffer_rsrc(Wr, Kc * (uint32_t)sizeof(TW));
  float wv[J];
#pragma unroll
  for (int j = 0; j < J; ++j) {
    const uint32_t off = (64u * (uint32_t)step_of(j) + (uint32_t)lane) * (uint32_t)sizeof(TW);
    wv[j] = RowLoad<TW>::get(rw, off);
  }
  bool bad = false;
#pragma unroll
  for (int j = 0; j < J; ++j) bad |= !isfinite(wv[j]);  // columns past K hold 0

  double gprev[4] = {0.0, 0.0, 0.0, 0.0};  // stored scales of earlier planes
#pragma unroll
  for (int i = 0; i < 4; ++i) {  // k <= 4: unrolled, so every plane index is a constant
    if (i >= k) break;
    double num = 0.0, den = 0.0;
    uint32_t* __restrict__ prow = planes + ((int64_t)i * N + n) * ldp;
    uint32_t wlo = 0u, whi = 0u;  // lane j: the two words of step 4 j + wave
    // the step limit, opaque to the compiler per pass: the per-step tests are then redone in
    // each pass instead of being kept live across passes as scalar masks
    int full_i = full;
    asm volatile("" : "+s"(full_i));
#pragma unroll
    for (int j = 0; j < J; ++j) {
      const int st = step_of(j);
      if (st > full_i) continue;  // wave-uniform: a step wholly past K (the loop stays unrolled)
      const bool valid = st < full_i || in_tail;
      const uint32_t col = 64u * (uint32_t)st + (uint32_t)lane;
      double R = (double)wv[j];
      bool b = nonneg_bits(wv[j]);
#pragma unroll
      for (int p = 0; p < i; ++p) {
        const double gh = HAS_H ? gprev[p] * (double)to_f32(h[(int64_t)p * K + (valid ? col : 0u)]) : gprev[p];
        R = b ? R - gh : R + gh;
        b = R >= 0.0;  // -0.0 >= 0 holds: sign(0) = +1
      }
      if (HAS_H) {
        const double hi = (double)to_f32(h[(int64_t)i * K + (valid ? col : 0u)]);
        if (valid) {
          num += fabs(R) * hi;
          den += hi * hi;
        }
      } else if (valid) {
        num += fabs(R);
      }
      const uint64_t m = __ballot(valid && b);
      wlo = lane == j ? (uint32_t)m : wlo;
      whi = lane == j ? (uint32_t)(m >> 32) : whi;
      // one step at a time: each ballot is consumed at once instead of piling up in scalar
      // registers (other resident waves hide the fp64 latency)
      __builtin_amdgcn_sched_barrier(0);
    }
    // lane j < J stores words 2 s and 2 s + 1 of step s = 4 j + wave
    {
      const uint32_t w0 = 2u * (uint32_t)(kRowBlockWaves * lane + wave);
      if (lane < J && w0 < Kw) prow[w0] = wlo;
      if (lane < J && w0 + 1u < Kw) prow[w0 + 1u] = whi;
    }
    num = wave_sum(num);
    if (HAS_H) den = wave_sum(den);
    if (lane == 0) {
      part[i & 1][wave][0] = num;
      part[i & 1][wave][1] = den;
    }
    __syncthreads();
    double tn = 0.0, td = 0.0;
#pragma unroll
    for (int v = 0; v < kRowBlockWaves; ++v) {
      tn += part[i & 1][v][0];
      td += part[i & 1][v][1];
    }
    if (!HAS_H) td = (double)K;
    const double q = td > 0.0 ? tn / td : 0.0;
    double stored;
    if (wave == 0 && lane == 0) {
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

// steps of 64 columns per wave (J) for a row of K columns, or 0 when the row does not fit
inline int row_block_steps(int64_t K) {
  const int64_t steps = (K + 63) / 64;
  const int64_t J = (steps + kRowBlockWaves - 1) / kRowBlockWaves;
  if (J <= 8) return 8;
  if (J <= 16) return 16;
  if (J <= 32) return 32;
  if (J <= 48) return 48;
  if (J <= 64) return 64;
  return 0;
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
  const uint32_t Kc = (uint32_t)K;
  const uint32_t Kw = (Kc + 31u) >> 5;
  const int64_t G = (K + group - 1) / group;
  // the row through a buffer resource: the loads of a chunk are issued unconditionally (a
  // column past K reads 0); steps wholly past K are skipped by a wave-uniform test
  const __amdgpu_buffer_rsrc_t rw = buffer_rsrc(W + n * ldw, Kc * (uint32_t)sizeof(TW));
  const int full = (int)(Kc >> 6);
  const bool in_tail = (uint32_t)lane < (Kc & 63u);
  bool bad = false;
  for (int c0 = 0; 64 * c0 < (int)Kc; c0 += kPackSteps) {  // c0: first step of the chunk
    float wv[kPackSteps];
#pragma unroll
    for (int j = 0; j < kPackSteps; ++j)
      wv[j] = RowLoad<TW>::get(rw, (64u * (uint32_t)(c0 + j) + (uint32_t)lane) * (uint32_t)sizeof(TW));
    uint32_t word[4] = {0u, 0u, 0u, 0u};
#pragma unroll
    for (int j = 0; j < kPackSteps; ++j) {
      const int st = c0 + j;
      if (st > full) continue;  // wave-uniform
      const bool valid = st < full || in_tail;
      const uint32_t col = 64u * (uint32_t)st + (uint32_t)lane;
      const float w = wv[j];
      bad |= !isfinite(w);  // columns past K hold 0
      // columns of this lane's group that exist (the last group of a row may be short)
      const uint32_t gq = (valid ? col : Kc - 1u) / (uint32_t)group;
      const uint32_t gstart = gq * (uint32_t)group;
      const uint32_t gend = gstart + (uint32_t)group < Kc ? gstart + (uint32_t)group : Kc;
      const double cnt = (double)(gend - gstart);
      const bool leader = valid && (col == gstart);
      double R = (double)w;
      bool b = nonneg_bits(w);
#pragma unroll
      for (int i = 0; i < 4; ++i) {  // k <= 4
        if (i < k) {
          const double sum = group_sum(valid ? fabs(R) : 0.0, group);
          const double q = sum / cnt;
          double stored;
          if (leader) {
            stored = ScaleRound<TS>::store(g + ((int64_t)i * N + n) * G + gq, q);
          } else {
            TS tmp;
            stored = ScaleRound<TS>::store(&tmp, q);
          }
          const uint64_t m = __ballot(valid && b);
          word[i] = lane == ((2 * j) & 63) ? (uint32_t)m : word[i];
          word[i] = lane == ((2 * j + 1) & 63) ? (uint32_t)(m >> 32) : word[i];
          R = b ? R - stored : R + stored;
          b = R >= 0.0;
        }
      }
    }
    // lanes 0 .. 2 kPackSteps - 1 hold the chunk's words
    const uint32_t w0 = 2u * (uint32_t)c0;
    if (lane < 2 * kPackSteps && w0 + (uint32_t)lane < Kw) {
#pragma unroll
      for (int i = 0; i < 4; ++i)
        if (i < k) planes[((int64_t)i * N + n) * ldp + w0 + lane] = word[i];
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
  const int J = group == 0 ? row_block_steps(K) : 0;
  if (J != 0) {
    const dim3 rgrid((unsigned)N), rblock(64 * kRowBlockWaves);
    const TW* Wt = static_cast<const TW*>(W);
    const TS* ht = static_cast<const TS*>(h);
    TS* gt = static_cast<TS*>(g);
    auto go = [&](auto has_h) {
      constexpr bool H = decltype(has_h)::value;
      switch (J) {
        case 8: pack_rows_block_kernel<TW, TS, 8, H><<<rgrid, rblock, 0, s>>>(Wt, N, K, ldw, k, ht, planes, ldp, gt, d_status); break;
        case 16: pack_rows_block_kernel<TW, TS, 16, H><<<rgrid, rblock, 0, s>>>(Wt, N, K, ldw, k, ht, planes, ldp, gt, d_status); break;
        case 32: pack_rows_block_kernel<TW, TS, 32, H><<<rgrid, rblock, 0, s>>>(Wt, N, K, ldw, k, ht, planes, ldp, gt, d_status); break;
        case 48: pack_rows_block_kernel<TW, TS, 48, H><<<rgrid, rblock, 0, s>>>(Wt, N, K, ldw, k, ht, planes, ldp, gt, d_status); break;
        default: pack_rows_block_kernel<TW, TS, 64, H><<<rgrid, rblock, 0, s>>>(Wt, N, K, ldw, k, ht, planes, ldp, gt, d_status); break;
      }
    };
    if (ht) go(std::true_type{});
    else go(std::false_type{});
  } else if (group == 0) {
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
