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
    TY* __restrict__ y, const TS* __restrict__ mu, int zero_one) {
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
        // a +-1 plane contributes 2 T - S, a {0, 1} plane T; a row offset mu adds mu S (h = 1)
        yacc[r][m] += gi * (zero_one ? T : 2.0f * T - S);
        if (i == 0 && mu && row < N) yacc[r][m] += to_f32(mu[row]) * S;
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

// ---------------------------------------------------------------------------
// LUT kernel (M = 1, h = 1): byte subset-sum tables in LDS.
//
// For a 1024-column slice of x, the block builds 128 tables, one per 8-column group:
// T_grp[b] = sum of x over the set bits of b (fp32, 256 entries). One lookup then stands
// for 8 weight bits of a row, so a plane row costs 1 LDS read and 2 VALU ops per byte
// instead of a masked add per bit; y uses the masked-add identity per lane,
// P = sum_i g_i (2 T_i - S), S being the lane's 32-column sum of x.
//
// LDS layout (128 KB): group grp = 4 s + q of the slice (s = word 0..31, q = byte 0..3)
// lives in region q >> 1 at slot (q & 1) * 32 + s; entry b of a table is at byte address
// region << 16 | b << 8 | slot << 2. The 32 lanes of a half wave look up the 32 words of
// one row: lane s always reads slot s (mod 32), so the 32 reads hit 32 different banks
// whatever the bytes are. The address is one v_perm of the weight word with a per-lane
// constant holding the slot bytes and the region byte.
//
// Work split: block = (slice, row block); 8 waves, each wave takes `pairs` row pairs
// (half 0 / half 1 of the wave take the two rows of a pair). The plane words of all the
// wave's rows are loaded before the tables are built, so HBM latency overlaps the build.
// Each row's lane partials are summed by five DPP steps inside each 32-lane half.
// Split-K: the slices of a row meet in one 64-bit fixed-point accumulator per row (see
// below), so the result is deterministic and no second launch is needed.
// ---------------------------------------------------------------------------
constexpr int kLutSliceCols = 1024;
constexpr int kLutSliceWords = 32;
constexpr int kLutThreads = 1024;
constexpr int kLutWaves = 16;
constexpr int kLutTableBytes = 128 * 1024;

template <typename T> struct BufElem;
template <> struct BufElem<__half> {
  using raw = uint32_t;
  __device__ static __forceinline__ uint32_t load(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff) {
    return buf_u16(r, voff, soff);
  }
  __device__ static __forceinline__ float f32(uint32_t v) { return __half2float(__ushort_as_half((uint16_t)v)); }
};
template <> struct BufElem<float> {
  using raw = uint32_t;
  __device__ static __forceinline__ uint32_t load(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff) {
    return buf_u32(r, voff, soff);
  }
  __device__ static __forceinline__ float f32(uint32_t v) { return __uint_as_float(v); }
};

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
constexpr int kLutXChunks = 2;  // 16-byte chunks of x per thread in the |x| sum (more: a loop)

template <typename TX> __device__ __forceinline__ float chunk_abs_sum(u32x4 c);
template <> __device__ __forceinline__ float chunk_abs_sum<__half>(u32x4 c) {
  float s = 0.0f;
#pragma unroll
  for (int d = 0; d < 4; ++d) {
    const uint32_t w = c[d];
    s += fabsf(__half2float(__ushort_as_half((uint16_t)(w & 0xffffu)))) +
         fabsf(__half2float(__ushort_as_half((uint16_t)(w >> 16))));
  }
  return s;
}
template <> __device__ __forceinline__ float chunk_abs_sum<float>(u32x4 c) {
  return (fabsf(__uint_as_float(c[0])) + fabsf(__uint_as_float(c[1]))) +
         (fabsf(__uint_as_float(c[2])) + fabsf(__uint_as_float(c[3])));
}

// a scale kept in a full 32-bit register (loading fp16 values into separate registers keeps
// the compiler from packing pairs, which would force a wait right after each load)
template <typename TS> struct RawScale;
template <> struct RawScale<__half> {
  using type = uint32_t;
  __device__ static __forceinline__ uint32_t load(const __half* p) {
    return (uint32_t)*reinterpret_cast<const uint16_t*>(p);
  }
  __device__ static __forceinline__ float f32(uint32_t v) { return __half2float(__ushort_as_half((uint16_t)v)); }
};
template <> struct RawScale<float> {
  using type = float;
  __device__ static __forceinline__ float load(const float* p) { return *p; }
  __device__ static __forceinline__ float f32(float v) { return v; }
};

// Split-K handoff through one 64-bit atomic per row. Each block adds its row partial p as
// a fixed-point integer q = rint(p * 2^(30 - e)), where 2^e is the smallest power of two above
// U = sum_i |g_i[row]| * sum_c |x_c|, a bound on |p| for every slice (so |q| < 2^31, and the
// scaling by a power of two is exact), plus a bias 2^48 and a count unit 2^56:
//   word = n * 2^56 + n * 2^48 + sum q      (n contributions so far; no field overflows for n <= 127)
// Integer addition is exact and order-free, so the result does not depend on which block
// arrives first; the quantisation error is at most n * 2^-31 * U. The block whose fetch_add
// brings the count to n_slices decodes the sum, writes y and stores 0 back for the next call.
// Every block computes U from the same data with the same instruction sequence, hence
// bit-identically.
constexpr uint64_t kAccCount = 1ull << 56;
constexpr uint64_t kAccBias = 1ull << 48;

// One block per compute unit (its tables take 128 KB of LDS), i.e. 4 waves per SIMD: the
// register budget is 128 per lane, and the scheduler need not trade loads in flight for
// occupancy it cannot get.
template <typename TX, typename TS, typename TY, int KP, int PAIRS>
__global__ __launch_bounds__(kLutThreads) __attribute__((amdgpu_waves_per_eu(1, 4))) void gemv_lut_kernel(
    const uint32_t* __restrict__ planes, int64_t ldp, const TS* __restrict__ g, int64_t N,
    int64_t K, const TX* __restrict__ x, TY* __restrict__ y, unsigned long long* __restrict__ acc_rows,
    int n_slices) {
  constexpr int kRowsPerBlock = 2 * kLutWaves * PAIRS;
  // tables at LDS offset 0 (so a lookup address is the v_perm result itself); 64 bytes after them
  extern __shared__ __align__(16) uint8_t lds[];
  float* red = reinterpret_cast<float*>(lds + kLutTableBytes);
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int s = lane & 31;
  const int half = lane >> 5;
  const int slice = blockIdx.x % n_slices;
  const int rb = blockIdx.x / n_slices;
  const int64_t row_first = (int64_t)rb * kRowsPerBlock;
  const int64_t row_lim = row_first + kRowsPerBlock < N ? row_first + kRowsPerBlock : N;
  const int64_t row_wave = row_first + (int64_t)wave * 2 * PAIRS;
  const uint32_t ldp_b = (uint32_t)ldp * 4u;

  // Every load goes through a buffer resource: offsets are 32-bit (the host checks that the
  // arrays fit), anything past the end reads as 0. Rows past N and words past ceil(K/32) may
  // read padding, the next plane or zeros: their columns' tables are all zero and their rows'
  // partials are never published, so they contribute nothing.
  const __amdgpu_buffer_rsrc_t rp = buffer_rsrc(planes, (uint32_t)((uint64_t)KP * N * ldp * 4));
  const __amdgpu_buffer_rsrc_t rg = buffer_rsrc(g, (uint32_t)((uint64_t)KP * N * sizeof(TS)));
  const __amdgpu_buffer_rsrc_t rx = buffer_rsrc(x, (uint32_t)((uint64_t)K * sizeof(TX)));

  // 0a. all of x in 16-byte chunks (through a resource that ends at the last full chunk, so a
  // chunk is either whole or 0) plus the < 16-byte tail, for sum |x| (the fixed-point scale)
  constexpr int kElemPerChunk = 16 / (int)sizeof(TX);
  const uint32_t full_chunks = (uint32_t)((K * (int64_t)sizeof(TX)) / 16);
  const __amdgpu_buffer_rsrc_t rxc = buffer_rsrc(x, full_chunks * 16u);
  u32x4 xc[kLutXChunks];
#pragma unroll
  for (int m = 0; m < kLutXChunks; ++m)
    xc[m] = __builtin_amdgcn_raw_buffer_load_b128(rxc, (int)(((uint32_t)tid + (uint32_t)m * kLutThreads) * 16u), 0, 0);
  uint32_t xt[kElemPerChunk];
#pragma unroll
  for (int j = 0; j < kElemPerChunk; ++j) {
    const uint32_t c = full_chunks * kElemPerChunk + j;  // tail element (or past K: reads 0)
    xt[j] = BufElem<TX>::load(rx, c * (uint32_t)sizeof(TX), 0);  // every lane loads, lane 0 adds
  }

  // 0b. the 8 activations of this thread's table group (16 bytes at a 16-byte boundary for fp16;
  // the one chunk that straddles K comes from the tail loads above)
  const int R = wave & 1;
  const int grp = 4 * s + 2 * R + half;
  const uint32_t col0 = (uint32_t)slice * kLutSliceCols + 8u * grp;
  uint32_t xr[8];
  if (sizeof(TX) == 2) {
    const u32x4 c = __builtin_amdgcn_raw_buffer_load_b128(rxc, (int)(col0 * 2u), 0, 0);
    const bool straddle = col0 == full_chunks * 8u;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      xr[2 * j] = straddle ? xt[2 * j] : (c[j] & 0xffffu);
      xr[2 * j + 1] = straddle ? xt[2 * j + 1] : (c[j] >> 16);
    }
  } else {
#pragma unroll
    for (int j = 0; j < 8; ++j) xr[j] = BufElem<TX>::load(rx, (col0 + j) * (uint32_t)sizeof(TX), 0);
  }

  // every wave's x loads enter the memory pipeline before any wave's plane loads: requests
  // return in order, so the table build must not queue behind the weight stream
  __builtin_amdgcn_sched_barrier(0);
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_sched_barrier(0);

  // 1. plane words and row scales of this lane's rows, all in flight before the build and
  // consumed below in issue order. Per lane: one base offset; per (row pair, plane): a
  // uniform offset.
  const uint32_t wv = ((uint32_t)(row_wave + half) * ldp_b) + ((uint32_t)slice * kLutSliceWords + s) * 4u;
  const uint32_t gv = (uint32_t)(row_wave + half) * (uint32_t)sizeof(TS);
  uint32_t wd[PAIRS][KP];
  uint32_t gr[PAIRS][KP];
#pragma unroll
  for (int t = 0; t < PAIRS; ++t) {
#pragma unroll
    for (int i = 0; i < KP; ++i) {
      wd[t][i] = buf_u32(rp, wv, ((uint32_t)i * (uint32_t)N + 2u * t) * ldp_b);
      gr[t][i] = BufElem<TS>::load(rg, gv, ((uint32_t)i * (uint32_t)N + 2u * t) * (uint32_t)sizeof(TS));
    }
  }


  __builtin_amdgcn_sched_barrier(0);

  // 2. tables: wave w builds entries b in [32 (w >> 1), +32) of groups with q = 2 (w & 1) + half
  {
    float xv[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) xv[j] = BufElem<TX>::f32(xr[j]);
    float L[16];
    L[0] = 0.0f;
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int n = 0; n < (1 << j); ++n) L[(1 << j) + n] = L[n] + xv[j];
    const int hb = wave >> 1;
    const uint32_t slot_byte = (uint32_t)((half ? 128 : 0) + 4 * s);
    uint8_t* tab = lds + ((uint32_t)R << 16) + slot_byte;
#pragma unroll
    for (int hh = 0; hh < 2; ++hh) {
      const int hi = 2 * hb + hh;  // high nibble
      float H = 0.0f;
#pragma unroll
      for (int j = 0; j < 4; ++j)
        if ((hi >> j) & 1) H += xv[4 + j];
#pragma unroll
      for (int lo = 0; lo < 16; ++lo) {
        const int b = hi * 16 + lo;
        *reinterpret_cast<float*>(tab + ((uint32_t)b << 8)) = H + L[lo];
      }
    }
  }
  // sum |x| over all of x, the same way in every block; the chunk loads were issued first,
  // so this waits on nothing the table build did not already wait on
  {
    float xa = 0.0f;
#pragma unroll
    for (int m = 0; m < kLutXChunks; ++m) xa += chunk_abs_sum<TX>(xc[m]);
    float tail = 0.0f;  // every lane sums the tail (its loads must not sink below the plane loads)
#pragma unroll
    for (int j = 0; j < kElemPerChunk; ++j) tail += fabsf(BufElem<TX>::f32(xt[j]));
    xa += tid == 0 ? tail : 0.0f;
    if (full_chunks > (uint32_t)(kLutXChunks * kLutThreads)) {  // very long rows: the rest, uniform branch
      for (uint32_t c = (uint32_t)(tid + kLutXChunks * kLutThreads); c < full_chunks; c += kLutThreads)
        xa += chunk_abs_sum<TX>(__builtin_amdgcn_raw_buffer_load_b128(rxc, (int)(c * 16u), 0, 0));
    }
    xa = wave_sum_dpp(xa);
    if (lane == 63) red[wave] = xa;
  }
  __syncthreads();

  // 3. lookups: one v_perm + one LDS read per weight byte
  const uint32_t cst = (uint32_t)(4 * s) | ((uint32_t)(128 + 4 * s) << 8) | (0u << 16) | (1u << 24);
  // selector bytes: [0] slot byte of cst (q & 1), [1] weight byte q, [2] region byte of cst (2 + (q >> 1)), [3] zero
  const uint32_t sel0 = 0x0C020400u, sel1 = 0x0C020501u, sel2 = 0x0C030600u, sel3 = 0x0C030701u;
  const float S = lds_f32(__builtin_amdgcn_perm(0xffffffffu, cst, sel0)) +
                  lds_f32(__builtin_amdgcn_perm(0xffffffffu, cst, sel1)) +
                  lds_f32(__builtin_amdgcn_perm(0xffffffffu, cst, sel2)) +
                  lds_f32(__builtin_amdgcn_perm(0xffffffffu, cst, sel3));
  float P[PAIRS];
#pragma unroll
  for (int t = 0; t < PAIRS; ++t) {
    float acc = 0.0f;
#pragma unroll
    for (int i = 0; i < KP; ++i) {
      const uint32_t w = wd[t][i];
      const float T = lds_f32(__builtin_amdgcn_perm(w, cst, sel0)) +
                      lds_f32(__builtin_amdgcn_perm(w, cst, sel1)) +
                      lds_f32(__builtin_amdgcn_perm(w, cst, sel2)) +
                      lds_f32(__builtin_amdgcn_perm(w, cst, sel3));
      acc += BufElem<TS>::f32(gr[t][i]) * (2.0f * T - S);
    }
    P[t] = acc;
  }

  float X = 0.0f;
#pragma unroll
  for (int w = 0; w < kLutWaves; ++w) X += red[w];

  // 4. per-row sums over the 32 lanes of each half (lanes 31 / 63 hold them), then one
  // fixed-point atomic per row; the contribution that completes the count writes y.
  float V[PAIRS];
#pragma unroll
  for (int t = 0; t < PAIRS; ++t) V[t] = half_wave_sum(P[t]);
  // issue every row's atomic first, then look at the returned words (one round trip in all)
  unsigned long long old[PAIRS], add[PAIRS];
  int ex[PAIRS];
#pragma unroll
  for (int t = 0; t < PAIRS; ++t) {
    const int64_t row = row_wave + 2 * t + half;
    float gsum = 0.0f;
#pragma unroll
    for (int i = 0; i < KP; ++i) gsum += fabsf(BufElem<TS>::f32(gr[t][i]));
    const float U = gsum * X;
    ex[t] = U > 0.0f ? __builtin_amdgcn_frexp_expf(U) : 0;  // U < 2^ex
    const int q = U > 0.0f ? (int)rintf(ldexpf(V[t], 30 - ex[t])) : 0;
    add[t] = kAccCount + kAccBias + (unsigned long long)(long long)q;
    old[t] = 0ull;
    if (s == 31 && row < row_lim)
      old[t] = __hip_atomic_fetch_add(&acc_rows[row], add[t], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
#pragma unroll
  for (int t = 0; t < PAIRS; ++t) {
    const int64_t row = row_wave + 2 * t + half;
    const unsigned long long now = old[t] + add[t];
    if (s == 31 && row < row_lim && (now >> 56) == (unsigned long long)n_slices) {
      const long long total = (long long)(now & (kAccCount - 1)) - (long long)n_slices * (long long)kAccBias;
      store_out<TY>(&y[row], ldexpf((float)total, ex[t] - 30));
      __hip_atomic_store(&acc_rows[row], 0ull, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
  }
}

// The LUT kernel addresses its arrays with 32-bit buffer offsets and counts slices in 7 bits.
bool lut_fits(int k, int64_t N, int64_t K, int64_t ldp, size_t sx, size_t ss) {
  const uint64_t lim = 0xffffffffull;
  const int64_t n_slices = (K + kLutSliceCols - 1) / kLutSliceCols;
  return n_slices <= 127 && (uint64_t)k * N * ldp * 4 < lim && (uint64_t)k * N * ss < lim && (uint64_t)K * sx < lim &&
         (uint64_t)(N + 2 * kLutWaves * 8) * ldp * 4 < lim;
}

struct LutPlan {
  int n_slices, pairs, n_blocks;
};


// Row pairs per wave are a compile-time class (so every load is branch-free); the plan picks
// the smallest class that spreads the (slice, row block) grid over the compute units.
constexpr int kPairClasses[4] = {2, 4, 6, 8};

LutPlan lut_plan(int64_t N, int64_t K, int cus) {
  LutPlan p;
  p.n_slices = (int)((K + kLutSliceCols - 1) / kLutSliceCols);
  int64_t blocks_per_slice = cus / p.n_slices;
  if (blocks_per_slice < 1) blocks_per_slice = 1;
  const int64_t rows = (N + blocks_per_slice - 1) / blocks_per_slice;
  const int64_t need = (rows + 2 * kLutWaves - 1) / (2 * kLutWaves);
  p.pairs = kPairClasses[3];
  for (int c = 0; c < 4; ++c)
    if (kPairClasses[c] >= need) { p.pairs = kPairClasses[c]; break; }
  const int64_t rows_pb = 2LL * kLutWaves * p.pairs;
  p.n_blocks = (int)(((N + rows_pb - 1) / rows_pb) * p.n_slices);
  return p;
}

size_t lut_workspace_bytes(int64_t N, int64_t) { return zero_region_bytes(N); }

template <typename TX, typename TS, typename TY, int KP, int PAIRS>
hipError_t launch_lut_kp(const LutPlan& p, const uint32_t* planes, int64_t ldp, const void* g, int64_t N,
                         int64_t K, const void* x, void* y, unsigned long long* acc, hipStream_t s) {
  constexpr size_t lds = kLutTableBytes + 64;
  static bool attr_set = false;  // per instantiation
  if (!attr_set) {
    const hipError_t e = hipFuncSetAttribute((const void*)gemv_lut_kernel<TX, TS, TY, KP, PAIRS>,
                                             hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return e;
    attr_set = true;
  }
  gemv_lut_kernel<TX, TS, TY, KP, PAIRS><<<p.n_blocks, kLutThreads, lds, s>>>(
      planes, ldp, static_cast<const TS*>(g), N, K, static_cast<const TX*>(x), static_cast<TY*>(y), acc,
      p.n_slices);
  return hipGetLastError();
}

template <typename TX, typename TS, typename TY, int KP>
hipError_t launch_lut_pairs(const LutPlan& p, const uint32_t* planes, int64_t ldp, const void* g, int64_t N,
                            int64_t K, const void* x, void* y, unsigned long long* acc, hipStream_t s) {
  switch (p.pairs) {
    case 2: return launch_lut_kp<TX, TS, TY, KP, 2>(p, planes, ldp, g, N, K, x, y, acc, s);
    case 4: return launch_lut_kp<TX, TS, TY, KP, 4>(p, planes, ldp, g, N, K, x, y, acc, s);
    case 6: return launch_lut_kp<TX, TS, TY, KP, 6>(p, planes, ldp, g, N, K, x, y, acc, s);
    default: return launch_lut_kp<TX, TS, TY, KP, 8>(p, planes, ldp, g, N, K, x, y, acc, s);
  }
}

template <typename TX, typename TS, typename TY>
hipError_t launch_lut(const uint32_t* planes, int64_t ldp, const void* g, int k, int64_t N, int64_t K,
                      const void* x, void* y, void* ws, hipStream_t s) {
  const LutPlan p = lut_plan(N, K, device_cu_count());
  unsigned long long* acc = static_cast<unsigned long long*>(ws);
  switch (k) {
    case 1: return launch_lut_pairs<TX, TS, TY, 1>(p, planes, ldp, g, N, K, x, y, acc, s);
    case 2: return launch_lut_pairs<TX, TS, TY, 2>(p, planes, ldp, g, N, K, x, y, acc, s);
    case 3: return launch_lut_pairs<TX, TS, TY, 3>(p, planes, ldp, g, N, K, x, y, acc, s);
    case 4: return launch_lut_pairs<TX, TS, TY, 4>(p, planes, ldp, g, N, K, x, y, acc, s);
    default: return hipErrorInvalidValue;
  }
}

template <typename TX, typename TS, typename TY>
hipError_t launch_direct(const uint32_t* planes, int64_t ldp, const void* g, const void* h, int k,
                         int64_t N, int64_t K, const void* x, int64_t M, void* y, const void* mu, int zero_one,
                         hipStream_t s) {
  const int64_t rows_per_block = (int64_t)kRowsPerWave * kWavesPerBlock;
  const unsigned gx = (unsigned)((N + rows_per_block - 1) / rows_per_block);
  if (M == 1) {
    gemv_direct_kernel<TX, TS, TY, 1><<<dim3(gx, 1), dim3(256), 0, s>>>(
        planes, ldp, static_cast<const TS*>(g), static_cast<const TS*>(h), k, N, K,
        static_cast<const TX*>(x), M, static_cast<TY*>(y), static_cast<const TS*>(mu), zero_one);
  } else {
    gemv_direct_kernel<TX, TS, TY, 4><<<dim3(gx, (unsigned)((M + 3) / 4)), dim3(256), 0, s>>>(
        planes, ldp, static_cast<const TS*>(g), static_cast<const TS*>(h), k, N, K,
        static_cast<const TX*>(x), M, static_cast<TY*>(y), static_cast<const TS*>(mu), zero_one);
  }
  return hipGetLastError();
}

template <typename TX, typename TS>
hipError_t launch_y(rb_dtype y_dtype, const uint32_t* planes, int64_t ldp, const void* g,
                    const void* h, int k, int64_t N, int64_t K, const void* x, int64_t M, void* y,
                    void* ws, const void* mu, int zero_one, hipStream_t s) {
  if (M == 1 && h == nullptr && mu == nullptr && !zero_one && lut_fits(k, N, K, ldp, sizeof(TX), sizeof(TS))) {
    if (y_dtype == RB_F16) return launch_lut<TX, TS, __half>(planes, ldp, g, k, N, K, x, y, ws, s);
    return launch_lut<TX, TS, float>(planes, ldp, g, k, N, K, x, y, ws, s);
  }
  if (y_dtype == RB_F16) return launch_direct<TX, TS, __half>(planes, ldp, g, h, k, N, K, x, M, y, mu, zero_one, s);
  return launch_direct<TX, TS, float>(planes, ldp, g, h, k, N, K, x, M, y, mu, zero_one, s);
}

template <typename TX>
hipError_t launch_s(rb_dtype scale_dtype, rb_dtype y_dtype, const uint32_t* planes, int64_t ldp,
                    const void* g, const void* h, int k, int64_t N, int64_t K, const void* x,
                    int64_t M, void* y, void* ws, const void* mu, int zero_one, hipStream_t s) {
  if (scale_dtype == RB_F16)
    return launch_y<TX, __half>(y_dtype, planes, ldp, g, h, k, N, K, x, M, y, ws, mu, zero_one, s);
  return launch_y<TX, float>(y_dtype, planes, ldp, g, h, k, N, K, x, M, y, ws, mu, zero_one, s);
}

}  // namespace

size_t zero_region_bytes(int64_t N) {
  return (size_t)(((N * 8 + 255) / 256) * 256);  // one 64-bit accumulator per row
}

// compute units of the current device (cached per device)
int device_cu_count() {
  static int cached[64] = {0};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  if (cached[dev] == 0) {
    int cus = 0;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0) cus = 256;
    cached[dev] = cus;
  }
  return cached[dev];
}

// Batches of a few rows on the matrix cores: the MFMA kernel's time is nearly flat in M up to
// 16 (4096x11008, k = 2: 13.6 us at M = 4 and 14.7 us at M = 16), while the nibble kernel
// streams the planes once per activation row (5.6 us per row). Measured crossovers on
// 4096x4096, 11008x4096, 4096x11008 (k = 1, 2) fall at M = 3..4: M = 3 goes to the matrix
// cores on the two oblong layers (4096x11008, k = 2: 13.8 against 17.4 us; 11008x4096, k = 2:
// 14.5 against 15.3 us, k = 1: 11.1 against 11.6 us) and stays on the nibble passes on
// 4096x4096 (10.0 against 10.3 us); M = 2 goes there on 28672x8192 (2^27 bits and more). With
// column scales h likewise. The kernel takes fp16 x, K a multiple of 64, an even ldp, and h
// only as fp16 (16-byte aligned).
static bool gemv_on_matrix_cores(int k, int64_t N, int64_t K, int64_t ldp, int64_t M, const void* h, rb_dtype x_dtype,
                                 rb_dtype scale_dtype) {
  if (M < 2 || x_dtype != RB_F16 || K % 64 != 0 || ldp % 2 != 0) return false;
  if (K > (int64_t(1) << 22) || ldp > (int64_t(1) << 20)) return false;
  if (h != nullptr && (scale_dtype != RB_F16 || (reinterpret_cast<uintptr_t>(h) & 15u) != 0)) return false;
  return M >= 4 || (M == 3 && (K >= 2 * N || N >= 2 * K)) || (double)k * (double)N * (double)K >= 134217728.0;
}

// Workspace: first the LUT path's region (M = 1: one 64-bit accumulator per row; the general-h
// chain's fp32 row sums), zero between calls; after it, for K a multiple of 64, the K-chunk
// partial sums of the matrix-core kernel at M = 16 (written before they are read, so their
// contents do not matter). Sized for M = 16 whatever M is asked for, so one workspace serves
// every batch size of a layer.
size_t gemv_workspace_bytes(int k, int64_t N, int64_t K, int64_t) {
  return lut_workspace_bytes(N, K) + (K % 64 == 0 ? gemm_small_workspace_bytes(k, N, K, 16) : 0u);
}

hipError_t launch_gemv_variant(const uint32_t* planes, int64_t ldp, const void* g, const void* h,
                               const void* mu, int zero_one, rb_dtype scale_dtype, int k, int64_t N, int64_t K,
                               const void* x, rb_dtype x_dtype, int64_t M, void* y, rb_dtype y_dtype, void* ws,
                               hipStream_t s) {
  // two activation rows with h = 1 where the one-build nibble kernel applies: one launch that
  // reads the planes once and runs the table build and lookups once per row
  if (mu == nullptr && !zero_one && h == nullptr &&
      gemv_nib_rows_fits(k, N, K, ldp, M, x_dtype, scale_dtype, y_dtype))
    return launch_gemv_nib_rows(planes, ldp, g, k, N, K, x, M, y, s);
  if (mu == nullptr && !zero_one && ws != nullptr &&
      gemv_on_matrix_cores(k, N, K, ldp, M, h, x_dtype, scale_dtype))
    return launch_gemm_small(planes, ldp, g, h, scale_dtype, k, N, K, x, M, y, y_dtype,
                             static_cast<char*>(ws) + lut_workspace_bytes(N, K), s);
  // one activation row, h = 1: the whole-row nibble-table kernel where it applies (fp16
  // data, k <= 2), else the byte-table kernel (plain product only) or the direct kernel
  if (M == 1 && h == nullptr && gemv_nib_fits(k, N, K, ldp, x_dtype, scale_dtype, y_dtype)) {
    const hipError_t e =
        launch_gemv_nib(planes, ldp, g, scale_dtype, k, N, K, x, x_dtype, y, y_dtype, mu, zero_one, s);
    if (e != hipErrorNotSupported) return e;
  }
  // one activation row with column scales h (fp16): the nibble kernel once per plane, x (.) h_i
  // in its tables, the planes' sums chained in fp32 through the workspace (left zero)
  // (and per activation row for a few rows whose starts stay 16-byte aligned)
  if (M <= 16 && (M == 1 || K % 8 == 0) && h != nullptr && mu == nullptr && ws != nullptr &&
      gemv_nib_h_fits(k, N, K, ldp, h, x_dtype, scale_dtype, y_dtype)) {
    for (int64_t m = 0; m < M; ++m) {
      const hipError_t e = launch_gemv_nib_h(planes, ldp, g, h, k, N, K, static_cast<const __half*>(x) + m * K,
                                             static_cast<__half*>(y) + m * N, zero_one, static_cast<float*>(ws), s);
      if (e != hipSuccess) return e;
    }
    return hipSuccess;
  }
  // a few activation rows (fp16, h = 1, rows of x that stay 16-byte aligned): the nibble kernel
  // once per row. Each row re-reads the planes, but a row costs about what the M = 1 product
  // does, against ~3 VALU operations per weight bit and batch row in the direct kernel.
  if (M > 1 && M <= 16 && h == nullptr && K % 8 == 0 &&
      gemv_nib_fits(k, N, K, ldp, x_dtype, scale_dtype, y_dtype)) {
    for (int64_t m = 0; m < M; ++m) {
      const hipError_t e = launch_gemv_nib(planes, ldp, g, scale_dtype, k, N, K, static_cast<const __half*>(x) + m * K,
                                           x_dtype, static_cast<__half*>(y) + m * N, y_dtype, mu, zero_one, s);
      if (e != hipSuccess) return e;
    }
    return hipSuccess;
  }
  if (x_dtype == RB_F16)
    return launch_s<__half>(scale_dtype, y_dtype, planes, ldp, g, h, k, N, K, x, M, y, ws, mu, zero_one, s);
  return launch_s<float>(scale_dtype, y_dtype, planes, ldp, g, h, k, N, K, x, M, y, ws, mu, zero_one, s);
}

hipError_t launch_gemv(const uint32_t* planes, int64_t ldp, const void* g, const void* h,
                       rb_dtype scale_dtype, int k, int64_t N, int64_t K, const void* x,
                       rb_dtype x_dtype, int64_t M, void* y, rb_dtype y_dtype, void* ws, hipStream_t s) {
  return launch_gemv_variant(planes, ldp, g, h, nullptr, 0, scale_dtype, k, N, K, x, x_dtype, M, y, y_dtype, ws, s);
}

}  // namespace rb
