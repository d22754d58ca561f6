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
// codeword with ties to the lowest index. With cnt (the E-step of the learning loop), each
// block is also counted for the M-step: cnt[j][v] += 1 and cnt[j][t] += bit t for its
// codeword j (integer atomics, spread over this long, ALU-bound kernel).
__global__ __launch_bounds__(256) void encode_kernel(const uint32_t* __restrict__ plane, int64_t ldp,
                                                     int64_t N, int64_t K,
                                                     const uint32_t* __restrict__ codebook, int c,
                                                     int v, uint16_t* __restrict__ idx,
                                                     uint32_t* __restrict__ cnt) {
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
  if (cnt) {
#pragma unroll
    for (int p = 0; p < kPatternsPerThread; ++p) {
      if (base + p < total) {
        uint32_t* __restrict__ row = cnt + (int64_t)(best[p] & 0xffffu) * (v + 1);
        atomicAdd(row + v, 1u);
        for (uint32_t b = pat[p]; b; b &= b - 1u) atomicAdd(row + __builtin_ctz(b), 1u);
      }
    }
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

// ---------------------------------------------------------------------------
// LUT product (M = 1, v = 20, group = 16).
//
// [BTC 2.1.2] LUT-GEMM replaces the dequantised dot product by sums of input blocks that
// are precomputed once and then accumulated by weight pattern. Here the precomputed sums
// are nibble tables over x: for every 4 consecutive columns, T[e] = sum_j (bit j of e ? +x
// : -x) over the 4 columns, for all 16 sign patterns e (the +-1 form, so no separate sum of
// x is needed). The codeword patterns of a row, concatenated, are exactly its sign bits; a
// 16-column scale group is 4 nibbles, so
//   y[n] = sum_q s[n][q] * (T[e_4q] + T[e_4q+1] + T[e_4q+2] + T[e_4q+3]).
// An 80-column unit (lcm of v = 20 and group = 16) is 4 codewords, 5 scale groups and 20
// nibbles; lane l of a row's wave takes units l and l + 64 of a phase.
//
// Layout: entry e of every table of a phase lies in one 8 KB row of LDS (entry-major),
// table slot 21 u + i for nibble i of unit u (20 nibbles + 1 pad slot per unit). The slot
// stride 21 is odd, so the 64 lanes of a wave, which read the same nibble i of 64
// consecutive units, hit 64 different banks whatever the pattern values; a lookup address is
// (e << 13) + 84 u + 4 i (4 i is the instruction's immediate offset).
//
// A block is 16 waves, one output row each, and runs the whole row: at most two phases of
// up to 97 units (15520 columns) whose tables are rebuilt in place, so the result needs no
// cross-block reduction, is deterministic and uses no workspace.
// ---------------------------------------------------------------------------
constexpr int kCbThreads = 1024;
constexpr int kCbRowsPerBlock = kCbThreads / 64;
constexpr int kCbUnitCols = 80;
constexpr int kCbSlots = 21;
constexpr int kCbEntryShift = 13;                                   // 8 KB per entry row
constexpr int kCbMaxUnits = (1 << kCbEntryShift) / (4 * kCbSlots);  // 97 units per phase
constexpr size_t kCbLdsBytes = (size_t)16 << kCbEntryShift;          // 128 KB

typedef uint32_t cb_u32x2 __attribute__((ext_vector_type(2)));

// the 16 +-x sums of one nibble table, written to its slot (x4: the 4 columns' activations)
__device__ __forceinline__ void cb_build_table(const float x4[4], uint32_t slot) {
  float lo[4], hi[4];
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    lo[e] = ((e & 1) ? x4[0] : -x4[0]) + ((e & 2) ? x4[1] : -x4[1]);
    hi[e] = ((e & 1) ? x4[2] : -x4[2]) + ((e & 2) ? x4[3] : -x4[3]);
  }
  typedef __attribute__((address_space(3))) float lds_f32p;
#pragma unroll
  for (int e = 0; e < 16; ++e)
    *(lds_f32p*)(size_t)(((uint32_t)e << kCbEntryShift) + slot * 4u) = lo[e & 3] + hi[e >> 2];
}

// 4 fp16 activations of one table from a b64 load; columns >= K are 0
__device__ __forceinline__ void cb_x4(cb_u32x2 raw, int64_t col0, int64_t K, float x4[4]) {
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const uint32_t h = (raw[j >> 1] >> (16 * (j & 1))) & 0xffffu;
    x4[j] = col0 + j < K ? __half2float(__ushort_as_half((uint16_t)h)) : 0.0f;
  }
}

// address of the nibble at bit 4i of d (i < 8) within entry-major tables: (nibble << 13) | base
template <int I>
__device__ __forceinline__ uint32_t cb_addr(uint32_t d, uint32_t base) {
  constexpr int sh = 4 * I;
  const uint32_t t = sh <= kCbEntryShift ? (d << (kCbEntryShift - sh)) : (d >> (sh - kCbEntryShift));
  return (t & (15u << kCbEntryShift)) | base;
}

// table value of nibble I of a unit (I < 20; nibble I lives in dword I / 8 at bit 4 (I % 8))
template <int I>
__device__ __forceinline__ float cb_nib(const uint32_t d[3], uint32_t base) {
  return lds_f32(cb_addr<I % 8>(d[I / 8], base) + 4u * I);
}

// +-x sum of the 16 columns of scale group R of a unit (nibbles 4R .. 4R+3)
template <int R>
__device__ __forceinline__ float cb_group(const uint32_t d[3], uint32_t base) {
  return (cb_nib<4 * R>(d, base) + cb_nib<4 * R + 1>(d, base)) +
         (cb_nib<4 * R + 2>(d, base) + cb_nib<4 * R + 3>(d, base));
}

template <int NPH>
__global__ __launch_bounds__(kCbThreads) __attribute__((amdgpu_waves_per_eu(1, 4))) void codebook_lut_kernel(
    const uint16_t* __restrict__ idx, const uint32_t* __restrict__ codebook, int c,
    const __half* __restrict__ s, int64_t N, int64_t K, const __half* __restrict__ x, __half* __restrict__ y,
    int units_per_phase) {
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int64_t n = (int64_t)blockIdx.x * kCbRowsPerBlock + wave;
  const int64_t nb = (K + 19) / 20;   // codeword blocks per row
  const int64_t G = (K + 15) / 16;    // scale groups per row
  const int UP = units_per_phase;
  const uint32_t OOB = 0x80000000u;

  // resources: x (whole dwords, the tail column masked below), this wave's idx and scale rows
  // (a row past N has no bytes, so it reads 0), the codebook
  const __amdgpu_buffer_rsrc_t rx = buffer_rsrc(x, (uint32_t)(((K * 2) + 3) & ~3ll));
  const __amdgpu_buffer_rsrc_t ri = buffer_rsrc(idx + (n < N ? n : 0) * nb, n < N ? (uint32_t)(nb * 2) : 0u);
  const __amdgpu_buffer_rsrc_t rs = buffer_rsrc(s + (n < N ? n : 0) * G, n < N ? (uint32_t)(G * 2) : 0u);
  const __amdgpu_buffer_rsrc_t rc = buffer_rsrc(codebook, (uint32_t)c * 4u);

  // 1. activations of this thread's tables (tables t and t + 1024 of each phase)
  cb_u32x2 xr[NPH][2];
#pragma unroll
  for (int ph = 0; ph < NPH; ++ph)
#pragma unroll
    for (int it = 0; it < 2; ++it) {
      const int p = tid + it * kCbThreads;
      const int64_t nib = (int64_t)20 * ph * UP + p;  // global nibble index
      const uint32_t off = p < 20 * UP ? (uint32_t)(nib * 8) : OOB;
      xr[ph][it] = __builtin_bit_cast(cb_u32x2, __builtin_amdgcn_raw_buffer_load_b64(rx, (int)off, 0, 0));
    }
  // activations first, in every wave, then the row data: requests return in order and the
  // table build must not wait behind the index stream
  __builtin_amdgcn_sched_barrier(0);
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_sched_barrier(0);

  // 2. indices and scales of this lane's units: the 4 indices of a unit are one 8-byte load,
  // its 5 scales one 12-byte load from the dword boundary at or below them. A dword that
  // straddles the end of a row's indices or scales may read as 0, so the row's last index and
  // last scale are also loaded alone and put in place (entries past the row's end meet
  // columns past K, whose activations are 0, so their values do not matter).
  typedef uint32_t cb_u32x3 __attribute__((ext_vector_type(3)));
  cb_u32x2 idw[NPH][2];
  cb_u32x3 scw[NPH][2];
#pragma unroll
  for (int ph = 0; ph < NPH; ++ph)
#pragma unroll
    for (int it = 0; it < 2; ++it) {
      const int ul = lane + 64 * it;
      const int64_t ug = (int64_t)ph * UP + ul;
      const bool ok = ul < UP;  // units past the phase read 0 through the row resources
      idw[ph][it] = __builtin_bit_cast(
          cb_u32x2, __builtin_amdgcn_raw_buffer_load_b64(ri, ok ? (int)(ug * 8) : (int)OOB, 0, 0));
      scw[ph][it] = __builtin_bit_cast(
          cb_u32x3, __builtin_amdgcn_raw_buffer_load_b96(rs, ok ? (int)((ug * 10) & ~3ll) : (int)OOB, 0, 0));
    }
  const uint32_t id_last = buf_u16(ri, (uint32_t)((nb - 1) * 2), 0);
  const uint32_t sc_last = buf_u16(rs, (uint32_t)((G - 1) * 2), 0);
  __builtin_amdgcn_sched_barrier(0);
  uint32_t id[NPH][2][4], sc[NPH][2][5];
#pragma unroll
  for (int ph = 0; ph < NPH; ++ph)
#pragma unroll
    for (int it = 0; it < 2; ++it) {
      const int64_t ug = (int64_t)ph * UP + lane + 64 * it;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const uint32_t v = (idw[ph][it][r >> 1] >> (16 * (r & 1))) & 0xffffu;
        id[ph][it][r] = 4 * ug + r == nb - 1 ? id_last : v;
      }
      // the unit's scales start 0 or 2 bytes into the loaded dwords
      const uint32_t sh = (uint32_t)((ug * 10) & 3) * 8u;
      const cb_u32x3 d = scw[ph][it];
      const uint32_t q[3] = {__builtin_amdgcn_alignbit(d[1], d[0], sh), __builtin_amdgcn_alignbit(d[2], d[1], sh),
                             d[2] >> sh};
#pragma unroll
      for (int r = 0; r < 5; ++r) {
        const uint32_t v = (q[r >> 1] >> (16 * (r & 1))) & 0xffffu;
        sc[ph][it][r] = 5 * ug + r == G - 1 ? sc_last : v;
      }
    }

  // 3. codewords (indices are < c by contract; clamped so a bad index cannot read past the codebook)
  uint32_t cw[NPH][2][4];
#pragma unroll
  for (int ph = 0; ph < NPH; ++ph)
#pragma unroll
    for (int it = 0; it < 2; ++it)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const uint32_t i = id[ph][it][r] < (uint32_t)c ? id[ph][it][r] : (uint32_t)(c - 1);
        cw[ph][it][r] = buf_u32(rc, i * 4u, 0);
      }
  __builtin_amdgcn_sched_barrier(0);

  float acc = 0.0f;
#pragma unroll
  for (int ph = 0; ph < NPH; ++ph) {
    // 4. tables of this phase (after every wave is done with the previous phase's)
    if (ph > 0) __syncthreads();
#pragma unroll
    for (int it = 0; it < 2; ++it) {
      // threads past the phase's tables write the pad slot of unit 0, which no lookup reads
      // (no branch: the activation loads above must not sink into one)
      const int p = tid + it * kCbThreads;
      const int u = p / 20, i = p - 20 * (p / 20);
      float x4[4];
      cb_x4(xr[ph][it], (int64_t)4 * (20 * (int64_t)ph * UP + p), K, x4);
      cb_build_table(x4, p < 20 * UP ? (uint32_t)(kCbSlots * u + i) : (uint32_t)(kCbSlots - 1));
    }
    __syncthreads();
    // 5. lookups: per unit 20 nibbles in 5 scale groups
#pragma unroll
    for (int it = 0; it < 2; ++it) {
      const int ul = lane + 64 * it;
      if (ul < UP) {
        uint32_t w[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) w[r] = cw[ph][it][r] & 0xfffffu;
        const uint32_t d[3] = {w[0] | (w[1] << 20), (w[1] >> 12) | (w[2] << 8) | (w[3] << 28), w[3] >> 4};
        const uint32_t base = (uint32_t)(kCbSlots * 4 * ul);
        float sf[5];
#pragma unroll
        for (int r = 0; r < 5; ++r) sf[r] = __half2float(__ushort_as_half((uint16_t)sc[ph][it][r]));
        acc += sf[0] * cb_group<0>(d, base);
        acc += sf[1] * cb_group<1>(d, base);
        acc += sf[2] * cb_group<2>(d, base);
        acc += sf[3] * cb_group<3>(d, base);
        acc += sf[4] * cb_group<4>(d, base);
      }
    }
  }
  acc = wave_sum_dpp(acc);
  if (lane == 63 && n < N) y[n] = __float2half_rn(acc);
}

// ---------------------------------------------------------------------------------------------
// binary K-means: M-step and the distinct patterns
// ---------------------------------------------------------------------------------------------
__global__ __launch_bounds__(256) void fill_u32_kernel(uint32_t* __restrict__ p, int64_t n, uint32_t val) {
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (int64_t)gridDim.x * 256) p[i] = val;
}

// M-step as a counting sort of the blocks by codeword, then a vote per codeword:
//   hist     members[c] = number of blocks with idx == c              (one atomic per block)
//   offsets  start[c] = exclusive prefix sum of members (one block)
//   scatter  each block's pattern goes to bucket[start[c] + cursor[c]++] (one atomic per block)
//   vote     thread c counts each bit over its bucket and sets the bits with 2 ones >= members
//            (sum of +-1 >= 0: ties go to +1); a codeword without members keeps its value.
// The order inside a bucket depends on the scheduling, the counts do not: the result is exact.
__global__ __launch_bounds__(256) void mstep_hist_kernel(const uint16_t* __restrict__ idx, int64_t total, int c,
                                                         uint32_t* __restrict__ members) {
  for (int64_t e = (int64_t)blockIdx.x * 256 + threadIdx.x; e < total; e += (int64_t)gridDim.x * 256) {
    const uint32_t id = idx[e];
    if (id < (uint32_t)c) atomicAdd(members + id, 1u);  // indices must be < c; others are skipped
  }
}

constexpr int kScanThreads = 1024;

// start[c] = sum of members[0..c), in two passes: each block of 1024 codewords scans its own
// range (exclusive, in LDS) and writes its total; then each block adds the totals of the
// blocks before it.
__global__ __launch_bounds__(kScanThreads) void mstep_scan_local_kernel(const uint32_t* __restrict__ members, int c,
                                                                        uint32_t* __restrict__ start,
                                                                        uint32_t* __restrict__ totals) {
  __shared__ uint32_t scan[2][kScanThreads];
  const int t = threadIdx.x;
  const int i = blockIdx.x * kScanThreads + t;
  const uint32_t mine = i < c ? members[i] : 0u;
  scan[0][t] = mine;
  __syncthreads();
  int src = 0;
  for (int off = 1; off < kScanThreads; off <<= 1) {  // inclusive scan, double-buffered
    scan[src ^ 1][t] = scan[src][t] + (t >= off ? scan[src][t - off] : 0u);
    src ^= 1;
    __syncthreads();
  }
  if (i < c) start[i] = scan[src][t] - mine;
  if (t == kScanThreads - 1) totals[blockIdx.x] = scan[src][t];
}

__global__ __launch_bounds__(kScanThreads) void mstep_scan_add_kernel(const uint32_t* __restrict__ totals, int c,
                                                                      uint32_t* __restrict__ start) {
  uint32_t pre = 0u;
  for (unsigned b = 0; b < blockIdx.x; ++b) pre += totals[b];  // at most 63 totals
  const int i = blockIdx.x * kScanThreads + threadIdx.x;
  if (i < c) start[i] += pre;
}

__global__ __launch_bounds__(256) void mstep_scatter_kernel(const uint32_t* __restrict__ plane, int64_t ldp,
                                                            int64_t N, int64_t K, int v,
                                                            const uint16_t* __restrict__ idx, int c,
                                                            const uint32_t* __restrict__ start,
                                                            uint32_t* __restrict__ cursor,
                                                            uint32_t* __restrict__ bucket) {
  const int64_t nb = (K + v - 1) / v;
  const int64_t total = N * nb;
  for (int64_t e = (int64_t)blockIdx.x * 256 + threadIdx.x; e < total; e += (int64_t)gridDim.x * 256) {
    const uint32_t id = idx[e];
    if (id >= (uint32_t)c) continue;
    const int64_t n = e / nb;
    const uint32_t b = extract_block(plane + n * ldp, K, (e - n * nb) * v, v);
    bucket[start[id] + atomicAdd(cursor + id, 1u)] = b;
  }
}

// one wave per codeword: its bucket is read 64 blocks at a time and each bit's count is the
// popcount of a ballot; bits with 2 ones >= members are set (ties go to +1)
__global__ __launch_bounds__(256) void mstep_vote_kernel(const uint32_t* __restrict__ members,
                                                         const uint32_t* __restrict__ start,
                                                         const uint32_t* __restrict__ bucket, int c, int v,
                                                         uint32_t* __restrict__ codebook,
                                                         uint32_t* __restrict__ counts) {
  const int lane = threadIdx.x & 63;
  const int id = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (id >= c) return;  // uniform per wave
  const uint32_t n = members[id];
  if (counts && lane == 0) counts[id] = n;
  if (n == 0) return;
  const uint32_t* __restrict__ bk = bucket + start[id];
  uint32_t ones[32];
#pragma unroll
  for (int t = 0; t < 32; ++t) ones[t] = 0u;
  for (uint32_t j0 = 0; j0 < n; j0 += 64) {
    const bool ok = j0 + (uint32_t)lane < n;
    const uint32_t b = ok ? bk[j0 + lane] : 0u;
#pragma unroll
    for (int t = 0; t < 32; ++t)
      if (t < v) ones[t] += (uint32_t)__popcll(__ballot((b >> t) & 1u));
  }
  uint32_t w = 0u;
#pragma unroll
  for (int t = 0; t < 32; ++t)
    if (t < v && 2ull * ones[t] >= n) w |= 1u << t;
  if (lane == 0) codebook[id] = w;
}

// the vote from the counters cnt[c][v + 1] filled by the counting E-step
__global__ __launch_bounds__(256) void mstep_vote_counts_kernel(const uint32_t* __restrict__ cnt, int c, int v,
                                                                uint32_t* __restrict__ codebook) {
  const int id = blockIdx.x * 256 + threadIdx.x;
  if (id >= c) return;
  const uint32_t* __restrict__ row = cnt + (int64_t)id * (v + 1);
  const uint64_t n = row[v];
  if (n == 0) return;
  uint32_t w = 0u;
  for (int t = 0; t < v; ++t) w |= (2ull * row[t] >= n ? 1u : 0u) << t;
  codebook[id] = w;
}

// bitmap of the 2^v possible patterns: bit p set when pattern p occurs
__global__ __launch_bounds__(256) void distinct_mark_kernel(const uint32_t* __restrict__ plane, int64_t ldp,
                                                            int64_t N, int64_t K, int v,
                                                            uint32_t* __restrict__ bitmap) {
  const int64_t nb = (K + v - 1) / v;
  const int64_t total = N * nb;
  for (int64_t e = (int64_t)blockIdx.x * 256 + threadIdx.x; e < total; e += (int64_t)gridDim.x * 256) {
    const int64_t n = e / nb;
    const uint32_t b = extract_block(plane + n * ldp, K, (e - n * nb) * v, v);
    atomicOr(bitmap + (b >> 5), 1u << (b & 31u));
  }
}

constexpr int kDistinctThreads = 1024;

// One block: M = number of set bits -> *n_distinct. If M < c, the patterns in ascending order
// go to codebook[0..M) and codebook[M..c) repeats the largest one. Thread t owns a contiguous
// range of bitmap words; its first output position is the exclusive scan of the ranges' counts.
__global__ __launch_bounds__(kDistinctThreads) void distinct_compact_kernel(const uint32_t* __restrict__ bitmap,
                                                                            int64_t nwords, int c,
                                                                            uint32_t* __restrict__ codebook,
                                                                            int32_t* __restrict__ n_distinct) {
  __shared__ uint32_t scan[2][kDistinctThreads];
  __shared__ int32_t top;
  const int t = threadIdx.x;
  const int64_t per = (nwords + kDistinctThreads - 1) / kDistinctThreads;
  const int64_t lo = (int64_t)t * per < nwords ? (int64_t)t * per : nwords;
  const int64_t hi = lo + per < nwords ? lo + per : nwords;
  uint32_t mine = 0u;
  int32_t last = -1;
  for (int64_t w = lo; w < hi; ++w) {
    const uint32_t b = bitmap[w];
    mine += (uint32_t)__popc(b);
    if (b) last = (int32_t)(w * 32 + 31 - __builtin_clz(b));
  }
  if (t == 0) top = -1;
  scan[0][t] = mine;
  __syncthreads();
  if (last >= 0) atomicMax(&top, last);
  int src = 0;
  for (int off = 1; off < kDistinctThreads; off <<= 1) {  // inclusive scan, double-buffered
    scan[src ^ 1][t] = scan[src][t] + (t >= off ? scan[src][t - off] : 0u);
    src ^= 1;
    __syncthreads();
  }
  const uint32_t total = scan[src][kDistinctThreads - 1];
  if (t == 0) *n_distinct = (int32_t)total;
  if (total >= (uint32_t)c) return;
  uint32_t pos = scan[src][t] - mine;
  for (int64_t w = lo; w < hi; ++w) {
    uint32_t b = bitmap[w];
    while (b) {
      codebook[pos++] = (uint32_t)(w * 32) + (uint32_t)__builtin_ctz(b);
      b &= b - 1u;
    }
  }
  for (int64_t i = (int64_t)total + t; i < c; i += kDistinctThreads) codebook[i] = (uint32_t)top;
}

unsigned stride_grid(int64_t items) {
  const int64_t b = (items + 255) / 256;
  return (unsigned)(b < 1 ? 1 : b > (1 << 20) ? (1 << 20) : b);
}

}  // namespace

hipError_t launch_codebook_encode(const uint32_t* plane, int64_t ldp, int64_t N, int64_t K,
                                  const uint32_t* codebook, int c, int v, uint16_t* idx,
                                  hipStream_t s) {
  const int64_t nb = (K + v - 1) / v;
  const int64_t total = N * nb;
  const int64_t per_block = 256 * kPatternsPerThread;
  const unsigned grid = (unsigned)((total + per_block - 1) / per_block);
  encode_kernel<<<grid, 256, 0, s>>>(plane, ldp, N, K, codebook, c, v, idx, nullptr);
  return hipGetLastError();
}

size_t codebook_gemv_workspace_bytes(int64_t, int64_t, int64_t) { return 0; }

template <int NPH>
hipError_t launch_codebook_lut(const uint16_t* idx, const uint32_t* codebook, int c, const void* s, int64_t N,
                               int64_t K, const void* x, void* y, int units_per_phase, hipStream_t st) {
  static bool attr_set = false;  // per instantiation
  if (!attr_set) {
    const hipError_t e = hipFuncSetAttribute((const void*)codebook_lut_kernel<NPH>,
                                             hipFuncAttributeMaxDynamicSharedMemorySize, (int)kCbLdsBytes);
    if (e != hipSuccess) return e;
    attr_set = true;
  }
  const unsigned grid = (unsigned)((N + kCbRowsPerBlock - 1) / kCbRowsPerBlock);
  codebook_lut_kernel<NPH><<<grid, kCbThreads, kCbLdsBytes, st>>>(
      idx, codebook, c, static_cast<const __half*>(s), N, K, static_cast<const __half*>(x),
      static_cast<__half*>(y), units_per_phase);
  return hipGetLastError();
}

hipError_t launch_codebook_gemv(const uint16_t* idx, const uint32_t* codebook, int c, int v,
                                const void* s, int group, int64_t N, int64_t K, const void* x,
                                int64_t M, void* y, void*, hipStream_t st) {
  // the LUT path: one activation row, the pages' block and group sizes, rows of at most two
  // phases, and 32-bit byte offsets into the index and scale arrays
  const int64_t units = (K + kCbUnitCols - 1) / kCbUnitCols;
  const int64_t phases = (units + kCbMaxUnits - 1) / kCbMaxUnits;
  if (M == 1 && v == 20 && group == 16 && phases <= 2 && N * ((K + 19) / 20) * 2 < 0x7fffffffll &&
      N * ((K + 15) / 16) * 2 < 0x7fffffffll) {
    const int up = (int)((units + phases - 1) / phases);
    if (phases == 1) return launch_codebook_lut<1>(idx, codebook, c, s, N, K, x, y, up, st);
    return launch_codebook_lut<2>(idx, codebook, c, s, N, K, x, y, up, st);
  }
  const dim3 grid((unsigned)((N + 3) / 4), (unsigned)M);
  codebook_gemv_kernel<<<grid, 256, 0, st>>>(idx, codebook, c, v, static_cast<const __half*>(s), group,
                                             N, K, static_cast<const __half*>(x), M,
                                             static_cast<__half*>(y));
  return hipGetLastError();
}

// workspace, used by one step at a time: the standalone M-step's members, start, cursor ([c]
// each), block totals (64) and bucket (one word per block); the learning loop's counters
// [c][v + 1]; the 2^v-bit bitmap of the distinct count
size_t codebook_learn_workspace_bytes(int64_t N, int64_t K, int c, int v) {
  const size_t blocks = (size_t)N * (size_t)((K + v - 1) / v);
  const size_t mstep = 4u * (3u * (size_t)c + 64u + blocks);
  const size_t counters = 4u * (size_t)c * (size_t)(v + 1);
  const size_t bitmap = v <= 24 ? ((size_t)1 << (v > 5 ? v - 3 : 2)) : 0u;
  size_t m = mstep > counters ? mstep : counters;
  return m > bitmap ? m : bitmap;
}

hipError_t launch_codebook_mstep(const uint32_t* plane, int64_t ldp, int64_t N, int64_t K, int v,
                                 const uint16_t* idx, uint32_t* codebook, int c, uint32_t* counts, void* ws,
                                 hipStream_t s) {
  uint32_t* members = static_cast<uint32_t*>(ws);
  uint32_t* start = members + c;
  uint32_t* cursor = start + c;
  uint32_t* totals = cursor + c;
  uint32_t* bucket = totals + 64;
  const int64_t total = N * ((K + v - 1) / v);
  const unsigned nscan = (unsigned)((c + kScanThreads - 1) / kScanThreads);
  fill_u32_kernel<<<stride_grid(3 * (int64_t)c), 256, 0, s>>>(members, 3 * (int64_t)c, 0u);
  mstep_hist_kernel<<<stride_grid(total), 256, 0, s>>>(idx, total, c, members);
  mstep_scan_local_kernel<<<nscan, kScanThreads, 0, s>>>(members, c, start, totals);
  mstep_scan_add_kernel<<<nscan, kScanThreads, 0, s>>>(totals, c, start);
  mstep_scatter_kernel<<<stride_grid(total), 256, 0, s>>>(plane, ldp, N, K, v, idx, c, start, cursor, bucket);
  mstep_vote_kernel<<<(unsigned)((c + 3) / 4), 256, 0, s>>>(members, start, bucket, c, v, codebook, counts);
  return hipGetLastError();
}

hipError_t launch_codebook_distinct(const uint32_t* plane, int64_t ldp, int64_t N, int64_t K, int v,
                                    uint32_t* codebook, int c, int32_t* n_distinct, void* ws, hipStream_t s) {
  uint32_t* bitmap = static_cast<uint32_t*>(ws);
  const int64_t nwords = v > 5 ? (int64_t)1 << (v - 5) : 1;
  fill_u32_kernel<<<stride_grid(nwords), 256, 0, s>>>(bitmap, nwords, 0u);
  const int64_t total = N * ((K + v - 1) / v);
  distinct_mark_kernel<<<stride_grid(total), 256, 0, s>>>(plane, ldp, N, K, v, bitmap);
  distinct_compact_kernel<<<1, kDistinctThreads, 0, s>>>(bitmap, nwords, c, codebook, n_distinct);
  return hipGetLastError();
}

hipError_t launch_codebook_learn(const uint32_t* plane, int64_t ldp, int64_t N, int64_t K, int v,
                                 uint32_t* codebook, int c, int iters, uint16_t* idx, int32_t* n_distinct,
                                 void* ws, hipStream_t s) {
  hipError_t e = launch_codebook_distinct(plane, ldp, N, K, v, codebook, c, n_distinct, ws, s);
  // each iteration: the E-step counts the members and their bits as it assigns them, then the
  // vote replaces the codewords (a codeword without members keeps its value)
  uint32_t* cnt = static_cast<uint32_t*>(ws);
  const int64_t ncnt = (int64_t)c * (v + 1);
  const int64_t total = N * ((K + v - 1) / v);
  const unsigned egrid = (unsigned)((total + 256 * kPatternsPerThread - 1) / (256 * kPatternsPerThread));
  for (int it = 0; it < iters && e == hipSuccess; ++it) {
    fill_u32_kernel<<<stride_grid(ncnt), 256, 0, s>>>(cnt, ncnt, 0u);
    encode_kernel<<<egrid, 256, 0, s>>>(plane, ldp, N, K, codebook, c, v, idx, cnt);
    mstep_vote_counts_kernel<<<(unsigned)((c + 255) / 256), 256, 0, s>>>(cnt, c, v, codebook);
    e = hipGetLastError();
  }
  if (e == hipSuccess) e = launch_codebook_encode(plane, ldp, N, K, codebook, c, v, idx, s);
  return e;
}

}  // namespace rb
