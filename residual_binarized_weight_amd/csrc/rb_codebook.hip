// rb_codebook.hip -- sub-1-bit binary codebook: encode and product (gfx950).
//
// [BTC-LLM page, 2.1.1] The sign matrix is cut into v-column +-1 sub-vectors; each is
// replaced by the index of its nearest codeword in Hamming distance (XOR + popcount).
// [BTC-LLM page, 2.1.2 and 3.2.1] The product runs on the indices with one scale per
// 16 weights, without dequantising the matrix.
#include "rb_device.hpp"
#include "rb_internal.h"

#include <type_traits>

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

// extract_block from the two words already loaded: lo = word col / 32 of the row, hi = the next
// (their loads may be clamped; words at or past Kw count as zero here)
__device__ __forceinline__ uint32_t block_from_words(uint32_t lo, uint32_t hi, int64_t col, int64_t K, int64_t Kw,
                                                     int v) {
  const int64_t w = col >> 5;
  const uint64_t both = ((uint64_t)(w + 1 < Kw ? hi : 0u) << 32) | (w < Kw ? lo : 0u);
  const uint32_t vmask = v == 32 ? 0xffffffffu : ((1u << v) - 1u);
  uint32_t b = (uint32_t)(both >> (col & 31)) & vmask;
  const int64_t real = K - col;  // columns of this block that exist
  if (real < v) b |= vmask & ~((1u << real) - 1u);
  return b;
}

// the two words block_from_words needs, loaded unconditionally at clamped addresses
__device__ __forceinline__ void load_block_words(const uint32_t* __restrict__ prow, int64_t col, int64_t Kw,
                                                 uint32_t& lo, uint32_t& hi) {
  const int64_t w = col >> 5;
  lo = prow[w < Kw ? w : Kw - 1];
  hi = prow[w + 1 < Kw ? w + 1 : Kw - 1];
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

// M-step as one radix pass of the blocks on the high byte of their codeword index, then counts
// per codeword in LDS (no global atomics; idx and the plane are read in order, never gathered):
//   hist     chunk q of 8192 blocks: H[bucket][q] = its blocks with idx >> 8 == bucket
//   scan     per bucket, H[bucket][.] becomes the exclusive prefix over the chunks, and
//            btot[bucket] the bucket's total
//   scatter  chunk q extracts each block's v-bit pattern and writes it to Rp, and the low byte of
//            its index to Rb (v > 24) or to Rp's top byte (v <= 24), at the bucket's start +
//            H[bucket][q] + a rank from an LDS counter (the order inside a bucket is the
//            scheduler's)
//   vote     one block per slice of up to 4096 consecutive records of one bucket: members and
//            ones per bit of each of the bucket's 256 codewords, counted with LDS atomics and
//            written as the slice's table
//   finish   per codeword, the sums over its bucket's slices; a bit is set when 2 ones >=
//            members (ties go to +1); a codeword without members keeps its value.
// Integer counts, so the result does not depend on any order: exact and deterministic.
constexpr int kMsChunk = 8192;    // blocks per histogram / scatter chunk
constexpr int kMsThreads = 256;   // one thread per bucket in the chunk kernels
constexpr int kMsBuckets = 256;   // idx >> 8

// buckets' exclusive starts from their totals, in LDS (one thread per bucket)
__device__ __forceinline__ void ms_bucket_starts(const uint32_t* __restrict__ btot, uint32_t* start, int tid) {
  start[tid] = btot[tid];
  __syncthreads();
  for (int off = 1; off < kMsBuckets; off <<= 1) {  // inclusive scan in place (Hillis-Steele)
    const uint32_t add = tid >= off ? start[tid - off] : 0u;
    __syncthreads();
    start[tid] += add;
    __syncthreads();
  }
  const uint32_t incl = start[tid];
  __syncthreads();
  start[tid] = incl - btot[tid];
  __syncthreads();
}

__global__ __launch_bounds__(kMsThreads) void mstep_hist_kernel(const uint16_t* __restrict__ idx, int64_t total,
                                                                int c, int64_t nchunk, uint32_t* __restrict__ H) {
  __shared__ uint32_t h[kMsBuckets];
  const int tid = threadIdx.x;
  h[tid] = 0u;
  __syncthreads();
  const int64_t e0 = (int64_t)blockIdx.x * kMsChunk;
  constexpr int kU = 8;  // indices per thread loaded together, at clamped addresses
  for (int k0 = 0; k0 < kMsChunk / kMsThreads; k0 += kU) {
    uint32_t id[kU];
#pragma unroll
    for (int u = 0; u < kU; ++u) {
      const int64_t e = e0 + (k0 + u) * kMsThreads + tid;
      id[u] = e < total ? (uint32_t)idx[e] : 0xffffffffu;  // past the end: skipped below
    }
#pragma unroll
    for (int u = 0; u < kU; ++u)
      if (id[u] < (uint32_t)c) atomicAdd(&h[id[u] >> 8], 1u);  // indices >= c are skipped
  }
  __syncthreads();
  H[(int64_t)tid * nchunk + blockIdx.x] = h[tid];
}

// block b: exclusive prefix of H[b][0 .. nchunk) over the chunks, 256 at a time with a carry
__global__ __launch_bounds__(kMsThreads) void mstep_scan_kernel(uint32_t* __restrict__ H, int64_t nchunk,
                                                                uint32_t* __restrict__ btot) {
  __shared__ uint32_t t[kMsThreads];
  const int tid = threadIdx.x;
  uint32_t* __restrict__ row = H + (int64_t)blockIdx.x * nchunk;
  uint32_t carry = 0u;
  for (int64_t q0 = 0; q0 < nchunk; q0 += kMsThreads) {
    const int64_t q = q0 + tid;
    const uint32_t mine = q < nchunk ? row[q] : 0u;
    t[tid] = mine;
    __syncthreads();
    for (int off = 1; off < kMsThreads; off <<= 1) {
      const uint32_t add = tid >= off ? t[tid - off] : 0u;
      __syncthreads();
      t[tid] += add;
      __syncthreads();
    }
    if (q < nchunk) row[q] = carry + t[tid] - mine;
    carry += t[kMsThreads - 1];
    __syncthreads();
  }
  if (tid == 0) btot[blockIdx.x] = carry;
}

__global__ __launch_bounds__(kMsThreads) void mstep_scatter_kernel(const uint32_t* __restrict__ plane, int64_t ldp,
                                                                   int64_t K, int v, const uint16_t* __restrict__ idx,
                                                                   int64_t total, int c, int64_t nchunk,
                                                                   const uint32_t* __restrict__ H,
                                                                   const uint32_t* __restrict__ btot,
                                                                   uint32_t* __restrict__ Rp, uint8_t* __restrict__ Rb) {
  __shared__ uint32_t cur[kMsBuckets];
  const int tid = threadIdx.x;
  ms_bucket_starts(btot, cur, tid);
  cur[tid] += H[(int64_t)tid * nchunk + blockIdx.x];
  __syncthreads();
  const uint32_t nb = (uint32_t)((K + v - 1) / v);  // blocks per row; total < 2^32
  const int64_t Kw = (K + 31) >> 5;
  const uint32_t e0 = blockIdx.x * (uint32_t)kMsChunk;
  constexpr int kU = 4;  // blocks per thread whose loads are in flight together
  for (int k0 = 0; k0 < kMsChunk / kMsThreads; k0 += kU) {
    uint32_t id[kU], lo[kU], hi[kU];
    int64_t col[kU];
    bool ok[kU];
#pragma unroll
    for (int u = 0; u < kU; ++u) {  // loads at clamped addresses, unconditionally
      const int64_t e64 = (int64_t)e0 + (k0 + u) * kMsThreads + tid;
      ok[u] = e64 < total;
      const uint32_t e = ok[u] ? (uint32_t)e64 : (uint32_t)(total - 1);
      id[u] = idx[e];
      const uint32_t n = e / nb;
      col[u] = (int64_t)(e - n * nb) * v;
      load_block_words(plane + (int64_t)n * ldp, col[u], Kw, lo[u], hi[u]);
    }
#pragma unroll
    for (int u = 0; u < kU; ++u) {
      if (!ok[u] || id[u] >= (uint32_t)c) continue;  // indices >= c are skipped
      const uint32_t pat = block_from_words(lo[u], hi[u], col[u], K, Kw, v);
      const uint32_t pos = atomicAdd(&cur[id[u] >> 8], 1u);
      if (v <= 24) {  // one word per record: the index byte above the pattern
        Rp[pos] = pat | (id[u] << 24);
      } else {
        Rp[pos] = pat;
        Rb[pos] = (uint8_t)(id[u] & 0xffu);
      }
    }
  }
}

constexpr int kMsVoteThreads = 1024;  // the vote's block
constexpr int kMsVoteUnroll = 4;      // members in flight per thread
constexpr int kMsSlice = kMsVoteThreads * kMsVoteUnroll;  // members per vote block

// A bucket's members are cut into slices of kMsSlice, so a popular bucket does not hold up the
// launch: slice counts per bucket = ceil(members / kMsSlice), their exclusive prefix gives each
// bucket's first slice. Computed in LDS by the first 256 threads of any block size (every thread
// passes the barriers): start[b] = first member, first[b] = first slice, nsl[b] = slices.
__device__ __forceinline__ void ms_slices(const uint32_t* __restrict__ btot, uint32_t* start, uint32_t* first,
                                          uint32_t* nsl, int tid) {
  const bool own = tid < kMsBuckets;
  const uint32_t m = own ? btot[tid] : 0u;
  const uint32_t ns = (m + kMsSlice - 1) / kMsSlice;
  if (own) {
    start[tid] = m;
    first[tid] = ns;
    nsl[tid] = ns;
  }
  __syncthreads();
  for (int off = 1; off < kMsBuckets; off <<= 1) {  // inclusive scans in place (Hillis-Steele)
    const uint32_t a0 = (own && tid >= off) ? start[tid - off] : 0u;
    const uint32_t a1 = (own && tid >= off) ? first[tid - off] : 0u;
    __syncthreads();
    if (own) {
      start[tid] += a0;
      first[tid] += a1;
    }
    __syncthreads();
  }
  if (own) {
    start[tid] -= m;
    first[tid] -= ns;
  }
  __syncthreads();
}

// one slice: its members' counts (members, ones per bit) per codeword of the bucket, written as
// P[slice][t][256] (t = 0..v-1 the bits, t = v the members); blocks past the last slice exit
__global__ __launch_bounds__(kMsVoteThreads) void mstep_vote_kernel(int v, const uint32_t* __restrict__ Rp,
                                                                    const uint8_t* __restrict__ Rb,
                                                                    const uint32_t* __restrict__ btot,
                                                                    uint32_t* __restrict__ P) {
  // [codeword][W]: counters t = 2 k (low half) and 2 k + 1 (high half) of word k, t = v the
  // members; a slice holds at most 4096 records, so 16 bits never carry
  __shared__ uint32_t cnt[kMsBuckets * 17];
  __shared__ uint32_t start[kMsBuckets], first[kMsBuckets], nsl[kMsBuckets];
  const int tid = threadIdx.x;
  const int stride = v + 1;
  const int W = (v + 2) / 2;
  for (int i = tid; i < kMsBuckets * W; i += kMsVoteThreads) cnt[i] = 0u;
  ms_slices(btot, start, first, nsl, tid);
  const uint32_t slice = blockIdx.x;
  if (slice >= first[kMsBuckets - 1] + nsl[kMsBuckets - 1]) return;  // whole block
  // the bucket whose slices cover this one: the last with first <= slice. It is never empty: an
  // empty bucket shares its first slice with the next bucket, and slice < the total slice count.
  int bk = 0;
  for (int step = kMsBuckets / 2; step > 0; step >>= 1)
    if (first[bk + step] <= slice) bk += step;
  const uint32_t j = slice - first[bk];
  const uint32_t lo = start[bk] + j * (uint32_t)kMsSlice;
  const uint32_t hi = min(lo + (uint32_t)kMsSlice, start[bk] + btot[bk]);
  uint32_t pat[kMsVoteUnroll], r[kMsVoteUnroll];
  bool live[kMsVoteUnroll];
#pragma unroll
  for (int u = 0; u < kMsVoteUnroll; ++u) {  // the slice's records, all loads issued first
    const uint32_t q = lo + (uint32_t)(u * kMsVoteThreads + tid);
    live[u] = q < hi;
    const uint32_t rec = live[u] ? Rp[q] : 0u;
    if (v <= 24) {  // the index byte sits above the pattern
      pat[u] = rec & 0xffffffu;
      r[u] = rec >> 24;
    } else {
      pat[u] = rec;
      r[u] = live[u] ? (uint32_t)Rb[q] : 0u;
    }
  }
#pragma unroll
  for (int u = 0; u < kMsVoteUnroll; ++u) {
    if (!live[u]) continue;
    uint32_t* row = cnt + r[u] * (uint32_t)W;
    const uint64_t all = (uint64_t)pat[u] | (1ull << v);  // the pattern's bits, then the member
    for (int k = 0; k < W; ++k) {
      const uint32_t add = (uint32_t)((all >> (2 * k)) & 1u) | ((uint32_t)((all >> (2 * k + 1)) & 1u) << 16);
      if (add) atomicAdd(row + k, add);
    }
  }
  __syncthreads();
  uint32_t* __restrict__ out = P + (size_t)slice * (size_t)(kMsBuckets * stride);
  for (int i = tid; i < kMsBuckets * stride; i += kMsVoteThreads) {
    const int t = i / kMsBuckets, cw = i % kMsBuckets;
    out[i] = (cnt[cw * W + (t >> 1)] >> (16 * (t & 1))) & 0xffffu;
  }
}

// block b, thread = codeword 256 b + tid: sums the bucket's slices and votes; a bit is set when
// 2 ones >= members (ties go to +1); a codeword without members keeps its value. All v + 1 sums
// stay in registers, so each slice costs one round of loads.
// one wave per SIMD at most (256 blocks of 4 waves): registers for all v + 1 loads of a slice
// in flight matter more than occupancy
__global__ __launch_bounds__(kMsBuckets) __attribute__((amdgpu_waves_per_eu(1, 2))) void mstep_finish_kernel(const uint32_t* __restrict__ P,
                                                                  const uint32_t* __restrict__ btot, int v, int c,
                                                                  uint32_t* __restrict__ codebook,
                                                                  uint32_t* __restrict__ counts) {
  __shared__ uint32_t start[kMsBuckets], first[kMsBuckets], nsl[kMsBuckets];
  const int tid = threadIdx.x;
  ms_slices(btot, start, first, nsl, tid);
  const uint32_t id = blockIdx.x * (uint32_t)kMsBuckets + (uint32_t)tid;
  if (id >= (uint32_t)c) return;
  const size_t per = (size_t)kMsBuckets * (size_t)(v + 1);
  const uint32_t* __restrict__ base = P + (size_t)first[blockIdx.x] * per + tid;
  const uint32_t ns = nsl[blockIdx.x];
  uint32_t acc[33];
#pragma unroll
  for (int t = 0; t < 33; ++t) acc[t] = 0u;
  for (uint32_t j = 0; j < ns; ++j) {  // rows past v re-read row v (no branch, so no wait per load)
    const uint32_t* __restrict__ src = base + (size_t)j * per;
#pragma unroll
    for (int t = 0; t < 33; ++t) acc[t] += src[(t < v ? t : v) * kMsBuckets];
  }
  uint32_t n = 0u;
#pragma unroll
  for (int t = 0; t < 33; ++t) n = t == v ? acc[t] : n;
  if (counts) counts[id] = n;
  if (n == 0u) return;
  uint32_t w = 0u;
#pragma unroll
  for (int t = 0; t < 32; ++t)
    if (t < v) w |= (2ull * acc[t] >= n ? 1u : 0u) << t;
  codebook[id] = w;
}

// slices the vote may need: floor(total / kMsSlice) full ones plus at most one partial slice per
// non-empty bucket (buckets at or past ceil(c / 256) are empty)
int64_t ms_max_slices(int64_t total, int c) {
  const int64_t nbk = ((int64_t)c + kMsBuckets - 1) / kMsBuckets;
  return total / kMsSlice + (nbk < total ? nbk : total);
}

// words before the slice tables: the records' patterns (one word each) and index bytes, chunk
// histograms, bucket totals, rounded up to 64
int64_t ms_head_words(int64_t total) {
  const int64_t nchunk = (total + kMsChunk - 1) / kMsChunk;
  return (total + (total + 3) / 4 + (int64_t)kMsBuckets * nchunk + kMsBuckets + 63) & ~(int64_t)63;
}

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

// distinct count: a flag byte per possible pattern, then the bitmap of the 2^v patterns (bit p
// set when pattern p occurs), then its count and list
constexpr int kMarkPerThread = 4;  // blocks per thread, their loads in flight together

// map[p] = 1 for every pattern p that occurs: plain byte stores, no atomics (every writer of a
// byte stores the same value, and the per-XCD caches merge their dirty bytes when written back)
__global__ __launch_bounds__(256) void distinct_mark_kernel(const uint32_t* __restrict__ plane, int64_t ldp,
                                                            int64_t K, int v, int64_t total,
                                                            uint8_t* __restrict__ map) {
  const uint32_t nb = (uint32_t)((K + v - 1) / v);  // blocks per row; total < 2^32
  const int64_t Kw = (K + 31) >> 5;
  uint32_t lo[kMarkPerThread], hi[kMarkPerThread];
  int64_t col[kMarkPerThread];
  bool ok[kMarkPerThread];
#pragma unroll
  for (int u = 0; u < kMarkPerThread; ++u) {  // loads at clamped addresses, unconditionally
    const int64_t e64 = ((int64_t)blockIdx.x * kMarkPerThread + u) * 256 + threadIdx.x;
    ok[u] = e64 < total;
    const uint32_t e = ok[u] ? (uint32_t)e64 : (uint32_t)(total - 1);
    const uint32_t n = e / nb;
    col[u] = (int64_t)(e - n * nb) * v;
    load_block_words(plane + (int64_t)n * ldp, col[u], Kw, lo[u], hi[u]);
  }
#pragma unroll
  for (int u = 0; u < kMarkPerThread; ++u)
    if (ok[u]) map[block_from_words(lo[u], hi[u], col[u], K, Kw, v)] = 1u;
}

// bitmap word w = the flags map[32 w .. 32 w + 31] as bits (npat = 2^v flags)
__global__ __launch_bounds__(256) void distinct_pack_kernel(const uint8_t* __restrict__ map, int64_t npat,
                                                            int64_t nwords, uint32_t* __restrict__ bitmap) {
  const int64_t w = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (w >= nwords) return;
  uint32_t word = 0u;
  if (npat >= 32) {  // 32 whole flags, eight 4-byte loads (the workspace is 4-byte aligned)
    const uint32_t* src = reinterpret_cast<const uint32_t*>(map + w * 32);
    uint32_t part[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) part[i] = src[i];
#pragma unroll
    for (int i = 0; i < 8; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j) word |= (((part[i] >> (8 * j)) & 0xffu) != 0u ? 1u : 0u) << (4 * i + j);
  } else {
    for (int64_t i = 0; i < npat; ++i) word |= (map[i] != 0u ? 1u : 0u) << i;
  }
  bitmap[w] = word;
}

constexpr int kDistinctThreads = 1024;

// One block: M = number of set bits -> *n_distinct. If M < c, the patterns in ascending order
// go to codebook[0..M) and codebook[M..c) repeats the largest one. Thread t owns a contiguous
// range of bitmap words; its first output position is the exclusive scan of the ranges' counts.
// one block on the whole chip: registers for a batch of loads matter more than occupancy
__global__ __launch_bounds__(kDistinctThreads) __attribute__((amdgpu_waves_per_eu(4, 4))) void distinct_compact_kernel(const uint32_t* __restrict__ bitmap,
                                                                            int64_t nwords, int c,
                                                                            uint32_t* __restrict__ codebook,
                                                                            int32_t* __restrict__ n_distinct) {
  __shared__ uint32_t scan[2][kDistinctThreads];
  __shared__ int32_t top;
  __shared__ uint32_t count;
  const int t = threadIdx.x;
  constexpr int kB = 8;  // words per batch, loaded together at clamped addresses
  // the count alone first, with coalesced reads (thread t takes words t, t + 1024, ...): when it
  // reaches c, nothing is listed
  {
    uint32_t n = 0u;
    for (int64_t w0 = t; w0 < nwords; w0 += (int64_t)kDistinctThreads * kB) {
      uint32_t b[kB];
#pragma unroll
      for (int u = 0; u < kB; ++u) {
        const int64_t w = w0 + (int64_t)u * kDistinctThreads;
        b[u] = bitmap[w < nwords ? w : nwords - 1];
      }
#pragma unroll
      for (int u = 0; u < kB; ++u) n += w0 + (int64_t)u * kDistinctThreads < nwords ? (uint32_t)__popc(b[u]) : 0u;
    }
    if (t == 0) count = 0u;
    __syncthreads();
    atomicAdd(&count, n);
    __syncthreads();
    if (count >= (uint32_t)c) {  // the whole block leaves here
      if (t == 0) *n_distinct = (int32_t)count;
      return;
    }
  }
  // fewer than c: thread t owns a contiguous range of words, listed in ascending order
  const int64_t per = (nwords + kDistinctThreads - 1) / kDistinctThreads;
  const int64_t lo = (int64_t)t * per < nwords ? (int64_t)t * per : nwords;
  const int64_t hi = lo + per < nwords ? lo + per : nwords;
  uint32_t mine = 0u;
  int32_t last = -1;
  for (int64_t w0 = lo; w0 < hi; w0 += kB) {
    uint32_t b[kB];
#pragma unroll
    for (int u = 0; u < kB; ++u) b[u] = bitmap[w0 + u < hi ? w0 + u : hi - 1];
#pragma unroll
    for (int u = 0; u < kB; ++u) {  // selects, no branches: the loads stay ahead of their uses
      const uint32_t bu = w0 + u < hi ? b[u] : 0u;
      mine += (uint32_t)__popc(bu);
      last = bu ? (int32_t)((w0 + u) * 32 + 31 - __builtin_clz(bu)) : last;
    }
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

// ---------------------------------------------------------------------------------------------
// Nearest-codeword table (v <= 24): the encode result of every one of the 2^v patterns, found by
// a breadth-first search over the hypercube from all codewords at once.
//   layer 0      T[C[i]] = (0, the lowest i holding that codeword)
//   layer d + 1  a pattern p not reached yet, with neighbours q = p ^ (1 << t) at distance d,
//                gets (d + 1, the lowest index among those neighbours' entries)
// Why that is the brute-force answer (nearest in Hamming distance, ties to the lowest index):
// if p's nearest codewords lie at distance d + 1, each of them lies at distance d from some
// neighbour q of p (one step along a shortest path), no neighbour is nearer than d to the
// codebook, so those q sit exactly at distance d, and every nearest codeword of such a q is a
// nearest codeword of p. The minimum of the neighbours' indices is therefore the lowest index
// among p's nearest codewords. Entries are (distance << 24) | index, 0xffffffff = not reached; a
// layer reads only entries of distance d and writes only distance d + 1, so no launch reads what
// it writes. flag[d] is nonzero when some pattern has distance d: once a layer reaches nothing,
// every pattern has been reached (the hypercube is connected) and the later layers return at once.
// ---------------------------------------------------------------------------------------------
constexpr uint32_t kTableUnreached = 0xffffffffu;
constexpr int kTableMaxV = 24;

__global__ __launch_bounds__(256) void table_seed_kernel(const uint32_t* __restrict__ codebook, int c, int v,
                                                         uint32_t* __restrict__ table, uint32_t* __restrict__ flag) {
  const uint32_t mask = (1u << v) - 1u;
  for (int i = blockIdx.x * 256 + threadIdx.x; i < c; i += gridDim.x * 256)
    atomicMin(&table[codebook[i] & mask], (uint32_t)i);  // distance 0; codewords hold v bits
  if (blockIdx.x == 0 && threadIdx.x == 0) flag[0] = 1u;
}

// VMAX >= v, a multiple of 4: the neighbour loop's unrolled length
template <int VMAX>
__global__ __launch_bounds__(256) void table_layer_kernel(uint32_t* __restrict__ table, int v, int d,
                                                          uint32_t* __restrict__ flag) {
  if (flag[d] == 0u) return;  // nothing at distance d: everything is reached
  __shared__ int any;
  if (threadIdx.x == 0) any = 0;
  __syncthreads();
  const uint32_t p = blockIdx.x * 256u + threadIdx.x;  // the grid covers the 2^v patterns (more when v < 8)
  if (p < (1u << v) && table[p] == kTableUnreached) {
    uint32_t e[VMAX];
#pragma unroll
    for (int t = 0; t < VMAX; ++t)  // all neighbours' loads in flight; bits past v re-read bit v - 1
      e[t] = table[p ^ (1u << (t < v ? t : v - 1))];
    uint32_t best = kTableUnreached;
#pragma unroll
    for (int t = 0; t < VMAX; ++t)
      if ((e[t] >> 24) == (uint32_t)d) best = (e[t] & 0xffffffu) < best ? (e[t] & 0xffffffu) : best;
    if (best != kTableUnreached) {
      table[p] = ((uint32_t)(d + 1) << 24) | best;
      any = 1;
    }
  }
  __syncthreads();
  if (threadIdx.x == 0 && any) flag[d + 1] = 1u;
}

// encode by lookup: the same blocks as encode_kernel, the same answer; kEncPerThread blocks per
// thread, each stage's loads in flight together
constexpr int kEncPerThread = 4;

__global__ __launch_bounds__(256) void encode_table_kernel(const uint32_t* __restrict__ plane, int64_t ldp, int64_t K,
                                                           int v, int64_t total, const uint32_t* __restrict__ table,
                                                           uint16_t* __restrict__ idx) {
  const uint32_t nb = (uint32_t)((K + v - 1) / v);  // blocks per row; total < 2^32
  const int64_t Kw = (K + 31) >> 5;
  uint32_t lo[kEncPerThread], hi[kEncPerThread], ent[kEncPerThread];
  int64_t col[kEncPerThread], e[kEncPerThread];
#pragma unroll
  for (int u = 0; u < kEncPerThread; ++u) {
    e[u] = ((int64_t)blockIdx.x * kEncPerThread + u) * 256 + threadIdx.x;
    const uint32_t ec = e[u] < total ? (uint32_t)e[u] : (uint32_t)(total - 1);
    const uint32_t n = ec / nb;
    col[u] = (int64_t)(ec - n * nb) * v;
    load_block_words(plane + (int64_t)n * ldp, col[u], Kw, lo[u], hi[u]);
  }
#pragma unroll
  for (int u = 0; u < kEncPerThread; ++u) ent[u] = table[block_from_words(lo[u], hi[u], col[u], K, Kw, v)];
#pragma unroll
  for (int u = 0; u < kEncPerThread; ++u)
    if (e[u] < total) idx[e[u]] = (uint16_t)(ent[u] & 0xffffu);
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

// workspace, used by one step at a time: the standalone M-step's records (a pattern word and an
// index byte per block), chunk histograms (256 per 8192 blocks), bucket totals (256) and slice counts (256 (v + 1)
// words per slice of 4096 members); the learning loop's
// counters [c][v + 1]; the 2^v-byte map (rounded up to 16 bytes) and 2^v-bit bitmap of the
// distinct count
size_t codebook_learn_workspace_bytes(int64_t N, int64_t K, int c, int v) {
  const size_t blocks = (size_t)N * (size_t)((K + v - 1) / v);
  const size_t mstep = 4u * ((size_t)ms_head_words((int64_t)blocks) +
                             (size_t)ms_max_slices((int64_t)blocks, c) * kMsBuckets * (size_t)(v + 1));
  const size_t counters = 4u * (size_t)c * (size_t)(v + 1);
  const size_t bitmap = v <= 24 ? ((((size_t)1 << v) + 15u) & ~(size_t)15) + ((size_t)1 << (v > 5 ? v - 3 : 2)) : 0u;
  const size_t table = codebook_use_table(N, K, c, v) ? codebook_table_bytes(v) : 0u;
  size_t m = mstep > counters ? mstep : counters;
  m = m > table ? m : table;
  return m > bitmap ? m : bitmap;
}

hipError_t launch_codebook_mstep(const uint32_t* plane, int64_t ldp, int64_t N, int64_t K, int v,
                                 const uint16_t* idx, uint32_t* codebook, int c, uint32_t* counts, void* ws,
                                 hipStream_t s) {
  const int64_t total = N * ((K + v - 1) / v);
  const int64_t nchunk = (total + kMsChunk - 1) / kMsChunk;
  if (total <= 0) return hipSuccess;
  if (total > 0xffffffffLL) return hipErrorInvalidValue;  // block positions are 32-bit words
  uint32_t* Rp = static_cast<uint32_t*>(ws);
  uint8_t* Rb = reinterpret_cast<uint8_t*>(Rp + total);
  uint32_t* H = Rp + total + (total + 3) / 4;
  uint32_t* btot = H + (int64_t)kMsBuckets * nchunk;
  uint32_t* P = Rp + ms_head_words(total);
  mstep_hist_kernel<<<(unsigned)nchunk, kMsThreads, 0, s>>>(idx, total, c, nchunk, H);
  mstep_scan_kernel<<<kMsBuckets, kMsThreads, 0, s>>>(H, nchunk, btot);
  mstep_scatter_kernel<<<(unsigned)nchunk, kMsThreads, 0, s>>>(plane, ldp, K, v, idx, total, c, nchunk, H, btot, Rp,
                                                               Rb);
  mstep_vote_kernel<<<(unsigned)ms_max_slices(total, c), kMsVoteThreads, 0, s>>>(v, Rp, Rb, btot, P);
  mstep_finish_kernel<<<(unsigned)((c + kMsBuckets - 1) / kMsBuckets), kMsBuckets, 0, s>>>(P, btot, v, c, codebook,
                                                                                           counts);
  return hipGetLastError();
}

hipError_t launch_codebook_distinct(const uint32_t* plane, int64_t ldp, int64_t N, int64_t K, int v,
                                    uint32_t* codebook, int c, int32_t* n_distinct, void* ws, hipStream_t s) {
  // workspace: the 2^v-byte map (rounded up to 16 bytes), then the 2^v-bit bitmap
  const int64_t npat = (int64_t)1 << v;
  const int64_t nwords = v > 5 ? (int64_t)1 << (v - 5) : 1;
  uint8_t* map = static_cast<uint8_t*>(ws);
  uint32_t* bitmap = reinterpret_cast<uint32_t*>(map + ((npat + 15) & ~(int64_t)15));
  const int64_t total = N * ((K + v - 1) / v);
  if (total > 0xffffffffLL) return hipErrorInvalidValue;  // block positions are 32-bit
  fill_u32_kernel<<<stride_grid((npat + 3) / 4), 256, 0, s>>>(reinterpret_cast<uint32_t*>(map), (npat + 3) / 4, 0u);
  if (total > 0) {
    const int64_t grid = (total + 256 * kMarkPerThread - 1) / (256 * kMarkPerThread);
    distinct_mark_kernel<<<(unsigned)grid, 256, 0, s>>>(plane, ldp, K, v, total, map);
  }
  distinct_pack_kernel<<<(unsigned)((nwords + 255) / 256), 256, 0, s>>>(map, npat, nwords, bitmap);
  distinct_compact_kernel<<<1, kDistinctThreads, 0, s>>>(bitmap, nwords, c, codebook, n_distinct);
  return hipGetLastError();
}

// the table and the layer flags (one word per possible distance 0..v, 32 of them)
size_t codebook_table_bytes(int v) { return v >= 1 && v <= kTableMaxV ? ((size_t)4 << v) + 128u : 0u; }

hipError_t launch_codebook_table(const uint32_t* codebook, int c, int v, void* ws, hipStream_t s) {
  uint32_t* table = static_cast<uint32_t*>(ws);
  const int64_t np = (int64_t)1 << v;
  uint32_t* flag = table + np;
  fill_u32_kernel<<<stride_grid(np), 256, 0, s>>>(table, np, kTableUnreached);
  fill_u32_kernel<<<1, 256, 0, s>>>(flag, 32, 0u);
  table_seed_kernel<<<(unsigned)((c + 255) / 256 < 1024 ? (c + 255) / 256 : 1024), 256, 0, s>>>(codebook, c, v, table,
                                                                                                 flag);
  const unsigned grid = (unsigned)((np + 255) / 256);
  auto layers = [&](auto vmax) {
    for (int d = 0; d < v; ++d) table_layer_kernel<decltype(vmax)::value><<<grid, 256, 0, s>>>(table, v, d, flag);
  };
  switch ((v + 3) / 4) {
    case 1: layers(std::integral_constant<int, 4>{}); break;
    case 2: layers(std::integral_constant<int, 8>{}); break;
    case 3: layers(std::integral_constant<int, 12>{}); break;
    case 4: layers(std::integral_constant<int, 16>{}); break;
    case 5: layers(std::integral_constant<int, 20>{}); break;
    default: layers(std::integral_constant<int, kTableMaxV>{}); break;
  }
  return hipGetLastError();
}

hipError_t launch_codebook_encode_table(const uint32_t* plane, int64_t ldp, int64_t N, int64_t K,
                                        const uint32_t* codebook, int c, int v, uint16_t* idx, void* ws,
                                        hipStream_t s) {
  const hipError_t e = launch_codebook_table(codebook, c, v, ws, s);
  if (e != hipSuccess) return e;
  const int64_t total = N * ((K + v - 1) / v);
  if (total > 0xffffffffLL) return hipErrorInvalidValue;  // block positions are 32-bit
  if (total > 0)
    encode_table_kernel<<<(unsigned)((total + 256 * kEncPerThread - 1) / (256 * kEncPerThread)), 256, 0, s>>>(
        plane, ldp, K, v, total, static_cast<const uint32_t*>(ws), idx);
  return hipGetLastError();
}

// The table pays when the brute-force search would score many more (pattern, codeword) pairs
// than the table's search visits entries (about 2^v times the few layers that do work).
bool codebook_use_table(int64_t N, int64_t K, int c, int v) {
  if (v < 1 || v > kTableMaxV) return false;
  const double pairs = (double)N * (double)((K + v - 1) / v) * (double)c;
  return pairs > 64.0 * (double)((int64_t)1 << v);
}

hipError_t launch_codebook_learn(const uint32_t* plane, int64_t ldp, int64_t N, int64_t K, int v,
                                 uint32_t* codebook, int c, int iters, uint16_t* idx, int32_t* n_distinct,
                                 void* ws, hipStream_t s) {
  hipError_t e = launch_codebook_distinct(plane, ldp, N, K, v, codebook, c, n_distinct, ws, s);
  if (codebook_use_table(N, K, c, v)) {
    // each iteration: the table of the current codebook, the lookups, then the counting-sort
    // M-step (the workspace holds one of them at a time)
    for (int it = 0; it < iters && e == hipSuccess; ++it) {
      e = launch_codebook_encode_table(plane, ldp, N, K, codebook, c, v, idx, ws, s);
      if (e == hipSuccess) e = launch_codebook_mstep(plane, ldp, N, K, v, idx, codebook, c, nullptr, ws, s);
    }
    if (e == hipSuccess) e = launch_codebook_encode_table(plane, ldp, N, K, codebook, c, v, idx, ws, s);
    return e;
  }
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
