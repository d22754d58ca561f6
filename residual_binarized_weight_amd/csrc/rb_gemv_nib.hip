// rb_gemv_nib.hip -- whole-row nibble-table product for one activation row (gfx950).
//
// [RaBiT summary page, background "Residual binarization"] y = sum_i g_i (.) (B_i x): the k
// paths need only additions and one scale per row and plane. With h = 1 every plane is
// multiplied by the same x, so one set of precomputed partial sums of x serves all of them
// (the idea the BTC-LLM page's LUT-GEMM describes in 2.1.2).
//
// Tables: for each run of 4 columns ("nibble" q), T_q[e] = sum of the x_c whose bit is set
// in the 4-bit pattern e (T_q[0] = 0). Per row and plane, Sum_c B x = 2 T - S with
// T = sum over nibbles of T_q[bits] and S = sum of x (the masked-add identity), so
//   y[n] = sum_i g_i[n] * (2 T_i[n] - S).
// 16 entries per 4 columns is 4 table bytes per column, so the tables of a whole row pass
// through LDS in a few double-buffered phases of 4096 columns (up to four: K <= 16384) and a
// block can own complete rows: no cross-block reduction, deterministic, no workspace.
//
// Layout: entry e of all tables of a phase is one 4 KB row of LDS (entry-major);
// nibble i of word w sits in slot 8 w + (i ^ a(w)), a(w) = ((w >> 2) ^ ((w >> 5) & 1)) & 7.
// Lane l of a wave reads word 64 j + l, so for a fixed i the lanes of each 32-lane half
// land in 32 different banks of a 32-bank LDS (lanes that share w mod 4 differ in a), and
// the 64 lanes in 64 different banks of a 64-bank one, whatever the bit values. A lookup
// address is (e << 12) | (32 l + 4 (i ^ a_l)), plus the immediate 2048 j (a does not
// depend on j); it is assembled by one byte permute per nibble (see the lookups).
//
// A block is 16 waves with RW rows each. Instantiated for fp16 activations, scales and
// outputs and k <= 2 (the byte-table kernel in rb_gemv.hip covers the other cases).
#include "rb_device.hpp"
#include "rb_internal.h"

namespace rb {
namespace {

constexpr int kNibWaves = 16;  // waves per block, RW rows each (8 measured slower: fewer waves keep LDS less busy)
constexpr int kNibB0Waves = 8;  // waves that build the first phase's tables
constexpr uint32_t kNibOob = 0x80000000u;  // an offset past every resource below

typedef uint32_t nib_u32x2 __attribute__((ext_vector_type(2)));

// 4 activations of nibble q (columns 4q .. 4q+3), in raw form; columns >= K become 0 later
template <typename TX> struct NibX;
template <> struct NibX<__half> {
  using raw = nib_u32x2;
  __device__ static __forceinline__ raw load(__amdgpu_buffer_rsrc_t r, uint32_t off) {
    return __builtin_bit_cast(raw, __builtin_amdgcn_raw_buffer_load_b64(r, (int)off, 0, 0));
  }
  static constexpr uint32_t bytes = 8;
  __device__ static __forceinline__ float get(raw v, int j) {
    return __half2float(__ushort_as_half((uint16_t)((v[j >> 1] >> (16 * (j & 1))) & 0xffffu)));
  }
};

template <typename TS> struct NibScale;
template <> struct NibScale<__half> {
  __device__ static __forceinline__ uint32_t load(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff) {
    return buf_u16(r, voff, soff);
  }
  __device__ static __forceinline__ float f32(uint32_t v) { return __half2float(__ushort_as_half((uint16_t)v)); }
};

template <typename T> __device__ __forceinline__ void nib_store(T* p, float v);
template <> __device__ __forceinline__ void nib_store<__half>(__half* p, float v) { *p = __float2half_rn(v); }

// Phases of 128 words (4096 columns): 16 entry rows of 4 KB = 64 KB of tables, two buffers
// (buffer b at byte 65536 b). Phase p + 1 is built while phase p is looked up.
constexpr int kNibPhaseWords = 128;
constexpr int kNibTables = 8 * kNibPhaseWords;  // 1024 nibble tables per phase: one per thread
constexpr int kNibSH = 12;                      // entry row = 4 KB
constexpr uint32_t kNibBuf = 65536u;

// WV waves per block, RW rows per wave (row r of wave w of block b: (b * WV + w) * RW + r)
// VAR: the product variants, compiled separately so that none costs the others registers:
// bit 0 reads the plane bits as {0, 1}, bit 1 adds a row offset, bit 2 (one plane per pass)
// multiplies the activations by that plane's column scales h before the tables are built and
// chains the passes of k planes through an fp32 row sum: acc_mode bit 0 adds the sum of the
// passes before (acc_io[n]), bit 1 writes the sum for the next pass instead of y (the last
// pass zeroes acc_io[n] after reading it); bit 3 (with bit 2 and KP = 2) runs both planes in
// one pass instead, plane 0's phases and then plane 1's, each phase's tables built from x times
// the column scales of its plane (two sums S, no chaining); 0 is the plain product.
template <typename TX, typename TS, typename TY, int KP, int NPH, int RW, int WV, int VAR>
__global__ __launch_bounds__(64 * WV) __attribute__((amdgpu_waves_per_eu(1, 4))) void gemv_nib_kernel(
    const uint32_t* __restrict__ planes, int64_t ldp, const TS* __restrict__ g, int64_t N, int64_t K,
    const TX* __restrict__ x, TY* __restrict__ y, const TS* __restrict__ mu, int zero_one,
    const TX* __restrict__ hrow, float* __restrict__ acc_io, int acc_mode) {
  extern __shared__ __align__(16) uint8_t lds[];
  constexpr bool kSeq = (VAR & 8) != 0;
  static_assert(!kSeq || (KP == 2 && (VAR & 4) != 0), "planes in sequence: two planes with column scales");
  constexpr int NV = kSeq ? 2 * NPH : NPH;  // phases run (plane 1's after plane 0's)
  float* red = reinterpret_cast<float*>(lds + (NV == 1 ? 1 : 2) * kNibBuf);  // after the table buffers
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  constexpr int kThreads = 64 * WV;
  static_assert(kThreads == kNibTables, "one table per thread from phase 1 on");
  // phase 0 is built by the first kNibB0Waves waves alone, kTB0 tables per thread
  constexpr int kB0Threads = 64 * kNibB0Waves;
  constexpr int kTB0 = kNibTables / kB0Threads;
  const bool b0 = wave < kNibB0Waves;  // wave-uniform
  const int64_t n0 = ((int64_t)blockIdx.x * WV + wave) * RW;
  const uint32_t Kw = (uint32_t)((K + 31) >> 5);
  const uint32_t Kc = (uint32_t)K;
  const uint32_t ldp_b = (uint32_t)ldp * 4u;

  // the row offsets (if any): a wave's row is uniform, so each is one scalar-cache load of the
  // aligned dword holding it, issued first; it does not wait behind the vector loads, and its
  // raw bits stay in scalar registers until the epilogue. The aligned dword never reaches a page
  // the offset array does not touch (its half-word neighbour is the array's or inside the same
  // 4-byte unit), so the load cannot fault.
  uint32_t mr[RW];
  if constexpr ((VAR & 2) != 0) {
    typedef __attribute__((address_space(4))) const uint32_t nib_const_u32;
#pragma unroll
    for (int r = 0; r < RW; ++r) {
      const int64_t row = n0 + r < N ? n0 + r : N - 1;
      const uintptr_t a = reinterpret_cast<uintptr_t>(mu) + 2u * (uintptr_t)row;
      const uint32_t w = *reinterpret_cast<nib_const_u32*>(a & ~(uintptr_t)3);
      mr[r] = (a & 2u) ? (w >> 16) : (w & 0xffffu);
    }
  }

  // plane words and scales through 32-bit offsets (the host checks k N ldp * 4 < 2^31), x
  // through whole dwords (a column past K inside the last one is masked); past the end: 0
  const __amdgpu_buffer_rsrc_t rp = buffer_rsrc(planes, (uint32_t)((uint64_t)KP * N * ldp * 4));
  const __amdgpu_buffer_rsrc_t rg = buffer_rsrc(g, (uint32_t)((uint64_t)KP * N * sizeof(TS)));
  const __amdgpu_buffer_rsrc_t rx = buffer_rsrc(x, (uint32_t)((uint64_t)((K * sizeof(TX) + 3) & ~3ull)));

  // 1. the activations of this thread's tables: phase 0's nibbles b * kB0Threads + tid in the
  // first waves (issued before anything else), then nibble tid of every later phase
  typename NibX<TX>::raw x0[kTB0];
  typename NibX<TX>::raw xr[NPH];
  if (b0) {
#pragma unroll
    for (int b = 0; b < kTB0; ++b)
      x0[b] = NibX<TX>::load(rx, (uint32_t)(b * kB0Threads + tid) * NibX<TX>::bytes);
  }
#pragma unroll
  for (int p = 1; p < NPH; ++p) xr[p] = NibX<TX>::load(rx, (uint32_t)(p * kNibTables + tid) * NibX<TX>::bytes);
  // h mode: this plane's column scales, in the same pattern as the activations
  typename NibX<TX>::raw h0[kTB0];
  typename NibX<TX>::raw hr[NPH];
  typename NibX<TX>::raw h10[kTB0];  // planes in sequence: plane 1's column scales (else unused)
  typename NibX<TX>::raw h1r[NPH];
  if constexpr ((VAR & 4) != 0) {
    const __amdgpu_buffer_rsrc_t rh = buffer_rsrc(hrow, (uint32_t)((uint64_t)((K * sizeof(TX) + 3) & ~3ull)));
    if (b0) {
#pragma unroll
      for (int b = 0; b < kTB0; ++b)
        h0[b] = NibX<TX>::load(rh, (uint32_t)(b * kB0Threads + tid) * NibX<TX>::bytes);
    }
#pragma unroll
    for (int p = 1; p < NPH; ++p) hr[p] = NibX<TX>::load(rh, (uint32_t)(p * kNibTables + tid) * NibX<TX>::bytes);
    if constexpr (kSeq) {
      const __amdgpu_buffer_rsrc_t rh1 =
          buffer_rsrc(hrow + K, (uint32_t)((uint64_t)((K * sizeof(TX) + 3) & ~3ull)));
      if (b0) {
#pragma unroll
        for (int b = 0; b < kTB0; ++b)
          h10[b] = NibX<TX>::load(rh1, (uint32_t)(b * kB0Threads + tid) * NibX<TX>::bytes);
      }
#pragma unroll
      for (int p = 1; p < NPH; ++p)
        h1r[p] = NibX<TX>::load(rh1, (uint32_t)(p * kNibTables + tid) * NibX<TX>::bytes);
    }
  }
  // activations first, in every wave: requests return in order, and the table build must not
  // queue behind the weight stream
  __builtin_amdgcn_sched_barrier(0);
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_sched_barrier(0);

  // 2. this wave's rows' plane words (lane l: words 128 p + l and 128 p + 64 + l) and scales
  uint32_t wd[RW][NPH][2][KP];
#pragma unroll
  for (int r = 0; r < RW; ++r) {
    const uint32_t row_off = (uint32_t)(n0 + r) * ldp_b;
#pragma unroll
    for (int p = 0; p < NPH; ++p)
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const uint32_t w = (uint32_t)(kNibPhaseWords * p + 64 * j + lane);
        const uint32_t voff = w < Kw ? row_off + 4u * w : kNibOob;
#pragma unroll
        for (int i = 0; i < KP; ++i) wd[r][p][j][i] = buf_u32(rp, voff, (uint32_t)i * (uint32_t)N * ldp_b);
      }
  }
  uint32_t gr[RW][KP];
#pragma unroll
  for (int r = 0; r < RW; ++r)
#pragma unroll
    for (int i = 0; i < KP; ++i)
      gr[r][i] = NibScale<TS>::load(rg, (uint32_t)(n0 + r) * (uint32_t)sizeof(TS),
                                    (uint32_t)i * (uint32_t)N * (uint32_t)sizeof(TS));
  __builtin_amdgcn_sched_barrier(0);

  // Lookup addresses by byte splicing. Lane l's slot offset 32 l + 4 (i ^ a(l)) is
  // 256 (l >> 3) + [32 (l & 7) + 4 (i ^ a(l))]: its low byte depends on i, its bits 8-10 are
  // l >> 3. The address (e << 12) | offset | 65536 buffer therefore has byte 0 = the low byte,
  // byte 1 = (e << 4) | (l >> 3), byte 2 = the buffer. Per word, nibble e of each byte's high
  // half OR (l >> 3) gives every nibble's byte 1 (two words: odd nibbles w & 0xf0f0f0f0, even
  // ones (w << 4) & 0xf0f0f0f0), and one v_perm per nibble joins it with cb[buffer][i] (bytes
  // 0 and 2): 11 operations per word instead of 15.
  uint32_t cb[2][8];
  const int al = ((lane >> 2) ^ ((lane >> 5) & 1)) & 7;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    cb[0][i] = 32u * (uint32_t)(lane & 7) + 4u * (uint32_t)(i ^ al);
    cb[1][i] = cb[0][i] | kNibBuf;
  }
  const uint32_t lh4 = (uint32_t)(lane >> 3) * 0x01010101u;

  float xs = 0.0f;  // this thread's share of sum x (of the current plane's x h in sequence)
  // table q of phase p (run as phase vp) into buffer vp % 2, from the 4 activations in `raw`
  auto build_one = [&](int vp, int p, uint32_t q, typename NibX<TX>::raw raw, typename NibX<TX>::raw hraw) {
    typedef __attribute__((address_space(3))) float lds_f32p;
    const uint32_t Q = (uint32_t)(p * kNibTables) + q;
    float xv[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      float v = NibX<TX>::get(raw, j);
      if constexpr ((VAR & 4) != 0) v *= NibX<TX>::get(hraw, j);  // exact: fp16 x fp16 fits fp32
      xv[j] = 4u * Q + (uint32_t)j < Kc ? v : 0.0f;
    }
    xs += (xv[0] + xv[1]) + (xv[2] + xv[3]);
    const uint32_t w = q >> 3, i = q & 7;
    const uint32_t slot = 8u * w + (i ^ (((w >> 2) ^ ((w >> 5) & 1u)) & 7u));
    const uint32_t base = (uint32_t)(vp & 1) * kNibBuf + slot * 4u;
    const float lo[4] = {0.0f, xv[0], xv[1], xv[0] + xv[1]};
    const float hi[4] = {0.0f, xv[2], xv[3], xv[2] + xv[3]};
    // entry 0 is 0 for every table: written by each buffer's first build only. Tables wholly
    // past K are read only at entry 0 (their words are 0), so they need no other entry.
    if (vp < 2) *(lds_f32p*)(size_t)base = 0.0f;
    if (4u * Q < Kc) {
#pragma unroll
      for (int e = 1; e < 16; ++e) {
        const float v = (e & 3) == 0 ? hi[e >> 2] : ((e >> 2) == 0 ? lo[e & 3] : lo[e & 3] + hi[e >> 2]);
        *(lds_f32p*)(size_t)(((uint32_t)e << kNibSH) + base) = v;
      }
    }
  };
  // phase p's tables: phase 0 by the first waves (their activations arrive first: the
  // memory returns to a block's waves in launch order), later phases one per thread
  auto build = [&](int vp) {
    const int p = kSeq ? vp % NPH : vp;
    const bool second = kSeq && vp >= NPH;  // plane 1's phase
    if (p == 0) {
      if (b0) {
#pragma unroll
        for (int b = 0; b < kTB0; ++b) {
          typename NibX<TX>::raw hb = h0[b];
          if constexpr (kSeq) hb = second ? h10[b] : hb;
          build_one(vp, 0, (uint32_t)(b * kB0Threads + tid), x0[b], hb);
        }
      }
    } else {
      typename NibX<TX>::raw hp = hr[p];
      if constexpr (kSeq) hp = second ? h1r[p] : hp;
      build_one(vp, p, (uint32_t)tid, xr[p], hp);
    }
    if (p == NPH - 1) {
      // every column has been seen: publish this wave's share of sum x (a barrier follows)
      const float xw = wave_sum_dpp(xs);
      if (lane == 63) red[(second ? WV : 0) + wave] = xw;
      if constexpr (kSeq) xs = 0.0f;
    }
  };

  float acc[RW][KP];
#pragma unroll
  for (int r = 0; r < RW; ++r)
#pragma unroll
    for (int i = 0; i < KP; ++i) acc[r][i] = 0.0f;

  build(0);
  __builtin_amdgcn_sched_barrier(0);
  __syncthreads();
  __builtin_amdgcn_sched_barrier(0);
#pragma unroll
  for (int vp = 0; vp < NV; ++vp) {
    const int p = kSeq ? vp % NPH : vp;
    // 3. the next phase's tables (activations only: no wait on the weight stream)
    if (vp + 1 < NV) build(vp + 1);
    __builtin_amdgcn_sched_barrier(0);
    // 4. lookups in this phase's buffer: one LDS read per 4 weight bits. A lane past the row's
    // last word holds 0 (its load was out of range) and reads entry 0, which is 0 in every
    // table; only a group of 64 words wholly past it is skipped (a wave-uniform test: a
    // per-lane one would put the reads under exec masks and wait for them inside)
#pragma unroll
    for (int r = 0; r < RW; ++r)
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        if (p == NPH - 1 && (uint32_t)(kNibPhaseWords * p + 64 * j) >= Kw) continue;
#pragma unroll
        for (int i = 0; i < KP; ++i) {
          if (kSeq && i != vp / NPH) continue;  // in sequence: this phase's plane only
          const uint32_t w = wd[r][p][j][i];
          const uint32_t o = 2048u * (uint32_t)j;
          const uint32_t* c = cb[vp & 1];
          const uint32_t ev = ((w << 4) & 0xf0f0f0f0u) | lh4;  // byte m: nibble 2 m
          const uint32_t od = (w & 0xf0f0f0f0u) | lh4;         // byte m: nibble 2 m + 1
          // selector: byte 0 <- c byte 0, byte 1 <- word byte m, byte 2 <- c byte 2, byte 3 <- 0
          auto at = [&](uint32_t src, uint32_t ci, uint32_t m) {
            return lds_f32(__builtin_amdgcn_perm(src, ci, 0x0c020000u | ((4u + m) << 8)) + o);
          };
          float t = (at(ev, c[0], 0) + at(od, c[1], 0)) + (at(ev, c[2], 1) + at(od, c[3], 1));
          t += (at(ev, c[4], 2) + at(od, c[5], 2)) + (at(ev, c[6], 3) + at(od, c[7], 3));
          acc[r][i] += t;
        }
      }
    // the next phase's tables are complete, and this phase's buffer is free for phase p + 2
    if (vp + 1 < NV) {
      __builtin_amdgcn_sched_barrier(0);
      __syncthreads();
      __builtin_amdgcn_sched_barrier(0);
    }
  }

  // 5. row sums; sum x over the block, read in the same order by every wave. A +-1 plane
  // contributes 2 T - S, a {0, 1} plane T; a row offset mu adds mu S.
  float S = 0.0f;
#pragma unroll
  for (int w = 0; w < WV; ++w) S += red[w];
  float S1 = 0.0f;  // in sequence: plane 1's sum of x h
  if constexpr (kSeq) {
#pragma unroll
    for (int w = 0; w < WV; ++w) S1 += red[WV + w];
  }
  constexpr float ta = (VAR & 1) != 0 ? 1.0f : 2.0f;
  const float ts = (VAR & 1) != 0 ? 0.0f : S;
  const float ts1 = (VAR & 1) != 0 ? 0.0f : S1;
#pragma unroll
  for (int r = 0; r < RW; ++r) {
    float v = 0.0f;
#pragma unroll
    for (int i = 0; i < KP; ++i)
      v += NibScale<TS>::f32(gr[r][i]) * (ta * wave_sum_dpp(acc[r][i]) - (kSeq && i == 1 ? ts1 : ts));
    if (lane == 63 && n0 + r < N) {
      if constexpr ((VAR & 2) != 0) v += NibScale<TS>::f32(mr[r]) * S;
      if constexpr ((VAR & 4) != 0) {
        if (acc_mode & 1) v += acc_io[n0 + r];
        if (acc_mode & 2) {
          acc_io[n0 + r] = v;
        } else {
          nib_store<TY>(&y[n0 + r], v);
          if (acc_mode & 1) acc_io[n0 + r] = 0.0f;
        }
      } else {
        nib_store<TY>(&y[n0 + r], v);
      }
    }
  }
}

// the variant arguments, passed through the launchers unchanged
struct NibExtra {
  const void* mu = nullptr;
  int zero_one = 0;
  const void* h = nullptr;
  float* acc = nullptr;
  int acc_mode = 0;
};

template <typename TX, typename TS, typename TY, int KP, int NPH, int RW, int VAR, int WV = kNibWaves>
hipError_t launch_nib_shape(const uint32_t* planes, int64_t ldp, const void* g, int64_t N, int64_t K,
                            const void* x, void* y, const NibExtra& ex, hipStream_t s) {
  // one phase needs one table buffer (two blocks fit on a compute unit), more need two; the
  // block's sums of x (one per plane in sequence) follow the buffers
  constexpr int NV = (VAR & 8) != 0 ? 2 * NPH : NPH;
  constexpr size_t lds = (NV == 1 ? 1 : 2) * (size_t)kNibBuf + ((VAR & 8) != 0 ? 128 : 64);
  static bool attr_set = false;  // per instantiation
  if (!attr_set) {
    const hipError_t e = hipFuncSetAttribute((const void*)gemv_nib_kernel<TX, TS, TY, KP, NPH, RW, WV, VAR>,
                                             hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return e;
    attr_set = true;
  }
  const unsigned grid = (unsigned)((N + WV * RW - 1) / (WV * RW));
  gemv_nib_kernel<TX, TS, TY, KP, NPH, RW, WV, VAR><<<grid, 64 * WV, lds, s>>>(
      planes, ldp, static_cast<const TS*>(g), N, K, static_cast<const TX*>(x), static_cast<TY*>(y),
      static_cast<const TS*>(ex.mu), ex.zero_one, static_cast<const TX*>(ex.h), ex.acc, ex.acc_mode);
  return hipGetLastError();
}

// rows per wave: the smallest count that puts at most one block on each compute unit, up
// to the most whose plane words still fit in registers next to the lookups' temporaries at
// 16 waves per block (larger counts spill; planes in sequence hold both planes' scales too)
constexpr int nib_max_rows(int kp, int nph, bool seq) {
  return seq ? (nph == 1 ? 3 : nph == 2 ? 2 : 1) : kp == 1 ? (nph <= 3 ? 3 : 2) : (nph == 1 ? 3 : nph <= 3 ? 2 : 1);
}

template <typename TX, typename TS, typename TY, int KP, int NPH, int VAR>
hipError_t launch_nib_rows(int rw, const uint32_t* planes, int64_t ldp, const void* g, int64_t N, int64_t K,
                           const void* x, void* y, const NibExtra& ex, hipStream_t s) {
  constexpr int kMax = nib_max_rows(KP, NPH, (VAR & 8) != 0);
  if (rw > kMax) rw = kMax;
  if constexpr (kMax >= 3) {
    if (rw == 3) return launch_nib_shape<TX, TS, TY, KP, NPH, 3, VAR>(planes, ldp, g, N, K, x, y, ex, s);
  }
  if constexpr (kMax >= 2) {
    if (rw == 2) return launch_nib_shape<TX, TS, TY, KP, NPH, 2, VAR>(planes, ldp, g, N, K, x, y, ex, s);
  }
  return launch_nib_shape<TX, TS, TY, KP, NPH, 1, VAR>(planes, ldp, g, N, K, x, y, ex, s);
}

// ---------------------------------------------------------------------------
// One build for the whole row: K from 4097 up to 10240 columns in LDS, plus a short tail
// ---------------------------------------------------------------------------
// The tables hold sums of +-x, T[e] = sum_j (bit j of e ? +x_j : -x_j), so a +-1 plane needs
// no sum of x (Sum_c B x = sum over nibbles of T[bits]) and entry 0 is written like the others.
// All of a row's tables are built once, with one block barrier, and then looked up with no
// further barrier: 64-word groups of 32 KB (16 entry rows of 2 KB), group j at 32 KB j, nibble i
// of word 64 j + l in slot 8 l + (i ^ a(l)) of every entry row (the swizzle of the phased
// kernel above, the same 64 distinct banks per lookup). Five groups fill the 160 KB of LDS
// (320 words). Words past that (at most 32 of them, whole words) are the tail: one lane per
// half word forms the +-x products of its 16 columns in every plane with v_dot2_f32_f16, no table.
// A lookup address is (j >> 1) << 16 | e << 11 | (l >> 3) << 8 | low byte, plus the immediate
// 32 KB (j & 1): byte 1 holds the nibble and l >> 3, joined with the lane's constant bytes by
// one byte permute as above.
constexpr int kSbGroupWords = 64;
constexpr int kSbMaxGroups = 5;
constexpr uint32_t kSbGroupBytes = 32768u;
constexpr int kSbSH = 11;  // entry row = 2 KB

// MR activation rows (x [MR][K], y [MR][N]): the weights are loaded once, and the tables are
// built and looked up once per activation row, one row after the other in the same LDS (a
// barrier before each rebuild); the next row's activations are fetched behind the weights.
// HM (column scales h, fp16 [KP][K], one activation row): one pass per plane instead, its
// tables built from x (.) h_i (fp16 x fp16 is exact in fp32) and looked up with that plane's
// words only; the passes' row sums add up in fp32 before y is written.
template <int KP, int NG, bool TAIL, int RW, int MR, bool HM = false>
__global__ __launch_bounds__(64 * kNibWaves) __attribute__((amdgpu_waves_per_eu(1, 4))) void gemv_nib1_kernel(
    const uint32_t* __restrict__ planes, int64_t ldp, const __half* __restrict__ g, int64_t N, int64_t K,
    const __half* __restrict__ x, __half* __restrict__ y, const __half* __restrict__ hcol) {
  static_assert(!HM || (MR == 1 && RW == 1), "column scales: one activation row, one row per wave");
  constexpr int NPASS = HM ? KP : MR;  // table builds
  static_assert(NPASS <= 2, "at most two table builds");
  typedef __attribute__((address_space(3))) float lds_f32p;
  constexpr int WV = kNibWaves;
  constexpr int kTables = 8 * kSbGroupWords * NG;               // tables of the row
  constexpr int kTB = (kTables + 64 * WV - 1) / (64 * WV);         // per thread (the last one partial)
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int64_t n0 = ((int64_t)blockIdx.x * WV + wave) * RW;
  const uint32_t Kw = (uint32_t)((K + 31) >> 5);
  const uint32_t Kc = (uint32_t)K;
  const uint32_t ldp_b = (uint32_t)ldp * 4u;
  const __amdgpu_buffer_rsrc_t rp = buffer_rsrc(planes, (uint32_t)((uint64_t)KP * N * ldp * 4));
  const __amdgpu_buffer_rsrc_t rg = buffer_rsrc(g, (uint32_t)((uint64_t)KP * N * 2));
  // x rows start 16-byte aligned when MR > 1 (K a multiple of 8)
  const __amdgpu_buffer_rsrc_t rx =
      buffer_rsrc(x, (uint32_t)((uint64_t)(((MR - 1) * K * 2 + K * 2 + 3) & ~3ll)));
  // h rows start 16-byte aligned (K a multiple of 8, h 16-byte aligned)
  const __amdgpu_buffer_rsrc_t rh = buffer_rsrc(hcol, HM ? (uint32_t)((uint64_t)KP * K * 2) : 0u);

  // 1. the activations of this thread's tables (nibbles tid + 1024 b), then of its tail word.
  // With several activation rows, row m + 1's table activations are fetched once row m's
  // tables are built and its tail activations once row m's lookups are done (one register
  // set each: two would spill)
  uint32_t tq = (uint32_t)tid;  // opaque per activation row (see the row loop)
  // With several activation rows, the threads past the last table (the upper 512 of the last
  // round) build a copy of the table 512 below theirs: the same activations and the same
  // operations write the same bits to the same place, and with every thread building in every
  // round no load sits under a branch (the compiler moved such a load behind the weights,
  // where the first build waited for all of them)
  constexpr bool kDup = MR > 1;
  auto table_of = [&](int b) -> uint32_t {
    const uint32_t q = (uint32_t)(b * 64 * WV) + tq;
    return kDup && (b * WV + wave) * 64 >= kTables ? q - 512u : q;
  };
  auto table_live = [&](int b) -> bool {  // uniform per wave (the table count is a multiple of 512)
    return kDup || (uint32_t)(b * 64 * WV) + tq < (uint32_t)kTables;
  };
  // tail: lane l < 2 TW takes half l & 1 (16 columns) of word 320 + (l >> 1), every plane
  constexpr uint32_t kTail0 = (uint32_t)(kSbGroupWords * NG);
  const uint32_t TW = TAIL ? Kw - kTail0 : 1u;
  const uint32_t tword = kTail0 + ((uint32_t)lane >> 1);
  const uint32_t thalf = (uint32_t)lane & 1u;
  const bool tlive = TAIL && (uint32_t)lane < 2u * TW;
  nib_u32x2 xq[kTB], hq[kTB];
  uint32_t xt[8], ht[8];
  static_assert(kTB <= 3, "at most three tables per thread");
  // the table values of row m of x (or of h) into q, the tail values into t
  auto load_q = [&](__amdgpu_buffer_rsrc_t r, int m, nib_u32x2 (&q)[kTB]) {
    const uint32_t xrow = (uint32_t)m * (uint32_t)K * 2u;
    // written out (a loop here was left rolled inside the row lambda)
    auto one = [&](int b) {
      q[b] = table_live(b) ? __builtin_bit_cast(nib_u32x2, __builtin_amdgcn_raw_buffer_load_b64(
                                                            r, (int)(xrow + 8u * table_of(b)), 0, 0))
                           : nib_u32x2{0u, 0u};
    };
    one(0);
    if constexpr (kTB > 1) one(1);
    if constexpr (kTB > 2) one(2);
  };
  auto load_t = [&](__amdgpu_buffer_rsrc_t r, int m, uint32_t (&t)[8]) {
    if constexpr (TAIL) {
      const uint32_t xo = tlive ? (uint32_t)m * (uint32_t)K * 2u + 64u * tword + 32u * thalf : kNibOob;
#pragma unroll
      for (int v = 0; v < 2; ++v) {
        const auto q4 = __builtin_amdgcn_raw_buffer_load_b128(r, (int)(xo + 16u * v), 0, 0);
#pragma unroll
        for (int c = 0; c < 4; ++c) t[4 * v + c] = q4[c];
      }
    }
  };
  auto load_xq = [&](int m) { load_q(rx, m, xq); };
  auto load_xt = [&](int m) { load_t(rx, m, xt); };
  load_xq(0);
  if constexpr (HM) load_q(rh, 0, hq);
  load_xt(0);
  if constexpr (HM) load_t(rh, 0, ht);
  __builtin_amdgcn_sched_barrier(0);
  __builtin_amdgcn_s_barrier();  // every wave's activations are requested before any weights
  __builtin_amdgcn_sched_barrier(0);

  // 2. the tail words (first: their steps run among the first lookups), plane words (lane l:
  // word 64 j + l of each group), the scales
  uint32_t wd[RW][NG][KP];
  uint32_t wt[RW][KP];
  if constexpr (TAIL) {
#pragma unroll
    for (int r = 0; r < RW; ++r)
#pragma unroll
      for (int i = 0; i < KP; ++i)
        wt[r][i] = buf_u32(rp, tlive ? (uint32_t)(n0 + r) * ldp_b + 4u * tword : kNibOob,
                           (uint32_t)i * (uint32_t)N * ldp_b);
  }
#pragma unroll
  for (int r = 0; r < RW; ++r) {
    const uint32_t row_off = (uint32_t)(n0 + r) * ldp_b;
#pragma unroll
    for (int j = 0; j < NG; ++j) {
      const uint32_t w = (uint32_t)(kSbGroupWords * j + lane);
      // with a tail every group word lies inside the row
      const uint32_t voff = (TAIL || w < Kw) ? row_off + 4u * w : kNibOob;
#pragma unroll
      for (int i = 0; i < KP; ++i) wd[r][j][i] = buf_u32(rp, voff, (uint32_t)i * (uint32_t)N * ldp_b);
    }
  }
  uint32_t gr[RW][KP];
#pragma unroll
  for (int r = 0; r < RW; ++r)
#pragma unroll
    for (int i = 0; i < KP; ++i)
      gr[r][i] = buf_u16(rg, (uint32_t)(n0 + r) * 2u, (uint32_t)i * (uint32_t)N * 2u);
  __builtin_amdgcn_sched_barrier(0);

  // 3. the tables: entry e = lo[e & 3] + hi[e >> 2], lo = {-x0-x1, x0-x1, x1-x0, x0+x1}
  auto build = [&](int b) {
    if (!table_live(b)) return;
    const uint32_t q = table_of(b);
    float xv[4];
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      float v = __half2float(__ushort_as_half((uint16_t)((xq[b][c >> 1] >> (16 * (c & 1))) & 0xffffu)));
      if constexpr (HM) v *= __half2float(__ushort_as_half((uint16_t)((hq[b][c >> 1] >> (16 * (c & 1))) & 0xffffu)));
      xv[c] = (TAIL || 4u * q + (uint32_t)c < Kc) ? v : 0.0f;  // with a tail every table column is < K
    }
    const float s01 = xv[0] + xv[1], d01 = xv[0] - xv[1];
    const float s23 = xv[2] + xv[3], d23 = xv[2] - xv[3];
    const float lo[4] = {-s01, d01, -d01, s01};
    const float hi[4] = {-s23, d23, -d23, s23};
    const uint32_t w = q >> 3, i = q & 7, wl = w & 63u;
    const uint32_t slot = 8u * wl + (i ^ (((wl >> 2) ^ ((wl >> 5) & 1u)) & 7u));
    uint32_t base = (w >> 6) * kSbGroupBytes + slot * 4u;
    // opaque: the 16 entry rows are then immediate offsets (at most 30 KB) from one address
    // register; otherwise groups past 64 KB had an OR per write
    asm volatile("" : "+v"(base));
#pragma unroll
    for (int e = 0; e < 16; ++e)
      *(lds_f32p*)(size_t)(((uint32_t)e << kSbSH) + base) = lo[e & 3] + hi[e >> 2];
  };
  // 4. lookups: one LDS read per 4 weight bits. A lane past the row's last word holds 0 and
  // reads entry 0 of a table whose activations are 0.
  const int al = ((lane >> 2) ^ ((lane >> 5) & 1)) & 7;
  uint32_t cb[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) cb[i] = 32u * (uint32_t)(lane & 7) + 4u * (uint32_t)(i ^ al);
  uint32_t lh = (uint32_t)(lane >> 3) * 0x01010101u;
  // the tail (step 5 below) is spread over the lookups, a few of its steps after each word's
  // LDS reads are issued: its ALU work fills the wait for them instead of running at the end,
  // when every wave of the compute unit would run it at once
  typedef _Float16 nib_h2 __attribute__((ext_vector_type(2)));
  const nib_h2 neg1 = __builtin_bit_cast(nib_h2, 0xBC00BC00u);
  float tt[RW][KP];
  uint32_t w2[RW][KP];  // the lane's 16 bits: byte 2 h of the word in byte 0, byte 2 h + 1 in byte 2
  // 5. tail step (c, plane i): columns c and c + 8 of the lane's 16 as one fp16 pair; bits c and
  // c + 8 moved to the two sign positions flip them, and the dot product with (-1, -1) gives +x
  // for a set bit, -x for a clear one. With h the pair of h is flipped (and negated) instead and
  // dotted with the pair of x: -(+-h) x = +-(h x), exact products in fp32.
  auto tail_step = [&](int r, int c, int i) {
    const uint32_t sel = (c & 1) ? 0x07060302u : 0x05040100u;
    const uint32_t pr = __builtin_amdgcn_perm(xt[4 + (c >> 1)], xt[c >> 1], sel);
    if constexpr (HM) {
      const uint32_t ph = __builtin_amdgcn_perm(ht[4 + (c >> 1)], ht[c >> 1], sel);
      const uint32_t v = ph ^ (~(w2[r][i] << (15 - c)) & 0x80008000u);
      tt[r][i] = __builtin_amdgcn_fdot2(__builtin_bit_cast(nib_h2, v), __builtin_bit_cast(nib_h2, pr), tt[r][i], false);
    } else {
      const uint32_t v = pr ^ ((w2[r][i] << (15 - c)) & 0x80008000u);
      tt[r][i] = __builtin_amdgcn_fdot2(__builtin_bit_cast(nib_h2, v), neg1, tt[r][i], false);
    }
  };
  constexpr int kPlanesPerPass = HM ? 1 : KP;
  constexpr int kSteps = 8 * kPlanesPerPass;
  // Without a tail the lookups are software-pipelined: the 8 reads of word n + 1 are issued
  // before the sums of word n, so each wave keeps two words' reads in flight and its ALU work
  // runs while they are served (in straight order the compiler waits for every word's reads
  // before computing the next word's addresses): 28672x8192 with two rows per wave 23.6 ->
  // 21.8 us (k = 2), 14.1 -> 13.1 us (k = 1). With the tail, whose steps already fill those
  // waits, the straight order measured 1 % faster and is kept.
  constexpr bool kPipe = !TAIL;
  constexpr int kW = NG * RW * kPlanesPerPass;  // looked-up words per pass, in (group, row, plane) order
  // plane of word wi in pass m (with h: the pass's plane)
  auto plane_of = [&](int m, int wi) { return HM ? m : wi % KP; };
  auto issue = [&](int m, int wi, float (&e)[8]) {
    const int j = wi / (RW * kPlanesPerPass), r = (wi / kPlanesPerPass) % RW, i = plane_of(m, wi);
    const uint32_t w = wd[r][j][i];
    const uint32_t hiw = (uint32_t)(j >> 1) << 16;
    const uint32_t o = kSbGroupBytes * (uint32_t)(j & 1);
    const uint32_t ev = ((w << 3) & 0x78787878u) | lh;  // byte m: nibble 2 m in bits 3-6
    const uint32_t od = ((w >> 1) & 0x78787878u) | lh;  // byte m: nibble 2 m + 1
#pragma unroll
    for (int m = 0; m < 4; ++m) {
      e[2 * m] = lds_f32(__builtin_amdgcn_perm(ev, cb[2 * m] | hiw, 0x0c020000u | ((4u + m) << 8)) + o);
      e[2 * m + 1] = lds_f32(__builtin_amdgcn_perm(od, cb[2 * m + 1] | hiw, 0x0c020000u | ((4u + m) << 8)) + o);
    }
  };
  float vh[RW];  // with h: the row sums of the passes so far
#pragma unroll
  for (int r = 0; r < RW; ++r) vh[r] = 0.0f;
  // one activation row per call; rows after the first run in a loop that is not unrolled, which
  // keeps the registers those of one row (unrolled, the compiler kept every row's addresses and
  // activations live and spilled). The first row is outside the loop: at the loop's head the
  // compiler waits for every load in flight, which must not delay the first table build.
  auto row = [&](int m) {
    if (m > 0) {  // every wave is done with the previous row's tables
      __syncthreads();
      __builtin_amdgcn_sched_barrier(0);
    }
    build(0);  // written out, as the loads
    if constexpr (kTB > 1) build(1);
    if constexpr (kTB > 2) build(2);
    if (m + 1 < NPASS) {  // the next pass's table values, behind the weights
      if constexpr (HM) load_q(rh, m + 1, hq);
      else load_xq(m + 1);
    }
    __builtin_amdgcn_sched_barrier(0);
    __syncthreads();
    __builtin_amdgcn_sched_barrier(0);
    float acc[RW][KP];
#pragma unroll
    for (int r = 0; r < RW; ++r)
#pragma unroll
      for (int i = 0; i < KP; ++i) {
        acc[r][i] = 0.0f;
        tt[r][i] = 0.0f;
        // after the build: waits for the tail words, not before it
        if constexpr (TAIL) w2[r][i] = __builtin_amdgcn_perm(wt[r][i], wt[r][i], thalf ? 0x0c030c02u : 0x0c010c00u);
      }
    float ebuf[2][8];
    if constexpr (kPipe) issue(m, 0, ebuf[0]);
#pragma unroll
    for (int wi = 0; wi < kW; ++wi) {
      if constexpr (kPipe) {
        if (wi + 1 < kW) issue(m, wi + 1, ebuf[(wi + 1) & 1]);
        __builtin_amdgcn_sched_barrier(0);
      } else {
        issue(m, wi, ebuf[wi & 1]);
      }
      if constexpr (TAIL) {  // this word's share of the tail steps (RW = 1 with a tail)
#pragma unroll
        for (int st = (kSteps * wi) / kW; st < (kSteps * (wi + 1)) / kW; ++st)
          tail_step(0, st / kPlanesPerPass, HM ? m : st % KP);
      }
      const float* e = ebuf[wi & 1];
      float t = (e[0] + e[1]) + (e[2] + e[3]);
      t += (e[4] + e[5]) + (e[6] + e[7]);
      acc[(wi / kPlanesPerPass) % RW][plane_of(m, wi)] += t;
      // (in the row loop, keep each word's tail steps with it: hoisted together they hold
      // 8 k shifted words live through the lookups)
      if constexpr (kPipe || NPASS > 1) __builtin_amdgcn_sched_barrier(0);
    }
    if constexpr (TAIL) {
#pragma unroll
      for (int r = 0; r < RW; ++r)
#pragma unroll
        for (int i = 0; i < KP; ++i) acc[r][i] += tt[r][i];
      if (m + 1 < NPASS) {
        if constexpr (HM) load_t(rh, m + 1, ht);
        else load_xt(m + 1);
      }
    }

    // 6. row sums of activation row m (with h: the pass's plane, added up over the passes)
#pragma unroll
    for (int r = 0; r < RW; ++r) {
      float v = 0.0f;
#pragma unroll
      for (int i = 0; i < KP; ++i)
        if (!HM || i == m) v += __half2float(__ushort_as_half((uint16_t)gr[r][i])) * wave_sum_dpp(acc[r][i]);
      if constexpr (HM) {
        vh[r] += v;
        if (m + 1 == NPASS && lane == 63 && n0 + r < N) y[n0 + r] = __float2half_rn(vh[r]);
      } else {
        if (lane == 63 && n0 + r < N) y[(int64_t)m * N + n0 + r] = __float2half_rn(v);
      }
    }
    if constexpr (NPASS > 1) {
      // everything the table and lookup addresses and the row sums derive from is the same in
      // every trip: hoisted out of the loop, those values would stay live across it (about 80
      // registers, which spill) and the first trip would wait for every load before its table
      // build; opaque copies made at the end of each trip (when every load has arrived) keep
      // them inside the loop
      asm volatile("" : "+v"(lh), "+v"(tq));
#pragma unroll
      for (int r = 0; r < RW; ++r) {
#pragma unroll
        for (int j = 0; j < NG; ++j)
#pragma unroll
          for (int i = 0; i < KP; ++i) asm volatile("" : "+v"(wd[r][j][i]));
#pragma unroll
        for (int i = 0; i < KP; ++i) {
          asm volatile("" : "+v"(gr[r][i]));
          if constexpr (TAIL) asm volatile("" : "+v"(wt[r][i]));
        }
      }
#pragma unroll
      for (int i = 0; i < 8; ++i) asm volatile("" : "+v"(cb[i]));
    }
  };
  if constexpr (HM) {  // the planes' passes, written out (the pass picks plane registers)
    row(0);
    if constexpr (KP > 1) row(1);
  } else {
    row(0);
#pragma unroll 1
    for (int m = 1; m < MR; ++m) row(m);
  }
}

// the single-build kernel's reach: K above one phase of the phased kernel, at most 320 words
// in LDS, and a tail of at most 32 whole words (one lane per half word)
bool nib1_fits(int kp, int64_t K) {
  const int64_t Kw = (K + 31) / 32;
  if (K <= 32 * kNibPhaseWords) return false;
  if (Kw <= kSbMaxGroups * kSbGroupWords) return true;
  return K % 32 == 0 && Kw - kSbMaxGroups * kSbGroupWords <= 32;
}

template <int KP, int NG, bool TAIL, int RW, int MR = 1, bool HM = false>
hipError_t launch_nib1_shape(const uint32_t* planes, int64_t ldp, const void* g, int64_t N, int64_t K,
                             const void* x, void* y, hipStream_t s, const void* hcol = nullptr) {
  constexpr size_t lds = (size_t)NG * kSbGroupBytes;
  static bool attr_set = false;  // per instantiation
  if (!attr_set) {
    const hipError_t e = hipFuncSetAttribute((const void*)gemv_nib1_kernel<KP, NG, TAIL, RW, MR, HM>,
                                             hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return e;
    attr_set = true;
  }
  const unsigned grid = (unsigned)((N + kNibWaves * RW - 1) / (kNibWaves * RW));
  gemv_nib1_kernel<KP, NG, TAIL, RW, MR, HM><<<grid, 64 * kNibWaves, lds, s>>>(
      planes, ldp, static_cast<const __half*>(g), N, K, static_cast<const __half*>(x), static_cast<__half*>(y),
      static_cast<const __half*>(hcol));
  return hipGetLastError();
}

template <int KP, int NG, bool TAIL>
hipError_t launch_nib1_ng(int rw, const uint32_t* planes, int64_t ldp, const void* g, int64_t N, int64_t K,
                          const void* x, void* y, hipStream_t s) {
  if constexpr (!TAIL) {  // two rows per wave with the tail's registers would spill
    if (rw >= 2) return launch_nib1_shape<KP, NG, TAIL, 2>(planes, ldp, g, N, K, x, y, s);
  }
  return launch_nib1_shape<KP, NG, TAIL, 1>(planes, ldp, g, N, K, x, y, s);
}

template <int KP>
hipError_t launch_nib1(const uint32_t* planes, int64_t ldp, const void* g, int64_t N, int64_t K, const void* x,
                       void* y, hipStream_t s) {
  const int64_t Kw = (K + 31) / 32;
  const int64_t cus = device_cu_count();
  const int rw = (N + kNibWaves - 1) / kNibWaves <= cus ? 1 : 2;
  const int64_t ng = Kw >= kSbMaxGroups * kSbGroupWords ? kSbMaxGroups : (Kw + kSbGroupWords - 1) / kSbGroupWords;
  const bool tail = Kw > kSbMaxGroups * kSbGroupWords;
  switch (ng) {
    case 3: return launch_nib1_ng<KP, 3, false>(rw, planes, ldp, g, N, K, x, y, s);
    case 4: return launch_nib1_ng<KP, 4, false>(rw, planes, ldp, g, N, K, x, y, s);
    default:
      return tail ? launch_nib1_ng<KP, 5, true>(rw, planes, ldp, g, N, K, x, y, s)
                  : launch_nib1_ng<KP, 5, false>(rw, planes, ldp, g, N, K, x, y, s);
  }
}

// two activation rows (h = 1, plain product): one launch, the weights read once. Measured on
// 4096x11008 (us, against two single-row launches or the matrix cores): M = 2 k = 2 9.8 against
// 10.8, k = 1 7.1 against 8.6; M = 3 k = 2 15.4 against 13.3 and M = 4 19.5 against 13.4 on the
// matrix cores, so only M = 2 takes this path. Each further row costs a table build, its
// barriers and a full set of lookups (about 4.2 us here), which the matrix cores undercut.
constexpr int kNibMaxRows = 2;

template <int KP, int MR>
hipError_t launch_nib1_rows(const uint32_t* planes, int64_t ldp, const void* g, int64_t N, int64_t K,
                            const void* x, void* y, hipStream_t s) {
  const int64_t Kw = (K + 31) / 32;
  const int64_t ng = Kw >= kSbMaxGroups * kSbGroupWords ? kSbMaxGroups : (Kw + kSbGroupWords - 1) / kSbGroupWords;
  const bool tail = Kw > kSbMaxGroups * kSbGroupWords;
  switch (ng) {
    case 3: return launch_nib1_shape<KP, 3, false, 1, MR>(planes, ldp, g, N, K, x, y, s);
    case 4: return launch_nib1_shape<KP, 4, false, 1, MR>(planes, ldp, g, N, K, x, y, s);
    default:
      return tail ? launch_nib1_shape<KP, 5, true, 1, MR>(planes, ldp, g, N, K, x, y, s)
                  : launch_nib1_shape<KP, 5, false, 1, MR>(planes, ldp, g, N, K, x, y, s);
  }
}

template <int KP>
hipError_t launch_nib1_rows_m(int64_t M, const uint32_t* planes, int64_t ldp, const void* g, int64_t N, int64_t K,
                              const void* x, void* y, hipStream_t s) {
  if (M == 2) return launch_nib1_rows<KP, 2>(planes, ldp, g, N, K, x, y, s);
  return hipErrorNotSupported;
}

// column scales h (fp16 [KP][K]), one activation row: one pass per plane in one launch
template <int KP>
hipError_t launch_nib1_h(const uint32_t* planes, int64_t ldp, const void* g, const void* h, int64_t N, int64_t K,
                         const void* x, void* y, hipStream_t s) {
  const int64_t Kw = (K + 31) / 32;
  const int64_t ng = Kw >= kSbMaxGroups * kSbGroupWords ? kSbMaxGroups : (Kw + kSbGroupWords - 1) / kSbGroupWords;
  const bool tail = Kw > kSbMaxGroups * kSbGroupWords;
  switch (ng) {
    case 3: return launch_nib1_shape<KP, 3, false, 1, 1, true>(planes, ldp, g, N, K, x, y, s, h);
    case 4: return launch_nib1_shape<KP, 4, false, 1, 1, true>(planes, ldp, g, N, K, x, y, s, h);
    default:
      return tail ? launch_nib1_shape<KP, 5, true, 1, 1, true>(planes, ldp, g, N, K, x, y, s, h)
                  : launch_nib1_shape<KP, 5, false, 1, 1, true>(planes, ldp, g, N, K, x, y, s, h);
  }
}

template <typename TX, typename TS, typename TY, int KP, int VAR>
hipError_t launch_nib_kp(const uint32_t* planes, int64_t ldp, const void* g, int64_t N, int64_t K,
                         const void* x, void* y, const NibExtra& ex, hipStream_t s) {
  if constexpr (VAR == 0) {
    if (nib1_fits(KP, K)) return launch_nib1<KP>(planes, ldp, g, N, K, x, y, s);
  }
  const int64_t phases = ((K + 31) / 32 + kNibPhaseWords - 1) / kNibPhaseWords;
  const int64_t cus = device_cu_count();
  int rw = 3;
  for (int c = 1; c <= 3; ++c)
    if ((N + kNibWaves * c - 1) / (kNibWaves * c) <= cus) {
      rw = c;
      break;
    }
  switch (phases) {
    case 1: return launch_nib_rows<TX, TS, TY, KP, 1, VAR>(rw, planes, ldp, g, N, K, x, y, ex, s);
    case 2: return launch_nib_rows<TX, TS, TY, KP, 2, VAR>(rw, planes, ldp, g, N, K, x, y, ex, s);
    case 3: return launch_nib_rows<TX, TS, TY, KP, 3, VAR>(rw, planes, ldp, g, N, K, x, y, ex, s);
    default: return launch_nib_rows<TX, TS, TY, KP, 4, VAR>(rw, planes, ldp, g, N, K, x, y, ex, s);
  }
}

template <int KP>
hipError_t launch_nib_var(const uint32_t* planes, int64_t ldp, const void* g, int64_t N, int64_t K, const void* x,
                          void* y, const NibExtra& ex, hipStream_t s) {
  const int var = (ex.zero_one ? 1 : 0) | (ex.mu ? 2 : 0) | (ex.h ? 4 : 0);
  switch (var) {
    case 0: return launch_nib_kp<__half, __half, __half, KP, 0>(planes, ldp, g, N, K, x, y, ex, s);
    case 1: return launch_nib_kp<__half, __half, __half, KP, 1>(planes, ldp, g, N, K, x, y, ex, s);
    case 2: return launch_nib_kp<__half, __half, __half, KP, 2>(planes, ldp, g, N, K, x, y, ex, s);
    case 3: return launch_nib_kp<__half, __half, __half, KP, 3>(planes, ldp, g, N, K, x, y, ex, s);
    default:
      if constexpr (KP == 1) {  // h mode: one plane per pass, no row offset
        if (var == 4) return launch_nib_kp<__half, __half, __half, 1, 4>(planes, ldp, g, N, K, x, y, ex, s);
        if (var == 5) return launch_nib_kp<__half, __half, __half, 1, 5>(planes, ldp, g, N, K, x, y, ex, s);
      } else {  // two planes with h: in sequence in one pass
        if (var == 4) return launch_nib_kp<__half, __half, __half, 2, 12>(planes, ldp, g, N, K, x, y, ex, s);
        if (var == 5) return launch_nib_kp<__half, __half, __half, 2, 13>(planes, ldp, g, N, K, x, y, ex, s);
      }
      return hipErrorNotSupported;
  }
}

}  // namespace

bool gemv_nib_fits(int k, int64_t N, int64_t K, int64_t ldp, rb_dtype x_dtype, rb_dtype scale_dtype,
                   rb_dtype y_dtype) {
  const uint64_t lim = 0x7fffffffull;
  return x_dtype == RB_F16 && scale_dtype == RB_F16 && y_dtype == RB_F16 && (k == 1 || k == 2) &&
         (K + 31) / 32 <= 4 * kNibPhaseWords && (uint64_t)k * N * ldp * 4 < lim && (uint64_t)k * N * 4 < lim &&
         (uint64_t)K * 4 + 16 < lim && (uint64_t)(N + kNibWaves * 3) * ldp * 4 < lim;
}

bool gemv_nib_rows_fits(int k, int64_t N, int64_t K, int64_t ldp, int64_t M, rb_dtype x_dtype, rb_dtype scale_dtype,
                        rb_dtype y_dtype) {
  // (planes of 2^27 bits and more go to the matrix cores from M = 2 on)
  return M >= 2 && M <= kNibMaxRows && K % 8 == 0 && nib1_fits(k, K) && (double)k * N * K < 134217728.0 &&
         gemv_nib_fits(k, N, K, ldp, x_dtype, scale_dtype, y_dtype) && (uint64_t)M * (uint64_t)K * 2u < 0x7fffffffull;
}

hipError_t launch_gemv_nib_rows(const uint32_t* planes, int64_t ldp, const void* g, int k, int64_t N, int64_t K,
                                const void* x, int64_t M, void* y, hipStream_t s) {
  if (k == 1) return launch_nib1_rows_m<1>(M, planes, ldp, g, N, K, x, y, s);
  if (k == 2) return launch_nib1_rows_m<2>(M, planes, ldp, g, N, K, x, y, s);
  return hipErrorNotSupported;
}

hipError_t launch_gemv_nib(const uint32_t* planes, int64_t ldp, const void* g, rb_dtype scale_dtype, int k,
                           int64_t N, int64_t K, const void* x, rb_dtype x_dtype, void* y, rb_dtype y_dtype,
                           const void* mu, int zero_one, hipStream_t s) {
  if (x_dtype != RB_F16 || scale_dtype != RB_F16 || y_dtype != RB_F16) return hipErrorNotSupported;
  switch (k) {
    case 1: {
      NibExtra ex;
      ex.mu = mu;
      ex.zero_one = zero_one;
      return launch_nib_var<1>(planes, ldp, g, N, K, x, y, ex, s);
    }
    case 2: {
      NibExtra ex;
      ex.mu = mu;
      ex.zero_one = zero_one;
      return launch_nib_var<2>(planes, ldp, g, N, K, x, y, ex, s);
    }
    default: return hipErrorNotSupported;
  }
}

// general h, one activation row: one single-plane pass per plane with x (.) h_i in the tables;
// the passes add up in acc (one fp32 per row, zero on entry and on return) and the last one
// writes y. K must be a multiple of 4 and h 8-byte aligned (each pass reads h_i in 8-byte units).
bool gemv_nib_h_fits(int k, int64_t N, int64_t K, int64_t ldp, const void* h, rb_dtype x_dtype,
                     rb_dtype scale_dtype, rb_dtype y_dtype) {
  return k >= 1 && k <= 4 && K % 4 == 0 && (reinterpret_cast<uintptr_t>(h) & 7u) == 0 &&
         gemv_nib_fits(1, N, K, ldp, x_dtype, scale_dtype, y_dtype) &&
         (uint64_t)k * N * ldp * 4 < 0x7fffffffull;
}

hipError_t launch_gemv_nib_h(const uint32_t* planes, int64_t ldp, const void* g, const void* h, int k, int64_t N,
                             int64_t K, const void* x, void* y, int zero_one, float* acc, hipStream_t s) {
  // 4096 < K within the one-build kernel's reach (K a multiple of 8, h 16-byte aligned, +-1
  // planes, one row per wave fills at most one block per compute unit): every plane's pass in
  // one launch, with one table build per plane. 4096x11008 k = 2 8.66 -> 8.35 us, k = 1 4.97 ->
  // 4.85, 4096x8192 k = 2 6.38 -> 5.69; 28672x8192 measured 32.7 against 31.2 (more blocks than
  // compute units: the phased kernel's three rows per wave share its builds) and keeps that.
  if (!zero_one && (k == 1 || k == 2) && nib1_fits(k, K) && K % 8 == 0 &&
      (reinterpret_cast<uintptr_t>(h) & 15u) == 0 && N <= (int64_t)kNibWaves * device_cu_count())
    return k == 1 ? launch_nib1_h<1>(planes, ldp, g, h, N, K, x, y, s) : launch_nib1_h<2>(planes, ldp, g, h, N, K, x, y, s);
  if (k == 2) {  // both planes in one pass (h_1 follows h_0 at h + K); acc is not used
    NibExtra ex;
    ex.zero_one = zero_one;
    ex.h = h;
    return launch_nib_var<2>(planes, ldp, g, N, K, x, y, ex, s);
  }
  for (int i = 0; i < k; ++i) {
    NibExtra ex;
    ex.zero_one = zero_one;
    ex.h = static_cast<const __half*>(h) + (int64_t)i * K;
    ex.acc = acc;
    ex.acc_mode = (i > 0 ? 1 : 0) | (i + 1 < k ? 2 : 0);
    const hipError_t e = launch_nib_var<1>(planes + (int64_t)i * N * ldp, ldp,
                                           static_cast<const __half*>(g) + (int64_t)i * N, N, K, x, y, ex, s);
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

}  // namespace rb
