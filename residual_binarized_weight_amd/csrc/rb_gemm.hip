// rb_gemm.hip -- batched product on the matrix cores (gfx950 MFMA).
//
// [RaBiT summary page, background "Residual binarization"] y = sum_i g_i (.) (B_i (h_i (.) x))
// for a batch of activation rows X [M][K]. For batches that can feed the matrix cores, the
// bits of each plane are expanded in registers into the fp16 B operand of
// v_mfma_f32_32x32x16_f16 (A = activations staged in LDS), with fp32 accumulation.
//
// Operand order. The MFMA contracts its 16 K slots in any order, as long as A and B agree,
// so the slots are permuted to make the bit expansion cheap: within a 32-column word,
// operand dword e of lane half hh at k-step t holds columns j and j+16 with
// j = 8t + 4hh + e, i.e. bits j and j+16, which one left shift by 15-j moves onto the two
// fp16 sign positions (15, 31). One AND-OR (or AND-XOR) then puts the sign on a fixed
// magnitude pair:
//   fold mode  (fp16 g, h = 1): +-|g_i[n]|, the sign of g folded into the bits; every
//              plane then adds into the same fp32 accumulator (products are exact)
//   ones mode  (fp32 g, h = 1): +-1, and y += g_i * acc_i in fp32 after each plane
//   h mode     (fp16 g and h):  +-h_i[c], and y += g_i * acc_i in fp32 after each plane
//   merge mode (fp16 g, h = 1, k = 2, two or more batch tiles): the two planes' weights
//              +-g_0 +-g_1 of a column formed as one fp16 operand by a packed fma of the
//              plane-1 signs with g_1 onto the plane-0 operand, so one MFMA serves both
//              planes. The sum is rounded once to fp16 (relative error at most 2^-11 of
//              |g_0| + |g_1|); both scales are first multiplied by the power of two that
//              puts |g_0| + |g_1| in [2^14, 2^15), so no operand is subnormal or overflows,
//              and the row's sum is divided by it at the end.
// The activations are staged in LDS in the same permuted order, 128 columns per stage,
// rows padded to 272 B so the 16-byte A reads of consecutive rows hit distinct banks.
//
// Tiles: a block is 4 waves; wave w owns 32 weight rows (one MFMA column tile) and the MT
// 32-row batch tiles of its block, so each expanded B operand feeds MT MFMAs and each A
// read feeds one MFMA per plane. Plane words are prefetched kDepth stages ahead in
// registers; the next activation stage is loaded into registers while the current one is
// multiplied, then written to the other LDS buffer (one barrier per stage).
#include "rb_device.hpp"
#include "rb_internal.h"

namespace rb {
namespace {

typedef _Float16 h8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x2g __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4g __attribute__((ext_vector_type(4)));

constexpr int kGemmWaves = 4;                   // waves per K group
constexpr int kGemmGroupThreads = 64 * kGemmWaves;
constexpr int kGemmTileN = 32 * kGemmWaves;     // weight rows per block
constexpr int kStageCols = 128;                 // columns per stage: 4 words per plane row
constexpr int kStageWords = kStageCols / 32;
constexpr int kRowBytes = kStageCols * 2 + 16;  // 16 groups of 16 B + pad
constexpr int kDepth = 2;                       // plane-word prefetch distance in stages

enum { kModeFold = 0, kModeOnes = 1, kModeH = 2, kModeMerge = 3 };
typedef _Float16 h2g __attribute__((ext_vector_type(2)));

template <typename T> __device__ __forceinline__ void gemm_store(T* p, float v);
template <> __device__ __forceinline__ void gemm_store<float>(float* p, float v) { *p = v; }
template <> __device__ __forceinline__ void gemm_store<__half>(__half* p, float v) { *p = __float2half_rn(v); }

template <typename TS> __device__ __forceinline__ float scale_f32(const TS* p);
template <> __device__ __forceinline__ float scale_f32<__half>(const __half* p) { return __half2float(*p); }
template <> __device__ __forceinline__ float scale_f32<float>(const float* p) { return *p; }

// two groups (hh = 0, 1) of word w, k-step t from 8 consecutive values at column 32w + 8t
// (lo) and 8 at column 32w + 8t + 16 (hi): dword e of group hh = (lo[4hh + e], hi[4hh + e])
__device__ __forceinline__ void interleave(const u32x4g lo, const u32x4g hi, u32x4g& g0, u32x4g& g1) {
  g0[0] = __builtin_amdgcn_perm(hi[0], lo[0], 0x05040100u);
  g0[1] = __builtin_amdgcn_perm(hi[0], lo[0], 0x07060302u);
  g0[2] = __builtin_amdgcn_perm(hi[1], lo[1], 0x05040100u);
  g0[3] = __builtin_amdgcn_perm(hi[1], lo[1], 0x07060302u);
  g1[0] = __builtin_amdgcn_perm(hi[2], lo[2], 0x05040100u);
  g1[1] = __builtin_amdgcn_perm(hi[2], lo[2], 0x07060302u);
  g1[2] = __builtin_amdgcn_perm(hi[3], lo[3], 0x05040100u);
  g1[3] = __builtin_amdgcn_perm(hi[3], lo[3], 0x07060302u);
}

// buffer resource over [base, base + bytes): loads at or past `bytes` return 0
__device__ __forceinline__ __amdgpu_buffer_rsrc_t gemm_rsrc(const void* base, int64_t bytes) {
  const uint32_t n = bytes <= 0 ? 0u : (bytes >= 0x7fffffffll ? 0x7fffffffu : (uint32_t)bytes);
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)n, 0x00020000);
}
constexpr uint32_t kOob = 0x80000000u;  // an offset past every resource above

__device__ __forceinline__ u32x4g buf_load16(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return __builtin_bit_cast(u32x4g, __builtin_amdgcn_raw_buffer_load_b128(r, (int)off, 0, 0));
}

// activation stage in registers: MT units per thread, unit q = (row, word w, k-step t)
template <int MT>
struct XStage {
  u32x4g lo[MT], hi[MT];
};

// rows past M and columns past K read as 0 (the resource ends at the block's last row;
// a column past K gets an out-of-range offset)
template <int MT>
__device__ __forceinline__ void load_x_stage(XStage<MT>& r, __amdgpu_buffer_rsrc_t rx, int64_t K, int64_t kend,
                                             int64_t k0, int tid) {
#pragma unroll
  for (int u = 0; u < MT; ++u) {
    const int q = tid + u * kGemmGroupThreads;  // 0 .. 256 MT - 1
    const int row = q >> 3, wt = q & 7;         // wt = 2 w + t
    const int64_t c = k0 + 32 * (wt >> 1) + 8 * (wt & 1);
    const uint32_t off = c < kend ? (uint32_t)((row * K + c) * 2) : kOob;
    r.lo[u] = buf_load16(rx, off);
    r.hi[u] = buf_load16(rx, off + 32u);
  }
}

template <int MT>
__device__ __forceinline__ void store_x_stage(const XStage<MT>& r, uint8_t* buf, int tid) {
#pragma unroll
  for (int u = 0; u < MT; ++u) {
    const int q = tid + u * kGemmGroupThreads;
    const int row = q >> 3, wt = q & 7;
    u32x4g g0, g1;
    interleave(r.lo[u], r.hi[u], g0, g1);
    // group index 4 w + 2 t + hh = 2 wt + hh. Lanes with wt >= 4 write their odd group
    // first: then the 8 lanes of a row cover 8 different 16-byte bank groups in each of
    // the two stores (in order, groups 2wt, 2wt+1 would put wt and wt+4 on the same banks)
    const bool swap = wt >= 4;
    *reinterpret_cast<u32x4g*>(buf + row * kRowBytes + (2 * wt + (swap ? 1 : 0)) * 16) = swap ? g1 : g0;
    *reinterpret_cast<u32x4g*>(buf + row * kRowBytes + (2 * wt + (swap ? 0 : 1)) * 16) = swap ? g0 : g1;
  }
}

// h stage (h mode): one plane's h over the stage, in the same 16 groups; every thread
// loads the unit of tid % 8 (so no load sits in a branch) and threads 0..7 store it.
// Columns past K read as 0.
struct HStage {
  u32x4g lo, hi;
};

__device__ __forceinline__ void load_h_stage(HStage& r, __amdgpu_buffer_rsrc_t rh, int64_t kend, int64_t k0, int tid) {
  const int u = tid & 7;
  const int64_t c = k0 + 32 * (u >> 1) + 8 * (u & 1);
  const uint32_t off = c < kend ? (uint32_t)(c * 2) : kOob;
  r.lo = buf_load16(rh, off);
  r.hi = buf_load16(rh, off + 32u);
}

__device__ __forceinline__ void store_h_stage(const HStage& r, uint8_t* hbuf, int tid) {
  if (tid < 8) {
    u32x4g g0, g1;
    interleave(r.lo, r.hi, g0, g1);
    *reinterpret_cast<u32x4g*>(hbuf + (2 * tid) * 16) = g0;
    *reinterpret_cast<u32x4g*>(hbuf + (2 * tid + 1) * 16) = g1;
  }
}

// B operand from complemented bits `nw` at k-step t, lane half hh: dword e carries the
// signs of bits j, j+16 (j = 8t + 4hh + e) on the magnitude pair base[e]
template <int MODE>
__device__ __forceinline__ h8 expand_b(uint32_t nw, int t, int hh, u32x4g base) {
  u32x4g d;
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const int j = 8 * t + 4 * hh + e;
    const uint32_t sgn = (nw << (15 - j)) & 0x80008000u;
    d[e] = MODE == kModeH ? (base[e] ^ sgn) : (base[e] | sgn);
  }
  return __builtin_bit_cast(h8, d);
}

// merge mode: dword e of the operand is fma(+-1 of plane 1, g_1 pair, +-g_0 of plane 0), the
// signs from the complemented bits nw0 (sign of g_0 folded in) and nw1 as in expand_b
__device__ __forceinline__ h8 expand_merge(uint32_t nw0, uint32_t nw1, int t, int hh, uint32_t base0,
                                           uint32_t g1pair) {
  u32x4g d;
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const int j = 8 * t + 4 * hh + e;
    const uint32_t b0 = base0 | ((nw0 << (15 - j)) & 0x80008000u);
    const uint32_t b1 = 0x3C003C00u | ((nw1 << (15 - j)) & 0x80008000u);
    const h2g r = __builtin_elementwise_fma(__builtin_bit_cast(h2g, b1), __builtin_bit_cast(h2g, g1pair),
                                            __builtin_bit_cast(h2g, b0));
    d[e] = __builtin_bit_cast(uint32_t, r);
  }
  return __builtin_bit_cast(h8, d);
}

// KP = planes multiplied per pass (fold and merge modes: all k; otherwise 1).
// A group runs nch stages (group 0's count). The plane words of a stage past its half (or
// past K in a 64-column tail) are whatever the row holds there, and they meet activations
// that read as 0, so they add +-0 (a non-finite g, which no finite W packs to, would turn
// that row's +-0 into NaN). Activations are fetched XD stages ahead: kDepth for one 32-row
// batch tile, whose MFMAs per stage are too few to cover a load's latency, else 1.
// NG wave groups per block. MSPLIT (two groups): they take two halves of the batch, else
// NG parts of K. blockIdx.z splits K further into chunks of kz columns (a multiple of
// the stage width) when the row and batch tiles alone would leave compute units idle; each
// chunk's partial sums then go to part[z][M][N] (fp32) for gemm_reduce_kernel, else to y.
// With a K split the grid's x extent is rounded up to a multiple of 8 (blocks past the row
// tiles return at once), so that every chunk of row tile x runs on the same XCD, x % 8
// (consecutive blocks go to consecutive XCDs), where the reduce reads its partials.
template <typename TS, typename TY, int MT, int MODE, int KP, int NG, bool MSPLIT>
__global__ __launch_bounds__(kGemmGroupThreads * NG) void gemm_small_kernel(
    const uint32_t* __restrict__ planes, int64_t ldp, const TS* __restrict__ g, const __half* __restrict__ h,
    int k, int64_t N, int64_t K, const __half* __restrict__ x, int64_t M, TY* __restrict__ y, int64_t kz,
    float* __restrict__ part) {
  extern __shared__ __align__(16) uint8_t smem[];
  static_assert(!MSPLIT || NG == 2, "the batch split takes two groups");
  if ((int64_t)blockIdx.x * kGemmTileN >= N) return;  // padding of the grid (uniform per block)
  // the K groups' hand-over below fits in the groups' activation buffers
  static_assert((NG - 1) * kGemmWaves * MT * 16 * 64 * 4 <= NG * 2 * MT * 32 * kRowBytes, "hand-over space");
  const int tid_all = threadIdx.x;
  const int lane = tid_all & 63;
  const int wave_all = __builtin_amdgcn_readfirstlane(tid_all >> 6);  // uniform: keeps resources scalar
  const int grp = NG == 1 ? 0 : wave_all / kGemmWaves;  // group of this wave
  const int wave = wave_all % kGemmWaves;   // wave within its group
  const int tid = tid_all % kGemmGroupThreads;
  constexpr int NH = MODE == kModeH ? KP : 1;  // h mode: one h stage and one accumulator per plane
  uint8_t* const gbase = smem + grp * (2 * MT * 32 * kRowBytes + 512 * NH);
  uint8_t* const xbuf0 = gbase;
  uint8_t* const xbuf1 = gbase + MT * 32 * kRowBytes;
  uint8_t* const hbuf0 = gbase + 2 * MT * 32 * kRowBytes;  // plane q's h stage at + 256 q
  uint8_t* const hbuf1 = hbuf0 + 256 * NH;

  const int nl = lane & 31;
  const int hh = lane >> 5;
  const int64_t n0 = (int64_t)blockIdx.x * kGemmTileN + wave * 32;  // wave's first row
  const int64_t n = n0 + nl;
  const int64_t nc = n < N ? n : N - 1;  // rows past N repeat the last row and are not stored
  const int64_t rb = n0 < N ? n0 : N - 1;
  // batch split: group g takes batch rows [m_base, m_base + 32 MT) of the block's 64 MT;
  // K split: group g takes columns [g kh, (g + 1) kh) of the chunk, kh a whole number of
  // stages, and every group runs group 0's stage count (stages past a group's columns read
  // activations as 0)
  const int64_t m_base = MSPLIT ? ((int64_t)blockIdx.y * NG + grp) * MT * 32 : (int64_t)blockIdx.y * MT * 32;
  const int64_t m_left = M - m_base;
  const int64_t m_rows = m_left < 0 ? 0 : (m_left < MT * 32 ? m_left : MT * 32);
  // this block's K chunk [kz0, kz1); the group split below works inside it
  const int64_t kz0 = (int64_t)blockIdx.z * kz;
  const int64_t kz1 = kz0 + kz < K ? kz0 + kz : K;
  const int64_t kl = kz1 - kz0;
  const int64_t kh_raw = (((kl + NG - 1) / NG + kStageCols - 1) / kStageCols) * kStageCols;
  const int64_t kh = (MSPLIT || NG == 1) ? kl : (kh_raw < kl ? kh_raw : kl);
  const int64_t g0 = MSPLIT ? 0 : ((int64_t)grp * kh < kl ? (int64_t)grp * kh : kl);  // group's columns
  const int64_t g1 = MSPLIT ? kh : (g0 + kh < kl ? g0 + kh : kl);                     // in the chunk
  const int64_t kbeg = kz0 + g0;
  const int64_t kend = kz0 + g1;
  const int nch = (int)((kh + kStageCols - 1) / kStageCols);
  const __amdgpu_buffer_rsrc_t rx = gemm_rsrc(x + (m_rows > 0 ? m_base : 0) * K, m_rows * K * 2);
  const uint32_t lane_off = (uint32_t)((nc - rb) * ldp * 4 + kbeg / 8);  // 4 bytes per 32 columns

  f32x16 yacc[MT];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) yacc[mt] = (f32x16){};

  constexpr int XD = MT == 1 ? kDepth : 1;  // activation stages in flight (divides kDepth)
  const int passes = (MODE == kModeFold || MODE == kModeMerge) ? 1 : k / KP;
  // merge mode: plane 0's |g_0| 2^sh pair (its sign folded into the bits), g_1 2^sh in both
  // halves, and 2^-sh for the row's sum
  uint32_t mbase = 0u, mg1 = 0u, msgn = 0u;
  float mscale = 1.0f;
  if constexpr (MODE == kModeMerge) {
    const float g0 = __half2float(*reinterpret_cast<const __half*>(g + nc));
    const float g1 = __half2float(*reinterpret_cast<const __half*>(g + N + nc));
    const float m = fabsf(g0) + fabsf(g1);
    int ex = 0;
    (void)frexpf(m, &ex);  // m = f 2^ex, f in [0.5, 1)
    const int sh = m > 0.0f && __builtin_isfinite(m) ? 15 - ex : 0;
    const uint32_t a = (uint32_t)__half_as_ushort(__float2half_rn(ldexpf(g0, sh)));  // exact: a power of two
    const uint32_t b = (uint32_t)__half_as_ushort(__float2half_rn(ldexpf(g1, sh)));
    mbase = (a & 0x7fffu) | ((a & 0x7fffu) << 16);
    msgn = (a & 0x8000u) ? 0xffffffffu : 0u;
    mg1 = b | (b << 16);
    mscale = ldexpf(1.0f, -sh);
  }
  for (int pass = 0; pass < passes; ++pass) {
    const int i0 = (MODE == kModeFold || MODE == kModeMerge) ? 0 : pass * KP;
    __amdgpu_buffer_rsrc_t rw[KP];
    u32x4g base[KP];
    uint32_t gsgn[KP];
#pragma unroll
    for (int p = 0; p < KP; ++p) {
      const int i = i0 + p;
      const int64_t first = (int64_t)i * N + rb;
      rw[p] = gemm_rsrc(planes + first * ldp, ((int64_t)k * N - first) * ldp * 4);
      if (MODE == kModeFold) {
        const uint32_t gb = (uint32_t)__half_as_ushort(*reinterpret_cast<const __half*>(g + (int64_t)i * N + nc));
        const uint32_t mag = gb & 0x7fffu;
        const uint32_t pair = mag | (mag << 16);
        base[p] = (u32x4g){pair, pair, pair, pair};
        gsgn[p] = (gb & 0x8000u) ? 0xffffffffu : 0u;
      } else {
        base[p] = (u32x4g){0x3C003C00u, 0x3C003C00u, 0x3C003C00u, 0x3C003C00u};  // +-1
        gsgn[p] = 0u;
      }
    }
    __amdgpu_buffer_rsrc_t rh[NH];
#pragma unroll
    for (int q = 0; q < NH; ++q) rh[q] = gemm_rsrc(MODE == kModeH ? h + (int64_t)(i0 + q) * K : x, K * 2);

    f32x16 acc[NH][MT];
#pragma unroll
    for (int q = 0; q < NH; ++q)
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) acc[q][mt] = (f32x16){};

    // prologue: plane words of stages 0 .. kDepth-1, activation stage 0
    u32x4g wr[kDepth][KP];
#pragma unroll
    for (int d = 0; d < kDepth; ++d)
#pragma unroll
      for (int p = 0; p < KP; ++p) wr[d][p] = buf_load16(rw[p], lane_off + 16u * d);
    // activation (and h) stages ride a ring of XD register slots: stage c sits in slot
    // c % XD from its load, XD stages ahead, until it is written to LDS at the end of stage c-1
    XStage<MT> xq[XD];
    HStage hq[XD][NH];
#pragma unroll
    for (int j = 0; j < XD; ++j) {
      load_x_stage<MT>(xq[j], rx, K, kend, kbeg + (int64_t)j * kStageCols, tid);
      if (MODE == kModeH) {
#pragma unroll
        for (int q = 0; q < NH; ++q) load_h_stage(hq[j][q], rh[q], kend, kbeg + (int64_t)j * kStageCols, tid);
      }
    }
    __syncthreads();  // the previous pass may still read buffer 0
    store_x_stage<MT>(xq[0], xbuf0, tid);
    if (MODE == kModeH) {
#pragma unroll
      for (int q = 0; q < NH; ++q) store_h_stage(hq[0][q], hbuf0 + 256 * q, tid);
    }
    __syncthreads();

    for (int cb = 0; cb < nch; cb += kDepth) {
#pragma unroll
      for (int d = 0; d < kDepth; ++d) {
        const int c = cb + d;
        if (c >= nch) break;  // uniform: every wave of the block runs nch stages
        u32x4g cur[KP];
#pragma unroll
        for (int p = 0; p < KP; ++p) cur[p] = wr[d][p];
        load_x_stage<MT>(xq[d % XD], rx, K, kend, kbeg + (int64_t)(c + XD) * kStageCols, tid);
        if (MODE == kModeH) {
#pragma unroll
          for (int q = 0; q < NH; ++q)
            load_h_stage(hq[d % XD][q], rh[q], kend, kbeg + (int64_t)(c + XD) * kStageCols, tid);
        }
#pragma unroll
        for (int p = 0; p < KP; ++p) wr[d][p] = buf_load16(rw[p], lane_off + 16u * (uint32_t)(c + kDepth));
        // keep the loads at the top of the stage: they must be in flight during its MFMAs
        __builtin_amdgcn_sched_barrier(0);

        const uint8_t* xb = (d & 1) ? xbuf1 : xbuf0;  // kDepth is even: stage parity = d parity
        const uint8_t* hb = (d & 1) ? hbuf1 : hbuf0;
        // A fragments of step s = 2 w + t are read one step ahead of their MFMAs
        h8 anext[MT];
#pragma unroll
        for (int mt = 0; mt < MT; ++mt)
          anext[mt] = *reinterpret_cast<const h8*>(xb + (mt * 32 + nl) * kRowBytes + hh * 16);
#pragma unroll
        for (int w = 0; w < kStageWords; ++w) {
#pragma unroll
          for (int t = 0; t < 2; ++t) {
            const int r = 4 * w + 2 * t + hh;
            h8 a[MT];
#pragma unroll
            for (int mt = 0; mt < MT; ++mt) a[mt] = anext[mt];
            if (2 * w + t + 1 < 2 * kStageWords) {
              const int rn = 2 * (2 * w + t + 1) + hh;
#pragma unroll
              for (int mt = 0; mt < MT; ++mt)
                anext[mt] = *reinterpret_cast<const h8*>(xb + (mt * 32 + nl) * kRowBytes + rn * 16);
            }
            if constexpr (MODE == kModeMerge) {
              const h8 b = expand_merge(~cur[0][w] ^ msgn, ~cur[1][w], t, hh, mbase, mg1);
#pragma unroll
              for (int mt = 0; mt < MT; ++mt)
                acc[0][mt] = __builtin_amdgcn_mfma_f32_32x32x16_f16(a[mt], b, acc[0][mt], 0, 0, 0);
              continue;
            }
#pragma unroll
            for (int p = 0; p < KP; ++p) {
              u32x4g bp = base[p];
              if (MODE == kModeH) bp = *reinterpret_cast<const u32x4g*>(hb + 256 * p + r * 16);
              const uint32_t nwd = ~cur[p][w] ^ gsgn[p];
              const h8 b = expand_b<MODE>(nwd, t, hh, bp);
              const int q = MODE == kModeH ? p : 0;  // fold and ones modes: one sum
#pragma unroll
              for (int mt = 0; mt < MT; ++mt)
                acc[q][mt] = __builtin_amdgcn_mfma_f32_32x32x16_f16(a[mt], b, acc[q][mt], 0, 0, 0);
            }
          }
        }
        __builtin_amdgcn_sched_barrier(0);
        store_x_stage<MT>(xq[(d + 1) % XD], (d & 1) ? xbuf0 : xbuf1, tid);
        if (MODE == kModeH) {
#pragma unroll
          for (int q = 0; q < NH; ++q) store_h_stage(hq[(d + 1) % XD][q], ((d & 1) ? hbuf0 : hbuf1) + 256 * q, tid);
        }
        __syncthreads();
      }
    }

    if (MODE == kModeFold) {
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) yacc[mt] = acc[0][mt];
    } else if (MODE == kModeMerge) {
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) yacc[mt] = acc[0][mt] * mscale;
    } else {
#pragma unroll
      for (int q = 0; q < NH; ++q) {  // planes in order, as one pass per plane would add them
        const float gi = scale_f32<TS>(g + (int64_t)(i0 + q) * N + nc);
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) yacc[mt] += gi * acc[q][mt];
      }
    }
  }

  // groups 1 .. NG-1 hand their sums to group 0 through LDS (the stage loop ended on a
  // barrier, so the activation buffers are free); group 0 adds them in group order and stores
  float* const ex = reinterpret_cast<float*>(smem);
  if (NG > 1 && !MSPLIT && grp > 0) {
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
      for (int j = 0; j < 16; ++j) ex[((((grp - 1) * kGemmWaves + wave) * MT + mt) * 16 + j) * 64 + lane] = yacc[mt][j];
  }
  if (NG > 1 && !MSPLIT) {
    __syncthreads();
    if (grp > 0) return;
#pragma unroll
    for (int gq = 1; gq < NG; ++gq)
#pragma unroll
      for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int j = 0; j < 16; ++j)
          yacc[mt][j] += ex[((((gq - 1) * kGemmWaves + wave) * MT + mt) * 16 + j) * 64 + lane];
  }

  // D of the 32x32 MFMA: lane l holds column n = l % 32 of the tile, element j holds
  // batch row 8 (j / 4) + 4 (l / 32) + j % 4
  if (n < N) {
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
#pragma unroll
      for (int j = 0; j < 16; ++j) {
        const int64_t m = m_base + mt * 32 + 8 * (j >> 2) + 4 * hh + (j & 3);
        if (m < M) {
          if (part)
            part[((int64_t)blockIdx.z * M + m) * N + n] = yacc[mt][j];
          else
            gemm_store<TY>(&y[m * N + n], yacc[mt][j]);
        }
      }
    }
  }
}

// y[m][n] = sum over the z chunks of part[z][m][n], in chunk order. Block (x, m) takes the
// 128 rows of tile x in batch row m; gridDim.x is the product kernel's padded x extent (a
// multiple of 8), so the block runs on the XCD whose L2 holds that tile's partials. All nz
// (<= kMaxChunks) loads are issued before the first add, so their latencies overlap.
constexpr int kMaxChunks = 16;
template <typename TY>
__global__ __launch_bounds__(kGemmTileN) void gemm_reduce_kernel(const float* __restrict__ part, int64_t N, int64_t M,
                                                                 int nz, TY* __restrict__ y) {
  const int64_t n = (int64_t)blockIdx.x * kGemmTileN + threadIdx.x;
  if (n >= N) return;
  const int64_t MN = M * N;
  const int64_t e = (int64_t)blockIdx.y * N + n;
  float v[kMaxChunks];
#pragma unroll
  for (int z = 0; z < kMaxChunks; ++z) v[z] = z < nz ? part[(int64_t)z * MN + e] : 0.0f;
  float s = 0.0f;
#pragma unroll
  for (int z = 0; z < kMaxChunks; ++z)
    if (z < nz) s += v[z];
  gemm_store<TY>(&y[e], s);
}

// batch rows per block for M (as launch_mt picks the tiles)
int64_t gemm_m_per_block(int64_t M, int mode_h) {
  if (M <= 32) return 32;
  if (M <= 64) return 64;
  if (M <= 128 || mode_h) return 128;
  return 256;
}

// K chunks per (row tile, batch tile): enough blocks for about one per compute unit (256),
// each chunk at least 8 stages (1024 columns) long; 1 when the tiles alone fill the part.
// (Measured on 4096 x 11008: two blocks per unit with 512-column chunks, or at most 4 chunks
// from M = 128 on, were both slower at every M.)
int gemm_k_split(int64_t N, int64_t K, int64_t M, int mode_h) {
  const int64_t tiles = ((N + kGemmTileN - 1) / kGemmTileN) * ((M + gemm_m_per_block(M, mode_h) - 1) /
                                                              gemm_m_per_block(M, mode_h));
  if (tiles >= 192) return 1;
  int64_t z = (256 + tiles - 1) / tiles;
  const int64_t zmax = K / (8 * kStageCols);
  if (z > zmax) z = zmax;
  if (z > kMaxChunks) z = kMaxChunks;
  return z < 1 ? 1 : (int)z;
}

// chunk width for z chunks: a whole number of stages
int64_t gemm_k_chunk(int64_t K, int z) {
  const int64_t stages = (K + kStageCols - 1) / kStageCols;
  return ((stages + z - 1) / z) * kStageCols;
}

// Fewer chunks when the grid would not spread evenly: blocks beyond `slots` (the compute
// units) put a second block on some units, which then finish last, so the count with the
// smallest ceil(blocks / slots) / z wins (86 row tiles: 3 chunks make 258 blocks, two on two
// units; 2 chunks make 172 blocks, one per unit). Measured on 11008x4096, k = 2, M = 4 / 16:
// 18.1 / 19.6 us with 3 chunks (two blocks fit a unit at once), 14.4 / 15.3 us with 2. Never
// more than z0, which sizes the workspace.
int gemm_fit_split(int z0, int64_t tiles, int64_t slots) {
  if (slots < 1) slots = 1;
  int best = z0;
  double best_cost = (double)((tiles * z0 + slots - 1) / slots) / z0;
  for (int z = z0 - 1; z >= 1; --z) {
    const double c = (double)((tiles * z + slots - 1) / slots) / z;
    if (c < best_cost) { best = z; best_cost = c; }
  }
  return best;
}

template <int MT, int NG, int NH>
constexpr size_t gemm_lds_bytes() {
  return (size_t)NG * (2 * MT * 32 * kRowBytes + 512 * NH);
}

template <typename TS, typename TY, int MT, int MODE, int KP, int NG, bool MSPLIT>
hipError_t launch_one(const uint32_t* planes, int64_t ldp, const void* g, const void* h, int k, int64_t N,
                      int64_t K, const void* x, int64_t M, void* y, float* ws, hipStream_t s) {
  constexpr size_t lds = gemm_lds_bytes<MT, NG, MODE == kModeH ? KP : 1>();
  static bool attr_set = false;  // per instantiation
  if (!attr_set) {
    const void* fn = (const void*)gemm_small_kernel<TS, TY, MT, MODE, KP, NG, MSPLIT>;
    const hipError_t e = hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return e;
    attr_set = true;
  }
  const int64_t m_per_block = (int64_t)32 * MT * (MSPLIT ? NG : 1);
  const unsigned gx = (unsigned)((N + kGemmTileN - 1) / kGemmTileN);
  const unsigned gy = (unsigned)((M + m_per_block - 1) / m_per_block);
  int nz = gemm_k_split(N, K, M, MODE == kModeH);
  if (nz > 1) nz = gemm_fit_split(nz, (int64_t)gx * gy, (int64_t)device_cu_count());
  const int64_t kz = nz > 1 ? gemm_k_chunk(K, nz) : K;
  float* part = nz > 1 ? ws : nullptr;
  const unsigned gxp = nz > 1 ? (gx + 7u) / 8u * 8u : gx;  // K split: x extent padded to whole XCD rounds
  gemm_small_kernel<TS, TY, MT, MODE, KP, NG, MSPLIT><<<dim3(gxp, gy, (unsigned)nz), kGemmGroupThreads * NG, lds, s>>>(
      planes, ldp, static_cast<const TS*>(g), static_cast<const __half*>(h), k, N, K,
      static_cast<const __half*>(x), M, static_cast<TY*>(y), kz, part);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || nz == 1) return e;
  gemm_reduce_kernel<TY><<<dim3(gxp, (unsigned)M), kGemmTileN, 0, s>>>(part, N, M, nz, static_cast<TY*>(y));
  return hipGetLastError();
}

// Batch tiles per wave and the wave groups: up to 64 batch rows the two groups split K (two
// waves per SIMD on a grid of N / 128 blocks); beyond, they split the block's batch rows
// (64 or 128 each), which keeps the grid at one block per 128 weight rows and 256 batch
// rows. (One group with 8 tiles per wave, so each expanded operand feeds 8 MFMAs, measured
// slower at M = 256: one wave per SIMD hides less than the halved expansion work saves.)
template <typename TS, typename TY, int MODE, int KP>
hipError_t launch_mt(const uint32_t* planes, int64_t ldp, const void* g, const void* h, int k, int64_t N,
                     int64_t K, const void* x, int64_t M, void* y, float* ws, hipStream_t s) {
  if (M <= 32) return launch_one<TS, TY, 1, MODE, KP, 2, false>(planes, ldp, g, h, k, N, K, x, M, y, ws, s);
  if (M <= 64) return launch_one<TS, TY, 2, MODE, KP, 2, false>(planes, ldp, g, h, k, N, K, x, M, y, ws, s);
  // h mode stages h as well and keeps at most two batch tiles (four would spill registers)
  if (M <= 128 || MODE == kModeH) return launch_one<TS, TY, 2, MODE, KP, 2, true>(planes, ldp, g, h, k, N, K, x, M, y, ws, s);
  if constexpr (MODE != kModeH) return launch_one<TS, TY, 4, MODE, KP, 2, true>(planes, ldp, g, h, k, N, K, x, M, y, ws, s);
  return hipErrorNotSupported;
}

template <typename TY>
hipError_t launch_y(rb_dtype scale_dtype, const uint32_t* planes, int64_t ldp, const void* g, const void* h,
                    int k, int64_t N, int64_t K, const void* x, int64_t M, void* y, float* ws, hipStream_t s) {
  // h mode, one 32-row batch tile, even k: two planes per sweep of K (the activation stages and
  // the start-up shared), each with its own accumulator
  if (h != nullptr && M <= 32 && k % 2 == 0)
    return launch_one<__half, TY, 1, kModeH, 2, 2, false>(planes, ldp, g, h, k, N, K, x, M, y, ws, s);
  if (h != nullptr) return launch_mt<__half, TY, kModeH, 1>(planes, ldp, g, h, k, N, K, x, M, y, ws, s);
  if (scale_dtype == RB_F32) return launch_mt<float, TY, kModeOnes, 1>(planes, ldp, g, h, k, N, K, x, M, y, ws, s);
  switch (k) {
    case 1: return launch_mt<__half, TY, kModeFold, 1>(planes, ldp, g, h, k, N, K, x, M, y, ws, s);
    case 2:
      // two or more batch tiles: both planes in one MFMA operand (one MFMA per step instead of
      // two; measured faster where each operand feeds several tiles)
      if (M > 32) return launch_mt<__half, TY, kModeMerge, 2>(planes, ldp, g, h, k, N, K, x, M, y, ws, s);
      return launch_mt<__half, TY, kModeFold, 2>(planes, ldp, g, h, k, N, K, x, M, y, ws, s);
    case 3: return launch_mt<__half, TY, kModeFold, 3>(planes, ldp, g, h, k, N, K, x, M, y, ws, s);
    default: return launch_mt<__half, TY, kModeFold, 4>(planes, ldp, g, h, k, N, K, x, M, y, ws, s);
  }
}

}  // namespace

// the K-split partial sums (fp32 [z][M][N]) when the tiles alone would leave compute units idle
size_t gemm_small_workspace_bytes(int, int64_t N, int64_t K, int64_t M) {
  const int nz = gemm_k_split(N, K, M, 0) > gemm_k_split(N, K, M, 1) ? gemm_k_split(N, K, M, 0)
                                                                       : gemm_k_split(N, K, M, 1);
  return nz > 1 ? (size_t)nz * (size_t)M * (size_t)N * sizeof(float) : 0u;
}

hipError_t launch_gemm_small(const uint32_t* planes, int64_t ldp, const void* g, const void* h,
                             rb_dtype scale_dtype, int k, int64_t N, int64_t K, const void* x, int64_t M,
                             void* y, rb_dtype y_dtype, void* ws, hipStream_t s) {
  float* wsf = static_cast<float*>(ws);
  if (y_dtype == RB_F16) return launch_y<__half>(scale_dtype, planes, ldp, g, h, k, N, K, x, M, y, wsf, s);
  return launch_y<float>(scale_dtype, planes, ldp, g, h, k, N, K, x, M, y, wsf, s);
}

}  // namespace rb
