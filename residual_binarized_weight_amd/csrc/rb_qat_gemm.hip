// rb_qat_gemm.hip -- the coupled-training layer's forward product on the matrix cores.
//
// [RaBiT, "Method step details", Algorithm 2] the layer multiplies its input by the effective
// weight re-derived from the shared full-precision weight on every forward: Y = X What^T,
// X [M][K] and What [N][K] in fp16 or bf16 (both K-contiguous), fp32 accumulation, Y in fp32
// or the operand type.
//
// Tiles. A block is 8 waves (two per SIMD, so one wave's LDS reads and barrier waits overlap
// the other's MFMAs) and owns a 128 (batch rows) x 256 (weight rows) tile of Y; wave w owns
// rows 64 (w & 1) .. +63 of the batch tile and 64 (w >> 1) .. +63 of the weight tile, i.e.
// 2 x 2 output tiles of 32 x 32 (v_mfma_f32_32x32x16_{bf16,f16}, 4 accumulators of 16 fp32
// per lane). K advances in tiles of 32 columns held in a ring of 6 LDS stages (24 KB
// each: the 128 x 32 slice of X, then the 256 x 32 slice of What). The stages are filled by
// direct-to-LDS buffer loads (16 bytes per lane, 1 KB per wave instruction = 16 rows of 64
// bytes), issued 5 tiles ahead of the multiplication: a wave waits only for its own loads of
// the tile it is about to read (vmcnt), then one barrier per tile makes every wave's loads
// visible and frees the stage of the tile before. Each tile's fragments are read from LDS one
// tile ahead of its MFMAs; every fragment read feeds 2 MFMAs.
//
// Stage layout: row r takes 64 bytes, its 16-byte chunk c (columns 8c .. 8c+7) in slot
// c ^ f(r), f(r) = ((r >> 1) ^ (r >> 3)) & 3, which spreads the rows of a fragment read over
// the bank groups.
//
// MFMA operand layout (32 x 32 x 16): lane l supplies row l % 32 of its operand at the 8
// consecutive columns 8 (l / 32) .. +7 of the 16-column step; D lane l holds output column
// l % 32 (a weight row) and, in element j, batch row 8 (j / 4) + 4 (l / 32) + j % 4.
//
// Grid. Consecutive blocks go to consecutive XCDs; tile indices are dealt so that XCD x owns
// one contiguous run of them, weight-row tile major, so the blocks of an XCD share What rows
// (and all of X) through that XCD's L2.
#include "rb_device.hpp"
#include "rb_internal.h"

namespace rb {
namespace {

typedef _Float16 q_h8 __attribute__((ext_vector_type(8)));
typedef __bf16 q_b8 __attribute__((ext_vector_type(8)));
typedef float q_f16x __attribute__((ext_vector_type(16)));
typedef uint32_t q_u4 __attribute__((ext_vector_type(4)));

constexpr int kQM = 128;                  // batch rows per block
constexpr int kQN = 256;                  // weight rows per block
constexpr int kQK = 32;                   // columns per K tile
constexpr int kQRowB = kQK * 2;           // bytes per staged row
constexpr int kQABytes = kQM * kQRowB;    // X slice: 8 KB
constexpr int kQStage = kQABytes + kQN * kQRowB;  // + What slice: 24 KB
constexpr int kQStages = 6;               // ring depth: 144 KB of LDS
constexpr int kQLead = kQStages - 1;      // tiles loaded ahead
constexpr int kQThreads = 512;
constexpr int kQGroups = kQStage / 1024;  // 1 KB load groups per tile: 24
constexpr int kQGroupsPerWave = kQGroups / (kQThreads / 64);  // 3
constexpr uint32_t kQOob = 0x80000000u;  // an offset past every resource below
constexpr int kQXcds = 8;

// s_waitcnt with vmcnt = n and the other counters left alone (gfx9 encoding: vmcnt in bits
// 3:0 and 15:14, expcnt 6:4, lgkmcnt 11:8)
constexpr int q_vmcnt(int n) { return (n & 15) | ((n >> 4) << 14) | (7 << 4) | (15 << 8); }
static_assert((kQLead - 1) * kQGroupsPerWave < 64, "vmcnt holds at most 63");
constexpr int q_lgkmcnt0 = 15 | (3 << 14) | (7 << 4);  // lgkmcnt = 0, the others left alone

template <bool BF16> struct QMfma;
template <> struct QMfma<true> {
  __device__ static __forceinline__ q_f16x run(q_u4 a, q_u4 b, q_f16x c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(q_b8, a), __builtin_bit_cast(q_b8, b), c, 0, 0, 0);
  }
};
template <> struct QMfma<false> {
  __device__ static __forceinline__ q_f16x run(q_u4 a, q_u4 b, q_f16x c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(q_h8, a), __builtin_bit_cast(q_h8, b), c, 0, 0, 0);
  }
};

template <typename TY, bool BF16> struct QStore;
template <bool BF16> struct QStore<float, BF16> {
  __device__ static __forceinline__ void put(float* p, float v) { *p = v; }
};
template <> struct QStore<uint16_t, true> {  // bf16, nearest even
  __device__ static __forceinline__ void put(uint16_t* p, float v) {
    *p = __bfloat16_as_ushort(__float2bfloat16(v));
  }
};
template <> struct QStore<uint16_t, false> {  // fp16, nearest even
  __device__ static __forceinline__ void put(uint16_t* p, float v) { *p = __half_as_ushort(__float2half_rn(v)); }
};

typedef __attribute__((address_space(3))) q_u4 q_lds_u4;
typedef __attribute__((address_space(3))) void q_lds_void;
__device__ __forceinline__ q_u4 q_lds_read(uint32_t addr) { return *(q_lds_u4*)(size_t)addr; }

// X [M][ldx], What [N][ldw] (element strides; both 16-byte aligned, strides multiples of 8,
// K a multiple of 32, M ldx and N ldw times 2 bytes below 2^31 -- checked by the launcher).
// Rows past M or N read as 0 through the buffer resources (and only meet outputs that are not
// stored); every staged chunk lies inside K.
template <bool BF16, typename TY>
__global__ __launch_bounds__(kQThreads) void qat_gemm_tn_kernel(const uint16_t* __restrict__ X, int64_t ldx,
                                                                const uint16_t* __restrict__ Wh, int64_t ldw,
                                                                int64_t M, int64_t N, int64_t K, TY* __restrict__ Y,
                                                                int64_t ldy, int64_t tiles_m, int64_t tiles,
                                                                int64_t per_xcd) {
  extern __shared__ __align__(16) uint8_t q_smem[];
  // tile indices as wave-uniform 32-bit values (the division is done in vector registers; read
  // back as scalars, the buffer resources built from them stay scalar)
  const uint32_t b = blockIdx.x;
  const uint32_t t = (b % kQXcds) * (uint32_t)per_xcd + b / kQXcds;  // this XCD's run of tiles
  if (t >= (uint32_t)tiles) return;  // uniform per block: grid padding
  const int64_t m0 = (int64_t)__builtin_amdgcn_readfirstlane(t % (uint32_t)tiles_m) * kQM;
  const int64_t n0 = (int64_t)__builtin_amdgcn_readfirstlane(t / (uint32_t)tiles_m) * kQN;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave & 1, wn = wave >> 1;  // wn 0..3
  const int lr = lane & 31, hh = lane >> 5;

  // buffer resources start at the block's first row; a row past M (N) lies past the end
  const int64_t ma = m0 < M ? M - m0 : 0, na = n0 < N ? N - n0 : 0;
  const __amdgpu_buffer_rsrc_t rx = buffer_rsrc(X + m0 * ldx, (uint32_t)(ma * ldx * 2));
  const __amdgpu_buffer_rsrc_t rw = buffer_rsrc(Wh + n0 * ldw, (uint32_t)(na * ldw * 2));

  // load group G = wave + 8 i of a tile (1 KB at LDS offset 1024 G): groups 0..7 are X rows
  // 16 G .. +15, groups 8..23 What rows 16 (G - 8) .. +15. Lane l fills slot l % 4 of row
  // l / 4 of the group with the chunk that belongs there: c = slot ^ f(row).
  auto swz = [](uint32_t r) { return ((r >> 1) ^ (r >> 3)) & 3u; };
  uint32_t goff[kQGroupsPerWave];
#pragma unroll
  for (int i = 0; i < kQGroupsPerWave; ++i) {
    const int G = wave + 8 * i;
    const uint32_t r = (uint32_t)(16 * (G < 8 ? G : G - 8) + (lane >> 2));
    goff[i] = (uint32_t)((int64_t)r * (G < 8 ? ldx : ldw) * 2 + ((lane & 3) ^ swz(r)) * 16);
  }
  auto dma = [&](int64_t tk) {  // tile tk into its stage; a tile past K loads nothing
    const bool live = tk * kQK < K;
    const uint32_t kb = (uint32_t)(tk * kQK * 2);
    uint8_t* const base = q_smem + (int)(tk % kQStages) * kQStage;
#pragma unroll
    for (int i = 0; i < kQGroupsPerWave; ++i) {
      const int G = wave + 8 * i;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(G < 8 ? rx : rw, (q_lds_void*)(base + G * 1024), 16,
                                               live ? goff[i] + kb : kQOob, 0, 0, 0);
    }
  };

  q_f16x acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) acc[i][j] = (q_f16x){};

  // fragment rows of the lane (f is the same for rows 32 apart)
  const uint32_t ra = (uint32_t)(wm * 64 + lr), rb = (uint32_t)(wn * 64 + lr);
  const uint32_t sa = swz(ra), sb = swz(rb);
  const uint32_t lds0 = (uint32_t)(size_t)(__attribute__((address_space(3))) uint8_t*)q_smem;
  // two fragment sets: a tile's 2 steps of 16 columns, 2 X and 2 What fragments each
  q_u4 fr[2][2][4];
  auto read = [&](int p, int64_t tk) {  // all fragments of tile tk into set p
    const uint32_t st = lds0 + (uint32_t)((tk % kQStages) * kQStage);
#pragma unroll
    for (int s = 0; s < 2; ++s) {
      const uint32_t c = (uint32_t)(2 * s + hh);
#pragma unroll
      for (int i = 0; i < 2; ++i) fr[p][s][i] = q_lds_read(st + (ra + 32u * i) * kQRowB + 16u * (c ^ sa));
#pragma unroll
      for (int j = 0; j < 2; ++j) fr[p][s][2 + j] = q_lds_read(st + kQABytes + (rb + 32u * j) * kQRowB + 16u * (c ^ sb));
    }
  };

  // Trip kt: a wave's own loads of tile kt + 1 have landed once at most those of the
  // kQLead - 2 tiles after it are in flight; the barrier after that wait covers every wave's
  // loads, and every wave is then done with tile kt - 1, whose stage takes the loads of tile
  // kt + kQLead. (The raw barrier: with __syncthreads the compiler would also wait for every
  // load in flight.) Tile kt + 1's fragments are read while tile kt's 16 MFMAs run.
  const int64_t ntile = K / kQK;
#pragma unroll
  for (int j = 0; j < kQLead; ++j) dma(j);
  __builtin_amdgcn_s_waitcnt(q_vmcnt((kQLead - 1) * kQGroupsPerWave));  // tile 0
  __builtin_amdgcn_s_barrier();
  read(0, 0);
  __builtin_amdgcn_s_waitcnt(q_lgkmcnt0);  // as at the end of each pair of trips below
  auto trip = [&](int p, int64_t kt) {
    __builtin_amdgcn_s_waitcnt(q_vmcnt((kQLead - 2) * kQGroupsPerWave));
    __builtin_amdgcn_s_barrier();
    dma(kt + kQLead);
    // unconditional (after the last tile it reads a stage of no use): under a branch the
    // compiler would wait for these reads before the MFMAs below
    read(p ^ 1, kt + 1);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int s = 0; s < 2; ++s)
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j) acc[i][j] = QMfma<BF16>::run(fr[p][s][i], fr[p][s][2 + j], acc[i][j]);
    __builtin_amdgcn_sched_barrier(0);
  };
  // pairs of trips with no branch inside, then the last odd one
  int64_t kt = 0;
  for (; kt + 2 <= ntile; kt += 2) {
    trip(0, kt);
    trip(1, kt + 1);
    // set 0's reads (issued before trip kt + 1's MFMAs) are done by now; saying so here keeps
    // the compiler, which cannot count LDS reads across the loop's back edge, from waiting for
    // the next trip's fresh reads before its MFMAs
    __builtin_amdgcn_s_waitcnt(q_lgkmcnt0);
  }
  if (kt < ntile) trip(0, kt);
  // the loads past the last tile (out of range, issued to keep the counts uniform) end before
  // the block does, so none writes LDS the next block on this compute unit may hold
  __builtin_amdgcn_s_waitcnt(q_vmcnt(0));

  // D: lane column lr is weight row n, element e batch row 8 (e / 4) + 4 hh + e % 4
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int64_t n = n0 + wn * 64 + j * 32 + lr;
    if (n >= N) continue;
#pragma unroll
    for (int i = 0; i < 2; ++i) {
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const int64_t m = m0 + wm * 64 + i * 32 + 8 * (e >> 2) + 4 * hh + (e & 3);
        if (m < M) QStore<TY, BF16>::put(Y + m * ldy + n, acc[i][j][e]);
      }
    }
  }
}

template <bool BF16, typename TY>
hipError_t launch_tn(const void* X, int64_t ldx, const void* Wh, int64_t ldw, int64_t M, int64_t N, int64_t K,
                     void* Y, int64_t ldy, hipStream_t s) {
  constexpr size_t lds = (size_t)kQStages * kQStage;
  static bool attr_set = false;  // per instantiation
  if (!attr_set) {
    const hipError_t e = hipFuncSetAttribute((const void*)qat_gemm_tn_kernel<BF16, TY>,
                                             hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return e;
    attr_set = true;
  }
  const int64_t tiles_m = (M + kQM - 1) / kQM;
  const int64_t tiles = tiles_m * ((N + kQN - 1) / kQN);
  const int64_t per_xcd = (tiles + kQXcds - 1) / kQXcds;
  const int64_t grid = per_xcd * kQXcds;
  if (grid > 0x7fffffff) return hipErrorInvalidConfiguration;  // tile indices are 32-bit
  qat_gemm_tn_kernel<BF16, TY><<<dim3((uint32_t)grid), kQThreads, lds, s>>>(
      static_cast<const uint16_t*>(X), ldx, static_cast<const uint16_t*>(Wh), ldw, M, N, K, static_cast<TY*>(Y), ldy,
      tiles_m, tiles, per_xcd);
  return hipGetLastError();
}

}  // namespace

bool qat_gemm_tn_supported(const void* X, int64_t ldx, const void* Wh, int64_t ldw, int64_t M, int64_t N, int64_t K) {
  const auto a16 = [](const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; };
  if (!a16(X) || !a16(Wh) || ldx % 8 != 0 || ldw % 8 != 0 || K % kQK != 0) return false;
  // 32-bit buffer offsets: each operand's rows (and one chunk past the last column) must stay
  // below 2^31 bytes, the out-of-range marker
  return M * ldx * 2 < (int64_t(1) << 31) && N * ldw * 2 < (int64_t(1) << 31);
}

hipError_t launch_qat_gemm_tn(const void* X, rb_dtype a_dtype, int64_t ldx, const void* Wh, int64_t ldw, int64_t M,
                              int64_t N, int64_t K, void* Y, rb_dtype y_dtype, int64_t ldy, hipStream_t s) {
  if (a_dtype == RB_BF16) {
    if (y_dtype == RB_F32) return launch_tn<true, float>(X, ldx, Wh, ldw, M, N, K, Y, ldy, s);
    return launch_tn<true, uint16_t>(X, ldx, Wh, ldw, M, N, K, Y, ldy, s);
  }
  if (y_dtype == RB_F32) return launch_tn<false, float>(X, ldx, Wh, ldw, M, N, K, Y, ldy, s);
  return launch_tn<false, uint16_t>(X, ldx, Wh, ldw, M, N, K, Y, ldy, s);
}

}  // namespace rb
