// rb_svid.hip -- function-aware initialization of the k residual paths (gfx950).
//
// [RaBiT, "Method step details", Algorithm 1]
//   W' = s_out^a_out (.) W (.) s_in^a_in   (I/O channel importance: rows by output, columns by
//                                           input importance)
//   T sweeps; in each, path i = 1..k in turn (Gauss-Seidel: the other paths at their latest
//   values): R_i = W' - sum_{j != i} g'_j (.) B_j (.) h'_j, B_i = sign(R_i) (0 -> +1), and
//   (g'_i, h'_i) the rank-1 fit of |R_i| (top singular pair, split evenly:
//   g' = sqrt(sigma) u, h' = sqrt(sigma) v). The paths start at zero, so the first sweep is
//   the greedy residual SVID. Finally g_i = g'_i / s_out^a_out, h_i = h'_i / s_in^a_in.
//
// The top singular pair comes from power iteration on |R_i|, which is never stored: every
// pass forms R_i from W and the other paths' sign planes and scales on the fly.
//   row pass     t = |R| v^        (one wave per row; v^ = v / ||v||)
//   column pass  p_b = |R|^T t     over a 64-row tile, its columns split over 16 blocks
//                                  (per-tile partial sums in the workspace)
//   reduce       v = sum_b p_b     (fixed order; partial sums of v^2 per 64 columns)
// P alternations of row + column pass, then a last row pass that also writes B_i's bits, and a
// finalize step: sigma = ||t||, g'_i = t / sqrt(sigma), h'_i = sqrt(sigma) v^. Each step warm-
// starts from the path's previous h'_i (ones in the first sweep). |R| is nonnegative and the
// start is positive, so the iteration stays in the positive cone and finds the Perron pair.
// Every sum has a fixed order, so the result is deterministic. Arithmetic is fp32.
//
// W is fp32, row-major with a row stride that is a multiple of 4 floats (16-byte rows): a lane
// handles 4 consecutive columns per step with one 16-byte load. Vectors over K live in the
// workspace padded with zeros to a multiple of 4, so columns past K contribute 0.
#include "rb_device.hpp"
#include "rb_internal.h"

namespace rb {
namespace {

typedef float svid_f32x4 __attribute__((ext_vector_type(4)));

constexpr int kSvidRowWaves = 4;   // rows per block of the row pass (one wave each)
constexpr int kSvidTileRows = 64;  // rows per tile of the column pass
constexpr int kSvidColSplit = 16;  // blocks per row tile of the column pass (each 1/16 of K)
constexpr int kSvidRedCols = 64;   // columns per block of the reduction (and per norm partial)
constexpr int kSvidRedGroups = 16; // tile groups per block of the reduction
constexpr int kSvidThreads = 256;
constexpr uint32_t kSvidOob = 0x80000000u;

struct SvidWs {
  float* fo;       // [N] s_out^a_out
  float* fi;       // [K4] s_in^a_in (0 past K)
  float* gp;       // [k][N] scaled-domain row scales
  float* hp;       // [k][K4] scaled-domain column scales (0 past K)
  float* t;        // [N] row-pass result
  float* v;        // [K4] power vector
  float* nrmv;     // [nvb] partial sums of v^2
  float* colpart;  // [ntile][K4] column-pass partial sums
};

__host__ __device__ inline int64_t svid_round4(int64_t K) { return (K + 3) & ~int64_t(3); }
__host__ __device__ inline int64_t svid_align64(int64_t n) { return (n + 63) & ~int64_t(63); }  // floats (256 B)

inline size_t svid_ws_floats(int k, int64_t N, int64_t K, SvidWs* w, float* base) {
  const int64_t K4 = svid_round4(K);
  const int64_t nvb = (K4 + kSvidRedCols - 1) / kSvidRedCols;
  const int64_t ntile = (N + kSvidTileRows - 1) / kSvidTileRows;
  int64_t off = 0;
  auto take = [&](int64_t n) {
    const int64_t o = off;
    off += svid_align64(n);
    return base ? base + o : nullptr;
  };
  SvidWs tmp;
  tmp.fo = take(N);
  tmp.fi = take(K4);
  tmp.gp = take((int64_t)k * svid_align64(N));
  tmp.hp = take((int64_t)k * svid_align64(K4));
  tmp.t = take(N);
  tmp.v = take(K4);
  tmp.nrmv = take(nvb);
  tmp.colpart = take(ntile * K4);
  if (w) *w = tmp;
  return (size_t)off;
}

// ||v||^2 from the per-block partial sums, in a fixed order (every wave gets the same value)
__device__ __forceinline__ float svid_norm2(const float* __restrict__ nrmv, int nvb) {
  float s = 0.0f;
  for (int b = 0; b < nvb; ++b) s += nrmv[b];
  return s;
}

// The 4 residual values of row n at columns 4q .. 4q+3:
//   R = fo_n W fi - sum_j g'_j[n] (b ? +h'_j : -h'_j), with g'_i taken as 0 for the fitted path
// (planes: [k][N][ldp] words; the 4 bits of the chunk are bits 4 (q % 8) .. +3 of word q / 8)
struct SvidOther {
  float g;
  svid_f32x4 h;
  uint32_t bits;
};

template <int KP>
__device__ __forceinline__ svid_f32x4 svid_residual(float fo_n, svid_f32x4 w, svid_f32x4 fi, const SvidOther (&o)[KP]) {
  svid_f32x4 r;
#pragma unroll
  for (int c = 0; c < 4; ++c) r[c] = fo_n * w[c] * fi[c];
#pragma unroll
  for (int j = 0; j < KP; ++j) {
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const float gh = o[j].g * o[j].h[c];
      r[c] -= ((o[j].bits >> c) & 1u) ? gh : -gh;
    }
  }
  return r;
}

__device__ __forceinline__ svid_f32x4 svid_ld4(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return __builtin_bit_cast(svid_f32x4, __builtin_amdgcn_raw_buffer_load_b128(r, (int)off, 0, 0));
}

// Row pass: t[n] = sum_k |R_nk| v^_k. With PACK, also B_i[n] = bits of (R >= 0).
template <int KP, bool PACK>
__global__ __launch_bounds__(kSvidThreads) void svid_row_kernel(const float* __restrict__ W, int64_t N, int64_t K,
                                                               int64_t ldw, int i, uint32_t* __restrict__ planes,
                                                               int64_t ldp, SvidWs ws, int nvb) {
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int64_t n = (int64_t)blockIdx.x * kSvidRowWaves + wave;
  if (n >= N) return;  // uniform per wave
  const int64_t K4 = svid_round4(K);
  const int64_t nq = K4 / 4;  // 4-column chunks
  const uint32_t Kw = (uint32_t)((K + 31) >> 5);
  const __amdgpu_buffer_rsrc_t rw = buffer_rsrc(W + n * ldw, (uint32_t)K * 4u);
  const __amdgpu_buffer_rsrc_t rfi = buffer_rsrc(ws.fi, (uint32_t)K4 * 4u);
  const __amdgpu_buffer_rsrc_t rv = buffer_rsrc(ws.v, (uint32_t)K4 * 4u);
  const float inv_nv = rsqrtf(svid_norm2(ws.nrmv, nvb));
  const float fo_n = ws.fo[n];
  // every path of this row; the path being fitted gets g = 0 (its own bits do not enter R)
  float og[KP];
  __amdgpu_buffer_rsrc_t rh[KP], rb[KP];
#pragma unroll
  for (int j = 0; j < KP; ++j) {
    og[j] = j == i ? 0.0f : ws.gp[(int64_t)j * svid_align64(N) + n];
    rh[j] = buffer_rsrc(ws.hp + (int64_t)j * svid_align64(K4), (uint32_t)K4 * 4u);
    rb[j] = buffer_rsrc(planes + ((int64_t)j * N + n) * ldp, Kw * 4u);
  }
  float acc = 0.0f;
#pragma unroll 8
  for (int64_t q0 = 0; q0 < nq; q0 += 64) {
    const int64_t q = q0 + lane;
    const bool in = q < nq;
    const uint32_t off = in ? (uint32_t)(q * 16) : kSvidOob;
    const uint32_t boff = in ? (uint32_t)(q >> 3) * 4u : kSvidOob;  // q < nq keeps q / 8 < Kw
    const svid_f32x4 w = svid_ld4(rw, off);
    const svid_f32x4 fi = svid_ld4(rfi, off);
    const svid_f32x4 v = svid_ld4(rv, off);
    SvidOther o[KP];
#pragma unroll
    for (int j = 0; j < KP; ++j) {
      o[j].g = og[j];
      o[j].h = svid_ld4(rh[j], off);
      o[j].bits = (buf_u32(rb[j], boff, 0u) >> (4u * (uint32_t)(q & 7))) & 15u;
    }
    const svid_f32x4 r = svid_residual(fo_n, w, fi, o);
#pragma unroll
    for (int c = 0; c < 4; ++c) acc += fabsf(r[c]) * (v[c] * inv_nv);
    if (PACK) {
      // nibble of this lane's 4 columns (columns past K give 0), then OR over the 8 lanes
      // of a word: lane 8 m holds word q0 / 8 + m
      uint32_t nib = 0u;
#pragma unroll
      for (int c = 0; c < 4; ++c) nib |= (r[c] >= 0.0f && 4 * q + c < K) ? (1u << c) : 0u;
      uint32_t word = in ? nib << (4u * (uint32_t)(lane & 7)) : 0u;
      word |= __shfl_xor(word, 1, 64);
      word |= __shfl_xor(word, 2, 64);
      word |= __shfl_xor(word, 4, 64);
      const uint32_t wi = (uint32_t)(q >> 3);
      if ((lane & 7) == 0 && in && wi < Kw) planes[((int64_t)i * N + n) * ldp + wi] = word;
    }
  }
  acc = wave_sum(acc);
  if (lane == 0) ws.t[n] = acc;
}

// Column pass over rows 16 b .. 16 b + 15: colpart[b][k] = sum_n |R_nk| t_n.
template <int KP>
__global__ __launch_bounds__(kSvidThreads) void svid_col_kernel(const float* __restrict__ W, int64_t N, int64_t K,
                                                               int64_t ldw, int i, const uint32_t* __restrict__ planes,
                                                               int64_t ldp, SvidWs ws) {
  const int64_t K4 = svid_round4(K);
  const int64_t nq = K4 / 4;
  const uint32_t Kw = (uint32_t)((K + 31) >> 5);
  const int64_t n0 = (int64_t)blockIdx.x * kSvidTileRows;
  const int rows = (int)((N - n0) < kSvidTileRows ? (N - n0) : kSvidTileRows);
  const __amdgpu_buffer_rsrc_t rfi = buffer_rsrc(ws.fi, (uint32_t)K4 * 4u);
  __amdgpu_buffer_rsrc_t rh[KP];
#pragma unroll
  for (int j = 0; j < KP; ++j) rh[j] = buffer_rsrc(ws.hp + (int64_t)j * svid_align64(K4), (uint32_t)K4 * 4u);
  // this block's share of the columns: chunk range blockIdx.y of kSvidColSplit
  const int64_t qper = (nq + kSvidColSplit - 1) / kSvidColSplit;
  const int64_t qend = (blockIdx.y + 1) * qper < nq ? (blockIdx.y + 1) * qper : nq;
  for (int64_t q = blockIdx.y * qper + threadIdx.x; q < qend; q += kSvidThreads) {
    const uint32_t off = (uint32_t)(q * 16);
    const uint32_t boff = (uint32_t)(q >> 3) * 4u;  // q < nq keeps q / 8 < Kw
    const uint32_t sh = 4u * (uint32_t)(q & 7);
    const svid_f32x4 fi = svid_ld4(rfi, off);
    svid_f32x4 hj[KP];
#pragma unroll
    for (int j = 0; j < KP; ++j) hj[j] = svid_ld4(rh[j], off);
    svid_f32x4 acc = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll 8
    for (int r = 0; r < rows; ++r) {
      const int64_t n = n0 + r;
      const svid_f32x4 w = svid_ld4(buffer_rsrc(W + n * ldw, (uint32_t)K * 4u), off);
      SvidOther o[KP];
#pragma unroll
      for (int j = 0; j < KP; ++j) {
        o[j].g = j == i ? 0.0f : ws.gp[(int64_t)j * svid_align64(N) + n];
        o[j].h = hj[j];
        o[j].bits = (buf_u32(buffer_rsrc(planes + ((int64_t)j * N + n) * ldp, Kw * 4u), boff, 0u) >> sh) & 15u;
      }
      const svid_f32x4 res = svid_residual(ws.fo[n], w, fi, o);
      const float tn = ws.t[n];
#pragma unroll
      for (int c = 0; c < 4; ++c) acc[c] += fabsf(res[c]) * tn;
    }
    *reinterpret_cast<svid_f32x4*>(ws.colpart + (int64_t)blockIdx.x * K4 + 4 * q) = acc;
  }
}

// v[k] = sum over tiles of colpart[b][k]: 16 groups of tiles summed in order, then the groups in
// order; nrmv[block] = sum of v^2 over the block's 64 columns (a fixed butterfly)
__global__ __launch_bounds__(kSvidRedCols * kSvidRedGroups) void svid_reduce_kernel(int64_t K4, int64_t ntile,
                                                                                    SvidWs ws) {
  __shared__ float part[kSvidRedGroups][kSvidRedCols];
  const int tx = threadIdx.x & (kSvidRedCols - 1), ty = threadIdx.x / kSvidRedCols;
  const int64_t k = (int64_t)blockIdx.x * kSvidRedCols + tx;
  const int64_t per = (ntile + kSvidRedGroups - 1) / kSvidRedGroups;
  const int64_t b0 = ty * per, b1 = (ty + 1) * per < ntile ? (ty + 1) * per : ntile;
  float s = 0.0f;
  if (k < K4)
    for (int64_t b = b0; b < b1; ++b) s += ws.colpart[b * K4 + k];
  part[ty][tx] = s;
  __syncthreads();
  if (ty == 0) {  // wave 0: one column per lane
    float v = 0.0f;
#pragma unroll
    for (int gq = 0; gq < kSvidRedGroups; ++gq) v += part[gq][tx];
    if (k < K4) ws.v[k] = v;
    const float s2 = wave_sum(k < K4 ? v * v : 0.0f);
    if (tx == 0) ws.nrmv[blockIdx.x] = s2;
  }
}

// start vector: ones over the K columns (first sweep) or the path's previous h'_i; nrmv as above
__global__ __launch_bounds__(kSvidRedCols) void svid_vinit_kernel(int64_t K, int i, int first, SvidWs ws) {
  const int64_t K4 = svid_round4(K);
  const int64_t k = (int64_t)blockIdx.x * kSvidRedCols + threadIdx.x;
  float s = 0.0f;
  if (k < K4) {
    s = first ? (k < K ? 1.0f : 0.0f) : ws.hp[(int64_t)i * svid_align64(K4) + k];
    ws.v[k] = s;
  }
  const float s2 = wave_sum(s * s);
  if (threadIdx.x == 0) ws.nrmv[blockIdx.x] = s2;
}

// sigma = ||t|| (every block sums all of t in the same order), g'_i = t / sqrt(sigma),
// h'_i = sqrt(sigma) v / ||v||
__global__ __launch_bounds__(kSvidThreads) void svid_finalize_kernel(int64_t N, int64_t K, int i, int nvb,
                                                                    SvidWs ws) {
  __shared__ float part[kSvidThreads / 64];
  float s = 0.0f;
  for (int64_t n = threadIdx.x; n < N; n += kSvidThreads) s += ws.t[n] * ws.t[n];
  s = wave_sum(s);
  if ((threadIdx.x & 63) == 0) part[threadIdx.x >> 6] = s;
  __syncthreads();
  float sig2 = 0.0f;
  for (int wv = 0; wv < kSvidThreads / 64; ++wv) sig2 += part[wv];
  const float sq = sqrtf(sqrtf(sig2));  // sqrt(sigma)
  const float inv_nv = rsqrtf(svid_norm2(ws.nrmv, nvb));
  const int64_t K4 = svid_round4(K);
  const int64_t e = (int64_t)blockIdx.x * kSvidThreads + threadIdx.x;
  if (e < N) ws.gp[(int64_t)i * svid_align64(N) + e] = sig2 > 0.0f ? ws.t[e] / sq : 0.0f;
  if (e < K4) ws.hp[(int64_t)i * svid_align64(K4) + e] = sig2 > 0.0f ? sq * ws.v[e] * inv_nv : 0.0f;
}

// fo, fi from the importance vectors; scaled-domain scales start at zero
__global__ __launch_bounds__(kSvidThreads) void svid_prep_kernel(int64_t N, int64_t K, int k,
                                                                const float* __restrict__ s_in,
                                                                const float* __restrict__ s_out, float a_in,
                                                                float a_out, SvidWs ws) {
  const int64_t K4 = svid_round4(K);
  const int64_t e = (int64_t)blockIdx.x * kSvidThreads + threadIdx.x;
  if (e < N) {
    ws.fo[e] = s_out ? powf(s_out[e], a_out) : 1.0f;
    for (int j = 0; j < k; ++j) ws.gp[(int64_t)j * svid_align64(N) + e] = 0.0f;
  }
  if (e < K4) {
    ws.fi[e] = e < K ? (s_in ? powf(s_in[e], a_in) : 1.0f) : 0.0f;
    for (int j = 0; j < k; ++j) ws.hp[(int64_t)j * svid_align64(K4) + e] = 0.0f;
  }
}

// g_i = g'_i / fo, h_i = h'_i / fi (the original domain)
__global__ __launch_bounds__(kSvidThreads) void svid_output_kernel(int64_t N, int64_t K, int k, float* __restrict__ g,
                                                                  float* __restrict__ h, SvidWs ws) {
  const int64_t K4 = svid_round4(K);
  const int64_t e = (int64_t)blockIdx.x * kSvidThreads + threadIdx.x;
  for (int j = 0; j < k; ++j) {
    if (e < N) g[(int64_t)j * N + e] = ws.gp[(int64_t)j * svid_align64(N) + e] / ws.fo[e];
    if (e < K) h[(int64_t)j * K + e] = ws.hp[(int64_t)j * svid_align64(K4) + e] / ws.fi[e];
  }
}

template <int KP>
hipError_t run_svid(const float* W, int64_t N, int64_t K, int64_t ldw, int T, int P, const float* s_in,
                    const float* s_out, float a_in, float a_out, uint32_t* planes, int64_t ldp, float* g,
                    float* h, void* wsp, hipStream_t s) {
  SvidWs ws;
  svid_ws_floats(KP, N, K, &ws, static_cast<float*>(wsp));
  const int64_t K4 = svid_round4(K);
  const int nvb = (int)((K4 + kSvidRedCols - 1) / kSvidRedCols);
  const int64_t ntile = (N + kSvidTileRows - 1) / kSvidTileRows;
  const int64_t nmax = N > K4 ? N : K4;
  const unsigned gvec = (unsigned)((nmax + kSvidThreads - 1) / kSvidThreads);
  const unsigned grow = (unsigned)((N + kSvidRowWaves - 1) / kSvidRowWaves);
  svid_prep_kernel<<<gvec, kSvidThreads, 0, s>>>(N, K, KP, s_in, s_out, a_in, a_out, ws);
  for (int t = 0; t < T; ++t) {
    for (int i = 0; i < KP; ++i) {
      svid_vinit_kernel<<<nvb, kSvidRedCols, 0, s>>>(K, i, t == 0, ws);
      for (int p = 0; p < P; ++p) {
        svid_row_kernel<KP, false><<<grow, kSvidThreads, 0, s>>>(W, N, K, ldw, i, planes, ldp, ws, nvb);
        svid_col_kernel<KP><<<dim3((unsigned)ntile, kSvidColSplit), kSvidThreads, 0, s>>>(W, N, K, ldw, i, planes,
                                                                                    ldp, ws);
        svid_reduce_kernel<<<nvb, kSvidRedCols * kSvidRedGroups, 0, s>>>(K4, ntile, ws);
      }
      svid_row_kernel<KP, true><<<grow, kSvidThreads, 0, s>>>(W, N, K, ldw, i, planes, ldp, ws, nvb);
      svid_finalize_kernel<<<gvec, kSvidThreads, 0, s>>>(N, K, i, nvb, ws);
    }
  }
  svid_output_kernel<<<gvec, kSvidThreads, 0, s>>>(N, K, KP, g, h, ws);
  return hipGetLastError();
}

}  // namespace

size_t svid_workspace_bytes(int k, int64_t N, int64_t K) { return svid_ws_floats(k, N, K, nullptr, nullptr) * 4; }

hipError_t launch_svid_init(const float* W, int64_t N, int64_t K, int64_t ldw, int k, int T, int P,
                            const float* s_in, const float* s_out, float a_in, float a_out, uint32_t* planes,
                            int64_t ldp, float* g, float* h, void* ws, hipStream_t s) {
  switch (k) {
    case 1: return run_svid<1>(W, N, K, ldw, T, P, s_in, s_out, a_in, a_out, planes, ldp, g, h, ws, s);
    case 2: return run_svid<2>(W, N, K, ldw, T, P, s_in, s_out, a_in, a_out, planes, ldp, g, h, ws, s);
    case 3: return run_svid<3>(W, N, K, ldw, T, P, s_in, s_out, a_in, a_out, planes, ldp, g, h, ws, s);
    default: return run_svid<4>(W, N, K, ldw, T, P, s_in, s_out, a_in, a_out, planes, ldp, g, h, ws, s);
  }
}

}  // namespace rb
