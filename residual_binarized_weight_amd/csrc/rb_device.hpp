// rb_device.hpp -- device helpers shared by the librb kernels (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <hip/hip_fp16.h>
#include <hip/hip_bf16.h>
#include <stdint.h>

#define RB_WAVE 64

namespace rb {

// ---------------------------------------------------------------------------
// element loads: every supported storage type widened exactly
// ---------------------------------------------------------------------------
__device__ __forceinline__ float to_f32(float v) { return v; }
__device__ __forceinline__ float to_f32(__half v) { return __half2float(v); }
__device__ __forceinline__ float to_f32(__hip_bfloat16 v) { return __bfloat162float(v); }

// raw sign-bit test: true for +0.0, -0.0 and every value >= 0 (so sign(0) = +1),
// independent of any denormal flushing of the arithmetic.
__device__ __forceinline__ bool nonneg_bits(float v) {
  uint32_t b = __float_as_uint(v);
  return (b >> 31) == 0u || (b & 0x7fffffffu) == 0u;
}

// ---------------------------------------------------------------------------
// round a double to the nearest fp16 (ties to even), directly (no double rounding
// through fp32). Only exact operations (scaling by powers of two) and rint() in the
// default round-to-nearest-even mode are used.
// ---------------------------------------------------------------------------
__device__ __forceinline__ uint16_t f64_to_f16_bits_rne(double d) {
  const uint16_t sgn = (uint16_t)((__double_as_longlong(d) >> 48) & 0x8000);
  const double a = fabs(d);
  if (a != a) return (uint16_t)(sgn | 0x7e00);
  if (a >= 65520.0) return (uint16_t)(sgn | 0x7c00);           // 65504 + half an ulp and up -> inf
  if (a < 6.103515625e-05) {                                     // below 2^-14: subnormal grid 2^-24
    const double m = rint(a * 16777216.0);                       // m <= 1024 (1024 = smallest normal)
    return (uint16_t)(sgn | (uint16_t)m);
  }
  int e;
  (void)frexp(a, &e);                                            // a = f * 2^e, f in [0.5, 1)
  int E = e - 1;                                                 // 2^E <= a < 2^(E+1), -14 <= E <= 15
  double m = rint(ldexp(a, 10 - E));                             // in [1024, 2048]
  if (m == 2048.0) { m = 1024.0; E += 1; }
  return (uint16_t)(sgn | (uint16_t)((E + 15) << 10) | (uint16_t)(m - 1024.0));
}

__device__ __forceinline__ double f16_bits_to_f64(uint16_t b) {
  return (double)__half2float(__ushort_as_half(b));
}

// round a double to the scale storage type; returns the stored value widened back to double.
template <typename TS> struct ScaleRound;
template <> struct ScaleRound<__half> {
  __device__ static __forceinline__ double store(__half* p, double v) {
    const uint16_t b = f64_to_f16_bits_rne(v);
    *reinterpret_cast<uint16_t*>(p) = b;
    return f16_bits_to_f64(b);
  }
};
template <> struct ScaleRound<float> {
  __device__ static __forceinline__ double store(float* p, double v) {
    const float f = __double2float_rn(v);
    *p = f;
    return (double)f;
  }
};

// ---------------------------------------------------------------------------
// wave-wide butterfly sums. Each stage adds a lane's value to its partner's; IEEE
// addition is commutative, so every lane ends with the bit-identical total and the
// order is fixed (deterministic run to run).
// ---------------------------------------------------------------------------
__device__ __forceinline__ double wave_sum(double v) {
#pragma unroll
  for (int s = 32; s >= 1; s >>= 1) v += __shfl_xor(v, s, RB_WAVE);
  return v;
}
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int s = 32; s >= 1; s >>= 1) v += __shfl_xor(v, s, RB_WAVE);
  return v;
}
// sum over aligned groups of `width` lanes (width a power of two <= 64)
__device__ __forceinline__ double group_sum(double v, int width) {
  for (int s = width >> 1; s >= 1; s >>= 1) v += __shfl_xor(v, s, RB_WAVE);
  return v;
}

// ---------------------------------------------------------------------------
// buffer loads, absolute LDS reads and DPP reductions
// ---------------------------------------------------------------------------
// Raw buffer resource over [base, base + bytes): loads through it take a 32-bit byte offset
// (per-lane VGPR + uniform SGPR/immediate part, no 64-bit address math) and return 0 past
// the end instead of faulting.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t buffer_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
}
__device__ __forceinline__ uint32_t buf_u32(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff) {
  return __builtin_amdgcn_raw_buffer_load_b32(r, (int)voff, (int)soff, 0);
}
__device__ __forceinline__ uint32_t buf_u16(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff) {
  return (uint32_t)__builtin_amdgcn_raw_buffer_load_b16(r, (int)voff, (int)soff, 0);
}
// LDS read at an absolute LDS byte address. A kernel that declares no static LDS has its
// dynamic LDS at address 0, so a computed table offset is usable as the address itself.
typedef __attribute__((address_space(3))) const float lds_cf32;
__device__ __forceinline__ float lds_f32(uint32_t byte_addr) {
  return *(lds_cf32*)(size_t)byte_addr;
}

// sum over each 32-lane half of the wave; the total lands in lanes 16..31 and 48..63
__device__ __forceinline__ float half_wave_sum(float v) {
  v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0xB1, 0xF, 0xF, false));   // quad [1,0,3,2]
  v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x4E, 0xF, 0xF, false));   // quad [2,3,0,1]
  v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x141, 0xF, 0xF, false));  // row_half_mirror
  v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x140, 0xF, 0xF, false));  // row_mirror
  v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x142, 0xA, 0xF, false));  // row_bcast:15
  return v;
}

// sum over the whole wave; the total lands in lane 63
__device__ __forceinline__ float wave_sum_dpp(float v) {
  v = half_wave_sum(v);  // lanes 16..31 and 48..63 hold the two half sums
  v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x143, 0x8, 0xF, false));  // row_bcast:31
  return v;
}

}  // namespace rb
