// rb_api.cpp -- C ABI of librb: host-side validation, then one enqueue per call.
//
// Every check below runs before any HIP call, so an invalid call returns its status
// without touching the device (and can be tested on a machine with no GPU).
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>
#include <cstdio>
#include <cstdlib>

#include "../../include/rb.h"
#include "rb_internal.h"

namespace {

bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }

bool valid_dtype(rb_dtype d) { return d == RB_F32 || d == RB_F16 || d == RB_BF16; }

bool is_pow2_in(int32_t v, int32_t lo, int32_t hi) {
  return v >= lo && v <= hi && (v & (v - 1)) == 0;
}

constexpr int64_t kMaxDim = (int64_t(1) << 31) - 1;
constexpr int64_t kQatMaxDim = int64_t(1) << 28;  // N and K of the training layer (32-bit byte offsets)

bool act_dtype(rb_dtype d) { return d == RB_F16 || d == RB_BF16; }
bool elem_aligned(const void* p, rb_dtype d) { return aligned(p, d == RB_F32 ? 4 : 2); }

// shapes shared by the training-layer calls
rb_status check_qat_layer(int64_t N, int64_t K, int32_t k, const float* g, const float* h,
                          const uint32_t* planes, int64_t ldp, const void* What, int64_t ldwh, rb_dtype a_dtype) {
  if (!g || !h || !planes || !What) return RB_ERR_INVALID_ARG;
  if (k < 1 || k > 4 || N < 1 || K < 1 || N > kQatMaxDim || K > kQatMaxDim) return RB_ERR_INVALID_ARG;
  if (ldp < (K + 31) / 32 || ldwh < K || ldwh > kMaxDim) return RB_ERR_INVALID_ARG;
  if (!valid_dtype(a_dtype)) return RB_ERR_INVALID_ARG;
  if (!act_dtype(a_dtype)) return RB_ERR_UNSUPPORTED;
  if (!aligned(g, 4) || !aligned(h, 4) || !aligned(planes, 4) || !elem_aligned(What, a_dtype))
    return RB_ERR_MISALIGNED;
  return RB_OK;
}

rb_status from_hip(hipError_t e) {
  if (e == hipSuccess) return RB_OK;
  if (std::getenv("RB_LOG")) std::fprintf(stderr, "librb: launch failed: %s\n", hipGetErrorString(e));
  return RB_ERR_HIP;
}

void log_call(const char* what, int64_t N, int64_t K, int64_t M, int k) {
  if (std::getenv("RB_LOG")) std::fprintf(stderr, "librb: %s N=%lld K=%lld M=%lld k=%d\n", what,
                                          (long long)N, (long long)K, (long long)M, k);
}

rb_status check_product_args(const uint32_t* planes, int64_t ldp, const void* g, rb_dtype scale_dtype,
                             int32_t k, int64_t N, int64_t K, const void* x, rb_dtype x_dtype,
                             int64_t M, void* y, rb_dtype y_dtype, int64_t max_m) {
  if (!planes || !g || !x || !y) return RB_ERR_INVALID_ARG;
  if (k < 1 || k > 4) return RB_ERR_INVALID_ARG;
  if (N < 1 || K < 1 || N > kMaxDim || K > kMaxDim) return RB_ERR_INVALID_ARG;
  if (M < 1) return RB_ERR_INVALID_ARG;
  if (ldp < (K + 31) / 32) return RB_ERR_INVALID_ARG;
  if (!valid_dtype(scale_dtype) || !valid_dtype(x_dtype) || !valid_dtype(y_dtype)) return RB_ERR_INVALID_ARG;
  if (scale_dtype == RB_BF16 || x_dtype == RB_BF16 || y_dtype == RB_BF16) return RB_ERR_UNSUPPORTED;
  if (M > max_m) return RB_ERR_UNSUPPORTED;
  if (!aligned(planes, 16) || !aligned(x, 16) || !aligned(y, 16)) return RB_ERR_MISALIGNED;
  if (!aligned(g, scale_dtype == RB_F32 ? 4 : 2)) return RB_ERR_MISALIGNED;
  return RB_OK;
}

}  // namespace

extern "C" {

int rb_version(void) { return 100; }

const char* rb_status_string(rb_status s) {
  switch (s) {
    case RB_OK: return "RB_OK";
    case RB_ERR_INVALID_ARG: return "RB_ERR_INVALID_ARG: an argument is out of range or NULL";
    case RB_ERR_UNSUPPORTED: return "RB_ERR_UNSUPPORTED: valid arguments this build does not implement";
    case RB_ERR_MISALIGNED: return "RB_ERR_MISALIGNED: a pointer is not aligned as required";
    case RB_ERR_WORKSPACE: return "RB_ERR_WORKSPACE: workspace missing or too small";
    case RB_ERR_HIP: return "RB_ERR_HIP: a kernel launch failed";
  }
  return "RB_ERR_UNKNOWN";
}

// rb_gemm_small's K-chunk partials: scratch, after the zero region (none when K is not split)
static size_t gemm_small_ws(int k, int64_t N, int64_t K, int64_t M) {
  const size_t p = rb::gemm_small_workspace_bytes(k, N, K, M);
  return p > 0 ? rb::zero_region_bytes(N) + p : 0u;
}

size_t rb_workspace_bytes(rb_op op, int32_t k, int64_t N, int64_t K, int64_t M) {
  if (k < 1 || k > 4 || N < 1 || K < 1 || M < 1) return 0;
  switch (op) {
    case RB_OP_GEMV: return rb::gemv_workspace_bytes(k, N, K, M);
    case RB_OP_GEMM_SMALL: return gemm_small_ws(k, N, K, M);
    case RB_OP_CODEBOOK_GEMV: return rb::codebook_gemv_workspace_bytes(N, K, M);
    case RB_OP_SVID_INIT: return (N > kMaxDim || K > kMaxDim) ? 0 : rb::zero_region_bytes(N) + rb::svid_workspace_bytes(k, N, K);
    case RB_OP_QAT_BACKWARD:
      return (N > kQatMaxDim || K > kQatMaxDim) ? 0 : rb::zero_region_bytes(N) + rb::qat_backward_workspace_bytes(k, N, K);
    default: return 0;
  }
}

double rb_storage_bits_per_weight(int64_t N, int64_t K, int32_t k, rb_dtype scale_dtype, int32_t has_h) {
  if (N < 1 || K < 1 || k < 1 || k > 4 || !valid_dtype(scale_dtype)) return -1.0;
  const double sbits = scale_dtype == RB_F32 ? 32.0 : 16.0;
  const double per_plane = (double)N + (has_h ? (double)K : 0.0);
  return (double)k + sbits * (double)k * per_plane / ((double)N * (double)K);
}

rb_status rb_pack(const void* W, rb_dtype w_dtype, int64_t N, int64_t K, int64_t ldw, int32_t k,
                  int32_t group, const void* h, rb_dtype scale_dtype, uint32_t* planes, int64_t ldp,
                  void* g, int32_t* d_status, void* stream) {
  if (!W || !planes || !g) return RB_ERR_INVALID_ARG;
  if (!valid_dtype(w_dtype) || !valid_dtype(scale_dtype)) return RB_ERR_INVALID_ARG;
  if (scale_dtype == RB_BF16) return RB_ERR_UNSUPPORTED;
  if (N < 1 || K < 1 || N > kMaxDim || K > kMaxDim) return RB_ERR_INVALID_ARG;
  if (ldw < K || ldp < (K + 31) / 32) return RB_ERR_INVALID_ARG;
  if (k < 1 || k > 4) return RB_ERR_INVALID_ARG;
  if (group != 0 && !is_pow2_in(group, 2, 64)) return RB_ERR_INVALID_ARG;
  if (group != 0 && h != nullptr) return RB_ERR_UNSUPPORTED;
  if (!aligned(planes, 16)) return RB_ERR_MISALIGNED;
  if (!aligned(W, w_dtype == RB_F32 ? 4 : 2) || !aligned(g, scale_dtype == RB_F32 ? 4 : 2) ||
      (h && !aligned(h, scale_dtype == RB_F32 ? 4 : 2)) || (d_status && !aligned(d_status, 4)))
    return RB_ERR_MISALIGNED;
  log_call("rb_pack", N, K, 0, k);
  return from_hip(rb::launch_pack(W, w_dtype, N, K, ldw, k, group, h, scale_dtype, planes, ldp, g,
                                  d_status, static_cast<hipStream_t>(stream)));
}

}  // extern "C"

namespace rb {
rb_status gemv_args_status(const uint32_t* planes, int64_t ldp, const void* g, const void* h, rb_dtype scale_dtype,
                           int32_t k, int64_t N, int64_t K, const void* x, rb_dtype x_dtype, int64_t M, void* y,
                           rb_dtype y_dtype) {
  rb_status st = check_product_args(planes, ldp, g, scale_dtype, k, N, K, x, x_dtype, M, y, y_dtype, 16);
  if (st != RB_OK) return st;
  if (h && !aligned(h, scale_dtype == RB_F32 ? 4 : 2)) return RB_ERR_MISALIGNED;
  return RB_OK;
}
}  // namespace rb

extern "C" {

rb_status rb_gemv(const uint32_t* planes, int64_t ldp, const void* g, const void* h,
                  rb_dtype scale_dtype, int32_t k, int64_t N, int64_t K, const void* x,
                  rb_dtype x_dtype, int64_t M, void* y, rb_dtype y_dtype, void* ws, size_t ws_bytes,
                  void* stream) {
  rb_status st = rb::gemv_args_status(planes, ldp, g, h, scale_dtype, k, N, K, x, x_dtype, M, y, y_dtype);
  if (st != RB_OK) return st;
  const size_t need = rb::gemv_workspace_bytes(k, N, K, M);
  if (need > 0 && (!ws || ws_bytes < need)) return RB_ERR_WORKSPACE;
  if (ws && !aligned(ws, 16)) return RB_ERR_MISALIGNED;
  log_call("rb_gemv", N, K, M, k);
  return from_hip(rb::launch_gemv(planes, ldp, g, h, scale_dtype, k, N, K, x, x_dtype, M, y, y_dtype,
                                  ws, static_cast<hipStream_t>(stream)));
}

rb_status rb_gemv_variant(const uint32_t* planes, int64_t ldp, const void* g, const void* h, const void* mu,
                          int32_t zero_one, rb_dtype scale_dtype, int32_t k, int64_t N, int64_t K, const void* x,
                          rb_dtype x_dtype, int64_t M, void* y, rb_dtype y_dtype, void* ws, size_t ws_bytes,
                          void* stream) {
  rb_status st = check_product_args(planes, ldp, g, scale_dtype, k, N, K, x, x_dtype, M, y, y_dtype, 16);
  if (st != RB_OK) return st;
  if (zero_one != 0 && zero_one != 1) return RB_ERR_INVALID_ARG;
  if (mu && h) return RB_ERR_UNSUPPORTED;
  if (h && !aligned(h, scale_dtype == RB_F32 ? 4 : 2)) return RB_ERR_MISALIGNED;
  if (mu && !aligned(mu, scale_dtype == RB_F32 ? 4 : 2)) return RB_ERR_MISALIGNED;
  const size_t need = rb::gemv_workspace_bytes(k, N, K, M);
  if (need > 0 && (!ws || ws_bytes < need)) return RB_ERR_WORKSPACE;
  if (ws && !aligned(ws, 16)) return RB_ERR_MISALIGNED;
  log_call("rb_gemv_variant", N, K, M, k);
  return from_hip(rb::launch_gemv_variant(planes, ldp, g, h, mu, zero_one, scale_dtype, k, N, K, x, x_dtype, M, y,
                                          y_dtype, ws, static_cast<hipStream_t>(stream)));
}

rb_status rb_gemm_small(const uint32_t* planes, int64_t ldp, const void* g, const void* h,
                        rb_dtype scale_dtype, int32_t k, int64_t N, int64_t K, const void* x,
                        rb_dtype x_dtype, int64_t M, void* y, rb_dtype y_dtype, void* ws,
                        size_t ws_bytes, void* stream) {
  rb_status st = check_product_args(planes, ldp, g, scale_dtype, k, N, K, x, x_dtype, M, y, y_dtype, 4096);
  if (st != RB_OK) return st;
  if (x_dtype != RB_F16) return RB_ERR_UNSUPPORTED;
  if (K % 64 != 0 || ldp % 2 != 0) return RB_ERR_UNSUPPORTED;
  if (K > (int64_t(1) << 22) || ldp > (int64_t(1) << 20)) return RB_ERR_UNSUPPORTED;  // 32-bit offsets
  if (h && scale_dtype != RB_F16) return RB_ERR_UNSUPPORTED;  // h enters the fp16 operand
  if (h && !aligned(h, 16)) return RB_ERR_MISALIGNED;
  const size_t need = gemm_small_ws(k, N, K, M);
  if (need > 0 && (!ws || ws_bytes < need)) return RB_ERR_WORKSPACE;
  if (need > 0 && !aligned(ws, 4)) return RB_ERR_MISALIGNED;
  log_call("rb_gemm_small", N, K, M, k);
  void* scratch_ws = need > 0 ? static_cast<char*>(ws) + rb::zero_region_bytes(N) : nullptr;
  return from_hip(rb::launch_gemm_small(planes, ldp, g, h, scale_dtype, k, N, K, x, M, y, y_dtype, scratch_ws,
                                        static_cast<hipStream_t>(stream)));
}

rb_status rb_codebook_encode(const uint32_t* sign_plane, int64_t ldp, int64_t N, int64_t K,
                             const uint32_t* codebook, int32_t c, int32_t v, uint16_t* idx,
                             void* stream) {
  if (!sign_plane || !codebook || !idx) return RB_ERR_INVALID_ARG;
  if (N < 1 || K < 1 || N > kMaxDim || K > kMaxDim) return RB_ERR_INVALID_ARG;
  if (ldp < (K + 31) / 32) return RB_ERR_INVALID_ARG;
  if (c < 1 || c > 65536 || v < 1 || v > 32) return RB_ERR_INVALID_ARG;
  if (!aligned(sign_plane, 16) || !aligned(codebook, 4) || !aligned(idx, 2)) return RB_ERR_MISALIGNED;
  log_call("rb_codebook_encode", N, K, 0, 1);
  return from_hip(rb::launch_codebook_encode(sign_plane, ldp, N, K, codebook, c, v, idx,
                                             static_cast<hipStream_t>(stream)));
}

size_t rb_codebook_table_bytes(int32_t v) { return rb::codebook_table_bytes(v); }

rb_status rb_codebook_encode_table(const uint32_t* sign_plane, int64_t ldp, int64_t N, int64_t K,
                                   const uint32_t* codebook, int32_t c, int32_t v, uint16_t* idx, void* ws,
                                   size_t ws_bytes, void* stream) {
  if (!sign_plane || !codebook || !idx) return RB_ERR_INVALID_ARG;
  if (N < 1 || K < 1 || N > kMaxDim || K > kMaxDim) return RB_ERR_INVALID_ARG;
  if (ldp < (K + 31) / 32) return RB_ERR_INVALID_ARG;
  if (c < 1 || c > 65536 || v < 1 || v > 32) return RB_ERR_INVALID_ARG;
  if (v > 24) return RB_ERR_UNSUPPORTED;
  if (N * ((K + v - 1) / v) > 0xffffffffll) return RB_ERR_UNSUPPORTED;  // 32-bit block positions
  if (!ws || ws_bytes < rb::codebook_table_bytes(v)) return RB_ERR_WORKSPACE;
  if (!aligned(sign_plane, 16) || !aligned(codebook, 4) || !aligned(idx, 2) || !aligned(ws, 4))
    return RB_ERR_MISALIGNED;
  log_call("rb_codebook_encode_table", N, K, 0, 1);
  return from_hip(rb::launch_codebook_encode_table(sign_plane, ldp, N, K, codebook, c, v, idx, ws,
                                                   static_cast<hipStream_t>(stream)));
}

size_t rb_codebook_learn_workspace_bytes(int64_t N, int64_t K, int32_t c, int32_t v) {
  if (N < 1 || K < 1 || N > kMaxDim || K > kMaxDim || c < 1 || c > 65536 || v < 1 || v > 32) return 0;
  return rb::codebook_learn_workspace_bytes(N, K, c, v);
}

namespace {
rb_status check_learn_args(const uint32_t* plane, int64_t ldp, int64_t N, int64_t K, int32_t v, int32_t max_v,
                           const uint32_t* codebook, int32_t c, void* ws, size_t ws_bytes) {
  if (!plane || !codebook) return RB_ERR_INVALID_ARG;
  if (N < 1 || K < 1 || N > kMaxDim || K > kMaxDim) return RB_ERR_INVALID_ARG;
  if (ldp < (K + 31) / 32) return RB_ERR_INVALID_ARG;
  if (c < 1 || c > 65536 || v < 1 || v > max_v) return RB_ERR_INVALID_ARG;
  if (!aligned(plane, 16) || !aligned(codebook, 4)) return RB_ERR_MISALIGNED;
  if (N * ((K + v - 1) / v) > 0xffffffffll) return RB_ERR_UNSUPPORTED;  // 32-bit bucket positions
  if (!ws || ws_bytes < rb::codebook_learn_workspace_bytes(N, K, c, v)) return RB_ERR_WORKSPACE;
  if (!aligned(ws, 4)) return RB_ERR_MISALIGNED;
  return RB_OK;
}
}  // namespace

rb_status rb_codebook_mstep(const uint32_t* sign_plane, int64_t ldp, int64_t N, int64_t K, int32_t v,
                            const uint16_t* idx, uint32_t* codebook, int32_t c, uint32_t* counts, void* ws,
                            size_t ws_bytes, void* stream) {
  if (!idx) return RB_ERR_INVALID_ARG;
  rb_status st = check_learn_args(sign_plane, ldp, N, K, v, 32, codebook, c, ws, ws_bytes);
  if (st != RB_OK) return st;
  if (!aligned(idx, 2) || (counts && !aligned(counts, 4))) return RB_ERR_MISALIGNED;
  log_call("rb_codebook_mstep", N, K, 0, 1);
  return from_hip(rb::launch_codebook_mstep(sign_plane, ldp, N, K, v, idx, codebook, c, counts, ws,
                                            static_cast<hipStream_t>(stream)));
}

rb_status rb_codebook_distinct(const uint32_t* sign_plane, int64_t ldp, int64_t N, int64_t K, int32_t v,
                               uint32_t* codebook, int32_t c, int32_t* n_distinct, void* ws, size_t ws_bytes,
                               void* stream) {
  if (!n_distinct) return RB_ERR_INVALID_ARG;
  rb_status st = check_learn_args(sign_plane, ldp, N, K, v, 24, codebook, c, ws, ws_bytes);
  if (st != RB_OK) return st;
  if (!aligned(n_distinct, 4)) return RB_ERR_MISALIGNED;
  log_call("rb_codebook_distinct", N, K, 0, 1);
  return from_hip(rb::launch_codebook_distinct(sign_plane, ldp, N, K, v, codebook, c, n_distinct, ws,
                                               static_cast<hipStream_t>(stream)));
}

rb_status rb_codebook_learn(const uint32_t* sign_plane, int64_t ldp, int64_t N, int64_t K, int32_t v,
                            uint32_t* codebook, int32_t c, int32_t iters, uint16_t* idx, int32_t* n_distinct,
                            void* ws, size_t ws_bytes, void* stream) {
  if (!idx || !n_distinct) return RB_ERR_INVALID_ARG;
  if (iters < 0 || iters > 1000) return RB_ERR_INVALID_ARG;
  rb_status st = check_learn_args(sign_plane, ldp, N, K, v, 24, codebook, c, ws, ws_bytes);
  if (st != RB_OK) return st;
  if (!aligned(idx, 2) || !aligned(n_distinct, 4)) return RB_ERR_MISALIGNED;
  log_call("rb_codebook_learn", N, K, 0, 1);
  return from_hip(rb::launch_codebook_learn(sign_plane, ldp, N, K, v, codebook, c, iters, idx, n_distinct, ws,
                                            static_cast<hipStream_t>(stream)));
}

rb_status rb_codebook_gemv(const uint16_t* idx, const uint32_t* codebook, int32_t c, int32_t v,
                           const void* s, int32_t group, int64_t N, int64_t K, const void* x,
                           int64_t M, void* y, void* ws, size_t ws_bytes, void* stream) {
  if (!idx || !codebook || !s || !x || !y) return RB_ERR_INVALID_ARG;
  if (N < 1 || K < 1 || N > kMaxDim || K > kMaxDim) return RB_ERR_INVALID_ARG;
  if (c < 1 || c > 65536 || v < 1 || v > 32) return RB_ERR_INVALID_ARG;
  if (!is_pow2_in(group, 2, 64)) return RB_ERR_INVALID_ARG;
  if (M < 1) return RB_ERR_INVALID_ARG;
  if (M > 4) return RB_ERR_UNSUPPORTED;
  if (!aligned(idx, 2) || !aligned(codebook, 4) || !aligned(s, 2) || !aligned(x, 16) || !aligned(y, 16))
    return RB_ERR_MISALIGNED;
  const size_t need = rb::codebook_gemv_workspace_bytes(N, K, M);
  if (need > 0 && (!ws || ws_bytes < need)) return RB_ERR_WORKSPACE;
  log_call("rb_codebook_gemv", N, K, M, 1);
  return from_hip(rb::launch_codebook_gemv(idx, codebook, c, v, s, group, N, K, x, M, y, ws,
                                           static_cast<hipStream_t>(stream)));
}

rb_status rb_svid_init(const void* W, rb_dtype w_dtype, int64_t N, int64_t K, int64_t ldw, int32_t k,
                       int32_t T, int32_t P, const float* s_in, const float* s_out, float a_in, float a_out,
                       uint32_t* planes, int64_t ldp, float* g, float* h, void* ws, size_t ws_bytes,
                       void* stream) {
  if (!W || !planes || !g || !h) return RB_ERR_INVALID_ARG;
  if (!valid_dtype(w_dtype)) return RB_ERR_INVALID_ARG;
  if (w_dtype != RB_F32) return RB_ERR_UNSUPPORTED;
  // 16-byte column chunks address a row with 32-bit offsets: K <= 2^28
  if (N < 1 || K < 1 || N > kMaxDim || K > (int64_t(1) << 28)) return RB_ERR_INVALID_ARG;
  if (ldw < K || ldw % 4 != 0 || ldp < (K + 31) / 32) return RB_ERR_INVALID_ARG;
  if (k < 1 || k > 4 || T < 1 || T > 1000 || P < 1 || P > 64) return RB_ERR_INVALID_ARG;
  if (!std::isfinite(a_in) || !std::isfinite(a_out)) return RB_ERR_INVALID_ARG;
  if (!aligned(W, 16) || !aligned(planes, 16) || !aligned(g, 4) || !aligned(h, 4) ||
      !aligned(s_in, 4) || !aligned(s_out, 4))
    return RB_ERR_MISALIGNED;
  const size_t need = rb::zero_region_bytes(N) + rb::svid_workspace_bytes(k, N, K);
  if (!ws || ws_bytes < need) return RB_ERR_WORKSPACE;
  if (!aligned(ws, 16)) return RB_ERR_MISALIGNED;
  log_call("rb_svid_init", N, K, 1, k);
  return from_hip(rb::launch_svid_init(static_cast<const float*>(W), N, K, ldw, k, T, P, s_in, s_out, a_in,
                                       a_out, planes, ldp, g, h, static_cast<char*>(ws) + rb::zero_region_bytes(N),
                                       static_cast<hipStream_t>(stream)));
}

rb_status rb_qat_derive(const float* W, int64_t N, int64_t K, int64_t ldw, int32_t k, const float* g,
                        const float* h, uint32_t* planes, int64_t ldp, void* What, rb_dtype a_dtype,
                        int64_t ldwh, void* stream) {
  if (!W) return RB_ERR_INVALID_ARG;
  rb_status st = check_qat_layer(N, K, k, g, h, planes, ldp, What, ldwh, a_dtype);
  if (st != RB_OK) return st;
  if (ldw < K) return RB_ERR_INVALID_ARG;
  if (!aligned(W, 4)) return RB_ERR_MISALIGNED;
  log_call("rb_qat_derive", N, K, 0, k);
  return from_hip(rb::launch_qat_derive(W, N, K, ldw, k, g, h, planes, ldp, What, a_dtype, ldwh,
                                        static_cast<hipStream_t>(stream)));
}

rb_status rb_qat_forward(const float* W, int64_t N, int64_t K, int64_t ldw, int32_t k, const float* g,
                         const float* h, const void* X, rb_dtype a_dtype, int64_t M, int64_t ldx,
                         uint32_t* planes, int64_t ldp, void* What, int64_t ldwh, void* Y, rb_dtype y_dtype,
                         int64_t ldy, void* stream) {
  if (!W || !X || !Y) return RB_ERR_INVALID_ARG;
  rb_status st = check_qat_layer(N, K, k, g, h, planes, ldp, What, ldwh, a_dtype);
  if (st != RB_OK) return st;
  if (ldw < K || M < 1 || M > kMaxDim || ldx < K || ldx > kMaxDim || ldy < N || ldy > kMaxDim)
    return RB_ERR_INVALID_ARG;
  if (!valid_dtype(y_dtype)) return RB_ERR_INVALID_ARG;
  if (y_dtype != RB_F32 && y_dtype != a_dtype) return RB_ERR_UNSUPPORTED;
  if (!aligned(W, 4) || !elem_aligned(X, a_dtype) || !elem_aligned(Y, y_dtype)) return RB_ERR_MISALIGNED;
  log_call("rb_qat_forward", N, K, M, k);
  const hipStream_t s = static_cast<hipStream_t>(stream);
  rb_status r = from_hip(rb::launch_qat_derive(W, N, K, ldw, k, g, h, planes, ldp, What, a_dtype, ldwh, s));
  if (r != RB_OK) return r;
  return from_hip(rb::launch_qat_forward_gemm(X, a_dtype, M, ldx, What, ldwh, N, K, Y, y_dtype, ldy, s));
}

rb_status rb_qat_backward(const void* dY, rb_dtype a_dtype, int64_t M, int64_t lddy, const void* X, int64_t ldx,
                          const void* What, int64_t ldwh, const uint32_t* planes, int64_t ldp, const float* g,
                          const float* h, int32_t k, int64_t N, int64_t K, float* dW, int64_t lddw, void* dX,
                          rb_dtype dx_dtype, int64_t lddx, float* dg, float* dh, void* ws, size_t ws_bytes,
                          void* stream) {
  if (!dY || !X || !dW || !dX || !dg || !dh) return RB_ERR_INVALID_ARG;
  rb_status st = check_qat_layer(N, K, k, g, h, planes, ldp, What, ldwh, a_dtype);
  if (st != RB_OK) return st;
  if (M < 1 || M > kMaxDim || lddy < N || lddy > kMaxDim || ldx < K || ldx > kMaxDim || lddw < K ||
      lddw > kMaxDim || lddx < K || lddx > kMaxDim)
    return RB_ERR_INVALID_ARG;
  if (!valid_dtype(dx_dtype)) return RB_ERR_INVALID_ARG;
  if (dx_dtype != RB_F32 && dx_dtype != a_dtype) return RB_ERR_UNSUPPORTED;
  if (!elem_aligned(dY, a_dtype) || !elem_aligned(X, a_dtype) || !aligned(dW, 4) || !elem_aligned(dX, dx_dtype) ||
      !aligned(dg, 4) || !aligned(dh, 4))
    return RB_ERR_MISALIGNED;
  const size_t need = rb::zero_region_bytes(N) + rb::qat_backward_workspace_bytes(k, N, K);
  if (!ws || ws_bytes < need) return RB_ERR_WORKSPACE;
  if (!aligned(ws, 16)) return RB_ERR_MISALIGNED;
  log_call("rb_qat_backward", N, K, M, k);
  return from_hip(rb::launch_qat_backward(dY, a_dtype, M, lddy, X, ldx, What, ldwh, planes, ldp, g, h, k, N, K, dW,
                                          lddw, dX, dx_dtype, lddx, dg, dh,
                                          static_cast<char*>(ws) + rb::zero_region_bytes(N),
                                          static_cast<hipStream_t>(stream)));
}

rb_status rb_qat_matmul(const void* X, rb_dtype a_dtype, int64_t M, int64_t ldx, const void* What, int64_t ldwh,
                        int64_t N, int64_t K, void* Y, rb_dtype y_dtype, int64_t ldy, int32_t engine, void* stream) {
  if (!X || !What || !Y) return RB_ERR_INVALID_ARG;
  if (N < 1 || K < 1 || M < 1 || N > kMaxDim || K > kMaxDim || M > kMaxDim) return RB_ERR_INVALID_ARG;
  if (ldx < K || ldx > kMaxDim || ldwh < K || ldwh > kMaxDim || ldy < N || ldy > kMaxDim) return RB_ERR_INVALID_ARG;
  if (engine < RB_QAT_ENGINE_AUTO || engine > RB_QAT_ENGINE_ROCBLAS) return RB_ERR_INVALID_ARG;
  if (!valid_dtype(a_dtype) || !valid_dtype(y_dtype)) return RB_ERR_INVALID_ARG;
  if (!act_dtype(a_dtype) || (y_dtype != RB_F32 && y_dtype != a_dtype)) return RB_ERR_UNSUPPORTED;
  if (!elem_aligned(X, a_dtype) || !elem_aligned(What, a_dtype) || !elem_aligned(Y, y_dtype)) return RB_ERR_MISALIGNED;
  if (engine == RB_QAT_ENGINE_MFMA && !rb::qat_gemm_tn_supported(X, ldx, What, ldwh, M, N, K))
    return RB_ERR_UNSUPPORTED;
  log_call("rb_qat_matmul", N, K, M, engine);
  return from_hip(rb::launch_qat_forward_gemm(X, a_dtype, M, ldx, What, ldwh, N, K, Y, y_dtype, ldy,
                                              static_cast<hipStream_t>(stream), engine));
}

rb_status rb_qat_autotune(const void* X, const void* dY, rb_dtype a_dtype, int64_t M, int64_t ldx, int64_t lddy,
                          const void* What, int64_t ldwh, int64_t N, int64_t K, void* Y, rb_dtype y_dtype,
                          int64_t ldy, float* dW, int64_t lddw, void* dX, rb_dtype dx_dtype, int64_t lddx,
                          void* stream) {
  if (!X || !dY || !What || !Y || !dW || !dX) return RB_ERR_INVALID_ARG;
  if (N < 1 || K < 1 || N > kQatMaxDim || K > kQatMaxDim || M < 1 || M > kMaxDim) return RB_ERR_INVALID_ARG;
  if (ldx < K || ldx > kMaxDim || lddy < N || lddy > kMaxDim || ldwh < K || ldwh > kMaxDim || ldy < N ||
      ldy > kMaxDim || lddw < K || lddw > kMaxDim || lddx < K || lddx > kMaxDim)
    return RB_ERR_INVALID_ARG;
  if (!valid_dtype(a_dtype) || !valid_dtype(y_dtype) || !valid_dtype(dx_dtype)) return RB_ERR_INVALID_ARG;
  if (!act_dtype(a_dtype)) return RB_ERR_UNSUPPORTED;
  if ((y_dtype != RB_F32 && y_dtype != a_dtype) || (dx_dtype != RB_F32 && dx_dtype != a_dtype))
    return RB_ERR_UNSUPPORTED;
  if (!elem_aligned(X, a_dtype) || !elem_aligned(dY, a_dtype) || !elem_aligned(What, a_dtype) ||
      !elem_aligned(Y, y_dtype) || !aligned(dW, 4) || !elem_aligned(dX, dx_dtype))
    return RB_ERR_MISALIGNED;
  log_call("rb_qat_autotune", N, K, M, 0);
  return from_hip(rb::launch_qat_autotune(X, dY, a_dtype, M, ldx, lddy, What, ldwh, N, K, Y, y_dtype, ldy, dW, lddw,
                                          dX, dx_dtype, lddx, static_cast<hipStream_t>(stream)));
}

}  // extern "C"
