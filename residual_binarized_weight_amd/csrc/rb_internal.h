// rb_internal.h -- launchers behind the C ABI (arguments already validated by rb_api.cpp).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "../../include/rb.h"

namespace rb {

int device_cu_count();  // compute units of the current device (cached)

hipError_t launch_pack(const void* W, rb_dtype w_dtype, int64_t N, int64_t K, int64_t ldw, int k,
                       int group, const void* h, rb_dtype scale_dtype, uint32_t* planes, int64_t ldp,
                       void* g, int32_t* d_status, hipStream_t s);

// GEMV (M <= 16)
size_t gemv_workspace_bytes(int k, int64_t N, int64_t K, int64_t M);
// The first bytes of every workspace (256-byte multiple): the per-row accumulators that the
// GEMV calls need zero on entry and leave zero. Calls with scratch-only workspaces place
// their scratch after it and never write it, so one buffer can serve every call.
size_t zero_region_bytes(int64_t N);
// rb_gemv's host-side argument checks (everything but the workspace)
rb_status gemv_args_status(const uint32_t* planes, int64_t ldp, const void* g, const void* h, rb_dtype scale_dtype,
                           int32_t k, int64_t N, int64_t K, const void* x, rb_dtype x_dtype, int64_t M, void* y,
                           rb_dtype y_dtype);
hipError_t launch_gemv(const uint32_t* planes, int64_t ldp, const void* g, const void* h,
                       rb_dtype scale_dtype, int k, int64_t N, int64_t K, const void* x,
                       rb_dtype x_dtype, int64_t M, void* y, rb_dtype y_dtype, void* ws,
                       hipStream_t s);

// whole-row nibble-table GEMV (M = 1, h = 1); hipErrorNotSupported for types it does not cover
bool gemv_nib_fits(int k, int64_t N, int64_t K, int64_t ldp, rb_dtype x_dtype, rb_dtype scale_dtype,
                   rb_dtype y_dtype);
hipError_t launch_gemv_nib(const uint32_t* planes, int64_t ldp, const void* g, rb_dtype scale_dtype, int k,
                           int64_t N, int64_t K, const void* x, rb_dtype x_dtype, void* y, rb_dtype y_dtype,
                           const void* mu, int zero_one, hipStream_t s);
// general h at M = 1 (fp16): one single-plane nibble pass per plane, chained through acc
// (N floats, zero on entry and on return)
bool gemv_nib_h_fits(int k, int64_t N, int64_t K, int64_t ldp, const void* h, rb_dtype x_dtype,
                     rb_dtype scale_dtype, rb_dtype y_dtype);
hipError_t launch_gemv_nib_h(const uint32_t* planes, int64_t ldp, const void* g, const void* h, int k, int64_t N,
                             int64_t K, const void* x, void* y, int zero_one, float* acc, hipStream_t s);
// two activation rows (fp16, h = 1, plain product, 4096 < K within the one-build kernel's
// reach, K a multiple of 8, planes below 2^27 bits): one launch that reads the planes once
bool gemv_nib_rows_fits(int k, int64_t N, int64_t K, int64_t ldp, int64_t M, rb_dtype x_dtype, rb_dtype scale_dtype,
                        rb_dtype y_dtype);
hipError_t launch_gemv_nib_rows(const uint32_t* planes, int64_t ldp, const void* g, int k, int64_t N, int64_t K,
                                const void* x, int64_t M, void* y, hipStream_t s);
// the product with {0, 1} planes (zero_one) and/or a per-row offset mu (h must be NULL with mu)
hipError_t launch_gemv_variant(const uint32_t* planes, int64_t ldp, const void* g, const void* h,
                               const void* mu, int zero_one, rb_dtype scale_dtype, int k, int64_t N, int64_t K,
                               const void* x, rb_dtype x_dtype, int64_t M, void* y, rb_dtype y_dtype, void* ws,
                               hipStream_t s);

// small GEMM on the matrix cores
size_t gemm_small_workspace_bytes(int k, int64_t N, int64_t K, int64_t M);
hipError_t launch_gemm_small(const uint32_t* planes, int64_t ldp, const void* g, const void* h,
                             rb_dtype scale_dtype, int k, int64_t N, int64_t K, const void* x,
                             int64_t M, void* y, rb_dtype y_dtype, void* ws, hipStream_t s);

// binary codebook
hipError_t launch_codebook_encode(const uint32_t* plane, int64_t ldp, int64_t N, int64_t K,
                                  const uint32_t* codebook, int c, int v, uint16_t* idx,
                                  hipStream_t s);
size_t codebook_gemv_workspace_bytes(int64_t N, int64_t K, int64_t M);
size_t codebook_learn_workspace_bytes(int64_t N, int64_t K, int c, int v);
// the nearest-codeword table of all 2^v patterns (v <= 24), and encoding through it
size_t codebook_table_bytes(int v);
bool codebook_use_table(int64_t N, int64_t K, int c, int v);
hipError_t launch_codebook_encode_table(const uint32_t* plane, int64_t ldp, int64_t N, int64_t K,
                                        const uint32_t* codebook, int c, int v, uint16_t* idx, void* ws,
                                        hipStream_t s);
hipError_t launch_codebook_mstep(const uint32_t* plane, int64_t ldp, int64_t N, int64_t K, int v,
                                 const uint16_t* idx, uint32_t* codebook, int c, uint32_t* counts, void* ws,
                                 hipStream_t s);
hipError_t launch_codebook_distinct(const uint32_t* plane, int64_t ldp, int64_t N, int64_t K, int v,
                                    uint32_t* codebook, int c, int32_t* n_distinct, void* ws, hipStream_t s);
hipError_t launch_codebook_learn(const uint32_t* plane, int64_t ldp, int64_t N, int64_t K, int v,
                                 uint32_t* codebook, int c, int iters, uint16_t* idx, int32_t* n_distinct,
                                 void* ws, hipStream_t s);
hipError_t launch_codebook_gemv(const uint16_t* idx, const uint32_t* codebook, int c, int v,
                                const void* s, int group, int64_t N, int64_t K, const void* x,
                                int64_t M, void* y, void* ws, hipStream_t st);

// function-aware initialization (iterative residual SVID)
size_t svid_workspace_bytes(int k, int64_t N, int64_t K);
hipError_t launch_svid_init(const float* W, int64_t N, int64_t K, int64_t ldw, int k, int T, int P,
                            const float* s_in, const float* s_out, float a_in, float a_out, uint32_t* planes,
                            int64_t ldp, float* g, float* h, void* ws, hipStream_t s);

size_t qat_backward_workspace_bytes(int k, int64_t N, int64_t K);
hipError_t launch_qat_derive(const float* W, int64_t N, int64_t K, int64_t ldw, int k, const float* g,
                             const float* h, uint32_t* planes, int64_t ldp, void* What, rb_dtype what_dtype,
                             int64_t ldwh, hipStream_t stream);
// the forward product Y = X What^T: engine 0 the layer's choice (rocBLAS, or the matrix-core
// kernel where rb_qat_autotune timed it at least as fast for the shape), 1 the matrix-core
// kernel, 2 rocBLAS
hipError_t launch_qat_forward_gemm(const void* X, rb_dtype a_dtype, int64_t M, int64_t ldx, const void* What,
                                   int64_t ldwh, int64_t N, int64_t K, void* Y, rb_dtype y_dtype, int64_t ldy,
                                   hipStream_t stream, int engine = 0);
// the matrix-core kernel of that product (rb_qat_gemm.hip) and the operands it takes
bool qat_gemm_tn_supported(const void* X, int64_t ldx, const void* Wh, int64_t ldw, int64_t M, int64_t N, int64_t K);
hipError_t launch_qat_gemm_tn(const void* X, rb_dtype a_dtype, int64_t ldx, const void* Wh, int64_t ldw, int64_t M,
                              int64_t N, int64_t K, void* Y, rb_dtype y_dtype, int64_t ldy, hipStream_t s);
hipError_t launch_qat_backward(const void* dY, rb_dtype a_dtype, int64_t M, int64_t lddy, const void* X, int64_t ldx,
                               const void* What, int64_t ldwh, const uint32_t* planes, int64_t ldp, const float* g,
                               const float* h, int k, int64_t N, int64_t K, float* dW, int64_t lddw, void* dX,
                               rb_dtype dx_dtype, int64_t lddx, float* dg, float* dh, void* ws, hipStream_t stream);
hipError_t launch_qat_autotune(const void* X, const void* dY, rb_dtype a_dtype, int64_t M, int64_t ldx, int64_t lddy,
                               const void* What, int64_t ldwh, int64_t N, int64_t K, void* Y, rb_dtype y_dtype,
                               int64_t ldy, float* dW, int64_t lddw, void* dX, rb_dtype dx_dtype, int64_t lddx,
                               hipStream_t stream);

}  // namespace rb
