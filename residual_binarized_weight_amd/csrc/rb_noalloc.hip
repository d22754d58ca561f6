// rb_noalloc.hip -- rb_gemv for callers that cannot allocate device memory (code under graph
// capture, tight serving loops, harnesses that forbid hipMalloc): its workspace is a fixed
// device array of this library instead of a caller's buffer.
//
// The array is a file-scope __device__ object, so each GPU the library runs on holds its own
// copy at its own address, allocated when the code object is loaded and kept until the
// process ends. Host code never uses the array's name as an address (on the host it is only a
// stand-in symbol): the device address comes from hipGetSymbolAddress, taken once per device
// with that device current, and only that pointer reaches the kernels.
#include <hip/hip_runtime.h>

#include <mutex>

#include "../../include/rb.h"
#include "rb_internal.h"

namespace {

constexpr size_t kScratchBytes = size_t(4) << 20;  // 4 MB per device
constexpr int kMaxDevices = 64;

__device__ __align__(256) uint8_t scratch[kScratchBytes];

// clears the zero region: a kernel, not a memset node, so that the call can be captured
__global__ __launch_bounds__(256) void scratch_zero_kernel(uint4* __restrict__ p, size_t n16) {
  for (size_t i = (size_t)blockIdx.x * 256 + threadIdx.x; i < n16; i += (size_t)gridDim.x * 256)
    p[i] = make_uint4(0u, 0u, 0u, 0u);
}

std::mutex g_scratch_mutex;
void* g_scratch_ptr[kMaxDevices] = {};

// the device address of this device's array (nullptr if it cannot be obtained)
void* scratch_for_current_device() {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
  std::lock_guard<std::mutex> lock(g_scratch_mutex);
  if (g_scratch_ptr[dev] == nullptr) {
    void* ptr = nullptr;
    if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || ptr == nullptr) return nullptr;
    g_scratch_ptr[dev] = ptr;
  }
  return g_scratch_ptr[dev];
}

}  // namespace

extern "C" rb_status rb_gemv_noalloc(const uint32_t* planes, int64_t ldp, const void* g, const void* h,
                                     rb_dtype scale_dtype, int32_t k, int64_t N, int64_t K, const void* x,
                                     rb_dtype x_dtype, int64_t M, void* y, rb_dtype y_dtype, void* stream) {
  const rb_status st = rb::gemv_args_status(planes, ldp, g, h, scale_dtype, k, N, K, x, x_dtype, M, y, y_dtype);
  if (st != RB_OK) return st;
  const size_t need = rb::gemv_workspace_bytes(k, N, K, M);
  if (need > kScratchBytes) return RB_ERR_WORKSPACE;  // beyond the fixed array
  void* ws = scratch_for_current_device();
  if (ws == nullptr) return RB_ERR_HIP;
  const hipStream_t s = static_cast<hipStream_t>(stream);
  // the zero region must be zero on entry; the array keeps whatever the last call left, so it
  // is cleared here rather than trusted
  const size_t zr = need < rb::zero_region_bytes(N) ? need : rb::zero_region_bytes(N);
  if (zr > 0) {
    const size_t n16 = (zr + 15) / 16;
    const unsigned blocks = (unsigned)((n16 + 255) / 256 < 1024 ? (n16 + 255) / 256 : 1024);
    scratch_zero_kernel<<<blocks, 256, 0, s>>>(static_cast<uint4*>(ws), n16);
    if (hipGetLastError() != hipSuccess) return RB_ERR_HIP;
  }
  const hipError_t e = rb::launch_gemv(planes, ldp, g, h, scale_dtype, k, N, K, x, x_dtype, M, y, y_dtype, ws, s);
  return e == hipSuccess ? RB_OK : RB_ERR_HIP;
}
