// rb_gemm.hip -- batched product on the matrix cores (gfx950 MFMA). Work in progress.
#include "rb_device.hpp"
#include "rb_internal.h"

namespace rb {

size_t gemm_small_workspace_bytes(int, int64_t, int64_t, int64_t) { return 0; }

hipError_t launch_gemm_small(const uint32_t*, int64_t, const void*, const void*, rb_dtype, int, int64_t,
                             int64_t, const void*, int64_t, void*, rb_dtype, void*, hipStream_t) {
  return hipErrorNotSupported;
}

}  // namespace rb
