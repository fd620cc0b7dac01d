// nvfp4_gemm_w4a4_noalloc (include/nvfp4.h): nvfp4_gemm_w4a4 with the library's own scratch
// memory in place of a caller workspace, for callers that cannot allocate device memory.
//
// The scratch is a file-scope device array; this translation unit holds no kernels, so its
// code object (and the array) is loaded on a device only when the entry point first asks for
// the array's address there.  In host code the array's name is not a device address: every use
// goes through the address hipGetSymbolAddress returns for the current device, kept per device.
#include "../../include/nvfp4.h"

#include <hip/hip_runtime.h>

#include <mutex>

namespace {

__device__ __align__(256) unsigned char scratch[NVFP4_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;

// Device address of `scratch` on the current device (looked up once per device), or NULL with
// *err set when the device cannot be named or the lookup fails.
void *scratch_address(nvfp4_status *err) {
  static std::mutex mu;
  static void *addr[kMaxDevices] = {};
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) {
    (void)hipGetLastError();
    *err = NVFP4_ERR_HIP;
    return nullptr;
  }
  std::lock_guard<std::mutex> lock(mu);
  if (!addr[dev]) {
    void *p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) {
      (void)hipGetLastError();
      *err = NVFP4_ERR_HIP;
      return nullptr;
    }
    addr[dev] = p;
  }
  return addr[dev];
}

}  // namespace

extern "C" nvfp4_status nvfp4_gemm_w4a4_noalloc(const void *a_bf16, int64_t m, int64_t k,
                                                int64_t ld_a, const nvfp4_tensor *a_q,
                                                const nvfp4_tensor *w, void *y, int64_t ld_y,
                                                void *stream) {
  // The checks that need no device come first, so that they are testable without a GPU; the
  // product call repeats them with the rest.
  if (!w) return NVFP4_ERR_NULL;
  if (m < 0 || k <= 0 || k % 16 || w->rows < 1) return NVFP4_ERR_SHAPE;
  if (m == 0) return NVFP4_OK;
  if (nvfp4_gemm_workspace_bytes(m, w->rows, k) > (size_t)NVFP4_NOALLOC_SCRATCH_BYTES)
    return NVFP4_ERR_WORKSPACE;
  nvfp4_status err = NVFP4_OK;
  void *ws = scratch_address(&err);
  if (!ws) return err;
  return nvfp4_gemm_w4a4(a_bf16, m, k, ld_a, a_q, w, y, ld_y, ws,
                         (size_t)NVFP4_NOALLOC_SCRATCH_BYTES, stream);
}
