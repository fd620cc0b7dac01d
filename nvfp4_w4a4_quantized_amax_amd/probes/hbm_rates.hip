// Measurement program (not part of libnvfp4): the HBM rates the activation quantizer's two
// phases can reach at best on this device.  A read-only stream of 128 MiB (the 8192 x 8192 bf16
// input; 16-byte non-temporal loads, a max kept in registers) and a write-only stream of 37.7 MB
// (its packed codes and scales; 16-byte non-temporal stores), over 4 and 8 rotating buffers
// respectively (512 MiB and 302 MB, so that neither stream lives in the 256 MB Infinity Cache), at three grid sizes of 256-thread
// workgroups.  Each line is the mean of 40 back-to-back launches, launch gaps included.
//
//   usage: hbm_rates
#include <hip/hip_runtime.h>
#include <stdio.h>
#include <stdlib.h>
#define CK(x) do { hipError_t e_ = (x); if (e_ != hipSuccess) { printf("HIP error %s at %d\n", hipGetErrorString(e_), __LINE__); exit(1);} } while (0)
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
__global__ __launch_bounds__(256) void rd(const u32x4 *x, size_t n16, unsigned *out) {
  unsigned m = 0;
  size_t i = blockIdx.x * 256 + threadIdx.x, s = (size_t)gridDim.x * 256;
  for (; i + 3 * s < n16; i += 4 * s) {
    u32x4 a = __builtin_nontemporal_load(x + i), b = __builtin_nontemporal_load(x + i + s);
    u32x4 c = __builtin_nontemporal_load(x + i + 2 * s), d = __builtin_nontemporal_load(x + i + 3 * s);
    m = max(m, a[0] ^ b[1] ^ c[2] ^ d[3]);
  }
  for (; i < n16; i += s) { u32x4 a = __builtin_nontemporal_load(x + i); m = max(m, a[0]); }
  if (m == 0x12345678u) out[blockIdx.x] = m;
}
__global__ __launch_bounds__(256) void wr(u32x4 *y, size_t n16) {
  size_t i = blockIdx.x * 256 + threadIdx.x, s = (size_t)gridDim.x * 256;
  for (; i < n16; i += s) __builtin_nontemporal_store(u32x4{(unsigned)i, 1u, 2u, 3u}, y + i);
}
int main() {
  const size_t nin = 128ull << 20, nout = 37748736ull;  // 128 MiB, 32 MiB + 4 MiB
  u32x4 *x[4], *y[8];
  unsigned *o;
  for (int b = 0; b < 4; ++b) { CK(hipMalloc(&x[b], nin)); CK(hipMemset(x[b], b + 1, nin)); }
  for (int b = 0; b < 8; ++b) CK(hipMalloc(&y[b], nout));
  CK(hipMalloc(&o, 1 << 20));
  hipEvent_t a, e; CK(hipEventCreate(&a)); CK(hipEventCreate(&e));
  for (int grid : {1024, 2048, 4096}) {
    for (int mode = 0; mode < 2; ++mode) {
      for (int i = 0; i < 8; ++i) {
        if (mode == 0) hipLaunchKernelGGL(rd, dim3(grid), dim3(256), 0, 0, x[i % 4], nin / 16, o);
        else hipLaunchKernelGGL(wr, dim3(grid), dim3(256), 0, 0, y[i % 8], nout / 16);
      }
      CK(hipDeviceSynchronize());
      CK(hipEventRecord(a, 0));
      const int reps = 40;
      for (int i = 0; i < reps; ++i) {
        if (mode == 0) hipLaunchKernelGGL(rd, dim3(grid), dim3(256), 0, 0, x[i % 4], nin / 16, o);
        else hipLaunchKernelGGL(wr, dim3(grid), dim3(256), 0, 0, y[i % 8], nout / 16);
      }
      CK(hipEventRecord(e, 0)); CK(hipEventSynchronize(e));
      float ms; CK(hipEventElapsedTime(&ms, a, e));
      double us = ms * 1000 / reps, bytes = mode == 0 ? (double)nin : (double)nout;
      printf("%s grid %d: %.2f us, %.0f GB/s\n", mode == 0 ? "read 128MiB " : "write 37.7MB", grid, us, bytes / us / 1e3);
    }
  }
  return 0;
}
