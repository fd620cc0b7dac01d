// Measurement program (not part of libnvfp4): how fast the decode-shaped products' weight
// stream can be read at best.  The 14336 x 4096 FP4 weight codes (29.4 MB), 10 rotating copies
// (294 MB, past the 256 MB Infinity Cache), read-only, in the launch shape of the decode kernel
// (224 workgroups of 16 waves, four 16-row bands per workgroup, every load issued up front):
//   mode 0: the decode kernel's lane pattern: lane (i16, q) of wave w reads 16 bytes of band row
//           i16 at byte 64 * window + 16 * q, windows 2w and 2w + 1;
//   mode 1: the same bytes per workgroup read as contiguous 1 KiB chunks (16 bytes per lane);
//   mode 2: mode 0 with a 64 KiB LDS array written and read once (the size of the decode
//           kernel's reduction buffer).
// Each line: HIP events around 100 back-to-back launches, launch gaps included (two passes).
//
//   usage: decode_stream
#include <hip/hip_runtime.h>
#include <stdio.h>
#include <stdlib.h>
#define CK(x) do { hipError_t e_ = (x); if (e_ != hipSuccess) { printf("HIP error %s at %d\n", hipGetErrorString(e_), __LINE__); exit(1);} } while (0)
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
template <int MODE>
__global__ __launch_bounds__(1024) void k(const uint8_t *__restrict__ w, unsigned *out) {
  __shared__ u32x4 big[MODE == 2 ? 4096 : 1];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, i16 = lane & 15, q = lane >> 4;
  u32x4 acc = {0, 0, 0, 0};
  u32x4 v[8];
  if (MODE == 1) {
    // WG b owns bands b, b+224, b+448, b+672: 4 x 32 KiB contiguous; wave w reads 2 KiB of each.
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const size_t band = blockIdx.x + (size_t)j * gridDim.x;
      const uint8_t *base = w + band * 16 * 2048 + wave * 2048;
      v[2 * j] = *(const u32x4 *)(base + lane * 16);
      v[2 * j + 1] = *(const u32x4 *)(base + 1024 + lane * 16);
    }
  } else {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const size_t band = blockIdx.x + (size_t)j * gridDim.x;
      const uint8_t *row = w + (band * 16 + i16) * 2048 + q * 16;
      v[2 * j] = *(const u32x4 *)(row + (2 * wave) * 64);
      v[2 * j + 1] = *(const u32x4 *)(row + (2 * wave + 1) * 64);
    }
  }
#pragma unroll
  for (int j = 0; j < 8; ++j) acc ^= v[j];
  if (MODE == 2) {
    big[threadIdx.x] = acc;
    __syncthreads();
    acc ^= big[(threadIdx.x * 7) & 1023];
  }
  if ((acc.x ^ acc.y ^ acc.z ^ acc.w) == 0x9E3779B9u) out[blockIdx.x] = acc.x;
}
int main() {
  const size_t bytes = 14336ull * 2048ull;
  const int NW = 10;
  uint8_t *w[NW];
  for (int i = 0; i < NW; ++i) { CK(hipMalloc(&w[i], bytes)); CK(hipMemset(w[i], i + 1, bytes)); }
  unsigned *o; CK(hipMalloc(&o, 4096));
  hipEvent_t a, b; CK(hipEventCreate(&a)); CK(hipEventCreate(&b));
  for (int pass = 0; pass < 2; ++pass)
    for (int mode = 0; mode < 3; ++mode) {
      auto run = [&](int i) {
        if (mode == 0) hipLaunchKernelGGL(k<0>, dim3(224), dim3(1024), 0, 0, w[i % NW], o);
        if (mode == 1) hipLaunchKernelGGL(k<1>, dim3(224), dim3(1024), 0, 0, w[i % NW], o);
        if (mode == 2) hipLaunchKernelGGL(k<2>, dim3(224), dim3(1024), 0, 0, w[i % NW], o);
      };
      for (int i = 0; i < 20; ++i) run(i);
      CK(hipDeviceSynchronize());
      CK(hipEventRecord(a, 0));
      for (int i = 0; i < 100; ++i) run(i);
      CK(hipEventRecord(b, 0)); CK(hipEventSynchronize(b));
      float ms; CK(hipEventElapsedTime(&ms, a, b));
      printf("mode %d: %.2f us per call, %.0f GB/s\n", mode, ms * 10, bytes / (ms * 10) / 1e3);
    }
  return 0;
}
