// Measurement program (not part of libnvfp4): what it costs to start a kernel shaped like the
// single-read quantizer (one workgroup of 1024 threads with 136 KiB of LDS per CU, a trivial
// body) with an ordinary launch and with HIP's cooperative launch, which guarantees that all
// workgroups are resident at once.  Prints the device's cooperative-launch attribute, the
// occupancy, the result of one cooperative launch, then the time per launch of 100 back-to-back
// launches of each kind (twice).
//
//   usage: launch_cost
#include <hip/hip_runtime.h>
#include <stdio.h>
__global__ __launch_bounds__(1024, 1) void k_big(int *out) {
  __shared__ int buf[34 * 1024];
  buf[threadIdx.x] = threadIdx.x;
  __syncthreads();
  if (threadIdx.x == 0 && blockIdx.x == 0) out[0] = buf[5];
}
int main() {
  int coop = -1, cus = 0, occ = -1;
  (void)hipDeviceGetAttribute(&coop, hipDeviceAttributeCooperativeLaunch, 0);
  (void)hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, 0);
  (void)hipOccupancyMaxActiveBlocksPerMultiprocessor(&occ, (const void *)k_big, 1024, 0);
  printf("coop attr %d cus %d occupancy %d\n", coop, cus, occ);
  int *d = nullptr;
  if (hipMalloc(&d, 64) != hipSuccess) return 1;
  void *args[] = {(void *)&d};
  hipError_t e = hipLaunchCooperativeKernel((const void *)k_big, dim3(cus), dim3(1024), args, 0, 0);
  printf("cooperative launch: %s\n", hipGetErrorString(e));
  (void)hipGetLastError();
  (void)hipDeviceSynchronize();
  hipEvent_t a, b;
  (void)hipEventCreate(&a);
  (void)hipEventCreate(&b);
  for (int mode = 0; mode < 2; ++mode) {
    for (int rep = 0; rep < 2; ++rep) {
      (void)hipEventRecord(a, 0);
      for (int i = 0; i < 100; ++i) {
        if (mode == 0) hipLaunchKernelGGL(k_big, dim3(cus), dim3(1024), 0, 0, d);
        else (void)hipLaunchCooperativeKernel((const void *)k_big, dim3(cus), dim3(1024), args, 0, 0);
      }
      (void)hipEventRecord(b, 0);
      (void)hipEventSynchronize(b);
      float ms = 0;
      (void)hipEventElapsedTime(&ms, a, b);
      printf("%s: %.2f us per launch (err %s)\n", mode ? "cooperative" : "plain", ms * 10.0f,
             hipGetErrorString(hipGetLastError()));
    }
  }
  return 0;
}
