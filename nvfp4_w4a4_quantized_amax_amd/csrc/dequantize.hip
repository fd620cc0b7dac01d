// NVFP4 reconstruction for gfx950: value = code value * block scale * global scale ("NVFP4
// Explained: NVIDIA's 4-Bit Format for Faster AI Inference", section "How NVFP4 Represents a
// Value").  code * block scale is exact in fp32 (<= 6 significant bits); the product with the
// global scale is rounded once to fp32, then optionally to bf16 (nearest, ties to even).
#include "nvfp4_device.hpp"
#include "launch.hpp"

namespace nvfp4 {

typedef float float2_t __attribute__((ext_vector_type(2)));

// bf16 output: one thread = 8 consecutive values (one 32-bit word of codes, 16 bytes out).
__global__ __launch_bounds__(256) void k_dequantize_bf16(const uint8_t *__restrict__ codes,
                                                         int64_t ld_codes,
                                                         const uint8_t *__restrict__ scales,
                                                         int64_t ld_scales,
                                                         const float *__restrict__ gsp,
                                                         int64_t rows, int64_t cols,
                                                         int block_rows,
                                                         uint16_t *__restrict__ y, int64_t ld_y) {
  const float gs = *gsp;
  const int64_t per_row = cols / 8;
  const int64_t n = rows * per_row;
  for (int64_t u = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; u < n;
       u += (int64_t)gridDim.x * blockDim.x) {
    const int64_t r = u / per_row, c8 = u - r * per_row;
    const uint32_t q = *(const uint32_t *)(codes + r * ld_codes + c8 * 4);
    const int64_t srow = block_rows == 16 ? (r >> 4) : r;
    const float sb = e4m3_to_float(scales[srow * ld_scales + (c8 >> 1)]);
    float2_t g[4] = {__builtin_amdgcn_cvt_scalef32_pk_f32_fp4(q, 1.0f, 0),
                     __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(q, 1.0f, 1),
                     __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(q, 1.0f, 2),
                     __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(q, 1.0f, 3)};
    uint32_t h[8];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      h[2 * j] = f32_to_bf16_rne((g[j][0] * sb) * gs);
      h[2 * j + 1] = f32_to_bf16_rne((g[j][1] * sb) * gs);
    }
    ntstore16(y + r * ld_y + c8 * 8, make_uint4(h[0] | (h[1] << 16), h[2] | (h[3] << 16),
                                                h[4] | (h[5] << 16), h[6] | (h[7] << 16)));
  }
}

// fp32 output: one thread = 4 consecutive values (16 bits of codes, 16 bytes out), so that one
// store instruction of a wave covers 1 KiB of contiguous output.  With 8 values per thread the
// two 16-byte stores of a lane interleave at a 32-byte stride, and that form wrote at about a
// third of the HBM rate.
__global__ __launch_bounds__(256) void k_dequantize_f32(const uint8_t *__restrict__ codes,
                                                        int64_t ld_codes,
                                                        const uint8_t *__restrict__ scales,
                                                        int64_t ld_scales,
                                                        const float *__restrict__ gsp,
                                                        int64_t rows, int64_t cols,
                                                        int block_rows, float *__restrict__ y,
                                                        int64_t ld_y) {
  const float gs = *gsp;
  const int64_t per_row = cols / 4;
  const int64_t n = rows * per_row;
  for (int64_t u = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; u < n;
       u += (int64_t)gridDim.x * blockDim.x) {
    const int64_t r = u / per_row, c4 = u - r * per_row;
    const uint32_t q = *(const uint16_t *)(codes + r * ld_codes + c4 * 2);
    const int64_t srow = block_rows == 16 ? (r >> 4) : r;
    const float sb = e4m3_to_float(scales[srow * ld_scales + (c4 >> 2)]);
    const float2_t g0 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(q, 1.0f, 0);
    const float2_t g1 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(q, 1.0f, 1);
    ntstore16(y + r * ld_y + c4 * 4,
              make_uint4(__float_as_uint((g0[0] * sb) * gs), __float_as_uint((g0[1] * sb) * gs),
                         __float_as_uint((g1[0] * sb) * gs), __float_as_uint((g1[1] * sb) * gs)));
  }
}

static unsigned grid_for(int64_t units) {
  int64_t g = (units + 255) / 256;
  if (g > 8192) g = 8192;
  if (g < 1) g = 1;
  return (unsigned)g;
}

hipError_t launch_dequantize(const uint8_t *codes, int64_t ld_codes, const uint8_t *scales,
                             int64_t ld_scales, const float *gs, int64_t rows, int64_t cols,
                             int block_rows, void *y, int64_t ld_y, int out_f32,
                             hipStream_t stream) {
  if (out_f32)
    hipLaunchKernelGGL(k_dequantize_f32, dim3(grid_for(rows * (cols / 4))), dim3(256), 0, stream,
                       codes, ld_codes, scales, ld_scales, gs, rows, cols, block_rows, (float *)y,
                       ld_y);
  else
    hipLaunchKernelGGL(k_dequantize_bf16, dim3(grid_for(rows * (cols / 8))), dim3(256), 0,
                       stream, codes, ld_codes, scales, ld_scales, gs, rows, cols, block_rows,
                       (uint16_t *)y, ld_y);
  return hipGetLastError();
}

}  // namespace nvfp4
