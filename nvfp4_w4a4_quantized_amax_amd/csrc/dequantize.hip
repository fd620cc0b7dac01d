// NVFP4 reconstruction for gfx950: value = code value * block scale * global scale ("NVFP4
// Explained: NVIDIA's 4-Bit Format for Faster AI Inference", section "How NVFP4 Represents a
// Value").  code * block scale is exact in fp32 (<= 6 significant bits); the product with the
// global scale is rounded once to fp32, then optionally to bf16 (nearest, ties to even).
#include "nvfp4_device.hpp"
#include "launch.hpp"

namespace nvfp4 {

typedef float float2_t __attribute__((ext_vector_type(2)));

// One thread = 8 consecutive values (one 32-bit word of codes).
template <bool OUT_F32>
__global__ __launch_bounds__(256) void k_dequantize(const uint8_t *__restrict__ codes,
                                                    int64_t ld_codes,
                                                    const uint8_t *__restrict__ scales,
                                                    int64_t ld_scales, const float *__restrict__ gsp,
                                                    int64_t rows, int64_t cols, int block_rows,
                                                    void *__restrict__ y, int64_t ld_y) {
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
    float v[8];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      v[2 * j] = (g[j][0] * sb) * gs;
      v[2 * j + 1] = (g[j][1] * sb) * gs;
    }
    if (OUT_F32) {
      float *p = (float *)y + r * ld_y + c8 * 8;
      ntstore16(p, make_uint4(__float_as_uint(v[0]), __float_as_uint(v[1]), __float_as_uint(v[2]),
                              __float_as_uint(v[3])));
      ntstore16(p + 4, make_uint4(__float_as_uint(v[4]), __float_as_uint(v[5]),
                                  __float_as_uint(v[6]), __float_as_uint(v[7])));
    } else {
      uint4 o;
      o.x = f32_to_bf16_rne(v[0]) | (f32_to_bf16_rne(v[1]) << 16);
      o.y = f32_to_bf16_rne(v[2]) | (f32_to_bf16_rne(v[3]) << 16);
      o.z = f32_to_bf16_rne(v[4]) | (f32_to_bf16_rne(v[5]) << 16);
      o.w = f32_to_bf16_rne(v[6]) | (f32_to_bf16_rne(v[7]) << 16);
      ntstore16((uint16_t *)y + r * ld_y + c8 * 8, o);
    }
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
  const unsigned grid = grid_for(rows * (cols / 8));
  if (out_f32)
    hipLaunchKernelGGL(k_dequantize<true>, dim3(grid), dim3(256), 0, stream, codes, ld_codes,
                       scales, ld_scales, gs, rows, cols, block_rows, y, ld_y);
  else
    hipLaunchKernelGGL(k_dequantize<false>, dim3(grid), dim3(256), 0, stream, codes, ld_codes,
                       scales, ld_scales, gs, rows, cols, block_rows, y, ld_y);
  return hipGetLastError();
}

}  // namespace nvfp4
