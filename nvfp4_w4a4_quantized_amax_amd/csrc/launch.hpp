// Host-side launchers of the libnvfp4 kernels (internal; the public API is include/nvfp4.h).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace nvfp4 {

// Quantization (quantize.hip).  launch_amax picks the grid and the per-workgroup tile count;
// the matching encode launch must use the same two values so that each workgroup re-reads the
// data it read in pass 1.
hipError_t launch_amax(const void *x, int64_t rows, int64_t cols, int64_t ld_x, void *ws,
                       float *gs_out, int *grid_out, uint32_t *tiles_per_wg_out,
                       hipStream_t stream);
hipError_t launch_encode_1d(const void *x, int64_t rows, int64_t cols, int64_t ld_x,
                            uint8_t *codes, int64_t ld_codes, uint8_t *scales, int64_t ld_scales,
                            const void *ws, int grid, uint32_t tiles_per_wg, hipStream_t stream);
hipError_t launch_encode_2d(const void *w, int64_t rows, int64_t cols, int64_t ld_w,
                            uint8_t *codes, int64_t ld_codes, uint8_t *scales, int64_t ld_scales,
                            const void *ws, hipStream_t stream);
// One-workgroup quantization of a small tensor (rows * cols <= kSmallMaxElems); `dec`, when not
// NULL, receives code * block scale as fp16 (row stride ld_dec elements).
constexpr int64_t kSmallMaxElems = 1 << 17;
hipError_t launch_quantize_small(const void *x, int64_t rows, int64_t cols, int64_t ld_x,
                                 uint8_t *codes, int64_t ld_codes, uint8_t *scales,
                                 int64_t ld_scales, float *gs_out, _Float16 *dec, int64_t ld_dec,
                                 hipStream_t stream);

// Dequantization (dequantize.hip).
hipError_t launch_dequantize(const uint8_t *codes, int64_t ld_codes, const uint8_t *scales,
                             int64_t ld_scales, const float *gs, int64_t rows, int64_t cols,
                             int block_rows, void *y, int64_t ld_y, int out_f32,
                             hipStream_t stream);
// code * block scale as fp16 (global scale not applied), 1D blocks: the A operand of the
// small-M GEMM when A arrives already quantized.
hipError_t launch_decode_f16(const uint8_t *codes, int64_t ld_codes, const uint8_t *scales,
                             int64_t ld_scales, int64_t rows, int64_t cols, _Float16 *dec,
                             int64_t ld_dec, hipStream_t stream);

// GEMM (gemm.hip).
struct GemmOperand {
  const uint8_t *codes;
  int64_t ld_codes;
  const uint8_t *scales;
  int64_t ld_scales;
  const float *gs;
  int block_rows;
};

hipError_t launch_gemm_tile(const GemmOperand &a, const GemmOperand &w, int64_t m, int64_t n,
                            int64_t k, uint16_t *y, int64_t ld_y, hipStream_t stream);
// Small M (m <= 16): A given as decoded fp16 (code * scale, row stride ld_dec, gsA separate).
hipError_t launch_gemm_small_m(const _Float16 *a_dec, int64_t ld_dec, const float *gs_a,
                               const GemmOperand &w, int64_t m, int64_t n, int64_t k, uint16_t *y,
                               int64_t ld_y, hipStream_t stream);
hipError_t launch_grouped_gemm(const GemmOperand &a, const int32_t *row_index,
                               const int32_t *offsets, int32_t num_groups, const GemmOperand &w,
                               int64_t w_group_rows, int64_t n, int64_t k, int64_t total_rows,
                               uint16_t *y, int64_t ld_y, hipStream_t stream);

}  // namespace nvfp4
