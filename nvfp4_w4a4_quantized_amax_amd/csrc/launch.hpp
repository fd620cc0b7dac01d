// Host-side launchers of the libnvfp4 kernels (internal; the public API is include/nvfp4.h).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace nvfp4 {

// Quantization (quantize.hip).  Two passes (amax, then encode); `ws` holds the per-workgroup
// partial maxima between them (kWsHeaderBytes).
hipError_t launch_quantize(const void *x, int64_t rows, int64_t cols, int64_t ld_x, bool two_d,
                           uint8_t *codes, int64_t ld_codes, uint8_t *scales, int64_t ld_scales,
                           float *gs_out, void *ws, hipStream_t stream);
// Single-read 1D quantization: one persistent workgroup per CU holds its tiles in registers
// across a grid barrier.  Returns hipErrorNotSupported, having launched nothing, when the device
// cannot run it (then use launch_quantize).
hipError_t launch_quantize_persistent(const void *x, int64_t rows, int64_t cols, int64_t ld_x,
                                      uint8_t *codes, int64_t ld_codes, uint8_t *scales,
                                      int64_t ld_scales, float *gs_out, void *ws,
                                      hipStream_t stream);
// One-workgroup quantization (1D blocks) of a small tensor (rows * cols <= kSmallMaxElems).
// One CU reads the whole tensor, so past 64K values the single-read kernel is faster (32 x 4096:
// 14.6 us on one workgroup, 9.5 us on all CUs).
constexpr int64_t kSmallMaxElems = 1 << 16;
// An activation quantized inside a product call with at most this many values takes the
// two-kernel path (amax, then encode) instead of the single-read kernel: measured 3-4 us faster
// per call for 17-256 rows x 4096 ahead of the mid-size and split-K products, and 8-9 us for
// the 4096 x 2048 MoE activation, though on its own the single-read kernel is the faster
// quantize.  At 8192 x 8192 (prefill) the single-read kernel stays ahead.
constexpr int64_t kTwoPassBeforeProductMaxElems = (int64_t)1 << 23;
hipError_t launch_quantize_small(const void *x, int64_t rows, int64_t cols, int64_t ld_x,
                                 uint8_t *codes, int64_t ld_codes, uint8_t *scales,
                                 int64_t ld_scales, float *gs_out, hipStream_t stream);

// Dequantization (dequantize.hip).
hipError_t launch_dequantize(const uint8_t *codes, int64_t ld_codes, const uint8_t *scales,
                             int64_t ld_scales, const float *gs, int64_t rows, int64_t cols,
                             int block_rows, void *y, int64_t ld_y, int out_f32,
                             hipStream_t stream);

// GEMM (gemm.hip).
struct GemmOperand {
  const uint8_t *codes;
  int64_t ld_codes;
  const uint8_t *scales;
  int64_t ld_scales;
  const float *gs;
  int block_rows;
};

// K splits of the tiled product (m > 16) of m x k by n x k.  The launcher picks 64-row tiles
// (two resident workgroups per CU), 128-row or 256-row tiles (one per CU), all 256 columns
// wide.  A shape whose tiles fill fewer than half of the resident slots of a 256-CU device
// splits its 64-wide K windows so that tiles x splits fills the slots without a partial second
// round, keeping at least 4 windows per split and the fp32 partial sums (splits x m x n x 4
// bytes) no larger than W's packed codes (n x k / 2 bytes), or twice that for 256-row tiles,
// whose compute gains more from the split.  Depends on the shape only, so the workspace size
// does too.  1 = no split.
// Mid-size M (16 < M <= 128) takes 64 x 64 tiles with K split inside the workgroup
// (k_gemm_mid) when K is a multiple of 1024 (four quarters of whole 4-window rounds), the scale
// rows are 2-byte aligned (checked by the launcher) and the tiles give at least 128 workgroups.
// For M = 65-128 against a weight of at least 8192 rows with 16x16 tile scales and 16-byte
// aligned scale rows, the launcher takes 128-row tiles instead (one workgroup per CU, W read
// once: 0.7-1.8 us faster on the 14336 x 4096 weight); elsewhere 128-row tiles measured no
// faster.  On such a weight the 128-row tiles also serve M = 129-384 (gemm_uses_mid_wide; two
// or three row slices, W re-read from L2): 2-4 us faster than the 256 x 256 tiles with a K split
// at 14336 x 4096 (41-68 us against 45-70 us prequantized), but slower at M = 512 (89 against
// 74 us).  Otherwise past M = 128 the 256 x 256 tiles with their interleaved decode win.
inline bool gemm_uses_mid(int64_t m, int64_t n, int64_t k) {
  return m > 16 && m <= 128 && k > 0 && k % 1024 == 0 && ((m + 63) / 64) * ((n + 63) / 64) >= 128;
}

// The M = 129-384 shapes that take the mid-size kernel's 128-row tiles when W has 16x16 tile
// scales and 16-byte aligned scale rows (checked by the launcher; other layouts split K, so the
// workspace still covers the split).
inline bool gemm_uses_mid_wide(int64_t m, int64_t n, int64_t k) {
  return m > 128 && m <= 384 && k > 0 && k % 1024 == 0 && (n + 63) / 64 >= 128;
}

inline int gemm_k_splits(int64_t m, int64_t n, int64_t k) {
  if (m <= 16 || n % 4 != 0 || k <= 0 || gemm_uses_mid(m, n, k)) return 1;
  const int64_t bm = m <= 64 ? 64 : (m <= 128 ? 128 : 256);
  const int64_t slots = 256 * (m <= 64 ? 2 : 1);
  const int64_t tiles = ((m + bm - 1) / bm) * ((n + 255) / 256);
  if (2 * tiles > slots) return 1;
  const int64_t nwin = (k + 63) / 64;
  int64_t s = slots / tiles;
  if (s > nwin / 4) s = nwin / 4;
  const int64_t cap = k / ((m > 128 ? 4 : 8) * m);  // partial sums vs W's packed codes
  if (s > cap) s = cap;
  if (s > 16) s = 16;
  if (s < 2) return 1;
  const int64_t wps = (nwin + s - 1) / s;
  return (int)((nwin + wps - 1) / wps);  // every split keeps at least one window
}

// Tiled product for m > 16.  `part` (workspace, gemm_k_splits(m, n, k) x m x n floats, 16-byte
// aligned) receives the partial sums when K is split; it may be NULL when it is not.
hipError_t launch_gemm_tile(const GemmOperand &a, const GemmOperand &w, int64_t m, int64_t n,
                            int64_t k, uint16_t *y, int64_t ld_y, float *part,
                            hipStream_t stream);
// Decode-shaped product with the activation quantization fused in (1 <= m <= 16, k <= 4096):
// bf16 A is quantized inside the kernel; aq's codes / scales / gs, where not NULL, receive the
// quantized A (row strides aq.ld_codes / aq.ld_scales).  hipErrorNotSupported (nothing
// launched) for other shapes.
hipError_t launch_gemm_decode_fused(const void *a_bf16, int64_t ld_a, const GemmOperand &aq,
                                    const GemmOperand &w, int64_t m, int64_t n, int64_t k,
                                    uint16_t *y, int64_t ld_y, hipStream_t stream);
// Small M (m <= 16, decode-shaped): W streamed at full width, A decoded in registers.
hipError_t launch_gemm_small_m(const GemmOperand &a, const GemmOperand &w, int64_t m, int64_t n,
                               int64_t k, uint16_t *y, int64_t ld_y, hipStream_t stream);
// Weight-only product (bf16 A, NVFP4 W, 1 <= m <= 16); hipErrorNotSupported (nothing launched)
// for other m.
hipError_t launch_gemm_w4a16(const void *a_bf16, int64_t ld_a, const GemmOperand &w, int64_t m,
                             int64_t n, int64_t k, uint16_t *y, int64_t ld_y, hipStream_t stream);
hipError_t launch_grouped_gemm(const GemmOperand &a, const int32_t *row_index,
                               const int32_t *offsets, int32_t num_groups, const GemmOperand &w,
                               int64_t w_group_rows, int64_t n, int64_t k, int64_t total_rows,
                               uint16_t *y, int64_t ld_y, hipStream_t stream);

// MSE-observer block scales (mse.hip): amax pass, then a per-block search over 18 candidate
// scales; two_d selects 16x16 tiles.
hipError_t launch_quantize_mse(const void *x, int64_t rows, int64_t cols, int64_t ld_x, bool two_d,
                               uint8_t *codes, int64_t ld_codes, uint8_t *scales,
                               int64_t ld_scales, float *gs_out, void *ws, hipStream_t stream);
// MXFP4 (mxfp4.hip): quantize (one pass), dequantize, and the product on the scaled FP4 MFMA.
hipError_t launch_mx_quantize(const void *x, int64_t rows, int64_t cols, int64_t ld_x,
                              uint8_t *codes, int64_t ld_codes, uint8_t *scales, int64_t ld_scales,
                              hipStream_t stream);
hipError_t launch_mx_dequantize(const uint8_t *codes, int64_t ld_codes, const uint8_t *scales,
                                int64_t ld_scales, int64_t rows, int64_t cols, void *y,
                                int64_t ld_y, int out_f32, hipStream_t stream);
hipError_t launch_mx_gemm(const uint8_t *a_codes, int64_t ld_ac, const uint8_t *a_scales,
                          int64_t ld_as, const uint8_t *w_codes, int64_t ld_wc,
                          const uint8_t *w_scales, int64_t ld_ws, int64_t m, int64_t n, int64_t k,
                          uint16_t *y, int64_t ld_y, hipStream_t stream);
// Small M with bf16 activations in one launch; *launched is false when the shape does not fit
// (nothing launched).
hipError_t launch_mx_gemm_fused(const void *a_bf16, int64_t ld_a, uint8_t *aq_codes,
                                int64_t ld_aqc, uint8_t *aq_scales, int64_t ld_aqs,
                                const uint8_t *w_codes, int64_t ld_wc, const uint8_t *w_scales,
                                int64_t ld_ws, int64_t m, int64_t n, int64_t k, uint16_t *y,
                                int64_t ld_y, hipStream_t stream, bool *launched);

}  // namespace nvfp4
