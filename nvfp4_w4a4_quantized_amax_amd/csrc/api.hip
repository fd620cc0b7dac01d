// libnvfp4 C ABI (include/nvfp4.h): argument validation, workspace layout and kernel dispatch.
// Validation happens before any HIP call, so every error path is testable without a GPU.
#include "../../include/nvfp4.h"

#include <hip/hip_runtime.h>
#include <stdlib.h>

#include <vector>

#include "launch.hpp"
#include "nvfp4_device.hpp"

using namespace nvfp4;

namespace {

constexpr size_t kAlign = 256;

// Every size and leading dimension the calls accept lies in [0, 2^31): products of two of them
// (byte counts, element counts) then fit in 62 bits, so no size computation below can overflow.
constexpr int64_t kDimLimit = (int64_t)1 << 31;
inline bool dim_ok(int64_t v) { return v >= 0 && v < kDimLimit; }

inline size_t round_up(size_t v, size_t a) { return (v + a - 1) / a * a; }
inline bool aligned(const void *p, size_t a) { return ((uintptr_t)p % a) == 0; }

// Packed-A storage carved from a workspace (after the 4 KiB header).
struct PackedLayout {
  size_t gs_off, codes_off, scales_off, end;
  int64_t ld_codes, ld_scales;
};

PackedLayout packed_layout(int64_t rows, int64_t k) {
  PackedLayout L;
  L.ld_codes = (int64_t)round_up((size_t)(k / 2), 16);
  L.ld_scales = k / 16;
  size_t off = kWsHeaderBytes;
  L.gs_off = off;
  off += kAlign;
  L.codes_off = off;
  off = round_up(off + (size_t)rows * (size_t)L.ld_codes, kAlign);
  L.scales_off = off;
  off = round_up(off + (size_t)rows * (size_t)L.ld_scales, kAlign);
  L.end = off;
  return L;
}

constexpr int64_t kSmallM = 16;

// Workspace bytes for the split-K partial sums of the tiled product (after the packed A).
size_t partial_bytes(int64_t m, int64_t n, int64_t k) {
  if (m <= kSmallM || n <= 0) return 0;
  const int splits = gemm_k_splits(m, n, k);
  return splits > 1 ? round_up((size_t)splits * (size_t)m * (size_t)n * 4, kAlign) : 0;
}

// MXFP4 operand checks.
nvfp4_status check_mx_tensor(const mxfp4_tensor *t, int64_t rows, int64_t cols) {
  if (!t) return NVFP4_ERR_NULL;
  if (!t->codes || !t->scales) return NVFP4_ERR_NULL;
  if (t->rows != rows || t->cols != cols) return NVFP4_ERR_SHAPE;
  if (!dim_ok(rows) || !dim_ok(cols) || !dim_ok(t->ld_codes) || !dim_ok(t->ld_scales))
    return NVFP4_ERR_SHAPE;
  if (cols <= 0 || cols % 32 || rows < 0) return NVFP4_ERR_SHAPE;
  if (t->ld_codes < cols / 2 || t->ld_scales < cols / 32) return NVFP4_ERR_SHAPE;
  if (!aligned(t->codes, 16) || t->ld_codes % 16) return NVFP4_ERR_ALIGN;
  return NVFP4_OK;
}

// Quantized-A storage of the MXFP4 product in a workspace (scale rows padded to 4 bytes).
struct MxLayout {
  size_t codes_off, scales_off, end;
  int64_t ld_codes, ld_scales;
};

MxLayout mx_layout(int64_t rows, int64_t k) {
  MxLayout L;
  L.ld_codes = (int64_t)round_up((size_t)(k / 2), 16);
  L.ld_scales = (int64_t)round_up((size_t)(k / 32), 4);
  L.codes_off = 0;
  L.scales_off = round_up((size_t)rows * (size_t)L.ld_codes, kAlign);
  L.end = round_up(L.scales_off + (size_t)rows * (size_t)L.ld_scales, kAlign);
  return L;
}

// Shape/pointer checks of a quantized operand.
nvfp4_status check_tensor(const nvfp4_tensor *t, int64_t rows, int64_t cols, bool need_16b) {
  if (!t) return NVFP4_ERR_NULL;
  if (!t->codes || !t->scales || !t->global_scale) return NVFP4_ERR_NULL;
  if (t->reserved != 0) return NVFP4_ERR_UNSUPPORTED;
  if (t->block_rows != 1 && t->block_rows != 16) return NVFP4_ERR_UNSUPPORTED;
  if (t->rows != rows || t->cols != cols) return NVFP4_ERR_SHAPE;
  if (!dim_ok(rows) || !dim_ok(cols) || !dim_ok(t->ld_codes) || !dim_ok(t->ld_scales))
    return NVFP4_ERR_SHAPE;
  if (cols <= 0 || cols % 16 || rows < 0) return NVFP4_ERR_SHAPE;
  if (t->block_rows == 16 && rows % 16) return NVFP4_ERR_SHAPE;
  if (t->ld_codes < cols / 2 || t->ld_scales < cols / 16) return NVFP4_ERR_SHAPE;
  if (need_16b && (!aligned(t->codes, 16) || t->ld_codes % 16)) return NVFP4_ERR_ALIGN;
  if (!aligned(t->global_scale, 4)) return NVFP4_ERR_ALIGN;
  return NVFP4_OK;
}

nvfp4_status check_bf16_input(const void *x, int64_t rows, int64_t cols, int64_t ld) {
  if (!x) return NVFP4_ERR_NULL;
  if (!dim_ok(rows) || !dim_ok(cols) || !dim_ok(ld)) return NVFP4_ERR_SHAPE;
  if (cols <= 0 || cols % 16 || ld < cols) return NVFP4_ERR_SHAPE;
  if (!aligned(x, 16) || ld % 8) return NVFP4_ERR_ALIGN;
  // 32-bit chunk indexing inside the quantize kernels
  if (rows * (cols / 8) >= (int64_t)1 << 31) return NVFP4_ERR_SHAPE;
  return NVFP4_OK;
}

inline nvfp4_status hip_status(hipError_t e) { return e == hipSuccess ? NVFP4_OK : NVFP4_ERR_HIP; }

// NVFP4_DEBUG=1: host-side check of the grouped product's device-resident routing arrays (read
// on every grouped call, so a process may switch it on and off).
bool debug_checks() {
  const char *v = getenv("NVFP4_DEBUG");
  return v && v[0] == '1' && v[1] == '\0';
}

// Copies offsets[0..num_groups] and row_index[0..total_rows) to the host (ordered on `stream`)
// and checks them; NVFP4_ERR_HIP if a copy fails.
nvfp4_status check_routing(const int32_t *offsets, int32_t num_groups, const int32_t *row_index,
                           int64_t total_rows, int64_t tokens, hipStream_t stream) {
  hipStreamCaptureStatus capture = hipStreamCaptureStatusNone;
  if (hipStreamIsCapturing(stream, &capture) != hipSuccess) {
    (void)hipGetLastError();
    return NVFP4_OK;
  }
  if (capture != hipStreamCaptureStatusNone) return NVFP4_OK;
  std::vector<int32_t> off((size_t)num_groups + 1);
  std::vector<int32_t> ri(row_index ? (size_t)total_rows : 0);
  if (hipMemcpyAsync(off.data(), offsets, off.size() * sizeof(int32_t), hipMemcpyDeviceToHost,
                     stream) != hipSuccess)
    return NVFP4_ERR_HIP;
  if (row_index && hipMemcpyAsync(ri.data(), row_index, ri.size() * sizeof(int32_t),
                                  hipMemcpyDeviceToHost, stream) != hipSuccess)
    return NVFP4_ERR_HIP;
  if (hipStreamSynchronize(stream) != hipSuccess) return NVFP4_ERR_HIP;
  if (off[0] != 0) return NVFP4_ERR_SHAPE;
  for (int32_t g = 0; g < num_groups; ++g)
    if (off[(size_t)g + 1] < off[(size_t)g]) return NVFP4_ERR_SHAPE;
  if ((int64_t)off[(size_t)num_groups] > total_rows) return NVFP4_ERR_SHAPE;
  for (const int32_t r : ri)
    if (r < 0 || (int64_t)r >= tokens) return NVFP4_ERR_SHAPE;
  return NVFP4_OK;
}

// 1D quantization into explicit buffers, choosing the one-workgroup path for small tensors
// and, ahead of a product in the same call (before_product), the two-kernel path for
// mid-size ones.
nvfp4_status run_quantize_1d(const void *x, int64_t rows, int64_t cols, int64_t ld_x,
                             uint8_t *codes, int64_t ld_codes, uint8_t *scales, int64_t ld_scales,
                             float *gs, void *ws, hipStream_t stream, bool before_product) {
  if (rows * cols <= kSmallMaxElems)
    return hip_status(launch_quantize_small(x, rows, cols, ld_x, codes, ld_codes, scales,
                                            ld_scales, gs, stream));
  if (!(before_product && rows * cols <= kTwoPassBeforeProductMaxElems)) {
    const hipError_t e = launch_quantize_persistent(x, rows, cols, ld_x, codes, ld_codes, scales,
                                                    ld_scales, gs, ws, stream);
    if (e != hipErrorNotSupported) return hip_status(e);
  }
  return hip_status(launch_quantize(x, rows, cols, ld_x, false, codes, ld_codes, scales,
                                    ld_scales, gs, ws, stream));
}

}  // namespace

extern "C" {

const char *nvfp4_status_string(int status) {
  switch (status) {
    case NVFP4_OK: return "NVFP4_OK";
    case NVFP4_ERR_NULL: return "NVFP4_ERR_NULL: a required pointer is NULL";
    case NVFP4_ERR_SHAPE: return "NVFP4_ERR_SHAPE: invalid or unsupported sizes";
    case NVFP4_ERR_ALIGN: return "NVFP4_ERR_ALIGN: pointer or leading dimension misaligned";
    case NVFP4_ERR_WORKSPACE: return "NVFP4_ERR_WORKSPACE: workspace missing or too small";
    case NVFP4_ERR_HIP: return "NVFP4_ERR_HIP: a HIP kernel launch failed";
    case NVFP4_ERR_UNSUPPORTED: return "NVFP4_ERR_UNSUPPORTED: unsupported argument combination";
    default: return "unknown nvfp4 status";
  }
}

int nvfp4_version(void) { return 100; }

size_t nvfp4_quantize_workspace_bytes(int64_t rows, int64_t cols) {
  (void)rows;
  (void)cols;
  return kWsHeaderBytes;
}

size_t nvfp4_gemm_workspace_bytes(int64_t m, int64_t n, int64_t k) {
  if (m < 0 || k <= 0) return kWsHeaderBytes;
  if (!dim_ok(m) || !dim_ok(k) || n >= kDimLimit) return SIZE_MAX;  // no call accepts these
  return packed_layout(m, k).end + partial_bytes(m, n, k);
}

size_t nvfp4_grouped_gemm_workspace_bytes(int64_t tokens, int64_t k, int64_t total_rows,
                                          int32_t num_groups) {
  (void)total_rows;
  (void)num_groups;
  if (tokens < 0 || k <= 0) return kWsHeaderBytes;
  if (!dim_ok(tokens) || !dim_ok(k)) return SIZE_MAX;  // no call accepts these
  return packed_layout(tokens, k).end;
}

nvfp4_status nvfp4_quantize_1d(const void *x, int64_t rows, int64_t cols, int64_t ld_x,
                               const nvfp4_tensor *out, void *ws, size_t ws_bytes, void *stream) {
  if (!out) return NVFP4_ERR_NULL;
  if (rows == 0 && cols > 0 && cols % 16 == 0) return NVFP4_OK;  // nothing to compute or write
  nvfp4_status s = check_bf16_input(x, rows, cols, ld_x);
  if (s) return s;
  s = check_tensor(out, rows, cols, true);
  if (s) return s;
  if (out->block_rows != 1) return NVFP4_ERR_UNSUPPORTED;
  if (!ws) return NVFP4_ERR_WORKSPACE;
  if (ws_bytes < nvfp4_quantize_workspace_bytes(rows, cols) || !aligned(ws, kAlign))
    return NVFP4_ERR_WORKSPACE;
  return run_quantize_1d(x, rows, cols, ld_x, out->codes, out->ld_codes, out->scales,
                         out->ld_scales, out->global_scale, ws, (hipStream_t)stream, false);
}

nvfp4_status nvfp4_quantize_2d(const void *w, int64_t rows, int64_t cols, int64_t ld_w,
                               const nvfp4_tensor *out, void *ws, size_t ws_bytes, void *stream) {
  if (!out) return NVFP4_ERR_NULL;
  if (rows == 0 && cols > 0 && cols % 16 == 0) return NVFP4_OK;  // nothing to compute or write
  nvfp4_status s = check_bf16_input(w, rows, cols, ld_w);
  if (s) return s;
  if (rows % 16) return NVFP4_ERR_SHAPE;
  s = check_tensor(out, rows, cols, true);
  if (s) return s;
  if (out->block_rows != 16) return NVFP4_ERR_UNSUPPORTED;
  if (!ws) return NVFP4_ERR_WORKSPACE;
  if (ws_bytes < nvfp4_quantize_workspace_bytes(rows, cols) || !aligned(ws, kAlign))
    return NVFP4_ERR_WORKSPACE;
  return hip_status(launch_quantize(w, rows, cols, ld_w, true, out->codes, out->ld_codes,
                                    out->scales, out->ld_scales, out->global_scale, ws,
                                    (hipStream_t)stream));
}

nvfp4_status nvfp4_quantize_mse(const void *w, int64_t rows, int64_t cols, int64_t ld_w,
                                const nvfp4_tensor *out, void *ws, size_t ws_bytes, void *stream) {
  if (!out) return NVFP4_ERR_NULL;
  if (rows == 0 && cols > 0 && cols % 16 == 0) return NVFP4_OK;  // nothing to compute or write
  nvfp4_status s = check_bf16_input(w, rows, cols, ld_w);
  if (s) return s;
  s = check_tensor(out, rows, cols, false);
  if (s) return s;
  if (!aligned(out->codes, 8) || out->ld_codes % 8) return NVFP4_ERR_ALIGN;
  if (!ws) return NVFP4_ERR_WORKSPACE;
  if (ws_bytes < nvfp4_quantize_workspace_bytes(rows, cols) || !aligned(ws, kAlign))
    return NVFP4_ERR_WORKSPACE;
  return hip_status(launch_quantize_mse(w, rows, cols, ld_w, out->block_rows == 16, out->codes,
                                        out->ld_codes, out->scales, out->ld_scales,
                                        out->global_scale, ws, (hipStream_t)stream));
}

nvfp4_status nvfp4_dequantize(const nvfp4_tensor *q, void *y, int64_t ld_y, int out_dtype,
                              void *stream) {
  if (!q) return NVFP4_ERR_NULL;
  if (q->rows == 0 && q->cols > 0 && q->cols % 16 == 0) return NVFP4_OK;  // empty
  nvfp4_status s = check_tensor(q, q->rows, q->cols, false);
  if (s) return s;
  if (!y) return NVFP4_ERR_NULL;
  if (out_dtype != NVFP4_OUT_BF16 && out_dtype != NVFP4_OUT_F32) return NVFP4_ERR_UNSUPPORTED;
  if (ld_y < q->cols || !dim_ok(ld_y)) return NVFP4_ERR_SHAPE;
  if (!aligned(q->codes, 4) || q->ld_codes % 4 || !aligned(y, 16) || ld_y % 8)
    return NVFP4_ERR_ALIGN;
  if (q->rows == 0) return NVFP4_OK;
  return hip_status(launch_dequantize(q->codes, q->ld_codes, q->scales, q->ld_scales,
                                      q->global_scale, q->rows, q->cols, q->block_rows, y, ld_y,
                                      out_dtype == NVFP4_OUT_F32, (hipStream_t)stream));
}

nvfp4_status nvfp4_gemm_w4a4(const void *a_bf16, int64_t m, int64_t k, int64_t ld_a,
                             const nvfp4_tensor *a_q, const nvfp4_tensor *w, void *y,
                             int64_t ld_y, void *ws, size_t ws_bytes, void *stream) {
  if (!w) return NVFP4_ERR_NULL;
  if (m < 0 || k <= 0 || k % 16) return NVFP4_ERR_SHAPE;
  if (m == 0) return NVFP4_OK;  // empty product: nothing to compute or write
  if (!y) return NVFP4_ERR_NULL;
  const int64_t n = w->rows;
  nvfp4_status s = check_tensor(w, n, k, true);
  if (s) return s;
  if (n < 1 || n >= ((int64_t)1 << 30) || m >= ((int64_t)1 << 30)) return NVFP4_ERR_SHAPE;
  if (ld_y < n || !dim_ok(ld_y)) return NVFP4_ERR_SHAPE;
  if (!aligned(y, 4) || ld_y % 2) return NVFP4_ERR_ALIGN;
  if (a_bf16) {
    s = check_bf16_input(a_bf16, m, k, ld_a);
    if (s) return s;
    if (a_q) {
      s = check_tensor(a_q, m, k, true);
      if (s) return s;
      if (a_q->block_rows != 1) return NVFP4_ERR_UNSUPPORTED;
    }
  } else {
    s = check_tensor(a_q, m, k, true);
    if (s) return s;
    if (a_q->block_rows != 1) return NVFP4_ERR_UNSUPPORTED;
  }
  if (!ws) return NVFP4_ERR_WORKSPACE;
  if (ws_bytes < nvfp4_gemm_workspace_bytes(m, n, k) || !aligned(ws, kAlign))
    return NVFP4_ERR_WORKSPACE;
  if (m == 0) return NVFP4_OK;

  hipStream_t st = (hipStream_t)stream;
  uint8_t *base = (uint8_t *)ws;
  const PackedLayout L = packed_layout(m, k);
  GemmOperand A;
  A.block_rows = 1;
  if (a_q) {
    A.codes = a_q->codes;
    A.ld_codes = a_q->ld_codes;
    A.scales = a_q->scales;
    A.ld_scales = a_q->ld_scales;
    A.gs = a_q->global_scale;
  } else {
    A.codes = base + L.codes_off;
    A.ld_codes = L.ld_codes;
    A.scales = base + L.scales_off;
    A.ld_scales = L.ld_scales;
    A.gs = (const float *)(base + L.gs_off);
  }
  GemmOperand W{w->codes, w->ld_codes, w->scales, w->ld_scales, w->global_scale, w->block_rows};
  if (a_bf16 && m <= kSmallM) {
    // Decode shapes: the quantization of A runs inside the product kernel (the quantized A is
    // written only where the caller asked for it).
    GemmOperand AQ = A;
    if (!a_q) {
      AQ.codes = nullptr;
      AQ.scales = nullptr;
      AQ.gs = nullptr;
    }
    const hipError_t e = launch_gemm_decode_fused(a_bf16, ld_a, AQ, W, m, n, k, (uint16_t *)y,
                                                  ld_y, st);
    if (e != hipErrorNotSupported) return hip_status(e);
  }
  if (a_bf16) {
    s = run_quantize_1d(a_bf16, m, k, ld_a, (uint8_t *)A.codes, A.ld_codes, (uint8_t *)A.scales,
                        A.ld_scales, (float *)A.gs, ws, st, true);
    if (s) return s;
  }
  if (m <= kSmallM)
    return hip_status(launch_gemm_small_m(A, W, m, n, k, (uint16_t *)y, ld_y, st));
  float *part = partial_bytes(m, n, k) ? (float *)(base + L.end) : nullptr;
  return hip_status(launch_gemm_tile(A, W, m, n, k, (uint16_t *)y, ld_y, part, st));
}

nvfp4_status nvfp4_gemm_w4a16(const void *a_bf16, int64_t m, int64_t k, int64_t ld_a,
                              const nvfp4_tensor *w, void *y, int64_t ld_y, void *stream) {
  if (!w) return NVFP4_ERR_NULL;
  if (m < 0 || k <= 0 || k % 16) return NVFP4_ERR_SHAPE;
  if (m == 0) return NVFP4_OK;
  if (!a_bf16 || !y) return NVFP4_ERR_NULL;
  const int64_t n = w->rows;
  nvfp4_status s = check_tensor(w, n, k, true);
  if (s) return s;
  if (n < 1 || n >= ((int64_t)1 << 30)) return NVFP4_ERR_SHAPE;
  if (ld_y < n || !dim_ok(ld_y)) return NVFP4_ERR_SHAPE;
  if (!aligned(y, 4) || ld_y % 2) return NVFP4_ERR_ALIGN;
  s = check_bf16_input(a_bf16, m, k, ld_a);
  if (s) return s;
  if (m > kSmallM) return NVFP4_ERR_UNSUPPORTED;
  GemmOperand W{w->codes, w->ld_codes, w->scales, w->ld_scales, w->global_scale, w->block_rows};
  return hip_status(launch_gemm_w4a16(a_bf16, ld_a, W, m, n, k, (uint16_t *)y, ld_y,
                                      (hipStream_t)stream));
}

nvfp4_status nvfp4_grouped_gemm_w4a4(const void *a_bf16, int64_t tokens, int64_t k,
                                     int64_t ld_a, const nvfp4_tensor *a_q,
                                     const int32_t *row_index, int64_t total_rows,
                                     const int32_t *offsets, int32_t num_groups,
                                     const nvfp4_tensor *w, int64_t n, void *y, int64_t ld_y,
                                     void *ws, size_t ws_bytes, void *stream) {
  if (!w) return NVFP4_ERR_NULL;
  if (num_groups < 1) return NVFP4_ERR_SHAPE;
  if (num_groups > 1024) return NVFP4_ERR_UNSUPPORTED;
  if (tokens < 0 || total_rows < 0 || k <= 0 || k % 16 || n < 1) return NVFP4_ERR_SHAPE;
  if (total_rows == 0) return NVFP4_OK;  // no routed rows: nothing to compute or write
  if (tokens == 0) return NVFP4_ERR_SHAPE;  // rows to fill but no tokens to take them from
  if (!y || !offsets) return NVFP4_ERR_NULL;
  if (total_rows >= ((int64_t)1 << 30) || tokens >= ((int64_t)1 << 30)) return NVFP4_ERR_SHAPE;
  if (!row_index && tokens != total_rows) return NVFP4_ERR_SHAPE;
  if (!dim_ok(n)) return NVFP4_ERR_SHAPE;  // num_groups * n below stays within 2^41
  nvfp4_status s = check_tensor(w, (int64_t)num_groups * n, k, true);
  if (s) return s;
  if (w->block_rows == 16 && n % 16) return NVFP4_ERR_SHAPE;
  if (ld_y < n || !dim_ok(ld_y)) return NVFP4_ERR_SHAPE;
  if (!aligned(y, 4) || ld_y % 2) return NVFP4_ERR_ALIGN;
  if (a_bf16) {
    s = check_bf16_input(a_bf16, tokens, k, ld_a);
    if (s) return s;
    if (a_q) {
      s = check_tensor(a_q, tokens, k, true);
      if (s) return s;
      if (a_q->block_rows != 1) return NVFP4_ERR_UNSUPPORTED;
    }
  } else {
    s = check_tensor(a_q, tokens, k, true);
    if (s) return s;
    if (a_q->block_rows != 1) return NVFP4_ERR_UNSUPPORTED;
  }
  if (!ws) return NVFP4_ERR_WORKSPACE;
  if (ws_bytes < nvfp4_grouped_gemm_workspace_bytes(tokens, k, total_rows, num_groups) ||
      !aligned(ws, kAlign))
    return NVFP4_ERR_WORKSPACE;

  hipStream_t st = (hipStream_t)stream;
  if (debug_checks()) {
    s = check_routing(offsets, num_groups, row_index, total_rows, tokens, st);
    if (s) return s;
  }
  uint8_t *base = (uint8_t *)ws;
  const PackedLayout L = packed_layout(tokens, k);
  GemmOperand A;
  A.block_rows = 1;
  if (a_q) {
    A.codes = a_q->codes;
    A.ld_codes = a_q->ld_codes;
    A.scales = a_q->scales;
    A.ld_scales = a_q->ld_scales;
    A.gs = a_q->global_scale;
  } else {
    A.codes = base + L.codes_off;
    A.ld_codes = L.ld_codes;
    A.scales = base + L.scales_off;
    A.ld_scales = L.ld_scales;
    A.gs = (const float *)(base + L.gs_off);
  }
  if (a_bf16) {
    s = run_quantize_1d(a_bf16, tokens, k, ld_a, (uint8_t *)A.codes, A.ld_codes,
                        (uint8_t *)A.scales, A.ld_scales, (float *)A.gs, ws, st, true);
    if (s) return s;
  }
  GemmOperand W{w->codes, w->ld_codes, w->scales, w->ld_scales, w->global_scale, w->block_rows};
  return hip_status(launch_grouped_gemm(A, row_index, offsets, num_groups, W, n, n, k, total_rows,
                                        (uint16_t *)y, ld_y, st));
}

size_t nvfp4_mxfp4_gemm_workspace_bytes(int64_t m, int64_t k) {
  if (m <= 0 || k <= 0) return 0;
  if (!dim_ok(m) || !dim_ok(k)) return SIZE_MAX;  // no call accepts these
  return mx_layout(m, k).end;
}

nvfp4_status nvfp4_mxfp4_quantize(const void *x, int64_t rows, int64_t cols, int64_t ld_x,
                                  const mxfp4_tensor *out, void *stream) {
  if (!out) return NVFP4_ERR_NULL;
  if (rows == 0 && cols > 0 && cols % 32 == 0) return NVFP4_OK;  // nothing to compute or write
  nvfp4_status s = check_bf16_input(x, rows, cols, ld_x);
  if (s) return s;
  s = check_mx_tensor(out, rows, cols);
  if (s) return s;
  return hip_status(launch_mx_quantize(x, rows, cols, ld_x, out->codes, out->ld_codes,
                                       out->scales, out->ld_scales, (hipStream_t)stream));
}

nvfp4_status nvfp4_mxfp4_dequantize(const mxfp4_tensor *q, void *y, int64_t ld_y, int out_dtype,
                                    void *stream) {
  if (!q) return NVFP4_ERR_NULL;
  if (q->rows == 0 && q->cols > 0 && q->cols % 32 == 0) return NVFP4_OK;  // empty
  nvfp4_status s = check_mx_tensor(q, q->rows, q->cols);
  if (s) return s;
  if (!y) return NVFP4_ERR_NULL;
  if (out_dtype != NVFP4_OUT_BF16 && out_dtype != NVFP4_OUT_F32) return NVFP4_ERR_UNSUPPORTED;
  if (ld_y < q->cols || !dim_ok(ld_y)) return NVFP4_ERR_SHAPE;
  if (!aligned(y, 16) || ld_y % 8) return NVFP4_ERR_ALIGN;
  if (q->rows * (q->cols / 8) >= (int64_t)1 << 31) return NVFP4_ERR_SHAPE;
  return hip_status(launch_mx_dequantize(q->codes, q->ld_codes, q->scales, q->ld_scales, q->rows,
                                         q->cols, y, ld_y, out_dtype == NVFP4_OUT_F32,
                                         (hipStream_t)stream));
}

nvfp4_status nvfp4_mxfp4_gemm(const void *a_bf16, int64_t m, int64_t k, int64_t ld_a,
                              const mxfp4_tensor *a_q, const mxfp4_tensor *w, void *y,
                              int64_t ld_y, void *ws, size_t ws_bytes, void *stream) {
  if (!w) return NVFP4_ERR_NULL;
  if (m < 0 || k <= 0 || k % 32) return NVFP4_ERR_SHAPE;
  if (m == 0) return NVFP4_OK;  // empty product: nothing to compute or write
  if (!y) return NVFP4_ERR_NULL;
  const int64_t n = w->rows;
  nvfp4_status s = check_mx_tensor(w, n, k);
  if (s) return s;
  if (n < 1 || n >= ((int64_t)1 << 30) || m >= ((int64_t)1 << 30)) return NVFP4_ERR_SHAPE;
  if (ld_y < n || !dim_ok(ld_y)) return NVFP4_ERR_SHAPE;
  if (!aligned(y, 4) || ld_y % 2) return NVFP4_ERR_ALIGN;
  if (a_q) {
    s = check_mx_tensor(a_q, m, k);
    if (s) return s;
  }
  if (a_bf16) {
    s = check_bf16_input(a_bf16, m, k, ld_a);
    if (s) return s;
  } else if (!a_q) {
    return NVFP4_ERR_NULL;
  }
  const uint8_t *ac, *as;
  int64_t ld_ac, ld_as;
  hipStream_t st = (hipStream_t)stream;
  if (a_q) {
    ac = a_q->codes;
    as = a_q->scales;
    ld_ac = a_q->ld_codes;
    ld_as = a_q->ld_scales;
  } else {
    if (!ws) return NVFP4_ERR_WORKSPACE;
    if (ws_bytes < nvfp4_mxfp4_gemm_workspace_bytes(m, k) || !aligned(ws, kAlign))
      return NVFP4_ERR_WORKSPACE;
    const MxLayout L = mx_layout(m, k);
    ac = (const uint8_t *)ws + L.codes_off;
    as = (const uint8_t *)ws + L.scales_off;
    ld_ac = L.ld_codes;
    ld_as = L.ld_scales;
  }
  if (a_bf16) {
    // Small M: one launch that quantizes A itself (writing it only to a_q, if given).
    bool launched = false;
    const hipError_t e = launch_mx_gemm_fused(
        a_bf16, ld_a, a_q ? (uint8_t *)ac : nullptr, ld_ac, a_q ? (uint8_t *)as : nullptr, ld_as,
        w->codes, w->ld_codes, w->scales, w->ld_scales, m, n, k, (uint16_t *)y, ld_y, st,
        &launched);
    if (launched) return hip_status(e);
    s = hip_status(launch_mx_quantize(a_bf16, m, k, ld_a, (uint8_t *)ac, ld_ac, (uint8_t *)as,
                                      ld_as, st));
    if (s) return s;
  }
  return hip_status(launch_mx_gemm(ac, ld_ac, as, ld_as, w->codes, w->ld_codes, w->scales,
                                   w->ld_scales, m, n, k, (uint16_t *)y, ld_y, st));
}

}  // extern "C"
