/*
 * libnvfp4 — NVFP4 dynamic W4A4 quantization and quantized GEMM for AMD MI355X (gfx950).
 *
 * Plain C ABI: no C++ types, no exceptions, no torch types.  Every pointer named "device" is a
 * HIP device pointer; every call is asynchronous on `stream` (a hipStream_t passed as void*;
 * NULL means the default stream) and never synchronizes (except for the opt-in NVFP4_DEBUG
 * check of nvfp4_grouped_gemm_w4a4's routing arrays).  The caller owns every buffer; the
 * library allocates nothing per call and keeps no state between calls other than what is
 * written into the caller's workspace and a host counter that tags each call of the
 * single-read quantizer.  Calls may be captured into a HIP graph and replayed: on a capturing
 * stream the activation quantizer takes its two-kernel form (the single-read form's tag would
 * be frozen into the graph), and no call records memset or copy operations.
 *
 * The format (sources cited by page title and section):
 *  - element: 4-bit E2M1 code, 1 sign / 2 exponent / 1 mantissa bit, magnitudes
 *    0, 0.5, 1, 1.5, 2, 3, 4, 6 ("What is NVFP4? 4-bit AI inference on NVIDIA Blackwell
 *    explained", section "What does NVFP4 mean?");
 *  - one FP8 E4M3 block scale per 16 consecutive values and one FP32 global scale per tensor
 *    (same page, "Why does scaling matter so much?"; "NVFP4 Explained: NVIDIA's 4-Bit Format
 *    for Faster AI Inference", "Why the Block Scale Uses FP8 E4M3");
 *  - weights may use one scale per 16x16 tile, activations the 1D 16-element form (first page,
 *    "Why does scaling matter so much?");
 *  - reconstructed value = fp4 value x block scale x global scale ("NVFP4 Explained", section
 *    "How NVFP4 Represents a Value").
 *
 * Readings of what the pages leave open (fixed here, identical in the library and the oracle):
 *  - global scale gs = RN_fp32(amax / 2688), 2688 = 6 * 448; amax = max |x| over the tensor,
 *    recomputed on every call (dynamic quantization);
 *  - block scale = OCP E4M3 value nearest to the exact real bamax / (6 gs), ties to the even
 *    code, saturating at 448 (0x7E); bamax = 0 gives 0;
 *  - element code = nearest E2M1 magnitude to the exact real |x| / (sb gs), ties to the even
 *    code, saturating at 6; sign bit = signbit(x); sb = 0 gives magnitude 0;
 *  - packing: element 2j in the low nibble of byte j, element 2j+1 in the high nibble;
 *  - scales row-major: 1D rows x cols/16, 2D (16x16 tiles) rows/16 x cols/16;
 *  - blocks run along the contiguous axis; rows and cols must be multiples of 16 where blocks
 *    need it (cols always; rows for 16x16 tiles).
 * Codes, scales and gs are bit-exact for finite inputs with amax in [2^-96, bf16 max].
 * Inputs must be finite (NaN/Inf give unspecified codes, never a fault).
 *
 * Empty problems: a call with zero rows (rows == 0, m == 0, total_rows == 0) and otherwise
 * valid sizes computes and writes nothing (not even a global scale) and returns NVFP4_OK; its
 * data pointers may then be NULL.
 */
#ifndef NVFP4_H
#define NVFP4_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  NVFP4_OK = 0,
  NVFP4_ERR_NULL = 1,        /* a required pointer is NULL                                  */
  NVFP4_ERR_SHAPE = 2,       /* bad sizes: cols % 16, rows % 16 for 16x16 tiles, K mismatch,
                                num_groups < 1, sizes too large for 32-bit indexing, ...     */
  NVFP4_ERR_ALIGN = 3,       /* pointer or leading dimension misaligned (see each call)      */
  NVFP4_ERR_WORKSPACE = 4,   /* workspace NULL or smaller than the matching *_workspace_bytes */
  NVFP4_ERR_HIP = 5,         /* a HIP launch failed (the HIP error is lost; check hipGetLastError) */
  NVFP4_ERR_UNSUPPORTED = 6  /* argument combination not supported (e.g. block_rows not 1/16) */
} nvfp4_status;

typedef enum { NVFP4_OUT_BF16 = 0, NVFP4_OUT_F32 = 1 } nvfp4_out_dtype;

/* One NVFP4 matrix of rows x cols, cols contiguous.  All pointers are device pointers.
 *   codes        : packed E2M1 codes, row r starts at codes + r * ld_codes (bytes),
 *                  ld_codes >= cols / 2.
 *   scales       : E4M3 bytes; block_rows == 1: rows x cols/16, block_rows == 16:
 *                  rows/16 x cols/16; scale row i starts at scales + i * ld_scales (bytes).
 *   global_scale : 1 float (for stacked grouped weights: one float per group).
 *   block_rows   : 1 (1D 16-element blocks) or 16 (16x16 tiles).                           */
typedef struct {
  uint8_t *codes;
  int64_t ld_codes;
  uint8_t *scales;
  int64_t ld_scales;
  float *global_scale;
  int64_t rows;
  int64_t cols;
  int32_t block_rows;
  int32_t reserved; /* must be 0 */
} nvfp4_tensor;

/* Human-readable name of a status code (static string, never NULL). */
const char *nvfp4_status_string(int status);

/* Library version as 10000*major + 100*minor + patch. */
int nvfp4_version(void);

/* ---------------------------------------------------------------------------------------------
 * Workspace.  Every call that takes `ws` needs at least the matching number of bytes, 256-byte
 * aligned; its contents need no initialization and carry nothing from one call to the next.  Its
 * first 8 KiB hold the per-workgroup partial maxima of the amax pass (and the grid-barrier slots
 * of the single-read quantizer); the rest holds the quantized activations of the GEMM calls
 * and, for product shapes that split K across workgroups, their fp32 partial sums.
 * Calls that may overlap in time (different streams) need different workspaces.
 * Sizes: every row count, column count, K and leading dimension passed to this library must lie
 * below 2^31 (else NVFP4_ERR_SHAPE); for such sizes the workspace queries return SIZE_MAX.
 * ------------------------------------------------------------------------------------------- */
size_t nvfp4_quantize_workspace_bytes(int64_t rows, int64_t cols);
size_t nvfp4_gemm_workspace_bytes(int64_t m, int64_t n, int64_t k);
size_t nvfp4_grouped_gemm_workspace_bytes(int64_t tokens, int64_t k, int64_t total_rows,
                                          int32_t num_groups);

/* ---------------------------------------------------------------------------------------------
 * nvfp4_quantize_1d — dynamic activation quantization ("NVFP4 Explained", FAQ "Can NVFP4
 * quantize both weights and activations?": dynamically quantized activations; "NVFP4 Dynamic
 * Quantization in Practice", section "The Meaning and Advantages of W4A4": quantization
 * parameters determined in real time).
 *   x      : device bf16, rows x cols, row r at x + r * ld_x (elements); 16-byte aligned,
 *            ld_x % 8 == 0.
 *   out    : out->codes / scales / global_scale receive the result; out->rows == rows,
 *            out->cols == cols, out->block_rows == 1; codes 16-byte aligned, ld_codes % 16 == 0.
 * Computes amax (pass 1) then block scales and codes (pass 2).  cols % 16 == 0.
 * Large tensors run as one workgroup per compute unit that read the tensor once and wait for
 * each other between the passes (a two-kernel form, amax then encode, serves graph capture and
 * devices where one such workgroup per CU does not fit).  The wait is bounded: should other work
 * on the device keep some workgroups from starting, a workgroup that gives up waiting reads the
 * whole tensor for the maximum itself, so the result is the same, only slower.
 * ------------------------------------------------------------------------------------------- */
nvfp4_status nvfp4_quantize_1d(const void *x, int64_t rows, int64_t cols, int64_t ld_x,
                               const nvfp4_tensor *out, void *ws, size_t ws_bytes, void *stream);

/* nvfp4_quantize_2d — weight quantization with one scale per 16x16 tile ("What is NVFP4?",
 * section "Why does scaling matter so much?").  Same arguments as nvfp4_quantize_1d with
 * out->block_rows == 16; rows % 16 == 0 and cols % 16 == 0. */
nvfp4_status nvfp4_quantize_2d(const void *w, int64_t rows, int64_t cols, int64_t ld_w,
                               const nvfp4_tensor *out, void *ws, size_t ws_bytes, void *stream);

/* nvfp4_quantize_mse — offline weight quantization with MSE-observer block scales
 * ("Accelerating large language models with NVFP4 quantization", section "NVFP4 robustness with
 * scale-dependent variability": MSE-based observers as a calibration refinement).  Same
 * arguments as nvfp4_quantize_1d / nvfp4_quantize_2d; out->block_rows (1 or 16) picks the block
 * shape (rows % 16 == 0 for 16), and the result is an ordinary NVFP4 tensor.
 * The global scale is the amax one (as above).  Each block takes, among the E4M3 codes
 * c0 - 16 .. c0 + 1 around the amax-derived code c0 (clamped to 0 .. 126), the scale whose
 * reconstruction has the least squared error sum_i (x_i - code value_i * sb * gs)^2.  The
 * library evaluates that error in fp32:
 *   d_i = RN(code value_i * sb * gs), e_i = RN(x_i - d_i), the 16 values of a row block summed
 *   left to right as RN(e_i * e_i); a 16x16 tile combines its 16 row errors pairwise (row r
 *   with r ^ 1, then ^ 2, ^ 4, ^ 8);
 * so between candidates whose exact errors differ by less than this evaluation resolves it may
 * keep either: the chosen scale's exact error exceeds the exact minimum by at most the two
 * candidates' fp32 evaluation error bounds.  Equal fp32 errors go to the code nearest c0, then
 * the smaller code.  Elements are encoded as by the quantizer under the chosen scale (bit-exact).
 * Codes need 8-byte alignment here (ld_codes % 8 == 0). */
nvfp4_status nvfp4_quantize_mse(const void *w, int64_t rows, int64_t cols, int64_t ld_w,
                                const nvfp4_tensor *out, void *ws, size_t ws_bytes, void *stream);

/* nvfp4_dequantize — reconstruction ("NVFP4 Explained", section "How NVFP4 Represents a
 * Value"): y = RN_fp32(code value x block scale x global scale); NVFP4_OUT_BF16 rounds that
 * float to bf16 (nearest, ties to even).
 *   q  : quantized matrix (block_rows 1 or 16).
 *   y  : device output rows x cols, row r at y + r * ld_y (elements); 16-byte aligned,
 *        ld_y % 8 == 0. */
nvfp4_status nvfp4_dequantize(const nvfp4_tensor *q, void *y, int64_t ld_y, int out_dtype,
                              void *stream);

/* ---------------------------------------------------------------------------------------------
 * nvfp4_gemm_w4a4 — Y = A . W^T with both operands in NVFP4 ("NVFP4 Dynamic Quantization in
 * Practice", section "The Meaning and Advantages of W4A4": weights and activations both 4-bit,
 * matrix multiplication directly at low precision), FP32 accumulation, bf16 output:
 *   Y[m, n] = RN_bf16( RN_fp32(gsA * gsW) * sum_k (cA * sbA)[m, k] * (cW * sbW)[n, k] ).
 * A is m x k and W is n x k, both k-contiguous; Y is m x n.
 *   a_bf16 : if not NULL, device bf16 activations (m x k, row stride ld_a elements, 16-byte
 *            aligned, ld_a % 8 == 0) quantized dynamically inside the call (1D blocks).  a_q may
 *            then be NULL (the quantized A lives in the workspace) or name buffers that receive
 *            it.
 *            If NULL, a_q must describe an already quantized A (block_rows == 1).
 *   w      : quantized weights, n = w->rows, w->cols == k, block_rows 1 or 16.
 *   y      : device bf16 m x n, row stride ld_y elements; 4-byte aligned, ld_y % 2 == 0.
 * Quantized operands: codes 16-byte aligned, ld_codes % 16 == 0.  k % 16 == 0.
 * Accuracy (fp32 accumulation in unspecified order, then the bf16 store): for every element
 *   |Y - Y64| <= 1e-3 * ||Y64[m, :]||_2 + 2^-8 * |Y64[m, n]|,
 * Y64 being the exact product of the two dequantized operands.
 * ------------------------------------------------------------------------------------------- */
nvfp4_status nvfp4_gemm_w4a4(const void *a_bf16, int64_t m, int64_t k, int64_t ld_a,
                             const nvfp4_tensor *a_q, const nvfp4_tensor *w, void *y,
                             int64_t ld_y, void *ws, size_t ws_bytes, void *stream);

/* ---------------------------------------------------------------------------------------------
 * nvfp4_gemm_w4a4_noalloc — nvfp4_gemm_w4a4 without a caller workspace, for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops, harnesses that
 * forbid allocation).  Same arguments, results and errors as nvfp4_gemm_w4a4, with the
 * library's own scratch in place of `ws`: a static device array of NVFP4_NOALLOC_SCRATCH_BYTES
 * (64 MiB) per GPU, loaded on a device at the first call there and held until the process ends.
 *   - Shapes whose nvfp4_gemm_workspace_bytes(m, n, k) exceeds NVFP4_NOALLOC_SCRATCH_BYTES return
 *     NVFP4_ERR_WORKSPACE, launching nothing (e.g. activations quantized inside the call up to
 *     about 59 million values for k = 4096 without a K split).
 *   - The call allocates nothing (no hipMalloc / hipFree); its first call on a device looks up
 *     the array's device address (hipGetSymbolAddress) and keeps it.
 *   - Every call on one GPU shares that GPU's array and leaves its contents behind (nothing in
 *     it needs clearing between calls): calls that may overlap in time on one GPU (different
 *     streams, or host threads) race on it and must be serialized by the caller.
 * ------------------------------------------------------------------------------------------- */
#define NVFP4_NOALLOC_SCRATCH_BYTES (64u * 1024u * 1024u)
nvfp4_status nvfp4_gemm_w4a4_noalloc(const void *a_bf16, int64_t m, int64_t k, int64_t ld_a,
                                     const nvfp4_tensor *a_q, const nvfp4_tensor *w, void *y,
                                     int64_t ld_y, void *stream);

/* ---------------------------------------------------------------------------------------------
 * nvfp4_gemm_w4a16 — weight-only product: NVFP4 weights, 16-bit activations ("NVFP4 Dynamic
 * Quantization in Practice", section "The Meaning and Advantages of W4A4": in W4A16 the 4-bit
 * weights are reconstructed to 16-bit floating point for the multiply, which mainly relieves
 * memory-bound steps; "What is NVFP4?", section "What does W4A4 mean?"), FP32 accumulation,
 * bf16 output:
 *   Y[m, n] = RN_bf16( RN_fp32( gsW * sum_k A[m, k] * (cW * sbW)[n, k] ) ).
 * No activation scale: A's bf16 values are used as they are.
 *   a_bf16 : device bf16 m x k, row stride ld_a elements; 16-byte aligned, ld_a % 8 == 0.
 *   w      : quantized weights, n = w->rows, w->cols == k, block_rows 1 or 16; codes 16-byte
 *            aligned, ld_codes % 16 == 0.  k % 16 == 0.
 *   y      : device bf16 m x n, row stride ld_y; 4-byte aligned, ld_y % 2 == 0.
 * Decode shapes only: 1 <= m <= 16, else NVFP4_ERR_UNSUPPORTED (m == 0 returns NVFP4_OK).
 * No workspace.  Accuracy: the bound of nvfp4_gemm_w4a4, Y64 being the exact product of the
 * bf16 A and the dequantized W.
 * ------------------------------------------------------------------------------------------- */
nvfp4_status nvfp4_gemm_w4a16(const void *a_bf16, int64_t m, int64_t k, int64_t ld_a,
                              const nvfp4_tensor *w, void *y, int64_t ld_y, void *stream);

/* ---------------------------------------------------------------------------------------------
 * nvfp4_grouped_gemm_w4a4 — the mixture-of-experts form ("NVFP4 Dynamic Quantization in
 * Practice", section "The Practical Significance of Full Gemma-4 Quantization Coverage": tokens
 * are routed to a few experts while all experts stay resident).
 *   A (tokens x k) is quantized once with one global scale (or passed quantized in a_q), then
 *   routed row i (0 <= i < total_rows) reads A row row_index[i] (row i if row_index is NULL, in
 *   which case tokens == total_rows), and the rows offsets[g] .. offsets[g+1]-1 are multiplied by
 *   expert g's weights:  Y[i, :] = A[row_index[i], :] . W_g^T.
 *   row_index : device int32[total_rows] or NULL; values in [0, tokens).
 *   offsets   : device int32[num_groups + 1], non-decreasing, offsets[0] == 0,
 *               offsets[num_groups] <= total_rows (rows past it are left untouched).
 *   w         : all experts stacked: w->rows == num_groups * n, w->cols == k; expert g owns rows
 *               g*n .. g*n+n-1; w->global_scale points to num_groups floats (one per expert);
 *               n % 16 == 0 when block_rows == 16.
 *   y         : device bf16 total_rows x n, row stride ld_y.
 * Alignment rules as for nvfp4_gemm_w4a4.  Offsets and row indices live in device memory and
 * are trusted on the hot path (checked only for being non-NULL): values outside the rules above
 * make the kernels read and write out of bounds.  With the environment variable NVFP4_DEBUG=1 the
 * call first copies them to the host (on `stream`, then waits for it) and returns
 * NVFP4_ERR_SHAPE, launching nothing, when offsets[0] != 0, the offsets decrease, the last one
 * exceeds total_rows, or a row index lies outside [0, tokens).  The check is skipped on a stream
 * that is being captured into a graph (it would have to wait).
 * ------------------------------------------------------------------------------------------- */
nvfp4_status nvfp4_grouped_gemm_w4a4(const void *a_bf16, int64_t tokens, int64_t k,
                                     int64_t ld_a, const nvfp4_tensor *a_q,
                                     const int32_t *row_index, int64_t total_rows,
                                     const int32_t *offsets, int32_t num_groups,
                                     const nvfp4_tensor *w, int64_t n, void *y, int64_t ld_y,
                                     void *ws, size_t ws_bytes, void *stream);

/* =============================================================================================
 * MXFP4, the variant the pages contrast with NVFP4 ("What is NVFP4?", section "NVFP4 versus
 * MXFP4"; "NVFP4 Explained", section "Why the Block Scale Uses FP8 E4M3" and FAQ "What is the
 * difference between NVFP4 and MXFP4?"): the same E2M1 elements, one E8M0 power-of-two scale
 * per 32 consecutive values, no tensor scale.
 * Readings (identical in the library and the oracle):
 *  - block scale X = 2^e, e = floor(log2(bamax)) - 2 clamped to [-127, 127] (the conversion rule
 *    of the MX specification), -127 for an all-zero block; stored byte e + 127;
 *  - element code = nearest E2M1 value to x / X, ties to the even code, saturating at 6,
 *    sign bit = signbit(x); packing as NVFP4 (element 2j in the low nibble);
 *  - scales row-major, rows x cols/32 bytes.
 * Codes and scales are bit-exact for finite inputs.
 * ========================================================================================== */

/* One MXFP4 matrix of rows x cols (cols % 32 == 0), cols contiguous; device pointers.
 *   codes  : packed E2M1 codes, row r at codes + r * ld_codes; 16-byte aligned,
 *            ld_codes >= cols / 2 and a multiple of 16.
 *   scales : E8M0 bytes, row r at scales + r * ld_scales, ld_scales >= cols / 32.          */
typedef struct {
  uint8_t *codes;
  int64_t ld_codes;
  uint8_t *scales;
  int64_t ld_scales;
  int64_t rows;
  int64_t cols;
} mxfp4_tensor;

/* nvfp4_mxfp4_quantize — x (device bf16 rows x cols, row stride ld_x elements, 16-byte aligned,
 * ld_x % 8 == 0) into out (out->rows == rows, out->cols == cols).  One pass, no workspace:
 * every block is scaled on its own. */
nvfp4_status nvfp4_mxfp4_quantize(const void *x, int64_t rows, int64_t cols, int64_t ld_x,
                                  const mxfp4_tensor *out, void *stream);

/* nvfp4_mxfp4_dequantize — y = RN_fp32(code value * 2^(byte - 127)) (exact for every value the
 * quantizer produces from bf16), NVFP4_OUT_BF16 rounds that to bf16.  y: device rows x cols,
 * row stride ld_y elements, 16-byte aligned, ld_y % 8 == 0. */
nvfp4_status nvfp4_mxfp4_dequantize(const mxfp4_tensor *q, void *y, int64_t ld_y, int out_dtype,
                                    void *stream);

/* nvfp4_mxfp4_gemm — Y = A . W^T with both operands MXFP4, FP32 accumulation, bf16 output:
 *   Y[m, n] = RN_bf16( sum_k (cA * XA)[m, k] * (cW * XW)[n, k] ).
 * The products run on CDNA4's scaled FP4 MFMA, which applies the E8M0 scales itself.
 *   a_bf16 : if not NULL, device bf16 activations (m x k, ld_a as for the quantize) quantized
 *            to MXFP4 inside the call (written to a_q's buffers when a_q is not NULL; otherwise
 *            an intermediate, held in the workspace or, for m <= 4, inside the product kernel);
 *            if NULL, a_q is the already quantized A.
 *   w      : n = w->rows, w->cols == k.   y : device bf16 m x n, row stride ld_y, 4-byte
 *            aligned, ld_y % 2 == 0.   k % 32 == 0.
 *   ws     : nvfp4_mxfp4_gemm_workspace_bytes(m, k) bytes, 256-byte aligned (may be NULL with
 *            size 0 when a_bf16 is NULL or a_q receives the quantized A).
 * Accuracy: the bound of nvfp4_gemm_w4a4, Y64 being the exact product of the reconstructed
 * operands. */
size_t nvfp4_mxfp4_gemm_workspace_bytes(int64_t m, int64_t k);
nvfp4_status nvfp4_mxfp4_gemm(const void *a_bf16, int64_t m, int64_t k, int64_t ld_a,
                              const mxfp4_tensor *a_q, const mxfp4_tensor *w, void *y,
                              int64_t ld_y, void *ws, size_t ws_bytes, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* NVFP4_H */
