"""NVFP4 oracle: a plain, slow, float64 CPU definition of the format and of the W4A4 product.

TEST INFRASTRUCTURE ONLY.  Only the test-suite, the smoke check and the CPU-baseline leg of the
benchmark may import this module.  The library (the HIP kernels, the C ABI and its Python binding)
never imports, links or calls it, and this module imports nothing from the library.  It shares
no code, table or constant generator with the GPU path.

Sources (web pages, cited by title and section):
  [P1] "NVFP4 Dynamic Quantization in Practice: W4A4 Accelerated Deployment for the Full Gemma-4
       Model Family" (kongchang.com)
  [P2] "What is NVFP4? 4-bit AI inference on NVIDIA Blackwell explained" (hivenet.com)
  [P3] "NVFP4 Explained: NVIDIA's 4-Bit Format for Faster AI Inference" (quirkybit.io)
  [P4] "W4A8 vs NVFP4 quantization on GPUs" (fanout.sh)
  [P5] "Accelerating large language models with NVFP4 quantization" (developers.redhat.com)

What the pages fix:
  * element: E2M1, one sign bit, two exponent bits, one mantissa bit, magnitudes
    0, 0.5, 1, 1.5, 2, 3, 4, 6 ([P2] "What does NVFP4 mean?"; [P3] "How NVFP4 Represents a Value");
  * one FP8 E4M3 scale per 16 consecutive values, one FP32 scale per tensor
    ([P2] "Why does scaling matter so much?"; [P3] "Why the Block Scale Uses FP8 E4M3");
  * weights may share one scale per 16x16 block, activations use the 1D 16-element form
    ([P2] "Why does scaling matter so much?");
  * reconstructed value = fp4 value x block scale x global scale
    ([P3] "How NVFP4 Represents a Value"; [P2] "What does NVFP4 mean?");
  * activations are quantized dynamically, per call ([P1] "The Meaning and Advantages of W4A4";
    [P3] FAQ "Can NVFP4 quantize both weights and activations?").

What the pages leave open, and the reading taken here (each is listed in the design notes):
  R1  global scale gs = RN_fp32(amax / (6 * 448)): the largest block scale then lands on E4M3's
      maximum (the tensor scale "restores range" E4M3 lacks, [P5] "Why NVFP4 works", [P3] "Why the
      Block Scale Uses FP8 E4M3"); Figure 1 of [P5] prints gs = 0.00390625, which this gives at
      amax = 10.5.
  R2  E4M3 is the OCP variant: bias 7, max 448 (0x7E), 0x7F is NaN, no infinities.
  R3  block scale = the finite non-negative E4M3 value nearest to the exact real
      bamax / (6 * gs), ties to the even code, values above 448 give 448, bamax = 0 gives 0.
      It is fitted against the stored (rounded) gs.
  R4  element code = index of the E2M1 magnitude nearest to the exact real |x| / (sb * gs),
      ties to the even index, values above 5 give 6; sb = 0 gives magnitude 0; the sign bit is
      signbit(x) (so -0.0 and small negatives give 0x8).
  R5  packing: element 2j in the low nibble, 2j+1 in the high nibble; scales row-major; 1D scales
      are rows x cols/16, 2D scales are rows/16 x cols/16.
  R6  blocks run along the contiguous axis (cols); shapes must be multiples of 16.
  R7  dequantize = RN_fp32(code value * sb * gs); the bf16 form rounds that fp32 value (RNE).
  R8  GEMM Y = A . W^T is defined as the exact product of the two dequantized operands
      (reconstruction applied to both); the GPU accumulates in fp32 and writes bf16, so it is
      compared with a tolerance, not bit for bit.
  R9  inputs are finite (NaN/Inf raise here).
  R10 GEMM acceptance: |Y - Y64| <= 1e-3 * ||Y64[m, :]||_2 + 2^-8 * |Y64[m, n]|: the stated
      relative budget for the fp32 accumulation plus half a bf16 ulp for the bf16 output.
  R13 W4A16 (the weight-only contrast the pages draw): Y = A . W_hat^T with A's bf16 values
      taken exactly and W_hat the exact reconstruction of the NVFP4 weight; no activation
      scale.  Accepted with R10's bound.

Exactness: every threshold below is a product of at most 31 significant bits (a midpoint with
<= 7 bits times the 24-bit gs), so float64 holds it exactly and every comparison is the exact
real comparison.
"""

import numpy as np

# ---------------------------------------------------------------------------------------------
# Number formats
# ---------------------------------------------------------------------------------------------


def e2m1_decode(code):
    """Value of a 4-bit E2M1 code `s ee m` ([P2] "What does NVFP4 mean?": 1 sign, 2 exponent,
    1 mantissa bit).  Exponent bias 1; exponent field 0 is subnormal (0 or 0.5)."""
    code = int(code)
    s = (code >> 3) & 1
    e = (code >> 1) & 3
    m = code & 1
    if e == 0:
        mag = 0.5 * m
    else:
        mag = 2.0 ** (e - 1) * (1.0 + 0.5 * m)
    return -mag if s else mag


# Magnitudes of codes 0..7, derived from the bit layout above.
E2M1_MAG = np.array([e2m1_decode(c) for c in range(8)], dtype=np.float64)
E2M1_MAX = float(E2M1_MAG[-1])  # 6.0


def e4m3_decode(byte):
    """Value of an OCP FP8 E4M3 byte `s eeee mmm` (reading R2): bias 7, exponent field 0 is
    subnormal (m * 2^-9), 0x7F / 0xFF are NaN, there is no infinity."""
    byte = int(byte) & 0xFF
    s = byte >> 7
    e = (byte >> 3) & 0xF
    m = byte & 7
    if e == 0xF and m == 7:
        return float("nan")
    if e == 0:
        mag = m * 2.0 ** -9
    else:
        mag = (1.0 + m / 8.0) * 2.0 ** (e - 7)
    return -mag if s else mag


# Non-negative finite E4M3 values, codes 0x00..0x7E in increasing order (127 values).
E4M3_POS = np.array([e4m3_decode(b) for b in range(0x7F)], dtype=np.float64)
E4M3_MAX = float(E4M3_POS[-1])  # 448.0


def _nearest_index(values, grid_mid, ties_even=True):
    """For each non-negative value, the index into an increasing grid whose midpoints are
    `grid_mid` (len(grid)-1 of them) of the nearest grid point.  A value exactly on a midpoint
    goes to the even index.  Values beyond the last midpoint take the last index (nearest in
    the finite set).  All comparisons are exact float64 comparisons."""
    below = np.searchsorted(grid_mid, values, side="left")   # midpoints strictly below value
    at_or_below = np.searchsorted(grid_mid, values, side="right")
    tie = at_or_below != below                                # value equals midpoint `below`
    # On a tie between index j=below and j+1, take the even one.
    idx = np.where(tie & ((below & 1) == 1), below + 1, below)
    return idx


# ---------------------------------------------------------------------------------------------
# bf16 helpers (bf16 tensors are carried as uint16 bit patterns)
# ---------------------------------------------------------------------------------------------


def bf16_bits_to_f64(u16):
    u16 = np.asarray(u16, dtype=np.uint16)
    return (u16.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def f32_to_bf16_bits(f32):
    """Round float32 values to bf16 (round to nearest, ties to even) and return the bits."""
    f32 = np.ascontiguousarray(f32, dtype=np.float32)
    u = f32.view(np.uint32).astype(np.uint64)
    lsb = (u >> 16) & 1
    r = (u + 0x7FFF + lsb) >> 16
    return r.astype(np.uint16)


def _check_finite(x):
    if not np.all(np.isfinite(x)):
        raise ValueError("NVFP4 oracle: input must be finite (NaN/Inf are outside the format)")


# ---------------------------------------------------------------------------------------------
# Quantization steps
# ---------------------------------------------------------------------------------------------


def global_amax(x):
    """Per-tensor absolute maximum, recomputed on every call (dynamic quantization,
    [P1] "The Meaning and Advantages of W4A4")."""
    return float(np.max(np.abs(x))) if x.size else 0.0


def global_scale(amax):
    """FP32 tensor scale (reading R1): gs = RN_fp32(amax / (6 * 448)).

    amax and 2688 are exact in float32; float64 division followed by rounding to float32 is the
    correctly rounded float32 quotient (53 >= 2*24 + 2, so the double rounding is innocuous)."""
    return np.float32(amax / (E2M1_MAX * E4M3_MAX))


_E4M3_MID = (E4M3_POS[:-1] + E4M3_POS[1:]) / 2.0  # 126 midpoints, each <= 5 significant bits
_E2M1_MID = (E2M1_MAG[:-1] + E2M1_MAG[1:]) / 2.0  # 0.25 0.75 1.25 1.75 2.5 3.5 5


def block_scale_codes(bamax, gs):
    """E4M3 block-scale bytes for an array of block maxima (reading R3).

    The nearest E4M3 value to bamax / (6 gs) is found by comparing bamax with mid * 6 * gs for
    each E4M3 midpoint: exact in float64 (<= 5 + 2 + 24 significant bits)."""
    bamax = np.asarray(bamax, dtype=np.float64)
    gs = float(gs)
    if gs == 0.0:
        return np.zeros(bamax.shape, dtype=np.uint8)
    thresholds = _E4M3_MID * E2M1_MAX * gs  # exact
    idx = _nearest_index(bamax.ravel(), thresholds).reshape(bamax.shape)
    idx = np.where(bamax == 0.0, 0, idx)
    return idx.astype(np.uint8)  # the E4M3 byte equals its index among the positive values


def element_codes(x, sb_value, gs):
    """E2M1 codes (sign bit included) of elements x given each element's block-scale value
    (reading R4).  The nearest magnitude to |x| / (sb gs) is found by comparing |x| with
    mid * sb * gs for the 7 E2M1 midpoints: exact in float64 (<= 3 + 4 + 24 bits)."""
    x = np.asarray(x, dtype=np.float64)
    sb_value = np.broadcast_to(np.asarray(sb_value, dtype=np.float64), x.shape)
    a = np.abs(x)
    thr = _E2M1_MID[None, :] * (sb_value.reshape(-1, 1) * float(gs))  # exact
    av = a.reshape(-1, 1)
    below = np.sum(thr < av, axis=1)
    at_or_below = np.sum(thr <= av, axis=1)
    tie = at_or_below != below
    mag = np.where(tie & ((below & 1) == 1), below + 1, below)
    mag = np.where(sb_value.reshape(-1) == 0.0, 0, mag)
    sign = np.signbit(x.reshape(-1)).astype(np.int64)
    return ((sign << 3) | mag).reshape(x.shape).astype(np.uint8)


def pack_codes(codes):
    """Two codes per byte, element 2j in the low nibble (reading R5)."""
    codes = np.asarray(codes, dtype=np.uint8)
    return (codes[..., 0::2] | (codes[..., 1::2] << 4)).astype(np.uint8)


def unpack_codes(packed):
    packed = np.asarray(packed, dtype=np.uint8)
    out = np.empty(packed.shape[:-1] + (packed.shape[-1] * 2,), dtype=np.uint8)
    out[..., 0::2] = packed & 0xF
    out[..., 1::2] = packed >> 4
    return out


def _as_f64(x_bf16_bits):
    x = bf16_bits_to_f64(x_bf16_bits)
    _check_finite(x)
    return x


def quantize_1d(x_bf16_bits, row_chunk=256):
    """Dynamic 1D NVFP4 quantization of a bf16 matrix (R x C, C % 16 == 0): one E4M3 scale per
    16 consecutive row elements, one FP32 scale per tensor ([P2] "Why does scaling matter so
    much?"; [P3] "How NVFP4 Represents a Value").

    Returns (codes uint8 R x C/2, scales uint8 R x C/16, gs float32)."""
    x = _as_f64(x_bf16_bits)
    if x.shape[1] % 16:
        raise ValueError("cols must be a multiple of 16")
    gs = global_scale(global_amax(x))
    codes, scales = encode_1d(x_bf16_bits, gs, row_chunk)
    return codes, scales, gs


def encode_1d(x_bf16_bits, gs, row_chunk=256):
    """The block-scale and code steps of quantize_1d for given rows under a given global scale
    (1D blocks are row-local, so any subset of rows can be encoded on its own once gs is known).
    Returns (codes, scales)."""
    x = _as_f64(x_bf16_bits)
    R, C = x.shape
    codes = np.empty((R, C // 2), dtype=np.uint8)
    scales = np.empty((R, C // 16), dtype=np.uint8)
    for r0 in range(0, R, row_chunk):
        xb = x[r0:r0 + row_chunk].reshape(-1, C // 16, 16)
        bamax = np.max(np.abs(xb), axis=2)
        sbc = block_scale_codes(bamax, gs)
        sbv = E4M3_POS[sbc]
        c = element_codes(xb, sbv[:, :, None], gs)
        codes[r0:r0 + row_chunk] = pack_codes(c.reshape(-1, C))
        scales[r0:r0 + row_chunk] = sbc
    return codes, scales


def quantize_2d(w_bf16_bits):
    """2D NVFP4 quantization for weights: each 16x16 tile shares one E4M3 scale
    ([P2] "Why does scaling matter so much?": 16 x 16 weight blocks share scaling information).

    Returns (codes uint8 R x C/2, scales uint8 R/16 x C/16, gs float32)."""
    w = _as_f64(w_bf16_bits)
    R, C = w.shape
    if R % 16 or C % 16:
        raise ValueError("rows and cols must be multiples of 16")
    gs = global_scale(global_amax(w))
    codes, scales = encode_2d(w_bf16_bits, gs)
    return codes, scales, gs


def encode_2d(w_bf16_bits, gs):
    """The block-scale and code steps of quantize_2d for a band of whole 16-row tiles under a
    given global scale.  Returns (codes, scales)."""
    w = _as_f64(w_bf16_bits)
    R, C = w.shape
    tiles = np.abs(w).reshape(R // 16, 16, C // 16, 16)
    bamax = tiles.max(axis=(1, 3))
    sbc = block_scale_codes(bamax, gs)
    sbv_el = np.repeat(np.repeat(E4M3_POS[sbc], 16, axis=0), 16, axis=1)
    c = element_codes(w, sbv_el, gs)
    return pack_codes(c), sbc


def dequantize(codes, scales, gs, block_rows=1, out="f32"):
    """Reconstruction ([P3] "How NVFP4 Represents a Value"): value = fp4 x block scale x global
    scale, rounded once to float32 (reading R7); out="bf16" returns the RNE bf16 bits of that
    float32 value, out="f64" the exact product."""
    c = unpack_codes(codes)
    R, C = c.shape
    mag = E2M1_MAG[c & 7]
    sgn = np.where(c & 8, -1.0, 1.0)
    sb = E4M3_POS[np.asarray(scales, dtype=np.int64)]
    sb_el = np.repeat(sb, 16, axis=1)
    if block_rows == 16:
        sb_el = np.repeat(sb_el, 16, axis=0)
    exact = sgn * mag * sb_el * float(gs)  # <= 2 + 4 + 24 significant bits: exact
    if out == "f64":
        return exact
    f32 = exact.astype(np.float32)
    if out == "f32":
        return f32
    if out == "bf16":
        return f32_to_bf16_bits(f32)
    raise ValueError(out)


# ---------------------------------------------------------------------------------------------
# W4A4 product
# ---------------------------------------------------------------------------------------------


def gemm64(a_q, w_q):
    """Y = A . W^T over the dequantized operands, in float64 (reading R8).

    a_q, w_q: (codes, scales, gs, block_rows).  A is M x K, W is N x K, both K-contiguous.
    Each product of two decoded values is exact in float64; the sum over K is a float64 matmul."""
    a = dequantize(a_q[0], a_q[1], a_q[2], a_q[3], out="f64")
    w = dequantize(w_q[0], w_q[1], w_q[2], w_q[3], out="f64")
    return a @ w.T


def grouped_gemm64(a_q, row_index, offsets, w_list):
    """Grouped (mixture-of-experts) product ([P1] "The Practical Significance of Full Gemma-4
    Quantization Coverage": tokens are routed to a few experts).  Grouped row i reads quantized
    activation row row_index[i] (or row i when row_index is None); rows offsets[e]..offsets[e+1]
    are multiplied by expert e's weight w_list[e] (each with its own global scale)."""
    a = dequantize(a_q[0], a_q[1], a_q[2], a_q[3], out="f64")
    if row_index is not None:
        a = a[np.asarray(row_index, dtype=np.int64)]
    total = int(offsets[-1])
    n = w_list[0][0].shape[0]
    y = np.zeros((total, n), dtype=np.float64)
    for e, wq in enumerate(w_list):
        lo, hi = int(offsets[e]), int(offsets[e + 1])
        if hi > lo:
            w = dequantize(wq[0], wq[1], wq[2], wq[3], out="f64")
            y[lo:hi] = a[lo:hi] @ w.T
    return y


def gemm64_w4a16(a_bf16_bits, w_q):
    """Weight-only product W4A16 (reading R13): the weights are stored in NVFP4 and
    reconstructed to 16-bit floating point, the activations stay 16-bit
    ([P1] "The Meaning and Advantages of W4A4": W4A16 dequantizes the 4-bit weights for a
    high-precision multiply; [P2] "What does W4A4 mean?"; [P3] "What W4A4, W4A8, and W4A16
    Mean").

    a_bf16_bits: uint16 M x K (bf16 bit patterns), used at their exact values.
    w_q: (codes, scales, gs, block_rows) of the N x K weight.
    Y = A . W_hat^T in float64, W_hat the exact reconstruction (code value * block scale * gs)."""
    a = _as_f64(a_bf16_bits)
    w = dequantize(w_q[0], w_q[1], w_q[2], w_q[3], out="f64")
    return a @ w.T


def row_tolerance(y64, rel=1e-3):
    """Accumulation part of the acceptance bound: rel * ||Y64[m, :]||_2 (same bound for every
    column of row m)."""
    return rel * np.sqrt(np.sum(np.square(y64), axis=1, keepdims=True))


def gemm_tolerance(y64, rel=1e-3):
    """Acceptance bound per output element (reading R10): the accumulation budget
    rel * ||Y64[m, :]||_2 plus the rounding of the bf16 store, at most half a bf16 ulp of the
    value, i.e. 2^-8 * |Y64[m, n]| (bf16 keeps 8 significant bits).  Without the second term the
    bound fails on the exact product itself wherever one element dominates its row."""
    return row_tolerance(y64, rel) + np.abs(y64) * 2.0 ** -8


def storage_bits_per_value(rows, cols, block_rows=1):
    """Storage of a quantized tensor, in bits per value: packed codes + E4M3 scales + one FP32
    tensor scale ([P3] "How NVFP4 Represents a Value": about 4.5 bits per value before the
    per-tensor overhead)."""
    code_bytes = rows * cols // 2
    scale_bytes = (rows // block_rows) * (cols // 16)
    return {"with_tensor_scale": (code_bytes + scale_bytes + 4) * 8 / (rows * cols),
            "codes_and_block_scales": (code_bytes + scale_bytes) * 8 / (rows * cols)}
