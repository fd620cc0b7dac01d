"""MXFP4 oracle: a plain, slow, float64 CPU definition of the MXFP4 variant and its product.

TEST INFRASTRUCTURE ONLY, like `nvfp4_oracle` (whose number formats and rounding rule it
reuses): only the test-suite, the smoke check and the CPU-baseline leg of the benchmark may
import it; the library never imports, links or calls it.

What the pages fix ([P2] "NVFP4 versus MXFP4"; [P3] "Why Blocks of 16 Instead of Larger
Groups?", "Why the Block Scale Uses FP8 E4M3", FAQ "What is the difference between NVFP4 and
MXFP4?"; [P4] "Scale layout changes the real storage cost"):
  * the same E2M1 elements as NVFP4;
  * one scale per 32 consecutive values, stored as E8M0: an 8-bit power of two;
  * no tensor-wide scale;
  * NVFP4's finer blocks and fractional scales are said to give less quantization error.

What the pages leave open, and the reading taken here (listed in the design notes):
  R14 the E8M0 scale of a block is X = 2^e with e = floor(log2(bamax)) - 2, the conversion rule
      of the OCP Microscaling (MX) specification that defines the format (2 = the exponent of
      E2M1's largest value, 6 = 1.5 * 2^2); e is clamped to [-127, 127]; an all-zero block takes
      e = -127.  The stored byte is e + 127 (0xFF, NaN, is never produced).
  R15 element code = nearest E2M1 magnitude to the exact real |x| / X, ties to the even code,
      values above 5 give 6 (the block maximum lies in [4X, 8X), so it may saturate), sign bit =
      signbit(x): the rule of reading R4 with sb * gs replaced by X.
  R16 packing as NVFP4 (element 2j in the low nibble); scales row-major, rows x cols/32.
  R17 the MXFP4 product is the exact product of the two reconstructed operands (value = code
      value * X), accepted with the bound of reading R10.
"""

import numpy as np

from oracle import nvfp4_oracle as O

MX_BLOCK = 32
E8M0_BIAS = 127


def e8m0_decode(byte):
    """Value of an E8M0 scale byte: 2^(byte - 127); 0xFF is NaN."""
    byte = int(byte) & 0xFF
    if byte == 0xFF:
        return float("nan")
    return 2.0 ** (byte - E8M0_BIAS)


def shared_exponents(bamax):
    """Reading R14: e = floor(log2(bamax)) - 2, clamped to [-127, 127]; -127 for bamax == 0.

    frexp gives bamax = f * 2^t with f in [0.5, 1), so floor(log2(bamax)) = t - 1 exactly."""
    bamax = np.asarray(bamax, dtype=np.float64)
    _, t = np.frexp(bamax)
    e = t.astype(np.int64) - 1 - 2
    e = np.where(bamax == 0.0, -E8M0_BIAS, e)
    return np.clip(e, -E8M0_BIAS, E8M0_BIAS)


def quantize_mx(x_bf16_bits, row_chunk=256):
    """MXFP4 quantization of a bf16 matrix (R x C, C % 32 == 0): one E8M0 scale per 32
    consecutive row elements, E2M1 codes packed two per byte.  Rows are processed in chunks
    only to bound memory; every block is independent.

    Returns (codes uint8 R x C/2, scales uint8 R x C/32)."""
    x_bf16_bits = np.asarray(x_bf16_bits, dtype=np.uint16)
    if x_bf16_bits.ndim != 2 or x_bf16_bits.shape[1] % MX_BLOCK:
        raise ValueError("cols must be a multiple of 32")
    r, c = x_bf16_bits.shape
    codes = np.empty((r, c // 2), dtype=np.uint8)
    scales = np.empty((r, c // MX_BLOCK), dtype=np.uint8)
    for r0 in range(0, r, row_chunk):
        x = O._as_f64(x_bf16_bits[r0:r0 + row_chunk])
        blocks = x.reshape(x.shape[0], c // MX_BLOCK, MX_BLOCK)
        e = shared_exponents(np.max(np.abs(blocks), axis=2))         # rows x C/32
        scale_el = np.repeat(np.ldexp(1.0, e), MX_BLOCK, axis=1)     # 2^e per element
        codes[r0:r0 + row_chunk] = O.pack_codes(O.element_codes(x, scale_el, 1.0))  # R15
        scales[r0:r0 + row_chunk] = (e + E8M0_BIAS).astype(np.uint8)
    return codes, scales


def dequantize_mx(codes, scales, out="f64"):
    """Reconstruction: code value * 2^(byte - 127), exact in float64 (and in float32 for every
    value a bf16 input can produce)."""
    c = O.unpack_codes(codes)
    mag = O.E2M1_MAG[c & 7]
    sgn = np.where(c & 8, -1.0, 1.0)
    e = np.asarray(scales, dtype=np.int64) - E8M0_BIAS
    x = sgn * mag * np.repeat(np.ldexp(1.0, e), MX_BLOCK, axis=1)
    if out == "f64":
        return x
    f32 = x.astype(np.float32)
    if out == "f32":
        return f32
    if out == "bf16":
        return O.f32_to_bf16_bits(f32)
    raise ValueError(out)


def gemm64_mx(a_mx, w_mx):
    """Y = A . W^T over the reconstructed MXFP4 operands, in float64 (reading R17).
    a_mx, w_mx: (codes, scales) of A (M x K) and W (N x K)."""
    return dequantize_mx(*a_mx) @ dequantize_mx(*w_mx).T


def storage_bits_per_value(rows, cols):
    """Packed codes plus one 8-bit scale per 32 values ([P4] "Scale layout changes the real
    storage cost": group size sets the scale overhead per value)."""
    return (rows * cols // 2 + rows * cols // MX_BLOCK) * 8 / (rows * cols)
