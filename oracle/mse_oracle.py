"""MSE-observer block scales: a plain CPU definition (oracle) of the scale choice that minimizes a
block's squared reconstruction error, for offline weight quantization.

TEST INFRASTRUCTURE ONLY, like `nvfp4_oracle` (whose format, rounding rules and reconstruction
it reuses): only the test-suite, the smoke check and the CPU-baseline leg of the benchmark may
import it; the library never imports, links or calls it.

The pages name MSE-based observers as one of the calibration refinements tried on smaller
models ([P5] "Accelerating large language models with NVFP4 quantization", section "NVFP4
robustness with scale-dependent variability") without giving the procedure.  The readings taken
here (listed in the design notes):
  R18 the global scale stays R1's (amax based); only block scales change.  The candidates for a
      block are the E4M3 codes c0 - 16 .. c0 + 1 (clamped to 0 .. 126), c0 being R3's
      amax-derived code: two binades of smaller scales (which clip the block maximum but refine
      the rest) and the next larger one.  Each candidate encodes the block by R4 under its scale.
  R19 the error of a candidate is evaluated in fp32, in a fixed order, so that the decision is
      reproducible: d_i = RN_fp32(code value_i * sb * gs) (the reconstruction of R7),
      e_i = RN_fp32(x_i - d_i), and the error of 16 consecutive values of a row is the
      left-to-right fp32 sum of RN_fp32(e_i * e_i).  A 16x16 tile combines its 16 row errors
      by a pairwise tree: four rounds, each replacing the error of row r by RN_fp32(s_r + s_(r^k))
      for k = 1, 2, 4, 8.
  R20 the candidate with the smallest error wins; among equal errors, the one nearest to c0,
      then the smaller code (so an all-zero block keeps code 0).
"""

import numpy as np

from oracle import nvfp4_oracle as O

CAND_BELOW, CAND_ABOVE = 16, 1


def candidate_offsets():
    """Offsets from c0 in order of preference: nearest first, the smaller code first."""
    offs = [0]
    for d in range(1, CAND_BELOW + 1):
        offs.append(-d)
        if d <= CAND_ABOVE:
            offs.append(d)
    return offs


def _row_errors(x32, codes, sbv, gs):
    """fp32 error of each 16-value row segment (reading R19).  x32: (..., 16) float32 values;
    codes: (..., 16) E2M1 codes; sbv: (...) block-scale values (float64, exact)."""
    mag = O.E2M1_MAG[codes & 7] * np.where(codes & 8, -1.0, 1.0)
    d = (mag * sbv[..., None] * float(gs)).astype(np.float32)     # RN_fp32 of the exact product
    e = (x32 - d).astype(np.float32)
    sq = (e * e).astype(np.float32)
    s = sq[..., 0].copy()
    for i in range(1, 16):
        s = (s + sq[..., i]).astype(np.float32)
    return s


def _tile_tree(row_err):
    """Pairwise tree over the 16 row errors of each tile; row_err: (..., 16) float32."""
    s = row_err.copy()
    idx = np.arange(16)
    for k in (1, 2, 4, 8):
        s = (s + s[..., idx ^ k]).astype(np.float32)
    return s[..., 0]


def mse_scale_codes(x_bf16_bits, block_rows=1, gs=None):
    """Block-scale codes chosen by the MSE observer, and the global scale.
    x: R x C bf16 bits; block_rows 1 (16-value row blocks) or 16 (16x16 tiles).  gs defaults to
    the tensor's own (R1); passing it lets a subset of rows (whole tiles) be checked alone."""
    x = O._as_f64(x_bf16_bits)
    R, C = x.shape
    if gs is None:
        gs = O.global_scale(O.global_amax(x))
    x32 = x.astype(np.float32)                                      # exact: x is bf16
    if block_rows == 1:
        xb = x.reshape(R, C // 16, 16)
        xb32 = x32.reshape(R, C // 16, 16)
        c0 = O.block_scale_codes(np.max(np.abs(xb), axis=2), gs).astype(np.int64)
    else:
        if R % 16:
            raise ValueError("rows must be a multiple of 16 for 16x16 tiles")
        # (tile row, tile col, row in tile, 16 values)
        xb = x.reshape(R // 16, 16, C // 16, 16).transpose(0, 2, 1, 3)
        xb32 = x32.reshape(R // 16, 16, C // 16, 16).transpose(0, 2, 1, 3)
        c0 = O.block_scale_codes(np.max(np.abs(xb), axis=(2, 3)), gs).astype(np.int64)
    best_c = c0.copy()
    best_e = np.full(c0.shape, np.inf, dtype=np.float32)
    for d in candidate_offsets():
        c = np.clip(c0 + d, 0, 126)
        sbv = O.E4M3_POS[c]
        if block_rows == 1:
            codes = O.element_codes(xb, sbv[..., None], gs)
            err = _row_errors(xb32, codes, sbv, gs)
        else:
            codes = O.element_codes(xb, sbv[..., None, None], gs)
            err = _tile_tree(_row_errors(xb32, codes, np.broadcast_to(sbv[..., None], c.shape + (16,)), gs))
        better = err < best_e                                        # strict: earlier wins ties
        best_c = np.where(better, c, best_c)
        best_e = np.where(better, err, best_e)
    return best_c.astype(np.uint8), gs


def quantize_mse(x_bf16_bits, block_rows=1, gs=None):
    """NVFP4 quantization with MSE-observer block scales: returns (codes, scales, gs) in the
    same layout as quantize_1d (block_rows 1) or quantize_2d (block_rows 16)."""
    sc, gs = mse_scale_codes(x_bf16_bits, block_rows, gs)
    x = O._as_f64(x_bf16_bits)
    sbv = O.E4M3_POS[sc]
    if block_rows == 1:
        el = np.repeat(sbv, 16, axis=1)
    else:
        el = np.repeat(np.repeat(sbv, 16, axis=0), 16, axis=1)
    return O.pack_codes(O.element_codes(x, el, gs)), sc, gs
