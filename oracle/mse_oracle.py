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
  R19 the error of a candidate is the exact real squared error of the block,
      sum_i (x_i - code value_i * sb * gs)^2, over its 16 values (1D) or 256 values (16x16 tile).
  R20 the candidate with the smallest error wins; among equal errors, the one nearest to c0,
      then the smaller code (so an all-zero block keeps code 0).

How the exact minimum is computed.  Every difference x_i - d_i is exact in float64 (x_i has 8
significant bits, d_i = code value * sb * gs at most 30, and d_i is x_i's own nearest grid value,
so their exponents lie within a few binades of each other and the difference needs < 40 bits).
The squares and the sum are rounded: over n <= 256 non-negative terms the float64 sum is within a
relative n * 2^-53 < 2^-44 of the exact sum.  So two candidates whose float64 errors differ by
more than a relative 2^-40 are ordered correctly; the candidates within 2^-40 of the smallest
float64 error (near or exact ties, e.g. the all-zero block) are re-evaluated exactly with
rational arithmetic (fractions.Fraction) and R20 decides among the exact minima.
"""

from fractions import Fraction

import numpy as np

from oracle import nvfp4_oracle as O

CAND_BELOW, CAND_ABOVE = 16, 1
NEAR_TIE_REL = 2.0 ** -40


def candidate_offsets():
    """Offsets from c0 in order of preference (R20): nearest first, the smaller code first."""
    offs = [0]
    for d in range(1, CAND_BELOW + 1):
        offs.append(-d)
        if d <= CAND_ABOVE:
            offs.append(d)
    return offs


def _recon(codes, sbv, gs):
    """Exact reconstruction code value * sb * gs (<= 2 + 4 + 24 significant bits: exact)."""
    mag = O.E2M1_MAG[codes & 7] * np.where(codes & 8, -1.0, 1.0)
    return mag * sbv * float(gs)


def _exact_error(xvals, codes, sbv, gs):
    """Exact squared error of one block (flattened values, codes, scale value) as a Fraction."""
    g = Fraction(float(gs))
    s = Fraction(float(sbv))
    tot = Fraction(0)
    for x, c in zip(xvals, codes):
        mag = Fraction(float(O.E2M1_MAG[int(c) & 7]))
        d = (-mag if int(c) & 8 else mag) * s * g
        tot += (Fraction(float(x)) - d) ** 2
    return tot


def _blocks(x, block_rows):
    """View of the values as (..., n) blocks: 1D (R, C/16, 16); 2D (R/16, C/16, 256)."""
    R, C = x.shape
    if block_rows == 1:
        return x.reshape(R, C // 16, 16)
    if R % 16:
        raise ValueError("rows must be a multiple of 16 for 16x16 tiles")
    return x.reshape(R // 16, 16, C // 16, 16).transpose(0, 2, 1, 3).reshape(R // 16, C // 16, 256)


def _errors(xb, scale_codes, gs):
    """Float64 squared error of every block of xb (..., n) under the given scale codes (each
    element encoded by R4 under its block's scale).  Within a relative 2^-44 of exact."""
    sbv = O.E4M3_POS[np.asarray(scale_codes, dtype=np.int64)]
    codes = O.element_codes(xb, sbv[..., None], gs)
    return np.sum(np.square(xb - _recon(codes, sbv[..., None], gs)), axis=-1)


def block_errors(x_bf16_bits, scale_codes, gs, block_rows=1):
    """Float64 squared error of every block of a bf16 matrix under the given scale codes."""
    return _errors(_blocks(O._as_f64(x_bf16_bits), block_rows), scale_codes, gs)


def _choose(xb, gs):
    """R18-R20 for the blocks of xb (..., n): the exact-minimum candidate code of each block."""
    c0 = O.block_scale_codes(np.max(np.abs(xb), axis=-1), gs).astype(np.int64)
    offs = candidate_offsets()
    cands = np.stack([np.clip(c0 + d, 0, 126) for d in offs], axis=-1)       # (..., 18)
    errs = np.stack([_errors(xb, cands[..., j], gs) for j in range(len(offs))], axis=-1)
    emin = errs.min(axis=-1, keepdims=True)
    near = errs <= emin * (1.0 + NEAR_TIE_REL)
    # Blocks whose near-minimal candidates all name one code are decided by float64 alone.
    first = np.argmax(near, axis=-1)
    best = np.take_along_axis(cands, first[..., None], axis=-1)[..., 0]
    unique = np.all(~near | (cands == best[..., None]), axis=-1)
    # The rest: exact rational errors of the near-minimal candidates, R20 among the exact minima
    # (candidates are listed in preference order, so the first exact minimum wins).
    for idx in zip(*np.nonzero(~unique)):
        vals = xb[idx]
        exact = {}
        for j in np.nonzero(near[idx])[0]:
            c = int(cands[idx + (j,)])
            if c not in exact:
                codes = O.element_codes(vals, O.E4M3_POS[c], gs)
                exact[c] = _exact_error(vals, codes, O.E4M3_POS[c], gs)
        emin_exact = min(exact.values())
        for j in range(len(offs)):
            c = int(cands[idx + (j,)])
            if c in exact and exact[c] == emin_exact:
                best[idx] = c
                break
    return best


def mse_scale_codes(x_bf16_bits, block_rows=1, gs=None, row_chunk=512):
    """Block-scale codes chosen by the MSE observer, and the global scale.
    x: R x C bf16 bits; block_rows 1 (16-value row blocks) or 16 (16x16 tiles).  gs defaults to
    the tensor's own (R1); passing it lets a subset of rows (whole tiles) be checked alone.
    Rows are processed in chunks (blocks never cross a chunk: it is a multiple of 16 rows)."""
    x = O._as_f64(x_bf16_bits)
    R, C = x.shape
    if block_rows == 16 and R % 16:
        raise ValueError("rows must be a multiple of 16 for 16x16 tiles")
    if gs is None:
        gs = O.global_scale(O.global_amax(x))
    out = np.empty((R // block_rows, C // 16), dtype=np.uint8)
    for r0 in range(0, R, row_chunk):
        xb = _blocks(x[r0:r0 + row_chunk], block_rows)
        out[r0 // block_rows:(r0 + xb.shape[0] * block_rows) // block_rows] = _choose(xb, gs)
    return out, gs


def quantize_mse(x_bf16_bits, block_rows=1, gs=None):
    """NVFP4 quantization with MSE-observer block scales: returns (codes, scales, gs) in the
    same layout as quantize_1d (block_rows 1) or quantize_2d (block_rows 16)."""
    sc, gs = mse_scale_codes(x_bf16_bits, block_rows, gs)
    return encode_with_scales(x_bf16_bits, sc, gs, block_rows) + (gs,)


def encode_with_scales(x_bf16_bits, scale_codes, gs, block_rows=1):
    """Codes of every element under given block-scale codes (R4), packed: (codes, scales)."""
    x = O._as_f64(x_bf16_bits)
    sbv = O.E4M3_POS[np.asarray(scale_codes, dtype=np.int64)]
    if block_rows == 1:
        el = np.repeat(sbv, 16, axis=1)
    else:
        el = np.repeat(np.repeat(sbv, 16, axis=0), 16, axis=1)
    return O.pack_codes(O.element_codes(x, el, gs)), np.asarray(scale_codes, dtype=np.uint8)


def fp32_evaluation_bound(x_bf16_bits, scale_codes, gs, block_rows=1):
    """Upper bound on |E_fp32 - E| for every block, E the exact squared error under the given
    scale codes and E_fp32 any fp32 evaluation that computes d_i = RN(code value * sb * gs),
    e_i = RN(x_i - d_i), RN(e_i^2) and sums the n squares in any order (u = 2^-24):
      |e^_i - e_i| <= delta_i = u (1 + u) |d_i| + u |e_i|,
      |RN(e^_i^2) - e_i^2| <= delta_i (2 |e_i| + delta_i) + u (|e_i| + delta_i)^2,
      summation: gamma_(n-1) = (n-1) u / (1 - (n-1) u) times the sum of the rounded squares.
    The bound is evaluated in float64 and widened by 1 % for that evaluation.  A library that
    evaluates errors this way may pick any candidate within the two candidates' bounds of the
    exact minimum; the GPU tests accept exactly that."""
    u = 2.0 ** -24
    xb = _blocks(O._as_f64(x_bf16_bits), block_rows)
    n = xb.shape[-1]
    sbv = O.E4M3_POS[np.asarray(scale_codes, dtype=np.int64)]
    codes = O.element_codes(xb, sbv[..., None], gs)
    d = np.abs(_recon(codes, sbv[..., None], gs))
    e = np.abs(xb - _recon(codes, sbv[..., None], gs))
    delta = u * (1 + u) * d + u * e
    per = delta * (2 * e + delta) + u * (e + delta) ** 2
    gamma = (n - 1) * u / (1 - (n - 1) * u)
    sq = (e + delta) ** 2 * (1 + u)
    return 1.01 * (np.sum(per, axis=-1) + gamma * np.sum(sq, axis=-1))
