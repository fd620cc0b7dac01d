"""Pins of the MSE-observer oracle (CPU only): blocks the amax scale already reconstructs exactly
keep it, all-zero blocks keep scale 0, the chosen scale is (up to the fp32 evaluation) the exact
minimum over the candidates, computed independently in rational arithmetic, and the observer
never does worse than the amax rule."""

from fractions import Fraction

import numpy as np
import pytest

from oracle import mse_oracle as M
from oracle import nvfp4_oracle as O
from nvfp4_w4a4_quantized_amax_amd import workloads as W

GRID = [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]   # E2M1 magnitudes ([P2] "What does NVFP4 mean?")


def e4m3_value(c):
    e, m = c >> 3, c & 7
    return Fraction(m, 512) if e == 0 else Fraction(8 + m, 8) * Fraction(2) ** (e - 7)


def nearest_grid(a):
    """Index of the nearest E2M1 magnitude to the rational a >= 0, ties to the even index."""
    best = None
    for i, g in enumerate(GRID):
        d = abs(a - Fraction(g))
        if best is None or d < best[0] or (d == best[0] and i % 2 == 0):
            best = (d, i)
    return best[1]


def exact_error(vals, c, gs):
    """Exact squared error of a block under scale code c: each element takes its nearest E2M1
    value (R4) and is reconstructed exactly."""
    sb = e4m3_value(c)
    g = Fraction(float(gs))
    tot = Fraction(0)
    for v in vals:
        if sb == 0:
            d = Fraction(0)
        else:
            i = nearest_grid(abs(v) / (sb * g))
            d = (-1 if v < 0 else 1) * Fraction(GRID[i]) * sb * g
        tot += (v - d) ** 2
    return tot


def test_candidate_order():
    assert M.candidate_offsets()[:4] == [0, -1, 1, -2]
    assert len(M.candidate_offsets()) == 18 and min(M.candidate_offsets()) == -16


def test_exactly_representable_blocks_keep_amax_scale():
    """gs = 2^-3 (amax 2688 / 8): a block whose maximum is 6 * sb * gs and whose other values
    lie on the grid of sb has error 0 under R3's own scale, so the observer keeps it."""
    rng = np.random.default_rng(1)
    gs = 2.0 ** -3
    codes = [0x38, 0x3C, 0x45, 0x50, 0x7E, 0x2B]
    rows = []
    for c in codes:
        sb = float(e4m3_value(c))
        v = np.array(GRID)[rng.integers(0, 8, 16)] * sb * gs * np.where(rng.random(16) < 0.5, -1, 1)
        v[3] = 6 * sb * gs
        rows.append(v)
    last = np.zeros(16)
    last[-1] = 2688 * gs          # the tensor maximum sets gs = 2^-3 exactly, in a block of its own
    x = np.concatenate(rows + [last])[None, :]
    u = W.to_bf16_bits(x)
    assert np.array_equal(O.bf16_bits_to_f64(u), x)
    sc, g = M.mse_scale_codes(u, 1)
    assert g == np.float32(gs)
    assert list(sc[0, :len(codes)]) == codes


def test_zero_blocks_keep_scale_zero():
    x = np.zeros((2, 64))
    x[1, 20] = 3.0
    sc, _ = M.mse_scale_codes(W.to_bf16_bits(x), 1)
    assert sc[0].tolist() == [0, 0, 0, 0] and sc[1, 0] == 0 and sc[1, 2] == 0


@pytest.mark.parametrize("seed", range(4))
def test_choice_is_the_exact_minimum(seed):
    """Independent exact check: for each block, the chosen code's exact error is the exact
    minimum over the candidates up to the fp32 evaluation of reading R19 (relative 2^-16)."""
    rng = np.random.default_rng(seed + 40)
    x = rng.standard_normal((3, 64)) * np.exp(rng.uniform(-4, 4, (3, 1)))
    x[1, :16] = rng.laplace(size=16) * 5
    x[2, 16:32] = np.where(rng.random(16) < 0.2, 20.0, 1.0) * rng.standard_normal(16)
    u = W.to_bf16_bits(x)
    sc, gs = M.mse_scale_codes(u, 1)
    c0 = O.block_scale_codes(np.abs(O.bf16_bits_to_f64(u)).reshape(3, 4, 16).max(axis=2), gs)
    for r in range(3):
        for b in range(4):
            vals = [Fraction(float(v)) for v in O.bf16_bits_to_f64(u[r, 16 * b:16 * b + 16])]
            cands = sorted({min(max(int(c0[r, b]) + d, 0), 126) for d in M.candidate_offsets()})
            errs = {c: exact_error(vals, c, gs) for c in cands}
            emin = min(errs.values())
            assert int(sc[r, b]) in errs
            assert errs[int(sc[r, b])] <= emin * (1 + Fraction(1, 2 ** 16)) + Fraction(1, 2 ** 300)


def test_never_worse_than_amax_and_often_better():
    rng = np.random.default_rng(7)
    w = W.to_bf16_bits(rng.standard_normal((64, 256)) * 0.02)
    xf = O.bf16_bits_to_f64(w)
    for br in (1, 16):
        base = (O.quantize_1d(w) + (1,)) if br == 1 else (O.quantize_2d(w) + (16,))
        mse = M.quantize_mse(w, br) + (br,)
        eb = (O.dequantize(*base, out="f64") - xf) ** 2
        em = (O.dequantize(*mse, out="f64") - xf) ** 2
        if br == 1:
            blk_b, blk_m = eb.reshape(64, 16, 16).sum(2), em.reshape(64, 16, 16).sum(2)
        else:
            blk_b = eb.reshape(4, 16, 16, 16).sum(axis=(1, 3))
            blk_m = em.reshape(4, 16, 16, 16).sum(axis=(1, 3))
        assert np.all(blk_m <= blk_b * (1 + 2.0 ** -16))
        assert np.mean(blk_m < blk_b * (1 - 2.0 ** -10)) > 0.2
        assert em.sum() < eb.sum()


def test_tile_form_matches_exact_minimum():
    """16x16 tiles: the chosen code's exact tile error is the exact minimum up to fp32."""
    rng = np.random.default_rng(11)
    w = W.to_bf16_bits(rng.standard_normal((16, 32)) * np.exp(rng.uniform(-2, 2, (16, 1))))
    sc, gs = M.mse_scale_codes(w, 16)
    xf = O.bf16_bits_to_f64(w)
    c0 = O.block_scale_codes(np.abs(xf).reshape(1, 16, 2, 16).max(axis=(1, 3)), gs)
    for t in range(2):
        vals = [Fraction(float(v)) for v in xf[:, 16 * t:16 * t + 16].ravel()]
        cands = sorted({min(max(int(c0[0, t]) + d, 0), 126) for d in M.candidate_offsets()})
        errs = {c: exact_error(vals, c, gs) for c in cands}
        assert errs[int(sc[0, t])] <= min(errs.values()) * (1 + Fraction(1, 2 ** 16))
