"""Pins for the CPU oracle: values the pages print, closed forms, brute force with exact rationals
and invariants of the format.  Each test is chosen so that a plausible slip in the oracle (a
dropped term, a wrong tie rule, a transposed operand, a wrong scale index, nibble order) fails.
CPU only."""

from fractions import Fraction

import numpy as np
import pytest
import torch

from oracle import nvfp4_oracle as O
from nvfp4_w4a4_quantized_amax_amd import workloads as W

# ---------------------------------------------------------------------------------------------
# Independent exact helpers (no oracle code): enumerate candidates with Fractions.
# ---------------------------------------------------------------------------------------------


def frac_of_bf16(u16):
    return Fraction(float(W.bf16_bits_to_float32(np.uint16(u16))))


def e4m3_candidates():
    """(byte, value) for the 127 non-negative finite OCP E4M3 values, from the bit layout."""
    out = []
    for b in range(0x7F):
        e, m = b >> 3, b & 7
        v = Fraction(m, 8) * Fraction(2) ** -6 if e == 0 else (1 + Fraction(m, 8)) * Fraction(2) ** (e - 7)
        out.append((b, v))
    return out


E2M1_PAGE = [Fraction(0), Fraction(1, 2), Fraction(1), Fraction(3, 2), Fraction(2), Fraction(3),
             Fraction(4), Fraction(6)]


def nearest_fp32(q):
    """Nearest float32 to the exact rational q >= 0 (ties to even), by search among neighbours."""
    if q == 0:
        return np.float32(0)
    approx = np.float32(float(q))
    cands = {approx, np.nextafter(approx, np.float32(np.inf)), np.nextafter(approx, np.float32(0))}
    best = None
    for c in sorted(cands):
        d = abs(Fraction(float(c)) - q)
        key = (d, int(np.array(c, dtype=np.float32).view(np.uint32)) & 1)
        if best is None or key < best[0]:
            best = (key, c)
    return np.float32(best[1])


def nearest_even(target, cands):
    """Index into cands (list of (code, value)) of the nearest value; ties to the even code."""
    best = None
    for code, v in cands:
        key = (abs(v - target), code & 1)
        if best is None or key < best[0]:
            best = (key, code, v)
    return best[1], best[2]


def brute_quantize(x_u16, block_rows=1):
    """Exact brute-force NVFP4 quantization of a tiny bf16 matrix: every E4M3 scale and every
    E2M1 magnitude is tried with exact rational distances."""
    R, C = x_u16.shape
    xs = [[frac_of_bf16(x_u16[r, c]) for c in range(C)] for r in range(R)]
    neg = [[bool(np.uint16(x_u16[r, c]) >> 15) for c in range(C)] for r in range(R)]
    amax = max(abs(v) for row in xs for v in row)
    gs = nearest_fp32(amax / 2688)
    gsf = Fraction(float(gs))
    scales = {}
    nbr = R // block_rows
    sc = np.zeros((nbr, C // 16), dtype=np.uint8)
    for br in range(nbr):
        for bc in range(C // 16):
            bamax = max(abs(xs[r][c]) for r in range(br * block_rows, (br + 1) * block_rows)
                        for c in range(bc * 16, bc * 16 + 16))
            if bamax == 0 or gsf == 0:
                code, val = 0, Fraction(0)
            else:
                code, val = nearest_even(bamax / (6 * gsf), e4m3_candidates())
            sc[br, bc] = code
            scales[(br, bc)] = val
    codes = np.zeros((R, C), dtype=np.uint8)
    values = [[None] * C for _ in range(R)]
    mags = list(enumerate(E2M1_PAGE))
    for r in range(R):
        for c in range(C):
            sb = scales[(r // block_rows, c // 16)]
            if sb == 0:
                idx, mv = 0, Fraction(0)
            else:
                idx, mv = nearest_even(abs(xs[r][c]) / (sb * gsf), mags)
            codes[r, c] = (8 if neg[r][c] else 0) | idx
            values[r][c] = (-1 if neg[r][c] else 1) * mv * sb * gsf
    packed = (codes[:, 0::2] | (codes[:, 1::2] << 4)).astype(np.uint8)
    return packed, sc, gs, values


def rand_bf16(rng, shape, scale=1.0, dist="normal"):
    if dist == "normal":
        a = rng.standard_normal(shape) * scale
    else:
        a = rng.laplace(0, 1, shape) * scale
    return W.to_bf16_bits(a)


# ---------------------------------------------------------------------------------------------
# Values printed on the pages
# ---------------------------------------------------------------------------------------------


def test_e2m1_magnitudes_are_the_pages_list(golden):
    g = golden("e2m1_magnitudes.txt")
    assert list(O.E2M1_MAG) == g["magnitudes"]
    assert g["sign_bits"] + g["exponent_bits"] + g["mantissa_bits"] == 4
    assert [O.e2m1_decode(c) for c in range(8, 16)] == [-v for v in g["magnitudes"]]
    assert O.E2M1_MAX == 6.0


def test_figure1_global_scale(golden):
    g = golden("figure1_global_scale.txt")
    assert O.global_scale(g["amax"]) == np.float32(g["global_scale"])
    # and a whole tensor whose absolute maximum is 10.5 carries that scale
    x = W.to_bf16_bits(np.array([[10.5] + [0.25] * 15]))
    assert O.quantize_1d(x)[2] == np.float32(g["global_scale"])


def test_storage_bits_and_ratios(golden):
    g = golden("format_constants.txt")
    b = O.storage_bits_per_value(4096, 4096, 1)
    assert b["codes_and_block_scales"] == g["bits_per_value"]
    assert b["with_tensor_scale"] > g["bits_per_value"]
    # the storage accountant on the page's INT4 example: 4-bit payload + FP16 scale per 128 / 32
    assert 4 + 16 / 128 == g["int4_g128_fp16_bits"]
    assert 16 / 32 == g["int4_g32_fp16_extra_bits"]
    # "about": 16 / 4.5 = 3.56 and 8 / 4.5 = 1.78
    assert abs(16 / b["codes_and_block_scales"] - g["ratio_vs_fp16"]) < 0.1
    assert abs(8 / b["codes_and_block_scales"] - g["ratio_vs_fp8"]) < 0.05
    b2 = O.storage_bits_per_value(4096, 4096, 16)
    assert b2["codes_and_block_scales"] == 4 + 8 / 256
    # the quantizer's real output sizes agree with the accountant
    x = rand_bf16(np.random.default_rng(5), (32, 64))
    codes, scales, _ = O.quantize_1d(x)
    assert (codes.nbytes + scales.nbytes) * 8 / x.size == g["bits_per_value"]
    assert scales.shape == (32, 64 // int(g["block_1d"]))
    codes2, scales2, _ = O.quantize_2d(x)
    assert scales2.shape == (32 // 16, 64 // 16)


def test_hand_derived_ties(golden):
    g = golden("e2m1_ties.txt")
    vals = [10.5] + g["x"] + [0.0] * 8
    neg = [10.5] + [-v for v in g["x"]] + [0.0] * 8
    x = W.to_bf16_bits(np.array([vals, neg]))
    assert np.all(W.bf16_bits_to_float32(x)[0, 1:8] == np.array(g["x"], dtype=np.float32))
    codes, scales, gs = O.quantize_1d(x)
    assert gs == np.float32(2.0 ** -8)
    assert list(scales[:, 0]) == [0x7E, 0x7E]
    c = O.unpack_codes(codes)
    assert list(c[0, 1:8]) == [int(v) for v in g["codes"]]
    assert list(c[1, 1:8]) == [int(v) for v in g["negative_codes"]]
    assert c[0, 0] == 7 and c[1, 0] == 7


# ---------------------------------------------------------------------------------------------
# Number formats against a library routine (torch's OCP float8_e4m3fn)
# ---------------------------------------------------------------------------------------------


def test_e4m3_decode_matches_torch():
    t = torch.arange(256, dtype=torch.uint8).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    mine = np.array([O.e4m3_decode(b) for b in range(256)])
    assert np.array_equal(np.isnan(t), np.isnan(mine))
    ok = ~np.isnan(t)
    assert np.array_equal(t[ok], mine[ok])
    assert O.E4M3_MAX == 448.0 and O.e4m3_decode(0x7E) == 448.0


def test_e4m3_rounding_matches_torch_cast():
    """Rounding an exact value to the E4M3 grid (the step behind the block scale) agrees with
    torch's round-to-nearest-even cast on random float32 values and on every midpoint."""
    rng = np.random.default_rng(11)
    v = np.concatenate([
        np.exp(rng.uniform(np.log(2.0 ** -11), np.log(448.0), 20000)),
        (O.E4M3_POS[:-1] + O.E4M3_POS[1:]) / 2,            # all 126 midpoints (exact in fp32)
        O.E4M3_POS, [449.0, 455.0, 463.9],                  # grid points, saturation region
    ]).astype(np.float32)
    tv = torch.from_numpy(v).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    mid = (O.E4M3_POS[:-1] + O.E4M3_POS[1:]) / 2
    mine = O._nearest_index(v.astype(np.float64), mid)
    assert np.array_equal(mine, tv.astype(np.int64))


# ---------------------------------------------------------------------------------------------
# Brute force with exact rationals
# ---------------------------------------------------------------------------------------------


def _brute_case(x, block_rows):
    if block_rows == 1:
        codes, scales, gs = O.quantize_1d(x)
    else:
        codes, scales, gs = O.quantize_2d(x)
    bc, bs, bgs, bvals = brute_quantize(x, block_rows)
    assert gs == bgs
    assert np.array_equal(scales, bs)
    assert np.array_equal(codes, bc)
    deq = O.dequantize(codes, scales, gs, block_rows, out="f64")
    exact = np.array([[float(v) for v in row] for row in bvals])
    assert np.array_equal(deq, exact)


@pytest.mark.parametrize("seed", range(6))
def test_brute_force_1d(seed):
    rng = np.random.default_rng(100 + seed)
    shape = [(1, 16), (2, 32), (3, 48), (4, 64), (2, 64), (1, 128)][seed]
    x = rand_bf16(rng, shape, scale=10.0 ** rng.uniform(-3, 3), dist=["normal", "laplace"][seed % 2])
    # plant zeros, a negative zero, an all-zero block and a tiny block
    xf = W.bf16_bits_to_float32(x).copy()
    xf.reshape(-1)[0] = -0.0
    if xf.size >= 32:
        xf.reshape(-1)[16:32] = 0.0
    if xf.size >= 48:
        xf.reshape(-1)[32:48] *= 1e-5
    _brute_case(W.to_bf16_bits(xf), 1)


@pytest.mark.parametrize("seed", range(3))
def test_brute_force_2d(seed):
    rng = np.random.default_rng(200 + seed)
    x = rand_bf16(rng, (32, 32), scale=0.02 * 10 ** seed)
    xf = W.bf16_bits_to_float32(x).copy()
    xf[16:32, 0:16] *= 1e-3           # one quiet tile
    _brute_case(W.to_bf16_bits(xf), 16)


def test_brute_force_constructed_ties():
    """Blocks whose elements sit exactly on E2M1 midpoints and whose bamax sits exactly on E4M3
    midpoints (amax = 10.5 makes gs = 2^-8, so 6 gs = 3/128)."""
    rows = []
    mids = [0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0]
    for sbv in [448.0, 1.75, 0.5, 0.0703125, 2.0 ** -9 * 3]:
        s = sbv * 2.0 ** -8
        row = [6 * s] + [m * s for m in mids] + [-m * s for m in mids] + [0.0]
        rows.append(row)
    e4_mid = [(1.0 + 1.5 / 8) * 2.0 ** -3, 1.9375 * 2, 1.0625 * 0.25]      # E4M3 midpoints
    for mu in e4_mid:
        rows.append([mu * 6 * 2.0 ** -8] + [2.0 ** -10] * 15)
    rows[0][0] = 10.5
    x = W.to_bf16_bits(np.array(rows))
    assert np.array_equal(W.bf16_bits_to_float32(x), np.array(rows, dtype=np.float32)), "not bf16-exact"
    _brute_case(x, 1)


# ---------------------------------------------------------------------------------------------
# Invariants of the format
# ---------------------------------------------------------------------------------------------


def _q1(x):
    return O.quantize_1d(x)


def test_amax_block_gets_top_scale_and_normal_blocks_reach_six():
    rng = np.random.default_rng(7)
    for scale in [1e-6, 0.02, 1.0, 300.0]:
        x = rand_bf16(rng, (64, 256), scale, "laplace")
        codes, scales, gs = _q1(x)
        xf = np.abs(W.bf16_bits_to_float32(x)).reshape(64, 16, 16)
        bamax = xf.max(axis=2)
        assert np.all(scales[bamax == bamax.max()] == 0x7E)
        mags = (O.unpack_codes(codes) & 7).reshape(64, 16, 16)
        normal = scales >= 8
        assert np.all(mags.max(axis=2)[normal] == 7)
        # ratio bound for normal scales: t = bamax / (6 gs) is rounded to 3 mantissa bits, so
        # t / sb lies in [1.0625 / 1.125, 1.0625]: bamax / (sb gs) in [5.667, 6.375], above 5
        r = bamax[normal] / (O.E4M3_POS[scales[normal]] * float(gs))
        assert r.min() >= 6 * 1.0625 / 1.125 and r.max() <= 6.375


def test_round_trip_idempotence():
    rng = np.random.default_rng(8)
    for scale in [0.02, 1.0, 1e4]:
        x = rand_bf16(rng, (32, 128), scale, "normal")
        codes, scales, gs = _q1(x)
        if not np.all((scales == 0) | (scales >= 8)):
            continue
        back = O.dequantize(codes, scales, gs, 1, out="bf16")
        c2, s2, g2 = _q1(back)
        assert g2 == gs and np.array_equal(s2, scales) and np.array_equal(c2, codes)


def test_power_of_two_equivariance_and_sign_symmetry():
    rng = np.random.default_rng(9)
    x = rand_bf16(rng, (16, 64), 1.0, "laplace")
    codes, scales, gs = _q1(x)
    for k in [-20, -1, 3, 7]:
        xk = W.to_bf16_bits(W.bf16_bits_to_float32(x).astype(np.float64) * 2.0 ** k)
        ck, sk, gk = _q1(xk)
        assert np.array_equal(ck, codes) and np.array_equal(sk, scales)
        assert gk == np.float32(gs * 2.0 ** k)
    xn = x ^ np.uint16(0x8000)
    cn, sn, gn = _q1(xn)
    assert gn == gs and np.array_equal(sn, scales)
    assert np.array_equal(cn, codes ^ np.uint8(0x88))


def test_2d_equals_1d_on_identical_rows():
    rng = np.random.default_rng(10)
    row = rand_bf16(rng, (1, 96), 0.5)
    x = np.repeat(row, 16, axis=0)
    c1, s1, g1 = _q1(row)
    c2, s2, g2 = O.quantize_2d(x)
    assert g1 == g2
    assert np.array_equal(s2[0], s1[0])
    assert np.array_equal(c2, np.repeat(c1, 16, axis=0))


def test_gather_commutes_with_quantize():
    rng = np.random.default_rng(12)
    x = rand_bf16(rng, (24, 64), 1.0)
    idx = np.concatenate([np.arange(24), rng.integers(0, 24, 40)])
    rng.shuffle(idx)
    c, s, g = _q1(x)
    cg, sg, gg = _q1(x[idx])
    assert gg == g and np.array_equal(cg, c[idx]) and np.array_equal(sg, s[idx])


def test_zero_tensor_and_signed_zero():
    x = np.zeros((2, 32), dtype=np.uint16)
    x[1, 3] = 0x8000
    c, s, g = _q1(x)
    assert g == 0 and not s.any()
    cu = O.unpack_codes(c)
    assert cu[1, 3] == 8 and cu.sum() == 8


def test_quantization_error_bound():
    """Each reconstructed value is within half a grid gap of the input (nearest rounding), and
    the relative error is smaller with 16-element blocks than with one scale per row
    ([P3] "Why Blocks of 16 Improve Accuracy")."""
    rng = np.random.default_rng(13)
    x = rand_bf16(rng, (64, 512), 1.0, "laplace")
    c, s, g = _q1(x)
    deq = O.dequantize(c, s, g, 1, out="f64")
    xf = W.bf16_bits_to_float32(x).astype(np.float64)
    sb_el = np.repeat(O.E4M3_POS[s], 16, axis=1) * float(g)
    mags = O.E2M1_MAG[O.unpack_codes(c) & 7]
    gap_up = np.interp(mags, O.E2M1_MAG[:-1], np.diff(O.E2M1_MAG), right=0)
    gap_dn = np.interp(mags, O.E2M1_MAG[1:], np.diff(O.E2M1_MAG), left=0)
    half = np.maximum(gap_up, gap_dn) / 2 * sb_el
    assert np.all(np.abs(deq - xf) <= half + 1e-300)
    # one scale per whole row (block = 512) is worse
    err16 = np.mean((deq - xf) ** 2)
    xr = xf.reshape(64, 1, 512)
    sbr = np.abs(xr).max(axis=2, keepdims=True) / 6
    mag = np.abs(xr) / sbr
    idx = np.argmin(np.abs(mag[..., None] - O.E2M1_MAG), axis=-1)
    err_row = np.mean((np.sign(xr) * O.E2M1_MAG[idx] * sbr - xr) ** 2)
    assert err16 < err_row


# ---------------------------------------------------------------------------------------------
# GEMM
# ---------------------------------------------------------------------------------------------


def test_gemm_identity_closed_form():
    """W = I quantized with 16x16 blocks: every diagonal tile has bamax 1 = amax, so it gets
    scale 448 and code 6, i.e. W_hat = 2688 gs_W I.  Then Y = 2688 gs_W A_hat exactly; this pins
    transposes, nibble order and scale indexing."""
    n = 512
    eye = W.to_bf16_bits(np.eye(n))
    wq = O.quantize_2d(eye)
    assert wq[2] == np.float32(1 / 2688)
    d = np.arange(n // 16)
    assert np.all(wq[1][d, d] == 0x7E) and wq[1].sum() == 0x7E * (n // 16)
    a = W.tiny()["a"]
    aq = O.quantize_1d(a)
    y = O.gemm64(aq + (1,), wq + (16,))
    ahat = O.dequantize(*aq, 1, out="f64")
    assert np.array_equal(y, ahat * (2688 * float(wq[2])))


def test_gemm_exact_small_brute_force():
    """Tiny A (3 x 32) and W (5 x 32): compare with an exact rational triple loop over the
    brute-force reconstructed values."""
    rng = np.random.default_rng(14)
    a = rand_bf16(rng, (3, 32), 1.0)
    w = rand_bf16(rng, (5, 32), 0.02)
    aq, wq = O.quantize_1d(a), O.quantize_1d(w)
    _, _, _, av = brute_quantize(a, 1)
    _, _, _, wv = brute_quantize(w, 1)
    y = O.gemm64(aq + (1,), wq + (1,))
    for m in range(3):
        for n in range(5):
            exact = sum(av[m][k] * wv[n][k] for k in range(32))
            assert abs(Fraction(y[m, n]) - exact) <= abs(exact) * Fraction(1, 2 ** 45) + Fraction(1, 2 ** 200)


def test_grouped_gemm_is_dense_per_group():
    rng = np.random.default_rng(15)
    tokens, k, n, e = 12, 32, 16, 3
    a = rand_bf16(rng, (tokens, k), 1.0)
    ws = [rand_bf16(rng, (n, k), 0.02) for _ in range(e)]
    wqs = [O.quantize_2d(w) + (16,) for w in ws]
    aq = O.quantize_1d(a) + (1,)
    row_index = np.array([0, 5, 7, 1, 2, 3, 4, 11, 9, 10], dtype=np.int32)
    offsets = np.array([0, 3, 3, 10], dtype=np.int32)
    y = O.grouped_gemm64(aq, row_index, offsets, wqs)
    full = [O.gemm64(aq, wq) for wq in wqs]
    for g in range(e):
        for i in range(offsets[g], offsets[g + 1]):
            assert np.array_equal(y[i], full[g][row_index[i]])


def test_row_tolerance_is_per_row_norm():
    y = np.array([[3.0, 4.0], [0.0, 1e-3]])
    t = O.row_tolerance(y)
    assert np.allclose(t[:, 0], [5e-3, 1e-6])


def test_gemm_tolerance_admits_the_bf16_store():
    """The bound must hold for the exact product rounded to bf16 (torch's RNE cast) on any
    data, including rows dominated by one element, and must not be looser than needed: an error
    of one full bf16 ulp on a dominant element exceeds it."""
    rng = np.random.default_rng(21)
    y = rng.standard_normal((64, 48)) * np.exp(rng.uniform(-20, 20, (64, 1)))
    y[::3, 0] *= 1e4                                   # dominant elements
    yb = torch.from_numpy(y).to(torch.bfloat16).double().numpy()
    assert np.all(np.abs(yb - y) <= O.gemm_tolerance(y))
    row = np.array([[1.0 + 2.0 ** -7 * 0.999, 1e-6]])   # just below 1 + 1/128
    one_ulp_off = row[0, 0] + 2.0 ** -7
    assert abs(one_ulp_off - row[0, 0]) > O.gemm_tolerance(row)[0, 0]


def test_dequantize_bf16_is_rne_of_fp32():
    codes = np.array([[0x17]], dtype=np.uint8)   # elements: code 7 (6.0), code 1 (0.5)
    codes = np.repeat(codes, 8, axis=1)
    scales = np.array([[0x45]], dtype=np.uint8)  # 1.625 * 2^1 = 3.25
    gs = np.float32(1.0000001)
    f32 = O.dequantize(codes, scales, gs, 1, out="f32")
    assert f32[0, 0] == np.float32(6 * 3.25 * np.float64(gs))
    b = O.dequantize(codes, scales, gs, 1, out="bf16")
    want = torch.from_numpy(f32).to(torch.bfloat16).view(torch.int16).numpy().astype(np.uint16)
    assert np.array_equal(b, want)


def test_f32_to_bf16_ties_match_torch_cast():
    """The fp32 -> bf16 rounding behind the bf16 dequantize, pinned against torch's cast (round
    to nearest, ties to even) on every exact tie: all fp32 patterns whose low half is 0x8000,
    with both signs, every finite exponent and every bf16 mantissa (so both parities of the
    kept bit), plus their neighbours 0x7FFF and 0x8001.  A round-half-up (or half-down) rule
    fails on the ties, a truncating one on the 0x8001 neighbours."""
    sign = np.arange(2, dtype=np.uint32)[:, None, None, None] << 31
    expo = np.arange(255, dtype=np.uint32)[None, :, None, None] << 23
    mant = np.arange(128, dtype=np.uint32)[None, None, :, None] << 16
    low = np.array([0x7FFF, 0x8000, 0x8001], dtype=np.uint32)[None, None, None, :]
    bits = (sign | expo | mant | low).ravel()
    f32 = bits.view(np.float32)
    got = O.f32_to_bf16_bits(f32)
    want = torch.from_numpy(f32.copy()).to(torch.bfloat16).view(torch.int16).numpy()
    want = want.astype(np.uint16)
    assert np.array_equal(got, want)
    ties = (bits & 0xFFFF) == 0x8000
    kept_odd = ((bits >> 16) & 1) == 1
    # on a tie the result is the even neighbour: up when the kept bit is odd, down when even
    assert np.all(got[ties & kept_odd] == ((bits[ties & kept_odd] >> 16) + 1).astype(np.uint16))
    assert np.all(got[ties & ~kept_odd] == (bits[ties & ~kept_odd] >> 16).astype(np.uint16))


# ---------------------------------------------------------------------------------------------
# W4A16 (weights NVFP4, activations bf16)
# ---------------------------------------------------------------------------------------------


def test_w4a16_permutation_closed_form():
    """W = P (a permutation with no fixed points and no 2-cycles, so a transposed operand
    differs) quantized with 1D blocks: each row's one nonzero block has bamax 1 = amax, scale
    448 and code 6, so W_hat = 2688 gs_W P and Y[m, i] = 2688 gs_W A[m, pi(i)] exactly."""
    n = 96
    pi = (np.arange(n) * 5 + 7) % n          # 5 is invertible mod 96; pi^2 != id
    assert np.all(pi != np.arange(n)) and np.any(pi[pi] != np.arange(n))
    p = np.zeros((n, n))
    p[np.arange(n), pi] = 1.0
    wq = O.quantize_1d(W.to_bf16_bits(p))
    assert wq[2] == np.float32(1 / 2688)
    rng = np.random.default_rng(31)
    a = rand_bf16(rng, (5, n), 3.0)
    y = O.gemm64_w4a16(a, wq + (1,))
    af = O.bf16_bits_to_f64(a)
    assert np.array_equal(y, af[:, pi] * (2688 * float(wq[2])))


def test_w4a16_exact_small_brute_force():
    """A (4 x 48, bf16) times a 2D-quantized W (16 x 48): exact rational triple loop over the
    bf16 values of A and the brute-force reconstruction of W."""
    rng = np.random.default_rng(32)
    a = rand_bf16(rng, (4, 48), 2.0)
    w = rand_bf16(rng, (16, 48), 0.05)
    wq = O.quantize_2d(w)
    _, _, _, wv = brute_quantize(w, 16)
    y = O.gemm64_w4a16(a, wq + (16,))
    for m in range(4):
        for n in range(16):
            exact = sum(frac_of_bf16(a[m, k]) * wv[n][k] for k in range(48))
            assert abs(Fraction(y[m, n]) - exact) <= abs(exact) * Fraction(1, 2 ** 45) + Fraction(1, 2 ** 200)


def test_w4a16_equals_w4a4_on_representable_activations():
    """When A is itself an NVFP4 reconstruction that bf16 holds exactly (global scale a power
    of two, so every value has at most 6 significant bits), the weight-only product of those
    bf16 values equals the W4A4 product of the quantized A."""
    rng = np.random.default_rng(33)
    x = rng.standard_normal((6, 64))
    x[0, 0] = 2688 * 2.0 ** -3                # amax = 2688 * 2^-3 -> gs = 2^-3 exactly
    x = np.clip(x, -x[0, 0], x[0, 0])
    aq = O.quantize_1d(W.to_bf16_bits(x))
    assert aq[2] == np.float32(2.0 ** -3)
    a_hat = O.dequantize(*aq, 1, out="f64")
    a_bits = W.to_bf16_bits(a_hat)
    assert np.array_equal(O.bf16_bits_to_f64(a_bits), a_hat)
    wq = O.quantize_2d(rand_bf16(rng, (32, 64), 0.02)) + (16,)
    assert np.array_equal(O.gemm64_w4a16(a_bits, wq), O.gemm64(aq + (1,), wq))


def test_rn_bf16_helper_against_exact_rounding():
    """The GPU tests' report of outputs equal to RN_bf16(Y64) rounds float64 values to bf16 once;
    pinned against exact rational rounding (nearest of the two bf16 neighbours, ties to the even
    one) on random values and on constructed ties."""
    import sys
    import os
    sys.path.insert(0, os.path.dirname(os.path.abspath(__file__)))
    from gpu_helpers import rn_bf16_f64
    rng = np.random.default_rng(3)
    v = rng.standard_normal(300) * np.exp(rng.uniform(-40, 40, 300))
    ties = np.array([1 + 2.0 ** -8, 1 + 3 * 2.0 ** -8, -(3 + 2.0 ** -6), 2.0 ** 20 * (1 + 2.0 ** -8)])
    v = np.concatenate([v, ties, [0.0, -0.0]])
    got = rn_bf16_f64(v)
    for x, g in zip(v, got):
        if x == 0:
            assert g == 0
            continue
        e = int(np.floor(np.log2(abs(x))))
        ulp = Fraction(2) ** (e - 7)
        fx = Fraction(float(x))
        lo = (fx / ulp).__floor__() * ulp
        hi = lo + ulp
        dlo, dhi = fx - lo, hi - fx
        if dlo < dhi or (dlo == dhi and (lo / ulp) % 2 == 0):
            want = lo
        else:
            want = hi
        assert Fraction(float(g)) == want, (x, g, float(want))
