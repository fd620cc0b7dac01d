"""GPU parity of the weight-only W4A16 product (bf16 activations, NVFP4 weights) against the
float64 oracle: |Y - Y64| <= 1e-3 * ||Y64[m, :]||_2 + 2^-8 |Y64[m, n]| for every element, with
Y64 the exact product of the bf16 A and the dequantized W.  The quantized W is first checked
byte for byte against the oracle's quantization of the same bf16 weights."""

import numpy as np
import pytest
import torch

from oracle import nvfp4_oracle as O
from nvfp4_w4a4_quantized_amax_amd import workloads as W
from gpu_helpers import assert_codes_equal, check_gemm, dev_bf16, host_q

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def nv():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from nvfp4_w4a4_quantized_amax_amd import nvfp4
    return nvfp4


def quantized_w(nv, w_u16, br, what):
    wq = (nv.quantize_2d if br == 16 else nv.quantize_1d)(dev_bf16(w_u16))
    ow = (O.quantize_2d(w_u16) if br == 16 else O.quantize_1d(w_u16)) + (br,)
    wc, ws, wg = host_q(wq)
    assert np.float32(wg) == ow[2]
    assert_codes_equal(wc, ow[0], what + " W codes")
    assert_codes_equal(ws, ow[1], what + " W scales")
    return wq, ow


# K <= 4096 runs the persistent form; larger K the one-band-per-workgroup form.  Ragged N and K
# (partial 128-wide windows, a single 16-value block) and every M from 1 to 16 appear.
@pytest.mark.parametrize("m,n,k,br", [
    (1, 512, 1024, 16), (7, 80, 1040, 1), (16, 512, 4096, 16), (3, 48, 16, 1), (1, 16, 32, 1),
    (12, 272, 4112, 16), (2, 256, 8192, 1), (16, 96, 14336, 16), (5, 1008, 2000, 16),
])
def test_shapes(nv, m, n, k, br):
    rng = np.random.default_rng(m * 11 + n * 5 + k)
    a = W.to_bf16_bits(W.normal_with_outliers(rng, m, k, 0.01, 20.0))
    w = W.to_bf16_bits(rng.standard_normal((n, k)) * 0.02)
    wq, ow = quantized_w(nv, w, br, f"{m}x{n}x{k}")
    y = nv.gemm_w4a16(dev_bf16(a), wq)
    assert y.shape == (m, n)
    check_gemm(y, O.gemm64_w4a16(a, ow), what=f"w4a16 {m}x{n}x{k} b{br}")


# A single activation row: K <= 4096 (K a multiple of 128) runs the band kernel; with N >= 8192
# and K = 8192 the GEMV form (no MFMA, no LDS reduction); other shapes the streaming form.
@pytest.mark.parametrize("n,k,br", [(1000, 2048, 1), (4112, 4096, 16), (272, 8192, 16),
                                    (48, 4096, 1), (18, 2048, 1), (8200, 2048, 1),
                                    (8208, 4096, 16), (8192, 8192, 1)])
def test_single_row_shapes(nv, n, k, br):
    rng = np.random.default_rng(n + k + br)
    a = W.to_bf16_bits(W.normal_with_outliers(rng, 1, k, 0.01, 20.0))
    w = W.to_bf16_bits(rng.standard_normal((n, k)) * 0.02)
    wq, ow = quantized_w(nv, w, br, f"1x{n}x{k}")
    y = nv.gemm_w4a16(dev_bf16(a), wq)
    check_gemm(y, O.gemm64_w4a16(a, ow), what=f"w4a16 single row 1x{n}x{k} b{br}")


def test_single_row_long_k_sampled(nv):
    """GEMV form with K = 8192 (8 blocks per lane) on 8192 x 8192 weights with 16x16 tiles:
    W checked byte for byte on sampled bands, Y on their columns."""
    rng = np.random.default_rng(77)
    n = k = 8192
    w = W.to_bf16_bits(rng.standard_normal((n, k)) * 0.02)
    a = W.to_bf16_bits(W.normal_with_outliers(rng, 1, k, 0.01, 20.0))
    wq = nv.quantize_2d(dev_bf16(w))
    wc, ws, wg = host_q(wq)
    gw = O.global_scale(float(np.max(np.abs(W.bf16_bits_to_float32(w)))))
    assert np.float32(wg) == gw
    bands = np.unique(np.concatenate([[0, 511], rng.choice(512, 20, replace=False)]))
    rows = (bands[:, None] * 16 + np.arange(16)).ravel()
    oc, os_ = O.encode_2d(w[rows], gw)
    assert_codes_equal(wc[rows], oc, "W codes")
    assert_codes_equal(ws[bands], os_, "W scales")
    y = nv.gemm_w4a16(dev_bf16(a), wq)
    check_gemm(y.cpu()[:, rows], O.gemm64_w4a16(a, (oc, os_, gw, 16)), what="w4a16 gemv 8192^2")


def test_permutation_closed_form(nv):
    """A permutation weight (1D blocks) gives W_hat = 2688 gs_W P, so Y[m, i] must be
    RN_bf16(A[m, pi(i)] * 2688 gs_W): pins the operand order, nibble order and scale indexing."""
    n = 256
    pi = (np.arange(n) * 37 + 11) % n
    p = np.zeros((n, n))
    p[np.arange(n), pi] = 1.0
    wq, ow = quantized_w(nv, W.to_bf16_bits(p), 1, "permutation")
    rng = np.random.default_rng(7)
    a = W.to_bf16_bits(rng.standard_normal((9, n)) * 4.0)
    y = nv.gemm_w4a16(dev_bf16(a), wq)
    y64 = O.bf16_bits_to_f64(a)[:, pi] * (2688 * float(ow[2]))
    check_gemm(y, y64, what="w4a16 permutation")


def test_rows_of_very_different_magnitude(nv):
    """bf16 activations are used as they are, with no scale of their own: rows near 1e-30 and
    near 1e30 in one call each meet their own row's bound."""
    rng = np.random.default_rng(8)
    k, n = 1024, 256
    a = rng.standard_normal((4, k))
    a[0] *= 1e-30
    a[1] *= 1e30
    a[2, ::2] *= 1e-25                          # mixed magnitudes inside a row
    a = W.to_bf16_bits(a)
    wq, ow = quantized_w(nv, W.to_bf16_bits(rng.standard_normal((n, k)) * 0.02), 16, "range")
    y = nv.gemm_w4a16(dev_bf16(a), wq)
    check_gemm(y, O.gemm64_w4a16(a, ow), what="w4a16 magnitudes")


def test_strided_activation_and_output(nv):
    """A is a column slice of a wider matrix (ld_a > k) and Y is written into a wider buffer;
    the padding columns of Y stay untouched."""
    rng = np.random.default_rng(9)
    m, n, k = 6, 128, 512
    full = W.to_bf16_bits(rng.standard_normal((m, k + 64)))
    wq, ow = quantized_w(nv, W.to_bf16_bits(rng.standard_normal((n, k)) * 0.02), 1, "strided")
    a_dev = dev_bf16(full)[:, 32:32 + k]
    ybuf = torch.full((m, n + 8), 7.0, dtype=torch.bfloat16, device="cuda")
    nv.gemm_w4a16(a_dev, wq, y=ybuf[:, :n])
    check_gemm(ybuf[:, :n], O.gemm64_w4a16(full[:, 32:32 + k], ow), what="w4a16 strided")
    assert torch.all(ybuf[:, n:] == 7.0)


def test_zero_activation_and_zero_weight(nv):
    rng = np.random.default_rng(10)
    w = W.to_bf16_bits(rng.standard_normal((64, 256)) * 0.02)
    wq, _ = quantized_w(nv, w, 16, "zero A")
    y = nv.gemm_w4a16(torch.zeros((3, 256), dtype=torch.bfloat16, device="cuda"), wq)
    assert torch.all(y == 0)
    zq, _ = quantized_w(nv, np.zeros((64, 256), dtype=np.uint16), 16, "zero W")
    y = nv.gemm_w4a16(dev_bf16(W.to_bf16_bits(rng.standard_normal((3, 256)))), zq)
    assert torch.all(y == 0)


def test_decode_config_full_size(nv):
    """The 14336 x 4096 decode weight (16x16 blocks) with the M = 1, 8, 16 activations as bf16:
    W's bytes on sampled 16-row bands, Y on the columns of those bands."""
    d = W.decode()
    w = d["w"]
    wq = nv.quantize_2d(dev_bf16(w))
    wc, ws, wg = host_q(wq)
    gw = O.global_scale(float(np.max(np.abs(W.bf16_bits_to_float32(w)))))
    assert np.float32(wg) == gw
    rng = np.random.default_rng(3)
    bands = np.unique(np.concatenate([[0, 895], rng.choice(896, 30, replace=False)]))
    rows = (bands[:, None] * 16 + np.arange(16)).ravel()
    oc, os_ = O.encode_2d(w[rows], gw)
    assert_codes_equal(wc[rows], oc, "decode W codes")
    assert_codes_equal(ws[bands], os_, "decode W scales")
    for m, a in d["a"].items():
        y = nv.gemm_w4a16(dev_bf16(a), wq)
        check_gemm(y.cpu()[:, rows], O.gemm64_w4a16(a, (oc, os_, gw, 16)),
                   what=f"w4a16 decode M={m}")


# 16x16-tile W scales with K = 2048 and 4096 and 4-byte aligned scale rows take the decode
# kernel's scalar scale loads; padded (2-byte aligned) rows take the vector loads.
@pytest.mark.parametrize("k", [2048, 4096])
@pytest.mark.parametrize("pad", [0, 2])
def test_scale_load_paths(nv, k, pad):
    rng = np.random.default_rng(3 * k + pad)
    n = 1040
    w = W.to_bf16_bits(rng.standard_normal((n, k)) * 0.02)
    scales = torch.full((n // 16, k // 16 + pad), 0xEE, dtype=torch.uint8, device="cuda")
    wq0 = nv.empty_qtensor(n, k, 16)
    wq = nv.QTensor(wq0.codes, scales[:, :k // 16], wq0.global_scale, n, k, 16)
    nv.quantize_2d(dev_bf16(w), out=wq)
    ow = O.quantize_2d(w) + (16,)
    wc, ws, wg = host_q(wq)
    assert_codes_equal(ws, ow[1], f"k={k} pad={pad} W scales")
    assert_codes_equal(wc, ow[0], f"k={k} pad={pad} W codes")
    for m in (1, 8, 16):
        a = W.to_bf16_bits(rng.standard_normal((m, k)))
        y = nv.gemm_w4a16(dev_bf16(a), wq)
        check_gemm(y, O.gemm64_w4a16(a, ow), what=f"w4a16 k={k} pad={pad} m={m}")


def test_rejects_prefill_shapes(nv):
    a = torch.zeros((17, 64), dtype=torch.bfloat16, device="cuda")
    wq = nv.quantize_1d(torch.zeros((32, 64), dtype=torch.bfloat16, device="cuda"))
    with pytest.raises(nv.Nvfp4Error) as e:
        nv.gemm_w4a16(a, wq)
    assert e.value.status == nv.ERR_UNSUPPORTED
