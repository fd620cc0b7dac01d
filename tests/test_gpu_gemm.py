"""GPU parity of the W4A4 GEMM paths against the float64 oracle:
|Y - Y64| <= 1e-3 * ||Y64[m, :]||_2 for every element, with Y64 the exact product of the two
dequantized operands.  The quantized operands the GEMM consumes are first checked byte for byte
against the oracle's quantization of the same bf16 inputs."""

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


def run_dense(nv, a_u16, w_u16, w_block_rows, what, check_aq=True):
    wq = (nv.quantize_2d if w_block_rows == 16 else nv.quantize_1d)(dev_bf16(w_u16))
    m, k = a_u16.shape
    aq = nv.empty_qtensor(m, k, 1)
    y = nv.gemm_w4a4(dev_bf16(a_u16), wq, a_q=aq)
    oa = O.quantize_1d(a_u16) + (1,)
    ow = (O.quantize_2d(w_u16) if w_block_rows == 16 else O.quantize_1d(w_u16)) + (w_block_rows,)
    wc, ws, wg = host_q(wq)
    assert np.float32(wg) == ow[2]
    assert_codes_equal(wc, ow[0], what + " W codes")
    assert_codes_equal(ws, ow[1], what + " W scales")
    if check_aq:
        ac, as_, ag = host_q(aq)
        assert np.float32(ag) == oa[2]
        assert_codes_equal(ac, oa[0], what + " A codes")
        assert_codes_equal(as_, oa[1], what + " A scales")
    y64 = O.gemm64(oa, ow)
    return check_gemm(y, y64, what=what), y, y64, aq, wq


def test_tiny_config(nv):
    d = W.tiny()
    worst, y, y64, _, _ = run_dense(nv, d["a"], d["w"], 1, "tiny")
    assert y.shape == (32, 512)


@pytest.mark.parametrize("m,n,k,br", [
    (1, 512, 1024, 16), (5, 512, 1024, 16), (16, 512, 1024, 16), (16, 80, 1040, 1),
    (8, 256, 4096, 16), (3, 48, 16, 1),
    (17, 256, 512, 16), (37, 80, 176, 1), (64, 512, 256, 16), (100, 272, 528, 16),
    (128, 256, 1024, 1), (300, 512, 2048, 16), (513, 1024, 4096, 16),
    # K split over workgroups (too few tiles for the device): 16 splits of 4 windows; 1D W;
    # K with a partial last window (5 splits, the tail in the last); the pipelined kernel with
    # 2 splits; N not a multiple of 4 (no split).
    (17, 1024, 4096, 16), (32, 4096, 4096, 16), (64, 1000, 2048, 1), (72, 768, 3088, 16),
    (200, 512, 4096, 16), (40, 514, 2048, 1),
    # 16 < M <= 512 with many 64-column tiles: K split over the 4 waves of each workgroup,
    # 64-row tiles up to M = 64, 128-row tiles above (ragged M and N; K = 1024 is a single
    # round of the window ring); 128-row tiles with too few of them take the split path.
    (40, 8200, 2048, 1), (100, 8256, 1024, 16), (300, 4160, 2048, 16), (128, 4096, 4096, 16),
])
def test_shapes(nv, m, n, k, br):
    rng = np.random.default_rng(m * 7 + n * 3 + k)
    a = W.normal_with_outliers(rng, m, k, 0.01, 20.0)
    w = rng.standard_normal((n, k)) * 0.02
    run_dense(nv, W.to_bf16_bits(a), W.to_bf16_bits(w), br, f"{m}x{n}x{k} b{br}")


@pytest.mark.parametrize("m", [1, 16, 200])
def test_prequantized_a(nv, m):
    rng = np.random.default_rng(m)
    a = W.to_bf16_bits(rng.standard_normal((m, 512)))
    w = W.to_bf16_bits(rng.standard_normal((256, 512)) * 0.02)
    aq = nv.quantize_1d(dev_bf16(a))
    wq = nv.quantize_2d(dev_bf16(w))
    y = nv.gemm_w4a4(aq, wq)
    y_fused = nv.gemm_w4a4(dev_bf16(a), wq)
    assert torch.equal(y, y_fused)
    y64 = O.gemm64(O.quantize_1d(a) + (1,), O.quantize_2d(w) + (16,))
    check_gemm(y, y64, what=f"prequantized m={m}")


# A single activation row: K <= 4096 takes the decode kernel, which quantizes the bf16
# activation inside it (the quantized A it writes is checked); K = 8192 a quantize launch and
# the small-M kernel.
@pytest.mark.parametrize("n,k,br", [(1000, 2048, 1), (4112, 4096, 16), (272, 8192, 16),
                                    (48, 4096, 1)])
def test_single_row_shapes(nv, n, k, br):
    rng = np.random.default_rng(n * 3 + k + br)
    a = W.to_bf16_bits(W.normal_with_outliers(rng, 1, k, 0.01, 20.0))
    w = W.to_bf16_bits(rng.standard_normal((n, k)) * 0.02)
    _, y, y64, aq, wq = run_dense(nv, a, w, br, f"single row 1x{n}x{k} b{br}")
    y_pre = nv.gemm_w4a4(aq, wq)          # the prequantized form of the same product
    assert torch.equal(y, y_pre)


def test_identity_weight_closed_form(nv):
    """W = I with 16x16 blocks makes W_hat = 2688 gs_W I: Y must be RN_bf16(A_hat * 2688 gs_W)
    up to the fp32 epilogue (pins transposes, nibble order and scale indexing on the GPU)."""
    a = W.tiny()["a"]
    eye = W.to_bf16_bits(np.eye(512))
    wq = nv.quantize_2d(dev_bf16(eye))
    y = nv.gemm_w4a4(dev_bf16(a), wq)
    oa = O.quantize_1d(a)
    ahat = O.dequantize(*oa, 1, out="f64")
    y64 = ahat * (2688 * float(O.quantize_2d(eye)[2]))
    check_gemm(y, y64, what="identity")


def test_decode_config_full_size(nv):
    """14336 x 4096 weights (16x16 blocks), activations M = 1, 8, 16 quantized inside the call.
    W's bytes are checked on sampled 16-row bands; outputs on the columns of those bands."""
    d = W.decode()
    w = d["w"]
    wq = nv.quantize_2d(dev_bf16(w))
    wc, ws, wg = host_q(wq)
    gw = O.global_scale(float(np.max(np.abs(W.bf16_bits_to_float32(w)))))
    assert np.float32(wg) == gw
    rng = np.random.default_rng(1)
    bands = np.unique(np.concatenate([[0, 895], rng.choice(896, 30, replace=False)]))
    rows = (bands[:, None] * 16 + np.arange(16)).ravel()
    oc, os_ = O.encode_2d(w[rows], gw)
    assert_codes_equal(wc[rows], oc, "decode W codes")
    assert_codes_equal(ws[bands], os_, "decode W scales")
    ow = (oc, os_, gw, 16)
    for m, a in d["a"].items():
        y = nv.gemm_w4a4(dev_bf16(a), wq)
        y64 = O.gemm64(O.quantize_1d(a) + (1,), ow)
        check_gemm(y.cpu()[:, rows], y64, what=f"decode M={m}")


@pytest.mark.parametrize("m", [17, 64, 200, 513])
def test_batched_decode_full_width(nv, m):
    """The 14336 x 4096 decode weight with M = 17, 64, 200 and 513 activation rows (quantized
    inside the call): 64- and 128-row tiles of 64 columns with K split over each workgroup's
    waves, then 256 x 256 tiles.  Outputs are checked on sampled 16-row bands of W."""
    d = W.decode()
    w = d["w"]
    wq = nv.quantize_2d(dev_bf16(w))
    wc, ws, wg = host_q(wq)
    gw = O.global_scale(float(np.max(np.abs(W.bf16_bits_to_float32(w)))))
    assert np.float32(wg) == gw
    rng = np.random.default_rng(100 + m)
    bands = np.unique(np.concatenate([[0, 895], rng.choice(896, 14, replace=False)]))
    rows = (bands[:, None] * 16 + np.arange(16)).ravel()
    oc, os_ = O.encode_2d(w[rows], gw)
    assert_codes_equal(wc[rows], oc, "W codes")
    assert_codes_equal(ws[bands], os_, "W scales")
    a = W.to_bf16_bits(W.normal_with_outliers(rng, m, 4096, 0.01, 20.0))
    y = nv.gemm_w4a4(dev_bf16(a), wq)
    y64 = O.gemm64(O.quantize_1d(a) + (1,), (oc, os_, gw, 16))
    check_gemm(y.cpu()[:, rows], y64, what=f"batched decode M={m}")


def test_prefill_config_full_size(nv):
    """8192^3 with the activation quantized inside the call: the quantized A (captured) and W
    are checked byte for byte on sampled rows / bands, Y on their cross product."""
    d = W.prefill()
    a, w = d["a"], d["w"]
    wq = nv.quantize_2d(dev_bf16(w))
    aq = nv.empty_qtensor(8192, 8192, 1)
    y = nv.gemm_w4a4(dev_bf16(a), wq, a_q=aq)
    ga = O.global_scale(float(np.max(np.abs(W.bf16_bits_to_float32(a)))))
    gw = O.global_scale(float(np.max(np.abs(W.bf16_bits_to_float32(w)))))
    ac, as_, ag = host_q(aq)
    wc, ws, wg = host_q(wq)
    assert np.float32(ag) == ga and np.float32(wg) == gw
    rng = np.random.default_rng(2)
    arows = np.unique(np.concatenate([[0, 8191], rng.choice(8192, 30, replace=False)]))
    bands = np.unique(np.concatenate([[0, 511], rng.choice(512, 14, replace=False)]))
    wrows = (bands[:, None] * 16 + np.arange(16)).ravel()
    oac, oas = O.encode_1d(a[arows], ga)
    owc, ows = O.encode_2d(w[wrows], gw)
    assert_codes_equal(ac[arows], oac, "prefill A codes")
    assert_codes_equal(as_[arows], oas, "prefill A scales")
    assert_codes_equal(wc[wrows], owc, "prefill W codes")
    assert_codes_equal(ws[bands], ows, "prefill W scales")
    y64 = O.gemm64((oac, oas, ga, 1), (owc, ows, gw, 16))
    ys = y.cpu()[arows][:, wrows]
    check_gemm(ys, y64, what="prefill sampled")
