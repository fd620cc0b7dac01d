"""GPU parity of the MSE-observer quantizer against the oracle: codes, scale bytes and the global
scale bit for bit (the observer's fp32 error evaluation is specified, so the decisions match);
the result is an ordinary NVFP4 tensor that the GEMM consumes."""

import numpy as np
import pytest
import torch

from oracle import mse_oracle as M
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


def check(nv, u16, br, what):
    q = nv.quantize_mse(dev_bf16(u16), br)
    c, s, g = host_q(q)
    oc, os_, og = M.quantize_mse(u16, br)
    assert np.float32(g) == og, what
    assert_codes_equal(s, os_, what + " scales")
    assert_codes_equal(c, oc, what + " codes")
    return q, (oc, os_, og, br)


def weights(rng, rows, cols, kind):
    if kind == "normal":
        x = rng.standard_normal((rows, cols)) * 0.02
    elif kind == "outliers":
        x = W.normal_with_outliers(rng, rows, cols, 0.01, 20.0) * 0.02
    else:
        x = rng.laplace(size=(rows, cols)) * rng.lognormal(size=(1, cols)) * 0.01
    return W.to_bf16_bits(x)


@pytest.mark.parametrize("kind", ["normal", "outliers", "laplace_gains"])
@pytest.mark.parametrize("rows,cols,br", [(64, 512, 1), (37, 1040, 1), (64, 512, 16),
                                          (48, 272, 16), (32, 80, 16)])
def test_shapes(nv, rows, cols, br, kind):
    rng = np.random.default_rng(rows + cols + br)
    check(nv, weights(rng, rows, cols, kind), br, f"mse {rows}x{cols} b{br} {kind}")


def test_edge_blocks(nv):
    """Zero blocks, a lone outlier, subnormal-scale blocks, exact grid blocks and -0.0."""
    x = np.zeros((16, 64))
    x[0, 5] = 100.0                              # tensor maximum
    x[1, :16] = np.linspace(-1, 1, 16) * 1e-3    # small block
    x[2, 16:32] = 6.0 * 2.0 ** -10               # constant block
    x[3, 32:48] = -0.0
    x[4, 48:64] = [1.0] * 15 + [7.0]
    x[5:9, :] = np.random.default_rng(3).standard_normal((4, 64)) * 1e-6
    u = W.to_bf16_bits(x)
    check(nv, u, 1, "edge 1d")
    check(nv, u, 16, "edge 2d")


def test_decode_weight_sampled_bands(nv):
    """The 14336 x 4096 decode weight with 16x16 tiles: sampled bands bit for bit (under the
    tensor's global scale), and the observer's total error below the amax rule's."""
    d = W.decode()
    w = d["w"]
    q = nv.quantize_mse(dev_bf16(w), 16)
    c, s, g = host_q(q)
    gw = O.global_scale(float(np.max(np.abs(W.bf16_bits_to_float32(w)))))
    assert np.float32(g) == gw
    rng = np.random.default_rng(5)
    bands = np.unique(np.concatenate([[0, 895], rng.choice(896, 24, replace=False)]))
    rows = (bands[:, None] * 16 + np.arange(16)).ravel()
    oc, os_, _ = M.quantize_mse(w[rows], 16, gs=gw)
    assert_codes_equal(c[rows], oc, "decode W codes")
    assert_codes_equal(s[bands], os_, "decode W scales")
    xf = O.bf16_bits_to_f64(w[rows])
    e_mse = np.sum((O.dequantize(oc, os_, gw, 16, out="f64") - xf) ** 2)
    base = O.encode_2d(w[rows], gw)
    e_amax = np.sum((O.dequantize(base[0], base[1], gw, 16, out="f64") - xf) ** 2)
    assert e_mse < e_amax


def test_gemm_consumes_mse_weights(nv):
    rng = np.random.default_rng(9)
    w = weights(rng, 256, 1024, "outliers")
    a = W.to_bf16_bits(rng.standard_normal((200, 1024)))
    wq, ow = check(nv, w, 16, "gemm weight")
    y = nv.gemm_w4a4(dev_bf16(a), wq)
    check_gemm(y, O.gemm64(O.quantize_1d(a) + (1,), ow), what="gemm with mse weights")
