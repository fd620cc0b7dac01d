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
    # 128-row tiles of the mid-size kernel on a wide 2D-scaled weight with several rounds of
    # the window ring (K = 4096); 1D-scaled weights with M > 128 on the pipelined 256 x 256
    # kernel (with and without a K split); M > 128 with K not a multiple of 64 (the
    # register-prefetch kernel with 256-row tiles), 2D and 1D.
    (65, 8192, 4096, 16), (200, 512, 4096, 1), (513, 1024, 1024, 1), (1024, 2048, 512, 1),
    (200, 256, 1040, 16), (150, 272, 528, 1),
    # M = 129-384 on a wide 2D-scaled weight: 128-row tiles of the mid-size kernel in two or
    # three row slices (ragged M and N); the same shape with 1D W scales splits K instead.
    (129, 8192, 1024, 16), (256, 8256, 2048, 16), (384, 8192, 1024, 16), (200, 8192, 1024, 1),
])
def test_shapes(nv, m, n, k, br):
    rng = np.random.default_rng(m * 7 + n * 3 + k)
    a = W.normal_with_outliers(rng, m, k, 0.01, 20.0)
    w = rng.standard_normal((n, k)) * 0.02
    run_dense(nv, W.to_bf16_bits(a), W.to_bf16_bits(w), br, f"{m}x{n}x{k} b{br}")


@pytest.mark.parametrize("br", [16, 1])
@pytest.mark.parametrize("m", [40, 100, 200])
def test_mid_kernel_strided_scales(nv, m, br):
    """Mid-size M on a wide weight whose scale rows are not 16-byte aligned (a strided view of
    a wider scale buffer): the mid-size kernel's form that loads scales 2 bytes at a time, and
    at M = 200 the 256 x 256 tiles with a K split (the 128-row tiles need aligned rows)."""
    rng = np.random.default_rng(m + br)
    n, k = 8192, 2048
    a = W.to_bf16_bits(W.normal_with_outliers(rng, m, k, 0.01, 20.0))
    w = W.to_bf16_bits(rng.standard_normal((n, k)) * 0.02)
    wq = (nv.quantize_2d if br == 16 else nv.quantize_1d)(dev_bf16(w))
    srows = n // br
    wide = torch.zeros((srows, k // 16 + 2), dtype=torch.uint8, device="cuda")
    wide[:, :k // 16] = wq.scales
    wq2 = nv.QTensor(wq.codes, wide[:, :k // 16], wq.global_scale, n, k, br)
    assert wq2.scales.stride(0) % 16 != 0
    aq = nv.quantize_1d(dev_bf16(a))
    y = nv.gemm_w4a4(aq, wq2)
    y_ref = nv.gemm_w4a4(aq, wq)
    ow = (O.quantize_2d(w) if br == 16 else O.quantize_1d(w)) + (br,)
    check_gemm(y, O.gemm64(O.quantize_1d(a) + (1,), ow), what=f"strided scales m={m} b{br}")
    check_gemm(y_ref, O.gemm64(O.quantize_1d(a) + (1,), ow), what=f"aligned scales m={m} b{br}")


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


# The decode kernels read a wave's scale bytes of a band with one scalar load when W has 16x16
# tile scales, K is 2048 or 4096 (every wave holds its whole share of windows) and the scale rows
# are 4-byte aligned; otherwise with vector loads.  Both, for A prequantized (the form that takes
# the scalar loads) and A quantized inside the call (the form that does not): bit-identical
# outputs, and the oracle's bound.
@pytest.mark.parametrize("k", [2048, 4096])
@pytest.mark.parametrize("pad", [0, 2])
def test_decode_scale_load_paths(nv, k, pad):
    rng = np.random.default_rng(k + pad)
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
        aq = nv.quantize_1d(dev_bf16(a))
        y = nv.gemm_w4a4(aq, wq)
        y_fused = nv.gemm_w4a4(dev_bf16(a), wq)
        assert torch.equal(y, y_fused), f"k={k} pad={pad} m={m}: prequantized and fused differ"
        check_gemm(y, O.gemm64(O.quantize_1d(a) + (1,), ow), what=f"k={k} pad={pad} m={m}")
    torch.cuda.synchronize()
    if pad:
        assert bool((scales[:, k // 16:] == 0xEE).all()), "padding of the scale rows written"


# A single activation row: K <= 4096 takes the decode kernel, whose first wave quantizes the
# bf16 activation for the whole workgroup (the quantized A it writes is checked; K = 2064 and
# 1040 leave the last waves' K slices short or empty); K = 8192 a quantize launch and the
# small-M kernel.
@pytest.mark.parametrize("n,k,br", [(1000, 2048, 1), (4112, 4096, 16), (272, 8192, 16),
                                    (48, 4096, 1), (528, 2064, 16), (100, 1040, 1),
                                    (64, 256, 16)])
def test_single_row_shapes(nv, n, k, br):
    rng = np.random.default_rng(n * 3 + k + br)
    a = W.to_bf16_bits(W.normal_with_outliers(rng, 1, k, 0.01, 20.0))
    w = W.to_bf16_bits(rng.standard_normal((n, k)) * 0.02)
    _, y, y64, aq, wq = run_dense(nv, a, w, br, f"single row 1x{n}x{k} b{br}")
    y_pre = nv.gemm_w4a4(aq, wq)          # the prequantized form of the same product
    assert torch.equal(y, y_pre)


# Decode shapes with A quantized inside the call read A with its row stride: one row by the
# first wave's loads, 2-16 rows through the LDS staging copy (K = 1040 leaves the last 1 KiB
# chunk of each staged row partly past the row's end).
@pytest.mark.parametrize("m,k", [(1, 1040), (6, 1040), (16, 4096), (2, 2064)])
def test_strided_activation_rows(nv, m, k):
    rng = np.random.default_rng(m * 31 + k)
    n, ld = 272, k + 72
    a_full = W.to_bf16_bits(W.normal_with_outliers(rng, m, ld, 0.01, 20.0))
    a = a_full[:, :k]
    w = W.to_bf16_bits(rng.standard_normal((n, k)) * 0.02)
    wq = nv.quantize_2d(dev_bf16(w))
    a_dev = dev_bf16(np.ascontiguousarray(a_full))[:, :k]
    assert a_dev.stride(0) == ld
    aq = nv.empty_qtensor(m, k, 1)
    y = nv.gemm_w4a4(a_dev, wq, a_q=aq)
    oa = O.quantize_1d(np.ascontiguousarray(a)) + (1,)
    ac, as_, ag = host_q(aq)
    assert np.float32(ag) == oa[2]
    assert_codes_equal(ac, oa[0], f"strided A {m}x{k} codes")
    assert_codes_equal(as_, oa[1], f"strided A {m}x{k} scales")
    y64 = O.gemm64(oa, O.quantize_2d(w) + (16,))
    check_gemm(y, y64, what=f"strided A {m}x{k}")


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


@pytest.fixture(scope="module")
def decode_w(nv):
    """The 14336 x 4096 decode weight (16x16 tiles) quantized on the GPU, checked byte for byte
    in full against the oracle; returns (workload, GPU tensor, oracle tensor, its float64
    reconstruction)."""
    d = W.decode(ms=(1, 8, 16))
    w = d["w"]
    wq = nv.quantize_2d(dev_bf16(w))
    wc, ws, wg = host_q(wq)
    oc, os_, og = O.quantize_2d(w)
    assert np.float32(wg) == og
    assert_codes_equal(ws, os_, "decode W scales")
    assert_codes_equal(wc, oc, "decode W codes")
    ow = (oc, os_, og, 16)
    return d, wq, ow, O.dequantize(*ow, out="f64")


def test_decode_config_full_size(nv, decode_w):
    """14336 x 4096 weights (16x16 blocks), activations M = 1, 8, 16 quantized inside the call:
    the quantized A the kernel writes and every output element against the oracle."""
    d, wq, ow, w64 = decode_w
    for m, a in d["a"].items():
        aq = nv.empty_qtensor(m, 4096, 1)
        y = nv.gemm_w4a4(dev_bf16(a), wq, a_q=aq)
        oa = O.quantize_1d(a) + (1,)
        ac, as_, ag = host_q(aq)
        assert np.float32(ag) == oa[2]
        assert_codes_equal(ac, oa[0], f"decode M={m} A codes")
        assert_codes_equal(as_, oa[1], f"decode M={m} A scales")
        y64 = O.dequantize(*oa, out="f64") @ w64.T
        check_gemm(y, y64, what=f"decode M={m}", min_agree=0.99)


@pytest.mark.parametrize("m", [17, 64, 65, 128, 200, 513])
def test_batched_decode_full_width(nv, decode_w, m):
    """The 14336 x 4096 decode weight with 17 to 513 activation rows (quantized inside the
    call): 64-row tiles of the mid-size kernel (M = 17, 64), its 128-row tiles on this wide
    weight (M = 65, 128; K = 4096 runs four rounds of the window ring), then 256 x 256 tiles
    with a K split (M = 200, 513).  Every output element against the oracle."""
    _, wq, ow, w64 = decode_w
    rng = np.random.default_rng(100 + m)
    a = W.to_bf16_bits(W.normal_with_outliers(rng, m, 4096, 0.01, 20.0))
    y = nv.gemm_w4a4(dev_bf16(a), wq)
    y64 = O.dequantize(*(O.quantize_1d(a) + (1,)), out="f64") @ w64.T
    check_gemm(y, y64, what=f"batched decode M={m}", min_agree=0.99)


def tile_cover(rng, n, tile, per_tile):
    """`per_tile` random indices in every `tile`-wide slice of range(n) (plus 0 and n - 1)."""
    idx = [t0 + rng.choice(min(tile, n - t0), min(per_tile, n - t0), replace=False)
           for t0 in range(0, n, tile)]
    return np.unique(np.concatenate(idx + [[0, n - 1]]))


def test_prefill_config_full_size(nv):
    """8192^3 with the activation quantized inside the call: the quantized A (captured) and W
    are checked byte for byte in full; Y on 528 rows x 528 columns chosen so that each of the
    1,024 output tiles of 256 x 256 holds 256 checked elements at random positions."""
    d = W.prefill()
    a, w = d["a"], d["w"]
    wq = nv.quantize_2d(dev_bf16(w))
    aq = nv.empty_qtensor(8192, 8192, 1)
    y = nv.gemm_w4a4(dev_bf16(a), wq, a_q=aq)
    ac, as_, ag = host_q(aq)
    wc, ws, wg = host_q(wq)
    oa = O.quantize_1d(a)
    assert np.float32(ag) == oa[2]
    assert_codes_equal(as_, oa[1], "prefill A scales")
    assert_codes_equal(ac, oa[0], "prefill A codes")
    del ac, as_
    ow = O.quantize_2d(w)
    assert np.float32(wg) == ow[2]
    assert_codes_equal(ws, ow[1], "prefill W scales")
    assert_codes_equal(wc, ow[0], "prefill W codes")
    del wc, ws
    rng = np.random.default_rng(2)
    rows = tile_cover(rng, 8192, 256, 16)
    cols = tile_cover(rng, 8192, 256, 16)
    assert len(rows) >= 512 and len(cols) >= 512
    a64 = O.dequantize(oa[0][rows], oa[1][rows], oa[2], 1, out="f64")
    w64 = O.dequantize(ow[0], ow[1], ow[2], 16, out="f64")[cols]
    y64 = a64 @ w64.T
    ys = y[torch.from_numpy(rows).cuda()][:, torch.from_numpy(cols).cuda()]
    check_gemm(ys, y64, what="prefill tile-covering sample", min_agree=0.99)
