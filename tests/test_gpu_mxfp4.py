"""GPU parity of the MXFP4 variant against the float64 oracle: codes and E8M0 scales bit for bit,
the reconstruction bit for bit, and the product on the scaled FP4 MFMA within
|Y - Y64| <= 1e-3 * ||Y64[m, :]||_2 + 2^-8 |Y64[m, n]|, Y64 the exact product of the two
reconstructed operands."""

import numpy as np
import pytest
import torch

from oracle import mxfp4_oracle as MX
from oracle import nvfp4_oracle as O
from nvfp4_w4a4_quantized_amax_amd import workloads as W
from gpu_helpers import assert_codes_equal, check_gemm, dev_bf16

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def nv():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from nvfp4_w4a4_quantized_amax_amd import nvfp4
    return nvfp4


def host_mx(q):
    torch.cuda.synchronize()
    return q.packed_codes().cpu().numpy(), q.packed_scales().cpu().numpy()


def check_quantize(nv, u16, what):
    q = nv.mxfp4_quantize(dev_bf16(u16))
    c, s = host_mx(q)
    oc, os_ = MX.quantize_mx(u16)
    assert_codes_equal(s, os_, what + " scales")
    assert_codes_equal(c, oc, what + " codes")
    return q, (oc, os_)


@pytest.mark.parametrize("rows,cols", [(1, 32), (3, 96), (64, 512), (37, 4128), (256, 2048)])
def test_quantize_shapes(nv, rows, cols):
    rng = np.random.default_rng(rows * 13 + cols)
    x = W.normal_with_outliers(rng, rows, cols, 0.01, 20.0) * np.exp(rng.uniform(-5, 5, (rows, 1)))
    check_quantize(nv, W.to_bf16_bits(x), f"{rows}x{cols}")


def test_quantize_edge_values(nv):
    """Zero blocks, signed zeros, bf16 subnormals (whole blocks of them), the largest bf16
    values, exact ties at every E2M1 midpoint and saturating maxima."""
    rows = []
    rows.append([0.0] * 32)
    rows.append([-0.0] * 16 + [0.0] * 16)
    rows.append([2.0 ** -133 * k for k in range(1, 33)])                   # subnormals only
    rows.append([2.0 ** -126 * (1 + k / 128) for k in range(32)])         # smallest normals
    rows.append([3.3e38, -3.3e38] + [1e38] * 30)
    mids = [0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0]
    rows.append([4.0] + mids + [-m for m in mids] + [0.0] * 17)           # X = 1: exact ties
    rows.append([7.96875, 6.5, 5.5, -7.0] + [1.0] * 28)                    # saturation, X = 1
    for e in (-100, -20, 30, 100):
        rows.append([v * 2.0 ** e for v in rows[5]])
    x = np.array(rows)
    check_quantize(nv, W.to_bf16_bits(x), "edge values")


def test_quantize_strided_input_and_padded_output(nv):
    rng = np.random.default_rng(3)
    full = W.to_bf16_bits(rng.standard_normal((40, 320)))
    x = dev_bf16(full)[:, 64:64 + 192]
    q = nv.empty_mxtensor(40, 192)
    q.codes.fill_(0xAB)
    q.scales.fill_(0xCD)
    nv.mxfp4_quantize(x, out=q)
    c, s = host_mx(q)
    oc, os_ = MX.quantize_mx(full[:, 64:64 + 192])
    assert_codes_equal(c, oc, "strided codes")
    assert_codes_equal(s, os_, "strided scales")
    torch.cuda.synchronize()
    assert torch.all(q.scales[:, 6:] == 0xCD)   # scale rows padded to 8 bytes stay untouched


def test_activation_config_sampled_rows(nv):
    """The 8192 x 8192 activation workload; every scale byte and the codes of 48 sampled rows."""
    x = W.activation()["x"]
    q = nv.mxfp4_quantize(dev_bf16(x))
    c, s = host_mx(q)
    rng = np.random.default_rng(5)
    rows = np.unique(np.concatenate([[0, 8191], rng.choice(8192, 46, replace=False)]))
    oc, os_ = MX.quantize_mx(x[rows])
    assert_codes_equal(c[rows], oc, "activation codes")
    assert_codes_equal(s[rows], os_, "activation scales")
    # every block's scale, from the block maxima alone
    blocks = np.abs(W.bf16_bits_to_float32(x).reshape(8192, 256, 32)).max(axis=2)
    assert_codes_equal(s, (MX.shared_exponents(blocks.astype(np.float64)) + 127).astype(np.uint8),
                       "activation all scales")


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
def test_dequantize(nv, dtype):
    rng = np.random.default_rng(6)
    x = W.to_bf16_bits(rng.standard_normal((33, 256)) * np.exp(rng.uniform(-60, 60, (33, 1))))
    q, oq = check_quantize(nv, x, "dequantize input")
    y = nv.mxfp4_dequantize(q, dtype)
    torch.cuda.synchronize()
    if dtype == torch.float32:
        want = MX.dequantize_mx(*oq, out="f32")
        assert np.array_equal(y.cpu().numpy().view(np.uint32), want.view(np.uint32))
    else:
        want = MX.dequantize_mx(*oq, out="bf16")
        assert np.array_equal(y.cpu().view(torch.int16).numpy().view(np.uint16), want)


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
def test_dequantize_ragged_strided(nv, dtype):
    """A shape that spans many workgroups with a ragged row count, written into rows of a wider
    matrix (ld_y = cols + 40): the view bit for bit against the oracle, the padding untouched."""
    rng = np.random.default_rng(61)
    rows, cols = 257, 1056
    x = W.to_bf16_bits(rng.standard_normal((rows, cols)) * np.exp(rng.uniform(-30, 30, (rows, 1))))
    q, oq = check_quantize(nv, x, "strided dequantize input")
    big = torch.full((rows, cols + 40), -3.0, dtype=dtype, device="cuda")
    nv.mxfp4_dequantize(q, dtype, out=big[:, :cols])
    torch.cuda.synchronize()
    host = big.cpu()
    assert bool((host[:, cols:] == -3.0).all()), "padding columns written"
    if dtype == torch.float32:
        want = MX.dequantize_mx(*oq, out="f32")
        assert np.array_equal(host[:, :cols].numpy().view(np.uint32), want.view(np.uint32))
    else:
        want = MX.dequantize_mx(*oq, out="bf16")
        got = host[:, :cols].contiguous().view(torch.int16).numpy().view(np.uint16)
        assert np.array_equal(got, want)


# M > 128 takes a pipelined kernel: the wide-window one when K is a multiple of 512 (one and
# three window pairs appear; 4100 x 4200 has more tiles than workgroups, so workgroups carry the
# pipeline from one ragged tile into the next), else the 64-wide one (one window, an odd window
# count).  M <= 128 with enough columns takes the mid-size kernel (covered below); the rest
# (small M and N, K = 32 mod 64) the direct one.  Ragged M and N appear on every path.
@pytest.mark.parametrize("m,n,k", [
    (1, 64, 64), (7, 96, 160), (16, 200, 2048), (129, 256, 64), (300, 512, 2048),
    (513, 1000, 4096), (256, 256, 192), (260, 300, 96), (300, 512, 512), (257, 384, 1536),
    (640, 272, 1024), (4100, 4200, 512),
])
def test_gemm_shapes(nv, m, n, k):
    rng = np.random.default_rng(m * 7 + n * 3 + k)
    a = W.to_bf16_bits(W.normal_with_outliers(rng, m, k, 0.01, 20.0))
    w = W.to_bf16_bits(rng.standard_normal((n, k)) * 0.02)
    wq, ow = check_quantize(nv, w, f"W {n}x{k}")
    aq = nv.empty_mxtensor(m, k)
    y = nv.mxfp4_gemm(dev_bf16(a), wq, a_q=aq)
    ac, as_ = host_mx(aq)
    oa = MX.quantize_mx(a)
    assert_codes_equal(ac, oa[0], "A codes")
    assert_codes_equal(as_, oa[1], "A scales")
    check_gemm(y, MX.gemm64_mx(oa, ow), what=f"mxfp4 {m}x{n}x{k}")
    # the prequantized form gives the same bits
    y2 = nv.mxfp4_gemm(aq, wq)
    assert torch.equal(y, y2)


# The mid-size kernel for M <= 128: each case names the (row tiles, column tiles, ring depth)
# form the shape selects, by M range and by the K multiple (4096, 2048 or 1024) that fits the
# ring; with too few 128-row tiles the 64-row form takes over.  With bf16 A and M <= 4 the
# kernel quantizes A itself (the 1x1 cases), checked through the a_q it writes.  W is checked on
# sampled rows and Y on the sampled columns (the ragged last columns always among them).
@pytest.mark.parametrize("m,n,k,form", [
    (1, 8200, 1024, "1x1 depth 4"), (3, 4100, 2048, "1x1 depth 8"), (4, 4096, 4096, "1x1 depth 16"),
    (17, 8192, 1024, "1x2 depth 4"), (32, 8256, 2048, "1x2 depth 8"), (9, 8200, 4096, "1x2 depth 16"),
    (40, 8192, 1024, "2x2 depth 4"), (64, 8200, 2048, "2x2 depth 8"), (97, 8200, 1024, "4x2 depth 4"),
    (128, 8192, 2048, "4x2 depth 8"), (100, 4100, 2048, "2x2 depth 4 (too few 128-row tiles)"),
    (4, 4100, 8192, "1x1 depth 16, A quantized by its own launch (M * K > 16384)"),
])
def test_gemm_mid_sizes(nv, m, n, k, form):
    rng = np.random.default_rng(m * 11 + n + k)
    a = W.to_bf16_bits(W.normal_with_outliers(rng, m, k, 0.01, 20.0))
    w = W.to_bf16_bits(rng.standard_normal((n, k)) * 0.02)
    wq = nv.mxfp4_quantize(dev_bf16(w))
    aq = nv.empty_mxtensor(m, k)
    y = nv.mxfp4_gemm(dev_bf16(a), wq, a_q=aq)
    cols = np.unique(np.concatenate([np.arange(n - 40, n), rng.choice(n - 40, 88, replace=False)]))
    wc, ws = host_mx(wq)
    ac, as_ = host_mx(aq)
    ow = MX.quantize_mx(w[cols])
    oa = MX.quantize_mx(a)
    assert_codes_equal(wc[cols], ow[0], f"{form}: W codes")
    assert_codes_equal(ws[cols], ow[1], f"{form}: W scales")
    assert_codes_equal(ac, oa[0], f"{form}: A codes")
    assert_codes_equal(as_, oa[1], f"{form}: A scales")
    check_gemm(y.cpu()[:, cols], MX.gemm64_mx(oa, ow), what=f"mxfp4 mid {form} {m}x{n}x{k}")
    assert torch.equal(y, nv.mxfp4_gemm(aq, wq))
    # without a_q (M <= 4: the activation quantized inside the product kernel, written nowhere)
    assert torch.equal(y, nv.mxfp4_gemm(dev_bf16(a), wq))


def test_gemm_unaligned_scale_rows(nv):
    """Scale rows 20 bytes apart (not 16-byte aligned) with K = 512: the 64-wide kernel takes
    the product, and it matches the wide kernel's on the same operands."""
    m, n, k = 384, 256, 512
    rng = np.random.default_rng(21)
    a = W.to_bf16_bits(W.normal_with_outliers(rng, m, k, 0.01, 20.0))
    w = W.to_bf16_bits(rng.standard_normal((n, k)) * 0.02)
    wq, ow = check_quantize(nv, w, "W")
    aq, oa = check_quantize(nv, a, "A")
    pad = nv.MxTensor(aq.codes, torch.zeros((m, 20), dtype=torch.uint8, device="cuda"), m, k)
    pad.scales[:, :16] = aq.packed_scales()
    y_pad = nv.mxfp4_gemm(pad, wq)
    y = nv.mxfp4_gemm(aq, wq)
    check_gemm(y_pad, MX.gemm64_mx(oa, ow), what="mxfp4 unaligned scales")
    assert torch.equal(y, y_pad)


def test_gemm_permutation_closed_form(nv):
    """W = P gives W_hat = P exactly (each 1 is magnitude 4 under scale 2^-2), so Y must be
    RN_bf16(A_hat[:, pi])."""
    n = 256
    pi = (np.arange(n) * 45 + 17) % n
    p = np.zeros((n, n))
    p[np.arange(n), pi] = 1.0
    wq, _ = check_quantize(nv, W.to_bf16_bits(p), "permutation")
    rng = np.random.default_rng(8)
    a = W.to_bf16_bits(rng.standard_normal((300, n)) * 3.0)
    y = nv.mxfp4_gemm(dev_bf16(a), wq)
    check_gemm(y, MX.dequantize_mx(*MX.quantize_mx(a))[:, pi], what="mxfp4 permutation")


def test_prefill_config_sampled(nv):
    """8192^3 (the prefill workload, both operands MXFP4): A and W checked byte for byte on
    sampled rows, Y on their cross product."""
    d = W.prefill()
    a, w = d["a"], d["w"]
    wq = nv.mxfp4_quantize(dev_bf16(w))
    aq = nv.empty_mxtensor(8192, 8192)
    y = nv.mxfp4_gemm(dev_bf16(a), wq, a_q=aq)
    ac, as_ = host_mx(aq)
    wc, ws = host_mx(wq)
    rng = np.random.default_rng(9)
    ar = np.unique(np.concatenate([[0, 8191], rng.choice(8192, 30, replace=False)]))
    wr = np.unique(np.concatenate([[0, 8191], rng.choice(8192, 62, replace=False)]))
    oa, ow = MX.quantize_mx(a[ar]), MX.quantize_mx(w[wr])
    assert_codes_equal(ac[ar], oa[0], "prefill A codes")
    assert_codes_equal(as_[ar], oa[1], "prefill A scales")
    assert_codes_equal(wc[wr], ow[0], "prefill W codes")
    assert_codes_equal(ws[wr], ow[1], "prefill W scales")
    check_gemm(y.cpu()[ar][:, wr], MX.gemm64_mx(oa, ow), what="mxfp4 prefill sampled")


def test_mxfp4_error_above_nvfp4_on_device(nv):
    """The pages' contrast, measured on the library's own outputs: on the activation-like tiny
    workload, NVFP4's reconstruction error is below MXFP4's."""
    a = W.tiny()["a"]
    x = dev_bf16(a)
    ref = torch.from_numpy(O.bf16_bits_to_f64(a))
    e_nv = (nv.dequantize(nv.quantize_1d(x)).double().cpu() - ref).pow(2).mean().item()
    e_mx = (nv.mxfp4_dequantize(nv.mxfp4_quantize(x)).double().cpu() - ref).pow(2).mean().item()
    assert e_nv < e_mx
