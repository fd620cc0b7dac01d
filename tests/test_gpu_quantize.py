"""GPU parity of quantize_1d / quantize_2d / dequantize against the CPU oracle: codes, scales and
the global scale must be byte-identical; dequantized values bit-identical."""

import numpy as np
import pytest
import torch

from oracle import nvfp4_oracle as O
from nvfp4_w4a4_quantized_amax_amd import workloads as W
from gpu_helpers import assert_codes_equal, dev_bf16, host_q

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def nv():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from nvfp4_w4a4_quantized_amax_amd import nvfp4
    return nvfp4


def check_1d(nv, x_u16, what):
    q = nv.quantize_1d(dev_bf16(x_u16))
    c, s, g = host_q(q)
    oc, os_, og = O.quantize_1d(x_u16)
    assert np.float32(g) == og, f"{what}: gs {g!r} vs {og!r}"
    assert_codes_equal(s, os_, what + " scales")
    assert_codes_equal(c, oc, what + " codes")
    return q


def check_2d(nv, w_u16, what):
    q = nv.quantize_2d(dev_bf16(w_u16))
    c, s, g = host_q(q)
    oc, os_, og = O.quantize_2d(w_u16)
    assert np.float32(g) == og, f"{what}: gs {g!r} vs {og!r}"
    assert_codes_equal(s, os_, what + " scales")
    assert_codes_equal(c, oc, what + " codes")
    return q


def test_tiny_round_trip(nv):
    d = W.tiny()
    for name in ("a", "w"):
        q = check_1d(nv, d[name], "tiny " + name)
        c, s, g = host_q(q)
        f32 = nv.dequantize(q, torch.float32).cpu().numpy()
        want = O.dequantize(c, s, g, 1, out="f32")
        assert np.array_equal(f32.view(np.uint32), want.view(np.uint32))
        b16 = nv.dequantize(q, torch.bfloat16).cpu().view(torch.int16).numpy().view(np.uint16)
        assert np.array_equal(b16, O.dequantize(c, s, g, 1, out="bf16"))


@pytest.mark.parametrize("rows,cols", [(1, 16), (3, 48), (17, 80), (130, 272), (64, 8192),
                                       (257, 1040), (2048, 4096)])
def test_ragged_shapes(nv, rows, cols):
    rng = np.random.default_rng(rows * 1000 + cols)
    x = W.to_bf16_bits(rng.laplace(0, 1, (rows, cols)) * np.exp(rng.standard_normal(cols)))
    check_1d(nv, x, f"{rows}x{cols}")


def test_activation_distribution_band(nv):
    """The activation workload's distribution (Laplace x log-normal column gains) on a 512-row
    band (the single-read path)."""
    x = W.activation(seed=1, rows=512, cols=8192)["x"]
    check_1d(nv, x, "activation band")


def test_strided_input(nv):
    rng = np.random.default_rng(3)
    big = W.to_bf16_bits(rng.standard_normal((300, 1024 + 64)))
    xt = dev_bf16(big)[:, 32:32 + 1024]
    assert xt.stride(0) == 1088
    q = nv.quantize_1d(xt)
    c, s, g = host_q(q)
    oc, os_, og = O.quantize_1d(np.ascontiguousarray(big[:, 32:32 + 1024]))
    assert np.float32(g) == og
    assert_codes_equal(s, os_, "strided scales")
    assert_codes_equal(c, oc, "strided codes")


def adversarial_rows():
    rows = []
    mids = [0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0]
    for sbv in [448.0, 1.75, 0.5, 0.0703125, 3 * 2.0 ** -9, 2.0 ** -9]:
        s = sbv * 2.0 ** -8
        row = [6 * s] + [m * s for m in mids] + [-m * s for m in mids] + [-0.0]
        rows.append(row)
    rows[0][0] = 10.5                                     # amax 10.5 -> gs = 2^-8 exactly
    for mu in [(1.0 + 1.5 / 8) * 2.0 ** -3, 1.9375 * 2, 1.0625 * 0.25, 1.9375 * 2.0 ** -7]:
        rows.append([mu * 6 * 2.0 ** -8] + [2.0 ** -10] * 15)  # block maxima on E4M3 midpoints
    rows.append([0.0] * 16)                               # zero block
    rows.append([-0.0] * 16)                              # negative zeros
    rows.append([1e-30] + [-1e-32] * 15)                  # scale underflows to 0
    return np.array(rows, dtype=np.float64)


def test_adversarial_ties_and_zeros(nv):
    x = W.to_bf16_bits(adversarial_rows())
    x = np.concatenate([x, x[::-1]], axis=1)  # two blocks per row
    check_1d(nv, x, "adversarial")
    # the same values in a tensor large enough for the multi-workgroup path
    big = np.tile(x, (512, 4))
    check_1d(nv, big, "adversarial, large")


@pytest.mark.parametrize("amax_sig", [21, 42, 63, 105, 128, 255])
@pytest.mark.parametrize("exp", [0, 100, -100])
def test_short_global_scales(nv, amax_sig, exp):
    """amax significands that are multiples of 21 make gs short (few bits), so exact E2M1 and
    E4M3 midpoints occur often and some block-scale mantissa has no single exact multiplier:
    those blocks take the two-term multiplier (exp = 0), or the exact slow path where gs lies
    outside the two-term range (exp = +-100: gs near 2^93 and 2^-110)."""
    rng = np.random.default_rng(amax_sig)
    x = rng.integers(-255, 256, size=(96, 512)).astype(np.float64) * 2.0 ** -4
    x[0, 0] = amax_sig * 2.0 ** -3
    x[np.abs(x) > amax_sig * 2.0 ** -3] = 0
    x = W.to_bf16_bits(x * 2.0 ** exp)
    check_1d(nv, x, f"short gs {amax_sig} x 2^{exp}")
    check_1d(nv, np.tile(x, (200, 1)), f"short gs {amax_sig} x 2^{exp}, large")


def test_extremes(nv):
    x = np.zeros((32, 64))
    x[0, 0] = 3.3e38                     # near bf16 max
    x[1, :16] = 1e-20
    x[2, 16:32] = -7.5e30
    x[3] = np.linspace(-1e38, 1e38, 64)
    check_1d(nv, W.to_bf16_bits(x), "extremes")
    z = np.zeros((40, 96), dtype=np.uint16)
    z[5, 7] = 0x8000
    check_1d(nv, z, "all zero")


def test_workspace_reuse_and_determinism(nv):
    rng = np.random.default_rng(5)
    a = W.to_bf16_bits(rng.standard_normal((1024, 2048)) * 100)
    b = W.to_bf16_bits(rng.standard_normal((1024, 2048)) * 0.01)
    q1 = check_1d(nv, a, "first")
    check_1d(nv, b, "second (smaller amax after larger)")
    q3 = check_1d(nv, a, "third")
    assert torch.equal(q1.codes, q3.codes) and torch.equal(q1.scales, q3.scales)


@pytest.mark.parametrize("rows,cols", [(16, 16), (32, 4096), (512, 4096), (48, 272)])
def test_quantize_2d(nv, rows, cols):
    rng = np.random.default_rng(rows + cols)
    w = W.to_bf16_bits(rng.standard_normal((rows, cols)) * 0.02)
    q = check_2d(nv, w, f"2d {rows}x{cols}")
    c, s, g = host_q(q)
    f32 = nv.dequantize(q, torch.float32).cpu().numpy()
    assert np.array_equal(f32.view(np.uint32), O.dequantize(c, s, g, 16, out="f32").view(np.uint32))


def test_activation_full_size(nv):
    """The 8192 x 8192 activation workload (the single-read path, as timed by the benchmark):
    the global scale and every code and scale byte of the whole tensor against the oracle."""
    x = W.activation()["x"]
    q = nv.quantize_1d(dev_bf16(x))
    c, s, g = host_q(q)
    oc, os_, og = O.quantize_1d(x)
    assert np.float32(g) == og
    assert_codes_equal(s, os_, "full-size scales")
    assert_codes_equal(c, oc, "full-size codes")
    # dequantize of the whole tensor, fp32 and bf16 outputs, bit for bit
    f32 = nv.dequantize(q, torch.float32).cpu().numpy()
    assert np.array_equal(f32.view(np.uint32), O.dequantize(oc, os_, og, 1, out="f32").view(np.uint32))
    del f32
    b16 = nv.dequantize(q, torch.bfloat16).cpu().view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(b16, O.dequantize(oc, os_, og, 1, out="bf16"))


@pytest.mark.parametrize("rows,cols,br", [(257, 1040, 1), (48, 272, 16), (130, 4112, 1)])
def test_dequantize_ragged(nv, rows, cols, br):
    """Dequantize (fp32 and bf16) on shapes that leave partial tiles, 1D and 16x16 scales."""
    rng = np.random.default_rng(rows * 3 + cols)
    x = W.to_bf16_bits(rng.laplace(0, 1, (rows, cols)) * np.exp(rng.standard_normal(cols)))
    q = (nv.quantize_2d if br == 16 else nv.quantize_1d)(dev_bf16(x))
    c, s, g = host_q(q)
    f32 = nv.dequantize(q, torch.float32).cpu().numpy()
    assert np.array_equal(f32.view(np.uint32), O.dequantize(c, s, g, br, out="f32").view(np.uint32))
    b16 = nv.dequantize(q, torch.bfloat16).cpu().view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(b16, O.dequantize(c, s, g, br, out="bf16"))


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
@pytest.mark.parametrize("rows,cols,br", [(257, 1040, 1), (48, 272, 16)])
def test_dequantize_strided_output(nv, rows, cols, br, dtype):
    """Dequantize into rows of a wider matrix (ld_y = cols + 24): every value of the view
    against the oracle, bit for bit, and the padding columns left as they were."""
    rng = np.random.default_rng(rows + 7 * cols)
    x = W.to_bf16_bits(rng.standard_normal((rows, cols)) * np.exp(rng.uniform(-4, 4, (rows, 1))))
    q = (nv.quantize_2d if br == 16 else nv.quantize_1d)(dev_bf16(x))
    c, s, g = host_q(q)
    big = torch.full((rows, cols + 24), -7.0, dtype=dtype, device="cuda")
    nv.dequantize(q, dtype, out=big[:, :cols])
    torch.cuda.synchronize()
    host = big.cpu()
    assert bool((host[:, cols:] == -7.0).all()), "padding columns written"
    if dtype == torch.float32:
        got = host[:, :cols].numpy().view(np.uint32)
        assert np.array_equal(got, O.dequantize(c, s, g, br, out="f32").view(np.uint32))
    else:
        got = host[:, :cols].contiguous().view(torch.int16).numpy().view(np.uint16)
        assert np.array_equal(got, O.dequantize(c, s, g, br, out="bf16"))


def test_empty_tensors(nv):
    """Zero-row inputs through the binding: every call succeeds and leaves its outputs alone."""
    x = torch.empty((0, 64), dtype=torch.bfloat16, device="cuda")
    q = nv.quantize_1d(x)
    assert q.codes.shape == (0, 32) and q.scales.shape == (0, 4)
    q2 = nv.quantize_2d(x)
    assert q2.scales.shape == (0, 4)
    assert nv.dequantize(q).shape == (0, 64)
    w = nv.quantize_2d(dev_bf16(W.to_bf16_bits(np.ones((32, 64)))))
    assert nv.gemm_w4a4(x, w).shape == (0, 32)
    torch.cuda.synchronize()


@pytest.mark.parametrize("path,spin", [("two_pass", ""), ("cooperative", ""), ("", "0")])
def test_other_quantize_paths(path, spin):
    """The two-kernel path, the cooperative launch of the single-read kernel (or the two-kernel
    path where the device refuses it), and the single-read kernel with a poll bound of 0, so
    that every workgroup takes the barrier's fallback (the whole-tensor maximum): selected
    through NVFP4_QUANT_PATH / NVFP4_QUANT_SPIN_LIMIT in a separate process (the library reads
    them once per process).  Every kernel ends normally in all three."""
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import os
    import subprocess
    import sys
    here = os.path.dirname(os.path.abspath(__file__))
    env = dict(os.environ)
    env.pop("NVFP4_QUANT_PATH", None)
    env.pop("NVFP4_QUANT_SPIN_LIMIT", None)
    if path:
        env["NVFP4_QUANT_PATH"] = path
    if spin:
        env["NVFP4_QUANT_SPIN_LIMIT"] = spin
    r = subprocess.run([sys.executable, "-u", os.path.join(here, "quantize_path_check.py")],
                       env=env, capture_output=True, text=True, timeout=110)
    assert r.returncode == 0, r.stdout[-2000:] + r.stderr[-2000:]
    assert r.stdout.count(" ok") == 4, r.stdout
