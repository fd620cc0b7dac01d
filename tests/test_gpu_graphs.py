"""Library calls captured in a HIP graph and replayed: every replay, on new input data copied in
between replays (eager work and a synchronization each time), must give the oracle's result or
the eager call's bits.  The inputs change their magnitude from replay to replay, so a global
scale left over from an earlier replay would show.  Calls under capture avoid the single-read
quantizer (its grid barrier tags slots with a per-call number that a graph would freeze)."""

import numpy as np
import pytest
import torch

from oracle import nvfp4_oracle as O
from oracle import mxfp4_oracle as MX
from nvfp4_w4a4_quantized_amax_amd import workloads as W
from gpu_helpers import assert_codes_equal, dev_bf16, host_q

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def nv():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from nvfp4_w4a4_quantized_amax_amd import nvfp4
    return nvfp4


def capture(fn):
    """Warm up on a side stream (allocations happen there), then capture one call."""
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        fn()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        fn()
    torch.cuda.synchronize()
    return g


def inputs(seed, rows, cols, count=4):
    rng = np.random.default_rng(seed)
    return [W.to_bf16_bits(W.normal_with_outliers(rng, rows, cols, 0.01, 20.0)
                           * np.exp(rng.uniform(-4, 4))) for _ in range(count)]


def test_quantize_1d_replays(nv):
    """512 x 1024 is above the one-workgroup size, so eager calls take the single-read path."""
    rows, cols = 512, 1024
    xs = inputs(31, rows, cols)
    x = dev_bf16(xs[0])
    q = nv.empty_qtensor(rows, cols, 1)
    g = capture(lambda: nv.quantize_1d(x, out=q))
    for u in xs[1:] + xs[:2]:
        x.copy_(dev_bf16(u))
        torch.cuda.synchronize()
        g.replay()
        c, s, gs = host_q(q)
        oc, os_, ogs = O.quantize_1d(u)
        assert np.float32(gs) == ogs
        assert_codes_equal(s, os_, "graph replay scales")
        assert_codes_equal(c, oc, "graph replay codes")


@pytest.mark.parametrize("m", [4, 256])
def test_gemm_w4a4_replays(nv, m):
    """Activations quantized inside the call: M = 4 by the decode kernel, M = 256 by the
    quantize kernels then the tiled product.  Each replay equals the eager call bit for bit."""
    n, k = 512, 1024
    rng = np.random.default_rng(32 + m)
    wq = nv.quantize_2d(dev_bf16(W.to_bf16_bits(rng.standard_normal((n, k)) * 0.02)))
    xs = inputs(33 + m, m, k)
    a = dev_bf16(xs[0])
    y = torch.empty((m, n), dtype=torch.bfloat16, device="cuda")
    g = capture(lambda: nv.gemm_w4a4(a, wq, y=y))
    for u in xs[1:] + xs[:2]:
        a.copy_(dev_bf16(u))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        got = y.clone()
        want = nv.gemm_w4a4(dev_bf16(u), wq)
        torch.cuda.synchronize()
        assert torch.equal(got, want)


@pytest.mark.parametrize("m,n,k", [(300, 256, 512), (2, 4096, 1024)])
def test_mxfp4_gemm_replays(nv, m, n, k):
    """M = 300: the quantize launch then the product; M = 2: one launch that quantizes A
    itself and writes it to a_q."""
    rng = np.random.default_rng(34 + m)
    wq = nv.mxfp4_quantize(dev_bf16(W.to_bf16_bits(rng.standard_normal((n, k)) * 0.02)))
    xs = inputs(35 + m, m, k)
    a = dev_bf16(xs[0])
    aq = nv.empty_mxtensor(m, k)
    y = torch.empty((m, n), dtype=torch.bfloat16, device="cuda")
    g = capture(lambda: nv.mxfp4_gemm(a, wq, y=y, a_q=aq))
    for u in xs[1:] + xs[:2]:
        a.copy_(dev_bf16(u))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        oc, os_ = MX.quantize_mx(u)
        assert_codes_equal(aq.packed_scales().cpu().numpy(), os_, "graph replay A scales")
        assert_codes_equal(aq.packed_codes().cpu().numpy(), oc, "graph replay A codes")
        got = y.clone()
        want = nv.mxfp4_gemm(dev_bf16(u), wq)
        torch.cuda.synchronize()
        assert torch.equal(got, want)
