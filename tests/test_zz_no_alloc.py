"""The allocation-free product, nvfp4_gemm_w4a4_noalloc, through the C ABI: its output must equal
nvfp4_gemm_w4a4's (same kernels, caller workspace) element for element, on consecutive calls
whose shapes shrink (so leftovers of a larger call sit in the shared scratch), and meet the
oracle's bound; shapes beyond the scratch are refused before any launch."""

import numpy as np
import pytest
import torch

from oracle import nvfp4_oracle as O
from nvfp4_w4a4_quantized_amax_amd import workloads as W
from gpu_helpers import check_gemm, dev_bf16

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def nv():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from nvfp4_w4a4_quantized_amax_amd import nvfp4
    return nvfp4


# (m, n, k): a K split over 5 workgroups (partial sums in the scratch), then a smaller product
# split 16 ways, the mid-size kernel, and a decode shape (activation quantized in the product
# kernel); activations quantized inside every call.
SEQUENCE = [(200, 512, 4096), (17, 1024, 4096), (40, 8192, 2048), (5, 512, 1024)]


def test_noalloc_matches_workspace_form(nv):
    rng = np.random.default_rng(31)
    cases = []
    for m, n, k in SEQUENCE:
        a = W.to_bf16_bits(W.normal_with_outliers(rng, m, k, 0.01, 20.0))
        w = W.to_bf16_bits(rng.standard_normal((n, k)) * 0.02)
        cases.append((a, w, nv.quantize_2d(dev_bf16(w))))
    for rnd in range(2):  # the whole sequence twice: each call after a larger one
        for (m, n, k), (a, w, wq) in zip(SEQUENCE, cases):
            ad = dev_bf16(a)
            y_ref = nv.gemm_w4a4(ad, wq)
            y = torch.full((m, n), float("nan"), dtype=torch.bfloat16, device="cuda")
            nv.gemm_w4a4_noalloc(ad, wq, y)
            torch.cuda.synchronize()
            assert torch.equal(y, y_ref), (rnd, m, n, k)
            if rnd == 0:
                y64 = O.gemm64(O.quantize_1d(a) + (1,), O.quantize_2d(w) + (16,))
                check_gemm(y, y64, what=f"noalloc {m}x{n}x{k}")


def test_noalloc_prequantized_and_refusal(nv):
    rng = np.random.default_rng(32)
    a = W.to_bf16_bits(rng.standard_normal((300, 2048)))
    w = W.to_bf16_bits(rng.standard_normal((1024, 2048)) * 0.02)
    aq = nv.quantize_1d(dev_bf16(a))
    wq = nv.quantize_2d(dev_bf16(w))
    y = torch.empty((300, 1024), dtype=torch.bfloat16, device="cuda")
    nv.gemm_w4a4_noalloc(aq, wq, y)
    assert torch.equal(y, nv.gemm_w4a4(aq, wq))
    # 16384 x 8192 activations quantized inside the call need 75.5 MB > 64 MiB of scratch
    big = nv.lib().nvfp4_gemm_workspace_bytes(16384, 1024, 8192)
    assert big > nv.NOALLOC_SCRATCH_BYTES
    a_big = torch.zeros((16384, 8192), dtype=torch.bfloat16, device="cuda")
    w_big = nv.empty_qtensor(1024, 8192, 16)
    y_big = torch.empty((16384, 1024), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(nv.Nvfp4Error) as ei:
        nv.gemm_w4a4_noalloc(a_big, w_big, y_big)
    assert ei.value.status == nv.ERR_WORKSPACE
