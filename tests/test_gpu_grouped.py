"""GPU parity of the grouped (mixture-of-experts) W4A4 GEMM against the float64 oracle."""

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


def quantize_experts(nv, w_stacked, experts, n):
    """Each expert's weights quantized on its own (own global scale) into one stacked tensor."""
    k = w_stacked.shape[1]
    wq = nv.empty_qtensor(experts * n, k, 16, n_global_scales=experts)
    for e in range(experts):
        part = nv.QTensor(wq.codes[e * n:(e + 1) * n], wq.scales[e * n // 16:(e + 1) * n // 16],
                          wq.global_scale[e:e + 1], n, k, 16)
        nv.quantize_2d(dev_bf16(w_stacked[e * n:(e + 1) * n]), out=part)
    return wq


def oracle_experts(w_stacked, experts, n):
    return [O.quantize_2d(w_stacked[e * n:(e + 1) * n]) + (16,) for e in range(experts)]


@pytest.mark.parametrize("tokens,hidden,experts,topk,n", [(256, 256, 8, 2, 128),
                                                           (300, 528, 16, 4, 80),
                                                           (64, 1024, 5, 5, 256)])
def test_small_moe(nv, tokens, hidden, experts, topk, n):
    d = W.moe(seed=tokens, tokens=tokens, hidden=hidden, experts=experts, topk=topk, n=n)
    wq = quantize_experts(nv, d["w"], experts, n)
    ri = torch.from_numpy(d["row_index"]).cuda()
    off = torch.from_numpy(d["offsets"]).cuda()
    total = int(d["offsets"][-1])
    aq = nv.empty_qtensor(tokens, hidden, 1)
    y = nv.grouped_gemm_w4a4(dev_bf16(d["a"]), ri, off, wq, n, total, a_q=aq)
    oa = O.quantize_1d(d["a"])
    ac, as_, ag = host_q(aq)
    assert np.float32(ag) == oa[2]
    assert_codes_equal(ac, oa[0], "moe A codes")
    ows = oracle_experts(d["w"], experts, n)
    wc, ws, wg = host_q(wq)
    for e in range(experts):
        assert np.float32(wg[e]) == ows[e][2]
        assert_codes_equal(wc[e * n:(e + 1) * n], ows[e][0], f"expert {e} codes")
    y64 = O.grouped_gemm64(oa + (1,), d["row_index"], d["offsets"], ows)
    check_gemm(y, y64, what="small moe")


def test_empty_groups_and_pregrouped_rows(nv):
    rng = np.random.default_rng(9)
    experts, n, k = 6, 64, 256
    counts = np.array([0, 40, 0, 0, 300, 1])
    offsets = np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)
    total = int(offsets[-1])
    a = W.to_bf16_bits(rng.standard_normal((total, k)))
    w = W.to_bf16_bits(rng.standard_normal((experts * n, k)) * 0.02)
    wq = quantize_experts(nv, w, experts, n)
    y = nv.grouped_gemm_w4a4(dev_bf16(a), None, torch.from_numpy(offsets).cuda(), wq, n, total)
    y64 = O.grouped_gemm64(O.quantize_1d(a) + (1,), None, offsets, oracle_experts(w, experts, n))
    check_gemm(y, y64, what="pregrouped")


def test_moe_config_full_size_sampled(nv):
    """4096 tokens, hidden 2048, 128 experts of 768 x 2048, top-8 Zipf routing: every output row
    of 12 sampled experts (including the hottest and the coldest) against the oracle."""
    d = W.moe()
    experts, n = d["experts"], d["n"]
    wq = quantize_experts(nv, d["w"], experts, n)
    ri = torch.from_numpy(d["row_index"]).cuda()
    off = torch.from_numpy(d["offsets"]).cuda()
    total = int(d["offsets"][-1])
    assert total == 4096 * 8
    y = nv.grouped_gemm_w4a4(dev_bf16(d["a"]), ri, off, wq, n, total).cpu()
    oa = O.quantize_1d(d["a"]) + (1,)
    ahat = O.dequantize(*oa, out="f64")
    counts = d["counts"]
    rng = np.random.default_rng(3)
    sample = np.unique(np.concatenate([[int(np.argmax(counts)), int(np.argmin(counts))],
                                       rng.choice(experts, 10, replace=False)]))
    wc, ws, wg = host_q(wq)
    for e in sample:
        ow = O.quantize_2d(d["w"][e * n:(e + 1) * n]) + (16,)
        assert np.float32(wg[e]) == ow[2]
        assert_codes_equal(wc[e * n:(e + 1) * n], ow[0], f"expert {e} codes")
        lo, hi = d["offsets"][e], d["offsets"][e + 1]
        y64 = ahat[d["row_index"][lo:hi]] @ O.dequantize(*ow, out="f64").T
        check_gemm(y[lo:hi], y64, what=f"expert {e} ({hi - lo} rows)")
