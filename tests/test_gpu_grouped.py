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


def quantize_experts(nv, w_stacked, experts, n, br=16):
    """Each expert's weights quantized on its own (own global scale) into one stacked tensor
    (16x16 tiles, or 1D blocks with br = 1)."""
    k = w_stacked.shape[1]
    wq = nv.empty_qtensor(experts * n, k, br, n_global_scales=experts)
    for e in range(experts):
        part = nv.QTensor(wq.codes[e * n:(e + 1) * n], wq.scales[e * n // br:(e + 1) * n // br],
                          wq.global_scale[e:e + 1], n, k, br)
        (nv.quantize_2d if br == 16 else nv.quantize_1d)(dev_bf16(w_stacked[e * n:(e + 1) * n]),
                                                        out=part)
    return wq


def oracle_experts(w_stacked, experts, n, br=16):
    q = O.quantize_2d if br == 16 else O.quantize_1d
    return [q(w_stacked[e * n:(e + 1) * n]) + (br,) for e in range(experts)]


# hidden 528 is not a multiple of 64 (the register-prefetch grouped kernel); br = 1 takes the 1D
# weight-scale forms of both grouped kernels.
@pytest.mark.parametrize("tokens,hidden,experts,topk,n,br", [(256, 256, 8, 2, 128, 16),
                                                              (300, 528, 16, 4, 80, 16),
                                                              (64, 1024, 5, 5, 256, 16),
                                                              (256, 512, 8, 2, 136, 1),
                                                              (300, 528, 16, 4, 72, 1)])
def test_small_moe(nv, tokens, hidden, experts, topk, n, br):
    d = W.moe(seed=tokens, tokens=tokens, hidden=hidden, experts=experts, topk=topk, n=n)
    wq = quantize_experts(nv, d["w"], experts, n, br)
    ri = torch.from_numpy(d["row_index"]).cuda()
    off = torch.from_numpy(d["offsets"]).cuda()
    total = int(d["offsets"][-1])
    aq = nv.empty_qtensor(tokens, hidden, 1)
    y = nv.grouped_gemm_w4a4(dev_bf16(d["a"]), ri, off, wq, n, total, a_q=aq)
    oa = O.quantize_1d(d["a"])
    ac, as_, ag = host_q(aq)
    assert np.float32(ag) == oa[2]
    assert_codes_equal(ac, oa[0], "moe A codes")
    ows = oracle_experts(d["w"], experts, n, br)
    wc, ws, wg = host_q(wq)
    for e in range(experts):
        assert np.float32(wg[e]) == ows[e][2]
        assert_codes_equal(wc[e * n:(e + 1) * n], ows[e][0], f"expert {e} codes")
        assert_codes_equal(ws[e * n // br:(e + 1) * n // br], ows[e][1], f"expert {e} scales")
    y64 = O.grouped_gemm64(oa + (1,), d["row_index"], d["offsets"], ows)
    check_gemm(y, y64, what="small moe")


@pytest.mark.parametrize("br", [16, 1])
def test_partial_last_tiles(nv, br):
    """Groups whose last 128-row tile holds 1 to 128 rows: the grouped kernel multiplies only
    the 32-row fragments of A that hold rows of the group (1, 2, 3 or 4 of them), and every
    class, with its boundary row counts, is checked against the oracle."""
    rng = np.random.default_rng(11 + br)
    counts = np.array([1, 31, 32, 33, 64, 65, 96, 97, 127, 128, 129, 160, 193, 250, 0, 5])
    experts, n, k, tokens = len(counts), 272, 512, 700
    offsets = np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)
    total = int(offsets[-1])
    row_index = rng.integers(0, tokens, total).astype(np.int32)
    a = W.to_bf16_bits(rng.standard_normal((tokens, k)))
    w = W.to_bf16_bits(rng.standard_normal((experts * n, k)) * 0.02)
    wq = quantize_experts(nv, w, experts, n, br)
    y = nv.grouped_gemm_w4a4(dev_bf16(a), torch.from_numpy(row_index).cuda(),
                             torch.from_numpy(offsets).cuda(), wq, n, total)
    y64 = O.grouped_gemm64(O.quantize_1d(a) + (1,), row_index, offsets,
                           oracle_experts(w, experts, n, br))
    check_gemm(y, y64, what=f"partial last tiles br={br}")


@pytest.mark.parametrize("k", [64, 48])
def test_most_groups_the_library_takes(nv, k):
    """1024 experts (the largest count the call accepts), most of them empty, a few rows in the
    others: the device scan of the offsets covers its whole range, in both grouped kernels (K a
    multiple of 64, and not)."""
    rng = np.random.default_rng(21 + k)
    experts, n, tokens = 1024, 16, 96
    counts = np.zeros(experts, dtype=np.int64)
    hot = rng.choice(experts, size=40, replace=False)
    counts[hot] = rng.integers(1, 20, size=40)
    counts[experts - 1] = 3  # the last group is not empty
    offsets = np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)
    total = int(offsets[-1])
    row_index = rng.integers(0, tokens, total).astype(np.int32)
    a = W.to_bf16_bits(rng.standard_normal((tokens, k)))
    w = W.to_bf16_bits(rng.standard_normal((experts * n, k)) * 0.02)
    wq = quantize_experts(nv, w, experts, n)
    y = nv.grouped_gemm_w4a4(dev_bf16(a), torch.from_numpy(row_index).cuda(),
                             torch.from_numpy(offsets).cuda(), wq, n, total)
    y64 = O.grouped_gemm64(O.quantize_1d(a) + (1,), row_index, offsets,
                           oracle_experts(w, experts, n))
    check_gemm(y, y64, what=f"1024 groups k={k}")


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


def test_moe_config_full_size(nv):
    """4096 tokens, hidden 2048, 128 experts of 768 x 2048, top-8 Zipf routing: the quantized
    tokens the call writes and every expert's weights byte for byte, then every output row of
    every expert (37 to 3,699 rows each) against a float64 product of the reconstructed
    operands."""
    d = W.moe()
    experts, n = d["experts"], d["n"]
    wq = quantize_experts(nv, d["w"], experts, n)
    ri = torch.from_numpy(d["row_index"]).cuda()
    off = torch.from_numpy(d["offsets"]).cuda()
    total = int(d["offsets"][-1])
    assert total == 4096 * 8
    aq = nv.empty_qtensor(4096, 2048, 1)
    y = nv.grouped_gemm_w4a4(dev_bf16(d["a"]), ri, off, wq, n, total, a_q=aq).cpu()
    oa = O.quantize_1d(d["a"]) + (1,)
    ac, as_, ag = host_q(aq)
    assert np.float32(ag) == oa[2]
    assert_codes_equal(ac, oa[0], "moe A codes")
    assert_codes_equal(as_, oa[1], "moe A scales")
    ahat = O.dequantize(*oa, out="f64")
    wc, ws, wg = host_q(wq)
    worst = 0.0
    for e in range(experts):
        ow = O.quantize_2d(d["w"][e * n:(e + 1) * n]) + (16,)
        assert np.float32(wg[e]) == ow[2]
        assert_codes_equal(wc[e * n:(e + 1) * n], ow[0], f"expert {e} codes")
        assert_codes_equal(ws[e * n // 16:(e + 1) * n // 16], ow[1], f"expert {e} scales")
        lo, hi = d["offsets"][e], d["offsets"][e + 1]
        y64 = ahat[d["row_index"][lo:hi]] @ O.dequantize(*ow, out="f64").T
        worst = max(worst, check_gemm(y[lo:hi], y64, what=f"expert {e} ({hi - lo} rows)",
                                      min_agree=0.99))
    print(f"moe: all {experts} experts, worst err/tol {worst:.4f}")


def test_debug_routing_checks(nv):
    """NVFP4_DEBUG=1: the grouped call copies its routing arrays to the host first and rejects
    bad ones with NVFP4_ERR_SHAPE, launching nothing; good ones give the same result as without
    the check.  (The environment variable is read on every grouped call.)"""
    import os
    d = W.moe(seed=7, tokens=64, hidden=256, experts=4, topk=2, n=64)
    wq = quantize_experts(nv, d["w"], 4, 64)
    a = dev_bf16(d["a"])
    total = int(d["offsets"][-1])
    ri = torch.from_numpy(d["row_index"]).cuda()
    off = torch.from_numpy(d["offsets"]).cuda()
    y_ref = nv.grouped_gemm_w4a4(a, ri, off, wq, 64, total)
    bad_cases = {
        "offsets[0] != 0": (ri, np.array([1, 40, 80, 100, 128], dtype=np.int32)),
        "decreasing offsets": (ri, np.array([0, 60, 50, 100, 128], dtype=np.int32)),
        "last offset past total_rows": (ri, np.array([0, 40, 80, 100, 129], dtype=np.int32)),
        "row index >= tokens": (torch.from_numpy(np.where(np.arange(total) == 5, 64,
                                                          d["row_index"]).astype(np.int32)).cuda(),
                                d["offsets"]),
        "negative row index": (torch.from_numpy(np.where(np.arange(total) == 9, -1,
                                                         d["row_index"]).astype(np.int32)).cuda(),
                               d["offsets"]),
    }
    old = os.environ.get("NVFP4_DEBUG")
    os.environ["NVFP4_DEBUG"] = "1"
    try:
        y = nv.grouped_gemm_w4a4(a, ri, off, wq, 64, total)
        assert torch.equal(y, y_ref)
        for what, (rix, offs) in bad_cases.items():
            y_bad = torch.full((total, 64), 7.0, dtype=torch.bfloat16, device="cuda")
            with pytest.raises(nv.Nvfp4Error) as ei:
                nv.grouped_gemm_w4a4(a, rix, torch.from_numpy(offs).cuda(), wq, 64, total,
                                     y=y_bad)
            assert ei.value.status == nv.ERR_SHAPE, what
            torch.cuda.synchronize()
            assert torch.all(y_bad == 7.0), what + ": output written"
    finally:
        if old is None:
            del os.environ["NVFP4_DEBUG"]
        else:
            os.environ["NVFP4_DEBUG"] = old
