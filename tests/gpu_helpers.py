"""Helpers shared by the GPU parity tests: moving bf16 bit patterns to the device and quantized
tensors back, and the oracle-side references."""

import numpy as np
import torch

from oracle import nvfp4_oracle as O


def dev_bf16(u16):
    """numpy uint16 bf16 bits -> contiguous torch bf16 on cuda:0."""
    return torch.from_numpy(np.ascontiguousarray(u16).view(np.int16)).view(torch.bfloat16).cuda()


def host_q(q):
    """QTensor -> (codes rows x cols/2, scales, gs) as numpy, padding stripped."""
    torch.cuda.synchronize()
    codes = q.codes[:, : q.cols // 2].cpu().numpy()
    scales = q.scales.cpu().numpy()
    gs = q.global_scale.cpu().numpy()
    return codes, scales, (gs[0] if gs.size == 1 else gs)


def bf16_to_f64(t):
    return t.float().cpu().numpy().astype(np.float64)


def assert_codes_equal(got, want, what=""):
    """Byte-exact comparison with a readable first mismatch."""
    got, want = np.asarray(got), np.asarray(want)
    assert got.shape == want.shape, (what, got.shape, want.shape)
    bad = np.argwhere(got != want)
    if bad.size:
        i = tuple(bad[0])
        raise AssertionError(f"{what}: {len(bad)} mismatches, first at {i}: got {got[i]:#x} "
                             f"want {want[i]:#x}")


def rn_bf16_f64(y):
    """RN_bf16 (nearest, ties to even) of float64 values, rounded once from float64 (values in
    bf16's normal range or zero; used only to report agreement)."""
    b = np.ascontiguousarray(y, dtype=np.float64).view(np.uint64)
    lsb = (b >> np.uint64(45)) & np.uint64(1)
    r = ((b + np.uint64((1 << 44) - 1) + lsb) >> np.uint64(45)) << np.uint64(45)
    return r.view(np.float64)


# Results of the last check_gemm calls (worst error / bound, share equal to RN_bf16(Y64)), for
# the report the config tests print.
LAST = {}


def check_gemm(y_gpu, y64, rel=1e-3, what="", min_agree=None):
    """|Y - Y64| <= rel * ||Y64[m, :]||_2 + 2^-8 |Y64[m, n]| for every element (accumulation
    budget plus the bf16 store's half ulp).  Also measures the share of outputs equal to
    RN_bf16(Y64), the exact product rounded once: with an accurate fp32 accumulation almost every
    output rounds to it, so `min_agree` (when given) is asserted as a floor.  Returns the worst
    error / bound ratio."""
    y = bf16_to_f64(y_gpu) if isinstance(y_gpu, torch.Tensor) else y_gpu
    tol = O.gemm_tolerance(y64, rel)
    err = np.abs(y - y64)
    ratio = np.where(tol > 0, err / np.where(tol > 0, tol, 1), np.where(err > 0, np.inf, 0))
    worst = float(ratio.max()) if ratio.size else 0.0
    agree = float(np.mean(y == rn_bf16_f64(y64))) if y.size else 1.0
    LAST[what] = (worst, agree)
    print(f"[check_gemm] {what}: max err/tol {worst:.4f}, equal to RN_bf16(Y64) {agree:.6f}",
          flush=True)
    assert worst <= 1.0, f"{what}: max err / tol = {worst:.3g}"
    if min_agree is not None:
        assert agree >= min_agree, f"{what}: only {agree:.5f} of outputs equal RN_bf16(Y64)"
    return worst
