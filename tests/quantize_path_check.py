"""Run as a separate process by test_gpu_quantize.py: quantizes a few tensors on whatever 1D path
NVFP4_QUANT_PATH selects, with the grid barrier's poll bound NVFP4_QUANT_SPIN_LIMIT (the library
reads both once per process), and compares every byte with the oracle.  With a poll bound of 0
every workgroup of the single-read kernel gives up on the barrier and reads the whole tensor for
the maximum; the status word of the workspace (its count of such workgroups) must then grow by
one per compute unit per call.  Prints one line per case; exit status 0 when all match."""

import os
import sys

import numpy as np

sys.path.insert(0, os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
sys.path.insert(0, os.path.dirname(os.path.abspath(__file__)))

from oracle import nvfp4_oracle as O  # noqa: E402
from nvfp4_w4a4_quantized_amax_amd import nvfp4 as nv  # noqa: E402
from nvfp4_w4a4_quantized_amax_amd import workloads as W  # noqa: E402
from gpu_helpers import assert_codes_equal, dev_bf16, host_q  # noqa: E402


def main():
    import torch
    path = os.environ.get("NVFP4_QUANT_PATH", "") + " spin=" + os.environ.get(
        "NVFP4_QUANT_SPIN_LIMIT", "default")
    # the default (ordinary) launch of the single-read kernel with a poll bound of 0
    spin0 = (os.environ.get("NVFP4_QUANT_SPIN_LIMIT") == "0"
             and not os.environ.get("NVFP4_QUANT_PATH"))
    ws = nv.Workspace.get(nv.lib().nvfp4_quantize_workspace_bytes(1, 16), "cuda")
    status_off = 8192 - 64
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    rng = np.random.default_rng(11)
    cases = {
        "activation band 512x8192": W.activation(seed=1, rows=512, cols=8192)["x"],
        "ragged 1000x1040": W.to_bf16_bits(rng.laplace(0, 1, (1000, 1040))),
        "strided 700x1024 (ld 1088)": None,
        # two-kernel path: 4 or 5 tiles per wave of the encode pass, the last tile partial
        "ragged 5001x4112": W.to_bf16_bits(rng.laplace(0, 1, (5001, 4112))),
    }
    big = W.to_bf16_bits(rng.standard_normal((700, 1088)))
    for name, x in cases.items():
        if x is None:
            xt = dev_bf16(big)[:, 32:32 + 1024]
            want = O.quantize_1d(np.ascontiguousarray(big[:, 32:32 + 1024]))
        else:
            xt = dev_bf16(x)
            want = O.quantize_1d(x)
        before = int(ws[status_off:status_off + 4].view(torch.int32).item())
        c, s, g = host_q(nv.quantize_1d(xt, ws=ws))
        after = int(ws[status_off:status_off + 4].view(torch.int32).item())
        if spin0:
            assert after - before == cus, (path, name, before, after, cus)
        assert np.float32(g) == want[2], (path, name, g, want[2])
        assert_codes_equal(s, want[1], f"{path} {name} scales")
        assert_codes_equal(c, want[0], f"{path} {name} codes")
        print(f"{path}: {name} ok", flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
