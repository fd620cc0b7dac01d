"""Run as a separate process by test_gpu_quantize.py: quantizes a few tensors on whatever 1D path
NVFP4_QUANT_PATH selects (the library reads it once per process) and compares every byte with
the oracle.  Prints one line per case; exit status 0 when all match."""

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
    path = os.environ.get("NVFP4_QUANT_PATH", "")
    rng = np.random.default_rng(11)
    cases = {
        "activation band 512x8192": W.activation(seed=1, rows=512, cols=8192)["x"],
        "ragged 1000x1040": W.to_bf16_bits(rng.laplace(0, 1, (1000, 1040))),
        "strided 700x1024 (ld 1088)": None,
    }
    big = W.to_bf16_bits(rng.standard_normal((700, 1088)))
    for name, x in cases.items():
        if x is None:
            xt = dev_bf16(big)[:, 32:32 + 1024]
            want = O.quantize_1d(np.ascontiguousarray(big[:, 32:32 + 1024]))
        else:
            xt = dev_bf16(x)
            want = O.quantize_1d(x)
        c, s, g = host_q(nv.quantize_1d(xt))
        assert np.float32(g) == want[2], (path, name, g, want[2])
        assert_codes_equal(s, want[1], f"{path} {name} scales")
        assert_codes_equal(c, want[0], f"{path} {name} codes")
        print(f"{path}: {name} ok", flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
