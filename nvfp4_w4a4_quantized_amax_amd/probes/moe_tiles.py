"""Measurement program (not part of libnvfp4): the grouped W4A4 product's time against its
tile count.  128 experts of 768 x 2048 (16x16 tile scales), 4096 tokens quantized beforehand
(so only the grouped product kernel runs), and routings with equal rows per expert (one round
of the 512 workgroup slots, 1.0, 1.5 and 2.25 rounds of 128 x 256 tiles) beside the Zipf(1.1)
top-8 routing of the MoE benchmark workload.  Each line: the best of 5 batches of 20 calls
(HIP events), the tile count, and TFLOP/s over the routed rows.

    python nvfp4_w4a4_quantized_amax_amd/probes/moe_tiles.py
"""
import os
import sys

import numpy as np
import torch

sys.path.insert(0, os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__)))))
from nvfp4_w4a4_quantized_amax_amd import nvfp4 as nv  # noqa: E402
from nvfp4_w4a4_quantized_amax_amd import workloads as W  # noqa: E402

E, N, K, TOKENS = 128, 768, 2048, 4096


def bf16(u16):
    return torch.from_numpy(np.ascontiguousarray(u16).view(np.int16)).view(torch.bfloat16).cuda()


def main():
    rng = np.random.default_rng(1)
    aq = nv.quantize_1d(bf16(W.to_bf16_bits(rng.standard_normal((TOKENS, K)))))
    wb = bf16(W.to_bf16_bits(rng.standard_normal((E * N, K)) * 0.02))
    wq = nv.empty_qtensor(E * N, K, 16, n_global_scales=E)
    for e in range(E):
        part = nv.QTensor(wq.codes[e * N:(e + 1) * N], wq.scales[e * N // 16:(e + 1) * N // 16],
                          wq.global_scale[e:e + 1], N, K, 16)
        nv.quantize_2d(wb[e * N:(e + 1) * N], out=part)

    def run(counts, label):
        counts = np.asarray(counts, dtype=np.int64)
        off = np.zeros(E + 1, dtype=np.int32)
        off[1:] = np.cumsum(counts)
        total = int(off[-1])
        ri = torch.from_numpy((np.arange(total) % TOKENS).astype(np.int32)).cuda()
        offd = torch.from_numpy(off).cuda()
        y = torch.empty((total, N), dtype=torch.bfloat16, device="cuda")
        tiles = int(sum((c + 127) // 128 for c in counts)) * (N // 256)
        call = lambda: nv.grouped_gemm_w4a4(aq, ri, offd, wq, N, total, y=y)  # noqa: E731
        for _ in range(5):
            call()
        torch.cuda.synchronize()
        best = 1e9
        for _ in range(5):
            s, t = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            s.record()
            for _ in range(20):
                call()
            t.record()
            torch.cuda.synchronize()
            best = min(best, s.elapsed_time(t) / 20 * 1000)
        print(f"{label:34s} rows {total:6d} tiles {tiles:5d}: {best:8.2f} us "
              f"{2 * total * N * K / best / 1e6:7.1f} TFLOP/s", flush=True)

    run([128] * E, "128 rows per expert")
    run([256] * 42 + [128] * 86, "170 row tiles (510 tiles)")
    run([256] * E, "256 rows per expert")
    run([384] * E, "384 rows per expert")
    run(W.moe()["counts"], "Zipf(1.1) top-8, 32768 rows")
    return 0


if __name__ == "__main__":
    sys.exit(main())
