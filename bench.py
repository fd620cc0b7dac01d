"""Benchmark of the NVFP4 W4A4 hot path on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-extra] [--no-cpu]

Prints ONE JSON line.  The headline step is the dynamic NVFP4 quantization of the 8192 x 8192
activation workload (Laplace(0,1) x LogNormal(0,1) column gains, seed 1): global amax, FP32
global scale, E4M3 scale per 16 values, E2M1 codes packed two per byte.  It is HBM-bound; its
algorithmic traffic is the bf16 input read once plus the packed outputs written once:
2.5625 bytes per value, 171,966,468 bytes per step.

Timing: K steps between two HIP events on the stream the library launches on, after W warm-up
steps, with synchronization on both sides.  Inputs are resident in HBM; the step rotates over
enough distinct input/output buffers (4 x 168 MiB) that no step finds its input in the 256 MB
Infinity Cache left there by the previous step.

"workloads" adds the other shapes the library serves (decode-, prefill- and MoE-shaped W4A4
GEMMs, activation quantization inside the call; the weight-only W4A16 form of the decode
shapes), each timed the same way with its own roofline.
"cpu_baseline" times the CPU oracle (test infrastructure, float64 numpy) on the same headline
input on the host.
"""

import argparse
import json
import os
import sys
import time

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, GB/s
FP16_MFMA_PEAK_TFLOPS = 2500.0  # MI355X dense fp16/bf16 MFMA, TFLOP/s
FP4_MFMA_PEAK_TFLOPS = 10100.0  # MI355X dense fp4 (and fp6) MFMA, TFLOP/s
METRIC = "W4A4 GEMM TFLOP/s + NVFP4 quantize GB/s, as % of MI355X roofline"


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=100)
    p.add_argument("--warmup", type=int, default=10)
    p.add_argument("--no-extra", action="store_true", help="headline workload only")
    p.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    p.add_argument("--only", default="", help="comma list of extra workloads to run")
    p.add_argument("--copy-calibration", action="store_true",
                   help="after the headline, run 5 plain device copies of the 128 MiB input "
                        "(reference dispatches for scaling the FETCH_SIZE / WRITE_SIZE counters)")
    return p.parse_args()


def timed(fn, steps, warmup, torch):
    """Average ms per call of fn(i) over `steps` calls, bracketed by HIP events on the current
    stream (the one the library launches on), after `warmup` calls."""
    for i in range(warmup):
        fn(i)
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    start.record(stream)
    for i in range(steps):
        fn(i)
    end.record(stream)
    torch.cuda.synchronize()
    return start.elapsed_time(end) / steps


def dev_bf16(torch, np, u16):
    return torch.from_numpy(np.ascontiguousarray(u16).view(np.int16)).view(torch.bfloat16).cuda()


def headline(args, torch, np, nv, W):
    rows = cols = 8192
    x_host = W.activation(seed=1, rows=rows, cols=cols)["x"]
    x0 = dev_bf16(torch, np, x_host)
    nbuf = 4
    xs = [x0] + [x0.clone() for _ in range(nbuf - 1)]
    qs = [nv.empty_qtensor(rows, cols, 1) for _ in range(nbuf)]
    ws = nv.Workspace.get(nv.lib().nvfp4_quantize_workspace_bytes(rows, cols), x0.device)

    def step(i):
        nv.quantize_1d(xs[i % nbuf], out=qs[i % nbuf], ws=ws)

    ms = timed(step, args.steps, args.warmup, torch)
    nbytes = rows * cols * 2 + rows * cols // 2 + rows * cols // 16 + 4
    gbs = nbytes / (ms * 1e-3) / 1e9
    if args.copy_calibration:
        dst = torch.empty_like(x0)
        for i in range(5):
            dst.copy_(xs[i % nbuf])
        torch.cuda.synchronize()
    return {"ms": ms, "bytes": nbytes, "gbs": gbs, "x_host": x_host}


TRAFFIC_FILE = os.path.join(os.path.dirname(os.path.abspath(__file__)), "profiles",
                            "k_quantize_persistent_activation_8192x8192_traffic.md")
QUANTIZE_SOURCES = ("quantize.hip", "nvfp4_device.hpp")


def quantize_source_hash():
    import hashlib
    h = hashlib.sha256()
    csrc = os.path.join(os.path.dirname(os.path.abspath(__file__)), "nvfp4_w4a4_quantized_amax_amd",
                        "csrc")
    for name in QUANTIZE_SOURCES:
        with open(os.path.join(csrc, name), "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def measured_traffic():
    """HBM bytes per launch of the headline kernel from the committed counter summary, or None
    when there is none or the kernel sources changed since the counters were taken."""
    try:
        text = open(TRAFFIC_FILE).read()
    except OSError:
        return None
    fields = {}
    for line in text.splitlines():
        if line.startswith("- ") and ": " in line:
            k, v = line[2:].split(": ", 1)
            fields[k.strip()] = v.strip().strip("`")
    if fields.get("source_sha256") != quantize_source_hash():
        return None
    try:
        return int(fields["traffic_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def extra_workloads(args, torch, np, nv, W, only):
    out = {}
    steps = max(10, args.steps // 2)
    warm = max(2, args.warmup)

    if not only or "decode" in only:
        # M = 1, 8, 16 (the decode configuration) and a batched M = 64 (split-K tiled product)
        d = W.decode(ms=(1, 8, 16, 64))
        wq0 = nv.quantize_2d(dev_bf16(torch, np, d["w"]))
        nw = 10  # 10 x 29.6 MB of weights > the 256 MB Infinity Cache
        wqs = [wq0] + [nv.QTensor(wq0.codes.clone(), wq0.scales.clone(), wq0.global_scale.clone(),
                                  wq0.rows, wq0.cols, 16) for _ in range(nw - 1)]
        n, k = 14336, 4096
        for m, a_host in d["a"].items():
            a = dev_bf16(torch, np, a_host)
            y = torch.empty((m, n), dtype=torch.bfloat16, device="cuda")
            ws = nv.Workspace.get(nv.lib().nvfp4_gemm_workspace_bytes(m, n, k), a.device)
            ms = timed(lambda i: nv.gemm_w4a4(a, wqs[i % nw], y=y, ws=ws), steps, warm, torch)
            nbytes = n * k // 2 + (n // 16) * (k // 16) + 4 + m * k * 2 + m * n * 2
            gbs = nbytes / (ms * 1e-3) / 1e9
            out[f"decode_m{m}"] = {
                "shape": [m, n, k], "ms": ms, "bound": "hbm", "achieved": gbs,
                "unit": "GB/s", "frac": gbs / HBM_PEAK_GBS,
                "tflops": 2 * m * n * k / (ms * 1e-3) / 1e12}
            if m > 16:  # the weight-only form serves m <= 16
                continue
            # Weight-only form of the same product: the bf16 A is used as is.
            ms = timed(lambda i: nv.gemm_w4a16(a, wqs[i % nw], y=y), steps, warm, torch)
            gbs = nbytes / (ms * 1e-3) / 1e9
            out[f"decode_w4a16_m{m}"] = {
                "shape": [m, n, k], "ms": ms, "bound": "hbm", "achieved": gbs,
                "unit": "GB/s", "frac": gbs / HBM_PEAK_GBS,
                "tflops": 2 * m * n * k / (ms * 1e-3) / 1e12}
        del wqs, wq0

    if not only or "prefill" in only:
        d = W.prefill()
        a = dev_bf16(torch, np, d["a"])
        wq = nv.quantize_2d(dev_bf16(torch, np, d["w"]))
        m = n = k = 8192
        y = torch.empty((m, n), dtype=torch.bfloat16, device="cuda")
        ws = nv.Workspace.get(nv.lib().nvfp4_gemm_workspace_bytes(m, n, k), a.device)
        ps = max(5, steps // 5)
        ms = timed(lambda i: nv.gemm_w4a4(a, wq, y=y, ws=ws), ps, warm, torch)
        tf = 2 * m * n * k / (ms * 1e-3) / 1e12
        out["prefill"] = {"shape": [m, n, k], "ms": ms, "bound": "mfma", "achieved": tf,
                          "unit": "TFLOP/s", "peak": FP16_MFMA_PEAK_TFLOPS,
                          "frac": tf / FP16_MFMA_PEAK_TFLOPS,
                          "note": "includes the dynamic quantization of A inside the call"}
        del a, wq, y

    if not only or "mxfp4" in only:
        # MXFP4 (E8M0 per 32 values): the headline activation quantized in one pass, and the
        # prefill product with both operands MXFP4 on the scaled FP4 MFMA.
        x = W.activation()["x"]
        xs = [dev_bf16(torch, np, x)] + [None] * 3
        for i in range(1, 4):
            xs[i] = xs[0].clone()
        qs = [nv.empty_mxtensor(8192, 8192) for _ in range(4)]
        ms = timed(lambda i: nv.mxfp4_quantize(xs[i % 4], out=qs[i % 4]), steps, warm, torch)
        nbytes = 8192 * 8192 * 2 + 8192 * 8192 // 2 + 8192 * 8192 // 32
        gbs = nbytes / (ms * 1e-3) / 1e9
        out["mxfp4_quantize"] = {"shape": [8192, 8192], "ms": ms, "bound": "hbm",
                                 "achieved": gbs, "unit": "GB/s", "frac": gbs / HBM_PEAK_GBS,
                                 "algorithmic_bytes": nbytes}
        del xs, qs
        d = W.prefill()
        a = dev_bf16(torch, np, d["a"])
        wq = nv.mxfp4_quantize(dev_bf16(torch, np, d["w"]))
        m = n = k = 8192
        y = torch.empty((m, n), dtype=torch.bfloat16, device="cuda")
        ws = nv.Workspace.get(nv.lib().nvfp4_mxfp4_gemm_workspace_bytes(m, k), a.device)
        ps = max(5, steps // 5)
        ms = timed(lambda i: nv.mxfp4_gemm(a, wq, y=y, ws=ws), ps, warm, torch)
        tf = 2 * m * n * k / (ms * 1e-3) / 1e12
        out["mxfp4_prefill"] = {"shape": [m, n, k], "ms": ms, "bound": "mfma", "achieved": tf,
                                "unit": "TFLOP/s", "peak": FP4_MFMA_PEAK_TFLOPS,
                                "frac": tf / FP4_MFMA_PEAK_TFLOPS,
                                "note": "includes the MXFP4 quantization of A inside the call"}
        del a, wq, y
        # Decode-shaped MXFP4 products against the decode weight (14336 x 4096) rotating over 10
        # copies so that W comes from HBM; the activation is quantized inside each call.
        d = W.decode(ms=(1, 16, 64))
        wq0 = nv.mxfp4_quantize(dev_bf16(torch, np, d["w"]))
        nw = 10
        wqs = [wq0] + [nv.MxTensor(wq0.codes.clone(), wq0.scales.clone(), wq0.rows, wq0.cols)
                       for _ in range(nw - 1)]
        n, k = 14336, 4096
        for m, a_host in d["a"].items():
            a = dev_bf16(torch, np, a_host)
            y = torch.empty((m, n), dtype=torch.bfloat16, device="cuda")
            ws = nv.Workspace.get(nv.lib().nvfp4_mxfp4_gemm_workspace_bytes(m, k), a.device)
            ms = timed(lambda i: nv.mxfp4_gemm(a, wqs[i % nw], y=y, ws=ws), steps, warm, torch)
            nbytes = n * k // 2 + n * k // 32 + m * k * 2 + m * n * 2
            gbs = nbytes / (ms * 1e-3) / 1e9
            out[f"mxfp4_decode_m{m}"] = {
                "shape": [m, n, k], "ms": ms, "bound": "hbm", "achieved": gbs, "unit": "GB/s",
                "frac": gbs / HBM_PEAK_GBS, "tflops": 2 * m * n * k / (ms * 1e-3) / 1e12,
                "note": "includes the MXFP4 quantization of A inside the call"}
        del wqs, wq0

    if not only or "mse" in only:
        # Offline weight quantization with MSE-observer block scales (16x16 tiles) of the decode
        # weight: 18 candidate scales per tile, so it is bound by vector ALU work, not HBM.
        d = W.decode()
        wdev = dev_bf16(torch, np, d["w"])
        q = nv.empty_qtensor(14336, 4096, 16)
        ws = nv.Workspace.get(nv.lib().nvfp4_quantize_workspace_bytes(14336, 4096), wdev.device)
        ms = timed(lambda i: nv.quantize_mse(wdev, 16, out=q, ws=ws), max(5, steps // 5), warm,
                   torch)
        vals = 14336 * 4096
        out["mse_quantize_2d"] = {"shape": [14336, 4096], "ms": ms, "bound": "alu",
                                  "gvalues_per_s": vals / (ms * 1e-3) / 1e9,
                                  "note": "offline; 18 candidate scales per 16x16 tile"}
        del wdev, q

    if not only or "moe" in only:
        d = W.moe()
        experts, n = d["experts"], d["n"]
        k = d["a"].shape[1]
        wq = nv.empty_qtensor(experts * n, k, 16, n_global_scales=experts)
        wdev = dev_bf16(torch, np, d["w"])
        for e in range(experts):
            part = nv.QTensor(wq.codes[e * n:(e + 1) * n], wq.scales[e * n // 16:(e + 1) * n // 16],
                              wq.global_scale[e:e + 1], n, k, 16)
            nv.quantize_2d(wdev[e * n:(e + 1) * n], out=part)
        del wdev
        a = dev_bf16(torch, np, d["a"])
        ri = torch.from_numpy(d["row_index"]).cuda()
        off = torch.from_numpy(d["offsets"]).cuda()
        total = int(d["offsets"][-1])
        y = torch.empty((total, n), dtype=torch.bfloat16, device="cuda")
        ws = nv.Workspace.get(nv.lib().nvfp4_grouped_gemm_workspace_bytes(4096, k, total, experts),
                              a.device)
        ms = timed(lambda i: nv.grouped_gemm_w4a4(a, ri, off, wq, n, total, y=y, ws=ws),
                   steps, warm, torch)
        flops = 2 * total * n * k
        tf = flops / (ms * 1e-3) / 1e12
        out["moe"] = {"shape": [total, n, k, experts], "ms": ms, "bound": "mfma",
                      "achieved": tf, "unit": "TFLOP/s", "peak": FP16_MFMA_PEAK_TFLOPS,
                      "frac": tf / FP16_MFMA_PEAK_TFLOPS,
                      "note": "includes the dynamic quantization of the 4096 x 2048 tokens"}
    return out


def cpu_baseline(x_host, nbytes):
    """The CPU oracle (float64 numpy, test infrastructure) quantizing the same 8192 x 8192
    input; numpy's elementwise work runs on one thread."""
    sys.path.insert(0, os.path.dirname(os.path.abspath(__file__)))
    from oracle import nvfp4_oracle as O
    t0 = time.perf_counter()
    O.quantize_1d(x_host)
    dt = time.perf_counter() - t0
    return {"value": nbytes / dt / 1e9, "unit": "GB/s", "cores": 1, "kind": "oracle",
            "sample": "the full 8192 x 8192 activation workload, one quantize_1d call "
                      f"({dt:.1f} s)"}


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported "
              "(the library has no multi-GPU path).", file=sys.stderr)
        sys.exit(2)
    import numpy as np
    import torch
    from nvfp4_w4a4_quantized_amax_amd import nvfp4 as nv
    from nvfp4_w4a4_quantized_amax_amd import workloads as W

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    h = headline(args, torch, np, nv, W)
    rec = {
        "metric": METRIC,
        "value": h["gbs"],
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": h["ms"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "activation quantize 8192x8192 bf16 (Laplace x LogNormal gains, "
                               "seed 1) -> NVFP4 1D-16", "rows": 8192, "cols": 8192,
                   "global_batch": 8192, "seq_len": 8192, "parallelism": "none"},
        "roofline": {"bound": "hbm", "achieved": h["gbs"], "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": h["gbs"] / HBM_PEAK_GBS, "traffic": measured_traffic(),
                     "kernel": "k_quantize_persistent (nvfp4_quantize_1d, single-read path)",
                     "algorithmic_bytes_per_launch": h["bytes"]},
    }
    if not args.no_extra:
        only = [s for s in args.only.split(",") if s]
        rec["workloads"] = extra_workloads(args, torch, np, nv, W, only)
    if not args.no_cpu:
        rec["cpu_baseline"] = cpu_baseline(h["x_host"], h["bytes"])
    print(json.dumps(rec), flush=True)


if __name__ == "__main__":
    main()
