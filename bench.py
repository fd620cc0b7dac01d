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
shapes; the dequantization of the headline activation; the MXFP4 variant and the MSE-observer
weight quantization), each timed the same way with its own roofline.
"accuracy" reports the error of each format on the same seeded inputs (dequantized tensors
against their bf16 inputs, products against the float64 product of the bf16 inputs).
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


def timed(fn, steps, warmup, torch, stats=True):
    """ms per call of fn(i): the average over `steps` calls bracketed by two HIP events on the
    current stream (the one the library launches on), after `warmup` calls.  With `stats`, a
    second pass times up to 10 batches of consecutive calls the same way (no event between the
    calls of a batch: an event per call adds its own gap to every small kernel) and adds the
    median, p10 and p90 of the batches' per-call times.  Returns (mean_ms, stats or None)."""
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
    mean = start.elapsed_time(end) / steps
    if not stats:
        return mean, None
    nb = min(10, steps)
    per_batch = max(1, steps // nb)
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(2 * nb)]
    i = 0
    for b in range(nb):
        ev[2 * b].record(stream)
        for _ in range(per_batch):
            fn(i)
            i += 1
        ev[2 * b + 1].record(stream)
    torch.cuda.synchronize()
    per = sorted(ev[2 * b].elapsed_time(ev[2 * b + 1]) / per_batch for b in range(nb))
    q = lambda f: per[min(len(per) - 1, int(round(f * (len(per) - 1))))]
    return mean, {"median_ms": q(0.5), "p10_ms": q(0.1), "p90_ms": q(0.9), "batches": nb,
                  "calls_per_batch": per_batch}


def clocks():
    """GPU clocks: the current shader (sclk) and memory (mclk) clock levels from sysfs (read as
    files, so nothing is started inside a process that uses the GPU), else the error."""
    import glob
    out = {}
    for dev in sorted(glob.glob("/sys/class/drm/card*/device")):
        rec = {}
        for name in ("pp_dpm_sclk", "pp_dpm_mclk", "pp_dpm_fclk"):
            try:
                lines = open(os.path.join(dev, name)).read().splitlines()
            except OSError:
                continue
            cur = [l.split(":", 1)[1].strip().rstrip(" *") for l in lines if l.strip().endswith("*")]
            rec[name] = cur[0] if cur else lines
        if rec:
            out[os.path.basename(os.path.dirname(dev))] = rec
    if out:
        return out
    # Fallback: amd-smi in a child process, except under a profiler whose preloaded library
    # would initialise the GPU in the child before it starts its own interpreter.
    if "rocprof" in os.environ.get("LD_PRELOAD", "") or "ROCPROF" in "".join(os.environ):
        return {"error": "no pp_dpm_* clock files readable; amd-smi skipped under a profiler"}
    import subprocess
    try:
        r = subprocess.run(["amd-smi", "metric", "--clock", "--json"], capture_output=True,
                           text=True, timeout=30)
        rep = json.loads(r.stdout)
        return {"amd-smi": [{k: v.get("clk") for k, v in g.get("clock", {}).items()
                             if isinstance(v, dict)} for g in rep.get("gpu_data", rep)]}
    except Exception as e:  # tool missing or output not JSON: say so
        return {"error": f"no pp_dpm_* clock files readable; amd-smi: {e}"}


def copy_bandwidth(torch):
    """Attainable HBM rate on this machine: a device-to-device copy of 1 GiB (torch's copy kernel),
    counted as bytes read plus bytes written; 10 timed copies cycling over 2 sources and 2
    destinations (4 GiB, far beyond the Infinity Cache)."""
    n = 1 << 30
    src = [torch.empty(n, dtype=torch.uint8, device="cuda").fill_(i) for i in range(2)]
    dst = [torch.empty(n, dtype=torch.uint8, device="cuda") for _ in range(2)]
    ms, st = timed(lambda i: dst[i % 2].copy_(src[(i // 2) % 2]), 10, 3, torch)
    del src, dst
    return {"copy_gbs_median": 2 * n / (st["median_ms"] * 1e-3) / 1e9,
            "copy_gbs_mean": 2 * n / (ms * 1e-3) / 1e9, "bytes_per_copy": 2 * n,
            "what": "torch device copy of 1 GiB, read + write bytes / time, median of batches"}


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

    ms, st = timed(step, args.steps, args.warmup, torch)
    nbytes = rows * cols * 2 + rows * cols // 2 + rows * cols // 16 + 4
    gbs = nbytes / (ms * 1e-3) / 1e9
    if args.copy_calibration:
        dst = torch.empty_like(x0)
        for i in range(5):
            dst.copy_(xs[i % nbuf])
        torch.cuda.synchronize()
    return {"ms": ms, "bytes": nbytes, "gbs": gbs, "x_host": x_host, "stats": st,
            "median_gbs": nbytes / (st["median_ms"] * 1e-3) / 1e9}


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


def _rec(ms, st, nbytes=None, flops=None, bound="hbm", peak=None, **extra):
    """One workload record: time per call (mean and per-call statistics) and its roofline."""
    r = {"ms": ms, "median_ms": st["median_ms"], "p10_ms": st["p10_ms"], "p90_ms": st["p90_ms"],
         "bound": bound}
    if nbytes is not None:
        r["algorithmic_bytes"] = nbytes
        r["gbs"] = nbytes / (ms * 1e-3) / 1e9
    if flops is not None:
        r["tflops"] = flops / (ms * 1e-3) / 1e12
    if bound == "hbm":
        r.update(achieved=r["gbs"], unit="GB/s", peak=HBM_PEAK_GBS, frac=r["gbs"] / HBM_PEAK_GBS)
    elif bound == "mfma":
        r.update(achieved=r["tflops"], unit="TFLOP/s", peak=peak, frac=r["tflops"] / peak)
    r.update(extra)
    return r


def extra_workloads(args, torch, np, nv, W, only):
    out = {}
    steps = max(10, args.steps // 2)
    warm = max(2, args.warmup)

    if not only or "decode" in only:
        # M = 1, 8, 16 (the decode configuration) and a batched M = 64 (mid-size product)
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
            nbytes = n * k // 2 + (n // 16) * (k // 16) + 4 + m * k * 2 + m * n * 2
            ms, st = timed(lambda i: nv.gemm_w4a4(a, wqs[i % nw], y=y, ws=ws), steps, warm, torch)
            out[f"decode_m{m}"] = _rec(ms, st, nbytes, 2 * m * n * k, shape=[m, n, k],
                                       note="activation quantized inside the call")
            if m > 16:  # the weight-only form serves m <= 16
                continue
            # The product alone, A already quantized (what the kernel's W stream costs).
            aq = nv.quantize_1d(a)
            ms, st = timed(lambda i: nv.gemm_w4a4(aq, wqs[i % nw], y=y, ws=ws), steps, warm,
                           torch)
            pbytes = nbytes - m * k * 2 + m * k // 2 + m * k // 16 + 4
            out[f"decode_prequantized_m{m}"] = _rec(ms, st, pbytes, 2 * m * n * k,
                                                    shape=[m, n, k])
            # Weight-only form of the same product: the bf16 A is used as is.
            ms, st = timed(lambda i: nv.gemm_w4a16(a, wqs[i % nw], y=y), steps, warm, torch)
            out[f"decode_w4a16_m{m}"] = _rec(ms, st, nbytes, 2 * m * n * k, shape=[m, n, k])
        del wqs, wq0

    if not only or "prefill" in only:
        # Three sets of (A, W, Y): 3 x (128 MiB + 36 MiB + 128 MiB) > 2 x the Infinity Cache.
        d = W.prefill()
        m = n = k = 8192
        a0 = dev_bf16(torch, np, d["a"])
        wq0 = nv.quantize_2d(dev_bf16(torch, np, d["w"]))
        ns = 3
        As = [a0] + [a0.clone() for _ in range(ns - 1)]
        Ws = [wq0] + [nv.QTensor(wq0.codes.clone(), wq0.scales.clone(), wq0.global_scale.clone(),
                                 m, k, 16) for _ in range(ns - 1)]
        Ys = [torch.empty((m, n), dtype=torch.bfloat16, device="cuda") for _ in range(ns)]
        ws = nv.Workspace.get(nv.lib().nvfp4_gemm_workspace_bytes(m, n, k), a0.device)
        ps = max(6, steps // 4)
        ms, st = timed(lambda i: nv.gemm_w4a4(As[i % ns], Ws[i % ns], y=Ys[i % ns], ws=ws), ps,
                       warm, torch)
        out["prefill"] = _rec(ms, st, None, 2 * m * n * k, "mfma", FP16_MFMA_PEAK_TFLOPS,
                              shape=[m, n, k],
                              note="includes the dynamic quantization of A inside the call; "
                                   "3 rotating input/output sets")
        aqs = [nv.quantize_1d(a) for a in As]
        ms, st = timed(lambda i: nv.gemm_w4a4(aqs[i % ns], Ws[i % ns], y=Ys[i % ns], ws=ws), ps,
                       warm, torch)
        out["prefill_prequantized"] = _rec(ms, st, None, 2 * m * n * k, "mfma",
                                           FP16_MFMA_PEAK_TFLOPS, shape=[m, n, k],
                                           note="A quantized beforehand (the product kernel)")
        del As, Ws, Ys, aqs

    if not only or "dequantize" in only:
        # Reconstruction of the quantized 8192 x 8192 activation (row a6), bf16 and fp32 out,
        # over 4 rotating inputs and outputs (4 x (36 MiB + 128 or 256 MiB), past the Infinity
        # Cache, so that neither side is served from it).
        q0 = nv.quantize_1d(dev_bf16(torch, np, W.activation(seed=1, rows=8192, cols=8192)["x"]))
        m = n = 8192
        qs = [q0] + [nv.QTensor(q0.codes.clone(), q0.scales.clone(), q0.global_scale.clone(),
                                m, n, 1) for _ in range(3)]
        inb = m * n // 2 + m * n // 16 + 4
        for dtype, name, esz in ((torch.bfloat16, "dequantize_bf16", 2),
                                 (torch.float32, "dequantize_f32", 4)):
            ys = [torch.empty((m, n), dtype=dtype, device="cuda") for _ in range(4)]
            ms, st = timed(lambda i: nv.dequantize(qs[i % 4], dtype, out=ys[i % 4]), steps, warm,
                           torch)
            out[name] = _rec(ms, st, inb + m * n * esz, shape=[m, n])
            del ys
        del qs, q0

    if not only or "moe" in only:
        d = W.moe()
        experts, n = d["experts"], d["n"]
        k = d["a"].shape[1]
        tokens = d["a"].shape[0]
        wq = nv.empty_qtensor(experts * n, k, 16, n_global_scales=experts)
        wdev = dev_bf16(torch, np, d["w"])
        for e in range(experts):
            part = nv.QTensor(wq.codes[e * n:(e + 1) * n], wq.scales[e * n // 16:(e + 1) * n // 16],
                              wq.global_scale[e:e + 1], n, k, 16)
            nv.quantize_2d(wdev[e * n:(e + 1) * n], out=part)
        del wdev
        ri = torch.from_numpy(d["row_index"]).cuda()
        off = torch.from_numpy(d["offsets"]).cuda()
        total = int(d["offsets"][-1])
        # Four sets of (tokens, expert weights, Y): 4 x 166 MB > 2 x the Infinity Cache.
        ns = 4
        a0 = dev_bf16(torch, np, d["a"])
        As = [a0] + [a0.clone() for _ in range(ns - 1)]
        Ws = [wq] + [nv.QTensor(wq.codes.clone(), wq.scales.clone(), wq.global_scale.clone(),
                                wq.rows, wq.cols, 16) for _ in range(ns - 1)]
        Ys = [torch.empty((total, n), dtype=torch.bfloat16, device="cuda") for _ in range(ns)]
        ws = nv.Workspace.get(nv.lib().nvfp4_grouped_gemm_workspace_bytes(tokens, k, total,
                                                                          experts), a0.device)
        ms, st = timed(lambda i: nv.grouped_gemm_w4a4(As[i % ns], ri, off, Ws[i % ns], n, total,
                                                      y=Ys[i % ns], ws=ws), steps, warm, torch)
        flops = 2 * total * n * k
        # Mixed roofline: the token quantize at HBM rate, then each expert at the slower of its
        # MFMA time and its HBM time (weights, gathered packed rows, bf16 outputs).
        bw, pk = HBM_PEAK_GBS * 1e9, FP16_MFMA_PEAK_TFLOPS * 1e12
        t_roof = (tokens * k * 2 + tokens * k // 2 + tokens * k // 16) / bw
        for rows in d["counts"]:
            rows = int(rows)
            wb = n * k // 2 + (n // 16) * (k // 16) + 4
            t_roof += max(2 * rows * n * k / pk, (wb + rows * (k // 2 + k // 16) + rows * n * 2) / bw)
        out["moe"] = _rec(ms, st, None, flops, "mfma", FP16_MFMA_PEAK_TFLOPS,
                          shape=[total, n, k, experts],
                          mixed_roofline_ms=t_roof * 1e3, mixed_roofline_frac=t_roof * 1e3 / ms,
                          note="includes the dynamic quantization of the 4096 x 2048 tokens; "
                               "4 rotating input/weight/output sets")
        del As, Ws, Ys

    if not only or "mxfp4" in only:
        # MXFP4 (E8M0 per 32 values): the headline activation quantized in one pass, and the
        # prefill product with both operands MXFP4 on the scaled FP4 MFMA.
        x = W.activation()["x"]
        xs = [dev_bf16(torch, np, x)] + [None] * 3
        for i in range(1, 4):
            xs[i] = xs[0].clone()
        qs = [nv.empty_mxtensor(8192, 8192) for _ in range(4)]
        nbytes = 8192 * 8192 * 2 + 8192 * 8192 // 2 + 8192 * 8192 // 32
        ms, st = timed(lambda i: nv.mxfp4_quantize(xs[i % 4], out=qs[i % 4]), steps, warm, torch)
        out["mxfp4_quantize"] = _rec(ms, st, nbytes, shape=[8192, 8192])
        del xs, qs
        d = W.prefill()
        a = dev_bf16(torch, np, d["a"])
        wq = nv.mxfp4_quantize(dev_bf16(torch, np, d["w"]))
        m = n = k = 8192
        y = torch.empty((m, n), dtype=torch.bfloat16, device="cuda")
        ws = nv.Workspace.get(nv.lib().nvfp4_mxfp4_gemm_workspace_bytes(m, k), a.device)
        ps = max(6, steps // 4)
        ms, st = timed(lambda i: nv.mxfp4_gemm(a, wq, y=y, ws=ws), ps, warm, torch)
        out["mxfp4_prefill"] = _rec(ms, st, None, 2 * m * n * k, "mfma", FP4_MFMA_PEAK_TFLOPS,
                                    shape=[m, n, k],
                                    note="includes the MXFP4 quantization of A inside the call")
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
            nbytes = n * k // 2 + n * k // 32 + m * k * 2 + m * n * 2
            ms, st = timed(lambda i: nv.mxfp4_gemm(a, wqs[i % nw], y=y, ws=ws), steps, warm,
                           torch)
            out[f"mxfp4_decode_m{m}"] = _rec(ms, st, nbytes, 2 * m * n * k, shape=[m, n, k],
                                             note="includes the MXFP4 quantization of A")
        del wqs, wq0

    if not only or "mse" in only:
        # Offline weight quantization with MSE-observer block scales (16x16 tiles) of the decode
        # weight: 18 candidate scales per tile, so it is bound by vector ALU work, not HBM.
        d = W.decode()
        wdev = dev_bf16(torch, np, d["w"])
        q = nv.empty_qtensor(14336, 4096, 16)
        ws = nv.Workspace.get(nv.lib().nvfp4_quantize_workspace_bytes(14336, 4096), wdev.device)
        ms, st = timed(lambda i: nv.quantize_mse(wdev, 16, out=q, ws=ws), max(5, steps // 5),
                       warm, torch)
        vals = 14336 * 4096
        out["mse_quantize_2d"] = _rec(ms, st, bound="alu", shape=[14336, 4096],
                                      gvalues_per_s=vals / (ms * 1e-3) / 1e9,
                                      note="offline; 18 candidate scales per 16x16 tile")
        del wdev, q
    return out


def accuracy(torch, np, nv, W):
    """Error of the formats the library serves on the seeded workloads, computed on the device
    from the library's own outputs: relative Frobenius norms ||Q(x) - x|| / ||x|| of the
    dequantized tensors against their bf16 inputs, and ||Y - Y64|| / ||Y64|| of the products
    against the float64 product of the same bf16 inputs (measurement only, not the path)."""
    def rel(a, b):
        a, b = a.double(), b.double()
        return float(torch.linalg.vector_norm(a - b) / torch.linalg.vector_norm(b))

    out = {"what": "relative Frobenius error against the bf16 inputs (quantize) or against the "
                   "float64 product of the bf16 inputs (products)"}
    x = dev_bf16(torch, np, W.activation(seed=1, rows=8192, cols=8192)["x"])
    out["activation_8192x8192"] = {
        "nvfp4_1d": rel(nv.dequantize(nv.quantize_1d(x)), x),
        "mxfp4": rel(nv.mxfp4_dequantize(nv.mxfp4_quantize(x)), x)}
    del x
    d = W.decode()  # the decode configuration: W, then A for M = 1, 8, 16
    w = dev_bf16(torch, np, d["w"])
    wq2, wq1 = nv.quantize_2d(w), nv.quantize_1d(w)
    wmse, wmx = nv.quantize_mse(w, 16), nv.mxfp4_quantize(w)
    out["decode_weight_14336x4096"] = {
        "nvfp4_2d": rel(nv.dequantize(wq2), w), "nvfp4_2d_mse_observer": rel(nv.dequantize(wmse), w),
        "nvfp4_1d": rel(nv.dequantize(wq1), w), "mxfp4": rel(nv.mxfp4_dequantize(wmx), w)}
    a = dev_bf16(torch, np, d["a"][16])
    y64 = a.double() @ w.double().t()
    out["decode_product_16x14336x4096"] = {
        "w4a4_nvfp4": rel(nv.gemm_w4a4(a, wq2), y64),
        "w4a4_nvfp4_mse_weights": rel(nv.gemm_w4a4(a, wmse), y64),
        "w4a16_nvfp4": rel(nv.gemm_w4a16(a, wq2), y64),
        "w4a4_mxfp4": rel(nv.mxfp4_gemm(a, wmx), y64)}
    del w, wq2, wq1, wmse, wmx, a, y64
    d = W.prefill()
    a, w = dev_bf16(torch, np, d["a"]), dev_bf16(torch, np, d["w"])
    y64 = a.double() @ w.double().t()
    out["prefill_product_8192x8192x8192"] = {
        "w4a4_nvfp4": rel(nv.gemm_w4a4(a, nv.quantize_2d(w)), y64),
        "w4a4_mxfp4": rel(nv.mxfp4_gemm(a, nv.mxfp4_quantize(w)), y64)}
    del a, w, y64
    torch.cuda.empty_cache()
    return out


def host_info():
    """Host cores as the CPU oracle sees them: os.cpu_count(), the affinity mask and the BLAS
    thread pools numpy's matmul uses."""
    import numpy as np
    np.ones((8, 8)) @ np.ones((8, 8))  # make sure the BLAS library is loaded
    info = {"os_cpu_count": os.cpu_count(), "affinity_cpus": len(os.sched_getaffinity(0))}
    try:
        import threadpoolctl
        info["blas"] = [{"api": p.get("internal_api"), "num_threads": p.get("num_threads")}
                        for p in threadpoolctl.threadpool_info() if p.get("user_api") == "blas"]
    except Exception as e:  # threadpoolctl missing or failing: say so
        info["blas"] = f"unknown ({e})"
    return info


def blas_threads(info):
    try:
        return max(p["num_threads"] for p in info["blas"])
    except (TypeError, ValueError, KeyError):
        return None


def cpu_baseline(x_host, nbytes, W, with_gemms=True):
    """The CPU oracle (float64 numpy, test infrastructure), timed on this host as it stands.

    Headline: quantize_1d of the same 8192 x 8192 input (numpy elementwise work: one thread).
    With `with_gemms`, bounded samples of the product configurations, each on the same seeded
    inputs as the GPU run and rated with the GPU rows' algorithmic bytes / flops:
      tiny   quantize A and W, then the float64 product (the whole 32 x 512 x 512 round trip);
      decode quantize A (M = 1, 8, 16), then the float64 product with the 14336 x 4096 weight
             (the weight's quantization is offline on both sides and not timed);
      moe    quantize the 4096 x 2048 tokens, then the float64 products of 16 of the 128
             experts (the first 16: the most-routed ones, 19,479 of the 32,768 rows), rated on
             the flops of those rows.
    The products run in numpy's BLAS with the threads host_info reports."""
    sys.path.insert(0, os.path.dirname(os.path.abspath(__file__)))
    import numpy as np
    from oracle import nvfp4_oracle as O
    info = host_info()
    t0 = time.perf_counter()
    O.quantize_1d(x_host)
    dt = time.perf_counter() - t0
    rec = {"value": nbytes / dt / 1e9, "unit": "GB/s", "cores": 1, "kind": "oracle",
           "sample": "the full 8192 x 8192 activation workload, one quantize_1d call "
                     f"({dt:.1f} s, numpy elementwise on one thread)", "host": info}
    if not with_gemms:
        return rec
    gemms = {}
    bt = blas_threads(info)
    d = W.tiny()
    t0 = time.perf_counter()
    O.gemm64(O.quantize_1d(d["a"]) + (1,), O.quantize_1d(d["w"]) + (1,))
    dt = time.perf_counter() - t0
    gemms["tiny"] = {"s": dt, "gflops": 2 * 32 * 512 * 512 / dt / 1e9, "threads": bt}
    d = W.decode()
    ow = O.quantize_2d(d["w"]) + (16,)
    n, k = 14336, 4096
    for m, a in d["a"].items():
        t0 = time.perf_counter()
        O.gemm64(O.quantize_1d(a) + (1,), ow)
        dt = time.perf_counter() - t0
        nb = n * k // 2 + (n // 16) * (k // 16) + 4 + m * k * 2 + m * n * 2
        gemms[f"decode_m{m}"] = {"s": dt, "gbs": nb / dt / 1e9, "threads": bt}
    del ow, d
    d = W.moe()
    n, e_s = d["n"], 16
    ws = [O.quantize_2d(d["w"][e * n:(e + 1) * n]) + (16,) for e in range(e_s)]  # offline
    off = d["offsets"][:e_s + 1]
    rows = int(off[-1])
    t0 = time.perf_counter()
    oa = O.quantize_1d(d["a"]) + (1,)
    O.grouped_gemm64(oa, d["row_index"][:rows], off, ws)
    dt = time.perf_counter() - t0
    gemms["moe_16_experts"] = {"s": dt, "rows": rows, "gflops": 2 * rows * n * 2048 / dt / 1e9,
                               "threads": bt, "note": "token quantize + the 16 experts' "
                                                      "products; their weight quantization "
                                                      "(offline) not timed"}
    rec["gemms"] = gemms
    return rec


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
        if not only or "accuracy" in only:
            rec["accuracy"] = accuracy(torch, np, nv, W)
    rec["roofline"]["median_gbs"] = h["median_gbs"]
    rec["roofline"]["per_call"] = h["stats"]
    rec["clocks"] = clocks()
    rec["attainable"] = copy_bandwidth(torch)
    if not args.no_cpu:
        rec["cpu_baseline"] = cpu_baseline(h["x_host"], h["bytes"], W, not args.no_extra)
    print(json.dumps(rec), flush=True)


if __name__ == "__main__":
    main()
