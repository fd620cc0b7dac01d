"""Build libnvfp4.so in-tree for gfx950 with hipcc (cross-compiles without a GPU).

    python -m nvfp4_w4a4_quantized_amax_amd.build [-v]
"""

import concurrent.futures
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
BUILD_DIR = os.path.join(HERE, "_build")
LIB_PATH = os.path.join(HERE, "libnvfp4.so")
SOURCES = ["quantize.hip", "dequantize.hip", "gemm.hip", "mxfp4.hip", "mse.hip", "api.hip",
           "noalloc.hip"]

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"
FLAGS = [
    "-O3", "-std=c++17", f"--offload-arch={ARCH}", "-fPIC", "-ffp-contract=off",
    # packed fp32 VALU forms are not used by this library
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function",
]


def _compile(src, verbose):
    obj = os.path.join(BUILD_DIR, os.path.splitext(src)[0] + ".o")
    cmd = [HIPCC, *FLAGS, "-c", os.path.join(CSRC, src), "-o", obj]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    msgs = "\n".join(l for l in (r.stdout + r.stderr).splitlines()
                     if "packed-fp32-ops" not in l)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{msgs}")
    if verbose and msgs.strip():
        print(msgs)
    return obj


PROBES = [("probes/mfma_routes.hip", "probes/mfma_routes"),
          ("probes/hbm_rates.hip", "probes/hbm_rates"),
          ("probes/launch_cost.hip", "probes/launch_cost"),
          ("probes/decode_stream.hip", "probes/decode_stream")]


def build_probes(verbose=False):
    """Measurement programs beside the library (not linked into it): built as executables."""
    outs = []
    for src, exe in PROBES:
        out = os.path.join(HERE, exe)
        cmd = [HIPCC, *[f for f in FLAGS if f not in ("-fPIC",)], os.path.join(HERE, src), "-o", out]
        if verbose:
            print(" ".join(cmd), flush=True)
        r = subprocess.run(cmd, capture_output=True, text=True)
        if r.returncode != 0:
            raise RuntimeError(f"hipcc failed on {src}:\n{r.stdout}{r.stderr}")
        outs.append(out)
    return outs


def build(verbose=False):
    os.makedirs(BUILD_DIR, exist_ok=True)
    with concurrent.futures.ThreadPoolExecutor(max_workers=4) as ex:
        objs = list(ex.map(lambda s: _compile(s, verbose), SOURCES))
    tmp = LIB_PATH + ".tmp"
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("link failed:\n" + r.stdout + r.stderr)
    os.replace(tmp, LIB_PATH)
    build_probes(verbose)
    return LIB_PATH


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
