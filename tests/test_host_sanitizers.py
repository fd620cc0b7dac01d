"""The library's host code under AddressSanitizer and UndefinedBehaviorSanitizer (CPU only).

Every source of libnvfp4 is compiled with the sanitizers on its host side only (the device code
is built as usual and never runs here) and linked with tests/host_checks.cpp, a C program that
drives each C-ABI entry point's validation with ordinary mistakes and with sizes at the edges of
int64_t.  Those calls all return before any HIP call, so no GPU is needed.  A signed overflow in
a size computation, an out-of-bounds read or any other undefined behaviour stops the program with
the sanitizer's report, and the test fails with it.
"""

import concurrent.futures
import os
import shutil
import subprocess

import pytest

from conftest import ROOT
from nvfp4_w4a4_quantized_amax_amd import build as B

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
# Sanitizers on the host pass only: each flag goes through -Xarch_host.
SAN = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
       "-Xarch_host", "-fno-sanitize-recover=undefined"]
FLAGS = ["--offload-arch=gfx950", "-O1", "-g", "-std=c++17", "-fPIC", "-fno-omit-frame-pointer",
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops", *SAN]


def _run(cmd):
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        msgs = "\n".join(l for l in (r.stdout + r.stderr).splitlines() if "packed-fp32" not in l)
        raise RuntimeError(f"{' '.join(cmd)}\n{msgs}")


@pytest.mark.timeout(600)
@pytest.mark.skipif(not shutil.which(HIPCC) and not os.path.exists(HIPCC), reason="no hipcc")
def test_host_code_under_asan_and_ubsan(tmp_path):
    jobs = [[HIPCC, *FLAGS, "-c", os.path.join(B.CSRC, s), "-o", str(tmp_path / (s + ".o"))]
            for s in B.SOURCES]
    jobs.append([HIPCC, *FLAGS, "-I", os.path.join(ROOT, "include"), "-x", "c++",
                 os.path.join(ROOT, "tests", "host_checks.cpp"), "-c", "-o",
                 str(tmp_path / "host_checks.o")])
    with concurrent.futures.ThreadPoolExecutor(max_workers=4) as ex:
        list(ex.map(_run, jobs))
    exe = str(tmp_path / "host_checks")
    objs = sorted(str(p) for p in tmp_path.glob("*.o"))
    _run([HIPCC, "--offload-arch=gfx950", *SAN, *objs, "-o", exe])
    env = dict(os.environ)
    # Leak reports would come from the HIP runtime's own process-lifetime state, not from the
    # library's validation; everything else stops the program.
    env["ASAN_OPTIONS"] = "detect_leaks=0:abort_on_error=0:exitcode=86"
    env["UBSAN_OPTIONS"] = "print_stacktrace=1:halt_on_error=1:exitcode=87"
    r = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=120)
    out = r.stdout + r.stderr
    assert r.returncode == 0, out
    assert "host checks passed" in r.stdout, out
    assert "runtime error" not in out and "AddressSanitizer" not in out, out
