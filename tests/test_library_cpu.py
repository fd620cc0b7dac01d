"""CPU-only checks of libnvfp4: the shared library loads, exports every function the public
header declares, and rejects bad arguments before touching the GPU (validation runs before any
HIP call, so these paths need no device)."""

import ctypes
import os
import re

import pytest

from conftest import ROOT

nv = pytest.importorskip("nvfp4_w4a4_quantized_amax_amd.nvfp4",
                         reason="libnvfp4.so not built")
L = nv.lib()
HEADER = os.path.join(ROOT, "include", "nvfp4.h")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(nvfp4_[a-z0-9_]+)\s*\(", text)))


def test_header_functions_are_exported():
    names = declared_functions()
    assert len(names) >= 10
    for n in names:
        assert hasattr(L, n), n
    assert set(names) == set(nv.EXPORTED)


def test_status_strings_and_version():
    for s in range(7):
        assert L.nvfp4_status_string(s).startswith(b"NVFP4_")
    assert b"unknown" in L.nvfp4_status_string(99)
    assert L.nvfp4_version() >= 100


def test_workspace_sizes():
    assert L.nvfp4_quantize_workspace_bytes(8192, 8192) == 8192
    small = L.nvfp4_gemm_workspace_bytes(16, 14336, 4096)
    big = L.nvfp4_gemm_workspace_bytes(8192, 8192, 8192)
    # packed A: codes + scales + global scale after the 4 KiB header
    assert big >= 8192 + 8192 * 4096 + 8192 * 512 + 4
    assert small >= 8192 + 16 * 2048 + 16 * 256 + 4
    assert L.nvfp4_grouped_gemm_workspace_bytes(4096, 2048, 32768, 128) >= 8192 + 4096 * 1024


FAKE = 0x100000  # aligned, never dereferenced: every call below fails validation first


def qt(rows, cols, block_rows=1, ld=None, codes=FAKE, gs=FAKE):
    ld = ld if ld is not None else max((cols // 2 + 15) // 16 * 16, 16)
    return nv.CTensor(codes, ld, FAKE, cols // 16, gs, rows, cols, block_rows, 0)


def q1d(x, rows, cols, ld, out, ws=FAKE, wsb=8192):
    return L.nvfp4_quantize_1d(x, rows, cols, ld, ctypes.byref(out), ws, wsb, None)


def test_quantize_validation():
    t = qt(32, 64)
    assert q1d(None, 32, 64, 64, t) == nv.ERR_NULL
    assert q1d(FAKE, 32, 60, 64, qt(32, 60)) == nv.ERR_SHAPE           # cols % 16
    assert q1d(FAKE, 32, 64, 32, t) == nv.ERR_SHAPE                     # ld < cols
    assert q1d(FAKE + 2, 32, 64, 64, t) == nv.ERR_ALIGN                 # x misaligned
    assert q1d(FAKE, 32, 64, 68, t) == nv.ERR_ALIGN                     # ld % 8
    assert q1d(FAKE, 32, 64, 64, qt(31, 64)) == nv.ERR_SHAPE            # out shape mismatch
    assert q1d(FAKE, 32, 64, 64, qt(32, 64, codes=None)) == nv.ERR_NULL
    assert q1d(FAKE, 32, 64, 64, qt(32, 64, codes=FAKE + 4)) == nv.ERR_ALIGN
    assert q1d(FAKE, 32, 64, 64, qt(32, 64, ld=40)) == nv.ERR_ALIGN     # ld_codes % 16
    assert q1d(FAKE, 32, 64, 64, qt(32, 64, block_rows=16)) == nv.ERR_UNSUPPORTED
    assert q1d(FAKE, 32, 64, 64, qt(32, 64, block_rows=3)) == nv.ERR_UNSUPPORTED
    assert q1d(FAKE, 32, 64, 64, t, ws=None) == nv.ERR_WORKSPACE
    assert q1d(FAKE, 32, 64, 64, t, wsb=100) == nv.ERR_WORKSPACE
    assert q1d(FAKE, 32, 64, 64, t, ws=FAKE + 16) == nv.ERR_WORKSPACE  # ws alignment
    bad = qt(32, 64)
    bad.reserved = 1
    assert q1d(FAKE, 32, 64, 64, bad) == nv.ERR_UNSUPPORTED
    # 2D needs rows % 16 and block_rows 16
    assert L.nvfp4_quantize_2d(FAKE, 24, 64, 64, ctypes.byref(qt(24, 64, 16)), FAKE, 8192,
                               None) == nv.ERR_SHAPE
    assert L.nvfp4_quantize_2d(FAKE, 32, 64, 64, ctypes.byref(qt(32, 64, 1)), FAKE, 8192,
                               None) == nv.ERR_UNSUPPORTED


def test_dequantize_validation():
    t = qt(32, 64)
    assert L.nvfp4_dequantize(None, FAKE, 64, 0, None) == nv.ERR_NULL
    assert L.nvfp4_dequantize(ctypes.byref(t), None, 64, 0, None) == nv.ERR_NULL
    assert L.nvfp4_dequantize(ctypes.byref(t), FAKE, 32, 0, None) == nv.ERR_SHAPE
    assert L.nvfp4_dequantize(ctypes.byref(t), FAKE, 64, 7, None) == nv.ERR_UNSUPPORTED
    assert L.nvfp4_dequantize(ctypes.byref(t), FAKE + 8, 64, 0, None) == nv.ERR_ALIGN


def gemm(a, m, k, ld_a, aq, w, y=FAKE, ld_y=None, ws=FAKE, wsb=1 << 40):
    ld_y = ld_y if ld_y is not None else (w.rows if w is not None else 128)
    return L.nvfp4_gemm_w4a4(a, m, k, ld_a, ctypes.byref(aq) if aq is not None else None,
                             ctypes.byref(w) if w is not None else None, y, ld_y, ws, wsb, None)


def test_gemm_validation():
    w = qt(128, 256, 16)
    assert gemm(FAKE, 64, 256, 256, None, None) == nv.ERR_NULL
    assert gemm(FAKE, 64, 256, 256, None, w, y=None) == nv.ERR_NULL
    assert gemm(None, 64, 256, 256, None, w) == nv.ERR_NULL              # no A at all
    assert gemm(FAKE, 64, 240, 240, None, w) == nv.ERR_SHAPE             # K mismatch
    assert gemm(FAKE, 64, 250, 256, None, qt(128, 250, 1)) == nv.ERR_SHAPE
    assert gemm(FAKE, 64, 256, 256, None, w, ld_y=100) == nv.ERR_SHAPE
    assert gemm(FAKE, 64, 256, 256, None, w, y=FAKE + 1) == nv.ERR_ALIGN
    assert gemm(FAKE, 64, 256, 256, qt(64, 256, 16), w) == nv.ERR_UNSUPPORTED
    assert gemm(None, 64, 256, 0, qt(64, 256, 16), w) == nv.ERR_UNSUPPORTED
    assert gemm(None, 64, 256, 0, qt(60, 256), w) == nv.ERR_SHAPE
    assert gemm(FAKE, 64, 256, 256, None, w, ws=None) == nv.ERR_WORKSPACE
    assert gemm(FAKE, 64, 256, 256, None, w, wsb=8192) == nv.ERR_WORKSPACE
    assert gemm(FAKE + 8, 64, 256, 256, None, w) == nv.ERR_ALIGN


def w4a16(a, m, k, w, ld_a=None, y=FAKE, ld_y=None):
    return L.nvfp4_gemm_w4a16(a, m, k, k if ld_a is None else ld_a,
                              ctypes.byref(w) if w is not None else None, y,
                              (w.rows if w is not None else 0) if ld_y is None else ld_y, None)


def test_w4a16_validation():
    w = qt(128, 256, 16)
    assert w4a16(FAKE, 8, 256, None) == nv.ERR_NULL
    assert w4a16(None, 8, 256, w) == nv.ERR_NULL
    assert w4a16(FAKE, 8, 256, w, y=None) == nv.ERR_NULL
    assert w4a16(FAKE, 8, 240, w) == nv.ERR_SHAPE                 # K mismatch
    assert w4a16(FAKE, 8, 250, qt(128, 250, 1)) == nv.ERR_SHAPE   # K % 16
    assert w4a16(FAKE, 8, 256, w, ld_y=100) == nv.ERR_SHAPE
    assert w4a16(FAKE, 8, 256, w, ld_a=100) == nv.ERR_SHAPE        # ld_a < k
    assert w4a16(FAKE, 8, 256, w, y=FAKE + 2) == nv.ERR_ALIGN
    assert w4a16(FAKE + 8, 8, 256, w) == nv.ERR_ALIGN              # A not 16-byte aligned
    assert w4a16(FAKE, 8, 256, w, ld_a=260) == nv.ERR_ALIGN        # ld_a % 8
    assert w4a16(FAKE, 17, 256, w) == nv.ERR_UNSUPPORTED           # decode shapes only
    assert w4a16(FAKE, -1, 256, w) == nv.ERR_SHAPE
    assert w4a16(None, 0, 256, w, y=None) == nv.OK                 # empty: nothing to do


def grouped(a, tokens, k, aq, ri, total, off, g, w, n, y=FAKE, ws=FAKE, wsb=1 << 40):
    return L.nvfp4_grouped_gemm_w4a4(a, tokens, k, k, ctypes.byref(aq) if aq else None, ri,
                                     total, off, g, ctypes.byref(w), n, y, n, ws, wsb, None)


def test_grouped_validation():
    w = qt(8 * 64, 128, 16)
    assert grouped(FAKE, 32, 128, None, FAKE, 64, None, 8, w, 64) == nv.ERR_NULL
    assert grouped(FAKE, 32, 128, None, FAKE, 64, FAKE, 0, w, 64) == nv.ERR_SHAPE
    assert grouped(FAKE, 32, 128, None, FAKE, 64, FAKE, 4096, w, 64) == nv.ERR_UNSUPPORTED
    assert grouped(FAKE, 32, 128, None, FAKE, 64, FAKE, 7, w, 64) == nv.ERR_SHAPE   # rows != 7*64
    assert grouped(FAKE, 32, 128, None, None, 64, FAKE, 8, w, 64) == nv.ERR_SHAPE   # no index
    assert grouped(FAKE, 32, 128, None, FAKE, 64, FAKE, 8, qt(8 * 40, 128, 16), 40) == \
        nv.ERR_SHAPE                                                               # n % 16
    assert grouped(FAKE, 32, 128, None, FAKE, 64, FAKE, 8, w, 64, ws=None) == nv.ERR_WORKSPACE


def mxt(rows, cols, ld=None, codes=FAKE, lds=None):
    ld = ld if ld is not None else max((cols // 2 + 15) // 16 * 16, 16)
    return nv.CMxTensor(codes, ld, FAKE, cols // 32 if lds is None else lds, rows, cols)


def test_mxfp4_validation():
    q = mxt(64, 256)
    Q = L.nvfp4_mxfp4_quantize
    assert Q(FAKE, 64, 256, 256, None, None) == nv.ERR_NULL
    assert Q(None, 64, 256, 256, ctypes.byref(q), None) == nv.ERR_NULL
    assert Q(FAKE, 64, 240, 240, ctypes.byref(mxt(64, 240)), None) == nv.ERR_SHAPE   # cols % 32
    assert Q(FAKE, 64, 256, 256, ctypes.byref(mxt(64, 288)), None) == nv.ERR_SHAPE   # cols mismatch
    assert Q(FAKE, 64, 256, 256, ctypes.byref(mxt(64, 256, ld=136)), None) == nv.ERR_ALIGN
    assert Q(FAKE, 64, 256, 256, ctypes.byref(mxt(64, 256, lds=4)), None) == nv.ERR_SHAPE
    assert Q(FAKE, 64, 256, 256, ctypes.byref(mxt(64, 256, codes=FAKE + 4)), None) == nv.ERR_ALIGN
    assert Q(FAKE + 2, 64, 256, 256, ctypes.byref(q), None) == nv.ERR_ALIGN
    D = L.nvfp4_mxfp4_dequantize
    assert D(ctypes.byref(q), None, 256, nv.OUT_F32, None) == nv.ERR_NULL
    assert D(ctypes.byref(q), FAKE, 256, 7, None) == nv.ERR_UNSUPPORTED
    assert D(ctypes.byref(q), FAKE, 128, nv.OUT_F32, None) == nv.ERR_SHAPE
    G = L.nvfp4_mxfp4_gemm
    w = mxt(128, 256)
    assert G(FAKE, 8, 256, 256, None, None, FAKE, 128, FAKE, 1 << 30, None) == nv.ERR_NULL
    assert G(FAKE, 8, 240, 240, None, ctypes.byref(w), FAKE, 128, FAKE, 1 << 30, None) == \
        nv.ERR_SHAPE                                                          # k % 32
    assert G(FAKE, 8, 224, 224, None, ctypes.byref(w), FAKE, 128, FAKE, 1 << 30, None) == \
        nv.ERR_SHAPE                                                          # K mismatch
    assert G(FAKE, 8, 256, 256, None, ctypes.byref(w), FAKE, 100, FAKE, 1 << 30, None) == \
        nv.ERR_SHAPE                                                          # ld_y < n
    assert G(FAKE, 8, 256, 256, None, ctypes.byref(w), FAKE, 128, None, 0, None) == \
        nv.ERR_WORKSPACE                                                      # A quantized inside
    assert G(None, 8, 256, 0, None, ctypes.byref(w), FAKE, 128, None, 0, None) == nv.ERR_NULL
    assert L.nvfp4_mxfp4_gemm_workspace_bytes(8, 256) >= 8 * 128 + 8 * 8
    # empty problems
    assert G(None, 0, 256, 0, None, ctypes.byref(w), None, 128, None, 0, None) == nv.OK
    assert Q(None, 0, 256, 256, ctypes.byref(mxt(0, 256)), None) == nv.OK


def test_empty_problems_need_no_buffers():
    """Zero rows: nothing is computed or written, NVFP4_OK is returned and the data pointers
    may be NULL (no GPU work is launched, so this runs without a device)."""
    def empty(rows, cols, br):
        return nv.CTensor(None, cols // 2, None, cols // 16, None, rows, cols, br, 0)
    q1, q2 = empty(0, 64, 1), empty(0, 64, 16)
    assert L.nvfp4_quantize_1d(None, 0, 64, 64, ctypes.byref(q1), None, 0, None) == nv.OK
    assert L.nvfp4_quantize_2d(None, 0, 64, 64, ctypes.byref(q2), None, 0, None) == nv.OK
    assert L.nvfp4_dequantize(ctypes.byref(q1), None, 64, nv.OUT_F32, None) == nv.OK
    w = empty(32, 64, 16)
    assert L.nvfp4_gemm_w4a4(None, 0, 64, 64, None, ctypes.byref(w), None, 32, None, 0,
                             None) == nv.OK
    assert L.nvfp4_grouped_gemm_w4a4(None, 4, 64, 64, None, None, 0, None, 2, ctypes.byref(w),
                                     16, None, 16, None, 0, None) == nv.OK
    # but bad sizes are still rejected, and rows to fill without tokens is an error
    assert L.nvfp4_quantize_1d(None, 0, 40, 64, ctypes.byref(q1), None, 0, None) != nv.OK
    assert L.nvfp4_grouped_gemm_w4a4(None, 0, 64, 64, None, None, 5, None, 2, ctypes.byref(w),
                                     16, None, 16, None, 0, None) == nv.ERR_SHAPE


def test_noalloc_validation():
    """The allocation-free product refuses, before touching a device, shapes whose workspace
    would exceed its fixed scratch, and the usual bad arguments."""
    w = qt(1024, 8192, 16)
    f = L.nvfp4_gemm_w4a4_noalloc
    assert f(FAKE, 16, 8192, 8192, None, None, FAKE, 1024, None) == nv.ERR_NULL
    assert f(FAKE, 16, 8200, 8200, None, ctypes.byref(w), FAKE, 1024, None) == nv.ERR_SHAPE
    assert f(FAKE, -1, 8192, 8192, None, ctypes.byref(w), FAKE, 1024, None) == nv.ERR_SHAPE
    assert f(FAKE, 0, 8192, 8192, None, ctypes.byref(w), FAKE, 1024, None) == nv.OK
    assert L.nvfp4_gemm_workspace_bytes(16384, 1024, 8192) > nv.NOALLOC_SCRATCH_BYTES
    assert f(FAKE, 16384, 8192, 8192, None, ctypes.byref(w), FAKE, 1024,
             None) == nv.ERR_WORKSPACE


def test_sizes_below_two_to_the_31():
    """Every size and leading dimension must lie below 2^31: larger ones are refused before any
    size arithmetic, and the workspace queries answer SIZE_MAX for them instead of a wrapped
    product (the same edges run under the sanitizers in test_host_sanitizers)."""
    size_max = 2 ** 64 - 1
    big = 1 << 31
    assert L.nvfp4_gemm_workspace_bytes(big, 4096, 4096) == size_max
    assert L.nvfp4_gemm_workspace_bytes(64, 4096, big) == size_max
    assert L.nvfp4_gemm_workspace_bytes(64, big, 4096) == size_max
    assert L.nvfp4_grouped_gemm_workspace_bytes(big, 4096, 64, 8) == size_max
    assert L.nvfp4_mxfp4_gemm_workspace_bytes(64, big) == size_max
    assert L.nvfp4_gemm_workspace_bytes(big - 1, 16, 4096) < size_max
    assert q1d(FAKE, big, 64, 64, qt(big, 64)) == nv.ERR_SHAPE
    assert q1d(FAKE, 32, 64, big, qt(32, 64)) == nv.ERR_SHAPE
    assert L.nvfp4_dequantize(ctypes.byref(qt(32, 64)), FAKE, big, 0, None) == nv.ERR_SHAPE
    w = qt(128, 256, 16)
    assert gemm(FAKE, 64, 256, 256, None, w, ld_y=big) == nv.ERR_SHAPE
    assert grouped(FAKE, 32, 128, None, FAKE, 64, FAKE, 8, qt(8 * 64, 128, 16), big) == \
        nv.ERR_SHAPE
