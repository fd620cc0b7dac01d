"""Thin Python binding of libnvfp4 (include/nvfp4.h): argument marshalling only.

Every step of the computation runs in the library's HIP kernels; PyTorch provides device
memory and the current stream.  Importing this module loads libnvfp4.so and raises if it has not
been built (`python -m nvfp4_w4a4_quantized_amax_amd.build`); there is no fallback.
"""

import ctypes
import os
from dataclasses import dataclass

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libnvfp4.so")

if not os.path.exists(LIB_PATH):
    raise ImportError(f"libnvfp4 is not built ({LIB_PATH} missing); run "
                      "`python -m nvfp4_w4a4_quantized_amax_amd.build` first")
_lib = ctypes.CDLL(LIB_PATH)

OK, ERR_NULL, ERR_SHAPE, ERR_ALIGN, ERR_WORKSPACE, ERR_HIP, ERR_UNSUPPORTED = range(7)
OUT_BF16, OUT_F32 = 0, 1

EXPORTED = (
    "nvfp4_status_string", "nvfp4_version", "nvfp4_quantize_workspace_bytes",
    "nvfp4_gemm_workspace_bytes", "nvfp4_grouped_gemm_workspace_bytes", "nvfp4_quantize_1d",
    "nvfp4_quantize_2d", "nvfp4_dequantize", "nvfp4_gemm_w4a4", "nvfp4_grouped_gemm_w4a4",
    "nvfp4_gemm_w4a16", "nvfp4_mxfp4_quantize", "nvfp4_mxfp4_dequantize",
    "nvfp4_mxfp4_gemm_workspace_bytes", "nvfp4_mxfp4_gemm", "nvfp4_quantize_mse",
    "nvfp4_gemm_w4a4_noalloc",
)


class CTensor(ctypes.Structure):
    """Mirror of `nvfp4_tensor`."""
    _fields_ = [("codes", ctypes.c_void_p), ("ld_codes", ctypes.c_int64),
                ("scales", ctypes.c_void_p), ("ld_scales", ctypes.c_int64),
                ("global_scale", ctypes.c_void_p), ("rows", ctypes.c_int64),
                ("cols", ctypes.c_int64), ("block_rows", ctypes.c_int32),
                ("reserved", ctypes.c_int32)]


class CMxTensor(ctypes.Structure):
    """Mirror of `mxfp4_tensor`."""
    _fields_ = [("codes", ctypes.c_void_p), ("ld_codes", ctypes.c_int64),
                ("scales", ctypes.c_void_p), ("ld_scales", ctypes.c_int64),
                ("rows", ctypes.c_int64), ("cols", ctypes.c_int64)]


_i64, _i32, _vp, _sz = ctypes.c_int64, ctypes.c_int32, ctypes.c_void_p, ctypes.c_size_t
_pt = ctypes.POINTER(CTensor)
_pmx = ctypes.POINTER(CMxTensor)

_lib.nvfp4_status_string.restype = ctypes.c_char_p
_lib.nvfp4_status_string.argtypes = [ctypes.c_int]
_lib.nvfp4_version.restype = ctypes.c_int
_lib.nvfp4_quantize_workspace_bytes.restype = _sz
_lib.nvfp4_quantize_workspace_bytes.argtypes = [_i64, _i64]
_lib.nvfp4_gemm_workspace_bytes.restype = _sz
_lib.nvfp4_gemm_workspace_bytes.argtypes = [_i64, _i64, _i64]
_lib.nvfp4_grouped_gemm_workspace_bytes.restype = _sz
_lib.nvfp4_grouped_gemm_workspace_bytes.argtypes = [_i64, _i64, _i64, _i32]
for _name in ("nvfp4_quantize_1d", "nvfp4_quantize_2d"):
    getattr(_lib, _name).restype = ctypes.c_int
    getattr(_lib, _name).argtypes = [_vp, _i64, _i64, _i64, _pt, _vp, _sz, _vp]
_lib.nvfp4_quantize_mse.restype = ctypes.c_int
_lib.nvfp4_quantize_mse.argtypes = [_vp, _i64, _i64, _i64, _pt, _vp, _sz, _vp]
_lib.nvfp4_dequantize.restype = ctypes.c_int
_lib.nvfp4_dequantize.argtypes = [_pt, _vp, _i64, ctypes.c_int, _vp]
_lib.nvfp4_gemm_w4a4.restype = ctypes.c_int
_lib.nvfp4_gemm_w4a4.argtypes = [_vp, _i64, _i64, _i64, _pt, _pt, _vp, _i64, _vp, _sz, _vp]
_lib.nvfp4_gemm_w4a4_noalloc.restype = ctypes.c_int
_lib.nvfp4_gemm_w4a4_noalloc.argtypes = [_vp, _i64, _i64, _i64, _pt, _pt, _vp, _i64, _vp]
NOALLOC_SCRATCH_BYTES = 64 * 1024 * 1024
_lib.nvfp4_gemm_w4a16.restype = ctypes.c_int
_lib.nvfp4_gemm_w4a16.argtypes = [_vp, _i64, _i64, _i64, _pt, _vp, _i64, _vp]
_lib.nvfp4_mxfp4_quantize.restype = ctypes.c_int
_lib.nvfp4_mxfp4_quantize.argtypes = [_vp, _i64, _i64, _i64, _pmx, _vp]
_lib.nvfp4_mxfp4_dequantize.restype = ctypes.c_int
_lib.nvfp4_mxfp4_dequantize.argtypes = [_pmx, _vp, _i64, ctypes.c_int, _vp]
_lib.nvfp4_mxfp4_gemm_workspace_bytes.restype = _sz
_lib.nvfp4_mxfp4_gemm_workspace_bytes.argtypes = [_i64, _i64]
_lib.nvfp4_mxfp4_gemm.restype = ctypes.c_int
_lib.nvfp4_mxfp4_gemm.argtypes = [_vp, _i64, _i64, _i64, _pmx, _pmx, _vp, _i64, _vp, _sz, _vp]
_lib.nvfp4_grouped_gemm_w4a4.restype = ctypes.c_int
_lib.nvfp4_grouped_gemm_w4a4.argtypes = [_vp, _i64, _i64, _i64, _pt, _vp, _i64, _vp, _i32, _pt,
                                         _i64, _vp, _i64, _vp, _sz, _vp]


def lib():
    return _lib


class Nvfp4Error(RuntimeError):
    def __init__(self, status, where):
        self.status = status
        super().__init__(f"{where}: {_lib.nvfp4_status_string(status).decode()}")


def _check(status, where):
    if status != OK:
        raise Nvfp4Error(status, where)


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(device):
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def _round_up(v, a):
    return (v + a - 1) // a * a


@dataclass
class QTensor:
    """An NVFP4 matrix in device memory: packed codes (rows x ld_codes bytes, ld_codes >=
    cols/2), E4M3 scales (rows x cols/16 for 1D blocks, rows/16 x cols/16 for 16x16 tiles) and
    the FP32 global scale(s)."""
    codes: torch.Tensor
    scales: torch.Tensor
    global_scale: torch.Tensor
    rows: int
    cols: int
    block_rows: int

    def c(self):
        return CTensor(self.codes.data_ptr(), self.codes.stride(0), self.scales.data_ptr(),
                       self.scales.stride(0), self.global_scale.data_ptr(), self.rows, self.cols,
                       self.block_rows, 0)

    def packed_codes(self):
        """Codes without row padding (rows x cols/2)."""
        return self.codes[:, : self.cols // 2]


def empty_qtensor(rows, cols, block_rows=1, device="cuda", n_global_scales=1):
    ld = max(_round_up(cols // 2, 16), 16)
    codes = torch.empty((rows, ld), dtype=torch.uint8, device=device)
    srows = rows if block_rows == 1 else rows // 16
    scales = torch.empty((srows, cols // 16), dtype=torch.uint8, device=device)
    gs = torch.empty((n_global_scales,), dtype=torch.float32, device=device)
    return QTensor(codes, scales, gs, rows, cols, block_rows)


class Workspace:
    """Device scratch for the library calls, grown on demand (one per device; calls on one
    device share it, so they must be ordered on one stream)."""
    _bufs = {}

    @classmethod
    def get(cls, nbytes, device):
        dev = torch.device(device)
        key = (dev.type, dev.index if dev.index is not None else torch.cuda.current_device())
        buf = cls._bufs.get(key)
        if buf is None or buf.numel() < nbytes:
            buf = torch.zeros(max(nbytes, 4096), dtype=torch.uint8, device=dev)
            cls._bufs[key] = buf
        return buf


def _ws(nbytes, device, ws):
    if ws is None:
        ws = Workspace.get(nbytes, device)
    return ws


def quantize_1d(x, out=None, ws=None):
    """Dynamic NVFP4 quantization of a bf16 matrix with 16-element blocks along rows."""
    assert x.dtype == torch.bfloat16 and x.dim() == 2 and x.stride(1) == 1
    rows, cols = x.shape
    if out is None:
        out = empty_qtensor(rows, cols, 1, x.device)
    ws = _ws(_lib.nvfp4_quantize_workspace_bytes(rows, cols), x.device, ws)
    ct = out.c()
    _check(_lib.nvfp4_quantize_1d(_ptr(x), rows, cols, x.stride(0), ctypes.byref(ct), _ptr(ws),
                                  ws.numel(), _stream(x.device)), "nvfp4_quantize_1d")
    return out


def quantize_2d(w, out=None, ws=None):
    """NVFP4 quantization of a bf16 weight matrix with one scale per 16x16 tile."""
    assert w.dtype == torch.bfloat16 and w.dim() == 2 and w.stride(1) == 1
    rows, cols = w.shape
    if out is None:
        out = empty_qtensor(rows, cols, 16, w.device)
    ws = _ws(_lib.nvfp4_quantize_workspace_bytes(rows, cols), w.device, ws)
    ct = out.c()
    _check(_lib.nvfp4_quantize_2d(_ptr(w), rows, cols, w.stride(0), ctypes.byref(ct), _ptr(ws),
                                  ws.numel(), _stream(w.device)), "nvfp4_quantize_2d")
    return out


def quantize_mse(w, block_rows=16, out=None, ws=None):
    """Offline NVFP4 weight quantization with MSE-observer block scales (1D blocks or 16x16
    tiles); the result is an ordinary QTensor."""
    assert w.dtype == torch.bfloat16 and w.dim() == 2 and w.stride(1) == 1
    rows, cols = w.shape
    if out is None:
        out = empty_qtensor(rows, cols, block_rows, w.device)
    ws = _ws(_lib.nvfp4_quantize_workspace_bytes(rows, cols), w.device, ws)
    ct = out.c()
    _check(_lib.nvfp4_quantize_mse(_ptr(w), rows, cols, w.stride(0), ctypes.byref(ct), _ptr(ws),
                                   ws.numel(), _stream(w.device)), "nvfp4_quantize_mse")
    return out


def dequantize(q, dtype=torch.float32, out=None):
    """code value x block scale x global scale, as float32 or bf16."""
    if out is None:
        out = torch.empty((q.rows, q.cols), dtype=dtype, device=q.codes.device)
    ct = q.c()
    code = OUT_F32 if dtype == torch.float32 else OUT_BF16
    _check(_lib.nvfp4_dequantize(ctypes.byref(ct), _ptr(out), out.stride(0), code,
                                 _stream(q.codes.device)), "nvfp4_dequantize")
    return out


def gemm_w4a4(a, w, y=None, a_q=None, ws=None):
    """Y = A . W^T (bf16 out).  `a` is a bf16 matrix (quantized inside the call; `a_q`, if given,
    receives the quantized A) or a QTensor with 1D blocks."""
    if isinstance(a, QTensor):
        m, k = a.rows, a.cols
        a_bf16, a_q = None, a
        dev = a.codes.device
    else:
        assert a.dtype == torch.bfloat16 and a.dim() == 2 and a.stride(1) == 1
        m, k = a.shape
        a_bf16, dev = a, a.device
    n = w.rows
    if y is None:
        y = torch.empty((m, n), dtype=torch.bfloat16, device=dev)
    ws = _ws(_lib.nvfp4_gemm_workspace_bytes(m, n, k), dev, ws)
    wc = w.c()
    ac = a_q.c() if a_q is not None else None
    _check(_lib.nvfp4_gemm_w4a4(_ptr(a_bf16), m, k, a_bf16.stride(0) if a_bf16 is not None else 0,
                                ctypes.byref(ac) if ac is not None else None, ctypes.byref(wc),
                                _ptr(y), y.stride(0), _ptr(ws), ws.numel(), _stream(dev)),
           "nvfp4_gemm_w4a4")
    return y


def gemm_w4a4_noalloc(a, w, y, a_q=None):
    """gemm_w4a4 with the library's own scratch instead of a workspace (nothing is allocated;
    `y` must be given).  Calls that overlap on one GPU race on that scratch."""
    if isinstance(a, QTensor):
        m, k = a.rows, a.cols
        a_bf16, a_q = None, a
        dev = a.codes.device
    else:
        assert a.dtype == torch.bfloat16 and a.dim() == 2 and a.stride(1) == 1
        m, k = a.shape
        a_bf16, dev = a, a.device
    wc = w.c()
    ac = a_q.c() if a_q is not None else None
    _check(_lib.nvfp4_gemm_w4a4_noalloc(
        _ptr(a_bf16), m, k, a_bf16.stride(0) if a_bf16 is not None else 0,
        ctypes.byref(ac) if ac is not None else None, ctypes.byref(wc), _ptr(y), y.stride(0),
        _stream(dev)), "nvfp4_gemm_w4a4_noalloc")
    return y


def gemm_w4a16(a, w, y=None):
    """Weight-only Y = A . W^T (bf16 out): `a` is a bf16 matrix of at most 16 rows, used as is;
    `w` a quantized weight."""
    assert a.dtype == torch.bfloat16 and a.dim() == 2 and a.stride(1) == 1
    m, k = a.shape
    n = w.rows
    if y is None:
        y = torch.empty((m, n), dtype=torch.bfloat16, device=a.device)
    wc = w.c()
    _check(_lib.nvfp4_gemm_w4a16(_ptr(a), m, k, a.stride(0), ctypes.byref(wc), _ptr(y),
                                 y.stride(0), _stream(a.device)), "nvfp4_gemm_w4a16")
    return y


def grouped_gemm_w4a4(a, row_index, offsets, w, n, total_rows, y=None, a_q=None, ws=None):
    """Grouped (MoE) W4A4 product.  `w` stacks all experts (num_groups * n rows) with one global
    scale per expert; `offsets` (int32, num_groups + 1) and `row_index` (int32, total_rows, or
    None) live on the device."""
    if isinstance(a, QTensor):
        tokens, k = a.rows, a.cols
        a_bf16, a_q = None, a
        dev = a.codes.device
    else:
        assert a.dtype == torch.bfloat16 and a.dim() == 2 and a.stride(1) == 1
        tokens, k = a.shape
        a_bf16, dev = a, a.device
    num_groups = offsets.numel() - 1
    if y is None:
        y = torch.empty((total_rows, n), dtype=torch.bfloat16, device=dev)
    ws = _ws(_lib.nvfp4_grouped_gemm_workspace_bytes(tokens, k, total_rows, num_groups), dev, ws)
    wc = w.c()
    ac = a_q.c() if a_q is not None else None
    _check(_lib.nvfp4_grouped_gemm_w4a4(
        _ptr(a_bf16), tokens, k, a_bf16.stride(0) if a_bf16 is not None else 0,
        ctypes.byref(ac) if ac is not None else None, _ptr(row_index), total_rows, _ptr(offsets),
        num_groups, ctypes.byref(wc), n, _ptr(y), y.stride(0), _ptr(ws), ws.numel(),
        _stream(dev)), "nvfp4_grouped_gemm_w4a4")
    return y


# ---------------------------------------------------------------------------------------------
# MXFP4
# ---------------------------------------------------------------------------------------------
@dataclass
class MxTensor:
    """An MXFP4 matrix in device memory: packed codes (rows x ld_codes bytes) and one E8M0
    scale byte per 32 values (rows x ld_scales bytes)."""
    codes: torch.Tensor
    scales: torch.Tensor
    rows: int
    cols: int

    def c(self):
        return CMxTensor(self.codes.data_ptr(), self.codes.stride(0), self.scales.data_ptr(),
                         self.scales.stride(0), self.rows, self.cols)

    def packed_codes(self):
        return self.codes[:, : self.cols // 2]

    def packed_scales(self):
        return self.scales[:, : self.cols // 32]


def empty_mxtensor(rows, cols, device="cuda"):
    codes = torch.empty((rows, max(_round_up(cols // 2, 16), 16)), dtype=torch.uint8,
                        device=device)
    scales = torch.empty((rows, max(_round_up(cols // 32, 4), 4)), dtype=torch.uint8,
                         device=device)
    return MxTensor(codes, scales, rows, cols)


def mxfp4_quantize(x, out=None):
    """MXFP4 quantization of a bf16 matrix: one E8M0 scale per 32 values along rows."""
    assert x.dtype == torch.bfloat16 and x.dim() == 2 and x.stride(1) == 1
    rows, cols = x.shape
    if out is None:
        out = empty_mxtensor(rows, cols, x.device)
    ct = out.c()
    _check(_lib.nvfp4_mxfp4_quantize(_ptr(x), rows, cols, x.stride(0), ctypes.byref(ct),
                                     _stream(x.device)), "nvfp4_mxfp4_quantize")
    return out


def mxfp4_dequantize(q, dtype=torch.float32, out=None):
    if out is None:
        out = torch.empty((q.rows, q.cols), dtype=dtype, device=q.codes.device)
    ct = q.c()
    code = OUT_F32 if out.dtype == torch.float32 else OUT_BF16
    _check(_lib.nvfp4_mxfp4_dequantize(ctypes.byref(ct), _ptr(out), out.stride(0), code,
                                       _stream(q.codes.device)), "nvfp4_mxfp4_dequantize")
    return out


def mxfp4_gemm(a, w, y=None, a_q=None, ws=None):
    """Y = A . W^T (bf16 out) with both operands MXFP4.  `a` is a bf16 matrix (quantized inside
    the call; `a_q`, if given, receives it) or an MxTensor."""
    if isinstance(a, MxTensor):
        m, k = a.rows, a.cols
        a_bf16, a_q, dev = None, a, a.codes.device
    else:
        assert a.dtype == torch.bfloat16 and a.dim() == 2 and a.stride(1) == 1
        m, k = a.shape
        a_bf16, dev = a, a.device
    n = w.rows
    if y is None:
        y = torch.empty((m, n), dtype=torch.bfloat16, device=dev)
    nbytes = _lib.nvfp4_mxfp4_gemm_workspace_bytes(m, k) if a_q is None else 0
    ws = _ws(nbytes, dev, ws) if nbytes else ws
    wc = w.c()
    ac = a_q.c() if a_q is not None else None
    _check(_lib.nvfp4_mxfp4_gemm(_ptr(a_bf16), m, k, a_bf16.stride(0) if a_bf16 is not None else 0,
                                 ctypes.byref(ac) if ac is not None else None, ctypes.byref(wc),
                                 _ptr(y), y.stride(0), _ptr(ws), ws.numel() if ws is not None else 0,
                                 _stream(dev)), "nvfp4_mxfp4_gemm")
    return y
