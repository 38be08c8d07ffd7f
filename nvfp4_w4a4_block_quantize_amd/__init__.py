"""Python binding of the NVFP4 W4A4 linear-layer library (libnvfp4.so).

Argument marshalling only: every operation runs in the HIP kernels behind the
C ABI declared in include/nvfp4.h.  torch provides device memory and the
current stream; there is no fallback path: if the library is missing or no
GPU is visible, the calls raise.

Functions carry the C names:
  nvfp4_amax_observe(x, amax_state)          -> amax_state
  nvfp4_gscale_from_amax(amax_state)         -> gscale
  nvfp4_kv_scale_from_amax(amax_state)       -> scale
  nvfp4_kv_quantize_fp8(x, scale)            -> E4M3 bytes
  nvfp4_quantize(x, gscale, mode)            -> (codes, scales)
  nvfp4_fuse_rescale(scales, k, rows, gs)    -> (g_star, lossy_blocks)
  nvfp4_gemm(a_codes, a_scales, a_gscale,
             w_codes, w_scales, w_gscale,
             out_dtype)                      -> c
"""
from __future__ import annotations

import ctypes
import os

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libnvfp4.so")

NVFP4_OK = 0
STATUS_NAMES = {0: "NVFP4_OK", 1: "NVFP4_ERR_NULL", 2: "NVFP4_ERR_SHAPE", 3: "NVFP4_ERR_ALIGN",
                4: "NVFP4_ERR_DTYPE", 5: "NVFP4_ERR_RANGE", 6: "NVFP4_ERR_DEVICE"}
F32, BF16, F16 = 0, 1, 2
GSCALE_STATIC, GSCALE_DYNAMIC = 0, 1
MAX_FUSED_MODULES = 64

# every symbol include/nvfp4.h declares, with (restype, argtypes)
_P = ctypes.c_void_p
_I64 = ctypes.c_int64
_I32 = ctypes.c_int32
SIGNATURES = {
    "nvfp4_quantize": (_I32, [_P, _I32, _I64, _I64, _I64, _P, _I32, _P, _P, _P]),
    "nvfp4_fuse_rescale": (_I32, [_P, _I64, _I32, _P, _P, _P, _P, _P]),
    "nvfp4_gemm": (_I32, [_I64, _I64, _I64, _P, _P, _P, _P, _P, _P, _P, _I32, _I64, _P]),
    "nvfp4_amax_observe": (_I32, [_P, _I32, _I64, _I64, _I64, _P, _P]),
    "nvfp4_gscale_from_amax": (_I32, [_P, _P, _P]),
    "nvfp4_kv_quantize_fp8": (_I32, [_P, _I32, _I64, _I64, _I64, _P, _P, _P]),
    "nvfp4_kv_scale_from_amax": (_I32, [_P, _P, _P]),
    "nvfp4_status_str": (ctypes.c_char_p, [_I32]),
    "nvfp4_abi_version": (_I32, []),
}

_lib = None


class Nvfp4Error(RuntimeError):
    def __init__(self, fn: str, status: int, msg: str):
        super().__init__(f"{fn}: {STATUS_NAMES.get(status, status)} ({msg})")
        self.status = status


def load_library(path: str | None = None):
    """Load libnvfp4.so (built in-tree by build.build()); raises if it is missing."""
    global _lib
    if _lib is not None and path is None:
        return _lib
    p = path or LIB_PATH
    if not os.path.exists(p):
        raise RuntimeError(f"{p} is missing: build it first (python -c 'import __graft_entry__ as g; g.build()')")
    lib = ctypes.CDLL(p)
    for name, (res, args) in SIGNATURES.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    if path is None:
        _lib = lib
    return lib


def status_str(status: int) -> str:
    return load_library().nvfp4_status_str(status).decode()


def _check(fn: str, status: int):
    if status != NVFP4_OK:
        raise Nvfp4Error(fn, status, status_str(status))


def _torch():
    import torch

    return torch


_DTYPES = {}


def _dtype_code(dtype) -> int:
    if not _DTYPES:
        torch = _torch()
        _DTYPES.update({torch.float32: F32, torch.bfloat16: BF16, torch.float16: F16})
    if dtype not in _DTYPES:
        raise TypeError(f"unsupported dtype {dtype}")
    return _DTYPES[dtype]


def _stream_ptr(stream=None, like=None) -> int:
    """hipStream_t of `stream`, else torch's current stream on the device of
    tensor `like` (or the current device).  torch's raw-stream accessor skips
    building a Stream object, which costs more than the rest of a call."""
    torch = _torch()
    if stream is not None:
        return int(stream.cuda_stream)
    raw = getattr(torch._C, "_cuda_getCurrentRawStream", None)
    index = like.get_device() if like is not None else torch.cuda.current_device()
    if raw is not None:
        return int(raw(index))
    return int(torch.cuda.current_stream(index).cuda_stream)


def _dev(t, name):
    if not t.is_cuda:
        raise ValueError(f"{name} must be a GPU tensor")
    return t.data_ptr()


def _same_device(t, like, name):
    if t.device != like.device:
        raise ValueError(f"{name} is on {t.device}, expected {like.device}")


def _bytes_arg(t, shape, name, like=None):
    """A uint8 tensor the library reads or writes as dense [rows][cols] bytes."""
    torch = _torch()
    if t.dtype != torch.uint8:
        raise ValueError(f"{name} must be uint8, got {t.dtype}")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if like is not None:
        _same_device(t, like, name)


def _scalar_f32(t, name, like=None):
    """A one-element float32 tensor (a global scale or an amax word)."""
    torch = _torch()
    if t.dtype != torch.float32 or t.numel() != 1:
        raise ValueError(f"{name} must be a float32 tensor with one element, got {t.dtype} with {t.numel()}")
    if like is not None:
        _same_device(t, like, name)


def nvfp4_quantize(x, gscale, mode: str = "static", codes=None, scales=None, stream=None):
    """Quantise a 2-D GPU tensor x (f32 / bf16 / f16, unit stride along columns).

    gscale: GPU float32 tensor with one element; read (mode='static') or
    written (mode='dynamic').  Returns (codes uint8 [rows, cols/2],
    scales uint8 [rows, cols/16]).
    """
    torch = _torch()
    if x.dim() != 2 or x.stride(1) != 1:
        raise ValueError("x must be 2-D with unit column stride")
    rows, cols = x.shape
    if codes is None:
        codes = torch.empty((rows, cols // 2), dtype=torch.uint8, device=x.device)
    if scales is None:
        scales = torch.empty((rows, cols // 16), dtype=torch.uint8, device=x.device)
    _bytes_arg(codes, (rows, cols // 2), "codes", x)
    _bytes_arg(scales, (rows, cols // 16), "scales", x)
    _scalar_f32(gscale, "gscale", x)
    if mode not in ("static", "dynamic"):
        raise ValueError(f"mode must be 'static' or 'dynamic', got {mode!r}")
    m = {"static": GSCALE_STATIC, "dynamic": GSCALE_DYNAMIC}[mode]
    st = load_library().nvfp4_quantize(_dev(x, "x"), _dtype_code(x.dtype), rows, cols, x.stride(0),
                                       _dev(gscale, "gscale"), m, _dev(codes, "codes"), _dev(scales, "scales"),
                                       _stream_ptr(stream, x))
    _check("nvfp4_quantize", st)
    return codes, scales


def nvfp4_amax_observe(x, amax_state, stream=None):
    """Fold max|x| of one calibration batch (2-D GPU tensor) into amax_state,
    a GPU float32 tensor with one element that starts at 0."""
    if x.dim() != 2 or x.stride(1) != 1:
        raise ValueError("x must be 2-D with unit column stride")
    rows, cols = x.shape
    _scalar_f32(amax_state, "amax_state", x)
    st = load_library().nvfp4_amax_observe(_dev(x, "x"), _dtype_code(x.dtype), rows, cols, x.stride(0),
                                           _dev(amax_state, "amax_state"), _stream_ptr(stream, x))
    _check("nvfp4_amax_observe", st)
    return amax_state


def nvfp4_gscale_from_amax(amax_state, gscale=None, stream=None):
    """Encode global scale fp32(2688 / amax) of the observed calibration set."""
    torch = _torch()
    if gscale is None:
        gscale = torch.empty(1, dtype=torch.float32, device=amax_state.device)
    _scalar_f32(amax_state, "amax_state")
    _scalar_f32(gscale, "gscale", amax_state)
    st = load_library().nvfp4_gscale_from_amax(_dev(amax_state, "amax_state"), _dev(gscale, "gscale"),
                                               _stream_ptr(stream, amax_state))
    _check("nvfp4_gscale_from_amax", st)
    return gscale


def nvfp4_kv_quantize_fp8(x, scale, out=None, stream=None):
    """Static FP8 E4M3 codes of a 2-D GPU tensor (one byte per element, uint8)."""
    torch = _torch()
    if x.dim() != 2 or x.stride(1) != 1:
        raise ValueError("x must be 2-D with unit column stride")
    rows, cols = x.shape
    if out is None:
        out = torch.empty((rows, cols), dtype=torch.uint8, device=x.device)
    _bytes_arg(out, (rows, cols), "out", x)
    _scalar_f32(scale, "scale", x)
    st = load_library().nvfp4_kv_quantize_fp8(_dev(x, "x"), _dtype_code(x.dtype), rows, cols, x.stride(0),
                                              _dev(scale, "scale"), _dev(out, "out"), _stream_ptr(stream, x))
    _check("nvfp4_kv_quantize_fp8", st)
    return out


def nvfp4_kv_scale_from_amax(amax_state, scale=None, stream=None):
    """Encode scale fp32(448 / amax) for nvfp4_kv_quantize_fp8."""
    torch = _torch()
    if scale is None:
        scale = torch.empty(1, dtype=torch.float32, device=amax_state.device)
    _scalar_f32(amax_state, "amax_state")
    _scalar_f32(scale, "scale", amax_state)
    st = load_library().nvfp4_kv_scale_from_amax(_dev(amax_state, "amax_state"), _dev(scale, "scale"),
                                                 _stream_ptr(stream, amax_state))
    _check("nvfp4_kv_scale_from_amax", st)
    return scale


def nvfp4_fuse_rescale(scales, k: int, module_rows, module_gscales, want_lossy: bool = True, stream=None):
    """Rewrite the stacked block scales of a fused group in place.

    Returns (g_star, lossy) where g_star is the shared encode scale (float)
    and lossy a GPU int64 tensor [1] (or None) counting changed blocks.
    """
    torch = _torch()
    n = len(module_rows)
    if len(module_gscales) != n:
        raise ValueError("module_rows and module_gscales differ in length")
    _bytes_arg(scales, (sum(int(r) for r in module_rows), int(k) // 16), "scales")
    rows_arr = (ctypes.c_int64 * n)(*[int(r) for r in module_rows])
    gs_arr = (ctypes.c_float * n)(*[float(g) for g in module_gscales])
    g_star = ctypes.c_float(0.0)
    lossy = torch.empty(1, dtype=torch.int64, device=scales.device) if want_lossy else None
    st = load_library().nvfp4_fuse_rescale(_dev(scales, "scales"), int(k), n, ctypes.cast(rows_arr, _P),
                                           ctypes.cast(gs_arr, _P), ctypes.addressof(g_star),
                                           None if lossy is None else lossy.data_ptr(), _stream_ptr(stream, scales))
    _check("nvfp4_fuse_rescale", st)
    return g_star.value, lossy


def nvfp4_gemm(a_codes, a_scales, a_gscale, w_codes, w_scales, w_gscale, out_dtype=None, out=None, stream=None):
    """C = A_hat W_hat^T from two quantised operands (K along the last axis)."""
    torch = _torch()
    m, kh = a_codes.shape
    n = w_codes.shape[0]
    k = kh * 2
    _bytes_arg(a_codes, (m, kh), "a_codes")
    _bytes_arg(a_scales, (m, k // 16), "a_scales", a_codes)
    _bytes_arg(w_codes, (n, kh), "w_codes", a_codes)
    _bytes_arg(w_scales, (n, k // 16), "w_scales", a_codes)
    _scalar_f32(a_gscale, "a_gscale", a_codes)
    _scalar_f32(w_gscale, "w_gscale", a_codes)
    if out is None:
        out = torch.empty((m, n), dtype=out_dtype or torch.float32, device=a_codes.device)
    if out.dim() != 2 or out.stride(1) != 1 or out.shape[0] != m or out.shape[1] < n:
        raise ValueError("out must be [m, >=n] with unit column stride")
    _same_device(out, a_codes, "out")
    st = load_library().nvfp4_gemm(m, n, k, _dev(a_codes, "a_codes"), _dev(a_scales, "a_scales"),
                                   _dev(a_gscale, "a_gscale"), _dev(w_codes, "w_codes"), _dev(w_scales, "w_scales"),
                                   _dev(w_gscale, "w_gscale"), _dev(out, "out"), _dtype_code(out.dtype),
                                   out.stride(0), _stream_ptr(stream, a_codes))
    _check("nvfp4_gemm", st)
    return out
