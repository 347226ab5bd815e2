"""ctypes binding of libfp8q.so: the C ABI of include/fp8q.h with the same names.

Argument marshalling only: torch tensors supply device pointers and the current HIP stream; every
step of the computation runs in the library's kernels.  Importing this module raises if the built
library is missing -- there is no fallback path.
"""
from __future__ import annotations

import ctypes
import os

import torch

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libfp8q.so")

OK, ERR_INVALID_ARG, ERR_UNSUPPORTED, ERR_HIP, ERR_NO_DEVICE = 0, -1, -2, -3, -4
E4M3, E5M2 = 0, 1
IN_F32, IN_BF16 = 0, 1
OUT_F32, OUT_BF16 = 0, 1
TENSOR, BLOCK, MX, MOSS, BLOCK_E8M0 = 0, 1, 2, 3, 4

EXPORTS = ("fp8q_init", "fp8q_last_error", "fp8_amax", "fp8_quantize", "fp8_quantize_dual", "fp8_history_update",
           "fp8_scaled_gemm", "fp8_history_merge", "fp8_auto_scale", "fp8_scale_to_e8m0", "fp8_block_dequantize")

if not os.path.exists(LIB_PATH):
    raise ImportError("libfp8q.so is not built (run __graft_entry__.build() or "
                      "python fp8_scaled_quantization_amd/build.py); there is no fallback path")

_L = ctypes.CDLL(LIB_PATH)
_P, _I64, _I = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int
_L.fp8q_init.restype = _I
_L.fp8q_init.argtypes = []
_L.fp8q_last_error.restype = ctypes.c_char_p
_L.fp8q_last_error.argtypes = []
_L.fp8_amax.restype = _I
_L.fp8_amax.argtypes = [_P, _I, _I64, _I64, _I64, _P, _P]
_L.fp8_quantize.restype = _I
_L.fp8_quantize.argtypes = [_I, _I, _P, _I, _I64, _I64, _I64, _I, _I, _I, _P, _I64, _P, _P, _I, _P, _P]
_L.fp8_quantize_dual.restype = _I
_L.fp8_quantize_dual.argtypes = [_I, _I, _P, _I, _I64, _I64, _I64, _P, _I64, _P, _P, _I64, _P, _P, _I, _P, _P]
_L.fp8_history_update.restype = _I
_L.fp8_history_update.argtypes = [_P, _I64, _P, _P, _I, _P]
_L.fp8_scaled_gemm.restype = _I
_L.fp8_scaled_gemm.argtypes = [_I, _P, _I, _P, _P, _I, _P, _P, _P, _I64, _I64, _I64, _I64, _I64, _P, _I, _I64, _P]
_L.fp8_history_merge.restype = _I
_L.fp8_history_merge.argtypes = [_P, _P, _I64, _P, _P, _P]
_L.fp8_auto_scale.restype = _I
_L.fp8_auto_scale.argtypes = [_P, _I, _P, ctypes.c_float, _I, _P, _P]
_L.fp8_scale_to_e8m0.restype = _I
_L.fp8_scale_to_e8m0.argtypes = [_P, _I64, _P, _P, _P]
_L.fp8_block_dequantize.restype = _I
_L.fp8_block_dequantize.argtypes = [_I, _I, _P, _I64, _I64, _I64, _P, _I, _I, _P, _I, _I64, _P]


class Fp8qError(RuntimeError):
    def __init__(self, code: int, msg: str):
        super().__init__("fp8q status %d: %s" % (code, msg))
        self.code = code


def lib():
    return _L


def _check(rc: int) -> None:
    if rc != OK:
        raise Fp8qError(rc, _L.fp8q_last_error().decode())


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream):
    if stream is not None:
        return ctypes.c_void_p(stream)
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def _in_kind(x: torch.Tensor) -> int:
    if x.dtype == torch.float32:
        return IN_F32
    if x.dtype == torch.bfloat16:
        return IN_BF16
    raise TypeError("input must be float32 or bfloat16, got %s" % x.dtype)


def _ld(x: torch.Tensor) -> int:
    if x.dim() != 2 or x.stride(1) != 1:
        raise ValueError("expected a 2-D row-major tensor (unit column stride)")
    return x.stride(0)


def init() -> None:
    _check(_L.fp8q_init())


# ------------------------------------------------------------------ the entry points
def fp8_amax(x: torch.Tensor, amax_out: torch.Tensor, stream=None) -> None:
    _check(_L.fp8_amax(_ptr(x), _in_kind(x), x.shape[0], x.shape[1], _ld(x), _ptr(amax_out), _stream(stream)))


def fp8_quantize(mode: int, fmt: int, x: torch.Tensor, q: torch.Tensor, scales=None, tensor_scale=None,
                 scale_is_input: bool = False, amax_out=None, block=(1, 128), transpose_out: bool = False,
                 stream=None) -> None:
    if q.dtype != torch.uint8:
        raise TypeError("q must be uint8")
    _check(_L.fp8_quantize(mode, fmt, _ptr(x), _in_kind(x), x.shape[0], x.shape[1], _ld(x),
                           int(block[0]), int(block[1]), int(bool(transpose_out)), _ptr(q), _ld(q),
                           _ptr(scales), _ptr(tensor_scale), int(bool(scale_is_input)), _ptr(amax_out),
                           _stream(stream)))


def fp8_quantize_dual(mode: int, fmt: int, x: torch.Tensor, q: torch.Tensor, scales, qt: torch.Tensor, scales_t,
                      tensor_scale=None, scale_is_input: bool = False, amax_out=None, stream=None) -> None:
    if q.dtype != torch.uint8 or qt.dtype != torch.uint8:
        raise TypeError("q and qt must be uint8")
    _check(_L.fp8_quantize_dual(mode, fmt, _ptr(x), _in_kind(x), x.shape[0], x.shape[1], _ld(x),
                                _ptr(q), _ld(q), _ptr(scales), _ptr(qt), _ld(qt), _ptr(scales_t),
                                _ptr(tensor_scale), int(bool(scale_is_input)), _ptr(amax_out), _stream(stream)))


def fp8_history_update(history: torch.Tensor, amax_new: torch.Tensor, scale: torch.Tensor, fmt: int,
                       stream=None) -> None:
    _check(_L.fp8_history_update(_ptr(history), history.numel(), _ptr(amax_new), _ptr(scale), fmt,
                                 _stream(stream)))


def fp8_scaled_gemm(mode: int, A: torch.Tensor, afmt: int, Ascale, B: torch.Tensor, bfmt: int, Bscale,
                    Aglobal, Bglobal, C: torch.Tensor, out_dtype: int, stream=None) -> None:
    M, K = A.shape
    N = B.shape[0]
    _check(_L.fp8_scaled_gemm(mode, _ptr(A), afmt, _ptr(Ascale), _ptr(B), bfmt, _ptr(Bscale),
                              _ptr(Aglobal), _ptr(Bglobal), M, N, K, _ld(A), _ld(B), _ptr(C), out_dtype,
                              _ld(C), _stream(stream)))


def fp8_history_merge(hist_dst: torch.Tensor, hist_src: torch.Tensor, scale_dst: torch.Tensor, scale_src: torch.Tensor,
                      stream=None) -> None:
    if hist_dst.numel() != hist_src.numel():
        raise ValueError("histories differ in length")
    _check(_L.fp8_history_merge(_ptr(hist_dst), _ptr(hist_src), hist_dst.numel(), _ptr(scale_dst), _ptr(scale_src),
                                _stream(stream)))


def fp8_auto_scale(state: torch.Tensor, rescale: bool, amax_now, lr: float, fmt: int, scale_out: torch.Tensor,
                   stream=None) -> None:
    _check(_L.fp8_auto_scale(_ptr(state), int(bool(rescale)), _ptr(amax_now), float(lr), fmt, _ptr(scale_out),
                             _stream(stream)))


def fp8_scale_to_e8m0(s: torch.Tensor, e8m0: torch.Tensor, bad_count: torch.Tensor, stream=None) -> None:
    if s.numel() != e8m0.numel() or e8m0.dtype != torch.uint8 or bad_count.dtype != torch.int32:
        raise TypeError("e8m0 must be uint8 with s's size and bad_count int32")
    _check(_L.fp8_scale_to_e8m0(_ptr(s), s.numel(), _ptr(e8m0), _ptr(bad_count), _stream(stream)))


def fp8_block_dequantize(mode: int, fmt: int, q: torch.Tensor, scales: torch.Tensor, out: torch.Tensor,
                         block=(128, 128), stream=None) -> None:
    out_dtype = OUT_BF16 if out.dtype == torch.bfloat16 else OUT_F32
    _check(_L.fp8_block_dequantize(mode, fmt, _ptr(q), q.shape[0], q.shape[1], _ld(q), _ptr(scales), int(block[0]),
                                   int(block[1]), _ptr(out), out_dtype, _ld(out), _stream(stream)))


# ------------------------------------------------------------------ allocating conveniences
def scale_shape(mode: int, out_rows: int, out_cols: int, block=(1, 128)):
    if mode == BLOCK:
        return (-(-out_rows // block[0]), -(-out_cols // block[1])), torch.float32
    if mode == BLOCK_E8M0:
        return (-(-out_rows // block[0]), -(-out_cols // block[1])), torch.uint8
    if mode in (MX, MOSS):
        return (out_rows, -(-out_cols // 32)), torch.uint8
    return None, None


def quantize(x: torch.Tensor, mode: int, fmt: int, block=(1, 128), transpose_out: bool = False,
             tensor_scale=None, scale_is_input: bool = False, amax_out=None, stream=None):
    """Allocate the outputs with torch and call fp8_quantize.  Returns (q, scales, tensor_scale, amax)."""
    R, Kc = (x.shape[1], x.shape[0]) if transpose_out else (x.shape[0], x.shape[1])
    q = torch.empty((R, Kc), dtype=torch.uint8, device=x.device)
    shp, dt = scale_shape(mode, R, Kc, block)
    scales = torch.empty(shp, dtype=dt, device=x.device) if shp is not None else None
    if mode in (TENSOR, MOSS) and tensor_scale is None:
        tensor_scale = torch.ones(1, dtype=torch.float32, device=x.device)
    if mode in (TENSOR, MOSS) and not scale_is_input and amax_out is None:
        amax_out = torch.zeros(1, dtype=torch.float32, device=x.device)
    fp8_quantize(mode, fmt, x, q, scales, tensor_scale, scale_is_input, amax_out, block, transpose_out, stream)
    return q, scales, tensor_scale, amax_out


def quantize_dual(x: torch.Tensor, mode: int, fmt: int, tensor_scale=None, scale_is_input: bool = False,
                  amax_out=None, stream=None):
    """Allocate both copies and call fp8_quantize_dual.  Returns (q, scales, qt, scales_t, tensor_scale, amax)."""
    R, C = x.shape
    q = torch.empty((R, C), dtype=torch.uint8, device=x.device)
    qt = torch.empty((C, R), dtype=torch.uint8, device=x.device)
    shp, dt = scale_shape(mode, R, C)
    shpt, _ = scale_shape(mode, C, R)
    scales = torch.empty(shp, dtype=dt, device=x.device) if shp is not None else None
    scales_t = torch.empty(shpt, dtype=dt, device=x.device) if shpt is not None else None
    if mode in (TENSOR, MOSS) and tensor_scale is None:
        tensor_scale = torch.ones(1, dtype=torch.float32, device=x.device)
    if mode in (TENSOR, MOSS) and not scale_is_input and amax_out is None:
        amax_out = torch.zeros(1, dtype=torch.float32, device=x.device)
    fp8_quantize_dual(mode, fmt, x, q, scales, qt, scales_t, tensor_scale, scale_is_input, amax_out, stream)
    return q, scales, qt, scales_t, tensor_scale, amax_out


def scaled_gemm(mode: int, A, afmt, Ascale, B, bfmt, Bscale, Aglobal=None, Bglobal=None,
                out_dtype: int = OUT_BF16, stream=None) -> torch.Tensor:
    C = torch.empty((A.shape[0], B.shape[0]), dtype=torch.bfloat16 if out_dtype == OUT_BF16 else torch.float32,
                    device=A.device)
    fp8_scaled_gemm(mode, A, afmt, Ascale, B, bfmt, Bscale, Aglobal, Bglobal, C, out_dtype, stream)
    return C


def scale_to_e8m0(s: torch.Tensor, stream=None) -> torch.Tensor:
    """Exact fp32 -> UE8M0 conversion; raises ValueError if any scale is not an exact power of two in
    range (the conversion never rounds: rounding block scales without re-quantizing corrupts weights)."""
    e = torch.empty(s.shape, dtype=torch.uint8, device=s.device)
    bad = torch.zeros(1, dtype=torch.int32, device=s.device)
    fp8_scale_to_e8m0(s.contiguous(), e, bad, stream)
    n = int(bad.item())
    if n:
        raise ValueError("%d of %d scales are not exact powers of two in [2^-127, 2^127]" % (n, s.numel()))
    return e


def block_dequantize(mode: int, fmt: int, q: torch.Tensor, scales: torch.Tensor, block=(128, 128),
                     out_dtype: int = OUT_BF16, stream=None) -> torch.Tensor:
    out = torch.empty(q.shape, dtype=torch.bfloat16 if out_dtype == OUT_BF16 else torch.float32, device=q.device)
    fp8_block_dequantize(mode, fmt, q, scales, out, block, stream)
    return out
