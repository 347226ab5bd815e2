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
    raise ImportError("libfp8q.so is not built (run python fp8_scaled_quantization_amd/build.py); "
                      "there is no fallback path")

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


# ------------------------------------------------------------------ argument checks
# The C ABI receives bare device pointers and cannot see a buffer's size or element type, so every
# wrapper checks here, before any pointer is passed, that each buffer has the shape and dtype the
# call will read or write (a buffer too small for what the kernels write would be written past its
# end) and that all of them live on one GPU.  Violations raise ValueError.
def _need(cond: bool, msg: str) -> None:
    if not cond:
        raise ValueError(msg)


def _mat(t, name: str, dtypes, shape=None) -> None:
    """A 2-D row-major (unit column stride) matrix of one of `dtypes`, optionally of `shape`."""
    _need(isinstance(t, torch.Tensor), "%s must be a torch tensor" % name)
    _need(t.dim() == 2 and t.stride(1) == 1,
          "%s must be a 2-D row-major tensor, got shape %s strides %s" % (name, tuple(t.shape), t.stride()))
    _need(t.dtype in dtypes, "%s must be %s, got %s" % (name, "/".join(str(d) for d in dtypes), t.dtype))
    if shape is not None:
        _need(tuple(t.shape) == tuple(shape), "%s must have shape %s, got %s" % (name, tuple(shape), tuple(t.shape)))


def _dense(t, name: str, dtype, shape) -> None:
    """A contiguous array of exactly `shape` (scale arrays are read densely, row-major)."""
    _need(isinstance(t, torch.Tensor), "%s must be a torch tensor" % name)
    _need(t.dtype == dtype, "%s must be %s, got %s" % (name, dtype, t.dtype))
    _need(tuple(t.shape) == tuple(shape), "%s must have shape %s, got %s" % (name, tuple(shape), tuple(t.shape)))
    _need(t.is_contiguous(), "%s must be contiguous" % name)


def _f32(t, name: str, n: int = 1) -> None:
    """At least n contiguous fp32 values (scales, amax, history, state)."""
    _need(isinstance(t, torch.Tensor), "%s must be a torch tensor" % name)
    _need(t.dtype == torch.float32, "%s must be float32, got %s" % (name, t.dtype))
    _need(t.numel() >= n and t.is_contiguous(), "%s must hold at least %d contiguous values" % (name, n))


def _same_gpu(*ts) -> None:
    ts = [t for t in ts if t is not None]
    _need(all(t.is_cuda for t in ts), "every buffer must be on a GPU")
    devs = {t.device.index for t in ts}
    _need(len(devs) <= 1, "every buffer must be on the same GPU")
    _need(not devs or devs == {torch.cuda.current_device()},
          "the buffers must be on the current device (the library launches there)")


# ------------------------------------------------------------------ the entry points
def fp8_amax(x: torch.Tensor, amax_out: torch.Tensor, stream=None) -> None:
    """amax_out[0] = max |x| over a 2-D fp32 or bf16 tensor (NaN if any element is NaN)."""
    _mat(x, "x", (torch.float32, torch.bfloat16))
    _f32(amax_out, "amax_out")
    _same_gpu(x, amax_out)
    _check(_L.fp8_amax(_ptr(x), _in_kind(x), x.shape[0], x.shape[1], _ld(x), _ptr(amax_out), _stream(stream)))


def fp8_quantize(mode: int, fmt: int, x: torch.Tensor, q: torch.Tensor, scales=None, tensor_scale=None,
                 scale_is_input: bool = False, amax_out=None, block=(1, 128), transpose_out: bool = False,
                 stream=None) -> None:
    """Cast x (2-D fp32/bf16) to FP8 bytes q under `mode`, writing the scales the mode uses: `scales`
    (BLOCK: fp32 per block; MX/MOSS/BLOCK_E8M0: E8M0 bytes) and, for TENSOR/MOSS, `tensor_scale`
    (derived from the amax, or read when scale_is_input).  transpose_out casts x^T.  Shapes are
    checked here (see scale_shape) before the call."""
    _mat(x, "x", (torch.float32, torch.bfloat16))
    R, Kc = (x.shape[1], x.shape[0]) if transpose_out else (x.shape[0], x.shape[1])
    _mat(q, "q", (torch.uint8,), (R, Kc))
    if mode in (BLOCK, BLOCK_E8M0):
        _need(len(block) == 2 and int(block[0]) > 0 and int(block[1]) > 0,
              "block must be two positive integers, got %s" % (block,))
    shp, dt = scale_shape(mode, R, Kc, block)
    if shp is not None:
        _dense(scales, "scales", dt, shp)
    if mode in (TENSOR, MOSS):
        _f32(tensor_scale, "tensor_scale")
        if not scale_is_input:
            _need(amax_out is not None, "amax_out is required when the scale is derived")
    if amax_out is not None:
        _f32(amax_out, "amax_out")
    _same_gpu(x, q, scales if shp is not None else None, tensor_scale if mode in (TENSOR, MOSS) else None, amax_out)
    _check(_L.fp8_quantize(mode, fmt, _ptr(x), _in_kind(x), x.shape[0], x.shape[1], _ld(x),
                           int(block[0]), int(block[1]), int(bool(transpose_out)), _ptr(q), _ld(q),
                           _ptr(scales), _ptr(tensor_scale), int(bool(scale_is_input)), _ptr(amax_out),
                           _stream(stream)))


def fp8_quantize_dual(mode: int, fmt: int, x: torch.Tensor, q: torch.Tensor, scales, qt: torch.Tensor, scales_t,
                      tensor_scale=None, scale_is_input: bool = False, amax_out=None, stream=None) -> None:
    """Both quantized copies of x in one call: q (rows x cols) grouped along each row and qt
    (cols x rows) grouped along each column, with their E8M0 scales (MX/MOSS) and one shared
    tensor scale (TENSOR/MOSS)."""
    _need(mode in (TENSOR, MX, MOSS), "fp8_quantize_dual: mode must be TENSOR, MX or MOSS")
    _mat(x, "x", (torch.float32, torch.bfloat16))
    R, C = x.shape
    _mat(q, "q", (torch.uint8,), (R, C))
    _mat(qt, "qt", (torch.uint8,), (C, R))
    if mode in (MX, MOSS):
        _dense(scales, "scales", torch.uint8, (R, -(-C // 32)))
        _dense(scales_t, "scales_t", torch.uint8, (C, -(-R // 32)))
    else:
        scales = scales_t = None
    if mode in (TENSOR, MOSS):
        _f32(tensor_scale, "tensor_scale")
        if not scale_is_input:
            _need(amax_out is not None, "amax_out is required when the scale is derived")
    if amax_out is not None:
        _f32(amax_out, "amax_out")
    _same_gpu(x, q, qt, scales, scales_t, tensor_scale if mode in (TENSOR, MOSS) else None, amax_out)
    _check(_L.fp8_quantize_dual(mode, fmt, _ptr(x), _in_kind(x), x.shape[0], x.shape[1], _ld(x),
                                _ptr(q), _ld(q), _ptr(scales), _ptr(qt), _ld(qt), _ptr(scales_t),
                                _ptr(tensor_scale), int(bool(scale_is_input)), _ptr(amax_out), _stream(stream)))


def fp8_history_update(history: torch.Tensor, amax_new: torch.Tensor, scale: torch.Tensor, fmt: int,
                       stream=None) -> None:
    """Delayed scaling: roll amax_new into the history window (newest at index 0) and set `scale`
    from the window's max for the next step (kept when that max is zero or non-finite)."""
    _f32(history, "history")
    _f32(amax_new, "amax_new")
    _f32(scale, "scale")
    _same_gpu(history, amax_new, scale)
    _check(_L.fp8_history_update(_ptr(history), history.numel(), _ptr(amax_new), _ptr(scale), fmt,
                                 _stream(stream)))


def fp8_scaled_gemm(mode: int, A: torch.Tensor, afmt: int, Ascale, B: torch.Tensor, bfmt: int, Bscale,
                    Aglobal, Bglobal, C: torch.Tensor, out_dtype: int, stream=None) -> None:
    """C = dequant(A) . dequant(B)^T for FP8 bytes A (M x K) and B (N x K) with the mode's scales
    (Ascale/Bscale per group or block; Aglobal/Bglobal fp32 tensor factors for TENSOR and MOSS, or
    a static activation scale as Aglobal for BLOCK without Ascale); C is fp32 or bf16 (out_dtype)."""
    _mat(A, "A", (torch.uint8,))
    M, K = A.shape
    _mat(B, "B", (torch.uint8,))
    N = B.shape[0]
    _need(B.shape[1] == K, "B must be N x K with K = %d (A's columns), got %s" % (K, tuple(B.shape)))
    _need(out_dtype in (OUT_F32, OUT_BF16), "out_dtype must be OUT_F32 or OUT_BF16")
    _mat(C, "C", (torch.bfloat16,) if out_dtype == OUT_BF16 else (torch.float32,), (M, N))
    nkb, ng = -(-K // 128), -(-K // 32)
    if mode in (TENSOR, MOSS):
        _f32(Aglobal, "Aglobal")
        _f32(Bglobal, "Bglobal")
    if mode in (BLOCK, BLOCK_E8M0):
        if Ascale is None:
            _f32(Aglobal, "Aglobal (static activation scale)")
        else:
            _dense(Ascale, "Ascale", torch.float32, (M, nkb))
        _dense(Bscale, "Bscale", torch.float32 if mode == BLOCK else torch.uint8, (-(-N // 128), nkb))
    elif mode in (MX, MOSS):
        _dense(Ascale, "Ascale", torch.uint8, (M, ng))
        _dense(Bscale, "Bscale", torch.uint8, (N, ng))
    else:
        _need(mode == TENSOR, "unknown mode %r" % (mode,))
        Ascale = Bscale = None
    if mode == MX or (mode in (BLOCK, BLOCK_E8M0) and Ascale is not None):
        Aglobal = None
    if mode in (MX, BLOCK, BLOCK_E8M0):
        Bglobal = None
    _same_gpu(A, B, C, Ascale, Bscale, Aglobal, Bglobal)
    _check(_L.fp8_scaled_gemm(mode, _ptr(A), afmt, _ptr(Ascale), _ptr(B), bfmt, _ptr(Bscale),
                              _ptr(Aglobal), _ptr(Bglobal), M, N, K, _ld(A), _ld(B), _ptr(C), out_dtype,
                              _ld(C), _stream(stream)))


def fp8_history_merge(hist_dst: torch.Tensor, hist_src: torch.Tensor, scale_dst: torch.Tensor, scale_src: torch.Tensor,
                      stream=None) -> None:
    """Merge two updates of one delayed-scaling state: history and scale become their elementwise
    max (NaN propagates)."""
    _f32(hist_dst, "hist_dst", 0)
    _f32(hist_src, "hist_src", 0)
    _need(hist_dst.numel() == hist_src.numel(), "histories differ in length")
    _f32(scale_dst, "scale_dst")
    _f32(scale_src, "scale_src")
    _same_gpu(hist_dst, hist_src, scale_dst, scale_src)
    _check(_L.fp8_history_merge(_ptr(hist_dst), _ptr(hist_src), hist_dst.numel(), _ptr(scale_dst), _ptr(scale_src),
                                _stream(stream)))


def fp8_auto_scale(state: torch.Tensor, rescale: bool, amax_now, lr: float, fmt: int, scale_out: torch.Tensor,
                   stream=None) -> None:
    """One step of automatic weight scaling: scale_out from the last measured weight max plus the
    learning rates since (state = [base, lr sum]); a rescale step takes amax_now as the new base."""
    _f32(state, "state", 2)
    _f32(scale_out, "scale_out")
    if rescale:
        _f32(amax_now, "amax_now")
    else:
        amax_now = None
    _same_gpu(state, scale_out, amax_now)
    _check(_L.fp8_auto_scale(_ptr(state), int(bool(rescale)), _ptr(amax_now), float(lr), fmt, _ptr(scale_out),
                             _stream(stream)))


def fp8_scale_to_e8m0(s: torch.Tensor, e8m0: torch.Tensor, bad_count: torch.Tensor, stream=None) -> None:
    """Exact conversion of power-of-two fp32 scales to UE8M0 bytes; anything else becomes 0xFF and is
    counted in bad_count[0]."""
    _f32(s, "s", 0)
    _need(e8m0.dtype == torch.uint8 and e8m0.numel() == s.numel() and e8m0.is_contiguous(),
          "e8m0 must be contiguous uint8 with s's size")
    _need(bad_count.dtype == torch.int32 and bad_count.numel() >= 1, "bad_count must hold one int32")
    _same_gpu(s, e8m0, bad_count)
    _check(_L.fp8_scale_to_e8m0(_ptr(s), s.numel(), _ptr(e8m0), _ptr(bad_count), _stream(stream)))


def fp8_block_dequantize(mode: int, fmt: int, q: torch.Tensor, scales: torch.Tensor, out: torch.Tensor,
                         block=(128, 128), stream=None) -> None:
    """out = decode(q) * block scale, one fp32 product per element, stored as fp32 or bf16 (RNE) by
    out's dtype; scales are fp32 (BLOCK) or UE8M0 bytes (BLOCK_E8M0)."""
    _need(mode in (BLOCK, BLOCK_E8M0), "mode must be BLOCK or BLOCK_E8M0")
    _need(len(block) == 2 and int(block[0]) > 0 and int(block[1]) > 0,
          "block must be two positive integers, got %s" % (block,))
    _mat(q, "q", (torch.uint8,))
    _mat(out, "out", (torch.bfloat16, torch.float32), tuple(q.shape))
    shp, dt = scale_shape(mode, q.shape[0], q.shape[1], block)
    _dense(scales, "scales", dt, shp)
    _same_gpu(q, out, scales)
    out_dtype = OUT_BF16 if out.dtype == torch.bfloat16 else OUT_F32
    _check(_L.fp8_block_dequantize(mode, fmt, _ptr(q), q.shape[0], q.shape[1], _ld(q), _ptr(scales), int(block[0]),
                                   int(block[1]), _ptr(out), out_dtype, _ld(out), _stream(stream)))


# ------------------------------------------------------------------ allocating conveniences
def scale_shape(mode: int, out_rows: int, out_cols: int, block=(1, 128)):
    """(shape, dtype) of the scale array fp8_quantize writes for an out_rows x out_cols output, or
    (None, None) when the mode has none."""
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
