"""ctypes binding of the C oracle (oracle.c) for numpy arrays on the host.

TEST INFRASTRUCTURE ONLY: imported by the tests, the package smoke check and the benchmark's
CPU-baseline leg, never by the product path.  Every function is a thin marshalling wrapper: the
arithmetic, and the page citation for it, live in oracle.c.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB_PATH = os.path.join(_HERE, "liboracle.so")

E4M3, E5M2 = 0, 1
IN_F32, IN_BF16 = 0, 1
TENSOR, BLOCK, MX, MOSS, BLOCK_E8M0 = 0, 1, 2, 3, 4
FP8_MAX = {E4M3: 448.0, E5M2: 57344.0}

_lib = None


def build(force: bool = False) -> str:
    """Compile oracle.c with plain gcc (no fast-math) into liboracle.so next to it."""
    if force or not os.path.exists(_LIB_PATH) or os.path.getmtime(_LIB_PATH) < os.path.getmtime(_SRC):
        tmp = _LIB_PATH + ".tmp%d" % os.getpid()
        subprocess.check_call(["gcc", "-O2", "-fopenmp", "-std=c11", "-fPIC", "-shared",
                               "-o", tmp, _SRC, "-lm"])
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH) or os.path.getmtime(_LIB_PATH) < os.path.getmtime(_SRC):
            build()
        L = ctypes.CDLL(_LIB_PATH)
        P, I64, I, F, D = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int, ctypes.c_float, ctypes.c_double
        sig = {
            "orc_fp8_max": (D, [I]),
            "orc_fp8_decode": (D, [I, I]),
            "orc_fp8_encode": (ctypes.c_uint8, [F, I]),
            "orc_fp8_encode_array": (None, [P, I64, I, P]),
            "orc_fp8_decode_array": (None, [P, I64, I, P]),
            "orc_amax": (F, [P, I, I64, I64, I64]),
            "orc_compute_scale": (F, [F, I, F]),
            "orc_quantize_value": (ctypes.c_uint8, [F, F, I]),
            "orc_quantize_tensor": (None, [P, I, I64, I64, I64, I, F, I, P, I64]),
            "orc_quantize_block": (None, [P, I, I64, I64, I64, I, I64, I64, I, P, I64, P]),
            "orc_quantize_mx": (None, [P, I, I64, I64, I64, I, I, P, I64, P]),
            "orc_quantize_moss": (None, [P, I, I64, I64, I64, I, I, P, I64, P, P]),
            "orc_quantize_moss_given": (None, [P, I, I64, I64, I64, I, I, F, P, I64, P]),
            "orc_history_roll_insert": (None, [P, I64, F]),
            "orc_history_max": (F, [P, I64]),
            "orc_delayed_step": (None, [P, I, I64, I64, I64, I, I, P, P, I64, P, I64, P]),
            "orc_dequantize": (None, [I, P, I, I64, I64, I64, P, I64, I64, P, P]),
            "orc_gemm_ref": (None, [P, P, I64, I64, I64, P, I64, P, P]),
            "orc_gemm_ref_terms": (None, [P, P, I64, I64, I64, I64, P, I64, P, P, P, P]),
            "orc_snr_db": (D, [P, P, I64]),
            "orc_quantize_block_e8m0": (None, [P, I, I64, I64, I64, I, I64, I64, I, P, I64, P]),
            "orc_scales_f32_to_e8m0": (I64, [P, I64, P]),
            "orc_history_merge": (None, [P, P, I64, P, F]),
            "orc_auto_scale_step": (F, [P, I, F, F, I]),
            "orc_block_dequantize": (None, [I, P, I, I64, I64, I64, P, I64, I64, I, P]),
        }
        for name, (res, args) in sig.items():
            fn = getattr(L, name)
            fn.restype = res
            fn.argtypes = args
        _lib = L
    return _lib


def _p(a: np.ndarray):
    return a.ctypes.data_as(ctypes.c_void_p)


def _input(x: np.ndarray):
    """(array, in_kind): fp32 arrays as-is, bf16 given as uint16 bit patterns."""
    x = np.ascontiguousarray(x)
    if x.dtype == np.float32:
        return x, IN_F32
    if x.dtype == np.uint16:
        return x, IN_BF16
    raise TypeError("oracle inputs are float32 or bf16 bit patterns (uint16), got %s" % x.dtype)


# ------------------------------------------------------------------ codec
def fp8_max(fmt: int) -> float:
    return lib().orc_fp8_max(fmt)


def decode(code: int, fmt: int) -> float:
    return lib().orc_fp8_decode(int(code), fmt)


def encode(v: float, fmt: int) -> int:
    return int(lib().orc_fp8_encode(float(np.float32(v)), fmt))


def encode_array(v: np.ndarray, fmt: int) -> np.ndarray:
    v = np.ascontiguousarray(v, dtype=np.float32)
    out = np.empty(v.shape, np.uint8)
    lib().orc_fp8_encode_array(_p(v), v.size, fmt, _p(out))
    return out


def decode_array(q: np.ndarray, fmt: int) -> np.ndarray:
    q = np.ascontiguousarray(q, dtype=np.uint8)
    out = np.empty(q.shape, np.float64)
    lib().orc_fp8_decode_array(_p(q), q.size, fmt, _p(out))
    return out


# ------------------------------------------------------------------ amax / scales
def amax(x: np.ndarray) -> np.float32:
    x, kind = _input(x)
    r, c = x.shape
    return np.float32(lib().orc_amax(_p(x), kind, r, c, c))


def compute_scale(a: float, fmt: int, fallback: float) -> np.float32:
    return np.float32(lib().orc_compute_scale(float(a), fmt, float(fallback)))


def quantize_value(x: float, s: float, fmt: int) -> int:
    return int(lib().orc_quantize_value(float(x), float(s), fmt))


# ------------------------------------------------------------------ schemes
def _out_shape(x, transpose):
    r, c = x.shape
    return (c, r) if transpose else (r, c)


def quantize_tensor(x: np.ndarray, fmt: int, scale: float, transpose: bool = False) -> np.ndarray:
    x, kind = _input(x)
    R, C = _out_shape(x, transpose)
    q = np.empty((R, C), np.uint8)
    lib().orc_quantize_tensor(_p(x), kind, x.shape[0], x.shape[1], x.shape[1], fmt,
                              float(scale), int(transpose), _p(q), C)
    return q


def quantize_tensor_current(x: np.ndarray, fmt: int, transpose: bool = False):
    """Current per-tensor scaling: scale = amax/MAX (fallback 1), then quantize."""
    s = compute_scale(amax(x), fmt, 1.0)
    return quantize_tensor(x, fmt, s, transpose), s


def quantize_block(x: np.ndarray, fmt: int, br: int, bc: int, transpose: bool = False):
    x, kind = _input(x)
    R, C = _out_shape(x, transpose)
    q = np.empty((R, C), np.uint8)
    s = np.empty(((R + br - 1) // br, (C + bc - 1) // bc), np.float32)
    lib().orc_quantize_block(_p(x), kind, x.shape[0], x.shape[1], x.shape[1], fmt, br, bc,
                             int(transpose), _p(q), C, _p(s))
    return q, s


def quantize_block_e8m0(x: np.ndarray, fmt: int, br: int, bc: int, transpose: bool = False):
    """UE8M0 block scaling: (q, e8m0 bytes [ceil(R/br)][ceil(C/bc)])."""
    x, kind = _input(x)
    R, C = _out_shape(x, transpose)
    q = np.empty((R, C), np.uint8)
    e = np.empty((-(-R // br), -(-C // bc)), np.uint8)
    lib().orc_quantize_block_e8m0(_p(x), kind, x.shape[0], x.shape[1], x.shape[1], fmt, br, bc, int(transpose),
                                  _p(q), C, _p(e))
    return q, e


def scales_f32_to_e8m0(s: np.ndarray):
    """Exact fp32 -> UE8M0 conversion of power-of-two scales: (bytes, count of inexact entries)."""
    s = np.ascontiguousarray(s, np.float32)
    out = np.empty(s.shape, np.uint8)
    bad = lib().orc_scales_f32_to_e8m0(_p(s), s.size, _p(out))
    return out, int(bad)


def quantize_mx(x: np.ndarray, fmt: int, transpose: bool = False):
    x, kind = _input(x)
    R, C = _out_shape(x, transpose)
    q = np.empty((R, C), np.uint8)
    e = np.empty((R, (C + 31) // 32), np.uint8)
    lib().orc_quantize_mx(_p(x), kind, x.shape[0], x.shape[1], x.shape[1], fmt, int(transpose),
                          _p(q), C, _p(e))
    return q, e


def quantize_moss(x: np.ndarray, fmt: int, transpose: bool = False):
    x, kind = _input(x)
    R, C = _out_shape(x, transpose)
    q = np.empty((R, C), np.uint8)
    e = np.empty((R, (C + 31) // 32), np.uint8)
    S = np.zeros(1, np.float32)
    lib().orc_quantize_moss(_p(x), kind, x.shape[0], x.shape[1], x.shape[1], fmt, int(transpose),
                            _p(q), C, _p(e), _p(S))
    return q, e, S[0]


def quantize_moss_given(x: np.ndarray, fmt: int, S: float, transpose: bool = False):
    """MOSS elements and local exponents for a known global factor S (e.g. a row sample)."""
    x, kind = _input(x)
    R, C = _out_shape(x, transpose)
    q = np.empty((R, C), np.uint8)
    e = np.empty((R, (C + 31) // 32), np.uint8)
    lib().orc_quantize_moss_given(_p(x), kind, x.shape[0], x.shape[1], x.shape[1], fmt, int(transpose),
                                  float(S), _p(q), C, _p(e))
    return q, e


# ------------------------------------------------------------------ delayed scaling
def history_roll_insert(hist: np.ndarray, a: float) -> None:
    assert hist.dtype == np.float32 and hist.flags.c_contiguous
    lib().orc_history_roll_insert(_p(hist), hist.size, float(a))


def history_max(hist: np.ndarray) -> np.float32:
    hist = np.ascontiguousarray(hist, np.float32)
    return np.float32(lib().orc_history_max(_p(hist), hist.size))


def delayed_step(x: np.ndarray, fmt: int, scale: np.ndarray, hist: np.ndarray, transpose: bool = False):
    """Flax in-step order: scale from max(history) (previous kept on zero/non-finite), quantize,
    then roll-insert amax(x).  `scale` (shape (1,) fp32) and `hist` are updated in place."""
    x, kind = _input(x)
    assert scale.dtype == np.float32 and hist.dtype == np.float32
    R, C = _out_shape(x, transpose)
    q = np.empty((R, C), np.uint8)
    a = np.zeros(1, np.float32)
    lib().orc_delayed_step(_p(x), kind, x.shape[0], x.shape[1], x.shape[1], fmt, int(transpose),
                           _p(scale), _p(hist), hist.size, _p(q), C, _p(a))
    return q, a[0]


def history_merge(hist_dst: np.ndarray, scale_dst: np.ndarray, hist_src: np.ndarray, scale_src: float) -> None:
    """Combine two branches' updated (history, scale) by elementwise max, in place in *_dst."""
    assert hist_dst.dtype == np.float32 and scale_dst.dtype == np.float32 and hist_dst.flags.c_contiguous
    hs = np.ascontiguousarray(hist_src, np.float32)
    assert hs.size == hist_dst.size
    lib().orc_history_merge(_p(hist_dst), _p(hs), hist_dst.size, _p(scale_dst), float(scale_src))


def auto_scale_step(state: np.ndarray, rescale: bool, amax_now: float, lr: float, fmt: int) -> np.float32:
    """One automatic-scaling step; `state` (fp32[2]: base, learning-rate sum) is updated in place."""
    assert state.dtype == np.float32 and state.size == 2 and state.flags.c_contiguous
    return np.float32(lib().orc_auto_scale_step(_p(state), int(bool(rescale)), float(amax_now), float(lr), fmt))


# ------------------------------------------------------------------ dequant / GEMM / SNR
def dequantize(mode: int, q: np.ndarray, fmt: int, scales=None, global_scale=None,
               block=(1, 128)) -> np.ndarray:
    """fp64 dequantized operand (rows x K): q times its scale(s), exact."""
    q = np.ascontiguousarray(q, np.uint8)
    rows, K = q.shape
    out = np.empty((rows, K), np.float64)
    g = np.array([1.0 if global_scale is None else global_scale], np.float32)
    if mode == BLOCK:
        sc = np.ascontiguousarray(scales, np.float32)
    elif mode in (MX, MOSS, BLOCK_E8M0):
        sc = np.ascontiguousarray(scales, np.uint8)
    else:
        sc = np.zeros(1, np.float32)
    lib().orc_dequantize(mode, _p(q), fmt, rows, K, K, _p(sc), block[0], block[1], _p(g), _p(out))
    return out


def block_dequantize(mode: int, q: np.ndarray, fmt: int, scales: np.ndarray, block=(128, 128), out_bf16: bool = True):
    """fl32(decode(q) * block scale), optionally rounded to bf16 (returned as uint16 bit patterns)."""
    q = np.ascontiguousarray(q, np.uint8)
    rows, K = q.shape
    sc = np.ascontiguousarray(scales, np.uint8 if mode == BLOCK_E8M0 else np.float32)
    out = np.empty((rows, K), np.uint16 if out_bf16 else np.float32)
    lib().orc_block_dequantize(mode, _p(q), fmt, rows, K, K, _p(sc), block[0], block[1], int(bool(out_bf16)), _p(out))
    return out


def gemm_ref(A: np.ndarray, B: np.ndarray, pairs: np.ndarray | None = None):
    """fp64 C = A @ B.T and D = |A| @ |B|.T over dequantized operands (rows x K each).
    With `pairs` (n x 2 int64 of (m, n)), only those entries are returned (1-D)."""
    A = np.ascontiguousarray(A, np.float64)
    B = np.ascontiguousarray(B, np.float64)
    M, K = A.shape
    N, K2 = B.shape
    assert K == K2
    if pairs is None:
        C = np.empty((M, N), np.float64)
        D = np.empty((M, N), np.float64)
        lib().orc_gemm_ref(_p(A), _p(B), M, N, K, None, 0, _p(C), _p(D))
        return C, D
    pairs = np.ascontiguousarray(pairs, np.int64)
    n = pairs.shape[0]
    C = np.empty(n, np.float64)
    D = np.empty(n, np.float64)
    lib().orc_gemm_ref(_p(A), _p(B), M, N, K, _p(pairs), n, _p(C), _p(D))
    return C, D


def gemm_ref_terms(A: np.ndarray, B: np.ndarray, pairs: np.ndarray | None = None, chunk: int = 128):
    """gemm_ref's C and D plus the error-size sums of a K-chunked accumulation: E (per chunk the
    largest |product|, summed) and Sigma (per chunk |sum of all earlier chunks|, summed).
    Returns (C, D, E, Sigma), full matrices or 1-D over `pairs`."""
    A = np.ascontiguousarray(A, np.float64)
    B = np.ascontiguousarray(B, np.float64)
    M, K = A.shape
    N, K2 = B.shape
    assert K == K2 and chunk > 0
    if pairs is None:
        out = [np.empty((M, N), np.float64) for _ in range(4)]
        lib().orc_gemm_ref_terms(_p(A), _p(B), M, N, K, chunk, None, 0, *(_p(o) for o in out))
        return tuple(out)
    pairs = np.ascontiguousarray(pairs, np.int64)
    assert pairs.ndim == 2 and pairs.shape[1] == 2
    assert pairs.size == 0 or (pairs[:, 0].min() >= 0 and pairs[:, 0].max() < M and pairs[:, 1].min() >= 0
                               and pairs[:, 1].max() < N)
    n = pairs.shape[0]
    out = [np.empty(n, np.float64) for _ in range(4)]
    lib().orc_gemm_ref_terms(_p(A), _p(B), M, N, K, chunk, _p(pairs), n, *(_p(o) for o in out))
    return tuple(out)


def snr_db(x: np.ndarray, xhat: np.ndarray) -> float:
    x = np.ascontiguousarray(x, np.float32)
    xhat = np.ascontiguousarray(xhat, np.float64)
    assert x.size == xhat.size
    return float(lib().orc_snr_db(_p(x), _p(xhat), x.size))
