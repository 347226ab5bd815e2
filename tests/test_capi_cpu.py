"""CPU checks of the C ABI library: it loads, exports every entry point declared in include/fp8q.h,
and rejects invalid arguments with the documented status codes before touching a device."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def L():
    from fp8_scaled_quantization_amd import _lib
    return _lib


def test_exports_match_header(L):
    hdr = open(os.path.join(ROOT, "include", "fp8q.h")).read()
    declared = set(re.findall(r"^(?:int|const char\*)\s+(\w+)\(", hdr, re.M))
    assert declared == set(L.EXPORTS)
    for name in declared:
        assert hasattr(L.lib(), name)


def _err(L):
    return L.lib().fp8q_last_error().decode()


def test_invalid_arguments(L):
    lib = L.lib()
    dummy = ctypes.c_void_p(16)
    # unknown mode / format / dtype
    assert lib.fp8_quantize(7, 0, dummy, 1, 4, 8, 8, 1, 128, 0, dummy, 16, dummy, dummy, 1, None, None) == L.ERR_INVALID_ARG
    assert "mode" in _err(L)
    assert lib.fp8_quantize(0, 5, dummy, 1, 4, 8, 8, 1, 128, 0, dummy, 16, dummy, dummy, 1, None, None) == L.ERR_INVALID_ARG
    assert lib.fp8_quantize(0, 0, dummy, 9, 4, 8, 8, 1, 128, 0, dummy, 16, dummy, dummy, 1, None, None) == L.ERR_INVALID_ARG
    # block sizes must be two positive integers
    assert lib.fp8_quantize(1, 0, dummy, 1, 4, 8, 8, 0, 128, 0, dummy, 16, dummy, None, 0, None, None) == L.ERR_INVALID_ARG
    assert "positive" in _err(L)
    # derived scale needs amax_out; TENSOR needs tensor_scale
    assert lib.fp8_quantize(0, 0, dummy, 1, 4, 8, 8, 1, 128, 0, dummy, 16, None, dummy, 0, None, None) == L.ERR_INVALID_ARG
    assert lib.fp8_quantize(0, 0, dummy, 1, 4, 8, 8, 1, 128, 0, dummy, 16, None, None, 1, None, None) == L.ERR_INVALID_ARG
    # alignment / multiples outside the kernels' limits
    assert lib.fp8_quantize(0, 0, dummy, 1, 4, 12, 12, 1, 128, 0, dummy, 16, None, dummy, 1, None, None) == L.ERR_UNSUPPORTED
    # dual cast: BLOCK is not a dual mode; NULL qt; a derived scale needs amax_out
    d = lib.fp8_quantize_dual
    assert d(1, 0, dummy, 1, 32, 32, 32, dummy, 32, dummy, dummy, 32, dummy, dummy, 1, None, None) == L.ERR_INVALID_ARG
    assert "mode" in _err(L)
    assert d(2, 0, dummy, 1, 32, 32, 32, dummy, 32, dummy, None, 32, dummy, None, 0, None, None) == L.ERR_INVALID_ARG
    assert d(3, 0, dummy, 1, 32, 32, 32, dummy, 32, dummy, dummy, 32, dummy, dummy, 0, None, None) == L.ERR_INVALID_ARG
    assert d(3, 0, dummy, 1, 32, 32, 32, dummy, 16, dummy, dummy, 32, dummy, dummy, 1, None, None) == L.ERR_INVALID_ARG
    # ld smaller than cols
    assert lib.fp8_amax(dummy, 1, 4, 16, 8, dummy, None) == L.ERR_INVALID_ARG
    # history length bounds
    assert lib.fp8_history_update(dummy, 0, dummy, dummy, 0, None) == L.ERR_INVALID_ARG
    assert lib.fp8_history_update(dummy, 5000, dummy, dummy, 0, None) == L.ERR_INVALID_ARG
    # GEMM: out_dtype is required, globals for TENSOR, scales for MX
    g = lib.fp8_scaled_gemm
    assert g(0, dummy, 0, None, dummy, 0, None, dummy, dummy, 16, 16, 32, 32, 32, dummy, 7, 16, None) == L.ERR_INVALID_ARG
    assert "out_dtype" in _err(L)
    assert g(0, dummy, 0, None, dummy, 0, None, None, None, 16, 16, 32, 32, 32, dummy, 0, 16, None) == L.ERR_INVALID_ARG
    assert g(2, dummy, 0, None, dummy, 0, None, None, None, 16, 16, 32, 32, 32, dummy, 0, 16, None) == L.ERR_INVALID_ARG
    assert g(0, dummy, 0, None, dummy, 0, None, dummy, dummy, 16, 16, 24, 32, 32, dummy, 0, 16, None) == L.ERR_UNSUPPORTED
    # BLOCK_E8M0 is a quantize and GEMM mode, not a dual mode; static activations need Aglobal
    assert lib.fp8_quantize(4, 0, dummy, 1, 4, 8, 8, 128, 0, 0, dummy, 16, dummy, None, 0, None, None) == L.ERR_INVALID_ARG
    assert d(4, 0, dummy, 1, 32, 32, 32, dummy, 32, dummy, dummy, 32, dummy, dummy, 1, None, None) == L.ERR_INVALID_ARG
    assert g(4, dummy, 0, None, dummy, 0, dummy, None, None, 16, 16, 128, 128, 128, dummy, 0, 16, None) == L.ERR_INVALID_ARG
    assert g(5, dummy, 0, dummy, dummy, 0, dummy, None, None, 16, 16, 128, 128, 128, dummy, 0, 16, None) == L.ERR_INVALID_ARG


def test_next_entry_points_reject_bad_arguments(L):
    lib = L.lib()
    dummy = ctypes.c_void_p(16)
    assert lib.fp8_history_merge(dummy, dummy, -1, dummy, dummy, None) == L.ERR_INVALID_ARG
    assert lib.fp8_history_merge(None, dummy, 8, dummy, dummy, None) == L.ERR_INVALID_ARG
    assert lib.fp8_auto_scale(dummy, 1, None, ctypes.c_float(1e-3), 0, dummy, None) == L.ERR_INVALID_ARG
    assert lib.fp8_auto_scale(dummy, 0, None, ctypes.c_float(-1.0), 0, dummy, None) == L.ERR_INVALID_ARG
    assert "learning rate" in _err(L)
    assert lib.fp8_auto_scale(dummy, 2, dummy, ctypes.c_float(1e-3), 0, dummy, None) == L.ERR_INVALID_ARG
    assert lib.fp8_auto_scale(dummy, 0, None, ctypes.c_float(1e-3), 3, dummy, None) == L.ERR_INVALID_ARG
    assert lib.fp8_scale_to_e8m0(dummy, 4, dummy, None, None) == L.ERR_INVALID_ARG
    bd = lib.fp8_block_dequantize
    assert bd(2, 0, dummy, 128, 128, 128, dummy, 128, 128, dummy, 1, 128, None) == L.ERR_INVALID_ARG
    assert bd(1, 0, dummy, 128, 128, 128, dummy, 0, 128, dummy, 1, 128, None) == L.ERR_INVALID_ARG
    assert bd(1, 0, dummy, 128, 128, 128, dummy, 128, 128, dummy, 5, 128, None) == L.ERR_INVALID_ARG
    assert bd(4, 0, dummy, 128, 128, 64, dummy, 128, 128, dummy, 1, 128, None) == L.ERR_INVALID_ARG


def test_null_pointers_rejected_at_extents_whose_product_overflows(L):
    """Extents of 2^32 x 2^32 multiply to 2^64, which wraps to 0 in 64-bit arithmetic: the NULL
    checks compare each extent with zero, so such a call is still rejected as invalid."""
    lib = L.lib()
    dummy = ctypes.c_void_p(16)
    big = 1 << 32
    g = lib.fp8_scaled_gemm
    assert g(0, dummy, 0, None, dummy, 0, None, dummy, dummy, big, big, 32, 32, 32, None, 0, big, None) == L.ERR_INVALID_ARG
    assert "NULL C" in _err(L)
    assert g(0, None, 0, None, None, 0, None, dummy, dummy, big, big, 32, 32, 32, dummy, 0, big, None) == L.ERR_INVALID_ARG
    assert "NULL A or B" in _err(L)
    assert lib.fp8_amax(None, 1, big, big, big, dummy, None) == L.ERR_INVALID_ARG
    assert lib.fp8_quantize(0, 0, None, 1, big, big, big, 1, 128, 0, None, big, None, dummy, 1, None, None) == L.ERR_INVALID_ARG
    assert "NULL x or q" in _err(L)
    bd = lib.fp8_block_dequantize
    assert bd(1, 0, None, big, big, big, None, 128, 128, None, 1, big, None) == L.ERR_INVALID_ARG
