"""FP8 quantize-then-scaled-GEMM for AMD MI355X (gfx950): C ABI library + thin Python binding.

The compute path is libfp8q.so (hand-written HIP kernels); see include/fp8q.h for the ABI.  The
binding is imported on first use of any library name, and raises ImportError if the library has
not been built: there is no fallback path.  `workloads` (seeded synthetic inputs) imports without it.
"""
_LIB_NAMES = ("BLOCK", "BLOCK_E8M0", "E4M3", "E5M2", "IN_BF16", "IN_F32", "MOSS", "MX", "OUT_BF16", "OUT_F32",
              "TENSOR", "Fp8qError", "fp8_amax", "fp8_history_update", "fp8_quantize", "fp8_quantize_dual",
              "fp8_scaled_gemm", "fp8_history_merge", "fp8_auto_scale", "fp8_scale_to_e8m0", "fp8_block_dequantize",
              "init", "quantize", "quantize_dual", "scaled_gemm", "scale_to_e8m0", "block_dequantize")

__all__ = list(_LIB_NAMES)


def __getattr__(name):
    if name in _LIB_NAMES:
        from . import _lib
        return getattr(_lib, name)
    raise AttributeError(name)
