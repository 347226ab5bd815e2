"""The Python binding rejects buffers whose shape, dtype or device does not match what the call
will read or write, before any pointer reaches the C ABI (which cannot see buffer sizes).  These
run on the CPU: every rejection happens before a device is touched, and buffers with the right
shapes but on the host are refused for not being on a GPU."""
import pytest
import torch

import fp8_scaled_quantization_amd as fq

u8, f32, bf16, i32 = torch.uint8, torch.float32, torch.bfloat16, torch.int32


def z(shape, dt):
    return torch.zeros(shape, dtype=dt)


def _raises(fn, text):
    with pytest.raises(ValueError, match=text):
        fn()


def test_gemm_rejects_output_dtype_and_shape():
    A, B = z((256, 512), u8), z((128, 512), u8)
    s = z(1, f32)
    _raises(lambda: fq.fp8_scaled_gemm(fq.TENSOR, A, 0, None, B, 0, None, s, s, z((256, 128), bf16), fq.OUT_F32),
            "C must be torch.float32")
    _raises(lambda: fq.fp8_scaled_gemm(fq.TENSOR, A, 0, None, B, 0, None, s, s, z((256, 128), f32), fq.OUT_BF16),
            "C must be torch.bfloat16")
    _raises(lambda: fq.fp8_scaled_gemm(fq.TENSOR, A, 0, None, B, 0, None, s, s, z((128, 256), f32), fq.OUT_F32),
            r"C must have shape \(256, 128\)")
    _raises(lambda: fq.fp8_scaled_gemm(fq.TENSOR, A, 0, None, z((128, 256), u8), 0, None, s, s, z((256, 128), f32),
                                       fq.OUT_F32), "B must be N x K")
    _raises(lambda: fq.fp8_scaled_gemm(fq.TENSOR, A, 0, None, B, 0, None, s, s, z((256, 128), f32), 7),
            "out_dtype")
    _raises(lambda: fq.fp8_scaled_gemm(fq.TENSOR, A.float(), 0, None, B, 0, None, s, s, z((256, 128), f32),
                                       fq.OUT_F32), "A must be torch.uint8")
    _raises(lambda: fq.fp8_scaled_gemm(fq.TENSOR, A.t(), 0, None, B, 0, None, s, s, z((512, 128), f32), fq.OUT_F32),
            "row-major")


def test_gemm_rejects_scale_arrays():
    A, B = z((256, 512), u8), z((128, 512), u8)
    C = z((256, 128), bf16)
    s = z(1, f32)
    # MX: u8 [rows][K/32]
    _raises(lambda: fq.fp8_scaled_gemm(fq.MX, A, 0, z((256, 8), u8), B, 0, z((128, 16), u8), None, None, C,
                                       fq.OUT_BF16), r"Ascale must have shape \(256, 16\)")
    _raises(lambda: fq.fp8_scaled_gemm(fq.MOSS, A, 0, z((256, 16), u8), B, 0, z((128, 16), f32), s, s, C,
                                       fq.OUT_BF16), "Bscale must be torch.uint8")
    _raises(lambda: fq.fp8_scaled_gemm(fq.MOSS, A, 0, z((256, 16), u8), B, 0, z((128, 16), u8), None, s, C,
                                       fq.OUT_BF16), "Aglobal")
    # BLOCK: fp32 [M][K/128] and [N/128][K/128]
    _raises(lambda: fq.fp8_scaled_gemm(fq.BLOCK, A, 0, z((256, 4), u8), B, 0, z((1, 4), f32), None, None, C,
                                       fq.OUT_BF16), "Ascale must be torch.float32")
    _raises(lambda: fq.fp8_scaled_gemm(fq.BLOCK, A, 0, z((256, 4), f32), B, 0, z((2, 4), f32), None, None, C,
                                       fq.OUT_BF16), r"Bscale must have shape \(1, 4\)")
    _raises(lambda: fq.fp8_scaled_gemm(fq.BLOCK_E8M0, A, 0, z((256, 4), f32), B, 0, z((1, 4), f32), None, None, C,
                                       fq.OUT_BF16), "Bscale must be torch.uint8")
    _raises(lambda: fq.fp8_scaled_gemm(fq.BLOCK, A, 0, z((4, 256), f32).t(), B, 0, z((1, 4), f32), None, None, C,
                                       fq.OUT_BF16), "Ascale must be contiguous")
    # static activations need the per-tensor scale
    _raises(lambda: fq.fp8_scaled_gemm(fq.BLOCK, A, 0, None, B, 0, z((1, 4), f32), None, None, C, fq.OUT_BF16),
            "static activation")


def test_quantize_rejects_outputs():
    x = z((64, 256), bf16)
    _raises(lambda: fq.fp8_quantize(fq.MX, 0, x, z((64, 256), u8), z((64, 4), u8), transpose_out=True),
            r"q must have shape \(256, 64\)")
    _raises(lambda: fq.fp8_quantize(fq.MX, 0, x, z((64, 256), u8), z((64, 4), u8)), r"scales must have shape \(64, 8\)")
    _raises(lambda: fq.fp8_quantize(fq.BLOCK, 0, x, z((64, 256), u8), z((64, 2), u8), block=(1, 128)),
            "scales must be torch.float32")
    _raises(lambda: fq.fp8_quantize(fq.BLOCK, 0, x, z((64, 256), u8), z((64, 2), f32), block=(0, 128)),
            "block must be two positive integers")
    _raises(lambda: fq.fp8_quantize(fq.TENSOR, 0, x, z((64, 256), f32), None, z(1, f32), True), "q must be torch.uint8")
    _raises(lambda: fq.fp8_quantize(fq.TENSOR, 0, x, z((64, 256), u8), None, z(1, f32), False, None),
            "amax_out is required")
    _raises(lambda: fq.fp8_quantize(fq.MOSS, 0, x, z((64, 256), u8), z((64, 8), u8), z(1, bf16), True),
            "tensor_scale must be float32")
    _raises(lambda: fq.fp8_quantize(fq.TENSOR, 0, x.int(), z((64, 256), u8), None, z(1, f32), True), "x must be")


def test_quantize_dual_and_others_reject():
    x = z((64, 256), bf16)
    _raises(lambda: fq.fp8_quantize_dual(fq.MX, 0, x, z((64, 256), u8), z((64, 8), u8), z((64, 256), u8),
                                         z((256, 2), u8)), r"qt must have shape \(256, 64\)")
    _raises(lambda: fq.fp8_quantize_dual(fq.MX, 0, x, z((64, 256), u8), z((64, 8), u8), z((256, 64), u8),
                                         z((256, 1), u8)), r"scales_t must have shape \(256, 2\)")
    _raises(lambda: fq.fp8_quantize_dual(fq.BLOCK, 0, x, z((64, 256), u8), None, z((256, 64), u8), None), "mode")
    _raises(lambda: fq.fp8_block_dequantize(fq.BLOCK, 0, z((256, 256), u8), z((2, 2), f32), z((256, 128), bf16)),
            r"out must have shape \(256, 256\)")
    _raises(lambda: fq.fp8_block_dequantize(fq.BLOCK_E8M0, 0, z((256, 256), u8), z((2, 2), f32), z((256, 256), bf16)),
            "scales must be torch.uint8")
    _raises(lambda: fq.fp8_history_update(z(1024, i32), z(1, f32), z(1, f32), 0), "history must be float32")
    _raises(lambda: fq.fp8_auto_scale(z(1, f32), False, None, 1e-4, 0, z(1, f32)), "state must hold at least 2")
    _raises(lambda: fq.fp8_auto_scale(z(2, f32), True, None, 1e-4, 0, z(1, f32)), "amax_now")
    _raises(lambda: fq.fp8_history_merge(z(1024, f32), z(512, f32), z(1, f32), z(1, f32)), "differ in length")
    _raises(lambda: fq.fp8_scale_to_e8m0(z(16, f32), z(8, u8), z(1, i32)), "e8m0 must be")
    _raises(lambda: fq.fp8_amax(x, z(1, bf16)), "amax_out must be float32")


def test_correct_shapes_on_the_host_are_refused_as_not_on_a_gpu():
    A, B = z((256, 512), u8), z((128, 512), u8)
    s = z(1, f32)
    _raises(lambda: fq.fp8_scaled_gemm(fq.TENSOR, A, 0, None, B, 0, None, s, s, z((256, 128), f32), fq.OUT_F32),
            "on a GPU")
    _raises(lambda: fq.fp8_quantize(fq.MX, 0, z((64, 256), bf16), z((64, 256), u8), z((64, 8), u8)), "on a GPU")
    _raises(lambda: fq.fp8_amax(z((64, 256), bf16), z(1, f32)), "on a GPU")
