"""GPU parity of the scaled FP8 GEMM against the oracle's fp64 product of the same quantized
operands, with the elementwise bound derived in tests/gpu_util.py: full comparison on small and
ragged shapes (several tiles and partial tiles), and at the workloads' full shapes, in the launch
configuration the benchmark times, every output of the fine-grained, MXFP8 and MOSS products
(tests/gpu_util.check_gemm_large)."""
import numpy as np
import pytest
import torch

from fp8_scaled_quantization_amd import workloads
from tests.gpu_util import DEV, check_gemm, check_gemm_large, host, reference_terms, sample_pairs, to_dev

pytestmark = pytest.mark.gpu

E4M3, E5M2 = 0, 1
TENSOR, BLOCK, MX, MOSS = 0, 1, 2, 3
OUT_F32, OUT_BF16 = 0, 1


@pytest.fixture(scope="module")
def fq():
    import fp8_scaled_quantization_amd as fq
    fq.init()
    return fq


def _quant_operand(fq, orc, x, mode, fmt, block, transpose=False, S=None):
    """Quantize on the GPU; return device tensors and the oracle's fp64 dequantized operand built
    from the GPU's bytes and scales (the casts themselves are checked bit-exactly elsewhere)."""
    xd = to_dev(x)
    if mode == MOSS and S is not None:
        q, sc, g, _ = fq.quantize(xd, mode, fmt, transpose_out=transpose, tensor_scale=S, scale_is_input=True)
    else:
        q, sc, g, _ = fq.quantize(xd, mode, fmt, block=block or (1, 128), transpose_out=transpose)
    hq = host(q)
    hs = host(sc) if sc is not None else None
    hg = np.float32(host(g)[0]) if g is not None else None
    return (q, sc, g), (hq, hs, hg)


def _deq(orc, mode, hq, hs, hg, fmt, block):
    return orc.dequantize(mode, hq, fmt, hs, hg, block=block)


def _run(fq, mode, A, afmt, B, bfmt, out):
    (qa, sa, ga), (qb, sb, gb) = A, B
    return fq.scaled_gemm(mode, qa, afmt, sa, qb, bfmt, sb, ga, gb, out_dtype=out)


SMALL = [(200, 136, 384), (128, 128, 128), (256, 384, 1024), (16, 64, 32), (300, 260, 272), (600, 400, 1152)]


@pytest.mark.parametrize("mode", [TENSOR, BLOCK, MX, MOSS])
@pytest.mark.parametrize("M,N,K", SMALL)
@pytest.mark.parametrize("fmts", [(E4M3, E4M3), (E5M2, E4M3), (E4M3, E5M2)])
def test_gemm_small_full(fq, orc, mode, M, N, K, fmts):
    if mode == BLOCK and K % 128:
        K = (K + 127) // 128 * 128
    afmt, bfmt = fmts
    xa = workloads.random_matrix(M * 3 + K, M, K, 2.0)
    xb = workloads.random_matrix(N * 5 + K, N, K, 0.05)
    ba, bb = ((1, 128), (128, 128)) if mode == BLOCK else ((1, 128), (1, 128))
    A, (hqa, hsa, hga) = _quant_operand(fq, orc, xa, mode, afmt, ba)
    B, (hqb, hsb, hgb) = _quant_operand(fq, orc, xb, mode, bfmt, bb)
    Ad = _deq(orc, mode, hqa, hsa, hga, afmt, ba)
    Bd = _deq(orc, mode, hqb, hsb, hgb, bfmt, bb)
    Cref, D, E, Sg = reference_terms(orc, Ad, Bd, promoted=mode == BLOCK)
    C32 = host(_run(fq, mode, A, afmt, B, bfmt, OUT_F32))
    Cbf = host(_run(fq, mode, A, afmt, B, bfmt, OUT_BF16))
    check_gemm(C32, Cbf, Cref, D, E, K, "mode %d %dx%dx%d" % (mode, M, N, K), Sg)


def test_gemm_per_tensor_small_exact_config(fq, orc):
    """16x32 @ 32x64 fp32 U[0,1), fp32 out: all products are non-negative, so D = |C_ref| and the
    elementwise relative error is held to 1e-5 outright, besides the general bound."""
    a, b = workloads.per_tensor_inputs()
    A, (hqa, _, hga) = _quant_operand(fq, orc, a, TENSOR, E4M3, None)
    B, (hqb, _, hgb) = _quant_operand(fq, orc, b, TENSOR, E4M3, None, transpose=True)
    Ad = orc.dequantize(TENSOR, hqa, E4M3, None, hga)
    Bd = orc.dequantize(TENSOR, hqb, E4M3, None, hgb)
    Cref, D, E, Sg = reference_terms(orc, Ad, Bd)
    C32 = host(_run(fq, TENSOR, A, E4M3, B, E4M3, OUT_F32))
    worst = check_gemm(C32, None, Cref, D, E, 32, "16x32x64", Sg)
    assert np.allclose(D, np.abs(Cref))
    rel = float(np.max(np.abs(C32 - Cref) / np.abs(Cref)))
    print("16x32x64 fp32 out: max elementwise relative error %.3g" % rel)
    assert rel <= 1e-5 and worst <= 1.0


def test_gemm_delayed_step_full(fq, orc):
    """One delayed-scaling step at 1024x2048 @ 2048x1024, full output comparison."""
    Araw, Braw, _ = workloads.delayed_inputs(3)
    A, (hqa, _, hga) = _quant_operand(fq, orc, Araw, TENSOR, E4M3, None)
    B, (hqb, _, hgb) = _quant_operand(fq, orc, Braw, TENSOR, E4M3, None, transpose=True)
    Ad = orc.dequantize(TENSOR, hqa, E4M3, None, hga)
    Bd = orc.dequantize(TENSOR, hqb, E4M3, None, hgb)
    Cref, D, E, Sg = reference_terms(orc, Ad, Bd)
    C32 = host(_run(fq, TENSOR, A, E4M3, B, E4M3, OUT_F32))
    Cbf = host(_run(fq, TENSOR, A, E4M3, B, E4M3, OUT_BF16))
    check_gemm(C32, Cbf, Cref, D, E, 2048, "delayed 1024x1024x2048", Sg)


def _sampled_check(fq, orc, mode, A, afmt, B, bfmt, deqA, deqB, M, N, K, seed, label):
    pairs = sample_pairs(M, N, 2048, seed)
    rows = np.unique(pairs[:, 0])
    cols = np.unique(pairs[:, 1])
    Ad = deqA(rows)
    Bd = deqB(cols)
    ri = np.searchsorted(rows, pairs[:, 0])
    ci = np.searchsorted(cols, pairs[:, 1])
    local = np.stack([ri, ci], 1).astype(np.int64)
    Cref, D, E, Sg = reference_terms(orc, Ad, Bd, local, promoted=mode == BLOCK)
    C32 = _run(fq, mode, A, afmt, B, bfmt, OUT_F32)
    Cbf = _run(fq, mode, A, afmt, B, bfmt, OUT_BF16)
    c32 = host(C32)[pairs[:, 0], pairs[:, 1]]
    cbf = host(Cbf)[pairs[:, 0], pairs[:, 1]]
    return check_gemm(c32, cbf, Cref, D, E, K, label, Sg)


def _rows_deq(orc, mode, hq, hs, hg, fmt, block):
    """Dequantize a subset of rows: block scales are expanded per row first."""
    def f(rows):
        q = np.ascontiguousarray(hq[rows])
        if mode == BLOCK:
            s = np.ascontiguousarray(hs[rows // block[0]])
            return orc.dequantize(BLOCK, q, fmt, s, None, block=(1, block[1]))
        if mode in (MX, MOSS):
            return orc.dequantize(mode, q, fmt, np.ascontiguousarray(hs[rows]), hg)
        return orc.dequantize(TENSOR, q, fmt, None, hg)
    return f


def _large_check(fq, orc, mode, A, afmt, B, bfmt, deqA, deqB, M, N, K, seed, label, full=True):
    C32 = _run(fq, mode, A, afmt, B, bfmt, OUT_F32)
    Cbf = _run(fq, mode, A, afmt, B, bfmt, OUT_BF16)
    return check_gemm_large(orc, C32, Cbf, deqA, deqB, M, N, K, seed, label, promoted=mode == BLOCK, full=full)


def test_gemm_fine_grained_full_size(fq, orc):
    X, W = workloads.fine_grained_inputs()
    A, (hqa, hsa, _) = _quant_operand(fq, orc, X, BLOCK, E4M3, (1, 128))
    B, (hqb, hsb, _) = _quant_operand(fq, orc, W, BLOCK, E4M3, (128, 128))
    _large_check(fq, orc, BLOCK, A, E4M3, B, E4M3, _rows_deq(orc, BLOCK, hqa, hsa, None, E4M3, (1, 128)),
                 _rows_deq(orc, BLOCK, hqb, hsb, None, E4M3, (128, 128)), 4096, 2048, 7168, 3, "fine-grained")


def test_gemm_mx_full_size(fq, orc):
    Araw, Braw = workloads.mx_inputs()
    A, (hqa, hsa, _) = _quant_operand(fq, orc, Araw, MX, E4M3, None)
    B, (hqb, hsb, _) = _quant_operand(fq, orc, Braw, MX, E4M3, None)
    _large_check(fq, orc, MX, A, E4M3, B, E4M3, _rows_deq(orc, MX, hqa, hsa, None, E4M3, None),
                 _rows_deq(orc, MX, hqb, hsb, None, E4M3, None), 8192, 8192, 8192, 4, "mx 8192^3")


@pytest.fixture(scope="module")
def moss_operands(fq, orc):
    """The MOSS workload's six quantized copies (device) with their host bytes and scales."""
    X, W, dY = workloads.moss_inputs()
    o = {}
    o["X"] = _quant_operand(fq, orc, X, MOSS, E4M3, None)
    o["W"] = _quant_operand(fq, orc, W, MOSS, E4M3, None)
    o["G"] = _quant_operand(fq, orc, dY, MOSS, E5M2, None)
    o["XT"] = _quant_operand(fq, orc, X, MOSS, E4M3, None, transpose=True, S=o["X"][0][2])
    o["WT"] = _quant_operand(fq, orc, W, MOSS, E4M3, None, transpose=True, S=o["W"][0][2])
    o["GT"] = _quant_operand(fq, orc, dY, MOSS, E5M2, None, transpose=True, S=o["G"][0][2])
    yield o
    o.clear()
    torch.cuda.empty_cache()


# Y = X W^T; dX = dY W (B = W^T, grouped along out); dW = dY^T X (A = dY^T, B = X^T, grouped along
# tokens).  Every output of each product at the workload's size.
@pytest.mark.parametrize("gemm", ["Y", "dX", "dW"])
def test_gemm_moss_forward_backward_full_size(fq, orc, moss_operands, gemm):
    a, af, b, bf, M, N, K, seed = {"Y": ("X", E4M3, "W", E4M3, 16384, 4096, 4096, 51),
                                   "dX": ("G", E5M2, "WT", E4M3, 16384, 4096, 4096, 52),
                                   "dW": ("GT", E5M2, "XT", E4M3, 4096, 4096, 16384, 53)}[gemm]
    # (the transposed copies were cast with the row-grouped copy's global scale, which they return)
    (Aq, (ha, has_, hag)), (Bq, (hb, hbs, hbg)) = moss_operands[a], moss_operands[b]
    _large_check(fq, orc, MOSS, Aq, af, Bq, bf, _rows_deq(orc, MOSS, ha, has_, hag, af, None),
                 _rows_deq(orc, MOSS, hb, hbs, hbg, bf, None), M, N, K, seed, "moss " + gemm)


# Shapes with enough 256 x 256 tiles (>= 192) to take the ping-pong kernel, with partial tiles in
# M and N and K of one, two and five 128-wide steps (the copy pipeline's start-up and drain cases).
# 256 x 256 ping-pong kernel (at least 192 tiles of 256 x 256), then the 256 x 128 one (fewer, but at
# least 192 tiles of 256 x 128), with partial tiles and a partial last scale quad.  The last three
# have more 256 x 256 tiles than a GPU has CUs, so workgroups loop over tiles: 288 tiles with
# partial ones in M and N, 1024 partial-edged tiles of one K step and 1024 full tiles of two K steps
# (each tile's pipeline fill goes out before the previous tile's stores).
PINGPONG = [(3000, 4000, 128), (3000, 4000, 256), (2900, 4100, 640), (2900, 2100, 640), (4096, 2048, 1152),
            (4000, 4500, 384), (8000, 8000, 128), (8192, 8192, 256)]


@pytest.mark.parametrize("mode", [TENSOR, MX, MOSS])
def test_gemm_persistent_full(fq, orc, mode):
    """Every output of a problem whose 272 tiles of 256 x 256 (17 x 16, the last row and column of
    tiles partial) exceed the GPU's CUs, so that workgroups loop over tiles, compared in full."""
    M, N, K = 4200, 4000, 256
    xa = workloads.random_matrix(71, M, K, 2.0)
    xb = workloads.random_matrix(72, N, K, 0.05)
    A, (hqa, hsa, hga) = _quant_operand(fq, orc, xa, mode, E4M3, None)
    B, (hqb, hsb, hgb) = _quant_operand(fq, orc, xb, mode, E4M3, None)
    Ad = _deq(orc, mode, hqa, hsa, hga, E4M3, (1, 128))
    Bd = _deq(orc, mode, hqb, hsb, hgb, E4M3, (1, 128))
    Cref, D, E, Sg = reference_terms(orc, Ad, Bd)
    C32 = host(_run(fq, mode, A, E4M3, B, E4M3, OUT_F32))
    Cbf = host(_run(fq, mode, A, E4M3, B, E4M3, OUT_BF16))
    check_gemm(C32, Cbf, Cref, D, E, K, "persistent mode %d %dx%dx%d" % (mode, M, N, K), Sg)


@pytest.mark.parametrize("mode", [TENSOR, MX, MOSS])
@pytest.mark.parametrize("M,N,K", [(4200, 4000, 1536), (4096, 4608, 1024)])
def test_gemm_stream_full(fq, orc, mode, M, N, K):
    """Every output of problems run by the streaming 256 x 256 kernel (more tiles than CUs, K steps
    a multiple of 4 and at least 8): 272 tiles with partial ones in M and N, so that some
    workgroups run two tiles and the rest one, with 12 K steps (an odd number of scale quads per
    tile, so the quad ring entry alternates from tile to tile); and 288 full tiles of 8 K steps."""
    xa = workloads.random_matrix(M + 3 * K, M, K, 2.0)
    xb = workloads.random_matrix(N + 5 * K, N, K, 0.05)
    A, (hqa, hsa, hga) = _quant_operand(fq, orc, xa, mode, E4M3, None)
    B, (hqb, hsb, hgb) = _quant_operand(fq, orc, xb, mode, E4M3, None)
    Ad = _deq(orc, mode, hqa, hsa, hga, E4M3, (1, 128))
    Bd = _deq(orc, mode, hqb, hsb, hgb, E4M3, (1, 128))
    Cref, D, E, Sg = reference_terms(orc, Ad, Bd)
    C32 = host(_run(fq, mode, A, E4M3, B, E4M3, OUT_F32))
    Cbf = host(_run(fq, mode, A, E4M3, B, E4M3, OUT_BF16))
    check_gemm(C32, Cbf, Cref, D, E, K, "stream mode %d %dx%dx%d" % (mode, M, N, K), Sg)


@pytest.mark.parametrize("mode", [TENSOR, MX, MOSS])
@pytest.mark.parametrize("M,N,K,fmts", [(2048, 2048, 128, (E4M3, E4M3)), (2000, 2100, 384, (E4M3, E4M3)),
                                        (2048, 2048, 1152, (E5M2, E4M3))])
def test_gemm_pipelined_mid_tiles_full(fq, orc, mode, M, N, K, fmts):
    """Every output of problems run by the pipelined kernel's 128 x 128 tiles (at least 256 of them,
    fewer than 192 of 256 x 128): in TENSOR mode its ring has 4 stages and the wait before a K step
    lets the next min(2, steps left) steps' loads stay in flight, so 1, 3 and 9 K steps cover every
    count; MX/MOSS take the 3-stage scale-quad schedule.  2000 x 2100 has partial tiles in M and N."""
    afmt, bfmt = fmts
    xa = workloads.random_matrix(M + 13 * K, M, K, 2.0)
    xb = workloads.random_matrix(N + 17 * K, N, K, 0.05)
    A, (hqa, hsa, hga) = _quant_operand(fq, orc, xa, mode, afmt, None)
    B, (hqb, hsb, hgb) = _quant_operand(fq, orc, xb, mode, bfmt, None)
    Ad = _deq(orc, mode, hqa, hsa, hga, afmt, (1, 128))
    Bd = _deq(orc, mode, hqb, hsb, hgb, bfmt, (1, 128))
    Cref, D, E, Sg = reference_terms(orc, Ad, Bd)
    C32 = host(_run(fq, mode, A, afmt, B, bfmt, OUT_F32))
    Cbf = host(_run(fq, mode, A, afmt, B, bfmt, OUT_BF16))
    check_gemm(C32, Cbf, Cref, D, E, K, "pipelined 128x128 mode %d %dx%dx%d" % (mode, M, N, K), Sg)


@pytest.mark.parametrize("mode", [TENSOR, MX, MOSS])
@pytest.mark.parametrize("M,N,K", PINGPONG)
@pytest.mark.parametrize("fmts", [(E4M3, E4M3), (E5M2, E4M3), (E4M3, E5M2)])
def test_gemm_pingpong_ragged_sampled(fq, orc, mode, M, N, K, fmts):
    afmt, bfmt = fmts
    xa = workloads.random_matrix(M + 7 * K, M, K, 2.0)
    xb = workloads.random_matrix(N + 11 * K, N, K, 0.05)
    A, (hqa, hsa, hga) = _quant_operand(fq, orc, xa, mode, afmt, None)
    B, (hqb, hsb, hgb) = _quant_operand(fq, orc, xb, mode, bfmt, None)
    _sampled_check(fq, orc, mode, A, afmt, B, bfmt, _rows_deq(orc, mode, hqa, hsa, hga, afmt, None),
                   _rows_deq(orc, mode, hqb, hsb, hgb, bfmt, None), M, N, K, M + N + K,
                   "pingpong mode %d %dx%dx%d" % (mode, M, N, K))


def test_gemm_determinism_and_k_zero(fq, orc):
    xa = workloads.random_matrix(1, 256, 512)
    xb = workloads.random_matrix(2, 192, 512)
    A, _ = _quant_operand(fq, orc, xa, MX, E4M3, None)
    B, _ = _quant_operand(fq, orc, xb, MX, E4M3, None)
    c1 = host(_run(fq, MX, A, E4M3, B, E4M3, OUT_F32))
    c2 = host(_run(fq, MX, A, E4M3, B, E4M3, OUT_F32))
    assert np.array_equal(c1, c2)
    z = fq.scaled_gemm(TENSOR, torch.zeros((8, 0), dtype=torch.uint8, device=DEV), E4M3, None,
                       torch.zeros((16, 0), dtype=torch.uint8, device=DEV), E4M3, None,
                       torch.ones(1, device=DEV), torch.ones(1, device=DEV), out_dtype=OUT_F32)
    assert np.all(host(z) == 0.0)


def test_gemm_operand_past_4gib(fq, orc):
    """An A operand of more than 2^32 bytes: the dispatcher's fallback kernel, which addresses with
    64-bit offsets.  Rows on both sides of the 4 GiB boundary and the last rows are checked."""
    M, N, K = (1 << 20) + 256, 128, 4096
    gen = torch.Generator(device=DEV)
    gen.manual_seed(11)
    A = torch.randint(0, 254, (M, K), dtype=torch.uint8, device=DEV, generator=gen)
    A[A == 0x7F] = 0x7E                                      # no NaN codes
    B, (hqb, _, hgb) = _quant_operand(fq, orc, workloads.random_matrix(12, N, K, 0.05), TENSOR, E4M3, None)
    qb, _, gb = B
    sa = torch.ones(1, dtype=torch.float32, device=DEV)
    boundary = (1 << 32) // K                                 # first row wholly past 4 GiB
    rows = np.unique(np.concatenate([np.arange(0, 64), np.arange(boundary - 64, boundary + 64),
                                     np.arange(M - 64, M)]))
    rt = torch.from_numpy(rows).to(DEV)
    c32 = host(fq.scaled_gemm(TENSOR, A, E4M3, None, qb, E4M3, None, sa, gb, out_dtype=OUT_F32)[rt])
    cbf = host(fq.scaled_gemm(TENSOR, A, E4M3, None, qb, E4M3, None, sa, gb, out_dtype=OUT_BF16)[rt])
    Ad = orc.dequantize(TENSOR, host(A[rt]), E4M3, None, np.float32(1.0))
    del A
    torch.cuda.empty_cache()
    Bd = orc.dequantize(TENSOR, hqb, E4M3, None, hgb)
    Cref, D, E, Sg = reference_terms(orc, Ad, Bd)
    check_gemm(c32, cbf, Cref, D, E, K, "A past 4 GiB", Sg)
