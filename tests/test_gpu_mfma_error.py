"""Characterization of the FP8 matrix instruction's accumulation error, measured through
fp8_scaled_gemm alone.  These two constants size the GEMM bound of tests/gpu_util.py:

  * one 128-wide K step from a zero accumulator: |C - C_ref| <= 2^-10 * max_k |a_k b_k| (the
    measured ratio, printed, is about 2^-11);
  * a K step whose accumulator input S already holds a large partial sum: the step's error stays
    within 2^-13 * |S| (measured about 2^-15) plus the step's own 2^-10 * max |a_k b_k|.

The reference is the oracle's fp64 product of the decoded FP8 operands (no rounding of its own at
these sizes), with the per-tensor scales 1 (TENSOR) or random E8M0 scales applied by the
instruction (MX).  Operands: N(0,1) x 8 with 0.1% of entries x50, encoded to FP8 by the oracle;
shapes of 1024 x 1024 (the small-problem kernel) and 4096 x 3072 outputs (the 256 x 256 kernel).
Reference: page "Flax FP8 量化实战指南 ...", section 2.2 (FP32-accumulated dot of the FP8 operands,
dequantized by the scales)."""
import numpy as np
import pytest
import torch

from tests.gpu_util import DEV, host

pytestmark = pytest.mark.gpu

E4M3, E5M2 = 0, 1
TENSOR, MX = 0, 2
OUT_F32 = 0
MAXV = {E4M3: 448.0, E5M2: 57344.0}


@pytest.fixture(scope="module")
def fq():
    import fp8_scaled_quantization_amd as fq
    fq.init()
    return fq


def _codes(orc, rng, rows, K, fmt, scale=8.0):
    x = rng.standard_normal((rows, K)) * scale
    x[rng.random((rows, K)) < 1e-3] *= 50.0
    return orc.encode_array(np.clip(x, -MAXV[fmt], MAXV[fmt]).astype(np.float32), fmt)


def _run(fq, orc, mode, qa, afmt, qb, bfmt, rng, erange=6):
    """GEMM of the FP8 codes with unit tensor scales (TENSOR) or random E8M0 scales 2^[-erange,
    erange] (MX); returns (C32 on the host, fp64 A, fp64 B) with A, B the exactly decoded (and
    scaled) operands."""
    M, K = qa.shape
    N = qb.shape[0]
    A = torch.from_numpy(qa).to(DEV)
    B = torch.from_numpy(qb).to(DEV)
    C = torch.empty((M, N), dtype=torch.float32, device=DEV)
    if mode == TENSOR:
        one = torch.ones(1, dtype=torch.float32, device=DEV)
        fq.fp8_scaled_gemm(TENSOR, A, afmt, None, B, bfmt, None, one, one, C, OUT_F32)
        Ad = orc.dequantize(TENSOR, qa, afmt, None, np.float32(1.0))
        Bd = orc.dequantize(TENSOR, qb, bfmt, None, np.float32(1.0))
    else:
        ea = rng.integers(127 - erange, 127 + erange + 1, (M, K // 32)).astype(np.uint8)
        eb = rng.integers(127 - erange, 127 + erange + 1, (N, K // 32)).astype(np.uint8)
        fq.fp8_scaled_gemm(MX, A, afmt, torch.from_numpy(ea).to(DEV), B, bfmt, torch.from_numpy(eb).to(DEV),
                           None, None, C, OUT_F32)
        Ad = orc.dequantize(MX, qa, afmt, ea)
        Bd = orc.dequantize(MX, qb, bfmt, eb)
    return host(C), Ad, Bd


@pytest.mark.parametrize("M,N", [(1024, 1024), (4096, 3072)])
@pytest.mark.parametrize("mode", [TENSOR, MX])
@pytest.mark.parametrize("fmts", [(E4M3, E4M3), (E5M2, E4M3)])
def test_one_k_step_from_zero(fq, orc, M, N, mode, fmts):
    afmt, bfmt = fmts
    rng = np.random.default_rng(M + N + 10 * mode + afmt)
    qa = _codes(orc, rng, M, 128, afmt)
    qb = _codes(orc, rng, N, 128, bfmt)
    C32, Ad, Bd = _run(fq, orc, mode, qa, afmt, qb, bfmt, rng)
    Cref, D, E, _ = orc.gemm_ref_terms(Ad, Bd)
    err = np.abs(C32.astype(np.float64) - Cref)
    ratio = float((err / np.maximum(E, 1e-300)).max())
    print("MFMA one K step, mode %d fmts %s, %d outputs: max |C - C_ref| / max|a b| = %.3g = 2^%.2f"
          % (mode, fmts, M * N, ratio, np.log2(max(ratio, 1e-300))))
    assert ratio <= 2.0 ** -10


@pytest.mark.parametrize("mode", [TENSOR, MX])
@pytest.mark.parametrize("fmts", [(E4M3, E4M3), (E5M2, E4M3)])
@pytest.mark.parametrize("small", [2.0, 0.25])
def test_accumulator_input_error(fq, orc, mode, fmts, small):
    """K = 256: the first 128-wide step holds one product a0*b0 of magnitude 2^14..2^16 (exact in
    fp32, so the accumulator entering the second step is exactly S = a0*b0), the second step 128
    products of N(0,1) x `small` operands (magnitudes ~2^2 or ~2^-4, so ~2^-12..2^-20 of S)."""
    afmt, bfmt = fmts
    M = N = 1024
    rng = np.random.default_rng(100 + 10 * mode + afmt + int(small * 4))

    def operand(rows, fmt):
        q = np.zeros((rows, 256), np.uint8)
        big = rng.uniform(128.0, 256.0, rows) * rng.choice([-1.0, 1.0], rows)
        q[:, 0] = orc.encode_array(big.astype(np.float32), fmt)
        q[:, 128:] = _codes(orc, rng, rows, 128, fmt, scale=small)
        return q

    qa, qb = operand(M, afmt), operand(N, bfmt)
    C32, Ad, Bd = _run(fq, orc, mode, qa, afmt, qb, bfmt, rng, erange=2)
    Cref, D, E, Sg = orc.gemm_ref_terms(Ad, Bd)
    S1 = Ad[:, :1] * Bd[:, 0][None, :]                 # the exact first-step partial
    assert np.array_equal(np.abs(S1), Sg)               # Sigma of a two-step sum is |S_1|
    E2 = E - np.abs(S1)                                 # the second step's largest |product|
    err = np.abs(C32.astype(np.float64) - Cref)
    # where S dominates the step's products by 2^6 or more, the error is the accumulator input's
    dom = np.abs(S1) >= 64.0 * E2
    ratio_s = float((err[dom] / np.abs(S1)[dom]).max())
    ratio_b = float((err / (2.0 ** -10 * E2 + 2.0 ** -13 * np.abs(S1))).max())
    print("MFMA accumulator input, mode %d fmts %s, second-step operands x%g: %d outputs with |S| >= 64 max|a b|, max |C - C_ref| / |S| "
          "= %.3g = 2^%.2f; over all %d, max err / (2^-10 E_2 + 2^-13 |S|) = %.3g"
          % (mode, fmts, small, int(dom.sum()), ratio_s, np.log2(max(ratio_s, 1e-300)), M * N, ratio_b))
    assert dom.sum() >= M * N // 4
    assert ratio_b <= 1.0 and ratio_s <= 2.0 ** -13
