"""Helpers shared by the GPU parity tests: host<->device transfer of the seeded inputs, oracle-side
dequantization of row samples, and the GEMM error bound.

GEMM tolerance.  The oracle's reference is the exact (fp64) product of the dequantized operands.
The library reduces K in 128-wide steps with gfx950's FP8 matrix instruction, whose own error is
characterized through the library by tests/test_gpu_mfma_error.py: one instruction adds its 128
products with an error of at most 2^-11 times the largest product magnitude, and adds its C input
with an error of about 2^-15 times |C|.  BLOCK scaling promotes every step into an FP32
accumulator (one more rounding of 2^-24 |acc| per step, plus the rounding of the block-scale
product fl(sx*sw)); the other schemes keep the whole K sum in the instruction's accumulator, so
step k also carries the C-input error of the running sum S_{k-1}.  The elementwise bound used in
the tests is therefore
    |C - C_ref| <= 2^-10 * E + 2^-13 * Sigma + (K/128 + 3) * 2^-24 * D,
with E = sum over 128-wide K steps of max_k |a_k b_k|, Sigma = sum over steps of |S_{k-1}| (exact
prefix sums of the per-step partial products; 0 for BLOCK), D = sum_k |a_k b_k| (all from the
oracle's gemm_ref_terms), i.e. margins of 2x and about 4x over the characterized constants.  The
bf16 output must equal round-to-nearest-even of the same kernel's fp32 output bit for bit, and its
normwise relative error must stay within 2e-3.
"""
from __future__ import annotations

import numpy as np
import torch

from fp8_scaled_quantization_amd import workloads

DEV = "cuda:0"

_MOSS_ORACLE = {}


def moss_oracle_copies(orc, key: str, x: np.ndarray, fmt: int):
    """The oracle's two MOSS copies of a full workload tensor (groups along its rows, and along its
    columns), cached for the tests that compare both the single and the dual cast against them:
    (q, e, qt, et, S)."""
    if key not in _MOSS_ORACLE:
        oq, oe, oS = orc.quantize_moss(x, fmt)
        oqt, oet = orc.quantize_moss_given(x, fmt, oS, transpose=True)
        _MOSS_ORACLE[key] = (oq, oe, oqt, oet, oS)
    return _MOSS_ORACLE[key]


def to_dev_bf16(bits: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).to(DEV)


def to_dev(x: np.ndarray) -> torch.Tensor:
    if x.dtype == np.uint16:
        return to_dev_bf16(x)
    return torch.from_numpy(np.ascontiguousarray(x)).to(DEV)


def host(t: torch.Tensor) -> np.ndarray:
    t = t.detach().cpu()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view(np.uint16)
    return t.numpy()


def same(got: np.ndarray, want: np.ndarray, label: str = "", show: int = 6) -> bool:
    """Bitwise equality that prints the count and the first mismatching positions on failure."""
    got = np.asarray(got)
    want = np.asarray(want)
    if got.shape != want.shape:
        print("%s: shape %s != %s" % (label, got.shape, want.shape))
        return False
    gb = got.view(np.uint8) if got.dtype != np.uint8 else got
    wb = want.view(np.uint8) if want.dtype != np.uint8 else want
    if got.dtype == want.dtype and np.array_equal(gb, wb):
        return True
    bad = np.argwhere(got != want) if got.dtype != np.float32 else np.argwhere(
        got.view(np.uint32) != want.astype(np.float32).view(np.uint32))
    print("%s: %d mismatches of %d" % (label, len(bad), got.size))
    for idx in bad[:show]:
        i = tuple(int(v) for v in idx)
        print("   at %s: got %r want %r" % (i, got[i], want[i]))
    return False


def bf16_rne_bits(x32: np.ndarray) -> np.ndarray:
    """fp32 -> bf16 bits by torch's round-to-nearest-even (an independent library conversion)."""
    return workloads.to_bf16_bits(x32)


def gemm_bound(E, D, K, Sigma=None):
    b = 2.0 ** -10 * E + (K / 128.0 + 3.0) * 2.0 ** -24 * D
    if Sigma is not None:
        b = b + 2.0 ** -13 * Sigma
    return b


def check_gemm(C32: np.ndarray, Cbf: np.ndarray | None, Cref: np.ndarray, D: np.ndarray, E: np.ndarray, K: int,
               label: str = "", Sigma=None):
    """Assert the elementwise bound on the fp32 output, bf16 == RNE(fp32), normwise bf16 error.
    Also prints the largest err/D and the largest err / max(|C_ref|, D/16) (an elementwise relative
    error floored at D/16), which is what a fixed 1e-5 relative tolerance would be compared with."""
    err = np.abs(C32.astype(np.float64) - Cref)
    bound = gemm_bound(E, D, K, Sigma)
    bad = err > bound
    worst = float((err / np.maximum(bound, 1e-300)).max()) if err.size else 0.0
    if err.size:
        floored = float((err / np.maximum(np.maximum(np.abs(Cref), D / 16.0), 1e-300)).max())
        print("%s: %d outputs, worst err/bound %.3g, max err/D %.3g, max err/max(|C|,D/16) %.3g"
              % (label, err.size, worst, float((err / np.maximum(D, 1e-300)).max()), floored))
    assert not bad.any(), "%s: %d of %d outputs exceed the bound; worst err/bound %.3g" % (
        label, int(bad.sum()), bad.size, worst)
    if Cbf is not None:
        assert np.array_equal(Cbf, bf16_rne_bits(C32)), "%s: bf16 output is not RNE(fp32 output)" % label
        cb = workloads.bf16_bits_to_f32(Cbf).astype(np.float64)
        nrm = np.linalg.norm(Cref)
        if nrm > 0:
            rel = np.linalg.norm(cb - Cref) / nrm
            print("%s: bf16 normwise relative error %.3g" % (label, rel))
            assert rel <= 2e-3, label
    return worst


def reference_terms(orc, Ad: np.ndarray, Bd: np.ndarray, pairs=None, promoted: bool = False):
    """(C_ref, D, E, Sigma) from the oracle; Sigma is None when every K step starts from zero
    (BLOCK promotion), so the bound drops that term."""
    C, D, E, S = orc.gemm_ref_terms(Ad, Bd, pairs)
    return C, D, E, (None if promoted else S)


def edge_indices(n: int, tile: int = 128) -> np.ndarray:
    """First and last index of every tile of `tile` along an axis of length n, and the last index."""
    return np.unique(np.clip(np.concatenate([np.arange(0, n, tile), np.arange(tile - 1, n, tile), [n - 1]]), 0, n - 1))


def check_gemm_large(orc, C32, Cbf, deqA, deqB, M: int, N: int, K: int, seed: int, label: str,
                     promoted: bool = False, n_random: int = 65536, tile: int = 128, full: bool = False) -> float:
    """Full-size GEMM parity.  With full=True every output is compared.  Otherwise three sets of
    outputs: every output of the rows on a tile edge (first and last row of every `tile` rows),
    every output of the columns on a tile edge, and n_random seeded outputs anywhere; a 128-edge
    grid contains the edges of every kernel's tiles (256 x 256, 256 x 128, 128 x 128).  C32 / Cbf
    are the device outputs (fp32 and bf16) of the same problem; deqA / deqB dequantize a list of
    operand rows with the oracle."""
    Aall, Ball = deqA(np.arange(M)), deqB(np.arange(N))
    if full:
        Cref, D, E, Sg = reference_terms(orc, Aall, Ball, promoted=promoted)
        del Aall, Ball
        return check_gemm(host(C32), host(Cbf), Cref, D, E, K, "%s, all %d outputs" % (label, M * N), Sg)
    er, ec = edge_indices(M, tile), edge_indices(N, tile)
    rng = np.random.default_rng(seed)
    pairs = np.stack([rng.integers(0, M, n_random), rng.integers(0, N, n_random)], 1).astype(np.int64)
    worst = 0.0
    rt = torch.from_numpy(er).to(C32.device)
    ct = torch.from_numpy(ec).to(C32.device)
    for name, (Ad, Bd, sel) in {
            "edge rows": (Aall[er], Ball, lambda t: host(t[rt])),
            "edge cols": (Aall, Ball[ec], lambda t: host(t[:, ct])),
    }.items():
        Cref, D, E, Sg = reference_terms(orc, Ad, Bd, promoted=promoted)
        worst = max(worst, check_gemm(sel(C32), sel(Cbf), Cref, D, E, K, "%s, %s" % (label, name), Sg))
    Cref, D, E, Sg = reference_terms(orc, Aall, Ball, pairs, promoted=promoted)
    pt = torch.from_numpy(pairs).to(C32.device)
    c32 = host(C32[pt[:, 0], pt[:, 1]])
    cbf = host(Cbf[pt[:, 0], pt[:, 1]])
    worst = max(worst, check_gemm(c32, cbf, Cref, D, E, K, "%s, %d random" % (label, n_random), Sg))
    return worst


def sample_pairs(M: int, N: int, n: int, seed: int, tile: int = 128) -> np.ndarray:
    """Seeded (m, n) sample: random pairs plus rows/cols on every tile edge and the last row/col."""
    rng = np.random.default_rng(seed)
    pairs = [np.stack([rng.integers(0, M, n), rng.integers(0, N, n)], 1)]
    edges_m = np.unique(np.clip(np.concatenate([np.arange(0, M, tile), np.arange(tile - 1, M, tile), [M - 1]]), 0, M - 1))
    edges_n = np.unique(np.clip(np.concatenate([np.arange(0, N, tile), np.arange(tile - 1, N, tile), [N - 1]]), 0, N - 1))
    pairs.append(np.stack([edges_m, rng.integers(0, N, len(edges_m))], 1))
    pairs.append(np.stack([rng.integers(0, M, len(edges_n)), edges_n], 1))
    return np.concatenate(pairs).astype(np.int64)
