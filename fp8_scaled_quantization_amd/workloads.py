"""Seeded synthetic inputs for the five FP8 workloads.

This module only draws random numbers and stores them as fp32 or bf16 bit patterns; it holds
none of the quantization or GEMM arithmetic.  It is shared by the tests (which feed the same
arrays to the CPU oracle and to the HIP library) and by the benchmark.

Distributions follow the workload descriptions of the source pages' FP8 recipes:
  per-tensor current scaling  A 16x32, B 32x64 fp32 ~ U[0,1)
  delayed scaling             16 steps, A_t 1024x2048, B_t 2048x1024 bf16 = sigma_t * N(0,1),
                              one sigma_t ~ LogU[0.1, 10] per step shared by A_t and B_t
  fine-grained 1x128/128x128  X 4096x7168 bf16 ~ N(0,1) with 0.1% of entries (seeded positions)
                              multiplied by 50; W 2048x7168 bf16 ~ 0.02 * N(0,1)
  MXFP8                       A, B 8192x8192 bf16, row r ~ sigma_r * N(0,1), sigma_r ~ LogU[1e-2, 1e2]
  MOSS forward+backward       X 16384x4096 ~ N(0,1) with 32 seeded channels (columns) x50,
                              W 4096x4096 ~ 0.02 * N(0,1), dY 16384x4096 ~ 1e-3 * N(0,1)
Every array is drawn with numpy's PCG64 generator from a fixed seed; fp32 -> bf16 is
round-to-nearest-even (torch's conversion), and those bf16 bytes are the input of record.
"""
from __future__ import annotations

import numpy as np
import torch

SEEDS = {1: 1, 2: 2, 3: 3, 4: 4, 5: 5}


def to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """fp32 array -> bf16 bit patterns (uint16), round to nearest even."""
    t = torch.from_numpy(np.ascontiguousarray(x, np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (np.ascontiguousarray(b, np.uint16).astype(np.uint32) << 16).view(np.float32)


def _rng(seed) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(seed))


def _normal(rng, shape, scale=1.0):
    return (rng.standard_normal(shape, dtype=np.float32) * np.float32(scale)).astype(np.float32)


def _log_uniform(rng, lo, hi, size):
    return np.exp(rng.uniform(np.log(lo), np.log(hi), size)).astype(np.float32)


# ------------------------------------------------------------------ workloads
def per_tensor_inputs(seed: int = SEEDS[1], m: int = 16, k: int = 32, n: int = 64):
    """A (m x k) and B (k x n), fp32 ~ U[0,1)."""
    rng = _rng(seed)
    A = rng.random((m, k), dtype=np.float32)
    B = rng.random((k, n), dtype=np.float32)
    return A, B


def delayed_inputs(step: int, seed: int = SEEDS[2], m: int = 1024, k: int = 2048, n: int = 1024):
    """Step `step` (0-based) of the delayed-scaling run: (A_t bf16 m x k, B_t bf16 k x n, sigma_t)."""
    child = np.random.SeedSequence(seed).spawn(step + 1)[step]
    rng = _rng(child)
    sigma = _log_uniform(rng, 0.1, 10.0, 1)[0]
    A = to_bf16_bits(_normal(rng, (m, k), sigma))
    B = to_bf16_bits(_normal(rng, (k, n), sigma))
    return A, B, sigma


def fine_grained_inputs(seed: int = SEEDS[3], m: int = 4096, k: int = 7168, n: int = 2048,
                        outlier_frac: float = 0.001, outlier_mult: float = 50.0):
    """X (m x k) bf16 ~ N(0,1) with round(frac*m*k) seeded entries x50; W (n x k) bf16 ~ 0.02 N(0,1)."""
    rng = _rng(seed)
    X = _normal(rng, (m, k))
    n_out = int(round(outlier_frac * m * k))
    idx = rng.choice(m * k, size=n_out, replace=False)
    X.reshape(-1)[idx] *= np.float32(outlier_mult)
    W = _normal(rng, (n, k), 0.02)
    return to_bf16_bits(X), to_bf16_bits(W)


def mx_inputs(seed: int = SEEDS[4], m: int = 8192, k: int = 8192, n: int = 8192):
    """A (m x k), B (n x k) bf16, each row r ~ sigma_r N(0,1), sigma_r ~ LogU[1e-2, 1e2]."""
    rng = _rng(seed)
    sa = _log_uniform(rng, 1e-2, 1e2, m)
    A = _normal(rng, (m, k)) * sa[:, None]
    sb = _log_uniform(rng, 1e-2, 1e2, n)
    B = _normal(rng, (n, k)) * sb[:, None]
    return to_bf16_bits(A), to_bf16_bits(B)


def moss_inputs(seed: int = SEEDS[5], tokens: int = 16384, d_in: int = 4096, d_out: int = 4096,
                n_outlier_channels: int = 32, outlier_mult: float = 50.0):
    """X (tokens x d_in) ~ N(0,1) with 32 seeded columns x50; W (d_out x d_in) ~ 0.02 N(0,1);
    dY (tokens x d_out) ~ 1e-3 N(0,1).  All bf16."""
    rng = _rng(seed)
    X = _normal(rng, (tokens, d_in))
    ch = rng.choice(d_in, size=min(n_outlier_channels, d_in), replace=False)
    X[:, ch] *= np.float32(outlier_mult)
    W = _normal(rng, (d_out, d_in), 0.02)
    dY = _normal(rng, (tokens, d_out), 1e-3)
    return to_bf16_bits(X), to_bf16_bits(W), to_bf16_bits(dY)


def random_matrix(seed: int, rows: int, cols: int, scale: float = 1.0, bf16: bool = True):
    """Generic seeded N(0, scale^2) matrix for edge-case and ragged-shape tests."""
    x = _normal(_rng(seed), (rows, cols), scale)
    return to_bf16_bits(x) if bf16 else x
