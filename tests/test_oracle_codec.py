"""Pins for the oracle's FP8 codec and amax, against sources other than the oracle itself:
the OCP bit-field definitions written as exact rationals (tests/brute.py), torch's CPU float8
conversions (an independent library implementation), and textbook round-to-nearest-even cases."""
import math
from fractions import Fraction

import numpy as np
import pytest
import torch

from tests import brute

E4M3, E5M2 = 0, 1
TORCH_FMT = {E4M3: torch.float8_e4m3fn, E5M2: torch.float8_e5m2}
MAX = {E4M3: 448.0, E5M2: 57344.0}


@pytest.mark.parametrize("fmt", [E4M3, E5M2])
def test_decode_all_codes_vs_torch_and_fields(orc, fmt):
    codes = np.arange(256, dtype=np.uint8)
    ours = orc.decode_array(codes, fmt)
    theirs = torch.from_numpy(codes.copy()).view(TORCH_FMT[fmt]).to(torch.float64).numpy()
    for c in range(256):
        exact = brute.fp8_value(c, fmt)
        if exact == "nan":
            assert math.isnan(ours[c]) and math.isnan(theirs[c])
        elif exact in ("inf", "-inf"):
            assert ours[c] == theirs[c] == (math.inf if exact == "inf" else -math.inf)
        else:
            assert ours[c] == theirs[c] == float(exact), (fmt, c)


def test_format_landmarks(orc):
    # largest finite, smallest subnormal, one, and the special codes of each format
    assert orc.decode(0x7E, E4M3) == 448.0 and math.isnan(orc.decode(0x7F, E4M3))
    assert orc.decode(0x01, E4M3) == 2.0 ** -9 and orc.decode(0x08, E4M3) == 2.0 ** -6
    assert orc.decode(0x38, E4M3) == 1.0
    assert orc.decode(0x7B, E5M2) == 57344.0 and orc.decode(0x7C, E5M2) == math.inf
    assert orc.decode(0x01, E5M2) == 2.0 ** -16 and orc.decode(0x3C, E5M2) == 1.0
    assert orc.fp8_max(E4M3) == 448.0 and orc.fp8_max(E5M2) == 57344.0


@pytest.mark.parametrize("v,fmt,want", [
    (1.0625, E4M3, 1.0),          # tie between 1.0 (mantissa 000) and 1.125 (001): even wins
    (1.1875, E4M3, 1.25),         # tie between 1.125 (001) and 1.25 (010): even wins
    (464.0, E4M3, 448.0),         # tie between 448 and (non-existent) 480 after clip is 448 anyway
    (2.0 ** -10, E4M3, 0.0),      # half the smallest subnormal ties to zero
    (3 * 2.0 ** -10, E4M3, 2.0 ** -8),   # 1.5 subnormal steps ties to the even step 2
    (1.125, E5M2, 1.0),           # tie between 1.0 (00) and 1.25 (01)
    (1.375, E5M2, 1.5),           # tie between 1.25 (01) and 1.5 (10)
    (2.0 ** -17, E5M2, 0.0),
])
def test_round_to_nearest_even_textbook(orc, v, fmt, want):
    v = min(v, MAX[fmt])
    assert orc.decode(orc.encode(v, fmt), fmt) == want


def _torch_encode(v: np.ndarray, fmt: int) -> np.ndarray:
    t = torch.from_numpy(np.ascontiguousarray(v, np.float32))
    return t.to(TORCH_FMT[fmt]).view(torch.uint8).numpy()


def _clip(v, fmt):
    M = np.float32(MAX[fmt])
    return np.where(v > M, M, np.where(v < -M, -M, v)).astype(np.float32)


@pytest.mark.parametrize("fmt", [E4M3, E5M2])
def test_encode_all_bf16_patterns_vs_torch(orc, fmt):
    bits = (np.arange(65536, dtype=np.uint32) << 16).view(np.float32)
    v = _clip(bits[np.isfinite(bits)], fmt)
    assert np.array_equal(orc.encode_array(v, fmt), _torch_encode(v, fmt))


@pytest.mark.parametrize("fmt", [E4M3, E5M2])
def test_encode_random_and_midpoint_windows_vs_torch(orc, fmt):
    rng = np.random.default_rng(11 + fmt)
    rand = rng.integers(0, 2 ** 32, 1 << 21, dtype=np.uint64).astype(np.uint32).view(np.float32)
    rand = _clip(rand[np.isfinite(rand)], fmt)
    # every midpoint between adjacent finite FP8 values, +-64 fp32 ulps around it, both signs
    vals = sorted(float(brute.fp8_value(c, fmt)) for c in brute.finite_codes(fmt) if c < 0x80)
    mids = np.array([(a + b) / 2 for a, b in zip(vals[:-1], vals[1:])], np.float32)
    offs = np.arange(-64, 65, dtype=np.int64)
    win = (mids.view(np.uint32).astype(np.int64)[:, None] + offs[None, :]).reshape(-1)
    win = win[(win >= 0) & (win < 0x7F800000)].astype(np.uint32).view(np.float32)
    v = np.concatenate([rand, win, -win, np.array([0.0, -0.0], np.float32)])
    v = _clip(v, fmt)
    assert np.array_equal(orc.encode_array(v, fmt), _torch_encode(v, fmt))


@pytest.mark.parametrize("fmt", [E4M3, E5M2])
def test_encode_vs_exhaustive_nearest_search(orc, fmt):
    rng = np.random.default_rng(5 + fmt)
    vals = sorted(float(brute.fp8_value(c, fmt)) for c in brute.finite_codes(fmt) if c < 0x80)
    mids = [(a + b) / 2 for a, b in zip(vals[:-1], vals[1:])]
    sample = list(rng.choice(mids, 150)) + list(rng.uniform(-MAX[fmt], MAX[fmt], 150))
    sample += list(np.exp(rng.uniform(-25, math.log(MAX[fmt]), 150)) * rng.choice([-1, 1], 150))
    sample += [0.0, -0.0, MAX[fmt], -MAX[fmt], 2.0 ** -30, -(2.0 ** -30)]
    for v in sample:
        v = float(np.float32(v))
        assert orc.encode(v, fmt) == brute.nearest_code(v, fmt), (fmt, v)


@pytest.mark.parametrize("fmt", [E4M3, E5M2])
def test_encode_nan_keeps_sign_and_matches_torch(orc, fmt):
    v = np.array([np.nan, -np.nan], np.float32)
    got = orc.encode_array(v, fmt)
    assert list(got) == [0x7F, 0xFF]
    assert np.array_equal(got, _torch_encode(v, fmt))


def test_amax_vs_numpy(orc):
    rng = np.random.default_rng(3)
    x = (rng.standard_normal((37, 53)) * 10).astype(np.float32)
    assert orc.amax(x) == np.abs(x).max()
    x[5, 7] = -1e30
    assert orc.amax(x) == np.float32(1e30)
    xb = (np.ascontiguousarray(x).view(np.uint32) >> 16).astype(np.uint16)   # truncated bf16 bits
    xf = (xb.astype(np.uint32) << 16).view(np.float32)
    assert orc.amax(xb) == np.abs(xf).max()
    assert orc.amax(np.array([[-0.0, 0.0]], np.float32)) == 0.0
    x[1, 1] = np.nan
    assert np.isnan(orc.amax(x))


def test_scale_rule_and_fallbacks(orc):
    # scale = amax / MAX as one fp32 division (numpy's float32 division is IEEE)
    for a in [1.0, 3.7, 1e-3, 12345.678, 448.0]:
        assert orc.compute_scale(a, E4M3, 1.0) == np.float32(a) / np.float32(448.0)
        assert orc.compute_scale(a, E5M2, 1.0) == np.float32(a) / np.float32(57344.0)
    # zero, non-finite and underflowing amax keep the fallback
    for a in [0.0, float("inf"), float("nan"), 1e-45]:
        assert orc.compute_scale(a, E4M3, 0.5) == np.float32(0.5)


def test_quantize_value_is_divide_clip_round(orc):
    rng = np.random.default_rng(9)
    x = (rng.standard_normal(20000) * 7).astype(np.float32)
    s = np.float32(0.0123)
    want = _torch_encode(_clip((torch.from_numpy(x) / torch.tensor(s)).numpy(), E4M3), E4M3)
    got = np.array([orc.quantize_value(v, s, E4M3) for v in x[:2000]], np.uint8)
    assert np.array_equal(got, want[:2000])
    # overflow beyond MAX saturates to the largest code (the clip happens before the cast)
    assert orc.quantize_value(1e6, 1.0, E4M3) == 0x7E
    assert orc.quantize_value(-1e6, 1.0, E4M3) == 0xFE
    assert orc.quantize_value(float("inf"), 1.0, E5M2) == 0x7B
    assert orc.quantize_value(float("nan"), 1.0, E4M3) == 0x7F
