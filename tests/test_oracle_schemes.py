"""Pins for the oracle's five scaling schemes, from what the pages and the mathematics fix:
library recomputations (numpy/torch), exact-rational minimality checks, invariants stated on the
MOSS page (global factor >= every local factor, local factors are powers of two in (0,1]), the
Flax page's worked example for delayed scaling, and special cases that reduce one scheme to
another."""
import json
import math
import os
from fractions import Fraction

import numpy as np
import pytest
import torch

from fp8_scaled_quantization_amd import workloads

E4M3, E5M2 = 0, 1
MAX = {E4M3: 448.0, E5M2: 57344.0}
TORCH_FMT = {E4M3: torch.float8_e4m3fn, E5M2: torch.float8_e5m2}
GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def torch_quant(xf32: np.ndarray, s, fmt):
    """Library recomputation: fp32 divide by a (broadcast) scale, clamp, torch's RNE cast."""
    v = torch.from_numpy(np.ascontiguousarray(xf32, np.float32)) / torch.as_tensor(np.asarray(s, np.float32))
    v = v.clamp(-MAX[fmt], MAX[fmt])
    return v.to(TORCH_FMT[fmt]).view(torch.uint8).numpy()


def f32(xb):
    return workloads.bf16_bits_to_f32(xb)


# ------------------------------------------------------------------ per-tensor current scaling
@pytest.mark.parametrize("fmt", [E4M3, E5M2])
def test_per_tensor_vs_library(orc, fmt):
    xb = workloads.random_matrix(21, 48, 160, 3.0)
    q, s = orc.quantize_tensor_current(xb, fmt)
    x = f32(xb)
    assert s == np.float32(np.abs(x).max()) / np.float32(MAX[fmt])
    assert np.array_equal(q, torch_quant(x, s, fmt))
    # the max-|x| element lands exactly on +-MAX
    i = np.unravel_index(np.argmax(np.abs(x)), x.shape)
    assert q[i] & 0x7F == (0x7E if fmt == E4M3 else 0x7B)
    # transposed output is the quantization of x.T
    qt = orc.quantize_tensor(xb, fmt, s, transpose=True)
    assert np.array_equal(qt, q.T)


def test_per_tensor_lossless_on_grid(orc):
    # values on the E4M3 grid times 2^j with amax = 448 * 2^j come back exactly
    from tests import brute
    grid = np.array([float(brute.fp8_value(c, E4M3)) for c in brute.finite_codes(E4M3)], np.float32)
    rng = np.random.default_rng(2)
    x = rng.choice(grid, (16, 64)).astype(np.float32) * np.float32(2.0 ** -5)
    x[0, 0] = np.float32(448.0 * 2.0 ** -5)
    q, s = orc.quantize_tensor_current(x, E4M3)
    assert s == np.float32(2.0 ** -5)
    assert np.array_equal(orc.decode_array(q, E4M3) * float(s), x.astype(np.float64))


def test_per_tensor_relative_error_bound(orc):
    xb = workloads.random_matrix(22, 64, 256)
    q, s = orc.quantize_tensor_current(xb, E4M3)
    x = f32(xb).astype(np.float64)
    xh = orc.decode_array(q, E4M3) * float(s)
    normal = np.abs(x) / float(s) >= 2.0 ** -6          # E4M3 normal range
    assert np.all(np.abs(x - xh)[normal] <= 2.0 ** -4 * np.abs(x)[normal] * (1 + 1e-6))


# ------------------------------------------------------------------ delayed scaling
def _merge_example(orc, merge):
    g = json.load(open(os.path.join(GOLDEN, "flax_fp32_max_grad_example.json")))
    inp = g["inputs"]
    results = []
    for v in (inp["x"], inp["y"]):
        scale = np.array([inp["scale"]], np.float32)
        hist = np.zeros(inp["history_len"], np.float32)
        orc.delayed_step(np.array([[v]], np.float32), E4M3, scale, hist)
        results.append((scale[0], hist.copy()))
    (s1, h1), (s2, h2) = results
    if merge == "max":
        return np.float32(max(s1, s2)), np.maximum(h1, h2), g["max_merge"]
    return np.float32(s1 + s2), h1 + h2, g["sum_merge"]


@pytest.mark.parametrize("merge", ["max", "sum"])
def test_delayed_worked_example(orc, merge):
    s, h, want = _merge_example(orc, merge)
    assert s == want["scale"]
    assert list(h[:len(want["history_head"])]) == want["history_head"]
    assert np.all(h[len(want["history_head"]):] == 0.0)
    assert h.size == 1024


def test_delayed_sixteen_steps_vs_numpy_replay(orc):
    """Replay of the update rule written with numpy's roll, step by step (the page's test style),
    against the oracle's in-step update, on scaled-down delayed-scaling workload steps."""
    scale = np.array([1.0], np.float32)
    hist = np.zeros(1024, np.float32)
    r_scale, r_hist = np.float32(1.0), np.zeros(1024, np.float32)
    for t in range(16):
        A, _, sigma = workloads.delayed_inputs(t, m=32, k=64, n=8)
        q, a = orc.delayed_step(A, E4M3, scale, hist)
        m = r_hist.max()
        if m > 0 and np.isfinite(m):
            r_scale = np.float32(m) / np.float32(448.0)
        x = f32(A)
        assert np.array_equal(q, torch_quant(x, r_scale, E4M3)), t
        r_hist = np.roll(r_hist, -1)
        r_hist[0] = np.abs(x).max()
        assert scale[0] == r_scale and np.array_equal(hist, r_hist) and a == r_hist[0]
    # after 16 steps the window holds the 16 amaxes: newest at 0, the previous ones at the end
    assert np.count_nonzero(hist) == 16 and hist[0] == a


def test_delayed_overflow_saturates(orc):
    # a step whose data is 100x the history's range saturates to +-MAX instead of overflowing
    scale = np.array([1.0], np.float32)
    hist = np.zeros(8, np.float32)
    orc.delayed_step(workloads.random_matrix(30, 16, 16, 1.0), E4M3, scale, hist)
    q, _ = orc.delayed_step(workloads.random_matrix(31, 16, 16, 100.0), E4M3, scale, hist)
    codes = q & 0x7F
    assert codes.max() == 0x7E and not np.any(codes == 0x7F)


def test_post_step_order_equals_in_step_order(orc):
    """Updating (history, scale) after each cast yields the same per-step scale as Flax's order."""
    scale = np.array([1.0], np.float32)
    hist = np.zeros(1024, np.float32)
    post_scale, post_hist = np.float32(1.0), np.zeros(1024, np.float32)
    for t in range(6):
        A, _, _ = workloads.delayed_inputs(t, m=16, k=32, n=8)
        q_in, a = orc.delayed_step(A, E4M3, scale, hist)
        q_post = orc.quantize_tensor(A, E4M3, post_scale)
        assert np.array_equal(q_in, q_post) and scale[0] == post_scale
        orc.history_roll_insert(post_hist, orc.amax(A))
        post_scale = orc.compute_scale(orc.history_max(post_hist), E4M3, post_scale)
        assert np.array_equal(post_hist, hist)


# ------------------------------------------------------------------ block scaling
@pytest.mark.parametrize("br,bc", [(1, 128), (128, 128), (32, 32)])
def test_block_vs_library(orc, br, bc):
    xb = workloads.random_matrix(40 + br, 256, 384, 2.0)
    x = f32(xb)
    x[3, 5] *= 50.0                                   # an outlier in one block
    xb = workloads.to_bf16_bits(x)
    x = f32(xb)
    q, s = orc.quantize_block(xb, E4M3, br, bc)
    assert s.shape == (256 // br, 384 // bc)
    blocks = x.reshape(256 // br, br, 384 // bc, bc)
    am = np.abs(blocks).max(axis=(1, 3))
    assert np.array_equal(s, am.astype(np.float32) / np.float32(448.0))
    sfull = np.repeat(np.repeat(s, br, 0), bc, 1)
    assert np.array_equal(q, torch_quant(x, sfull, E4M3))
    # every block's max element is +-448
    qb = (q & 0x7F).reshape(256 // br, br, 384 // bc, bc)
    assert np.all(qb.max(axis=(1, 3)) == 0x7E)


def test_block_weight_scale_shape_and_ragged(orc):
    # (ceil(out/128), ceil(in/128)) scales; 2048 x 7168 gives 16 x 56
    W = np.zeros((2048, 7168), np.float32)
    W[::97, ::89] = 1.0
    _, s = orc.quantize_block(W[:, :], E4M3, 128, 128)
    assert s.shape == (16, 56)
    # ragged: 200 x 300 with 128 x 128 blocks -> 2 x 3 scales, partial blocks use their own amax
    xb = workloads.random_matrix(44, 200, 300)
    q, s = orc.quantize_block(xb, E4M3, 128, 128)
    assert s.shape == (2, 3)
    x = f32(xb)
    assert s[1, 2] == np.float32(np.abs(x[128:, 256:]).max()) / np.float32(448.0)
    sfull = np.repeat(np.repeat(s, 128, 0), 128, 1)[:200, :300]
    assert np.array_equal(q, torch_quant(x, sfull, E4M3))


def test_block_whole_tensor_is_per_tensor_and_zero_block(orc):
    xb = workloads.random_matrix(45, 64, 256)
    qb, sb = orc.quantize_block(xb, E4M3, 64, 256)
    qt, st = orc.quantize_tensor_current(xb, E4M3)
    assert np.array_equal(qb, qt) and sb[0, 0] == st
    z = np.zeros((4, 256), np.float32)
    qz, sz = orc.quantize_block(z, E4M3, 1, 128)
    assert np.all(sz == 1.0) and np.all(qz == 0)


def test_block_transposed_is_block_of_transpose(orc):
    xb = workloads.random_matrix(46, 256, 128)
    q1, s1 = orc.quantize_block(xb, E4M3, 1, 128, transpose=True)
    q2, s2 = orc.quantize_block(np.ascontiguousarray(xb.T), E4M3, 1, 128)
    assert np.array_equal(q1, q2) and np.array_equal(s1, s2)


# ------------------------------------------------------------------ MX
def _exact_min_exponent_ok(amax: float, e: int, M: float) -> bool:
    """e is the smallest integer in [-127,127] with M*2^e >= amax, checked with exact rationals."""
    a, Mq = Fraction(amax), Fraction(M)
    ok_hi = Mq * Fraction(2) ** e >= a
    ok_lo = e == -127 or Mq * Fraction(2) ** (e - 1) < a
    return ok_hi and ok_lo


@pytest.mark.parametrize("fmt", [E4M3, E5M2])
def test_mx_exponents_minimal_and_no_clip(orc, fmt):
    xb, _ = workloads.mx_inputs(m=64, k=256, n=8)
    x = f32(xb)
    q, e = orc.quantize_mx(xb, fmt)
    assert e.shape == (64, 8)
    g = x.reshape(64, 8, 32)
    am = np.abs(g).max(axis=2)
    for r in range(64):
        for j in range(8):
            assert _exact_min_exponent_ok(float(am[r, j]), int(e[r, j]) - 127, MAX[fmt])
    # exact scaling never needs the clip, and elements are the library RNE of x * 2^-e
    f = np.ldexp(np.float32(1.0), -(e.astype(np.int32) - 127)).astype(np.float32)
    v = (g * f[:, :, None]).reshape(64, 256)
    assert np.abs(v).max() <= MAX[fmt]
    want = torch.from_numpy(v).to(TORCH_FMT[fmt]).view(torch.uint8).numpy()
    assert np.array_equal(q, want)


def test_mx_zero_group_and_transpose(orc):
    x = np.zeros((2, 64), np.float32)
    x[0, 40] = 3.0
    q, e = orc.quantize_mx(x, E4M3)
    assert list(e[0]) == [0, 127 + int(math.ceil(math.log2(3.0 / 448.0)))] and e[1, 0] == 0
    xb = workloads.random_matrix(47, 64, 96)
    q1, e1 = orc.quantize_mx(xb, E4M3, transpose=True)
    q2, e2 = orc.quantize_mx(np.ascontiguousarray(xb.T), E4M3)
    assert np.array_equal(q1, q2) and np.array_equal(e1, e2)


def test_mx_equals_moss_when_global_factor_is_one(orc):
    # a tensor whose amax is exactly MAX has S = fl(MAX/MAX) = 1, and then MOSS's local
    # exponents and elements coincide with MX's
    xb = workloads.random_matrix(48, 32, 256, 1.0)
    x = f32(xb)
    x[0, 0] = 448.0
    qm, em = orc.quantize_mx(x, E4M3)
    qs, es, S = orc.quantize_moss(x, E4M3)
    assert S == 1.0
    assert np.array_equal(qm, qs) and np.array_equal(em, es)


# ------------------------------------------------------------------ MOSS
@pytest.mark.parametrize("fmt", [E4M3, E5M2])
def test_moss_invariants(orc, fmt):
    X, W, dY = workloads.moss_inputs(tokens=64, d_in=256, d_out=128)
    for src, f in ((X, E4M3), (W, E4M3), (dY, E5M2)):
        if f != fmt:
            continue
        x = f32(src)
        q, e, S = orc.quantize_moss(src, fmt)
        assert S == np.float32(np.abs(x).max()) / np.float32(MAX[fmt])
        am = np.abs(x.reshape(x.shape[0], -1, 32)).max(axis=2)
        s_i = am.astype(np.float32) / np.float32(MAX[fmt])
        ee = e.astype(np.int64) - 127
        assert np.all(S >= s_i)                                   # global >= every local need
        assert np.all((ee <= 0) & (ee >= -127))                    # local factor 2^e in (0, 1]
        for r in range(x.shape[0]):
            for j in range(am.shape[1]):
                k = int(ee[r, j])
                lhs = Fraction(float(S)) * Fraction(2) ** k
                assert lhs >= Fraction(float(s_i[r, j]))            # no overflow
                if k > -127:
                    assert Fraction(float(S)) * Fraction(2) ** (k - 1) < Fraction(float(s_i[r, j]))


def _moss_local_exponents(x32: np.ndarray, S: np.float32, fmt) -> np.ndarray:
    """Smallest e in [-127, 0] with S * 2^e >= s_i, s_i = fl32(amax_i / MAX) per 32-group (0 when
    none), by exact float64 comparisons (S * 2^e is exact in float64 over this range)."""
    am = np.abs(x32.reshape(x32.shape[0], -1, 32)).max(axis=2).astype(np.float32)
    s_i = (am / np.float32(MAX[fmt])).astype(np.float64)
    e = np.zeros(s_i.shape, np.int64)
    S64 = float(S)
    for k in range(-1, -128, -1):                      # lower e while S * 2^k still covers s_i
        ok = (e == k + 1) & (np.ldexp(S64, k) >= s_i)
        e[ok] = k
    return e


@pytest.mark.parametrize("fmt", [E4M3, E5M2])
@pytest.mark.parametrize("s_factor", [1.0, 1.7, 3.0, 2.0 ** 12, 0.5])
def test_moss_bytes_by_library_recomputation(orc, fmt, s_factor):
    """MOSS elements and E8M0 bytes for a general global factor S, recomputed with torch: the
    local exponents by exact comparison, then an IEEE fp32 divide by S, an exact power-of-two
    multiply by 2^-e_i, a clamp to +-MAX and torch's RNE cast.  S factors above 1 leave headroom
    (many groups get e_i < 0, some values land in FP8 subnormals); 0.5 puts the tensor max past
    S * MAX, where e_i = 0 and the clamp saturates."""
    rng = np.random.default_rng(int(s_factor * 7) + fmt)
    x = rng.standard_normal((96, 256)) * np.exp(rng.uniform(-6, 6, (96, 1)))
    x[:, 5] *= 50.0
    if fmt == E5M2:
        x *= 1e-3
    xb = workloads.to_bf16_bits(x.astype(np.float32))
    x32 = f32(xb)
    S = np.float32(np.float32(np.abs(x32).max()) / np.float32(MAX[fmt]) * np.float32(s_factor))
    q, e = orc.quantize_moss_given(xb, fmt, S)
    e_want = _moss_local_exponents(x32, S, fmt)
    assert np.array_equal(e.astype(np.int64) - 127, e_want)
    v = torch.from_numpy(x32) / torch.tensor(S, dtype=torch.float32)
    up = torch.from_numpy(np.repeat(np.ldexp(1.0, -e_want), 32, axis=1).astype(np.float32))
    v = (v * up).clamp(-MAX[fmt], MAX[fmt])
    want = v.to(TORCH_FMT[fmt]).view(torch.uint8).numpy()
    assert np.array_equal(q, want)
    assert (e_want < 0).any() and (s_factor >= 1.0 or (e_want == 0).any())


def test_moss_dominates_per_tensor(orc):
    """With the same global S, each MOSS element is at least as close to fl(x/S) as the
    per-tensor element, so MOSS's SNR is never below per-tensor's."""
    X, _, _ = workloads.moss_inputs(tokens=128, d_in=256, d_out=64)
    x = f32(X)
    q, e, S = orc.quantize_moss(X, E4M3)
    qt = orc.quantize_tensor(X, E4M3, S)
    v = (x / S).astype(np.float64)
    loc = np.repeat(np.ldexp(1.0, e.astype(np.int64) - 127), 32, axis=1)
    err_moss = np.abs(v - orc.decode_array(q, E4M3) * loc)
    err_pt = np.abs(v - orc.decode_array(qt, E4M3))
    assert np.all(err_moss <= err_pt * (1 + 2.0 ** -20) + 1e-300)
    snr_m = orc.snr_db(x, orc.dequantize(3, q, E4M3, e, S))
    snr_t = orc.snr_db(x, orc.dequantize(0, qt, E4M3, None, S))
    assert snr_m >= snr_t


def test_moss_single_group_is_per_tensor(orc):
    xb = workloads.random_matrix(49, 1, 32)
    q, e, S = orc.quantize_moss(xb, E4M3)
    qt, st = orc.quantize_tensor_current(xb, E4M3)
    assert e[0, 0] == 127 and S == st and np.array_equal(q, qt)


def test_moss_transposed_copy_shares_global(orc):
    X, _, _ = workloads.moss_inputs(tokens=64, d_in=128, d_out=32)
    q, e, S = orc.quantize_moss(X, E4M3)
    qt, et, St = orc.quantize_moss(X, E4M3, transpose=True)
    assert S == St and qt.shape == (128, 64) and et.shape == (128, 2)
    q2, e2, _ = orc.quantize_moss(np.ascontiguousarray(X.T), E4M3)
    assert np.array_equal(qt, q2) and np.array_equal(et, e2)


def test_zero_tensor_fallbacks(orc):
    z = np.zeros((4, 64), np.float32)
    q, e, S = orc.quantize_moss(z, E4M3)
    assert S == 1.0 and np.all(e == 0) and np.all(q == 0)
    q, s = orc.quantize_tensor_current(z, E4M3)
    assert s == 1.0 and np.all(q == 0)
