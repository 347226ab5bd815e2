"""GPU parity of the amax, cast and history kernels against the CPU oracle (bit-exact bytes, scales,
E8M0 exponents and amax values), at the five workloads' shapes and on ragged and special inputs.
Every call goes through the C ABI (libfp8q.so) via the Python binding."""
import numpy as np
import pytest
import torch

from fp8_scaled_quantization_amd import workloads
from tests.gpu_util import DEV, host, moss_oracle_copies, same, to_dev

pytestmark = pytest.mark.gpu

E4M3, E5M2 = 0, 1
TENSOR, BLOCK, MX, MOSS = 0, 1, 2, 3


@pytest.fixture(scope="module")
def fq():
    import fp8_scaled_quantization_amd as fq
    fq.init()
    return fq


def _f32(t):
    return np.float32(host(t)[0])


# ------------------------------------------------------------------ amax
@pytest.mark.parametrize("shape,bf16", [((1000, 512), True), ((37, 64), False), ((4096, 7168), True)])
def test_amax(fq, orc, shape, bf16):
    x = workloads.random_matrix(100 + shape[0], shape[0], shape[1], 5.0, bf16=bf16)
    out = torch.zeros(1, dtype=torch.float32, device=DEV)
    fq.fp8_amax(to_dev(x), out)
    assert _f32(out) == orc.amax(x)


@pytest.mark.parametrize("bf16", [False, True])
def test_amax_strided_nan_empty(fq, orc, bf16):
    x = workloads.random_matrix(7, 64, 96, 1.0, bf16=bf16)
    xd = to_dev(x)[:, :64]                      # ld = 96 > cols = 64: the row-strided kernel
    out = torch.zeros(1, dtype=torch.float32, device=DEV)
    fq.fp8_amax(xd, out)
    assert _f32(out) == orc.amax(np.ascontiguousarray(x[:, :64]))
    x[3, 5] = np.uint16(0x7FC0) if bf16 else np.nan
    fq.fp8_amax(to_dev(x)[:, :64], out)
    assert np.isnan(_f32(out))
    fq.fp8_amax(to_dev(x), out)
    assert np.isnan(_f32(out))
    fq.fp8_amax(torch.zeros((0, 64), dtype=torch.float32, device=DEV), out)
    assert _f32(out) == 0.0
    fq.fp8_amax(to_dev(np.array([[-0.0] * 8], np.float32)), out)
    assert _f32(out) == 0.0


# ------------------------------------------------------------------ per-tensor current (16x32 @ 32x64)
def test_per_tensor_current_small(fq, orc):
    A, B = workloads.per_tensor_inputs()
    qa, _, sa, aa = fq.quantize(to_dev(A), TENSOR, E4M3)
    qb, _, sb, ab = fq.quantize(to_dev(B), TENSOR, E4M3, transpose_out=True)
    oqa, osa = orc.quantize_tensor_current(A, E4M3)
    oqb, osb = orc.quantize_tensor_current(B, E4M3, transpose=True)
    assert _f32(sa) == osa and _f32(sb) == osb
    assert _f32(aa) == orc.amax(A) and _f32(ab) == orc.amax(B)
    assert same(host(qa), oqa) and same(host(qb), oqb)


# ------------------------------------------------------------------ delayed scaling, 16 steps
def test_delayed_sixteen_steps_full_size(fq, orc):
    L = 1024
    st = {op: (torch.ones(1, dtype=torch.float32, device=DEV), torch.zeros(L, dtype=torch.float32, device=DEV))
          for op in "ab"}
    ost = {op: (np.ones(1, np.float32), np.zeros(L, np.float32)) for op in "ab"}
    amax = torch.zeros(1, dtype=torch.float32, device=DEV)
    for t in range(16):
        A, B, _ = workloads.delayed_inputs(t)
        for op, x, tr in (("a", A, False), ("b", B, True)):
            scale, hist = st[op]
            q, _, _, _ = fq.quantize(to_dev(x), TENSOR, E4M3, transpose_out=tr, tensor_scale=scale,
                                     scale_is_input=True, amax_out=amax)
            oq, oa = orc.delayed_step(x, E4M3, ost[op][0], ost[op][1], transpose=tr)
            assert _f32(amax) == oa, (t, op)
            assert same(host(q), oq), (t, op)
            fq.fp8_history_update(hist, amax, scale, E4M3)
            # device state after the post-step update == oracle state after its in-step update
            # plus the next step's scale rule
            nxt = orc.compute_scale(orc.history_max(ost[op][1]), E4M3, ost[op][0][0])
            assert same(host(hist), ost[op][1]), (t, op)
            assert _f32(scale) == nxt, (t, op)


def test_history_update_edge_cases(fq, orc):
    for L in (1, 7, 1024, 4096):
        hist = np.abs(np.random.default_rng(L).standard_normal(L)).astype(np.float32)
        hist[::3] = 0.0
        dh = to_dev(hist)
        scale = torch.tensor([0.5], dtype=torch.float32, device=DEV)
        oscale = np.float32(0.5)
        for a in (3.5, 0.0, float("nan"), 1e-30, 2.0):
            fq.fp8_history_update(dh, torch.tensor([a], dtype=torch.float32, device=DEV), scale, E5M2)
            orc.history_roll_insert(hist, a)
            oscale = orc.compute_scale(orc.history_max(hist), E5M2, oscale)
            assert np.array_equal(host(dh), hist, equal_nan=True), (L, a)
            assert _f32(scale) == oscale, (L, a)
    # a zero history keeps the old scale and the newest amax lands at index 0 (Flax page worked example)
    h = torch.zeros(1024, dtype=torch.float32, device=DEV)
    s = torch.ones(1, dtype=torch.float32, device=DEV)
    fq.fp8_history_update(h, torch.tensor([0.0], device=DEV), s, E4M3)
    assert _f32(s) == 1.0
    fq.fp8_history_update(h, torch.tensor([3.0], device=DEV), s, E4M3)
    assert host(h)[0] == 3.0 and _f32(s) == np.float32(3.0) / np.float32(448.0)


# ------------------------------------------------------------------ fine-grained block scaling
def test_block_full_size(fq, orc):
    X, W = workloads.fine_grained_inputs()
    qx, sx, _, _ = fq.quantize(to_dev(X), BLOCK, E4M3, block=(1, 128))
    qw, sw, _, _ = fq.quantize(to_dev(W), BLOCK, E4M3, block=(128, 128))
    assert tuple(sw.shape) == (16, 56) and tuple(sx.shape) == (4096, 56)
    oqx, osx = orc.quantize_block(X, E4M3, 1, 128)
    oqw, osw = orc.quantize_block(W, E4M3, 128, 128)
    assert same(host(sx), osx) and same(host(sw), osw)
    assert same(host(qx), oqx) and same(host(qw), oqw)


# ------------------------------------------------------------------ MX at full size
def test_mx_full_size(fq, orc):
    """Both 8192 x 8192 MXFP8 operands, every byte and every E8M0 exponent."""
    A, B = workloads.mx_inputs()
    for name, x in (("A", A), ("B", B)):
        q, e, _, _ = fq.quantize(to_dev(x), MX, E4M3)
        oq, oe = orc.quantize_mx(x, E4M3)
        assert same(host(e), oe, name + " e") and same(host(q), oq, name + " q")


def test_mx_past_2g_elements(fq, orc):
    """A bf16 input of more than 2^31 elements (4 GiB): the row kernel's 64-bit indexing; rows around
    element 2^31 and the last rows are checked."""
    rows, cols = (1 << 20) + 64, 2048
    gen = torch.Generator(device=DEV)
    gen.manual_seed(13)
    x = torch.randn(rows, cols, dtype=torch.bfloat16, device=DEV, generator=gen)
    q, e, _, _ = fq.quantize(x, MX, E4M3)
    boundary = (1 << 31) // cols
    sel = np.unique(np.concatenate([np.arange(0, 16), np.arange(boundary - 32, boundary + 32), np.arange(rows - 32, rows)]))
    st = torch.from_numpy(sel).to(DEV)
    hx, hq, he = host(x[st]), host(q[st]), host(e[st])
    del x, q, e
    torch.cuda.empty_cache()
    oq, oe = orc.quantize_mx(np.ascontiguousarray(hx), E4M3)
    assert same(hq, oq) and same(he, oe)


# ------------------------------------------------------------------ MOSS, six copies at full size
def test_moss_full_size_six_copies(fq, orc):
    """X, W (E4M3) and dY (E5M2) of the MOSS workload, each in both copies (groups along its rows
    and, transposed, along its columns with the same S): every byte and exponent, S and amax."""
    X, W, dY = workloads.moss_inputs()
    for name, x, fmt in (("X", X, E4M3), ("W", W, E4M3), ("dY", dY, E5M2)):
        xd = to_dev(x)
        q, e, S, am = fq.quantize(xd, MOSS, fmt)
        qt, et, _, _ = fq.quantize(xd, MOSS, fmt, transpose_out=True, tensor_scale=S, scale_is_input=True)
        oq, oe, oqt, oet, oS = moss_oracle_copies(orc, name, x, fmt)
        assert _f32(S) == oS and _f32(am) == orc.amax(x)
        assert same(host(e), oe, name + " e") and same(host(q), oq, name + " q")
        assert same(host(et), oet, name + " et") and same(host(qt), oqt, name + " qt")


# ------------------------------------------------------------------ every scheme, small shapes
CASES = [
    # (rows, cols, transpose, block)  -- fast row/transposed kernels and the generic fallback
    (256, 384, False, (1, 128)), (256, 384, True, (1, 128)), (384, 256, False, (128, 128)),
    (96, 200, False, (32, 32)), (100, 200, False, (1, 128)), (64, 40, False, (1, 128)),
    (40, 64, True, (1, 128)), (256, 72, True, (1, 128)), (200, 96, True, (128, 128)),
]


@pytest.mark.parametrize("mode", [TENSOR, BLOCK, MX, MOSS])
@pytest.mark.parametrize("fmt", [E4M3, E5M2])
@pytest.mark.parametrize("rows,cols,tr,block", CASES)
@pytest.mark.parametrize("bf16", [True, False])
def test_schemes_small_shapes(fq, orc, mode, fmt, rows, cols, tr, block, bf16):
    x = workloads.random_matrix(rows * 7 + cols, rows, cols, 3.0, bf16=bf16)
    if bf16:
        xf = workloads.bf16_bits_to_f32(x)
        xf[1, 3] *= 200.0
        x = workloads.to_bf16_bits(xf)
    else:
        x[1, 3] *= 200.0
    xd = to_dev(x)
    if mode == TENSOR:
        q, _, s, a = fq.quantize(xd, mode, fmt, transpose_out=tr)
        oq, os_ = orc.quantize_tensor_current(x, fmt, transpose=tr)
        assert _f32(s) == os_ and same(host(q), oq)
    elif mode == BLOCK:
        q, s, _, _ = fq.quantize(xd, mode, fmt, block=block, transpose_out=tr)
        oq, os_ = orc.quantize_block(x, fmt, block[0], block[1], transpose=tr)
        assert same(host(s), os_) and same(host(q), oq)
    elif mode == MX:
        q, e, _, _ = fq.quantize(xd, mode, fmt, transpose_out=tr)
        oq, oe = orc.quantize_mx(x, fmt, transpose=tr)
        assert same(host(e), oe) and same(host(q), oq)
    else:
        q, e, S, _ = fq.quantize(xd, mode, fmt, transpose_out=tr)
        oq, oe, oS = orc.quantize_moss(x, fmt, transpose=tr)
        assert _f32(S) == oS and same(host(e), oe) and same(host(q), oq)


# ------------------------------------------------------------------ special values and guards
def _special_matrix(seed):
    rng = np.random.default_rng(seed)
    x = (rng.standard_normal((64, 256)) * np.exp(rng.uniform(-30, 30, (64, 1)))).astype(np.float32)
    x[0, :8] = [np.nan, -np.nan, np.inf, -np.inf, -0.0, 0.0, 1e-45, -1e-40]
    x[5, 40] = 3e38
    x[7, 100:108] = [2.0 ** -100, -(2.0 ** -97), 2.0 ** -126, 1e-39, 5e-39, -6e-39, 2.0 ** 61, -(2.0 ** 60)]
    x[9] = 0.0
    x[10, 64:96] = np.float32(1e-30) * rng.standard_normal(32).astype(np.float32)
    return x


@pytest.mark.parametrize("mode", [TENSOR, BLOCK, MX, MOSS])
@pytest.mark.parametrize("fmt", [E4M3, E5M2])
@pytest.mark.parametrize("tr", [False, True])
def test_special_values(fq, orc, mode, fmt, tr):
    x = _special_matrix(3)
    if mode == MOSS:
        x[0, :4] = 1.0                  # keep the tensor amax finite so S is a real scale
    xd = to_dev(x)
    if mode == TENSOR:
        for s in (1.0, 3.7e-5, 1e-30, 1e30, 2.0 ** -64, 2.0 ** 64, 0.0123):
            sd = torch.tensor([s], dtype=torch.float32, device=DEV)
            q, _, _, _ = fq.quantize(xd, mode, fmt, transpose_out=tr, tensor_scale=sd, scale_is_input=True)
            assert same(host(q), orc.quantize_tensor(x, fmt, s, transpose=tr)), s
        # current scaling: 16384 values take the one-workgroup kernel, twice as many the amax pass
        # and the cast kernel
        for xc in (x, np.ascontiguousarray(np.concatenate([x, x[::-1]]))):
            q, _, s, _ = fq.quantize(to_dev(xc), mode, fmt, transpose_out=tr)
            oq, os_ = orc.quantize_tensor_current(xc, fmt, transpose=tr)
            assert (_f32(s) == os_) and same(host(q), oq)
    elif mode == BLOCK:
        q, s, _, _ = fq.quantize(xd, mode, fmt, block=(1, 128), transpose_out=tr)
        oq, os_ = orc.quantize_block(x, fmt, 1, 128, transpose=tr)
        assert same(host(s), os_) and same(host(q), oq)
    elif mode == MX:
        q, e, _, _ = fq.quantize(xd, mode, fmt, transpose_out=tr)
        oq, oe = orc.quantize_mx(x, fmt, transpose=tr)
        assert same(host(e), oe) and same(host(q), oq)
    else:
        for S in (None, 1e-20, 3.0):
            if S is None:
                q, e, Sd, _ = fq.quantize(xd, mode, fmt, transpose_out=tr)
                oq, oe, oS = orc.quantize_moss(x, fmt, transpose=tr)
                assert _f32(Sd) == oS
            else:
                sd = torch.tensor([S], dtype=torch.float32, device=DEV)
                q, e, _, _ = fq.quantize(xd, mode, fmt, transpose_out=tr, tensor_scale=sd, scale_is_input=True)
                oq, oe = orc.quantize_moss_given(x, fmt, S, transpose=tr)
            assert same(host(e), oe) and same(host(q), oq), S


@pytest.mark.parametrize("fmt", [E4M3, E5M2])
def test_all_bf16_patterns_and_midpoint_quotients(fq, orc, fmt):
    """Every bf16 bit pattern through the per-tensor cast at several scales, and fp32 dividends
    whose quotient lands within a few ulps of every FP8 rounding midpoint (the exact-division
    fast path must agree with IEEE division there)."""
    allb = np.arange(65536, dtype=np.uint16).reshape(256, 256)
    xd = to_dev(allb)
    # 0x3AFFFFFF and 0x3D61368B: scales whose two-term reciprocal is off for some bf16 significand
    # (1/s sits next to a rounding midpoint), so the bf16 casts must take the exact division there;
    # 0x3DB6DB6E: RN(1/s) > 1/s, where a careless two-term product turns -0 into +0
    odd = [float(np.array([b], np.uint32).view(np.float32)[0]) for b in (0x3AFFFFFF, 0x3D61368B, 0x3DB6DB6E)]
    for s in [1.0, 0.0123, 3.7e-5, 7.1e9, 2.0 ** -70] + odd:
        sd = torch.tensor([s], dtype=torch.float32, device=DEV)
        for tr in (False, True):
            q, _, _, _ = fq.quantize(xd, TENSOR, fmt, tensor_scale=sd, scale_is_input=True, transpose_out=tr)
            assert same(host(q), orc.quantize_tensor(allb, fmt, s, transpose=tr)), (s, tr)
            q, e, _, _ = fq.quantize(xd, MOSS, fmt, tensor_scale=sd, scale_is_input=True, transpose_out=tr)
            oq, oe = orc.quantize_moss_given(allb, fmt, s, transpose=tr)
            assert same(host(e), oe) and same(host(q), oq), (s, tr)
    q, e, _, _ = fq.quantize(xd, MX, fmt)
    oq, oe = orc.quantize_mx(allb, fmt)
    assert same(host(e), oe) and same(host(q), oq)
    from tests import brute
    vals = sorted(float(brute.fp8_value(c, fmt)) for c in brute.finite_codes(fmt) if c < 0x80)
    mids = np.array([(a + b) / 2 for a, b in zip(vals[:-1], vals[1:])], np.float64)
    rng = np.random.default_rng(fmt)
    for s in (np.float32(0.0123), np.float32(1.7e-3), np.float32(rng.uniform(1, 2)) * np.float32(2.0 ** -20)):
        base = (mids * float(s)).astype(np.float32)
        offs = np.arange(-8, 8, dtype=np.int64)
        xs = (base.view(np.uint32).astype(np.int64)[:, None] + offs[None, :]).astype(np.uint32).view(np.float32)
        xs = np.concatenate([xs.reshape(-1), -xs.reshape(-1)])
        xs = np.resize(xs, (len(xs) + 255) // 256 * 256).reshape(-1, 256)
        sd = torch.tensor([s], dtype=torch.float32, device=DEV)
        q, _, _, _ = fq.quantize(to_dev(xs), TENSOR, fmt, tensor_scale=sd, scale_is_input=True)
        assert same(host(q), orc.quantize_tensor(xs, fmt, s)), s
        # bf16 dividends next to the same midpoints (the two-term reciprocal path)
        xb = workloads.to_bf16_bits(xs)
        xb = np.concatenate([xb, (xb.astype(np.int64) + 1).astype(np.uint16), (xb.astype(np.int64) - 1).astype(np.uint16)])
        q, _, _, _ = fq.quantize(to_dev(xb), TENSOR, fmt, tensor_scale=sd, scale_is_input=True)
        assert same(host(q), orc.quantize_tensor(xb, fmt, s)), s


def test_cast_determinism(fq):
    X, _, _ = workloads.moss_inputs(tokens=2048, d_in=1024, d_out=64)
    xd = to_dev(X)
    a = [host(t) for t in fq.quantize(xd, MOSS, E4M3, transpose_out=True)[:3]]
    b = [host(t) for t in fq.quantize(xd, MOSS, E4M3, transpose_out=True)[:3]]
    assert all(np.array_equal(u, v) for u, v in zip(a, b))
