"""GPU parity of the dual-axis cast (fp8_quantize_dual): both copies of one operand -- groups along
its columns and, transposed, along its rows -- against the CPU oracle's single-copy casts, bit for
bit (FP8 bytes, E8M0 exponents, tensor scale, amax).  Shapes cover the one-pass kernel (rows and
cols multiples of 32, partial 128 x 64 tiles) and the two-cast path for other shapes."""
import numpy as np
import pytest
import torch

from fp8_scaled_quantization_amd import workloads
from tests.gpu_util import DEV, host, moss_oracle_copies, same, to_dev

pytestmark = pytest.mark.gpu

E4M3, E5M2 = 0, 1
TENSOR, MX, MOSS = 0, 2, 3


@pytest.fixture(scope="module")
def fq():
    import fp8_scaled_quantization_amd as fq
    fq.init()
    return fq


def _f32(t):
    return np.float32(host(t)[0])


SHAPES = [(32, 32), (128, 64), (96, 160), (256, 192), (160, 96), (384, 288),   # one pass
          (40, 64), (64, 40), (100, 200)]                                         # two single casts


@pytest.mark.parametrize("mode", [TENSOR, MX, MOSS])
@pytest.mark.parametrize("fmt", [E4M3, E5M2])
@pytest.mark.parametrize("rows,cols", SHAPES)
@pytest.mark.parametrize("bf16", [True, False])
def test_dual_small_shapes(fq, orc, mode, fmt, rows, cols, bf16):
    x = workloads.random_matrix(rows * 13 + cols, rows, cols, 3.0, bf16=bf16)
    if bf16:
        xf = workloads.bf16_bits_to_f32(x)
        xf[1, 3] *= 200.0
        xf[rows - 1, cols - 1] = -0.0
        x = workloads.to_bf16_bits(xf)
    else:
        x[1, 3] *= 200.0
        x[rows - 1, cols - 1] = -0.0
    xd = to_dev(x)
    q, s, qt, st, S, am = fq.quantize_dual(xd, mode, fmt)
    if mode == TENSOR:
        oq, os_ = orc.quantize_tensor_current(x, fmt)
        oqt, _ = orc.quantize_tensor_current(x, fmt, transpose=True)
        assert _f32(S) == os_ and _f32(am) == orc.amax(x)
        assert same(host(q), oq, "q") and same(host(qt), oqt, "qt")
    elif mode == MX:
        oq, oe = orc.quantize_mx(x, fmt)
        oqt, oet = orc.quantize_mx(x, fmt, transpose=True)
        assert same(host(s), oe, "e") and same(host(q), oq, "q")
        assert same(host(st), oet, "et") and same(host(qt), oqt, "qt")
    else:
        oq, oe, oS = orc.quantize_moss(x, fmt)
        oqt, oet, _ = orc.quantize_moss(x, fmt, transpose=True)
        assert _f32(S) == oS and _f32(am) == orc.amax(x)
        assert same(host(s), oe, "e") and same(host(q), oq, "q")
        assert same(host(st), oet, "et") and same(host(qt), oqt, "qt")


@pytest.mark.parametrize("fmt", [E4M3, E5M2])
def test_dual_given_scale_fused_amax_and_specials(fq, orc, fmt):
    """Given-scale TENSOR with the fused amax (delayed scaling), given-S MOSS, and special values
    (NaN, Inf, -0, subnormals, huge and tiny rows) through the one-pass kernel."""
    rng = np.random.default_rng(7 + fmt)
    x = (rng.standard_normal((96, 256)) * np.exp(rng.uniform(-30, 30, (96, 1)))).astype(np.float32)
    x[0, :8] = [np.nan, -np.nan, np.inf, -np.inf, -0.0, 0.0, 1e-45, -1e-40]
    x[5, 40] = 3e38
    x[7, 100:108] = [2.0 ** -100, -(2.0 ** -97), 2.0 ** -126, 1e-39, 5e-39, -6e-39, 2.0 ** 61, -(2.0 ** 60)]
    x[9] = 0.0
    for xin in (x, workloads.to_bf16_bits(x)):
        xd = to_dev(xin)
        for s in (1.0, 3.7e-5, 2.0 ** -64, 0.0123):
            sd = torch.tensor([s], dtype=torch.float32, device=DEV)
            am = torch.full((1,), 123.0, dtype=torch.float32, device=DEV)
            q, _, qt, _, _, _ = fq.quantize_dual(xd, TENSOR, fmt, tensor_scale=sd, scale_is_input=True, amax_out=am)
            assert same(host(q), orc.quantize_tensor(xin, fmt, s), "q") and \
                same(host(qt), orc.quantize_tensor(xin, fmt, s, transpose=True), "qt"), s
            oa = orc.amax(xin)
            assert (np.isnan(oa) and np.isnan(_f32(am))) or _f32(am) == oa
            assert _f32(sd) == np.float32(s)
        for S in (1e-20, 3.0, 0.0123):
            sd = torch.tensor([S], dtype=torch.float32, device=DEV)
            q, e, qt, et, _, _ = fq.quantize_dual(xd, MOSS, fmt, tensor_scale=sd, scale_is_input=True)
            oq, oe = orc.quantize_moss_given(xin, fmt, S)
            oqt, oet = orc.quantize_moss_given(xin, fmt, S, transpose=True)
            assert same(host(e), oe) and same(host(q), oq) and same(host(et), oet) and same(host(qt), oqt), S
        q, e, qt, et, _, _ = fq.quantize_dual(xd, MX, fmt)
        oq, oe = orc.quantize_mx(xin, fmt)
        oqt, oet = orc.quantize_mx(xin, fmt, transpose=True)
        assert same(host(e), oe) and same(host(q), oq) and same(host(et), oet) and same(host(qt), oqt)


def test_dual_moss_full_size(fq, orc):
    """The MOSS forward/backward operands at full size through the one-pass dual cast: S and amax
    exact, every byte and exponent of both copies against the oracle."""
    X, W, dY = workloads.moss_inputs()
    for name, x, fmt in (("X", X, E4M3), ("W", W, E4M3), ("dY", dY, E5M2)):
        q, e, qt, et, S, am = fq.quantize_dual(to_dev(x), MOSS, fmt)
        oq, oe, oqt, oet, oS = moss_oracle_copies(orc, name, x, fmt)
        assert _f32(S) == oS and _f32(am) == orc.amax(x)
        assert same(host(e), oe, name + " e") and same(host(q), oq, name + " q")
        assert same(host(et), oet, name + " et") and same(host(qt), oqt, name + " qt")


def test_dual_empty(fq):
    x = torch.empty((0, 64), dtype=torch.bfloat16, device=DEV)
    q, e, qt, et, S, am = fq.quantize_dual(x, MOSS, E4M3)
    assert _f32(S) == 1.0 and _f32(am) == 0.0 and q.numel() == 0 and qt.numel() == 0


# tall bf16 operands take the band-run kernel: runs of 4, 8 (with a partial last run) and 16 bands
RUN_SHAPES = [(4096, 64), (8576, 192), (16384, 128)]


@pytest.mark.parametrize("rows,cols", RUN_SHAPES)
@pytest.mark.parametrize("fmt", [E4M3, E5M2])
def test_dual_band_runs_bit_exact(fq, orc, rows, cols, fmt):
    xf = workloads.bf16_bits_to_f32(workloads.random_matrix(rows + 7 * cols, rows, cols, 1.0))
    xf[:, 5] *= 60.0                                                   # an outlier channel
    xf[rows // 3, :4] = [np.nan, np.inf, -np.inf, -0.0]                # specials in one band
    xf[rows - 1, cols - 1] = 1e-40
    xf[200:232, 17] = 0.0                                              # an all-zero 32-group
    x = workloads.to_bf16_bits(xf)
    xd = to_dev(x)
    q, s, qt, st, S, am = fq.quantize_dual(xd, MOSS, fmt)
    oq, oe, oS = orc.quantize_moss(x, fmt)
    oqt, oet, _ = orc.quantize_moss(x, fmt, transpose=True)
    assert _f32(S) == oS or (np.isnan(oS) and np.isnan(_f32(S)))
    assert same(host(s), oe, "e") and same(host(q), oq, "q") and same(host(st), oet, "et") and same(host(qt), oqt, "qt")
    q, s, qt, st, _, _ = fq.quantize_dual(xd, MX, fmt)
    oq, oe = orc.quantize_mx(x, fmt)
    oqt, oet = orc.quantize_mx(x, fmt, transpose=True)
    assert same(host(s), oe, "e") and same(host(q), oq, "q") and same(host(st), oet, "et") and same(host(qt), oqt, "qt")
    sd = torch.tensor([0.0123], dtype=torch.float32, device=DEV)
    am = torch.zeros(1, dtype=torch.float32, device=DEV)
    q, _, qt, _, _, _ = fq.quantize_dual(xd, TENSOR, fmt, tensor_scale=sd, scale_is_input=True, amax_out=am)
    assert same(host(q), orc.quantize_tensor(x, fmt, 0.0123), "q") and \
        same(host(qt), orc.quantize_tensor(x, fmt, 0.0123, transpose=True), "qt")
    assert np.isnan(_f32(am)) and np.isnan(orc.amax(x))
    xf[rows // 3, :4] = 1.0                                            # finite tensor: current scaling
    x = workloads.to_bf16_bits(xf)
    q, _, qt, _, S, am = fq.quantize_dual(to_dev(x), TENSOR, fmt)
    oq, os_ = orc.quantize_tensor_current(x, fmt)
    assert _f32(S) == os_ and _f32(am) == orc.amax(x)
    assert same(host(q), oq, "q") and same(host(qt), orc.quantize_tensor(x, fmt, os_, transpose=True), "qt")
    q, s, qt, st, S, _ = fq.quantize_dual(to_dev(x), MOSS, fmt)
    oq, oe, oS = orc.quantize_moss(x, fmt)
    oqt, oet, _ = orc.quantize_moss(x, fmt, transpose=True)
    assert _f32(S) == oS
    assert same(host(s), oe, "e") and same(host(q), oq, "q") and same(host(st), oet, "et") and same(host(qt), oqt, "qt")
