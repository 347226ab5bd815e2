"""GPU parity of the next-step entry points against the oracle, through the C ABI: history merge,
automatic weight scaling, UE8M0 block quantization, the exact fp32 -> UE8M0 conversion, block
dequantization (all bit-exact), and the block-scaled GEMM with UE8M0 weight scales and with a
static per-tensor activation scale (within the elementwise bound of tests/gpu_util.py)."""
import numpy as np
import pytest
import torch

from fp8_scaled_quantization_amd import workloads
from tests.gpu_util import DEV, check_gemm, host, reference_terms, same, to_dev

pytestmark = pytest.mark.gpu

E4M3, E5M2 = 0, 1
TENSOR, BLOCK, MX, MOSS, BLOCK_E8M0 = 0, 1, 2, 3, 4
OUT_F32, OUT_BF16 = 0, 1


@pytest.fixture(scope="module")
def fq():
    import fp8_scaled_quantization_amd as fq
    fq.init()
    return fq


def f32dev(a):
    return torch.from_numpy(np.ascontiguousarray(a, np.float32)).to(DEV)


# ------------------------------------------------------------------ history merge
@pytest.mark.parametrize("n", [1, 1024, 4000])
def test_history_merge_bit_exact(fq, orc, n):
    rng = np.random.default_rng(n)
    a = rng.standard_exponential(n).astype(np.float32)
    b = rng.standard_exponential(n).astype(np.float32)
    if n > 8:
        a[3], b[4], a[6], b[6] = np.nan, np.nan, -np.inf, 7.0
    sa, sb = np.array([0.5], np.float32), np.array([0.25], np.float32)
    hd, hs, sd, ss = f32dev(a), f32dev(b), f32dev(sa), f32dev(sb)
    fq.fp8_history_merge(hd, hs, sd, ss)
    want_h, want_s = a.copy(), sa.copy()
    orc.history_merge(want_h, want_s, b, sb[0])
    assert same(host(hd), want_h, "merged history") and same(host(sd), want_s, "merged scale")


def test_history_merge_worked_example_on_gpu(fq, orc):
    """Flax page section 5.3 on the device: two delayed-scaling uses of one state (scale 1, 1024
    zeros) by 2.0 and by 3.0, each followed by its history update, merged by max.  The page prints
    the scale each use quantized with (1.0) and the merged history ([3, 0, ...]); in this ABI's
    post-step order the state then carries the next step's scale, fl(max(history) / MAX)."""
    states = []
    for v in (2.0, 3.0):
        x = f32dev(np.array([[v, 0, 0, 0, 0, 0, 0, 0]], np.float32))
        scale = torch.ones(1, device=DEV)
        hist = torch.zeros(1024, device=DEV)
        amax = torch.zeros(1, device=DEV)
        q = torch.empty((1, 8), dtype=torch.uint8, device=DEV)
        fq.fp8_quantize(TENSOR, E4M3, x, q, None, scale, True, amax)
        used = host(scale)[0]                       # the scale this use quantized with
        fq.fp8_history_update(hist, amax, scale, E4M3)
        states.append((hist, scale, used))
    (h1, s1, u1), (h2, s2, u2) = states
    fq.fp8_history_merge(h1, h2, s1, s2)
    h, s = host(h1), host(s1)
    assert u1 == u2 == 1.0
    assert h[0] == 3.0 and np.all(h[1:] == 0.0) and h.size == 1024
    assert s[0] == orc.compute_scale(3.0, E4M3, 1.0)


# ------------------------------------------------------------------ automatic scaling
@pytest.mark.parametrize("fmt", [E4M3, E5M2])
def test_auto_scale_sequence_bit_exact(fq, orc, fmt):
    rng = np.random.default_rng(20 + fmt)
    steps, interval = 1100, 500
    lrs = rng.uniform(1e-5, 3e-4, steps).astype(np.float32)
    maxes = (0.05 + 0.01 * rng.standard_normal(steps)).astype(np.float32)
    state_d = torch.zeros(2, device=DEV)
    scale_d = torch.zeros(1, device=DEV)
    state_h = np.zeros(2, np.float32)
    got, want = [], []
    for t in range(steps):
        rescale = t % interval == 0
        amax_d = f32dev(maxes[t:t + 1]) if rescale else None
        fq.fp8_auto_scale(state_d, rescale, amax_d, float(lrs[t]), fmt, scale_d)
        got.append(host(scale_d)[0])
        want.append(orc.auto_scale_step(state_h, rescale, maxes[t], lrs[t], fmt))
    assert same(np.array(got, np.float32), np.array(want, np.float32), "auto scales")
    assert same(host(state_d), state_h, "auto-scale state")


# ------------------------------------------------------------------ UE8M0 block quantization
def _special_block_input(seed):
    x = workloads.bf16_bits_to_f32(workloads.random_matrix(seed, 256, 384, 0.02)).copy()
    x[0:128, 0:128] = 0.0                                 # all-zero block: e = -127
    x[5, 200] = np.nan                                    # NaN block
    x[130, 10] = np.inf                                   # Inf block: e = 127, clipped to MAX
    x[140, 300] = 3.0e38
    x[200, 260] = 1e-30
    return x


@pytest.mark.parametrize("fmt", [E4M3, E5M2])
@pytest.mark.parametrize("case", ["fine-grained W", "ragged", "blocks 32x32", "transposed", "specials"])
def test_block_e8m0_quantize_bit_exact(fq, orc, fmt, case):
    br, bc, transpose = 128, 128, False
    if case == "fine-grained W":
        _, W = workloads.fine_grained_inputs()
        x = W
    elif case == "ragged":
        x = workloads.random_matrix(31, 300, 264, 0.05)
    elif case == "blocks 32x32":
        x = workloads.random_matrix(32, 256, 512, 1.0)
        br = bc = 32
    elif case == "transposed":
        x = workloads.random_matrix(33, 384, 256, 1.0)
        transpose = True
    else:
        x = _special_block_input(34)
    q, e, _, _ = fq.quantize(to_dev(x), BLOCK_E8M0, fmt, block=(br, bc), transpose_out=transpose)
    wq, we = orc.quantize_block_e8m0(x, fmt, br, bc, transpose=transpose)
    assert same(host(q), wq, case + " bytes") and same(host(e), we, case + " E8M0")


def test_scale_to_e8m0_bit_exact(fq, orc):
    e = np.arange(-127, 128)
    s = np.concatenate([np.ldexp(np.float32(1.0), e).astype(np.float32),
                        np.array([3.0, 0.75, 0.0, -2.0, np.inf, np.nan, 2.0 ** -128, 1.0 + 2.0 ** -23], np.float32)])
    got = torch.empty(s.size, dtype=torch.uint8, device=DEV)
    bad = torch.full((1,), 99, dtype=torch.int32, device=DEV)
    fq.fp8_scale_to_e8m0(f32dev(s), got, bad)
    want, nbad = orc.scales_f32_to_e8m0(s)
    assert same(host(got), want, "e8m0 bytes") and int(host(bad)[0]) == nbad == 8
    with pytest.raises(ValueError):
        fq.scale_to_e8m0(f32dev(s))
    assert np.array_equal(host(fq.scale_to_e8m0(f32dev(s[:255]))), want[:255])


# ------------------------------------------------------------------ block dequantize
@pytest.mark.parametrize("mode", [BLOCK, BLOCK_E8M0])
@pytest.mark.parametrize("out", [OUT_BF16, OUT_F32])
@pytest.mark.parametrize("shape", [(2048, 7168), (300, 264), (256, 512)])
@pytest.mark.parametrize("fmt", [E4M3, E5M2])
def test_block_dequantize_bit_exact(fq, orc, mode, out, shape, fmt):
    R, C = shape
    x = workloads.random_matrix(R + C + mode, R, C, 0.05)
    if mode == BLOCK:
        wq, ws = orc.quantize_block(x, fmt, 128, 128)
    else:
        wq, ws = orc.quantize_block_e8m0(x, fmt, 128, 128)
    if shape == (256, 512):
        wq = np.arange(R * C, dtype=np.uint32).astype(np.uint8).reshape(R, C)     # every code, NaN included
    qd = torch.from_numpy(np.ascontiguousarray(wq)).to(DEV)
    sd = torch.from_numpy(np.ascontiguousarray(ws)).to(DEV)
    got = host(fq.block_dequantize(mode, fmt, qd, sd, (128, 128), out))
    want = orc.block_dequantize(mode, wq, fmt, ws, (128, 128), out_bf16=out == OUT_BF16)
    # NaN codes decode to NaN on both sides; a NaN's sign and payload carry no value, so NaN
    # positions are compared as a set and every other output bit for bit
    if out == OUT_F32:
        gnan, wnan = np.isnan(got), np.isnan(want)
        gb, wb = got.view(np.uint32), want.view(np.uint32)
    else:
        gnan, wnan = (got & 0x7FFF) > 0x7F80, (want & 0x7FFF) > 0x7F80
        gb, wb = got, want
    assert np.array_equal(gnan, wnan)
    assert same(gb[~wnan], wb[~wnan], "dequant")


# ------------------------------------------------------------------ GEMM: UE8M0 weights, static activations
def _offset_view(t, offset):
    """A copy of t that starts `offset` bytes into a fresh byte buffer (a view the caller might
    hand over when its scales sit inside a larger allocation)."""
    buf = torch.zeros(t.numel() * t.element_size() + 16, dtype=torch.uint8, device=t.device)
    v = buf[offset:offset + t.numel() * t.element_size()].view(t.dtype).view(t.shape)
    v.copy_(t)
    return v


def _gemm_case(fq, orc, M, N, K, wmode, static_a, seed, scale_offset=0):
    """Every output of one block-scaled GEMM against the oracle's fp64 product of the same bytes."""
    X = workloads.random_matrix(seed, M, K, 1.0)
    W = workloads.random_matrix(seed + 1, N, K, 0.02)
    if static_a:
        sa = np.float32(orc.amax(X) / 448.0 * 1.25)      # a supplied (calibrated) activation scale
        sad = f32dev(np.array([sa], np.float32))
        qx, _, _, _ = fq.quantize(to_dev(X), TENSOR, E4M3, tensor_scale=sad, scale_is_input=True)
        hqx = host(qx)
        deqA = lambda rows: orc.dequantize(TENSOR, np.ascontiguousarray(hqx[rows]), E4M3, None, sa)
        Ascale, Aglobal = None, sad
    else:
        qx, sx, _, _ = fq.quantize(to_dev(X), BLOCK, E4M3, block=(1, 128))
        hqx, hsx = host(qx), host(sx)
        deqA = lambda rows: orc.dequantize(BLOCK, np.ascontiguousarray(hqx[rows]), E4M3,
                                           np.ascontiguousarray(hsx[rows]), block=(1, 128))
        Ascale, Aglobal = sx, None
    qw, sw, _, _ = fq.quantize(to_dev(W), wmode, E4M3, block=(128, 128))
    hqw, hsw = host(qw), host(sw)
    if scale_offset:
        sw = _offset_view(sw, scale_offset)
        assert sw.data_ptr() % 4 == scale_offset % 4
    deqB = lambda rows: orc.dequantize(wmode, np.ascontiguousarray(hqw[rows]), E4M3,
                                       np.ascontiguousarray(hsw[rows // 128]), block=(1, 128))
    C32 = torch.empty((M, N), dtype=torch.float32, device=DEV)
    Cbf = torch.empty((M, N), dtype=torch.bfloat16, device=DEV)
    fq.fp8_scaled_gemm(wmode, qx, E4M3, Ascale, qw, E4M3, sw, Aglobal, None, C32, OUT_F32)
    fq.fp8_scaled_gemm(wmode, qx, E4M3, Ascale, qw, E4M3, sw, Aglobal, None, Cbf, OUT_BF16)
    label = "mode %d static %d %dx%dx%d" % (wmode, static_a, M, N, K)
    Ad, Bd = deqA(np.arange(M)), deqB(np.arange(N))
    Cref, D, E, _ = reference_terms(orc, Ad, Bd, promoted=True)
    return check_gemm(host(C32), host(Cbf), Cref, D, E, K, label)


@pytest.mark.parametrize("wmode", [BLOCK, BLOCK_E8M0])
@pytest.mark.parametrize("static_a", [False, True])
@pytest.mark.parametrize("M,N,K", [(200, 136, 384), (256, 384, 1024), (300, 260, 256)])
def test_block_gemm_weight_and_activation_scale_kinds(fq, orc, wmode, static_a, M, N, K):
    _gemm_case(fq, orc, M, N, K, wmode, static_a, M + N + K)


@pytest.mark.parametrize("offset", [1, 2, 3])
@pytest.mark.parametrize("M,N,K", [(256, 384, 1024), (300, 260, 256), (200, 136, 384)])
def test_block_gemm_ue8m0_weight_scales_at_any_byte(fq, orc, offset, M, N, K):
    """UE8M0 weight-block scales handed over at a byte offset of 1-3 within a word: the kernels
    must pick each scale's own byte, whatever the array's alignment."""
    _gemm_case(fq, orc, M, N, K, BLOCK_E8M0, False, M + N + K + offset, scale_offset=offset)


def test_gemm_misaligned_word_scales_are_refused(fq):
    """Scale arrays the kernels read in 4-byte words (MX/MOSS E8M0 rows, fp32 block scales) must
    be 4-byte aligned: an offset view is refused with FP8Q_ERR_UNSUPPORTED, not misread."""
    A = torch.zeros((256, 256), dtype=torch.uint8, device=DEV)
    e = torch.full((256, 8), 127, dtype=torch.uint8, device=DEV)
    C = torch.empty((256, 256), dtype=torch.bfloat16, device=DEV)
    with pytest.raises(fq.Fp8qError) as ei:
        fq.fp8_scaled_gemm(MX, A, E4M3, _offset_view(e, 1), A, E4M3, e, None, None, C, OUT_BF16)
    assert ei.value.code == -2


@pytest.mark.parametrize("wmode,static_a", [(BLOCK_E8M0, False), (BLOCK, True), (BLOCK_E8M0, True)])
def test_block_gemm_fine_grained_full_size(fq, orc, wmode, static_a):
    _gemm_case(fq, orc, 4096, 2048, 7168, wmode, static_a, 3)


# ------------------------------------------------------------------ delayed-scaling backward
def test_delayed_forward_backward_steps(fq, orc):
    """A linear layer trained with delayed scaling: three delayed states (input and kernel in E4M3,
    output gradient in E5M2) drive Y = X W^T, dX = dY W and dW = dY^T X ("Flax FP8 量化实战指南 ...",
    section 3.3: the backward quantizes the incoming gradient to E5M2 under its own state).  Each
    operand is quantized once into both layouts (post-step history updates), and every byte,
    amax, history and scale equals the oracle's in-step replay; the GEMMs are within the bound."""
    M, I, O, L = 640, 384, 256, 1024
    fmts = {"x": E4M3, "w": E4M3, "g": E5M2}
    dev_st = {k: (torch.ones(1, dtype=torch.float32, device=DEV), torch.zeros(L, dtype=torch.float32, device=DEV))
              for k in fmts}
    orc_st = {k: (np.ones(1, np.float32), np.zeros(L, np.float32)) for k in fmts}
    W0 = workloads.bf16_bits_to_f32(workloads.random_matrix(900, O, I, 0.02))
    for t in range(6):
        rng = np.random.default_rng(1000 + t)
        sig = np.float32(np.exp(rng.uniform(np.log(0.1), np.log(10.0))))
        raw = {"x": workloads.random_matrix(1100 + t, M, I, float(sig)),
               "w": workloads.to_bf16_bits(W0 + workloads.bf16_bits_to_f32(workloads.random_matrix(1200 + t, O, I, 1e-4))),
               "g": workloads.random_matrix(1300 + t, M, O, float(1e-3 * sig))}
        if t == 4:
            raw["g"] = np.zeros_like(raw["g"])          # an all-zero gradient keeps the previous scale
        dq, oq, used = {}, {}, {}
        for k, fmt in fmts.items():
            scale, hist = dev_st[k]
            amax = torch.zeros(1, dtype=torch.float32, device=DEV)
            q, _, qt, _, _, _ = fq.quantize_dual(to_dev(raw[k]), TENSOR, fmt, tensor_scale=scale,
                                                 scale_is_input=True, amax_out=amax)
            osc, ohist = orc_st[k]
            oq_rows, oa = orc.delayed_step(raw[k], fmt, osc, ohist)
            oq_cols = orc.quantize_tensor(raw[k], fmt, osc[0], transpose=True)
            assert np.float32(host(amax)[0]) == oa, (t, k)
            assert same(host(q), oq_rows, "%s rows t=%d" % (k, t)) and same(host(qt), oq_cols, "%s cols t=%d" % (k, t))
            used[k] = np.float32(osc[0])
            dq[k] = (q, qt, scale.clone())
            oq[k] = (oq_rows, oq_cols)
            fq.fp8_history_update(hist, amax, scale, fmt)
            nxt = orc.compute_scale(orc.history_max(ohist), fmt, osc[0])
            assert np.array_equal(host(hist), ohist) and np.float32(host(scale)[0]) == nxt, (t, k)
        deq = lambda k, which: orc.dequantize(TENSOR, oq[k][which], fmts[k], None, used[k])
        cases = (("Y", ("x", 0), ("w", 0), I), ("dX", ("g", 0), ("w", 1), O), ("dW", ("g", 1), ("x", 1), M))
        for name, (ka, wa), (kb, wb), K in cases:
            C32 = fq.scaled_gemm(TENSOR, dq[ka][wa], fmts[ka], None, dq[kb][wb], fmts[kb], None,
                                 dq[ka][2], dq[kb][2], out_dtype=OUT_F32)
            Cbf = fq.scaled_gemm(TENSOR, dq[ka][wa], fmts[ka], None, dq[kb][wb], fmts[kb], None,
                                 dq[ka][2], dq[kb][2], out_dtype=OUT_BF16)
            Ad, Bd = deq(ka, wa), deq(kb, wb)
            Cref, D, E, Sg = reference_terms(orc, Ad, Bd)
            check_gemm(host(C32), host(Cbf), Cref, D, E, K, "%s t=%d" % (name, t), Sg)
