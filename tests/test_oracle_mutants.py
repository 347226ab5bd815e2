"""The oracle's pins must catch plausible mistakes.  Each case plants one mistake in a copy of
oracle.c (a text edit of the copy; the oracle itself is untouched), builds it, and runs the
oracle's pin tests against it in a subprocess: at least one pin must fail.  A mistake that no pin
caught would mean a wrong oracle could pass its own tests."""
import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
ORACLE_C = os.path.join(ROOT, "oracle", "oracle.c")
PINS = ["tests/test_oracle_codec.py", "tests/test_oracle_schemes.py", "tests/test_oracle_gemm.py",
        "tests/test_oracle_next.py"]

# name: (text in oracle.c, replacement) -- each text occurs exactly once
MUTANTS = {
    "FP8 ties round away from zero": (
        "else r = (c % 2 == 0) ? c : c + 1;", "else r = c + 1;"),
    "FP8 rounding truncates": (
        "if (a > midpoint) r = c + 1;", "if (a > above) r = c + 1;"),
    "E4M3 subnormal step off by a factor 2": (
        "if (e == 0) v = m * ldexp(1.0, -9);", "if (e == 0) v = m * ldexp(1.0, -10);"),
    "E5M2 exponent bias off by one": (
        "else v = (1.0 + m / 4.0) * ldexp(1.0, e - 15);", "else v = (1.0 + m / 4.0) * ldexp(1.0, e - 16);"),
    "scale is MAX / amax": (
        "float s = amax / (float)orc_fp8_max(fmt);", "float s = (float)orc_fp8_max(fmt) / amax;"),
    "quantize multiplies by the scale": (
        "float v = x / s;", "float v = x * s;"),
    "amax of signed values": (
        "float v = load_elem(x, in_kind, r * ld + c);\n            if (isnan(v)) nan_seen = 1;\n"
        "            else if (fabsf(v) > m) m = fabsf(v);",
        "float v = load_elem(x, in_kind, r * ld + c);\n            if (isnan(v)) nan_seen = 1;\n"
        "            else if (v > m) m = v;"),
    "power-of-two exponent search is strict": (
        "if (base * ldexp(1.0, e) >= target) return e;", "if (base * ldexp(1.0, e) > target) return e;"),
    "MX scales by 2^e instead of 2^-e": (
        "float f = (float)ldexp(1.0, -e);                      /* 2^-e, exact in fp32 */",
        "float f = (float)ldexp(1.0, e);"),
    "MOSS multiplies by the global factor": (
        "float v = (t[r * C + c] / S) * f;", "float v = (t[r * C + c] * S) * f;"),
    "MOSS group scale without the division by MAX": (
        "float s_i = amax_f32(t, C, r, r + 1, c0, c1) / M;", "float s_i = amax_f32(t, C, r, r + 1, c0, c1);"),
    "UE8M0 block scales by 2^e instead of 2^-e": (
        "e8m0[bi * nbc + bj] = (uint8_t)(e + 127);\n            float f = (float)ldexp(1.0, -e);",
        "e8m0[bi * nbc + bj] = (uint8_t)(e + 127);\n            float f = (float)ldexp(1.0, e);"),
    "fp32 -> UE8M0 conversion off by one": (
        "out[i] = (uint8_t)(ex - 1 + 127);", "out[i] = (uint8_t)(ex + 127);"),
    "block scales stored transposed": (
        "scales[bi * nbc + bj] = s;", "scales[bj * nbr + bi] = s;"),
    "history shift drops the wrapped entry": (
        "hist[len - 1] = first;", "hist[len - 1] = 0.0f;"),
    "history merge adds": (
        "hist_dst[i] = max_nan(hist_dst[i], hist_src[i]);", "hist_dst[i] = hist_dst[i] + hist_src[i];"),
    "delayed step scales by the current amax": (
        "float s = orc_compute_scale(orc_history_max(hist, len), fmt, *scale);",
        "float s = orc_compute_scale(orc_amax(x, in_kind, rows, cols, ld), fmt, *scale);"),
    "automatic scaling adds this step's learning rate early": (
        "float predicted = state[0] + state[1];", "float predicted = state[0] + state[1] + lr;"),
    "MOSS dequantization drops the global factor": (
        "if (mode == ORC_MOSS) s *= (double)*global;", "if (mode == ORC_MOSS) s *= 1.0;"),
    "bf16 rounding is half-up": (
        "u += 0x7FFFu + lsb;", "u += 0x8000u;"),
    "GEMM pairs A with reversed B": (
        "double p = a[k] * b[k];", "double p = a[k] * b[K - 1 - k];"),
    "error-size E sums instead of taking the max": (
        "if (fabs(p) > mx) mx = fabs(p);", "mx += fabs(p);"),
    "error-size Sigma includes the current chunk": (
        "sig += fabs(prefix);\n        prefix += part;", "prefix += part;\n        sig += fabs(prefix);"),
    "SNR as 20 log10 of a power ratio": (
        "return 10.0 * log10(sig / noise);", "return 20.0 * log10(sig / noise);"),
    "SNR noise as absolute differences": (
        "noise += d * d;", "noise += fabs(d);"),
    "E4M3 decodes every top-exponent code as NaN": (
        "if (e == 15 && m == 7) return NAN;", "if (e == 15) return NAN;"),
    "NaN encodes without its sign": (
        "if (isnan(v)) return (uint8_t)(sign | 0x7F);", "if (isnan(v)) return (uint8_t)0x7F;"),
    "scale of an infinite amax is not the fallback": (
        "if (!(amax > 0.0f) || isinf(amax)) return fallback;", "if (!(amax > 0.0f)) return fallback;"),
    "history inserts the newest amax at the end": (
        "hist[0] = amax_new;", "hist[len - 1] = amax_new;"),
    "automatic scaling keeps the sum at a rescale": (
        "state[1] = 0.0f;", "state[1] = state[1];"),
    "block dequantization swaps the block extents": (
        "else if (mode == ORC_BLOCK) s = (double)((const float*)scales)[(r / br) * nbc + k / bc];",
        "else if (mode == ORC_BLOCK) s = (double)((const float*)scales)[(r / bc) * nbc + k / br];"),
    "UE8M0 dequantization negates the exponent": (
        "s = ldexp(1.0, (int)((const uint8_t*)scales)[(r / br) * nbc + k / bc] - 127);",
        "s = ldexp(1.0, 127 - (int)((const uint8_t*)scales)[(r / br) * nbc + k / bc]);"),
    "MOSS global factor from the first row only": (
        "float S = orc_compute_scale(orc_amax(x, in_kind, rows, cols, ld), fmt, 1.0f);",
        "float S = orc_compute_scale(orc_amax(x, in_kind, 1, cols, ld), fmt, 1.0f);"),
    "block fp32 scale fallback is zero": (
        "float s = orc_compute_scale(amax_f32(t, C, r0, r1, c0, c1), fmt, 1.0f);",
        "float s = orc_compute_scale(amax_f32(t, C, r0, r1, c0, c1), fmt, 0.0f);"),
    "transposed operand left untransposed": (
        "if (transpose) t[c * C + r] = v; else t[r * C + c] = v;",
        "if (transpose) t[r * R + c] = v; else t[r * C + c] = v;"),
    "bf16 input widened from the wrong bit position": (
        "uint32_t b = (uint32_t)((const uint16_t*)x)[idx] << 16;",
        "uint32_t b = (uint32_t)((const uint16_t*)x)[idx] << 15;"),
    "overflow becomes NaN instead of saturating": (
        "if (v > M) return M;",
        "if (v > M) return NAN;"),
    "negative overflow saturates to +MAX": (
        "if (v < -M) return -M;",
        "if (v < -M) return M;"),
    "MX group exponent from the whole row's amax": (
        "float am = amax_f32(t, C, r, r + 1, c0, c1);\n"
        "            int e = smallest_pow2_exponent(orc_fp8_max(fmt), (double)am, -127, 127);\n"
        "            e8m0[r * ng + g]",
        "float am = amax_f32(t, C, r, r + 1, 0, C);\n"
        "            int e = smallest_pow2_exponent(orc_fp8_max(fmt), (double)am, -127, 127);\n"
        "            e8m0[r * ng + g]"),
    "delayed step quantizes with the previous step's scale": (
        "orc_quantize_tensor(x, in_kind, rows, cols, ld, fmt, s, transpose, q, ldq);",
        "orc_quantize_tensor(x, in_kind, rows, cols, ld, fmt, *scale, transpose, q, ldq);"),
    "history merge keeps the destination's scale": (
        "*scale_dst = max_nan(*scale_dst, scale_src);",
        "*scale_dst = max_nan(*scale_dst, *scale_dst);"),
    "automatic scaling keeps the old base at a rescale": (
        "state[0] = amax_now;",
        "state[0] = state[0] > amax_now ? state[0] : amax_now;"),
    "fp32 -> UE8M0 conversion accepts any significand": (
        "if (m == 0.5 && ex - 1 >= -127 && ex - 1 <= 127) {",
        "if (ex - 1 >= -127 && ex - 1 <= 127) {"),
    "MX dequantization reads the scales column-major": (
        "s = ldexp(1.0, (int)((const uint8_t*)scales)[r * ng + k / 32] - 127);",
        "s = ldexp(1.0, (int)((const uint8_t*)scales)[(k / 32) * rows + r] - 127);"),
    "MOSS elements scaled by 2^e instead of 2^-e": (
        "float f = (float)ldexp(1.0, -e);\n            for (int64_t c = c0; c < c1; ++c) {\n"
        "                float v = (t[r * C + c] / S) * f;",
        "float f = (float)ldexp(1.0, e);\n            for (int64_t c = c0; c < c1; ++c) {\n"
        "                float v = (t[r * C + c] / S) * f;"),
    "tensor amax ignores NaN": (
        "    return nan_seen ? NAN : m;\n}\n\n/* ----------------------------------------------------------------"
        " scales",
        "    return m;\n}\n\n/* ---------------------------------------------------------------- scales"),
}


def _build(path_c):
    so = os.path.splitext(path_c)[0] + ".so"
    subprocess.run(["gcc", "-O2", "-fopenmp", "-std=c11", "-fPIC", "-shared", "-o", so, path_c, "-lm"],
                   check=True, capture_output=True)


def _pins_fail(path_c):
    env = dict(os.environ, FP8Q_ORACLE_SOURCE=path_c, OMP_NUM_THREADS="2")
    r = subprocess.run([sys.executable, "-m", "pytest", "-x", "-q", "-m", "not gpu", "-p", "no:cacheprovider"] + PINS,
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=900)
    return r.returncode, r.stdout[-600:]


def test_every_planted_mistake_fails_a_pin(tmp_path):
    src = open(ORACLE_C).read()
    # the control: an unchanged copy run through the same harness passes every pin
    paths = {"control (no mistake)": str(tmp_path / "control.c")}
    with open(paths["control (no mistake)"], "w") as f:
        f.write(src)
    for i, (name, (old, new)) in enumerate(MUTANTS.items()):
        assert src.count(old) == 1, name
        p = str(tmp_path / ("mutant%02d.c" % i))
        with open(p, "w") as f:
            f.write(src.replace(old, new))
        paths[name] = p
    for p in paths.values():
        _build(p)                              # every copy compiles (a build error would not count)
    with ThreadPoolExecutor(4) as ex:
        results = dict(zip(paths, ex.map(_pins_fail, paths.values())))
    rc, out = results.pop("control (no mistake)")
    assert rc == 0, "the unchanged oracle failed its pins in the harness: " + out
    # exit status 1: the pins ran and at least one failed
    missed = {n: out for n, (rc, out) in results.items() if rc != 1}
    assert not missed, "mistakes no pin caught (or runs that did not complete): %s" % missed
