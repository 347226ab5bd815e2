/*
 * oracle.c -- plain, slow, obviously-correct CPU oracle for FP8 quantize-then-scaled-GEMM.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product path may call, link or load this file or
 * the library built from it: only the tests, the package smoke check and the benchmark's
 * CPU-baseline leg use it.  It shares no code with the HIP kernels.
 *
 * Build: gcc -O2 -fopenmp -std=c11 -shared -fPIC (no -ffast-math, no intrinsics).
 *
 * Sources (cited by page title and section):
 *  [FLAX]  "Flax FP8 量化实战指南：从 fp8_ops 低层 API 到 Fp8DotGeneral / Fp8Einsum 的完整实现解析"
 *          section 1 (Q/DQ definition: scale = amax/MAX, quantize = clip(x/scale)),
 *          section 2.2 (quantize divides by the scale in the compute dtype, clips to +-MAX, casts;
 *                       current scaling; dequantize by a_scale*b_scale),
 *          section 2.3 (delayed scaling: scale from the max of the amax history, history rolled
 *                       by one with the newest amax written at index 0, zero/non-finite amax keeps
 *                       the old scale), section 5.1 (scale initialised to 1, history to 1024 zeros).
 *  [NANO]  "Nanochat的FP8训练模块", section "实现" (E4M3 max 448, E5M2 max 57344, gradients in E5M2,
 *          cast after a clamp to +-max).
 *  [HF]    "Transformers 中的细粒度 FP8 量化配置、DeepGEMM 加速路径与 UE8M0 缩放格式完全指南",
 *          section 一 (128x128 weight blocks, per-token groups of 128 along the input channels,
 *          weight_scale_inv of shape (ceil(out/128), ceil(in/128))), section 四 (static activation
 *          scheme: one supplied per-tensor activation scale), section 五 (dequantize: the block
 *          scale folded back into the weight, bf16 result), section 七 (UE8M0 block scales: one
 *          power-of-two byte per block; power-of-two scales stored in fp32 containers converted
 *          exactly; rounding fp32 scales up to UE8M0 without re-quantizing corrupts the output).
 *  [MOSS]  "MOSS:高效、精确的 FP8 LLM 训练,采用微尺度和自动尺度变换",
 *          section 1 (MXFP8: groups of 32 consecutive values, power-of-two shared scale from the
 *                     group's max, divide, store FP8),
 *          section 2 (SNR as signal power over quantization-noise power, in dB),
 *          section 4 (two-level scaling, steps 1-4: per-32 float scale, global factor = max of
 *                     them, E8M0 local factor in (0,1], effective scale = global * local,
 *                     FP32 factors applied once in the epilogue),
 *          section 5 (automatic weight scaling: the weight max grows by at most the learning
 *                     rate per step, so the scale is predicted from the last measured max plus
 *                     the learning rates since, and re-measured at the end of each interval).
 *
 * Readings where the pages leave a step open are listed in the design notes; the ones that
 * change arithmetic here are:
 *  - scales are dequantization multipliers: x ~= q * s;
 *  - the quotient x/s is one IEEE fp32 division, then clip to +-MAX (NaN passes), then
 *    round-to-nearest-even onto the OCP E4M3 / E5M2 grid;
 *  - a scale whose amax is zero, non-finite, or whose quotient amax/MAX underflows to zero falls
 *    back (current and block scaling: 1; delayed scaling: the previous scale);
 *  - MX exponent: the smallest e in [-127,127] with MAX*2^e >= amax (127 if none);
 *  - MOSS local exponent: the smallest e in [-127,0] with S*2^e >= s_i (0 if none); the
 *    element is fl(fl(x/S) * 2^-e), clipped, rounded;
 *  - E8M0 byte = e + 127;
 *  - UE8M0 block scale: the MX exponent rule applied to a whole 2-D block;
 *  - automatic scaling: predicted max = fl(base + sum of the learning rates since the last
 *    measurement) in fp32 (the sum accumulated in fp32 step by step);
 *  - merging two branches' updated history/scale pairs takes the elementwise max.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define ORC_E4M3 0
#define ORC_E5M2 1
#define ORC_IN_F32 0
#define ORC_IN_BF16 1
#define ORC_TENSOR 0
#define ORC_BLOCK 1
#define ORC_MX 2
#define ORC_MOSS 3
#define ORC_BLOCK_E8M0 4

/* ---------------------------------------------------------------- formats ---- */

/* Largest finite magnitude of each format: E4M3 (bias 7, S.1111.111 is NaN) gives 1.75*2^8,
 * E5M2 (bias 15, exponent 31 is Inf/NaN) gives 1.75*2^15.  [NANO] */
double orc_fp8_max(int fmt) { return fmt == ORC_E4M3 ? 448.0 : 57344.0; }

/* Largest finite magnitude code (sign bit clear). */
static int max_code(int fmt) { return fmt == ORC_E4M3 ? 0x7E : 0x7B; }

/* Decode one FP8 byte from its sign/exponent/mantissa fields (OCP definitions). */
double orc_fp8_decode(int code, int fmt) {
    int sign = (code >> 7) & 1;
    double v;
    if (fmt == ORC_E4M3) {
        int e = (code >> 3) & 15, m = code & 7;
        if (e == 15 && m == 7) return NAN;
        if (e == 0) v = m * ldexp(1.0, -9);                    /* subnormal: m/8 * 2^(1-7) */
        else v = (1.0 + m / 8.0) * ldexp(1.0, e - 7);
    } else {
        int e = (code >> 2) & 31, m = code & 3;
        if (e == 31) return m == 0 ? (sign ? -INFINITY : INFINITY) : NAN;
        if (e == 0) v = m * ldexp(1.0, -16);                   /* subnormal: m/4 * 2^(1-15) */
        else v = (1.0 + m / 4.0) * ldexp(1.0, e - 15);
    }
    return sign ? -v : v;
}

/* Round a finite fp32 value with |v| <= MAX to the nearest FP8 value, ties to the even code.
 * Every FP8 value, every midpoint between neighbours and every fp32 value is exact in double,
 * so the comparisons below are exact.  The sign is always kept (-0 -> 0x80).  NaN -> S.1111111. */
uint8_t orc_fp8_encode(float v, int fmt) {
    uint32_t bits;
    memcpy(&bits, &v, 4);
    int sign = (int)(bits >> 31) << 7;
    if (isnan(v)) return (uint8_t)(sign | 0x7F);
    double a = fabs((double)v);
    int top = max_code(fmt);
    /* c = largest magnitude code whose value is <= a (decode is increasing on 0..top) */
    int lo = 0, hi = top;
    while (lo < hi) {
        int mid = (lo + hi + 1) / 2;
        if (orc_fp8_decode(mid, fmt) <= a) lo = mid; else hi = mid - 1;
    }
    int c = lo;
    if (c == top) return (uint8_t)(sign | c);                 /* input is clipped: a == MAX */
    double below = orc_fp8_decode(c, fmt), above = orc_fp8_decode(c + 1, fmt);
    double midpoint = (below + above) / 2.0;
    int r;
    if (a > midpoint) r = c + 1;
    else if (a < midpoint) r = c;
    else r = (c % 2 == 0) ? c : c + 1;
    return (uint8_t)(sign | r);
}

void orc_fp8_encode_array(const float* v, int64_t n, int fmt, uint8_t* out) {
    #pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < n; ++i) out[i] = orc_fp8_encode(v[i], fmt);
}

void orc_fp8_decode_array(const uint8_t* q, int64_t n, int fmt, double* out) {
    for (int64_t i = 0; i < n; ++i) out[i] = orc_fp8_decode(q[i], fmt);
}

/* ---------------------------------------------------------------- inputs ----- */

static float load_elem(const void* x, int in_kind, int64_t idx) {
    if (in_kind == ORC_IN_F32) return ((const float*)x)[idx];
    uint32_t b = (uint32_t)((const uint16_t*)x)[idx] << 16;   /* bf16 -> fp32 is exact */
    float f;
    memcpy(&f, &b, 4);
    return f;
}

/* Materialise the logical operand as fp32, rows x cols, optionally transposed (then the result
 * is cols x rows).  Grouping along "K" always means along the last axis of this logical array. */
static float* logical_f32(const void* x, int in_kind, int64_t rows, int64_t cols, int64_t ld,
                          int transpose, int64_t* out_rows, int64_t* out_cols) {
    int64_t R = transpose ? cols : rows, C = transpose ? rows : cols;
    float* t = (float*)malloc((size_t)(R * C > 0 ? R * C : 1) * sizeof(float));
    for (int64_t r = 0; r < rows; ++r)
        for (int64_t c = 0; c < cols; ++c) {
            float v = load_elem(x, in_kind, r * ld + c);
            if (transpose) t[c * C + r] = v; else t[r * C + c] = v;
        }
    *out_rows = R;
    *out_cols = C;
    return t;
}

/* ---------------------------------------------------------------- amax ------- */

/* max |x| over a region; any NaN makes the result NaN.  [FLAX] section 1 */
static float amax_f32(const float* t, int64_t ldt, int64_t r0, int64_t r1, int64_t c0, int64_t c1) {
    float m = 0.0f;
    int nan_seen = 0;
    for (int64_t r = r0; r < r1; ++r)
        for (int64_t c = c0; c < c1; ++c) {
            float v = t[r * ldt + c];
            if (isnan(v)) nan_seen = 1;
            else if (fabsf(v) > m) m = fabsf(v);
        }
    return nan_seen ? NAN : m;
}

float orc_amax(const void* x, int in_kind, int64_t rows, int64_t cols, int64_t ld) {
    float m = 0.0f;
    int nan_seen = 0;
    for (int64_t r = 0; r < rows; ++r)
        for (int64_t c = 0; c < cols; ++c) {
            float v = load_elem(x, in_kind, r * ld + c);
            if (isnan(v)) nan_seen = 1;
            else if (fabsf(v) > m) m = fabsf(v);
        }
    return nan_seen ? NAN : m;
}

/* ---------------------------------------------------------------- scales ----- */

/* scale = amax / MAX as one fp32 division; zero, non-finite or underflowing amax keeps
 * `fallback`.  [FLAX] sections 1 and 2.3 */
float orc_compute_scale(float amax, int fmt, float fallback) {
    if (!(amax > 0.0f) || isinf(amax)) return fallback;
    float s = amax / (float)orc_fp8_max(fmt);
    if (s == 0.0f) return fallback;
    return s;
}

/* clip to [-MAX, MAX]; NaN passes through (comparisons with NaN are false).  [FLAX] section 2.2 */
static float clip_max(float v, int fmt) {
    float M = (float)orc_fp8_max(fmt);
    if (v > M) return M;
    if (v < -M) return -M;
    return v;
}

/* encode(clip(fl(x / s))).  [FLAX] section 2.2 */
uint8_t orc_quantize_value(float x, float s, int fmt) {
    float v = x / s;
    return orc_fp8_encode(clip_max(v, fmt), fmt);
}

/* ---------------------------------------------------------------- schemes ---- */

/* Per-tensor: q[r][c] = encode(clip(fl(x/s))).  With transpose the output is cols x rows. */
void orc_quantize_tensor(const void* x, int in_kind, int64_t rows, int64_t cols, int64_t ld, int fmt,
                         float s, int transpose, uint8_t* q, int64_t ldq) {
    int64_t R, C;
    float* t = logical_f32(x, in_kind, rows, cols, ld, transpose, &R, &C);
    #pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < R; ++r)
        for (int64_t c = 0; c < C; ++c) q[r * ldq + c] = orc_quantize_value(t[r * C + c], s, fmt);
    free(t);
}

/* Block scaling: one fp32 scale per (br x bc) block of the logical array, shape
 * [ceil(R/br)][ceil(C/bc)], scale = amax_block/MAX (fallback 1).  (1,128) is the per-token
 * activation scheme, (128,128) the weight scheme.  [HF] section 一 */
void orc_quantize_block(const void* x, int in_kind, int64_t rows, int64_t cols, int64_t ld, int fmt,
                        int64_t br, int64_t bc, int transpose, uint8_t* q, int64_t ldq, float* scales) {
    int64_t R, C;
    float* t = logical_f32(x, in_kind, rows, cols, ld, transpose, &R, &C);
    int64_t nbr = (R + br - 1) / br, nbc = (C + bc - 1) / bc;
    #pragma omp parallel for schedule(static)
    for (int64_t bi = 0; bi < nbr; ++bi) {
        for (int64_t bj = 0; bj < nbc; ++bj) {
            int64_t r0 = bi * br, r1 = r0 + br < R ? r0 + br : R;
            int64_t c0 = bj * bc, c1 = c0 + bc < C ? c0 + bc : C;
            float s = orc_compute_scale(amax_f32(t, C, r0, r1, c0, c1), fmt, 1.0f);
            scales[bi * nbc + bj] = s;
            for (int64_t r = r0; r < r1; ++r)
                for (int64_t c = c0; c < c1; ++c) q[r * ldq + c] = orc_quantize_value(t[r * C + c], s, fmt);
        }
    }
    free(t);
}

/* Smallest e in [lo, hi] with base * 2^e >= target (products exact in double); hi if none. */
static int smallest_pow2_exponent(double base, double target, int lo, int hi);

/* UE8M0 block scaling: one power-of-two scale 2^e per (br x bc) block, e = smallest integer in
 * [-127, 127] with MAX * 2^e >= amax_block (127 if none), stored as the byte e + 127 in
 * e8m0[ceil(R/br)][ceil(C/bc)]; element encode(clip(fl(x * 2^-e))) (exact scaling, so nothing
 * clips unless the block holds non-finite values).  [HF] section 七 */
void orc_quantize_block_e8m0(const void* x, int in_kind, int64_t rows, int64_t cols, int64_t ld, int fmt,
                             int64_t br, int64_t bc, int transpose, uint8_t* q, int64_t ldq, uint8_t* e8m0) {
    int64_t R, C;
    float* t = logical_f32(x, in_kind, rows, cols, ld, transpose, &R, &C);
    int64_t nbr = (R + br - 1) / br, nbc = (C + bc - 1) / bc;
    #pragma omp parallel for schedule(static)
    for (int64_t bi = 0; bi < nbr; ++bi) {
        for (int64_t bj = 0; bj < nbc; ++bj) {
            int64_t r0 = bi * br, r1 = r0 + br < R ? r0 + br : R;
            int64_t c0 = bj * bc, c1 = c0 + bc < C ? c0 + bc : C;
            float am = amax_f32(t, C, r0, r1, c0, c1);
            int e = smallest_pow2_exponent(orc_fp8_max(fmt), (double)am, -127, 127);
            e8m0[bi * nbc + bj] = (uint8_t)(e + 127);
            float f = (float)ldexp(1.0, -e);
            for (int64_t r = r0; r < r1; ++r)
                for (int64_t c = c0; c < c1; ++c)
                    q[r * ldq + c] = orc_fp8_encode(clip_max(t[r * C + c] * f, fmt), fmt);
        }
    }
    free(t);
}

/* Exact conversion of power-of-two scales held in fp32 to UE8M0 bytes: 2^e with e in [-127, 127]
 * becomes e + 127.  Any other value (not a power of two, zero, negative, non-finite, out of range)
 * cannot be represented exactly; it gets the byte 0xFF and is counted.  Returns that count.
 * [HF] section 七 (checkpoints that keep power-of-two UE8M0 scales in fp32 containers are converted
 * exactly on load) */
int64_t orc_scales_f32_to_e8m0(const float* s, int64_t n, uint8_t* out) {
    int64_t bad = 0;
    for (int64_t i = 0; i < n; ++i) {
        double v = (double)s[i];
        int ok = 0;
        if (v > 0.0 && !isinf(v) && !isnan(v)) {
            int ex;
            double m = frexp(v, &ex);                 /* v = m * 2^ex, m in [0.5, 1) */
            if (m == 0.5 && ex - 1 >= -127 && ex - 1 <= 127) {
                out[i] = (uint8_t)(ex - 1 + 127);
                ok = 1;
            }
        }
        if (!ok) {
            out[i] = 0xFF;
            ++bad;
        }
    }
    return bad;
}

static int smallest_pow2_exponent(double base, double target, int lo, int hi) {
    for (int e = lo; e <= hi; ++e)
        if (base * ldexp(1.0, e) >= target) return e;
    return hi;
}

/* MXFP8: per group of 32 consecutive values along the last axis, e = smallest integer with
 * MAX * 2^e >= amax_group, E8M0 byte e + 127, element encode(clip(fl(x * 2^-e))).  [MOSS] section 1 */
void orc_quantize_mx(const void* x, int in_kind, int64_t rows, int64_t cols, int64_t ld, int fmt,
                     int transpose, uint8_t* q, int64_t ldq, uint8_t* e8m0) {
    int64_t R, C;
    float* t = logical_f32(x, in_kind, rows, cols, ld, transpose, &R, &C);
    int64_t ng = (C + 31) / 32;
    #pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < R; ++r) {
        for (int64_t g = 0; g < ng; ++g) {
            int64_t c0 = g * 32, c1 = c0 + 32 < C ? c0 + 32 : C;
            float am = amax_f32(t, C, r, r + 1, c0, c1);
            int e = smallest_pow2_exponent(orc_fp8_max(fmt), (double)am, -127, 127);
            e8m0[r * ng + g] = (uint8_t)(e + 127);
            float f = (float)ldexp(1.0, -e);                      /* 2^-e, exact in fp32 */
            for (int64_t c = c0; c < c1; ++c) {
                float v = t[r * C + c] * f;
                q[r * ldq + c] = orc_fp8_encode(clip_max(v, fmt), fmt);
            }
        }
    }
    free(t);
}

/* MOSS two-level scaling with a given global factor S (steps 1, 3 and 4 below); used directly
 * for the second quantized copy of a tensor whose S is already known. */
void orc_quantize_moss_given(const void* x, int in_kind, int64_t rows, int64_t cols, int64_t ld, int fmt,
                             int transpose, float S, uint8_t* q, int64_t ldq, uint8_t* e8m0) {
    int64_t R, C;
    float* t = logical_f32(x, in_kind, rows, cols, ld, transpose, &R, &C);
    int64_t ng = (C + 31) / 32;
    float M = (float)orc_fp8_max(fmt);
    #pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < R; ++r) {
        for (int64_t g = 0; g < ng; ++g) {
            int64_t c0 = g * 32, c1 = c0 + 32 < C ? c0 + 32 : C;
            float s_i = amax_f32(t, C, r, r + 1, c0, c1) / M;
            int e = smallest_pow2_exponent((double)S, (double)s_i, -127, 0);
            e8m0[r * ng + g] = (uint8_t)(e + 127);
            float f = (float)ldexp(1.0, -e);
            for (int64_t c = c0; c < c1; ++c) {
                float v = (t[r * C + c] / S) * f;
                q[r * ldq + c] = orc_fp8_encode(clip_max(v, fmt), fmt);
            }
        }
    }
    free(t);
}

/* MOSS two-level scaling.  Step 1: s_i = fl(amax_i / MAX) per group of 32 along the last axis.
 * Step 2: global S = fl(amax_tensor / MAX) (= max_i s_i; fallback 1).  Step 3: local exponent
 * e_i = smallest e in [-127, 0] with S * 2^e >= s_i, stored as E8M0 byte e_i + 127.
 * Step 4: element encode(clip(fl(fl(x/S) * 2^-e_i))), so x ~= q * S * 2^e_i.  [MOSS] section 4 */
void orc_quantize_moss(const void* x, int in_kind, int64_t rows, int64_t cols, int64_t ld, int fmt,
                       int transpose, uint8_t* q, int64_t ldq, uint8_t* e8m0, float* S_out) {
    float S = orc_compute_scale(orc_amax(x, in_kind, rows, cols, ld), fmt, 1.0f);
    *S_out = S;
    orc_quantize_moss_given(x, in_kind, rows, cols, ld, fmt, transpose, S, q, ldq, e8m0);
}

/* ---------------------------------------------------------------- delayed ---- */

/* One history step: roll the window left by one (element i+1 moves to i, element 0 to the end),
 * then write the newest amax at index 0.  [FLAX] section 2.3 */
void orc_history_roll_insert(float* hist, int64_t len, float amax_new) {
    if (len <= 0) return;
    float first = hist[0];
    for (int64_t i = 0; i + 1 < len; ++i) hist[i] = hist[i + 1];
    hist[len - 1] = first;
    hist[0] = amax_new;
}

/* Max of the history window (NaN-propagating like amax). */
float orc_history_max(const float* hist, int64_t len) { return amax_f32(hist, len, 0, 1, 0, len); }

/* Flax's in-step order for one operand at step t: s_t from max(H_{t-1}) (previous scale kept on
 * zero/non-finite), then quantize x_t with s_t, then H_t = roll-insert of amax(x_t).
 * Updates *scale and hist in place, writes q.  [FLAX] section 2.3 */
void orc_delayed_step(const void* x, int in_kind, int64_t rows, int64_t cols, int64_t ld, int fmt,
                      int transpose, float* scale, float* hist, int64_t len, uint8_t* q, int64_t ldq,
                      float* amax_out) {
    float s = orc_compute_scale(orc_history_max(hist, len), fmt, *scale);
    orc_quantize_tensor(x, in_kind, rows, cols, ld, fmt, s, transpose, q, ldq);
    float a = orc_amax(x, in_kind, rows, cols, ld);
    orc_history_roll_insert(hist, len, a);
    *scale = s;
    if (amax_out) *amax_out = a;
}

/* Two uses of one delayed-scaling state (branches, micro-batches) each produce an updated
 * history and scale; they are combined by taking the larger value, element by element, not by
 * adding them (lax.max semantics: NaN propagates).  dst <- max(dst, src).  [FLAX] section 5.3 */
static float max_nan(float a, float b) {
    if (isnan(a) || isnan(b)) return NAN;
    return a > b ? a : b;
}
void orc_history_merge(float* hist_dst, const float* hist_src, int64_t len, float* scale_dst, float scale_src) {
    for (int64_t i = 0; i < len; ++i) hist_dst[i] = max_nan(hist_dst[i], hist_src[i]);
    *scale_dst = max_nan(*scale_dst, scale_src);
}

/* Automatic weight scaling, one step.  state[0] = base (the weight max measured at the start of
 * the current interval), state[1] = the sum of the learning rates applied since.  On a rescale
 * step (the interval's first) base <- amax_now (a fresh max-reduction of the weight) and the sum
 * restarts at 0.  The step's scale is fl(fl(base + sum) / MAX) (1.0 if that max is zero or
 * non-finite); then this step's learning rate is added to the sum.  The prediction is an upper
 * bound because each optimizer step moves a weight by at most the learning rate.
 * [MOSS] section 5 */
float orc_auto_scale_step(float* state, int rescale, float amax_now, float lr, int fmt) {
    if (rescale) {
        state[0] = amax_now;
        state[1] = 0.0f;
    }
    float predicted = state[0] + state[1];
    float s = orc_compute_scale(predicted, fmt, 1.0f);
    state[1] = state[1] + lr;
    return s;
}

/* ---------------------------------------------------------------- dequant ---- */

/* Dequantize one K-contiguous operand (rows x K) into fp64: q * scale, exact in double.
 * TENSOR: scale = *global.  BLOCK: fp32 scale per (br x bc) block, [ceil(rows/br)][K/bc].
 * BLOCK_E8M0: 2^(byte-127) per (br x bc) block.  MX: 2^(byte-127) per (row, 32-group).
 * MOSS: as MX times *global. */
void orc_dequantize(int mode, const uint8_t* q, int fmt, int64_t rows, int64_t K, int64_t ldq,
                    const void* scales, int64_t br, int64_t bc, const float* global, double* out) {
    int64_t ng = (K + 31) / 32, nbc = bc > 0 ? (K + bc - 1) / bc : 0;
    #pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < rows; ++r)
        for (int64_t k = 0; k < K; ++k) {
            double v = orc_fp8_decode(q[r * ldq + k], fmt), s;
            if (mode == ORC_TENSOR) s = (double)*global;
            else if (mode == ORC_BLOCK) s = (double)((const float*)scales)[(r / br) * nbc + k / bc];
            else if (mode == ORC_BLOCK_E8M0)
                s = ldexp(1.0, (int)((const uint8_t*)scales)[(r / br) * nbc + k / bc] - 127);
            else {
                s = ldexp(1.0, (int)((const uint8_t*)scales)[r * ng + k / 32] - 127);
                if (mode == ORC_MOSS) s *= (double)*global;
            }
            out[r * K + k] = v * s;
        }
}

/* fp32 -> bf16 bits, round to nearest even (NaN -> quiet NaN with the sign kept). */
static uint16_t bf16_rne(float f) {
    uint32_t u;
    memcpy(&u, &f, 4);
    if ((u & 0x7FFFFFFFu) > 0x7F800000u) return (uint16_t)((u >> 16) | 0x40u);
    uint32_t lsb = (u >> 16) & 1u;
    u += 0x7FFFu + lsb;
    return (uint16_t)(u >> 16);
}

/* Block dequantize of a (rows x K) FP8 weight: out[r][k] = fl(decode(q) * s_block) as fp32, or
 * that fp32 product rounded to bf16 (out_bf16 = 1; out is then uint16 bit patterns).  The block
 * scale is fp32 (BLOCK) or 2^(byte-127) (BLOCK_E8M0), [ceil(rows/br)][ceil(K/bc)].
 * [HF] section 五 (the block scale folded into the weight, bf16 result) */
void orc_block_dequantize(int mode, const uint8_t* q, int fmt, int64_t rows, int64_t K, int64_t ldq,
                          const void* scales, int64_t br, int64_t bc, int out_bf16, void* out) {
    int64_t nbc = (K + bc - 1) / bc;
    #pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < rows; ++r)
        for (int64_t k = 0; k < K; ++k) {
            float v = (float)orc_fp8_decode(q[r * ldq + k], fmt);    /* exact in fp32 */
            int64_t bi = (r / br) * nbc + k / bc;
            float s = mode == ORC_BLOCK_E8M0 ? (float)ldexp(1.0, (int)((const uint8_t*)scales)[bi] - 127)
                                             : ((const float*)scales)[bi];
            float p = v * s;                                        /* one fp32 rounding */
            if (out_bf16) ((uint16_t*)out)[r * K + k] = bf16_rne(p);
            else ((float*)out)[r * K + k] = p;
        }
}

/* ---------------------------------------------------------------- GEMM ------- */

/* C[m][n] = sum_k A[m][k] * B[n][k] in fp64 over the dequantized operands (both rows x K,
 * K-contiguous), and D[m][n] = sum_k |A[m][k]| * |B[n][k]| (the scale of rounding error).
 * If `pairs` is non-NULL, only the listed (m, n) pairs are computed into C[i], D[i].
 * [FLAX] section 2.2 (FP32-accumulated dot of the quantized operands, dequantized by the scales);
 * here the accumulation is fp64 so that the result is the product of the quantized operands. */
void orc_gemm_ref(const double* A, const double* B, int64_t M, int64_t N, int64_t K,
                  const int64_t* pairs, int64_t npairs, double* C, double* D) {
    if (pairs) {
        #pragma omp parallel for schedule(dynamic, 64)
        for (int64_t i = 0; i < npairs; ++i) {
            int64_t m = pairs[2 * i], n = pairs[2 * i + 1];
            double c = 0.0, d = 0.0;
            for (int64_t k = 0; k < K; ++k) {
                double p = A[m * K + k] * B[n * K + k];
                c += p;
                d += fabs(p);
            }
            C[i] = c;
            D[i] = d;
        }
        return;
    }
    #pragma omp parallel for schedule(dynamic, 1)
    for (int64_t m = 0; m < M; ++m)
        for (int64_t n = 0; n < N; ++n) {
            double c = 0.0, d = 0.0;
            for (int64_t k = 0; k < K; ++k) {
                double p = A[m * K + k] * B[n * K + k];
                c += p;
                d += fabs(p);
            }
            C[m * N + n] = c;
            D[m * N + n] = d;
        }
}

/* The same product with the two further sums that size the rounding error of a GEMM which
 * reduces K in chunks of `chunk` (the matrix instruction's K width), per (m, n):
 *   E[m][n]   = sum over chunks of max_{k in chunk} |A[m][k] * B[n][k]|,
 *   Sig[m][n] = sum over chunks j of |S_{j-1}|, with S_{j-1} the sum of the products of all chunks
 *               before chunk j (the running sum a whole-K accumulation feeds back as its input),
 * both in fp64.  C and D are exactly those of orc_gemm_ref.  The last chunk may be short. */
static void gemm_terms_one(const double* a, const double* b, int64_t K, int64_t chunk, double* c_out,
                           double* d_out, double* e_out, double* s_out) {
    double c = 0.0, d = 0.0, e = 0.0, sig = 0.0, prefix = 0.0;
    for (int64_t k0 = 0; k0 < K; k0 += chunk) {
        int64_t k1 = k0 + chunk < K ? k0 + chunk : K;
        double part = 0.0, mx = 0.0;
        for (int64_t k = k0; k < k1; ++k) {
            double p = a[k] * b[k];
            c += p;
            d += fabs(p);
            part += p;
            if (fabs(p) > mx) mx = fabs(p);
        }
        e += mx;
        sig += fabs(prefix);
        prefix += part;
    }
    *c_out = c;
    *d_out = d;
    *e_out = e;
    *s_out = sig;
}

void orc_gemm_ref_terms(const double* A, const double* B, int64_t M, int64_t N, int64_t K, int64_t chunk,
                        const int64_t* pairs, int64_t npairs, double* C, double* D, double* E, double* Sig) {
    if (pairs) {
        #pragma omp parallel for schedule(dynamic, 64)
        for (int64_t i = 0; i < npairs; ++i) {
            int64_t m = pairs[2 * i], n = pairs[2 * i + 1];
            gemm_terms_one(A + m * K, B + n * K, K, chunk, C + i, D + i, E + i, Sig + i);
        }
        return;
    }
    /* the longer axis is the parallel (outer) one, so a few rows against many columns (or the
     * reverse) reads each long operand's rows once */
    if (M >= N) {
        #pragma omp parallel for schedule(dynamic, 1)
        for (int64_t m = 0; m < M; ++m)
            for (int64_t n = 0; n < N; ++n)
                gemm_terms_one(A + m * K, B + n * K, K, chunk, C + m * N + n, D + m * N + n, E + m * N + n,
                               Sig + m * N + n);
    } else {
        #pragma omp parallel for schedule(dynamic, 1)
        for (int64_t n = 0; n < N; ++n)
            for (int64_t m = 0; m < M; ++m)
                gemm_terms_one(A + m * K, B + n * K, K, chunk, C + m * N + n, D + m * N + n, E + m * N + n,
                               Sig + m * N + n);
    }
}

/* ---------------------------------------------------------------- SNR -------- */

/* SNR in dB = 10 log10( sum x^2 / sum (x - xhat)^2 ), fp64; +inf when the noise is zero.
 * [MOSS] section 2 (ratio of signal power to quantization-noise power, then in decibels) */
double orc_snr_db(const float* x, const double* xhat, int64_t n) {
    double sig = 0.0, noise = 0.0;
    for (int64_t i = 0; i < n; ++i) {
        double v = (double)x[i], d = v - xhat[i];
        sig += v * v;
        noise += d * d;
    }
    if (noise == 0.0) return INFINITY;
    return 10.0 * log10(sig / noise);
}
