/*
 * fp8q.h -- C ABI of the FP8 quantize-then-scaled-GEMM library for AMD Instinct MI355X (gfx950).
 *
 * The computation: an amax reduction, a saturating round-to-nearest-even cast to OCP FP8 (E4M3 for
 * activations and weights, E5M2 for gradients) under one of five scaling schemes, and a GEMM over
 * the FP8 operands with FP32 accumulation and dequantisation by the scales.
 *
 * Sources (by page title and section):
 *  [FLAX] "Flax FP8 量化实战指南：从 fp8_ops 低层 API 到 Fp8DotGeneral / Fp8Einsum 的完整实现解析":
 *         section 1 (Q/DQ: scale = amax/MAX, x_fp8 = clip(x/scale), x ~= x_fp8 * scale),
 *         section 2.2 (current scaling; quantize = divide, clip to +-MAX, cast; FP32-accumulated
 *         dot; dequantize by a_scale * b_scale), section 2.3 (delayed scaling with an amax history),
 *         section 5.3 (a state used by several branches merges their updates by max).
 *  [NANO] "Nanochat的FP8训练模块", section "实现" (E4M3/E5M2 and their maxima; the three GEMMs of a
 *         linear layer's forward and backward; output dtype always given explicitly; operand-layout
 *         bookkeeping is where transposes silently go wrong).
 *  [HF]   "Transformers 中的细粒度 FP8 量化配置、DeepGEMM 加速路径与 UE8M0 缩放格式完全指南":
 *         section 一 (128x128 weight blocks, 1x128 per-token activation groups, weight_scale_inv
 *         of shape (ceil(out/128), ceil(in/128))), section 四 (block size is two positive ints;
 *         the static activation scheme with one supplied per-tensor activation scale), section 五
 *         (dequantize: block scales folded back into the weights), section 七 (UE8M0 block scales,
 *         exact conversion of power-of-two scales kept in fp32 containers).
 *  [MOSS] "MOSS:高效、精确的 FP8 LLM 训练,采用微尺度和自动尺度变换": section 1 (MXFP8: one
 *         power-of-two scale per 32 consecutive values), section 4 (two-level scaling: FP32 global
 *         factor = max of the per-32 factors, E8M0 local factor per 32 values, FP32 factors applied
 *         once in the GEMM epilogue), section 5 (automatic weight scaling: the scale predicted from
 *         the last measured weight max plus the learning rates since, re-measured every interval).
 *
 * Conventions for every entry point:
 *  - All data pointers are DEVICE pointers owned by the caller.  The library never allocates or
 *    frees, never synchronizes, and enqueues all work on `stream` (a hipStream_t passed as void*;
 *    NULL means the default stream).  Results are ready when the stream's work completes.
 *  - Every call returns an fp8q_status and never throws.  On a non-OK return nothing has been
 *    enqueued (argument errors) or the HIP error is reported (FP8Q_ERR_HIP); fp8q_last_error()
 *    gives a message for the calling thread.
 *  - Scales at the boundary are dequantisation multipliers everywhere: x ~= decode(q) * scale.
 *  - FP8 bytes are OCP e4m3fn (bias 7, max 448, no Inf, NaN = S.1111.111) and e5m2 (bias 15,
 *    max 57344).  E8M0 bytes hold e + 127 for a scale of 2^e.
 *  - Matrices are row-major with a leading dimension in elements (`ld`); every row pointer
 *    (base + r*ld*elem_size) must be 16-byte aligned.
 *  - Calls that share output buffers must be ordered by the caller (same stream or events).
 */
#ifndef FP8Q_H
#define FP8Q_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    FP8Q_OK = 0,
    FP8Q_ERR_INVALID_ARG = -1,   /* bad enum, shape, block size, alignment or NULL pointer */
    FP8Q_ERR_UNSUPPORTED = -2,   /* a valid request outside what the kernels implement */
    FP8Q_ERR_HIP = -3,           /* a HIP runtime call or kernel launch failed */
    FP8Q_ERR_NO_DEVICE = -4      /* no gfx950 device is current */
} fp8q_status;

typedef enum { FP8Q_E4M3 = 0, FP8Q_E5M2 = 1 } fp8q_fmt;
typedef enum { FP8Q_IN_F32 = 0, FP8Q_IN_BF16 = 1 } fp8q_in;
typedef enum { FP8Q_OUT_F32 = 0, FP8Q_OUT_BF16 = 1 } fp8q_out;
typedef enum {
    FP8Q_TENSOR = 0,   /* one fp32 scale for the tensor (current, delayed or static) */
    FP8Q_BLOCK = 1,    /* one fp32 scale per (block_r x block_c) block */
    FP8Q_MX = 2,       /* one E8M0 scale per 32 consecutive values along K */
    FP8Q_MOSS = 3,     /* fp32 global factor S times one E8M0 local factor per 32 values along K */
    FP8Q_BLOCK_E8M0 = 4 /* one power-of-two (UE8M0 byte) scale per (block_r x block_c) block */
} fp8q_mode;

/* Checks that the current device is gfx950 (FP8Q_ERR_NO_DEVICE otherwise) and, once per device,
 * sets the launch attributes of every GEMM kernel on it (FP8Q_ERR_HIP if that fails).  Every entry
 * point checks the device by itself, and a GEMM sets its kernel's attributes at its first launch;
 * calling fp8q_init on each device first means no later call does either, which a caller that
 * captures library calls into a HIP graph should arrange. */
int fp8q_init(void);

/* Message describing the calling thread's last non-OK status ("" if none). */
const char* fp8q_last_error(void);

/*
 * fp8_amax -- amax = max |x| over a rows x cols matrix ([FLAX] section 1).
 *   x         rows x cols, fp32 or bf16 (`in_dtype`), leading dimension ld >= cols.
 *   amax_out  one fp32 on the device.  It is overwritten (not accumulated into).  Any NaN in x
 *             gives NaN; -0 counts as 0; an empty matrix gives 0.
 * The reduction is an integer max over the sign-cleared bit patterns, so it is exact and
 * independent of reduction order.
 */
int fp8_amax(const void* x, int in_dtype, int64_t rows, int64_t cols, int64_t ld,
             float* amax_out, void* stream);

/*
 * fp8_quantize -- saturating round-to-nearest-even FP8 cast under one scaling scheme.
 *
 * The logical operand is x (rows x cols, leading dimension ld, fp32 or bf16).  With
 * transpose_out = 0 the output q is rows x cols; with transpose_out = 1 it is cols x rows
 * (q[c][r] quantizes x[r][c]).  "K" is the last axis of the OUTPUT: scale groups run along it.
 * ldq is q's leading dimension in bytes.  Every element is
 *     q = RNE8( clip( fl(x / scale), -MAX, +MAX ) )       with fl() one IEEE fp32 division,
 * MAX = 448 (E4M3) or 57344 (E5M2); NaN inputs give S.1111111 with the input's sign.
 *
 * mode FP8Q_TENSOR ([FLAX] sections 2.2, 2.3):
 *   scale_is_input = 1: *tensor_scale (device fp32) is the scale to use (delayed or static
 *     scaling); it is not modified.  If amax_out is non-NULL the amax of x is computed in the same
 *     pass and written to *amax_out (the value fp8_history_update consumes).
 *   scale_is_input = 0: current scaling.  amax_out must be non-NULL; the call writes
 *     amax = max|x| to *amax_out, scale = fl(amax / MAX) to *tensor_scale (1.0 when amax is 0,
 *     non-finite, or the quotient underflows to 0), then quantizes with it.
 *   scales, block_r, block_c are ignored.
 * mode FP8Q_BLOCK ([HF] section 一): one fp32 scale per (block_r x block_c) block of the OUTPUT,
 *   scale = fl(amax_block / MAX) (1.0 on zero/non-finite/underflow), written to `scales` as
 *   fp32[ceil(R/block_r)][ceil(K/block_c)] row-major (R, K = output rows, cols).
 *   (1,128) is the per-token activation scheme, (128,128) the weight scheme; both must be positive
 *   ([HF] section 四).  tensor_scale and scale_is_input are ignored; amax_out may be NULL.
 * mode FP8Q_MX ([MOSS] section 1): per group of 32 along K, e = smallest integer in [-127, 127]
 *   with MAX * 2^e >= amax_group (127 if none, e.g. a non-finite group), E8M0 byte e + 127 written
 *   to `scales` as u8[R][ceil(K/32)]; element = RNE8(clip(fl(x * 2^-e))).  block_r/block_c,
 *   tensor_scale and scale_is_input are ignored.
 * mode FP8Q_MOSS ([MOSS] section 4): global S = fl(amax_tensor / MAX) (1.0 on zero/non-finite/
 *   underflow); per group i of 32 along K, s_i = fl(amax_i / MAX) and e_i = smallest integer in
 *   [-127, 0] with S * 2^e_i >= s_i (0 if none), E8M0 byte e_i + 127 in `scales` u8[R][ceil(K/32)];
 *   element = RNE8(clip(fl(fl(x / S) * 2^-e_i))).  scale_is_input = 0: amax_out must be non-NULL,
 *   receives amax_tensor, and S is written to *tensor_scale.  scale_is_input = 1: *tensor_scale
 *   holds S (from an earlier call on the same source tensor, e.g. the other copy of a
 *   forward/backward pair) and is not modified.
 * mode FP8Q_BLOCK_E8M0 ([HF] section 七): per (block_r x block_c) block of the OUTPUT, e = smallest
 *   integer in [-127, 127] with MAX * 2^e >= amax_block (127 if none), E8M0 byte e + 127 written to
 *   `scales` as u8[ceil(R/block_r)][ceil(K/block_c)]; element = RNE8(clip(fl(x * 2^-e))) (exact
 *   scaling: nothing clips unless the block holds Inf).  (128,128) is the UE8M0 weight scheme.
 *
 * Limits (FP8Q_ERR_UNSUPPORTED otherwise): cols % 8 == 0, ld % 8 == 0 and a 16-byte aligned x.
 * fp32 pointers (tensor_scale, amax_out, FP8Q_BLOCK scales) must be 4-byte aligned
 * (FP8Q_ERR_INVALID_ARG otherwise); E8M0 scale arrays may start at any byte.
 * Any ldq >= K works (ldq % 16 == 0 with a 16-byte aligned q selects the vectorized kernels).
 * Ragged group tails (K not a multiple of the group) are handled with ceil semantics.
 */
int fp8_quantize(int mode, int fmt, const void* x, int in_dtype,
                 int64_t rows, int64_t cols, int64_t ld,
                 int block_r, int block_c, int transpose_out,
                 uint8_t* q, int64_t ldq, void* scales,
                 float* tensor_scale, int scale_is_input, float* amax_out,
                 void* stream);

/*
 * fp8_quantize_dual -- both quantized copies of one operand in a single pass over it: q (rows x
 * cols, groups along cols) and qt (cols x rows, groups along rows), byte-for-byte what
 * fp8_quantize writes with transpose_out = 0 and with transpose_out = 1 under the same tensor
 * scale.  A linear layer's forward and backward GEMMs need each operand grouped along two
 * different K axes ([NANO] "实现": the three GEMMs; [MOSS] section 4: S is per source tensor, so
 * both copies share it).
 *   mode: FP8Q_TENSOR, FP8Q_MX or FP8Q_MOSS (FP8Q_BLOCK gives FP8Q_ERR_INVALID_ARG).
 *   q, ldq, scales:     the transpose_out = 0 copy (scales u8[rows][ceil(cols/32)] for MX/MOSS).
 *   qt, ldqt, scales_t: the transpose_out = 1 copy (scales_t u8[cols][ceil(rows/32)] for MX/MOSS).
 *   tensor_scale, scale_is_input, amax_out: as in fp8_quantize (current scaling computes the amax
 *   and the scale once for both copies).
 * Limits (FP8Q_ERR_UNSUPPORTED otherwise): those of fp8_quantize.  rows % 32 == 0,
 * cols % 32 == 0, ldq % 16 == 0, ldqt % 16 == 0 and 16-byte aligned q, qt use the one-pass kernel;
 * other shapes are served by the two single-copy casts.
 */
int fp8_quantize_dual(int mode, int fmt, const void* x, int in_dtype,
                      int64_t rows, int64_t cols, int64_t ld,
                      uint8_t* q, int64_t ldq, void* scales,
                      uint8_t* qt, int64_t ldqt, void* scales_t,
                      float* tensor_scale, int scale_is_input, float* amax_out,
                      void* stream);

/*
 * fp8_history_update -- delayed-scaling state update ([FLAX] section 2.3), called after the cast
 * of step t with that step's amax a_t:
 *     history <- roll(history, -1) with history[0] = *amax_new   (newest at index 0)
 *     *scale_inout <- fl(max(history) / MAX), or unchanged if that max is 0, non-finite or the
 *                     quotient underflows.
 * history: device fp32[len], 1 <= len <= 4096 (the pages use 1024, initialised to zeros with the
 * scale initialised to 1).  The scale left in *scale_inout is the one step t+1 quantizes with,
 * which is exactly the scale Flax's in-step order computes at step t+1.
 */
int fp8_history_update(float* history, int64_t len, const float* amax_new,
                       float* scale_inout, int fmt, void* stream);

/*
 * fp8_scaled_gemm -- C = dequant(A) . dequant(B)^T with FP32 accumulation.
 *   A: M x K FP8 bytes (format afmt), leading dimension lda bytes.  B: N x K FP8 bytes (bfmt),
 *   leading dimension ldb bytes -- both K-contiguous, so C = A B^T; a K x N operand is brought
 *   to N x K once by fp8_quantize(..., transpose_out = 1) ([NANO] on layout bookkeeping).
 *   C: M x N, fp32 or bf16 (`out_dtype`, required, round-to-nearest-even), leading dimension ldc
 *   elements.
 * Scale arguments by mode:
 *   FP8Q_TENSOR: Aglobal = &s_a, Bglobal = &s_b (device fp32); C = (sum qa*qb) * fl(s_a * s_b)
 *                ([FLAX] section 2.2).  Ascale, Bscale unused.
 *   FP8Q_BLOCK:  Ascale fp32[M][ceil(K/128)] (1x128 per token), Bscale fp32[ceil(N/128)][ceil(K/128)]
 *                (128x128 weight blocks, [HF] section 一); every 128-wide K block's FP32 partial
 *                sum is scaled by fl(sa[m][kb] * sb[n/128][kb]) and accumulated in the main loop.
 *   FP8Q_MX:     Ascale u8 E8M0[M][ceil(K/32)], Bscale u8 E8M0[N][ceil(K/32)]; the power-of-two
 *                scales are applied by the matrix-core instruction ([MOSS] section 1).
 *   FP8Q_MOSS:   as MX, plus Aglobal = &S_A, Bglobal = &S_B applied once in the epilogue as
 *                fl(S_A * S_B) ([MOSS] section 4).
 *   FP8Q_BLOCK_E8M0: as FP8Q_BLOCK with Bscale u8 E8M0[ceil(N/128)][ceil(K/128)] (UE8M0 weight
 *                blocks, [HF] section 七): sb = 2^(byte - 127).
 *   Static activations ([HF] section 四, activation_scheme "static"): with FP8Q_BLOCK or
 *                FP8Q_BLOCK_E8M0, Ascale = NULL and Aglobal = &s_a give every 1x128 activation
 *                block the one per-tensor scale s_a (A quantized by fp8_quantize(FP8Q_TENSOR,
 *                scale_is_input = 1)); the K-block factor is then fl(s_a * sb[n/128][kb]).
 * Accumulation: FP8Q_TENSOR, FP8Q_MX and FP8Q_MOSS keep the whole K sum in the FP8 matrix
 * instruction's FP32 accumulator; FP8Q_BLOCK reduces each 128-wide K chunk from zero and adds its
 * scaled FP32 partial into an FP32 accumulator.
 * Limits (FP8Q_ERR_UNSUPPORTED otherwise): K % 16 == 0, lda/ldb % 16 == 0, 16-byte aligned A, B;
 * Ascale, Aglobal, Bglobal and Bscale 4-byte aligned (the kernels read scale arrays in 4-byte
 * words), except the UE8M0 Bscale of FP8Q_BLOCK_E8M0, which may start at any byte.
 * M, N, K need not be multiples of any tile size.
 */
int fp8_scaled_gemm(int mode, const uint8_t* A, int afmt, const void* Ascale,
                    const uint8_t* B, int bfmt, const void* Bscale,
                    const float* Aglobal, const float* Bglobal,
                    int64_t M, int64_t N, int64_t K, int64_t lda, int64_t ldb,
                    void* C, int out_dtype, int64_t ldc, void* stream);

/*
 * fp8_history_merge -- combine the updates of one delayed-scaling state that was used by two
 * branches ([FLAX] section 5.3: the Flax meta dtype adds by max, with -inf as its zero):
 *     hist_dst[i] <- max(hist_dst[i], hist_src[i]),  *scale_dst <- max(*scale_dst, *scale_src)
 * (a NaN on either side gives NaN).  hist_dst, hist_src: device fp32[len], len >= 0; scale_dst,
 * scale_src: device fp32[1].  Merging each branch's state into one accumulator in turn gives the
 * same result in any order.
 */
int fp8_history_merge(float* hist_dst, const float* hist_src, int64_t len,
                      float* scale_dst, const float* scale_src, void* stream);

/*
 * fp8_auto_scale -- one step of automatic weight scaling ([MOSS] section 5): the weight max grows
 * by at most the learning rate per optimizer step, so instead of a max-reduction of the weight the
 * scale is predicted.
 *   state: device fp32[2] owned by the caller, zero-initialised: state[0] = the weight max measured
 *          at the current interval's start, state[1] = the learning rates summed since.
 *   rescale = 1 on an interval's first step (every 500 steps on the page): state[0] <- *amax_now
 *          (the caller's fp8_amax of the current weight), state[1] <- 0.  rescale = 0: amax_now is
 *          not read (it may be NULL).
 *   Then *scale_out <- fl(fl(state[0] + state[1]) / MAX) (1.0 when that max is 0 or non-finite),
 *   and state[1] <- fl(state[1] + lr), lr being the learning rate of the optimizer step that
 *   follows this forward pass.
 * The scale is then used as the MOSS global factor (fp8_quantize(FP8Q_MOSS, scale_is_input = 1)) or
 * as a per-tensor scale (FP8Q_TENSOR).  With fp32 arithmetic the prediction is an upper bound of
 * the weight max up to the rounding of the running sum (a few ulps).
 */
int fp8_auto_scale(float* state, int rescale, const float* amax_now, float lr, int fmt,
                   float* scale_out, void* stream);

/*
 * fp8_scale_to_e8m0 -- exact conversion of power-of-two scales stored as fp32 into UE8M0 bytes
 * ([HF] section 七: checkpoints that keep UE8M0-style scales in fp32 containers are converted
 * exactly on load).  s: device fp32[n]; e8m0: device u8[n] gets e + 127 for s = 2^e, e in
 * [-127, 127].  Every other value (not a power of two, zero, negative, non-finite, out of range)
 * has no exact UE8M0 form: it gets 0xFF and is counted into *bad_count (device int32, overwritten).
 * A caller that requires exactness checks *bad_count == 0 (the Python binding raises ValueError).
 * Scales are never rounded up here: rounding fp32 block scales up to UE8M0 without re-quantizing
 * the weights silently changes them ([HF] section 七); use fp8_quantize(FP8Q_BLOCK_E8M0) instead.
 */
int fp8_scale_to_e8m0(const float* s, int64_t n, uint8_t* e8m0, int32_t* bad_count, void* stream);

/*
 * fp8_block_dequantize -- fold block scales back into an FP8 weight ([HF] section 五):
 *     out[r][c] = fl(decode(q[r][c]) * s[r / block_r][c / block_c])     (one fp32 rounding)
 * stored as fp32 or rounded to bf16 (round to nearest even; NaN stays NaN).
 *   mode FP8Q_BLOCK: scales fp32[ceil(rows/block_r)][ceil(cols/block_c)]; FP8Q_BLOCK_E8M0: the same
 *   shape of E8M0 bytes (s = 2^(byte - 127), so the product is exact).
 *   q: rows x cols FP8 bytes (fmt), leading dimension ldq bytes; out: rows x cols, leading
 *   dimension ldo elements, out_dtype FP8Q_OUT_F32 or FP8Q_OUT_BF16.
 * cols % 16 == 0, block_c % 16 == 0 and 16-byte aligned rows select the vectorized kernel; any
 * other shape is served element by element.
 */
int fp8_block_dequantize(int mode, int fmt, const uint8_t* q, int64_t rows, int64_t cols, int64_t ldq,
                         const void* scales, int block_r, int block_c,
                         void* out, int out_dtype, int64_t ldo, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* FP8Q_H */
