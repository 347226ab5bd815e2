// C ABI entry points (include/fp8q.h): argument validation, error reporting and dispatch to the
// kernel launchers.  No allocation, no synchronization: all work goes on the caller's stream.
#include <hip/hip_runtime.h>
#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include "../../include/fp8q.h"
#include "kernels.h"

namespace {

thread_local char g_err[512] = "";

int fail(int code, const char* fmt, ...) {
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_err, sizeof g_err, fmt, ap);
    va_end(ap);
    return code;
}

int check_launch(const char* what) {
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return fail(FP8Q_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
    return FP8Q_OK;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
bool aligned4(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 3u) == 0; }
// at most kSmallCastElems elements, tested without forming a product that could overflow
bool small_tensor(int64_t rows, int64_t cols) {
    return rows <= fp8q::kSmallCastElems && cols <= fp8q::kSmallCastElems && rows * cols <= fp8q::kSmallCastElems;
}

// Per-device result of the architecture check (up to 64 devices).
int g_arch_ok[64];   // 0 unknown, 1 gfx950, -1 other
// Per-device flag: the GEMM kernels' LDS limits have been set (fp8q_init).
int g_gemm_prepared[64];

int check_device() {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return fail(FP8Q_ERR_NO_DEVICE, "no HIP device is current");
    if (dev < 0 || dev >= 64) return fail(FP8Q_ERR_NO_DEVICE, "device index %d out of range", dev);
    if (g_arch_ok[dev] == 0) {
        hipDeviceProp_t p;
        if (hipGetDeviceProperties(&p, dev) != hipSuccess) return fail(FP8Q_ERR_NO_DEVICE, "cannot query device %d", dev);
        g_arch_ok[dev] = strncmp(p.gcnArchName, "gfx950", 6) == 0 ? 1 : -1;
    }
    if (g_arch_ok[dev] != 1) return fail(FP8Q_ERR_NO_DEVICE, "device %d is not gfx950 (MI355X)", dev);
    return FP8Q_OK;
}

bool valid_fmt(int f) { return f == FP8Q_E4M3 || f == FP8Q_E5M2; }
bool valid_in(int d) { return d == FP8Q_IN_F32 || d == FP8Q_IN_BF16; }

}  // namespace

extern "C" {

int fp8q_init(void) {
    g_err[0] = 0;
    int rc = check_device();
    if (rc) return rc;
    int dev = 0;
    (void)hipGetDevice(&dev);
    if (!g_gemm_prepared[dev]) {
        if (fp8q::prepare_gemm_kernels() != 0) return fail(FP8Q_ERR_HIP, "fp8q_init: setting the GEMM kernels' LDS limit failed");
        g_gemm_prepared[dev] = 1;
    }
    return FP8Q_OK;
}

const char* fp8q_last_error(void) { return g_err; }

int fp8_amax(const void* x, int in_dtype, int64_t rows, int64_t cols, int64_t ld, float* amax_out, void* stream) {
    g_err[0] = 0;
    if (!valid_in(in_dtype)) return fail(FP8Q_ERR_INVALID_ARG, "fp8_amax: in_dtype %d is not FP8Q_IN_F32/BF16", in_dtype);
    if (rows < 0 || cols < 0 || ld < cols) return fail(FP8Q_ERR_INVALID_ARG, "fp8_amax: bad shape rows=%lld cols=%lld ld=%lld",
                                                      (long long)rows, (long long)cols, (long long)ld);
    if (!amax_out || (!x && rows > 0 && cols > 0)) return fail(FP8Q_ERR_INVALID_ARG, "fp8_amax: NULL pointer");
    if (cols % 8 || ld % 8 || !aligned16(x)) return fail(FP8Q_ERR_UNSUPPORTED, "fp8_amax: cols and ld must be multiples of 8 and x 16-byte aligned");
    int rc = check_device();
    if (rc) return rc;
    hipStream_t st = static_cast<hipStream_t>(stream);
    fp8q::launch_amax(x, in_dtype == FP8Q_IN_BF16, rows, cols, ld, amax_out, st);
    return check_launch("fp8_amax");
}

int fp8_quantize(int mode, int fmt, const void* x, int in_dtype, int64_t rows, int64_t cols, int64_t ld,
                 int block_r, int block_c, int transpose_out, uint8_t* q, int64_t ldq, void* scales,
                 float* tensor_scale, int scale_is_input, float* amax_out, void* stream) {
    g_err[0] = 0;
    if (mode < FP8Q_TENSOR || mode > FP8Q_BLOCK_E8M0) return fail(FP8Q_ERR_INVALID_ARG, "fp8_quantize: unknown mode %d", mode);
    if (!valid_fmt(fmt)) return fail(FP8Q_ERR_INVALID_ARG, "fp8_quantize: fmt %d is not FP8Q_E4M3/E5M2", fmt);
    if (!valid_in(in_dtype)) return fail(FP8Q_ERR_INVALID_ARG, "fp8_quantize: in_dtype %d is not FP8Q_IN_F32/BF16", in_dtype);
    if (transpose_out != 0 && transpose_out != 1) return fail(FP8Q_ERR_INVALID_ARG, "fp8_quantize: transpose_out must be 0 or 1");
    if (rows < 0 || cols < 0 || ld < cols) return fail(FP8Q_ERR_INVALID_ARG, "fp8_quantize: bad shape rows=%lld cols=%lld ld=%lld",
                                                      (long long)rows, (long long)cols, (long long)ld);
    const int64_t R = transpose_out ? cols : rows, K = transpose_out ? rows : cols;
    if (ldq < K) return fail(FP8Q_ERR_INVALID_ARG, "fp8_quantize: ldq=%lld is smaller than the output row length %lld",
                             (long long)ldq, (long long)K);
    const bool empty = rows == 0 || cols == 0;
    if (!empty && (!x || !q)) return fail(FP8Q_ERR_INVALID_ARG, "fp8_quantize: NULL x or q");
    if ((mode == FP8Q_BLOCK || mode == FP8Q_BLOCK_E8M0) && (block_r <= 0 || block_c <= 0))
        return fail(FP8Q_ERR_INVALID_ARG, "fp8_quantize: block size (%d, %d) must be two positive integers", block_r, block_c);
    if (mode != FP8Q_TENSOR && !scales && !empty) return fail(FP8Q_ERR_INVALID_ARG, "fp8_quantize: NULL scales");
    const bool needs_amax = (mode == FP8Q_TENSOR || mode == FP8Q_MOSS) && !scale_is_input;
    if ((mode == FP8Q_TENSOR || mode == FP8Q_MOSS) && !tensor_scale)
        return fail(FP8Q_ERR_INVALID_ARG, "fp8_quantize: tensor_scale is required for TENSOR and MOSS");
    if (needs_amax && !amax_out)
        return fail(FP8Q_ERR_INVALID_ARG, "fp8_quantize: amax_out is required when the scale is derived (scale_is_input=0)");
    if (cols % 8 || ld % 8 || !aligned16(x))
        return fail(FP8Q_ERR_UNSUPPORTED, "fp8_quantize: needs cols %% 8 == 0, ld %% 8 == 0 and a 16-byte aligned x");
    if (!aligned4(tensor_scale) || !aligned4(amax_out) || (mode == FP8Q_BLOCK && !aligned4(scales)))
        return fail(FP8Q_ERR_INVALID_ARG, "fp8_quantize: fp32 scale and amax pointers must be 4-byte aligned");
    (void)R;
    int rc = check_device();
    if (rc) return rc;
    hipStream_t st = static_cast<hipStream_t>(stream);
    const bool bf16 = in_dtype == FP8Q_IN_BF16;

    fp8q::CastArgs a{};
    a.mode = mode;
    a.fmt = fmt;
    a.x = x;
    a.bf16 = bf16;
    a.rows = rows;
    a.cols = cols;
    a.ld = ld;
    a.transpose = transpose_out != 0;
    a.q = q;
    a.ldq = ldq;
    a.scales = scales;
    a.block_r = block_r;
    a.block_c = block_c;
    a.vec_out = ldq % 16 == 0 && aligned16(q);
    if (mode == FP8Q_TENSOR && needs_amax && !empty && small_tensor(rows, cols)) {
        // small tensor: amax, scale and cast in one launch
        a.amax_out = amax_out;
        a.scale_out = tensor_scale;
        fp8q::launch_cast_small_current(a, st);
        return check_launch("fp8_quantize");
    }
    if (mode == FP8Q_TENSOR || mode == FP8Q_MOSS) {
        if (needs_amax) {
            fp8q::launch_amax(x, bf16, rows, cols, ld, amax_out, st);
            a.amax_in = amax_out;
            a.scale_out = tensor_scale;
        } else {
            a.scale_in = tensor_scale;
            if (mode == FP8Q_TENSOR && amax_out) {
                fp8q::launch_zero_u32(amax_out, st);
                a.amax_out = amax_out;
            }
        }
    }
    if (needs_amax && empty) {
        // amax of an empty tensor is 0: the scale falls back to 1 (no cast kernel runs)
        fp8q::launch_fill_f32(tensor_scale, 1.0f, st);
    }
    fp8q::launch_cast(a, st);
    return check_launch("fp8_quantize");
}

int fp8_quantize_dual(int mode, int fmt, const void* x, int in_dtype, int64_t rows, int64_t cols, int64_t ld,
                      uint8_t* q, int64_t ldq, void* scales, uint8_t* qt, int64_t ldqt, void* scales_t,
                      float* tensor_scale, int scale_is_input, float* amax_out, void* stream) {
    g_err[0] = 0;
    if (mode != FP8Q_TENSOR && mode != FP8Q_MX && mode != FP8Q_MOSS)
        return fail(FP8Q_ERR_INVALID_ARG, "fp8_quantize_dual: mode %d is not FP8Q_TENSOR/MX/MOSS", mode);
    if (!valid_fmt(fmt)) return fail(FP8Q_ERR_INVALID_ARG, "fp8_quantize_dual: fmt %d is not FP8Q_E4M3/E5M2", fmt);
    if (!valid_in(in_dtype)) return fail(FP8Q_ERR_INVALID_ARG, "fp8_quantize_dual: in_dtype %d is not FP8Q_IN_F32/BF16", in_dtype);
    if (rows < 0 || cols < 0 || ld < cols)
        return fail(FP8Q_ERR_INVALID_ARG, "fp8_quantize_dual: bad shape rows=%lld cols=%lld ld=%lld", (long long)rows,
                    (long long)cols, (long long)ld);
    if (ldq < cols || ldqt < rows)
        return fail(FP8Q_ERR_INVALID_ARG, "fp8_quantize_dual: ldq=%lld / ldqt=%lld smaller than cols=%lld / rows=%lld",
                    (long long)ldq, (long long)ldqt, (long long)cols, (long long)rows);
    const bool empty = rows == 0 || cols == 0;
    if (!empty && (!x || !q || !qt)) return fail(FP8Q_ERR_INVALID_ARG, "fp8_quantize_dual: NULL x, q or qt");
    if (mode != FP8Q_TENSOR && !empty && (!scales || !scales_t))
        return fail(FP8Q_ERR_INVALID_ARG, "fp8_quantize_dual: NULL scales or scales_t");
    const bool needs_amax = (mode == FP8Q_TENSOR || mode == FP8Q_MOSS) && !scale_is_input;
    if ((mode == FP8Q_TENSOR || mode == FP8Q_MOSS) && !tensor_scale)
        return fail(FP8Q_ERR_INVALID_ARG, "fp8_quantize_dual: tensor_scale is required for TENSOR and MOSS");
    if (needs_amax && !amax_out)
        return fail(FP8Q_ERR_INVALID_ARG, "fp8_quantize_dual: amax_out is required when the scale is derived");
    if (cols % 8 || ld % 8 || !aligned16(x))
        return fail(FP8Q_ERR_UNSUPPORTED, "fp8_quantize_dual: needs cols %% 8 == 0, ld %% 8 == 0 and a 16-byte aligned x");
    const bool one_pass = rows % 32 == 0 && cols % 32 == 0 && ldq % 16 == 0 && ldqt % 16 == 0 && aligned16(q) &&
                          aligned16(qt);
    if (!one_pass) {
        // the two single-copy casts; the second uses the scale the first one used or derived
        int rc = fp8_quantize(mode, fmt, x, in_dtype, rows, cols, ld, 1, 1, 0, q, ldq, scales, tensor_scale,
                              scale_is_input, amax_out, stream);
        if (rc) return rc;
        return fp8_quantize(mode, fmt, x, in_dtype, rows, cols, ld, 1, 1, 1, qt, ldqt, scales_t, tensor_scale,
                            mode == FP8Q_MX ? 0 : 1, nullptr, stream);
    }
    int rc = check_device();
    if (rc) return rc;
    hipStream_t st = static_cast<hipStream_t>(stream);
    const bool bf16 = in_dtype == FP8Q_IN_BF16;
    if (needs_amax && empty) {
        fp8q::launch_fill_f32(amax_out, 0.0f, st);
        fp8q::launch_fill_f32(tensor_scale, 1.0f, st);
        return check_launch("fp8_quantize_dual");
    }
    fp8q::CastArgs a{};
    a.mode = mode;
    a.fmt = fmt;
    a.x = x;
    a.bf16 = bf16;
    a.rows = rows;
    a.cols = cols;
    a.ld = ld;
    a.transpose = true;
    a.q = qt;
    a.ldq = ldqt;
    a.scales = scales_t;
    a.q2 = q;
    a.ldq2 = ldq;
    a.scales2 = scales;
    a.vec_out = true;
    if (mode == FP8Q_TENSOR && needs_amax && !empty && small_tensor(rows, cols)) {
        // small tensor: amax, scale and both copies in one launch
        a.amax_out = amax_out;
        a.scale_out = tensor_scale;
        fp8q::launch_cast_small_current(a, st);
        return check_launch("fp8_quantize_dual");
    }
    if (mode == FP8Q_TENSOR || mode == FP8Q_MOSS) {
        if (needs_amax) {
            fp8q::launch_amax(x, bf16, rows, cols, ld, amax_out, st);
            a.amax_in = amax_out;
            a.scale_out = tensor_scale;
        } else {
            a.scale_in = tensor_scale;
            if (mode == FP8Q_TENSOR && amax_out) {
                fp8q::launch_zero_u32(amax_out, st);
                a.amax_out = amax_out;
            }
        }
    }
    fp8q::launch_cast_dual(a, st);
    return check_launch("fp8_quantize_dual");
}

int fp8_history_update(float* history, int64_t len, const float* amax_new, float* scale_inout, int fmt, void* stream) {
    g_err[0] = 0;
    if (!valid_fmt(fmt)) return fail(FP8Q_ERR_INVALID_ARG, "fp8_history_update: fmt %d is not FP8Q_E4M3/E5M2", fmt);
    if (len < 1 || len > 4096) return fail(FP8Q_ERR_INVALID_ARG, "fp8_history_update: len=%lld outside [1, 4096]", (long long)len);
    if (!history || !amax_new || !scale_inout) return fail(FP8Q_ERR_INVALID_ARG, "fp8_history_update: NULL pointer");
    int rc = check_device();
    if (rc) return rc;
    fp8q::launch_history(history, (int)len, amax_new, scale_inout, fmt, static_cast<hipStream_t>(stream));
    return check_launch("fp8_history_update");
}

int fp8_scaled_gemm(int mode, const uint8_t* A, int afmt, const void* Ascale, const uint8_t* B, int bfmt,
                    const void* Bscale, const float* Aglobal, const float* Bglobal, int64_t M, int64_t N, int64_t K,
                    int64_t lda, int64_t ldb, void* C, int out_dtype, int64_t ldc, void* stream) {
    g_err[0] = 0;
    if (mode < FP8Q_TENSOR || mode > FP8Q_BLOCK_E8M0) return fail(FP8Q_ERR_INVALID_ARG, "fp8_scaled_gemm: unknown mode %d", mode);
    if (!valid_fmt(afmt) || !valid_fmt(bfmt)) return fail(FP8Q_ERR_INVALID_ARG, "fp8_scaled_gemm: bad operand format");
    if (out_dtype != FP8Q_OUT_F32 && out_dtype != FP8Q_OUT_BF16)
        return fail(FP8Q_ERR_INVALID_ARG, "fp8_scaled_gemm: out_dtype %d is not FP8Q_OUT_F32/BF16 (it is required)", out_dtype);
    if (M < 0 || N < 0 || K < 0 || lda < K || ldb < K || ldc < N)
        return fail(FP8Q_ERR_INVALID_ARG, "fp8_scaled_gemm: bad shape M=%lld N=%lld K=%lld lda=%lld ldb=%lld ldc=%lld",
                    (long long)M, (long long)N, (long long)K, (long long)lda, (long long)ldb, (long long)ldc);
    if (M > 0 && N > 0 && !C) return fail(FP8Q_ERR_INVALID_ARG, "fp8_scaled_gemm: NULL C");
    if (M > 0 && N > 0 && K > 0 && (!A || !B)) return fail(FP8Q_ERR_INVALID_ARG, "fp8_scaled_gemm: NULL A or B");
    if ((mode == FP8Q_TENSOR || mode == FP8Q_MOSS) && (!Aglobal || !Bglobal))
        return fail(FP8Q_ERR_INVALID_ARG, "fp8_scaled_gemm: Aglobal and Bglobal are required for TENSOR and MOSS");
    const bool blocked = mode == FP8Q_BLOCK || mode == FP8Q_BLOCK_E8M0;
    const bool a_static = blocked && !Ascale && Aglobal;     // static per-tensor activation scale
    if (mode != FP8Q_TENSOR && K > 0 && M > 0 && N > 0 && ((!Ascale && !a_static) || !Bscale))
        return fail(FP8Q_ERR_INVALID_ARG, "fp8_scaled_gemm: Ascale (or, for BLOCK, a static Aglobal) and Bscale are "
                    "required for BLOCK, BLOCK_E8M0, MX and MOSS");
    if (K > 0 && (K % 16 || lda % 16 || ldb % 16 || !aligned16(A) || !aligned16(B)))
        return fail(FP8Q_ERR_UNSUPPORTED, "fp8_scaled_gemm: needs K, lda, ldb multiples of 16 and 16-byte aligned A, B");
    // scale arrays are read in 4-byte words, except UE8M0 weight-block scales (read byte by byte)
    if (!aligned4(Aglobal) || !aligned4(Bglobal) || !aligned4(Ascale) || (mode != FP8Q_BLOCK_E8M0 && !aligned4(Bscale)))
        return fail(FP8Q_ERR_UNSUPPORTED, "fp8_scaled_gemm: Ascale, Aglobal, Bglobal and (except for BLOCK_E8M0) Bscale "
                    "must be 4-byte aligned");
    int rc = check_device();
    if (rc) return rc;
    fp8q::GemmArgs g{};
    g.mode = mode;
    g.a_static = a_static;
    g.b_e8m0 = mode == FP8Q_BLOCK_E8M0;
    g.afmt = afmt;
    g.bfmt = bfmt;
    g.A = A;
    g.B = B;
    g.Ascale = Ascale;
    g.Bscale = Bscale;
    g.Aglobal = Aglobal;
    g.Bglobal = Bglobal;
    g.M = M;
    g.N = N;
    g.K = K;
    g.lda = lda;
    g.ldb = ldb;
    g.C = C;
    g.out_bf16 = out_dtype == FP8Q_OUT_BF16;
    g.ldc = ldc;
    fp8q::launch_gemm(g, static_cast<hipStream_t>(stream));
    return check_launch("fp8_scaled_gemm");
}

int fp8_history_merge(float* hist_dst, const float* hist_src, int64_t len, float* scale_dst, const float* scale_src,
                      void* stream) {
    g_err[0] = 0;
    if (len < 0) return fail(FP8Q_ERR_INVALID_ARG, "fp8_history_merge: len=%lld < 0", (long long)len);
    if (!scale_dst || !scale_src || (len > 0 && (!hist_dst || !hist_src)))
        return fail(FP8Q_ERR_INVALID_ARG, "fp8_history_merge: NULL pointer");
    int rc = check_device();
    if (rc) return rc;
    fp8q::launch_history_merge(hist_dst, hist_src, len, scale_dst, scale_src, static_cast<hipStream_t>(stream));
    return check_launch("fp8_history_merge");
}

int fp8_auto_scale(float* state, int rescale, const float* amax_now, float lr, int fmt, float* scale_out, void* stream) {
    g_err[0] = 0;
    if (!valid_fmt(fmt)) return fail(FP8Q_ERR_INVALID_ARG, "fp8_auto_scale: fmt %d is not FP8Q_E4M3/E5M2", fmt);
    if (rescale != 0 && rescale != 1) return fail(FP8Q_ERR_INVALID_ARG, "fp8_auto_scale: rescale must be 0 or 1");
    if (!state || !scale_out || (rescale && !amax_now)) return fail(FP8Q_ERR_INVALID_ARG, "fp8_auto_scale: NULL pointer");
    if (!(lr >= 0.0f) || lr == __builtin_huge_valf())
        return fail(FP8Q_ERR_INVALID_ARG, "fp8_auto_scale: the learning rate must be finite and >= 0");
    int rc = check_device();
    if (rc) return rc;
    fp8q::launch_auto_scale(state, rescale, amax_now, lr, fmt, scale_out, static_cast<hipStream_t>(stream));
    return check_launch("fp8_auto_scale");
}

int fp8_scale_to_e8m0(const float* s, int64_t n, uint8_t* e8m0, int32_t* bad_count, void* stream) {
    g_err[0] = 0;
    if (n < 0) return fail(FP8Q_ERR_INVALID_ARG, "fp8_scale_to_e8m0: n=%lld < 0", (long long)n);
    if (!bad_count || (n > 0 && (!s || !e8m0))) return fail(FP8Q_ERR_INVALID_ARG, "fp8_scale_to_e8m0: NULL pointer");
    int rc = check_device();
    if (rc) return rc;
    fp8q::launch_scale_to_e8m0(s, n, e8m0, bad_count, static_cast<hipStream_t>(stream));
    return check_launch("fp8_scale_to_e8m0");
}

int fp8_block_dequantize(int mode, int fmt, const uint8_t* q, int64_t rows, int64_t cols, int64_t ldq, const void* scales,
                         int block_r, int block_c, void* out, int out_dtype, int64_t ldo, void* stream) {
    g_err[0] = 0;
    if (mode != FP8Q_BLOCK && mode != FP8Q_BLOCK_E8M0)
        return fail(FP8Q_ERR_INVALID_ARG, "fp8_block_dequantize: mode %d is not FP8Q_BLOCK/BLOCK_E8M0", mode);
    if (!valid_fmt(fmt)) return fail(FP8Q_ERR_INVALID_ARG, "fp8_block_dequantize: fmt %d is not FP8Q_E4M3/E5M2", fmt);
    if (out_dtype != FP8Q_OUT_F32 && out_dtype != FP8Q_OUT_BF16)
        return fail(FP8Q_ERR_INVALID_ARG, "fp8_block_dequantize: out_dtype %d is not FP8Q_OUT_F32/BF16", out_dtype);
    if (block_r <= 0 || block_c <= 0)
        return fail(FP8Q_ERR_INVALID_ARG, "fp8_block_dequantize: block size (%d, %d) must be two positive integers",
                    block_r, block_c);
    if (rows < 0 || cols < 0 || ldq < cols || ldo < cols)
        return fail(FP8Q_ERR_INVALID_ARG, "fp8_block_dequantize: bad shape rows=%lld cols=%lld ldq=%lld ldo=%lld",
                    (long long)rows, (long long)cols, (long long)ldq, (long long)ldo);
    if (rows > 0 && cols > 0 && (!q || !scales || !out)) return fail(FP8Q_ERR_INVALID_ARG, "fp8_block_dequantize: NULL pointer");
    int rc = check_device();
    if (rc) return rc;
    fp8q::DequantArgs a{};
    a.e8m0 = mode == FP8Q_BLOCK_E8M0;
    a.fmt = fmt;
    a.q = q;
    a.rows = rows;
    a.cols = cols;
    a.ldq = ldq;
    a.scales = scales;
    a.block_r = block_r;
    a.block_c = block_c;
    a.out = out;
    a.out_bf16 = out_dtype == FP8Q_OUT_BF16;
    a.ldo = ldo;
    const int64_t esz = a.out_bf16 ? 2 : 4;
    a.vec = cols % 16 == 0 && block_c % 16 == 0 && ldq % 16 == 0 && (ldo * esz) % 16 == 0 && aligned16(q) && aligned16(out);
    fp8q::launch_block_dequantize(a, static_cast<hipStream_t>(stream));
    return check_launch("fp8_block_dequantize");
}

}  // extern "C"
