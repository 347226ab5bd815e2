// Delayed-scaling state merge, MOSS automatic weight scaling, exact fp32 -> UE8M0 scale conversion
// and 128x128 block dequantization.
//
//   history merge    two uses of one delayed-scaling state each update it; the updates combine by
//                    elementwise max, not by sum (page "Flax FP8 量化实战指南 ...", section 5.3).
//   automatic scale  the weight max grows by at most the learning rate per optimizer step, so the
//                    scale is predicted from the last measured max plus the learning rates since,
//                    with a fresh max-reduction at each interval start (page "MOSS:高效、精确的 FP8
//                    LLM 训练 ...", section 5).
//   UE8M0 scales     power-of-two block scales kept in fp32 containers are converted to E8M0
//                    bytes exactly; anything else is rejected (page "Transformers 中的细粒度 FP8
//                    量化配置 ...", section 七).
//   block dequantize the block scale folded back into the weight: fl32(decode(q) * s) in fp32 or
//                    rounded to bf16 (same page, section 五).
#include "common.cuh"
#include "kernels.h"

namespace fp8q {

// ------------------------------------------------------------------ history merge
__device__ __forceinline__ float max_nan(float a, float b) {
    if (a != a || b != b) return __builtin_nanf("");
    return a > b ? a : b;
}

__global__ __launch_bounds__(256) void history_merge_kernel(float* __restrict__ hist_dst, const float* __restrict__ hist_src,
                                                            int64_t len, float* __restrict__ scale_dst,
                                                            const float* __restrict__ scale_src) {
    for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < len; i += (int64_t)gridDim.x * 256)
        hist_dst[i] = max_nan(hist_dst[i], hist_src[i]);
    if (blockIdx.x == 0 && threadIdx.x == 0) *scale_dst = max_nan(*scale_dst, *scale_src);
}

int launch_history_merge(float* hist_dst, const float* hist_src, int64_t len, float* scale_dst, const float* scale_src,
                         hipStream_t st) {
    int64_t blocks = (len + 255) / 256;
    if (blocks < 1) blocks = 1;
    if (blocks > 1024) blocks = 1024;
    hipLaunchKernelGGL(history_merge_kernel, dim3((unsigned)blocks), dim3(256), 0, st, hist_dst, hist_src, len, scale_dst,
                       scale_src);
    return 0;
}

// ------------------------------------------------------------------ automatic scaling
// state[0] = the weight max measured at the interval start, state[1] = the learning rates summed
// since (fp32, one addition per step).
template <int FMT>
__global__ void auto_scale_kernel(float* __restrict__ state, int rescale, const float* __restrict__ amax_now, float lr,
                                  float* __restrict__ scale_out) {
    float base = state[0], sum = state[1];
    if (rescale) {
        base = *amax_now;
        sum = 0.0f;
    }
    const float predicted = base + sum;
    *scale_out = scale_from_amax<FMT>(predicted, 1.0f);
    state[0] = base;
    state[1] = sum + lr;
}

int launch_auto_scale(float* state, int rescale, const float* amax_now, float lr, int fmt, float* scale_out,
                      hipStream_t st) {
    if (fmt == kE4M3) hipLaunchKernelGGL(auto_scale_kernel<kE4M3>, dim3(1), dim3(1), 0, st, state, rescale, amax_now, lr, scale_out);
    else hipLaunchKernelGGL(auto_scale_kernel<kE5M2>, dim3(1), dim3(1), 0, st, state, rescale, amax_now, lr, scale_out);
    return 0;
}

// ------------------------------------------------------------------ fp32 -> UE8M0
// 2^e (e in [-127, 127]) -> e + 127: for normal powers of two that is the exponent field itself;
// 2^-127 is the one fp32 subnormal in range.  Anything else becomes 0xFF and is counted.
__global__ __launch_bounds__(256) void scale_to_e8m0_kernel(const float* __restrict__ s, int64_t n,
                                                            uint8_t* __restrict__ out, int32_t* __restrict__ bad) {
    int32_t nbad = 0;
    for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (int64_t)gridDim.x * 256) {
        const uint32_t b = __float_as_uint(s[i]);
        const uint32_t ef = b >> 23;                         // sign and exponent field
        uint32_t byte;
        if (b == 0x00400000u) byte = 0u;                     // 2^-127
        else if ((b & 0x7FFFFFu) == 0u && ef >= 1u && ef <= 254u) byte = ef;
        else {
            byte = 0xFFu;
            ++nbad;
        }
        out[i] = (uint8_t)byte;
    }
    if (nbad) atomicAdd(bad, nbad);
}

__global__ void zero_i32_kernel(int32_t* p) { *p = 0; }

int launch_scale_to_e8m0(const float* s, int64_t n, uint8_t* e8m0, int32_t* bad_count, hipStream_t st) {
    hipLaunchKernelGGL(zero_i32_kernel, dim3(1), dim3(1), 0, st, bad_count);
    if (n == 0) return 0;
    int64_t blocks = (n + 255) / 256;
    if (blocks > 1024) blocks = 1024;
    hipLaunchKernelGGL(scale_to_e8m0_kernel, dim3((unsigned)blocks), dim3(256), 0, st, s, n, e8m0, bad_count);
    return 0;
}

// ------------------------------------------------------------------ block dequantize
__device__ __forceinline__ uint32_t bf16_rne_bits(float f) {
    const uint32_t u = __float_as_uint(f);
    const uint32_t r = (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
    return (u & 0x7FFFFFFFu) > 0x7F800000u ? ((u >> 16) | 0x40u) : r;
}

// two FP8 codes (bytes 2 HI, 2 HI + 1 of w) -> fp32, exact
template <int FMT, bool HI>
__device__ __forceinline__ void decode2(uint32_t w, float& a, float& b) {
    typedef float f2 __attribute__((ext_vector_type(2)));
    f2 v = FMT == kE4M3 ? __builtin_amdgcn_cvt_pk_f32_fp8((int)w, HI) : __builtin_amdgcn_cvt_pk_f32_bf8((int)w, HI);
    a = v[0];
    b = v[1];
}

template <bool E8>
__device__ __forceinline__ float block_scale(const DequantArgs& a, int64_t r, int64_t c) {
    const int64_t nbc = (a.cols + a.block_c - 1) / a.block_c;
    const int64_t i = (r / a.block_r) * nbc + c / a.block_c;
    if (E8) return __builtin_amdgcn_ldexpf(1.0f, (int)static_cast<const uint8_t*>(a.scales)[i] - 127);
    return static_cast<const float*>(a.scales)[i];
}

// Vectorized: one thread per 16 consecutive bytes of a row (cols % 16 == 0, block_c % 16 == 0,
// 16-byte aligned rows), so the 16 values share one block scale.
template <int FMT, bool E8, bool BF16OUT>
__global__ __launch_bounds__(256) void block_dequant_vec_kernel(DequantArgs a) {
    const int64_t cpr = a.cols / 16, total = a.rows * cpr;
    for (int64_t g = (int64_t)blockIdx.x * 256 + threadIdx.x; g < total; g += (int64_t)gridDim.x * 256) {
        const int64_t r = g / cpr, c = (g - r * cpr) * 16;
        const uint4 w = *reinterpret_cast<const uint4*>(a.q + r * a.ldq + c);
        const float s = block_scale<E8>(a, r, c);
        const uint32_t ww[4] = {w.x, w.y, w.z, w.w};
        float p[16];
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            decode2<FMT, false>(ww[k], p[4 * k], p[4 * k + 1]);
            decode2<FMT, true>(ww[k], p[4 * k + 2], p[4 * k + 3]);
        }
#pragma unroll
        for (int k = 0; k < 16; ++k) p[k] = p[k] * s;                  // one fp32 rounding
        if (BF16OUT) {
            uint32_t o[8];
#pragma unroll
            for (int k = 0; k < 8; ++k) o[k] = bf16_rne_bits(p[2 * k]) | (bf16_rne_bits(p[2 * k + 1]) << 16);
            uint4* dst = reinterpret_cast<uint4*>(static_cast<uint16_t*>(a.out) + r * a.ldo + c);
            dst[0] = make_uint4(o[0], o[1], o[2], o[3]);
            dst[1] = make_uint4(o[4], o[5], o[6], o[7]);
        } else {
            float4* dst = reinterpret_cast<float4*>(static_cast<float*>(a.out) + r * a.ldo + c);
#pragma unroll
            for (int k = 0; k < 4; ++k) dst[k] = make_float4(p[4 * k], p[4 * k + 1], p[4 * k + 2], p[4 * k + 3]);
        }
    }
}

// Any shape: one element per thread.
template <int FMT, bool E8, bool BF16OUT>
__global__ __launch_bounds__(256) void block_dequant_any_kernel(DequantArgs a) {
    const int64_t total = a.rows * a.cols;
    for (int64_t g = (int64_t)blockIdx.x * 256 + threadIdx.x; g < total; g += (int64_t)gridDim.x * 256) {
        const int64_t r = g / a.cols, c = g - r * a.cols;
        float v, unused;
        decode2<FMT, false>((uint32_t)a.q[r * a.ldq + c], v, unused);
        const float p = v * block_scale<E8>(a, r, c);
        if (BF16OUT) static_cast<uint16_t*>(a.out)[r * a.ldo + c] = (uint16_t)bf16_rne_bits(p);
        else static_cast<float*>(a.out)[r * a.ldo + c] = p;
    }
}

template <int FMT, bool E8, bool BF16OUT>
static void dequant_launch(const DequantArgs& a, hipStream_t st) {
    const int64_t work = a.vec ? a.rows * (a.cols / 16) : a.rows * a.cols;
    int64_t blocks = (work + 255) / 256;
    if (blocks > 8192) blocks = 8192;
    if (blocks < 1) return;
    if (a.vec) hipLaunchKernelGGL((block_dequant_vec_kernel<FMT, E8, BF16OUT>), dim3((unsigned)blocks), dim3(256), 0, st, a);
    else hipLaunchKernelGGL((block_dequant_any_kernel<FMT, E8, BF16OUT>), dim3((unsigned)blocks), dim3(256), 0, st, a);
}

template <int FMT>
static void dequant_fmt(const DequantArgs& a, hipStream_t st) {
    if (a.e8m0) {
        if (a.out_bf16) dequant_launch<FMT, true, true>(a, st);
        else dequant_launch<FMT, true, false>(a, st);
    } else {
        if (a.out_bf16) dequant_launch<FMT, false, true>(a, st);
        else dequant_launch<FMT, false, false>(a, st);
    }
}

int launch_block_dequantize(const DequantArgs& a, hipStream_t st) {
    if (a.rows == 0 || a.cols == 0) return 0;
    if (a.fmt == kE4M3) dequant_fmt<kE4M3>(a, st);
    else dequant_fmt<kE5M2>(a, st);
    return 0;
}

}  // namespace fp8q
