// Device helpers shared by the FP8 cast, amax and GEMM kernels (gfx950 / CDNA4).
//
// FP8 formats are OCP e4m3fn (max 448) and e5m2 (max 57344).  gfx950's v_cvt_pk_{fp8,bf8}_f32
// rounds to nearest even and produces subnormals, but it does not saturate (values past MAX become
// NaN / Inf) and it maps every NaN to one fixed byte.  So every cast here clips first (v_med3) and
// lanes holding NaN take a slow path that writes S.1111111 with the input's sign.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fp8q {

constexpr int kE4M3 = 0;
constexpr int kE5M2 = 1;

template <int FMT> __device__ __forceinline__ constexpr float fmt_max() { return FMT == kE4M3 ? 448.0f : 57344.0f; }
// exponent EM and the mantissa threshold of MAX = 1.75 * 2^EM
template <int FMT> __device__ __forceinline__ constexpr int fmt_max_exp() { return FMT == kE4M3 ? 8 : 15; }

// ------------------------------------------------------------------ bf16 / fp32 loads
__device__ __forceinline__ float bf16lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

// 8 consecutive elements starting at p (16-byte aligned) into v[0..7] as fp32.
template <bool BF16>
__device__ __forceinline__ void load8(const void* p, float* v) {
    if (BF16) {
        uint4 w = *reinterpret_cast<const uint4*>(p);
        v[0] = bf16lo(w.x); v[1] = bf16hi(w.x); v[2] = bf16lo(w.y); v[3] = bf16hi(w.y);
        v[4] = bf16lo(w.z); v[5] = bf16hi(w.z); v[6] = bf16lo(w.w); v[7] = bf16hi(w.w);
    } else {
        float4 a = reinterpret_cast<const float4*>(p)[0];
        float4 b = reinterpret_cast<const float4*>(p)[1];
        v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w; v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
    }
}

__device__ __forceinline__ uint32_t absbits(float v) { return __float_as_uint(v) & 0x7FFFFFFFu; }

// max |x| of the 2N bf16 values packed two per word in w, as the fp32 bits of that magnitude:
// magnitudes of bf16 (and NaN above Inf) order like their 15-bit patterns, so one packed 16-bit
// max per word replaces an unpack, a mask and a max per value
template <int N>
__device__ __forceinline__ uint32_t bf16w_absmax(const uint32_t* w) {
    typedef unsigned short u16x2 __attribute__((ext_vector_type(2)));
    u16x2 m = {0, 0};
#pragma unroll
    for (int j = 0; j < N; ++j) m = __builtin_elementwise_max(m, __builtin_bit_cast(u16x2, w[j] & 0x7FFF7FFFu));
    return (uint32_t)max(m[0], m[1]) << 16;
}
// min over the same values of (|x| bits - 1) as fp32 bits, a zero wrapping to 0xFFFFFFFF: per
// 16-bit half (|x| - 1) wraps the same way, and (d << 16) | 0xFFFF maps it monotonically onto the
// fp32 difference, so the packed min gives the exact value
template <int N>
__device__ __forceinline__ uint32_t bf16w_minm1(const uint32_t* w) {
    typedef unsigned short u16x2 __attribute__((ext_vector_type(2)));
    const u16x2 one = {1, 1};
    u16x2 m = {0xFFFF, 0xFFFF};
#pragma unroll
    for (int j = 0; j < N; ++j) m = __builtin_elementwise_min(m, __builtin_bit_cast(u16x2, w[j] & 0x7FFF7FFFu) - one);
    return ((uint32_t)min(m[0], m[1]) << 16) | 0xFFFFu;
}

// ------------------------------------------------------------------ FP8 packing
// Four fp32 -> four FP8 bytes, byte i = code(v_i).  Inputs must already be clipped to +-MAX.
template <int FMT>
__device__ __forceinline__ uint32_t cvt4(float a, float b, float c, float d) {
    int w;
    if (FMT == kE4M3) {
        w = __builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false);
        w = __builtin_amdgcn_cvt_pk_fp8_f32(c, d, w, true);
    } else {
        w = __builtin_amdgcn_cvt_pk_bf8_f32(a, b, 0, false);
        w = __builtin_amdgcn_cvt_pk_bf8_f32(c, d, w, true);
    }
    return (uint32_t)w;
}

template <int FMT> __device__ __forceinline__ float clip(float v) {
    return __builtin_amdgcn_fmed3f(v, -fmt_max<FMT>(), fmt_max<FMT>());
}

// Slow-path element: v is the exact scaled value (may be NaN/Inf).  Clip keeping NaN, cast, and
// give NaN the byte S.1111111.
template <int FMT>
__device__ __forceinline__ uint32_t code_slow(float v) {
    if (v != v) return ((__float_as_uint(v) >> 24) & 0x80u) | 0x7Fu;
    float c = clip<FMT>(v);
    return cvt4<FMT>(c, c, c, c) & 0xFFu;
}

// ------------------------------------------------------------------ exact division
// q = RN(x / s) given y = RN(1 / s): one Markstein correction of q0 = RN(x * y).  Valid (bit-equal
// to the IEEE quotient) when s, y, x, x*y and the remainder stay in the normal range; callers
// guarantee that with the fast-path guards below and use IEEE division otherwise.
// The correction step turns a -0 quotient into +0 (-0 + +0 = +0), so the sign is taken from q0,
// which always carries the sign of x / s.
__device__ __forceinline__ float div_fast(float x, float s, float y) {
    float q0 = x * y;
    float r = __builtin_fmaf(-q0, s, x);
    return __builtin_copysignf(__builtin_fmaf(r, y, q0), q0);
}

// Uniform guard on the divisor: 2^-64 <= s <= 2^64.
__device__ __forceinline__ bool divisor_ok(float s) {
    uint32_t b = __float_as_uint(s);
    return b >= 0x1F800000u && b <= 0x5F800000u;
}
// Per-chunk guard on the dividends: every |x| <= 2^60 and finite, every nonzero |x| >= 2^-96.
// max_abs / min_abs_m1 are the chunk's max of |x| bits and min of (|x| bits - 1) (zero wraps).
__device__ __forceinline__ bool dividends_ok(uint32_t max_abs, uint32_t min_abs_m1) {
    return max_abs <= 0x5D800000u && min_abs_m1 >= 0x0F800000u - 1u;
}

// RN(1/s), correctly rounded (IEEE division).
__device__ __forceinline__ float recip_rn(float s) { return 1.0f / s; }

// Two-term reciprocal for bf16 dividends.  yh is 1/s rounded toward zero, so the residual
// 1 - s*yh (one fma) is >= 0 and yl = RN(residual * yh) is never negative: then x*yl carries the
// sign of x and a -0 dividend stays -0 through the fma.  yh + yl lies within about 2^-47 of 1/s,
// so fma(x, yh, x*yl) is RN(x/s) unless x/s lies that close to a rounding midpoint.  A bf16 x is m * 2^k with m one of 128
// significands in [1, 2), and every step scales exactly by 2^k while the results stay normal, so
// checking the 128 significands once decides the question for every bf16 dividend whose quotient
// (and x*yl) is a normal number; quotients below that are far under the FP8 range anyway.
__device__ __forceinline__ float recip_hi_rz(float s) {
    const float y = 1.0f / s;
    return __builtin_fmaf(-s, y, 1.0f) < 0.0f ? __uint_as_float(__float_as_uint(y) - 1u) : y;
}
__device__ __forceinline__ float recip_lo(float s, float yh) { return __builtin_fmaf(-s, yh, 1.0f) * yh; }
__device__ __forceinline__ float mul2(float x, float yh, float yl) { return __builtin_fmaf(x, yh, x * yl); }
// Wave-uniform: true when mul2 equals IEEE division by s for all 128 bf16 significands (all lanes of
// the wave must be active).
__device__ __forceinline__ bool mul2_exact_bf16(float s, float yh, float yl) {
    const int lane = threadIdx.x & 63;
    const float m1 = 1.0f + (float)lane * (1.0f / 128.0f), m2 = m1 + 0.5f;
    const bool ok = mul2(m1, yh, yl) == m1 / s && mul2(m2, yh, yl) == m2 / s;
    return __all(ok);
}

// scale = fl(amax / MAX); 1.0 (or `fallback`) on amax zero / non-finite / underflow.
template <int FMT>
__device__ __forceinline__ float scale_from_amax(float amax, float fallback) {
    if (!(amax > 0.0f) || __float_as_uint(amax) >= 0x7F800000u) return fallback;
    float s = amax / fmt_max<FMT>();
    return s == 0.0f ? fallback : s;
}

// ------------------------------------------------------------------ E8M0 exponents
// Normalize a positive finite float: v = m * 2^E with m in [1,2); returns E, and sets mbits to
// the 23 fraction bits of m.
__device__ __forceinline__ int norm_exp(float v, uint32_t& mbits) {
    int e;
    float fr = __builtin_frexpf(v, &e);        // v = fr * 2^e, fr in [0.5, 1)
    mbits = __float_as_uint(fr * 2.0f) & 0x7FFFFFu;
    return e - 1;
}

// MX: smallest e in [-127, 127] with MAX * 2^e >= amax (127 if none: non-finite amax).
template <int FMT>
__device__ __forceinline__ int mx_exponent(float amax) {
    if (!(amax > 0.0f)) return amax == 0.0f ? -127 : 127;   // NaN -> 127
    if (__float_as_uint(amax) >= 0x7F800000u) return 127;
    uint32_t mb;
    int E = norm_exp(amax, mb);
    int e = E - fmt_max_exp<FMT>() + (mb > 0x600000u ? 1 : 0);   // MAX mantissa is 1.75 = 1.11b
    return e < -127 ? -127 : (e > 127 ? 127 : e);
}

// fl(a / MAX) for a >= 0: the one-correction division where its guards hold, else IEEE division.
template <int FMT>
__device__ __forceinline__ float div_by_max(float a) {
    const uint32_t b = __float_as_uint(a);
    if (b >= 0x0F800000u && b <= 0x5D800000u) return div_fast(a, fmt_max<FMT>(), 1.0f / fmt_max<FMT>());
    return a / fmt_max<FMT>();
}

// S = ms * 2^ES, computed once per tensor for moss_exponent_p.
struct SParts {
    int ES;
    uint32_t ms;
};
__device__ __forceinline__ SParts s_parts(float S) {
    SParts p;
    p.ES = norm_exp(S, p.ms);
    return p;
}
// moss_exponent(S, s_i) with S given by its parts.
__device__ __forceinline__ int moss_exponent_p(const SParts& p, float s_i) {
    if (!(s_i > 0.0f)) return s_i == 0.0f ? -127 : 0;         // NaN -> 0
    if (__float_as_uint(s_i) >= 0x7F800000u) return 0;
    uint32_t mi;
    int Ei = norm_exp(s_i, mi);
    int e = Ei - p.ES + (mi > p.ms ? 1 : 0);
    return e < -127 ? -127 : (e > 0 ? 0 : e);
}

// MOSS: smallest e in [-127, 0] with S * 2^e >= s_i (0 if none), S > 0 finite.
__device__ __forceinline__ int moss_exponent(float S, float s_i) {
    if (!(s_i > 0.0f)) return s_i == 0.0f ? -127 : 0;         // NaN -> 0
    if (__float_as_uint(s_i) >= 0x7F800000u) return 0;
    uint32_t ms, mi;
    int ES = norm_exp(S, ms);
    int Ei = norm_exp(s_i, mi);
    int e = Ei - ES + (mi > ms ? 1 : 0);
    return e < -127 ? -127 : (e > 0 ? 0 : e);
}

// ------------------------------------------------------------------ reductions
__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) {
    for (int off = 32; off > 0; off >>= 1) {
        uint32_t o = (uint32_t)__shfl_xor((int)v, off, 64);
        v = v > o ? v : o;
    }
    return v;
}

// max over groups of G consecutive lanes (G = 1, 2, 4, 8, 16, 32, 64)
template <int G>
__device__ __forceinline__ uint32_t group_max_u32(uint32_t v) {
    for (int off = G / 2; off > 0; off >>= 1) {
        uint32_t o = (uint32_t)__shfl_xor((int)v, off, 64);
        v = v > o ? v : o;
    }
    return v;
}

}  // namespace fp8q
