// amax reduction and delayed-scaling history update kernels.
//
// amax = max |x| ("Flax FP8 量化实战指南 ...", section 1).  The reduction runs on the sign-cleared
// fp32 bit patterns as unsigned integers: for non-negative floats integer order is numeric order and
// every NaN pattern sorts above +Inf, so the result is exact, NaN-propagating and independent of the
// order in which workgroups finish.  Each workgroup reduces in registers and LDS and issues one
// global atomic max into the output, which a one-thread kernel zeroes first.
#include "common.cuh"
#include "kernels.h"

#include <string.h>

namespace fp8q {

__global__ void fill_u32_kernel(uint32_t* p, uint32_t v) { *p = v; }

// Same-address atomics serialize in L2 (on the order of 10 ns each), so the reductions below use at
// most kAmaxBlocks workgroups of 1024 threads, each issuing one atomic max.
constexpr int kAmaxThreads = 1024;
constexpr int64_t kAmaxBlocks = 256;
constexpr int kAmaxUnroll = 8;       // 16-byte loads in flight per thread

typedef unsigned short u16x2 __attribute__((ext_vector_type(2)));

// Running max of |x| over one 16-byte vector.  bf16: the sign-cleared 16-bit patterns are kept as
// two packed unsigned maxima (bf16 is the upper half of fp32, so the same integer order holds);
// fp32: the sign-cleared 32-bit patterns.
template <bool BF16>
__device__ __forceinline__ uint32_t vmax_acc(uint32_t m, uint4 w) {
    if (BF16) {
        u16x2 a = __builtin_bit_cast(u16x2, w.x & 0x7FFF7FFFu), b = __builtin_bit_cast(u16x2, w.y & 0x7FFF7FFFu);
        u16x2 c = __builtin_bit_cast(u16x2, w.z & 0x7FFF7FFFu), d = __builtin_bit_cast(u16x2, w.w & 0x7FFF7FFFu);
        u16x2 r = __builtin_elementwise_max(__builtin_elementwise_max(a, b), __builtin_elementwise_max(c, d));
        return __builtin_bit_cast(uint32_t, __builtin_elementwise_max(__builtin_bit_cast(u16x2, m), r));
    }
    return max(max(m, max(w.x & 0x7FFFFFFFu, w.y & 0x7FFFFFFFu)), max(w.z & 0x7FFFFFFFu, w.w & 0x7FFFFFFFu));
}

// packed accumulator -> fp32 |x| bit pattern
template <bool BF16>
__device__ __forceinline__ uint32_t vmax_final(uint32_t m) {
    return BF16 ? max(m & 0xFFFFu, m >> 16) << 16 : m;
}

__device__ __forceinline__ void block1024_atomic_max(uint32_t m, uint32_t* out) {
    __shared__ uint32_t red[16];
    m = wave_max_u32(m);
    if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = m;
    __syncthreads();
    if (threadIdx.x < 64) {
        uint32_t v = threadIdx.x < 16 ? red[threadIdx.x] : 0u;
        v = wave_max_u32(v);
        if (threadIdx.x == 0) atomicMax(out, v);
    }
}

// Contiguous tensor as nv 16-byte vectors; each thread keeps kAmaxUnroll loads in flight.
template <bool BF16>
__global__ __launch_bounds__(kAmaxThreads) void amax_flat_kernel(const uint4* __restrict__ x, int64_t nv,
                                                                 uint32_t* __restrict__ out) {
    constexpr int U = kAmaxUnroll, T = kAmaxThreads;
    const int64_t stride = (int64_t)gridDim.x * T * U;
    uint32_t m = 0;
    for (int64_t b = (int64_t)blockIdx.x * T * U + threadIdx.x; b < nv; b += stride) {
        uint4 w[U];
        if (b + (int64_t)(U - 1) * T < nv) {
#pragma unroll
            for (int u = 0; u < U; ++u) w[u] = x[b + u * T];
        } else {
#pragma unroll
            for (int u = 0; u < U; ++u) w[u] = b + u * T < nv ? x[b + u * T] : make_uint4(0u, 0u, 0u, 0u);
        }
#pragma unroll
        for (int u = 0; u < U; ++u) m = vmax_acc<BF16>(m, w[u]);
    }
    block1024_atomic_max(vmax_final<BF16>(m), out);
}

// Strided rows (ld > cols): workgroups stride over rows, threads over the row's 16-byte vectors.
template <bool BF16>
__global__ __launch_bounds__(kAmaxThreads) void amax_rows_kernel(const void* __restrict__ x, int64_t rows, int64_t cols,
                                                                 int64_t ld, uint32_t* __restrict__ out) {
    const size_t esz = BF16 ? 2 : 4;
    const int64_t vpr = cols * (int64_t)esz / 16;      // cols % 8 == 0: whole vectors per row
    uint32_t m = 0;
    for (int64_t r = blockIdx.x; r < rows; r += gridDim.x) {
        const uint4* row = reinterpret_cast<const uint4*>(static_cast<const char*>(x) + r * ld * (int64_t)esz);
        for (int64_t v = threadIdx.x; v < vpr; v += kAmaxThreads) m = vmax_acc<BF16>(m, row[v]);
    }
    block1024_atomic_max(vmax_final<BF16>(m), out);
}

int launch_amax(const void* x, bool bf16, int64_t rows, int64_t cols, int64_t ld, float* amax_out,
                hipStream_t st) {
    uint32_t* out = reinterpret_cast<uint32_t*>(amax_out);
    hipLaunchKernelGGL(fill_u32_kernel, dim3(1), dim3(1), 0, st, out, 0u);
    if (rows == 0 || cols == 0) return 0;
    const size_t esz = bf16 ? 2 : 4;
    if (ld == cols) {
        const int64_t nv = rows * cols * (int64_t)esz / 16;
        int64_t blocks = (nv + kAmaxThreads * kAmaxUnroll - 1) / (kAmaxThreads * kAmaxUnroll);
        if (blocks > kAmaxBlocks) blocks = kAmaxBlocks;
        const uint4* xv = static_cast<const uint4*>(x);
        if (bf16) hipLaunchKernelGGL(amax_flat_kernel<true>, dim3((unsigned)blocks), dim3(kAmaxThreads), 0, st, xv, nv, out);
        else hipLaunchKernelGGL(amax_flat_kernel<false>, dim3((unsigned)blocks), dim3(kAmaxThreads), 0, st, xv, nv, out);
    } else {
        const int64_t blocks = rows < kAmaxBlocks ? rows : kAmaxBlocks;
        if (bf16) hipLaunchKernelGGL(amax_rows_kernel<true>, dim3((unsigned)blocks), dim3(kAmaxThreads), 0, st, x, rows, cols, ld, out);
        else hipLaunchKernelGGL(amax_rows_kernel<false>, dim3((unsigned)blocks), dim3(kAmaxThreads), 0, st, x, rows, cols, ld, out);
    }
    return 0;
}

int launch_zero_u32(float* p, hipStream_t st) {
    hipLaunchKernelGGL(fill_u32_kernel, dim3(1), dim3(1), 0, st, reinterpret_cast<uint32_t*>(p), 0u);
    return 0;
}

int launch_fill_f32(float* p, float v, hipStream_t st) {
    uint32_t bits;
    memcpy(&bits, &v, 4);
    hipLaunchKernelGGL(fill_u32_kernel, dim3(1), dim3(1), 0, st, reinterpret_cast<uint32_t*>(p), bits);
    return 0;
}

// Delayed-scaling state update ("Flax FP8 量化实战指南 ...", section 2.3): the window is rolled left
// by one (element i+1 moves to i, element 0 to the end) and the newest amax is written at index 0;
// then scale = fl(max(window) / MAX) unless that max is zero or non-finite (or the quotient
// underflows), in which case the previous scale is kept.  One workgroup; len <= 4096.
template <int FMT>
__global__ __launch_bounds__(1024) void history_kernel(float* __restrict__ hist, int len,
                                                       const float* __restrict__ amax_new,
                                                       float* __restrict__ scale) {
    __shared__ float buf[4096];
    __shared__ uint32_t red[16];
    const int t = threadIdx.x;
    for (int i = t; i < len; i += 1024) buf[i] = hist[i];
    __syncthreads();
    const float a = *amax_new;
    uint32_t m = 0;
    for (int i = t; i < len; i += 1024) {
        float v = (i == 0) ? a : (i == len - 1 ? buf[0] : buf[i + 1]);
        if (len == 1) v = a;
        hist[i] = v;
        m = max(m, absbits(v));
    }
    m = wave_max_u32(m);
    if ((t & 63) == 0) red[t >> 6] = m;
    __syncthreads();
    if (t == 0) {
        uint32_t b = 0;
        for (int w = 0; w < 16; ++w) b = max(b, red[w]);
        // history entries are amaxes (non-negative or NaN), so the max bit pattern is the max value
        float hmax = __uint_as_float(b);
        float s = *scale;
        *scale = scale_from_amax<FMT>(hmax, s);
    }
}

int launch_history(float* hist, int len, const float* amax_new, float* scale, int fmt, hipStream_t st) {
    if (fmt == kE4M3)
        hipLaunchKernelGGL(history_kernel<kE4M3>, dim3(1), dim3(1024), 0, st, hist, len, amax_new, scale);
    else
        hipLaunchKernelGGL(history_kernel<kE5M2>, dim3(1), dim3(1024), 0, st, hist, len, amax_new, scale);
    return 0;
}

}  // namespace fp8q
