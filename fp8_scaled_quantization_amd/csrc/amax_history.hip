// amax reduction and delayed-scaling history update kernels.
//
// amax = max |x| ("Flax FP8 量化实战指南 ...", section 1).  The reduction runs on the sign-cleared
// fp32 bit patterns as unsigned integers: for non-negative floats integer order is numeric order and
// every NaN pattern sorts above +Inf, so the result is exact, NaN-propagating and independent of the
// order in which workgroups finish.  Each workgroup reduces in registers and LDS and issues one
// global atomic max.
#include "common.cuh"
#include "kernels.h"

#include <string.h>

namespace fp8q {

__global__ void fill_u32_kernel(uint32_t* p, uint32_t v) { *p = v; }

// Grid-stride amax over rows x cols (leading dimension ld).  Each thread handles 8 consecutive
// elements per step; cols % 8 == 0 and 16-byte aligned rows are guaranteed by the host.
template <bool BF16>
__global__ __launch_bounds__(256) void amax_kernel(const void* __restrict__ x, int64_t rows, int64_t cols,
                                                   int64_t ld, uint32_t* __restrict__ out) {
    const int64_t chunks_per_row = cols / 8;
    const int64_t total = rows * chunks_per_row;
    const size_t esz = BF16 ? 2 : 4;
    uint32_t m = 0;
    for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < total; i += (int64_t)gridDim.x * 256) {
        int64_t r = i / chunks_per_row, c = (i - r * chunks_per_row) * 8;
        float v[8];
        load8<BF16>(static_cast<const char*>(x) + (r * ld + c) * esz, v);
#pragma unroll
        for (int j = 0; j < 8; ++j) m = max(m, absbits(v[j]));
    }
    m = wave_max_u32(m);
    __shared__ uint32_t red[4];
    if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = m;
    __syncthreads();
    if (threadIdx.x == 0) {
        uint32_t b = max(max(red[0], red[1]), max(red[2], red[3]));
        atomicMax(out, b);
    }
}

int launch_amax(const void* x, bool bf16, int64_t rows, int64_t cols, int64_t ld, float* amax_out,
                hipStream_t st) {
    hipLaunchKernelGGL(fill_u32_kernel, dim3(1), dim3(1), 0, st, reinterpret_cast<uint32_t*>(amax_out), 0u);
    int64_t total = rows * (cols / 8);
    if (total == 0) return 0;
    int64_t blocks = (total + 255) / 256;
    if (blocks > kMaxReduceBlocks) blocks = kMaxReduceBlocks;
    if (bf16)
        hipLaunchKernelGGL(amax_kernel<true>, dim3((unsigned)blocks), dim3(256), 0, st, x, rows, cols, ld,
                           reinterpret_cast<uint32_t*>(amax_out));
    else
        hipLaunchKernelGGL(amax_kernel<false>, dim3((unsigned)blocks), dim3(256), 0, st, x, rows, cols, ld,
                           reinterpret_cast<uint32_t*>(amax_out));
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
