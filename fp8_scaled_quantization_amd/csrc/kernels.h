// Internal launcher interface between the C ABI (capi.hip) and the kernel files.
// All launchers enqueue on `st` and return 0; argument validation happens in capi.hip.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fp8q {

constexpr int64_t kMaxReduceBlocks = 256;    // cap on workgroups that each end with one same-address atomic
constexpr int kModeTensor = 0, kModeBlock = 1, kModeMX = 2, kModeMoss = 3;

int launch_amax(const void* x, bool bf16, int64_t rows, int64_t cols, int64_t ld, float* amax_out,
                hipStream_t st);
int launch_zero_u32(float* p, hipStream_t st);
int launch_fill_f32(float* p, float v, hipStream_t st);
int launch_history(float* hist, int len, const float* amax_new, float* scale, int fmt, hipStream_t st);

struct CastArgs {
    int mode, fmt;
    const void* x;
    bool bf16;
    int64_t rows, cols, ld;          // input x: rows x cols
    bool transpose;                  // output is cols x rows when set
    uint8_t* q;
    int64_t ldq;
    bool vec_out;                    // q rows are 16-byte aligned (vector stores allowed)
    void* scales;                    // BLOCK: float[]; MX/MOSS: uint8[]
    int block_r, block_c;            // BLOCK only
    const float* scale_in;           // TENSOR: scale to use; MOSS: global S to use
    const float* amax_in;            // TENSOR current / MOSS: tensor amax to derive the scale from
    float* scale_out;                // written by workgroup 0 when the scale is derived here
    float* amax_out;                 // fused amax (TENSOR with a given scale), may be null
    int tile_group;                  // transposed kernel: 128-row tile bands walked per column strip
    uint8_t* q2;                     // dual cast: the non-transposed copy (rows x cols), row stride ldq2,
    int64_t ldq2;                    //   with its E8M0 scales (MX, MOSS) in scales2 [rows][cols / 32];
    void* scales2;                   //   q / ldq / scales then hold the transposed copy
};

// Both copies of x in one pass (TENSOR, MX, MOSS; rows % 32 == 0, cols % 32 == 0, vector-aligned
// outputs): q2 gets the row-grouped copy, q the transposed one.
int launch_cast_dual(const CastArgs& a, hipStream_t st);

// Casts with the tensor scale (or S) either given (scale_in) or derived from amax_in.
int launch_cast(const CastArgs& a, hipStream_t st);

struct GemmArgs {
    int mode, afmt, bfmt;
    const uint8_t* A;
    const uint8_t* B;
    const void* Ascale;
    const void* Bscale;
    const float* Aglobal;
    const float* Bglobal;
    int64_t M, N, K, lda, ldb;
    void* C;
    bool out_bf16;
    int64_t ldc;
};
int launch_gemm(const GemmArgs& g, hipStream_t st);

}  // namespace fp8q
