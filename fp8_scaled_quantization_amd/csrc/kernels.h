// Internal launcher interface between the C ABI (capi.hip) and the kernel files.
// All launchers enqueue on `st` and return 0; argument validation happens in capi.hip.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fp8q {

constexpr int64_t kMaxReduceBlocks = 256;    // cap on workgroups that each end with one same-address atomic
constexpr int kModeTensor = 0, kModeBlock = 1, kModeMX = 2, kModeMoss = 3, kModeBlockE8 = 4;

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

// Per-tensor current scaling (TENSOR, scale derived) of a tensor of at most kSmallCastElems elements:
// amax, scale and cast in one single-workgroup launch; writes *amax_out and *scale_out.
constexpr int64_t kSmallCastElems = 16384;
int launch_cast_small_current(const CastArgs& a, hipStream_t st);

struct GemmArgs {
    int mode, afmt, bfmt;
    // BLOCK / BLOCK_E8M0 only: a_static = the activation operand has one per-tensor scale, *Aglobal
    // (Ascale unused); b_e8m0 = the 128x128 weight-block scales are E8M0 bytes (else fp32)
    bool a_static, b_e8m0;
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
// Sets the dynamic-LDS limit of every GEMM kernel on the current device (0 on success).
int prepare_gemm_kernels();

// Small state kernels and block dequantization (next.hip).
int launch_history_merge(float* hist_dst, const float* hist_src, int64_t len, float* scale_dst,
                         const float* scale_src, hipStream_t st);
int launch_auto_scale(float* state, int rescale, const float* amax_now, float lr, int fmt, float* scale_out,
                      hipStream_t st);
int launch_scale_to_e8m0(const float* s, int64_t n, uint8_t* e8m0, int32_t* bad_count, hipStream_t st);
struct DequantArgs {
    bool e8m0;                 // block scales are E8M0 bytes (else fp32)
    int fmt;
    const uint8_t* q;
    int64_t rows, cols, ldq;
    const void* scales;
    int block_r, block_c;
    void* out;
    bool out_bf16;
    int64_t ldo;
    bool vec;                  // 16-byte aligned rows (q, out) and cols % 16 == 0, block_c % 16 == 0
};
int launch_block_dequantize(const DequantArgs& a, hipStream_t st);

}  // namespace fp8q
