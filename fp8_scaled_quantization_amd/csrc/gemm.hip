// Scaled FP8 GEMM on gfx950 matrix cores: C = dequant(A) . dequant(B)^T, A: M x K, B: N x K, both
// K-contiguous FP8 bytes.
//
// Scale handling per scheme:
//   TENSOR  C = (sum qa*qb) * fl(s_a*s_b) in the epilogue (page "Flax FP8 量化实战指南 ...",
//           section 2.2: FP32-accumulated dot, dequantize by a_scale * b_scale);
//   BLOCK   each 128-wide K block's FP32 partial is multiplied by fl(sx[m][kb] * sw[n/128][kb]) and
//           accumulated in the main loop (page "Transformers 中的细粒度 FP8 量化配置 ...", section 一:
//           1x128 activation groups aligned with 128x128 weight blocks); sw may be an E8M0 power
//           of two (section 七) and sx one static per-tensor activation scale (section 四);
//   MX      the E8M0 scales of each 32-wide K group go into the block-scaled MFMA
//           (v_mfma_scale_f32_16x16x128_f8f6f4), so the main loop is matrix-core only (page "MOSS:
//           高效、精确的 FP8 LLM 训练 ...", sections 1 and 4);
//   MOSS    as MX, then fl(S_A*S_B) once in the epilogue (same page, section 4, step 4).
//
// This file holds the dispatch (launch_sel, at the end) to the kernels that run the schemes: the
// ping-pong kernels with 256 x 256 tiles for TENSOR/MX/MOSS with whole-K accumulation in the matrix
// core (gemm_pp.cuh: one tile per workgroup, or a persistent grid of one workgroup per CU when
// there are more tiles; gemm_pps.cuh: the persistent grid with a workgroup's tiles run as one
// stream of K steps, for bf16 output), the ping-pong kernel with 256 x 128 tiles (gemm_ppb.cuh:
// block scaling, and smaller TENSOR/MX/MOSS problems), the pipelined kernel for small problems
// (gemm_kernel.cuh), and the reference-tile kernel below for what those do not cover (K not a
// multiple of 128, operands past 32-bit offsets).
//
// Reference-tile kernel.  Accumulation: gfx950's FP8 MFMA adds its products (and its C input) with
// only ~12-15 bits kept below the largest term; this kernel computes each 128-wide K step by MFMAs
// starting from zero and adds it into a separate FP32 accumulator with VALU adds (a full-precision
// promotion every 128 K, which BLOCK needs anyway for its per-block scales).
//
// Tiling.  Block tile 128 x 128, K step 128 bytes, 256 threads = 4 waves in 2 x 2, wave tile
// 64 x 64 = 4 x 4 MFMA tiles of 16 x 16.  A and B K-tiles are double-buffered in LDS (64 KiB) with a
// 16-byte-chunk XOR swizzle (chunk ^ (row & 7)) so that both the coalesced global->LDS writes and
// the MFMA fragment reads are bank-conflict free.  MFMA operand layout for 16x16x128 (lane
// l = r + 16 g): bytes 0-15 hold A[r][16g .. 16g+15], bytes 16-31 hold A[r][64+16g .. 64+16g+15];
// the E8M0 scale of (row r, 32-group q) is taken from lane r + 16 q; C[4 (l/16) + i][l % 16] is
// element i of lane l.  Workgroups are remapped so that each XCD (one L2 each) works on a compact
// group of output tiles.
#include "common.cuh"
#include "gemm_kernel.cuh"
#include "gemm_pp.cuh"
#include "gemm_ppb.cuh"
#include "gemm_pps.cuh"
#include "kernels.h"

namespace fp8q {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v4f __attribute__((ext_vector_type(4)));

constexpr int BM = 128, BN = 128, BK = 128;
constexpr int kTileBytes = BM * BK;     // 16 KiB per operand tile

__device__ __forceinline__ int swz(int row, int chunk) { return row * BK + ((chunk ^ (row & 7)) << 4); }

__device__ __forceinline__ uint16_t f32_to_bf16_rne(float f) {
    uint32_t u = __float_as_uint(f);
    if ((u & 0x7FFFFFFFu) > 0x7F800000u) return (uint16_t)((u >> 16) | 0x40u);   // quiet NaN
    u += 0x7FFFu + ((u >> 16) & 1u);
    return (uint16_t)(u >> 16);
}

// Map the linear workgroup id to an output tile: first undo the round-robin XCD dispatch so that
// consecutive logical ids run on the same XCD, then walk tiles in groups of 8 tile-rows.
__device__ __forceinline__ void tile_coords(int64_t ntm, int64_t ntn, int64_t& tm, int64_t& tn) {
    int64_t nb = ntm * ntn;
    int64_t b = blockIdx.x;
    if (nb % 8 == 0) b = (b % 8) * (nb / 8) + b / 8;
    const int64_t GROUP_M = 8;
    int64_t per_group = GROUP_M * ntn;
    int64_t grp = b / per_group;
    int64_t first_m = grp * GROUP_M;
    int64_t gm = min(ntm - first_m, GROUP_M);
    int64_t in_grp = b - grp * per_group;
    tm = first_m + in_grp % gm;
    tn = in_grp / gm;
}

template <int MODE, int AFMT, int BFMT, bool OUT_BF16>
__global__ __launch_bounds__(256) void gemm_kernel(GemmArgs g) {
    extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
    uint8_t* sA = smem;                            // [2][BM*BK]
    uint8_t* sB = smem + 2 * kTileBytes;           // [2][BN*BK]
    uint32_t* sSa = reinterpret_cast<uint32_t*>(smem + 4 * kTileBytes);   // [2][BM] scale words
    uint32_t* sSb = sSa + 2 * BM;                                          // [2][BN]

    const int64_t M = g.M, N = g.N, K = g.K;
    const int64_t ntm = (M + BM - 1) / BM, ntn = (N + BN - 1) / BN;
    int64_t tm, tn;
    tile_coords(ntm, ntn, tm, tn);
    const int64_t m0 = tm * BM, n0 = tn * BN;
    const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
    const int wm = wave >> 1, wn = wave & 1;
    const int r16 = lane & 15, g4 = lane >> 4;
    const int64_t nk = (K + BK - 1) / BK;
    const int64_t ngroups = (K + 31) / 32;         // MX/MOSS scale row length
    const int64_t nkb = (K + 127) / 128;           // BLOCK scale row length

    // ---- global -> register prefetch of one K tile (4 chunks of A and 4 of B per thread)
    uint4 ra[4], rb[4];
    uint32_t rsa = 0, rsb = 0;
    auto load_tile = [&](int64_t kt) {
        const int64_t k0 = kt * BK;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int ch = t + 256 * i, row = ch >> 3, c = ch & 7;
            const int64_t k = k0 + c * 16;
            const bool kin = k < K;
            const int64_t ar = m0 + row, br = n0 + row;
            ra[i] = (kin && ar < M) ? *reinterpret_cast<const uint4*>(g.A + ar * g.lda + k) : make_uint4(0, 0, 0, 0);
            rb[i] = (kin && br < N) ? *reinterpret_cast<const uint4*>(g.B + br * g.ldb + k) : make_uint4(0, 0, 0, 0);
        }
        if (MODE == kModeMX || MODE == kModeMoss) {
            // scale bytes for groups 4kt .. 4kt+3 of one row; absent groups get E8M0 127 (= 1.0)
            const int row = t & 127;
            const bool isA = t < 128;
            const int64_t grow = (isA ? m0 : n0) + row;
            const int64_t lim = isA ? M : N;
            const uint8_t* sc = static_cast<const uint8_t*>(isA ? g.Ascale : g.Bscale);
            uint32_t w = 0;
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const int64_t grp = kt * 4 + q;
                uint32_t byte = (grow < lim && grp < ngroups) ? sc[grow * ngroups + grp] : 127u;
                w |= byte << (8 * q);
            }
            if (isA) rsa = w; else rsb = w;
        } else if (MODE == kModeBlock) {
            if (t < 128) {
                const int64_t grow = m0 + t;
                if (g.a_static) rsa = __float_as_uint(*g.Aglobal);
                else rsa = grow < M ? static_cast<const uint32_t*>(g.Ascale)[grow * nkb + kt] : 0u;
            }
        }
    };
    auto store_tile = [&](int buf) {
        uint8_t* a = sA + buf * kTileBytes;
        uint8_t* b = sB + buf * kTileBytes;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int ch = t + 256 * i, row = ch >> 3, c = ch & 7;
            *reinterpret_cast<uint4*>(a + swz(row, c)) = ra[i];
            *reinterpret_cast<uint4*>(b + swz(row, c)) = rb[i];
        }
        if (MODE == kModeMX || MODE == kModeMoss) {
            if (t < 128) sSa[buf * BM + t] = rsa; else sSb[buf * BN + (t - 128)] = rsb;
        } else if (MODE == kModeBlock) {
            if (t < 128) sSa[buf * BM + t] = rsa;
        }
    };

    v4f acc[4][4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = v4f{0.f, 0.f, 0.f, 0.f};

    if (nk > 0) {
        load_tile(0);
        store_tile(0);
    }
    __syncthreads();

    for (int64_t kt = 0; kt < nk; ++kt) {
        const int buf = kt & 1;
        if (kt + 1 < nk) load_tile(kt + 1);

        const uint8_t* a = sA + buf * kTileBytes;
        const uint8_t* b = sB + buf * kTileBytes;
        v8i fa[4], fb[4];
        int sca[4] = {0, 0, 0, 0}, scb[4] = {0, 0, 0, 0};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int ra_ = wm * 64 + i * 16 + r16;
            const int rb_ = wn * 64 + i * 16 + r16;
            uint4 lo = *reinterpret_cast<const uint4*>(a + swz(ra_, g4));
            uint4 hi = *reinterpret_cast<const uint4*>(a + swz(ra_, 4 + g4));
            fa[i] = v8i{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
            lo = *reinterpret_cast<const uint4*>(b + swz(rb_, g4));
            hi = *reinterpret_cast<const uint4*>(b + swz(rb_, 4 + g4));
            fb[i] = v8i{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
            if (MODE == kModeMX || MODE == kModeMoss) {
                // lane r16 + 16 q passes the scale of (row r16, group q), q = g4
                sca[i] = (int)((sSa[buf * BM + ra_] >> (8 * g4)) & 0xFFu);
                scb[i] = (int)((sSb[buf * BN + rb_] >> (8 * g4)) & 0xFFu);
            }
        }
        float rowscale[4][4];
        if (MODE == kModeBlock) {
            const int64_t nb = n0 / 128;
            const float sw = g.b_e8m0 ? __builtin_amdgcn_ldexpf(1.0f, (int)static_cast<const uint8_t*>(g.Bscale)[nb * nkb + kt] - 127)
                                      : static_cast<const float*>(g.Bscale)[nb * nkb + kt];
#pragma unroll
            for (int i = 0; i < 4; ++i)
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    rowscale[i][e] = __uint_as_float(sSa[buf * BM + wm * 64 + i * 16 + 4 * g4 + e]) * sw;
        }
        const v4f zero = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                v4f p;
                if (MODE == kModeMX || MODE == kModeMoss)
                    p = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(fa[i], fb[j], zero, AFMT, BFMT, 0, sca[i], 0, scb[j]);
                else
                    p = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(fa[i], fb[j], zero, AFMT, BFMT, 0, 0, 0, 0);
                if (MODE == kModeBlock) {
#pragma unroll
                    for (int e = 0; e < 4; ++e) acc[i][j][e] = __builtin_fmaf(rowscale[i][e], p[e], acc[i][j][e]);
                } else {
                    acc[i][j] += p;
                }
            }
        }
        if (kt + 1 < nk) {
            __syncthreads();               // everyone is done reading the buffer about to be refilled
            store_tile(buf ^ 1);
            __syncthreads();
        }
    }

    // ---- epilogue: global dequantisation factor, convert, store
    float f = 1.0f;
    if (MODE == kModeTensor || MODE == kModeMoss) f = (*g.Aglobal) * (*g.Bglobal);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int64_t col = n0 + wn * 64 + j * 16 + r16;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int64_t row = m0 + wm * 64 + i * 16 + 4 * g4 + e;
                if (row < M && col < N) {
                    const float v = (MODE == kModeTensor || MODE == kModeMoss) ? acc[i][j][e] * f : acc[i][j][e];
                    if (OUT_BF16) static_cast<uint16_t*>(g.C)[row * g.ldc + col] = f32_to_bf16_rne(v);
                    else static_cast<float*>(g.C)[row * g.ldc + col] = v;
                }
            }
        }
    }
}

constexpr size_t kGemmSmem = 4 * kTileBytes + 4 * 128 * sizeof(uint32_t);

template <int MODE, int AFMT, int BFMT, bool OUT>
static void launch_t(const GemmArgs& g, hipStream_t st) {
    const int64_t ntm = (g.M + BM - 1) / BM, ntn = (g.N + BN - 1) / BN;
    auto kern = gemm_kernel<MODE, AFMT, BFMT, OUT>;
    static bool attr_set = false;
    if (!attr_set) {
        (void)hipFuncSetAttribute(reinterpret_cast<const void*>(kern), hipFuncAttributeMaxDynamicSharedMemorySize, (int)kGemmSmem);
        attr_set = true;
    }
    hipLaunchKernelGGL(kern, dim3((unsigned)(ntm * ntn)), dim3(256), kGemmSmem, st, g);
}

// Pipelined kernels (gemm_kernel.cuh) for K % 128 == 0 and operands addressable with 32-bit
// buffer offsets; the reference-tile kernel above handles everything else (ragged K, huge operands).
template <int MODE, int AFMT, int BFMT, bool OUT, int BM_, int BN_, int WM, int WN, int S>
static void launch_v2(const GemmArgs& g, hipStream_t st) {
    const int64_t ntm = (g.M + BM_ - 1) / BM_, ntn = (g.N + BN_ - 1) / BN_;
    auto kern = g2::gemm_kernel<MODE, AFMT, BFMT, OUT, BM_, BN_, WM, WN, S>;
    constexpr size_t smem = g2::smem_bytes<MODE, BM_, BN_, S>();
    static bool attr_set = false;
    if (!attr_set) {
        (void)hipFuncSetAttribute(reinterpret_cast<const void*>(kern), hipFuncAttributeMaxDynamicSharedMemorySize, (int)smem);
        attr_set = true;
    }
    hipLaunchKernelGGL(kern, dim3((unsigned)(ntm * ntn)), dim3(64 * WM * WN), smem, st, g);
}

// Ping-pong kernel with 256 x 128 tiles (gemm_ppb.cuh): every BLOCK / BLOCK_E8M0 problem, and
// TENSOR/MX/MOSS problems too small for the 256 x 256 tiles.  K % 128 == 0.
template <int MODE, int AFMT, int BFMT, bool OUT, bool E8, bool AST>
static void launch_ppb_k(const GemmArgs& g, hipStream_t st) {
    const int64_t ntm = (g.M + ppb::BM - 1) / ppb::BM, ntn = (g.N + ppb::BN - 1) / ppb::BN;
    auto kern = ppb::gemm_ppb_kernel<MODE, AFMT, BFMT, OUT, E8, AST>;
    constexpr size_t smem = ppb::lds_bytes<MODE>();
    static bool attr_set = false;
    if (!attr_set) {
        (void)hipFuncSetAttribute(reinterpret_cast<const void*>(kern), hipFuncAttributeMaxDynamicSharedMemorySize, (int)smem);
        attr_set = true;
    }
    hipLaunchKernelGGL(kern, dim3((unsigned)(ntm * ntn)), dim3(512), smem, st, g);
}
template <int MODE, int AFMT, int BFMT, bool OUT>
static void launch_ppb(const GemmArgs& g, hipStream_t st) {
    if constexpr (MODE == kModeBlock) {
        if (g.b_e8m0) {
            if (g.a_static) launch_ppb_k<MODE, AFMT, BFMT, OUT, true, true>(g, st);
            else launch_ppb_k<MODE, AFMT, BFMT, OUT, true, false>(g, st);
        } else {
            if (g.a_static) launch_ppb_k<MODE, AFMT, BFMT, OUT, false, true>(g, st);
            else launch_ppb_k<MODE, AFMT, BFMT, OUT, false, false>(g, st);
        }
    } else {
        launch_ppb_k<MODE, AFMT, BFMT, OUT, false, false>(g, st);
    }
}

// Ping-pong kernel with 256 x 256 tiles (gemm_pp.cuh): TENSOR, MX and MOSS with K % 128 == 0.
// CUs of the current device, read once per device
static int64_t compute_units() {
    static int64_t cache[64] = {0};
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 0;
    if (cache[dev] == 0) {
        int n = 0;
        if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return 0;
        cache[dev] = n;
    }
    return cache[dev];
}

template <int MODE, int AFMT, int BFMT, bool OUT>
static void launch_pp(const GemmArgs& g, hipStream_t st) {
    const int64_t ntm = (g.M + pp::BM - 1) / pp::BM, ntn = (g.N + pp::BN - 1) / pp::BN;
    auto kern = pp::gemm_pp_kernel<MODE, AFMT, BFMT, OUT>;
    constexpr size_t smem = pp::lds_bytes<MODE>();
    static bool attr_set = false;
    if (!attr_set) {
        (void)hipFuncSetAttribute(reinterpret_cast<const void*>(kern), hipFuncAttributeMaxDynamicSharedMemorySize, (int)smem);
        attr_set = true;
    }
    // one workgroup per CU (the kernel's LDS and registers admit no second one), each looping over
    // tiles; a grid smaller than the tile count is a multiple of 8 so that every workgroup's tiles
    // stay on its XCD
    const int64_t ntiles = ntm * ntn;
    int64_t grid = compute_units();
    grid -= grid % 8;
    if (grid <= 0 || ntiles <= grid) grid = ntiles;
    const int64_t nk = g.K / pp::BK;
    if constexpr (OUT) {
        // workgroups with several tiles run them as one stream of K steps (gemm_pps.cuh)
        if (ntiles > grid && nk % 4 == 0 && nk >= pps::kMinSteps) {
            auto skern = pps::gemm_pps_kernel<MODE, AFMT, BFMT>;
            static bool sattr_set = false;
            if (!sattr_set) {
                (void)hipFuncSetAttribute(reinterpret_cast<const void*>(skern), hipFuncAttributeMaxDynamicSharedMemorySize,
                                          (int)smem);
                sattr_set = true;
            }
            hipLaunchKernelGGL(skern, dim3((unsigned)grid), dim3(512), smem, st, g);
            return;
        }
    }
    hipLaunchKernelGGL(kern, dim3((unsigned)grid), dim3(512), smem, st, g);
}

static bool fits_u32(int64_t bytes) { return bytes >= 0 && bytes < ((int64_t)1 << 32); }

// LDS stages of the pipelined kernel's tiles.  128 x 128 TENSOR tiles keep one more step's loads in
// flight (4 x 32 KiB; 2048 x 2048 x 4096 measured 30.3-31.1 us against 31.7-32.0 us with 3 stages);
// MX/MOSS keep the scale-quad schedule of 3 stages.  The 64 x 64 tiles keep 2 stages: at
// 1024 x 1024 x 2048 their 256 workgroups pull 64 MiB through L2 in ~9 us, and 6 stages made the
// call slower (10.2 us against 8.6 us per call in a replayed graph).
template <int MODE>
constexpr int small_stages() { return 2; }
template <int MODE>
constexpr int mid_stages() { return MODE == kModeTensor ? 4 : 3; }

template <int MODE, int AFMT, int BFMT, bool OUT>
static void launch_sel(const GemmArgs& g, hipStream_t st) {
    const bool fast = g.K > 0 && g.K % 128 == 0 && fits_u32(g.M * g.lda) && fits_u32(g.N * g.ldb) &&
                      fits_u32(g.M * (g.K / 32)) && fits_u32(g.N * (g.K / 32));
    if (!fast) {
        launch_t<MODE, AFMT, BFMT, OUT>(g, st);
        return;
    }
    if constexpr (MODE == kModeBlock) {
        // per-128 promotion with the block scales: the ping-pong kernel's 256 x 128 tiles
        launch_ppb<MODE, AFMT, BFMT, OUT>(g, st);
    } else {
        // whole-K accumulation on the matrix cores: the ping-pong kernel's 256 x 256 tiles when
        // there are enough of them to fill the GPU, else its 256 x 128 tiles, else the pipelined
        // kernel's 128 x 128 tiles, or 64 x 64 tiles when 128 x 128 ones would leave CUs idle
        // (1024 x 1024 x 2048: 8.8 us with 256 tiles of 64 x 64, 18 us with 64 of 128 x 128)
        const int64_t big_tiles = ((g.M + 255) / 256) * ((g.N + 255) / 256);
        const int64_t mid_tiles = ((g.M + 255) / 256) * ((g.N + 127) / 128);
        const int64_t small_tiles = ((g.M + 127) / 128) * ((g.N + 127) / 128);
        if (big_tiles >= 192) launch_pp<MODE, AFMT, BFMT, OUT>(g, st);
        else if (mid_tiles >= 192) launch_ppb<MODE, AFMT, BFMT, OUT>(g, st);
        else if (small_tiles >= 256) launch_v2<MODE, AFMT, BFMT, OUT, 128, 128, 2, 2, mid_stages<MODE>()>(g, st);
        else launch_v2<MODE, AFMT, BFMT, OUT, 64, 64, 2, 2, small_stages<MODE>()>(g, st);
    }
}

template <int MODE, int AFMT, int BFMT>
static void launch_out(const GemmArgs& g, hipStream_t st) {
    if (g.out_bf16) launch_sel<MODE, AFMT, BFMT, true>(g, st);
    else launch_sel<MODE, AFMT, BFMT, false>(g, st);
}

template <int MODE>
static void launch_fmt(const GemmArgs& g, hipStream_t st) {
    if (g.afmt == kE4M3 && g.bfmt == kE4M3) launch_out<MODE, 0, 0>(g, st);
    else if (g.afmt == kE5M2 && g.bfmt == kE4M3) launch_out<MODE, 1, 0>(g, st);
    else if (g.afmt == kE4M3 && g.bfmt == kE5M2) launch_out<MODE, 0, 1>(g, st);
    else launch_out<MODE, 1, 1>(g, st);
}

// The dynamic-LDS limit of every GEMM kernel the dispatcher can launch, set once per device by
// fp8q_init, so that no first launch has to set it (for example inside a stream capture).
template <class KERN>
static bool set_lds_limit(KERN kern, size_t bytes) {
    return hipFuncSetAttribute(reinterpret_cast<const void*>(kern), hipFuncAttributeMaxDynamicSharedMemorySize,
                               (int)bytes) == hipSuccess;
}
template <int MODE, int AF, int BF, bool OUT>
static bool prepare_combo() {
    bool ok = set_lds_limit(gemm_kernel<MODE, AF, BF, OUT>, kGemmSmem);
    if constexpr (MODE == kModeBlock) {
        ok &= set_lds_limit(ppb::gemm_ppb_kernel<MODE, AF, BF, OUT, false, false>, ppb::lds_bytes<MODE>());
        ok &= set_lds_limit(ppb::gemm_ppb_kernel<MODE, AF, BF, OUT, false, true>, ppb::lds_bytes<MODE>());
        ok &= set_lds_limit(ppb::gemm_ppb_kernel<MODE, AF, BF, OUT, true, false>, ppb::lds_bytes<MODE>());
        ok &= set_lds_limit(ppb::gemm_ppb_kernel<MODE, AF, BF, OUT, true, true>, ppb::lds_bytes<MODE>());
    } else {
        ok &= set_lds_limit(g2::gemm_kernel<MODE, AF, BF, OUT, 128, 128, 2, 2, mid_stages<MODE>()>,
                            g2::smem_bytes<MODE, 128, 128, mid_stages<MODE>()>());
        ok &= set_lds_limit(g2::gemm_kernel<MODE, AF, BF, OUT, 64, 64, 2, 2, small_stages<MODE>()>,
                            g2::smem_bytes<MODE, 64, 64, small_stages<MODE>()>());
        ok &= set_lds_limit(ppb::gemm_ppb_kernel<MODE, AF, BF, OUT, false, false>, ppb::lds_bytes<MODE>());
        ok &= set_lds_limit(pp::gemm_pp_kernel<MODE, AF, BF, OUT>, pp::lds_bytes<MODE>());
        if constexpr (OUT) ok &= set_lds_limit(pps::gemm_pps_kernel<MODE, AF, BF>, pp::lds_bytes<MODE>());
    }
    return ok;
}
template <int MODE, int AF, int BF>
static bool prepare_out() { return prepare_combo<MODE, AF, BF, false>() && prepare_combo<MODE, AF, BF, true>(); }
template <int MODE>
static bool prepare_mode() {
    return prepare_out<MODE, 0, 0>() && prepare_out<MODE, 1, 0>() && prepare_out<MODE, 0, 1>() && prepare_out<MODE, 1, 1>();
}
int prepare_gemm_kernels() {
    const bool ok = prepare_mode<kModeTensor>() && prepare_mode<kModeBlock>() && prepare_mode<kModeMX>() &&
                    prepare_mode<kModeMoss>();
    return ok ? 0 : -1;
}

int launch_gemm(const GemmArgs& g, hipStream_t st) {
    if (g.M == 0 || g.N == 0) return 0;
    switch (g.mode) {
        case kModeTensor: launch_fmt<kModeTensor>(g, st); break;
        case kModeBlock:
        case kModeBlockE8: launch_fmt<kModeBlock>(g, st); break;   // b_e8m0 / a_static select the scale kinds
        case kModeMX: launch_fmt<kModeMX>(g, st); break;
        default: launch_fmt<kModeMoss>(g, st); break;
    }
    return 0;
}

}  // namespace fp8q
