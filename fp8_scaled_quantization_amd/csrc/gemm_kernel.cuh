// Pipelined scaled FP8 GEMM kernel template for gfx950 (CDNA4): C = dequant(A) . dequant(B)^T.
//
// Scale handling per scheme (same arithmetic as the reference-tile kernel in gemm.hip):
//   TENSOR  C = (sum qa*qb) * fl(s_a*s_b) in the epilogue (page "Flax FP8 量化实战指南 ...",
//           section 2.2);
//   BLOCK   each 128-wide K block's FP32 partial is scaled by fl(sx[m][kb] * sw[n/128][kb]) and
//           accumulated in the main loop (page "Transformers 中的细粒度 FP8 量化配置 ...", section 一);
//   MX/MOSS E8M0 scales per 32-wide K group applied by v_mfma_scale_f32_16x16x128_f8f6f4; MOSS adds
//           fl(S_A*S_B) in the epilogue (page "MOSS:高效、精确的 FP8 LLM 训练 ...", sections 1, 4).
//
// Data movement.  A and B K-tiles (128 bytes of K per row) go from HBM straight into LDS with
// buffer_load_dwordx4 ... lds: no VGPR staging, and rows past M or N read as zero through the
// buffer's range check.  STAGES LDS buffers form a ring: while stage k is being multiplied, the
// loads for stage k + STAGES - 1 are in flight.  Each 16-byte chunk c of tile row r is stored at
// chunk position c ^ (r & 7), so both the DMA writes (8 rows per wave instruction) and the MFMA
// fragment reads are bank-conflict free; the swizzle is applied by choosing which global chunk
// each lane fetches.  Per-row scale words (4 E8M0 bytes or one fp32 per row and K step) travel
// the same way.
//
// Accumulation.  The FP8 MFMA keeps only ~12-15 bits below the largest term it adds (its
// products and its C input), so a long chain through one accumulator loses accuracy as the
// accumulator grows.  Partial products are chained through the MFMA for R consecutive 128-wide
// K steps (the accumulator input stays comparable to the products) and then added into a
// separate FP32 accumulator with VALU adds; BLOCK uses R = 1 because its scale changes every
// 128 K.
//
// MFMA operand layout for 16x16x128 (lane l = r + 16 g): bytes 0-15 hold A[r][16g .. 16g+15],
// bytes 16-31 hold A[r][64+16g .. 64+16g+15]; the E8M0 scale of (row r, 32-group q) is taken from
// lane r + 16 q; C[4 (l/16) + i][l % 16] is element i of lane l.
#pragma once
#include "common.cuh"
#include "kernels.h"

namespace fp8q {
namespace g2 {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) void* lds_ptr_t;

constexpr int BK = 128;
constexpr uint32_t kRsrcWord3 = 0x00020000u;   // raw buffer, 32-bit format field (gfx9 family)

typedef uint32_t rsrc_t __attribute__((ext_vector_type(4)));

// Raw buffer descriptor: base address, stride 0, range in bytes (loads past it return zero).
__device__ __forceinline__ rsrc_t make_rsrc(const void* base, uint32_t bytes) {
    const uint64_t a = reinterpret_cast<uint64_t>(base);
    // the descriptor must live in scalar registers: every field is wave-uniform
    return rsrc_t{(uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)a),
                  (uint32_t)__builtin_amdgcn_readfirstlane((int)((uint32_t)(a >> 32) & 0xFFFFu)),
                  (uint32_t)__builtin_amdgcn_readfirstlane((int)bytes), kRsrcWord3};
}

// One wave instruction: lane i loads 16 (or 4) bytes at rsrc + voff + soff into LDS address
// lds + 16 i (or 4 i).  Issued as inline assembly so that the compiler does not treat the LDS ring
// as written by every outstanding load (it would otherwise drain all loads before each LDS read);
// completion is tracked explicitly with vmcnt waits before the workgroup barrier.
__device__ __forceinline__ void dma16(uint32_t lds, rsrc_t rsrc, uint32_t voff, uint32_t soff) {
    asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tbuffer_load_dwordx4 %1, %2, %3 offen lds"
                 :: "s"(lds), "v"(voff), "s"(rsrc), "s"(__builtin_amdgcn_readfirstlane(soff)) : "memory", "m0");
}
__device__ __forceinline__ void dma4(uint32_t lds, rsrc_t rsrc, uint32_t voff, uint32_t soff) {
    asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tbuffer_load_dword %1, %2, %3 offen lds"
                 :: "s"(lds), "v"(voff), "s"(rsrc), "s"(__builtin_amdgcn_readfirstlane(soff)) : "memory", "m0");
}
// Workgroup barrier without the release fence of __syncthreads (whose vmcnt(0) would also wait for
// the loads still in flight for later stages); LDS visibility of a stage is established by each
// wave's vmcnt wait before it arrives here.
__device__ __forceinline__ void barrier_nofence() { asm volatile("s_barrier" ::: "memory"); }

__device__ __forceinline__ uint32_t lds_addr(const void* p) {
    return __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)(lds_ptr_t)p);
}

__device__ __forceinline__ uint16_t f32_to_bf16_rne(float f) {
    uint32_t u = __float_as_uint(f);
    if ((u & 0x7FFFFFFFu) > 0x7F800000u) return (uint16_t)((u >> 16) | 0x40u);
    u += 0x7FFFu + ((u >> 16) & 1u);
    return (uint16_t)(u >> 16);
}

// wait until at most n vector-memory operations of this wave are outstanding
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
    static_assert(N >= 0 && N < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((N & 0xF) | ((N >> 4) << 14) | (0x7 << 4) | (0xF << 8));
}

template <int BM, int BN>
struct Smem {
    static constexpr int kA = BM * BK, kB = BN * BK;
    static constexpr int kScale = (BM + BN) * 4;
    static constexpr int kStage = kA + kB + kScale;
};

template <int MODE, int BM, int BN, int NW, int A_LDS_PER_WAVE, int B_LDS_PER_WAVE, int SC_A_LDS, int SC_B_LDS>
__device__ __forceinline__ void issue_stage(uint8_t* smem, int64_t kt, int buf, int wave, int lane,
                                            rsrc_t ra, rsrc_t rb, rsrc_t rsa, rsrc_t rsb,
                                            const uint32_t* offA, const uint32_t* offB, int64_t ngroups, int64_t nkb) {
    using S = Smem<BM, BN>;
    constexpr bool SCALED = MODE == kModeMX || MODE == kModeMoss;

        uint8_t* st = smem + buf * S::kStage;
        const uint32_t koff = (uint32_t)(kt * BK);
#pragma unroll
        for (int j = 0; j < A_LDS_PER_WAVE; ++j) {
            uint8_t* dst = st + (wave * A_LDS_PER_WAVE + j) * 8 * BK;
            dma16(lds_addr(dst), ra, offA[j], koff);
        }
#pragma unroll
        for (int j = 0; j < B_LDS_PER_WAVE; ++j) {
            uint8_t* dst = st + S::kA + (wave * B_LDS_PER_WAVE + j) * 8 * BK;
            dma16(lds_addr(dst), rb, offB[j], koff);
        }
        // scale words: one dword per tile row, 64 rows per wave instruction (waves 0.. take turns)
        uint8_t* sc = st + S::kA + S::kB;
        if (SCALED) {
#pragma unroll
            for (int j = 0; j < SC_A_LDS + SC_B_LDS; ++j) {
                if (wave == j % NW) {
                    const bool isA = j < SC_A_LDS;
                    const int rowb = (isA ? j : j - SC_A_LDS) * 64;
                    uint8_t* dst = sc + (isA ? 0 : BM * 4) + rowb * 4;
                    const uint32_t off = (uint32_t)((rowb + lane) * ngroups);
                    // (two calls rather than a conditional expression over the resource type,
                    // which the host-side pass of the compiler does not instantiate)
                    if (isA) dma4(lds_addr(dst), rsa, off, (uint32_t)(kt * 4));
                    else dma4(lds_addr(dst), rsb, off, (uint32_t)(kt * 4));
                }
            }
        } else if (MODE == kModeBlock) {
#pragma unroll
            for (int j = 0; j < SC_A_LDS; ++j) {
                if (wave == j % NW) {
                    uint8_t* dst = sc + j * 64 * 4;
                    const uint32_t off = (uint32_t)((j * 64 + lane) * nkb * 4);
                    dma4(lds_addr(dst), rsa, off, (uint32_t)(kt * 4));
                }
            }
        }
    }

template <int MODE, int AFMT, int BFMT, bool OUT_BF16, int BM, int BN, int WAVES_M, int WAVES_N, int R, int STAGES>
__global__ __launch_bounds__(64 * WAVES_M * WAVES_N) void gemm_kernel(GemmArgs g) {
    constexpr int NT = 64 * WAVES_M * WAVES_N;
    constexpr int NW = WAVES_M * WAVES_N;
    constexpr int WTM = BM / WAVES_M, WTN = BN / WAVES_N;
    constexpr int TM = WTM / 16, TN = WTN / 16;
    constexpr bool SCALED = MODE == kModeMX || MODE == kModeMoss;
    // R == 0: no promotion, the MFMA's FP32 accumulator runs over the whole K (pages' design for
    // per-tensor, MX and MOSS scaling); R >= 1: promote every R K steps (BLOCK always promotes).
    constexpr bool FULL_CHAIN = MODE != kModeBlock && R == 0;
    constexpr int RR = MODE == kModeBlock ? 1 : (R == 0 ? 1 : R);
    static_assert(MODE != kModeBlock || BN == 128, "block-scaled B tiles must match the 128-row weight blocks");
    // 16-byte chunk loads per stage: (BM + BN) rows x 8 chunks; one wave instruction = 8 rows
    constexpr int ROWS_PER_WAVE_LD = 8;
    constexpr int A_LDS_PER_WAVE = BM / ROWS_PER_WAVE_LD / NW;   // loads of A per wave per stage
    constexpr int B_LDS_PER_WAVE = BN / ROWS_PER_WAVE_LD / NW;
    static_assert(BM % (ROWS_PER_WAVE_LD * NW) == 0 && BN % (ROWS_PER_WAVE_LD * NW) == 0, "tile/wave split");
    static_assert(BM % 64 == 0 && BN % 64 == 0, "scale-word loads cover 64 rows per wave instruction");
    constexpr int SC_A_LDS = (MODE == kModeTensor) ? 0 : (BM + 63) / 64;   // scale-word loads (64 rows each)
    constexpr int SC_B_LDS = SCALED ? (BN + 63) / 64 : 0;
    using S = Smem<BM, BN>;

    extern __shared__ __attribute__((aligned(16))) uint8_t smem[];

    const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
    const int wm = wave / WAVES_N, wn = wave % WAVES_N;
    const int r16 = lane & 15, g4 = lane >> 4;
    const int64_t M = g.M, N = g.N, K = g.K;
    const int64_t ntm = (M + BM - 1) / BM, ntn = (N + BN - 1) / BN;

    // ---- tile coordinates: undo the round-robin XCD dispatch, then group 8 tile-rows
    int64_t b = blockIdx.x;
    {
        const int64_t nb = ntm * ntn;
        if (nb % 8 == 0) b = (b % 8) * (nb / 8) + b / 8;
    }
    const int64_t per_group = 8 * ntn;
    const int64_t grp = b / per_group, first_m = grp * 8;
    const int64_t gm = min(ntm - first_m, (int64_t)8);
    const int64_t in_grp = b - grp * per_group;
    const int64_t m0 = (first_m + in_grp % gm) * BM, n0 = (in_grp / gm) * BN;

    const int64_t nk = K / BK;
    const int64_t ngroups = K / 32, nkb = K / 128;

    // ---- buffer resources (byte ranges end at the last row, so rows >= M / N read zero)
    const rsrc_t ra = make_rsrc(g.A + m0 * g.lda, (uint32_t)(max((int64_t)0, M - m0) * g.lda));
    const rsrc_t rb = make_rsrc(g.B + n0 * g.ldb, (uint32_t)(max((int64_t)0, N - n0) * g.ldb));
    // scale words: MX/MOSS one E8M0 byte per 32-group (4 per K step), BLOCK one fp32 per K step
    const uint8_t* sca_base = static_cast<const uint8_t*>(g.Ascale);
    const uint8_t* scb_base = static_cast<const uint8_t*>(g.Bscale);
    uint32_t sca_bytes = 0, scb_bytes = 0;
    if (SCALED) {
        sca_base += m0 * ngroups;
        sca_bytes = (uint32_t)(max((int64_t)0, M - m0) * ngroups);
        scb_base += n0 * ngroups;
        scb_bytes = (uint32_t)(max((int64_t)0, N - n0) * ngroups);
    } else if (MODE == kModeBlock) {
        sca_base += m0 * nkb * 4;
        sca_bytes = (uint32_t)(max((int64_t)0, M - m0) * nkb * 4);
    }
    const rsrc_t rsa = make_rsrc(sca_base, sca_bytes);
    const rsrc_t rsb = make_rsrc(scb_base, scb_bytes);

    // ---- per-lane global byte offsets of this wave's chunks (K offset added per stage)
    // lane i of a load covers tile row rbase + i/8 at LDS chunk position i%8, fetching global chunk
    // (i%8) ^ (row & 7) of that row.
    uint32_t offA[A_LDS_PER_WAVE], offB[B_LDS_PER_WAVE];
#pragma unroll
    for (int j = 0; j < A_LDS_PER_WAVE; ++j) {
        const int row = (wave * A_LDS_PER_WAVE + j) * 8 + (lane >> 3);
        offA[j] = (uint32_t)(row * g.lda) + (uint32_t)((((lane & 7) ^ (row & 7))) << 4);
    }
#pragma unroll
    for (int j = 0; j < B_LDS_PER_WAVE; ++j) {
        const int row = (wave * B_LDS_PER_WAVE + j) * 8 + (lane >> 3);
        offB[j] = (uint32_t)(row * g.ldb) + (uint32_t)((((lane & 7) ^ (row & 7))) << 4);
    }


    // vector-memory instructions each wave issues per stage (for the vmcnt wait): the scale-word
    // loads are dealt round-robin, so waves below SC_TOTAL % NW issue one more
    constexpr int SC_TOTAL = SC_A_LDS + SC_B_LDS;
    constexpr int LD_LO = A_LDS_PER_WAVE + B_LDS_PER_WAVE + SC_TOTAL / NW;
    constexpr int LD_HI = LD_LO + (SC_TOTAL % NW ? 1 : 0);
    const bool extra_sc = wave < SC_TOTAL % NW;
    static_assert((STAGES - 2) * LD_HI < 64, "vmcnt range");

    v4f acc[TM][TN], P[TM][TN];
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j) {
            acc[i][j] = v4f{0.f, 0.f, 0.f, 0.f};
            P[i][j] = v4f{0.f, 0.f, 0.f, 0.f};
        }

    // ---- prologue: stages 0 .. STAGES-2 in flight
#pragma unroll
    for (int s = 0; s < STAGES - 1; ++s) {
        if (s < nk) issue_stage<MODE, BM, BN, NW, A_LDS_PER_WAVE, B_LDS_PER_WAVE, SC_A_LDS, SC_B_LDS>(smem, s, s, wave, lane, ra, rb, rsa, rsb, offA, offB, ngroups, nkb);
    }

    // K loop in chains of RR steps (nk % RR == 0, checked by the host): inside a chain the MFMA
    // result is fed back as its C input; at the chain's end it is added into the FP32 accumulator.
    for (int64_t kc = 0; kc < nk; kc += RR) {
#pragma unroll
        for (int rr = 0; rr < RR; ++rr) {
            const int64_t kt = kc + rr;
            const int buf = (int)(kt % STAGES);
            // stage kt has landed once at most (STAGES-2) later stages are outstanding
            if (kt + STAGES - 2 < nk) {
                if (extra_sc) wait_vmcnt<(STAGES - 2) * LD_HI>();
                else wait_vmcnt<(STAGES - 2) * LD_LO>();
            } else {
                wait_vmcnt<0>();
            }
            barrier_nofence();
            if (kt + STAGES - 1 < nk)
                issue_stage<MODE, BM, BN, NW, A_LDS_PER_WAVE, B_LDS_PER_WAVE, SC_A_LDS, SC_B_LDS>(
                    smem, kt + STAGES - 1, (int)((kt + STAGES - 1) % STAGES), wave, lane, ra, rb, rsa, rsb, offA, offB, ngroups, nkb);

            const uint8_t* sa = smem + buf * S::kStage;
            const uint8_t* sb = sa + S::kA;
            const uint32_t* scw = reinterpret_cast<const uint32_t*>(sb + S::kB);

            v8i fb[TN];
            int scb[TN];
#pragma unroll
            for (int j = 0; j < TN; ++j) {
                const int row = wn * WTN + j * 16 + r16;
                const uint8_t* p = sb + row * BK;
                uint4 lo = *reinterpret_cast<const uint4*>(p + ((g4 ^ (row & 7)) << 4));
                uint4 hi = *reinterpret_cast<const uint4*>(p + (((4 + g4) ^ (row & 7)) << 4));
                fb[j] = v8i{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
                scb[j] = 0;
                if (SCALED) scb[j] = (int)((scw[BM + row] >> (8 * g4)) & 0xFFu);
            }
            float sw = 1.0f;
            float rsv[TM][4];
            if (MODE == kModeBlock) sw = static_cast<const float*>(g.Bscale)[(n0 / 128) * nkb + kt];
#pragma unroll
            for (int i = 0; i < TM; ++i) {
                const int row = wm * WTM + i * 16 + r16;
                const uint8_t* p = sa + row * BK;
                uint4 lo = *reinterpret_cast<const uint4*>(p + ((g4 ^ (row & 7)) << 4));
                uint4 hi = *reinterpret_cast<const uint4*>(p + (((4 + g4) ^ (row & 7)) << 4));
                const v8i fa = v8i{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
                int sca = 0;
                if (SCALED) sca = (int)((scw[row] >> (8 * g4)) & 0xFFu);
                float rs[4] = {1.f, 1.f, 1.f, 1.f};
                if (MODE == kModeBlock) {
#pragma unroll
                    for (int e = 0; e < 4; ++e)
                        rs[e] = __uint_as_float(scw[wm * WTM + i * 16 + 4 * g4 + e]) * sw;
                }
#pragma unroll
                for (int j = 0; j < TN; ++j) {
                    const v4f cin = (rr == 0 && !FULL_CHAIN) ? v4f{0.f, 0.f, 0.f, 0.f} : P[i][j];
                    if (SCALED)
                        P[i][j] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(fa, fb[j], cin, AFMT, BFMT, 0, sca, 0, scb[j]);
                    else
                        P[i][j] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(fa, fb[j], cin, AFMT, BFMT, 0, 0, 0, 0);
                }
                if (MODE == kModeBlock) {
#pragma unroll
                    for (int e = 0; e < 4; ++e) rsv[i][e] = rs[e];
                }
            }
            // promotion into the FP32 accumulators, after every MFMA of the step was issued
            if (MODE == kModeBlock) {
#pragma unroll
                for (int i = 0; i < TM; ++i)
#pragma unroll
                    for (int j = 0; j < TN; ++j)
#pragma unroll
                        for (int e = 0; e < 4; ++e) acc[i][j][e] = __builtin_fmaf(rsv[i][e], P[i][j][e], acc[i][j][e]);
            } else if (!FULL_CHAIN && rr == RR - 1) {
#pragma unroll
                for (int i = 0; i < TM; ++i)
#pragma unroll
                    for (int j = 0; j < TN; ++j) acc[i][j] += P[i][j];
            }
        }
    }

    // ---- epilogue
    if (FULL_CHAIN) {
#pragma unroll
        for (int i = 0; i < TM; ++i)
#pragma unroll
            for (int j = 0; j < TN; ++j) acc[i][j] = P[i][j];
    }
    float f = 1.0f;
    if (MODE == kModeTensor || MODE == kModeMoss) f = (*g.Aglobal) * (*g.Bglobal);
#pragma unroll
    for (int i = 0; i < TM; ++i) {
#pragma unroll
        for (int j = 0; j < TN; ++j) {
            const int64_t col = n0 + wn * WTN + j * 16 + r16;
            if (col >= N) continue;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int64_t row = m0 + wm * WTM + i * 16 + 4 * g4 + e;
                if (row < M) {
                    const float v = (MODE == kModeTensor || MODE == kModeMoss) ? acc[i][j][e] * f : acc[i][j][e];
                    if (OUT_BF16) static_cast<uint16_t*>(g.C)[row * g.ldc + col] = f32_to_bf16_rne(v);
                    else static_cast<float*>(g.C)[row * g.ldc + col] = v;
                }
            }
        }
    }
}

template <int BM, int BN, int STAGES>
constexpr size_t smem_bytes() { return (size_t)STAGES * Smem<BM, BN>::kStage; }

}  // namespace g2
}  // namespace fp8q
