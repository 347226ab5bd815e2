// Pipelined scaled FP8 GEMM kernel template for gfx950 (CDNA4): C = dequant(A) . dequant(B)^T.
//
// Scale handling per scheme (same arithmetic as the reference-tile kernel in gemm.hip):
//   TENSOR  C = (sum qa*qb) * fl(s_a*s_b) in the epilogue (page "Flax FP8 量化实战指南 ...",
//           section 2.2);
//   MX/MOSS E8M0 scales per 32-wide K group applied by v_mfma_scale_f32_16x16x128_f8f6f4; MOSS adds
//           fl(S_A*S_B) in the epilogue (page "MOSS:高效、精确的 FP8 LLM 训练 ...", sections 1, 4).
// Block scaling, which promotes every K step, has its own kernel (gemm_ppb.cuh).  The helpers
// below (descriptors, copies, waits, uniform loads) are shared with it and with gemm_pp.cuh.
//
// Data movement.  A and B K-tiles (128 bytes of K per row) go from HBM straight into LDS with
// buffer_load_dwordx4 ... lds: no VGPR staging, and rows past M or N read as zero through the
// buffer's range check.  STAGES LDS buffers form a ring: while stage k is being multiplied, the
// loads for stage k + STAGES - 1 are in flight.  Each 16-byte chunk c of tile row r is stored at
// chunk position c ^ (r & 7), so both the DMA writes (8 rows per wave instruction) and the MFMA
// fragment reads are bank-conflict free; the swizzle is applied by choosing which global chunk
// each lane fetches.  Per-row scales travel in 16-byte quads that cover four K steps (16 E8M0
// bytes), loaded every fourth step into a two-entry ring, so each wave
// instruction fetches four steps' worth of the 64 rows it touches.
//
// Accumulation.  The FP8 MFMA keeps only ~12-15 bits below the largest term it adds (its
// products and its C input).  TENSOR, MX and MOSS keep the whole K sum in the instruction's FP32
// accumulator, as the MOSS page's design keeps the main loop on the matrix cores.
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
typedef uint32_t rsrc_t __attribute__((ext_vector_type(4)));

constexpr int BK = 128;
constexpr int SQ = 4;                          // K steps per scale quad
constexpr uint32_t kRsrcWord3 = 0x00020000u;   // raw buffer, 32-bit format field (gfx9 family)

// Raw buffer descriptor: base address, stride 0, range in bytes (loads past it return zero).
__device__ __forceinline__ rsrc_t make_rsrc(const void* base, uint32_t bytes) {
    const uint64_t a = reinterpret_cast<uint64_t>(base);
    // the descriptor must live in scalar registers: every field is wave-uniform
    return rsrc_t{(uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)a),
                  (uint32_t)__builtin_amdgcn_readfirstlane((int)((uint32_t)(a >> 32) & 0xFFFFu)),
                  (uint32_t)__builtin_amdgcn_readfirstlane((int)bytes), kRsrcWord3};
}

// One wave instruction: lane i loads 16 bytes at rsrc + voff + soff into LDS address lds + 16 i.
// Issued as inline assembly so that the compiler does not treat the LDS ring as written by every
// outstanding load (it would otherwise drain all loads before each LDS read); completion is
// tracked explicitly with vmcnt waits before the workgroup barrier.
__device__ __forceinline__ void dma16(uint32_t lds, rsrc_t rsrc, uint32_t voff, uint32_t soff) {
    asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tbuffer_load_dwordx4 %1, %2, %3 offen lds"
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

// Read-only load of a wave-uniform value through the scalar cache (constant address space): it is
// tracked by lgkmcnt, so waiting for it does not also drain the LDS-bound buffer loads in flight.
__device__ __forceinline__ float load_uniform_f32(const float* p) {
    typedef __attribute__((address_space(4))) const float* cptr;
    const uint64_t a = reinterpret_cast<uint64_t>(p);
    const uint64_t u = (uint64_t)(uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)a) |
                       ((uint64_t)(uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)(a >> 32)) << 32);
    return *(cptr)u;
}

// Read-only load of the byte at p (wave-uniform address) through the scalar cache: the aligned
// 4-byte word holding it is fetched (an aligned word never crosses a page, so it is readable when
// the byte is) and the byte extracted.
__device__ __forceinline__ uint32_t load_uniform_u8(const uint8_t* p) {
    typedef __attribute__((address_space(4))) const uint32_t* cptr;
    const uint64_t a = reinterpret_cast<uint64_t>(p);
    const uint64_t u = (uint64_t)(uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)a) |
                       ((uint64_t)(uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)(a >> 32)) << 32);
    return (*(cptr)(u & ~(uint64_t)3) >> (8 * (uint32_t)(u & 3))) & 0xFFu;
}

// 128x128 weight-block scale of (n-block, k-block) index bi: fp32, or an E8M0 byte (2^(b - 127))
__device__ __forceinline__ float weight_block_scale(const GemmArgs& g, int64_t bi) {
    if (g.b_e8m0) return __builtin_amdgcn_ldexpf(1.0f, (int)load_uniform_u8(static_cast<const uint8_t*>(g.Bscale) + bi) - 127);
    return load_uniform_f32(static_cast<const float*>(g.Bscale) + bi);
}

// wait until at most N vector-memory operations of this wave are outstanding
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
    static_assert(N >= 0 && N < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((N & 0xF) | ((N >> 4) << 14) | (0x7 << 4) | (0xF << 8));
}

// Wait until at most r * PER vector-memory operations of this wave are outstanding, for a
// wave-uniform r in 0 .. R (the count must be an immediate, so each r has its own wait).
template <int PER, int R>
__device__ __forceinline__ void wait_steps(int r) {
    if constexpr (R == 0) {
        wait_vmcnt<0>();
    } else {
        if (r >= R) {
            wait_vmcnt<R * PER>();
            return;
        }
        wait_steps<PER, R - 1>(r);
    }
}

template <int MODE, int BM, int BN, int STAGES>
struct Layout {
    static constexpr bool SCALED = MODE == kModeMX || MODE == kModeMoss;
    static constexpr int kA = BM * BK, kB = BN * BK, kStage = kA + kB;
    static constexpr int kScRows = SCALED ? BM + BN : 0;
    static constexpr int kScQuad = kScRows * 16;              // one scale quad (4 K steps)
    static constexpr int kScBase = STAGES * kStage;
    static constexpr int kBytes = kScBase + 2 * kScQuad;
};

// Issue the loads of K step kt into stage buffer kt % STAGES, plus the scale quad every SQ steps.
// (A device function rather than a lambda: the host-side pass of the compiler does not emit kernels
// whose lambdas capture arrays by reference.)
template <int MODE, int BM, int BN, int STAGES, int NW, int A_LD, int B_LD, int SC_LD_TOTAL>
__device__ __forceinline__ void issue_step(uint8_t* smem, int64_t kt, int wave, int lane, rsrc_t ra, rsrc_t rb,
                                           rsrc_t rsa, rsrc_t rsb, const uint32_t* offA, const uint32_t* offB,
                                           int64_t sc_row) {
    using L = Layout<MODE, BM, BN, STAGES>;
    uint8_t* st = smem + (kt % STAGES) * L::kStage;
    const uint32_t koff = (uint32_t)(kt * BK);
#pragma unroll
    for (int j = 0; j < A_LD; ++j) dma16(lds_addr(st + (wave * A_LD + j) * 8 * BK), ra, offA[j], koff);
#pragma unroll
    for (int j = 0; j < B_LD; ++j) dma16(lds_addr(st + L::kA + (wave * B_LD + j) * 8 * BK), rb, offB[j], koff);
    if (L::kScRows > 0 && kt % SQ == 0) {
        uint8_t* sq = smem + L::kScBase + ((kt / SQ) & 1) * L::kScQuad;
        // 4 scale bytes per K step.  The K offset goes into the range-checked lane offset: with K
        // steps not a multiple of 4 the last quad of a row ends past the row, and on the array's
        // last row past its end, where the buffer range turns the excess into zeros.
        const uint32_t kq = (uint32_t)(kt * 4);
#pragma unroll
        for (int j = 0; j < SC_LD_TOTAL; ++j) {
            if (wave == j % NW) {
                const bool isA = j * 64 < BM;
                const int rowb = isA ? j * 64 : j * 64 - BM;
                const uint32_t off = (uint32_t)((rowb + lane) * sc_row) + kq;
                uint8_t* dst = sq + (isA ? 0 : BM * 16) + rowb * 16;
                if (isA) dma16(lds_addr(dst), rsa, off, 0u);
                else dma16(lds_addr(dst), rsb, off, 0u);
            }
        }
    }
}

template <int MODE, int AFMT, int BFMT, bool OUT_BF16, int BM, int BN, int WAVES_M, int WAVES_N, int STAGES>
__global__ __launch_bounds__(64 * WAVES_M * WAVES_N) void gemm_kernel(GemmArgs g) {
    constexpr int NW = WAVES_M * WAVES_N;
    constexpr int WTM = BM / WAVES_M, WTN = BN / WAVES_N;
    constexpr int TM = WTM / 16, TN = WTN / 16;
    using L = Layout<MODE, BM, BN, STAGES>;
    constexpr bool SCALED = L::SCALED;
    static_assert(MODE == kModeTensor || SCALED, "block scaling has its own kernel (gemm_ppb.cuh)");
    // 16-byte chunk loads per stage: (BM + BN) rows x 8 chunks; one wave instruction = 8 rows
    constexpr int A_LD = BM / 8 / NW, B_LD = BN / 8 / NW;
    static_assert(BM % (8 * NW) == 0 && BN % (8 * NW) == 0, "tile/wave split");
    constexpr int SC_LD_TOTAL = L::kScRows / 64;                 // scale-quad instructions (64 rows each)
    static_assert(L::kScRows % 64 == 0, "scale rows per wave instruction");
    constexpr int LD_LO = A_LD + B_LD;                           // per stage without scales
    constexpr int SC_LO = SC_LD_TOTAL / NW;                      // scale instructions of every wave
    // TENSOR takes deeper rings (no scale quads, so every step carries the same instruction count)
    static_assert(STAGES >= 2 && STAGES <= (SCALED ? 3 : 8), "stage count");
    static_assert(LD_LO + SC_LO + 1 < 64 && LD_LO * (STAGES - 2) < 64, "vmcnt range");

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

    // ---- buffer descriptors (ranges end at the last row, so rows >= M / N read zero)
    const rsrc_t ra = make_rsrc(g.A + m0 * g.lda, (uint32_t)(max((int64_t)0, M - m0) * g.lda));
    const rsrc_t rb = make_rsrc(g.B + n0 * g.ldb, (uint32_t)(max((int64_t)0, N - n0) * g.ldb));
    // per-row scale bytes: one E8M0 per 32-group, 4 bytes per K step
    const int64_t sc_row = 4 * nk;
    const uint8_t* sca_base = static_cast<const uint8_t*>(g.Ascale);
    const uint8_t* scb_base = static_cast<const uint8_t*>(g.Bscale);
    uint32_t sca_bytes = 0, scb_bytes = 0;
    if (SCALED) {
        sca_base += m0 * sc_row;
        sca_bytes = (uint32_t)(max((int64_t)0, M - m0) * sc_row);
        scb_base += n0 * sc_row;
        scb_bytes = (uint32_t)(max((int64_t)0, N - n0) * sc_row);
    }
    const rsrc_t rsa = make_rsrc(sca_base, sca_bytes);
    const rsrc_t rsb = make_rsrc(scb_base, scb_bytes);

    // ---- per-lane global byte offsets of this wave's chunks (the K offset is added per stage):
    // lane i of a load covers tile row base + i/8 at LDS chunk position i%8, fetching global chunk
    // (i%8) ^ (row & 7) of that row.
    uint32_t offA[A_LD], offB[B_LD];
#pragma unroll
    for (int j = 0; j < A_LD; ++j) {
        const int row = (wave * A_LD + j) * 8 + (lane >> 3);
        offA[j] = (uint32_t)(row * g.lda) + (uint32_t)(((lane & 7) ^ (row & 7)) << 4);
    }
#pragma unroll
    for (int j = 0; j < B_LD; ++j) {
        const int row = (wave * B_LD + j) * 8 + (lane >> 3);
        offB[j] = (uint32_t)(row * g.ldb) + (uint32_t)(((lane & 7) ^ (row & 7)) << 4);
    }
    // scale-quad instructions: instruction j covers scale rows [64 j, 64 j + 64) (A rows first);
    // wave j % NW issues it
    const bool extra_sc = (SC_LD_TOTAL % NW) > wave;

    // ---- per-lane LDS read offsets (loop invariant)
    uint32_t rdA[TM], rdB[TN];
#pragma unroll
    for (int i = 0; i < TM; ++i) rdA[i] = (uint32_t)((wm * WTM + i * 16 + r16) * BK);
#pragma unroll
    for (int j = 0; j < TN; ++j) rdB[j] = (uint32_t)((wn * WTN + j * 16 + r16) * BK);
    const uint32_t cLo = (uint32_t)((g4 ^ (r16 & 7)) << 4), cHi = (uint32_t)(((4 + g4) ^ (r16 & 7)) << 4);

    v4f acc[TM][TN];
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j) acc[i][j] = v4f{0.f, 0.f, 0.f, 0.f};

    // ---- prologue: steps 0 .. STAGES-2 in flight
#pragma unroll
    for (int s = 0; s < STAGES - 1; ++s)
        if (s < nk) issue_step<MODE, BM, BN, STAGES, NW, A_LD, B_LD, SC_LD_TOTAL>(smem, s, wave, lane, ra, rb, rsa, rsb, offA,
                                                                               offB, sc_row);

    for (int64_t kt = 0; kt < nk; ++kt) {
        // step kt has landed once only the later steps' loads (at most STAGES-2 of them) remain
        if (!SCALED) {
            wait_steps<LD_LO, STAGES - 2>((int)min((int64_t)(STAGES - 2), nk - 1 - kt));
        } else if (STAGES == 3 && kt + 1 < nk) {
            // one later step in flight: its instruction count depends on whether it carries scales
            if (L::kScRows > 0 && (kt + 1) % SQ == 0) {
                if (extra_sc) wait_vmcnt<LD_LO + SC_LO + 1>();
                else wait_vmcnt<LD_LO + SC_LO>();
            } else {
                wait_vmcnt<LD_LO>();
            }
        } else {
            wait_vmcnt<0>();
        }
        barrier_nofence();
        if (kt + STAGES - 1 < nk)
            issue_step<MODE, BM, BN, STAGES, NW, A_LD, B_LD, SC_LD_TOTAL>(smem, kt + STAGES - 1, wave, lane, ra, rb, rsa, rsb,
                                                                          offA, offB, sc_row);

        const uint8_t* sa = smem + (kt % STAGES) * L::kStage;
        const uint8_t* sb = sa + L::kA;
        const uint8_t* sq = smem + L::kScBase + ((kt / SQ) & 1) * L::kScQuad;
        const int qs = (int)(kt % SQ);          // which K step of the scale quad
        const uint32_t* sqA = reinterpret_cast<const uint32_t*>(sq);
        const uint32_t* sqB = reinterpret_cast<const uint32_t*>(sq + BM * 16);

        v8i fb[TN];
        int scb[TN];
#pragma unroll
        for (int j = 0; j < TN; ++j) {
            const uint4 lo = *reinterpret_cast<const uint4*>(sb + rdB[j] + cLo);
            const uint4 hi = *reinterpret_cast<const uint4*>(sb + rdB[j] + cHi);
            fb[j] = v8i{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
            scb[j] = 0;
            if (SCALED) scb[j] = (int)((sqB[(wn * WTN + j * 16 + r16) * 4 + qs] >> (8 * g4)) & 0xFFu);
        }

        // A fragments: the next subtile's reads are issued before this subtile's MFMAs
        v8i fa_next;
        int sca_next = 0;
        {
            const uint4 lo = *reinterpret_cast<const uint4*>(sa + rdA[0] + cLo);
            const uint4 hi = *reinterpret_cast<const uint4*>(sa + rdA[0] + cHi);
            fa_next = v8i{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
            if (SCALED) sca_next = (int)((sqA[(wm * WTM + r16) * 4 + qs] >> (8 * g4)) & 0xFFu);
        }
#pragma unroll
        for (int i = 0; i < TM; ++i) {
            const v8i fa = fa_next;
            const int sca = sca_next;
            if (i + 1 < TM) {
                const uint4 lo = *reinterpret_cast<const uint4*>(sa + rdA[i + 1] + cLo);
                const uint4 hi = *reinterpret_cast<const uint4*>(sa + rdA[i + 1] + cHi);
                fa_next = v8i{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
                if (SCALED) sca_next = (int)((sqA[(wm * WTM + (i + 1) * 16 + r16) * 4 + qs] >> (8 * g4)) & 0xFFu);
            }
#pragma unroll
            for (int j = 0; j < TN; ++j) {
                if (SCALED)
                    acc[i][j] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(fa, fb[j], acc[i][j], AFMT, BFMT, 0, sca, 0,
                                                                                  scb[j]);
                else
                    acc[i][j] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(fa, fb[j], acc[i][j], AFMT, BFMT, 0, 0, 0, 0);
            }
        }
    }

    // ---- epilogue
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

template <int MODE, int BM, int BN, int STAGES>
constexpr size_t smem_bytes() { return (size_t)Layout<MODE, BM, BN, STAGES>::kBytes; }

}  // namespace g2
}  // namespace fp8q
