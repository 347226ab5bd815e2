// Ping-pong scaled FP8 GEMM for gfx950 with 256 x 128 output tiles, 8 waves, two per SIMD: the
// kernel for problems whose 256 x 256 tiles would leave CUs idle, and for every block-scaled
// problem.  Per scheme:
//   BLOCK   the per-128-K promotion of the fine-grained scheme (page "Transformers 中的细粒度 FP8
//           量化配置 ...", section 一, and the COAT description on page "MOSS:高效、精确的 FP8 LLM
//           训练 ...", section 4):  acc[m][n] += fl(sx[m][kb] * sw[n / 128][kb]) * P_kb[m][n], where
//           P_kb is the matrix core's FP32 sum over the 128-wide K block kb, sx the activation's 1x128
//           scale (or one per-tensor scale for static activations), sw the 128x128 weight-block scale
//           (fp32, or an E8M0 byte).  A 128-column tile lies inside one weight block, so sw is one
//           value per K step for the whole tile;
//   TENSOR  whole-K accumulation in the MFMA, fl(s_a * s_b) in the epilogue (page "Flax FP8 量化实战
//           指南 ...", section 2.2);
//   MX/MOSS E8M0 scales per 32-wide K group applied by the MFMA; MOSS adds fl(S_A * S_B) in the
//           epilogue (MOSS page, sections 1 and 4).
//
// Schedule.  As in the 256 x 256 ping-pong kernel (gemm_pp.cuh): waves 0-3 (group 0) and 4-7
// (group 1) alternate a memory phase and a compute phase, group 1 one phase behind, so that on
// every SIMD one wave multiplies while the other moves data.  Wave (g, w) owns rows 64 w .. +64 and
// columns 64 g .. +64 of the tile: 16 MFMAs per K step.  Block scaling promotes each row block's
// partial sums while the MFMAs of the next row block run.  LDS holds three K stages (3 x 48 KiB) and
// a two-entry ring of scale quads (16 bytes per row = 4 K steps of fp32 row scales, or of four E8M0
// bytes).  In its memory phase for step k a wave reads its fragments and scales of step k, and sends
// its half of step k+2's copies (group 0: A rows 0-127 and B rows 0-63; group 1: the other halves)
// and, at a quad's first step, its share of the scale quad; stage (k+2) % 3 was last read in the
// memory phases for step k-1, which both ended before this phase.  It then waits for the copies it
// sent one memory phase earlier (step k+1), which gives every copy two phases to land.
#pragma once
#include "gemm_pp.cuh"

namespace fp8q {
namespace ppb {

using g2::make_rsrc;
using g2::rsrc_t;
using g2::v4f;
using g2::v8i;
using pp::barrier;
using pp::copy8;
using pp::frag;
using pp::wait_lgkm0;
using pp::wait_vm;
using pp::wait_vm0;

constexpr int BM = 256, BN = 128, BK = 128, STAGES = 3;
constexpr int kA = BM * BK, kB = BN * BK, kStage = kA + kB;   // 48 KiB per K step
constexpr int kScBase = STAGES * kStage;
// scale quad: A rows (and for MX/MOSS the B rows after them), 16 bytes per row
template <int MODE>
constexpr int quad_rows() { return MODE == kModeBlock ? BM : (MODE == kModeMX || MODE == kModeMoss) ? BM + BN : 0; }
template <int MODE>
constexpr size_t lds_bytes() { return (size_t)kScBase + 2 * (size_t)quad_rows<MODE>() * 16; }   // <= 156 KiB

// This wave's half of step s: group g, wave wi sends A rows 128 g + 32 wi .. +32 (4 copies) and
// B rows 64 g + 16 wi .. +16 (2 copies).  j selects one of the six.
// The data of step ks goes into the stage of step s (ks = s except past the last step, where the
// copies repeat the last step's data into a stage no step reads, which keeps the loop free of
// branches).
__device__ __forceinline__ void copy_one(uint32_t sbase, int s, int ks, int g, int wi, int j, rsrc_t ra, rsrc_t rb,
                                         uint32_t voffA, uint32_t voffB, uint32_t lda, uint32_t ldb) {
    const uint32_t st = sbase + (uint32_t)((s % STAGES) * kStage);
    const uint32_t koff = (uint32_t)ks * BK;
    if (j < 4) {
        const uint32_t r0 = (uint32_t)(128 * g + 32 * wi + 8 * j);
        copy8(st + r0 * BK, ra, voffA, r0 * lda, koff);
    } else {
        const uint32_t r0 = (uint32_t)(64 * g + 16 * wi + 8 * (j - 4));
        copy8(st + kA + r0 * BK, rb, voffB, r0 * ldb, koff);
    }
}

// One instruction of the scale quad of steps s .. s+3: quad rows r0 .. r0+64 (16 bytes each) from
// the scale array behind rs (rows of A from 0, rows of B from BM).  The K offset goes into the
// range-checked lane offset: the last quad of a row may end past the row (K steps not a multiple of
// 4), and past the array's end on its last row, where the buffer range turns the excess into zeros.
template <int MODE>
__device__ __forceinline__ void copy_quad(uint32_t sbase, int s, int r0, rsrc_t rs, uint32_t voffS, uint32_t sc_row) {
    const uint32_t sq = sbase + (uint32_t)(kScBase + ((s >> 2) & 1) * (quad_rows<MODE>() * 16));
    const uint32_t first = (uint32_t)(r0 < BM ? r0 : r0 - BM);
    copy8(sq + r0 * 16, rs, voffS + (uint32_t)s * 4, first * sc_row, 0u);
}
// The quad instructions of wave (g, wi): group 1 copies A rows 64 wi ..; for MX/MOSS waves 0 and 1
// of group 0 copy B rows 64 wi ...  Returns how many it issued.
template <int MODE>
__device__ __forceinline__ int wave_quads(int g, int wi) {
    if (MODE == kModeTensor) return 0;
    if (g == 1) return 1;
    return (MODE != kModeBlock && wi < 2) ? 1 : 0;
}
template <int MODE>
__device__ __forceinline__ void issue_quad(uint32_t sbase, int s, int g, int wi, rsrc_t rsa, rsrc_t rsb, uint32_t voffS,
                                           uint32_t sc_row) {
    if (MODE == kModeTensor) return;
    if (g == 1) copy_quad<MODE>(sbase, s, 64 * wi, rsa, voffS, sc_row);
    else if (MODE != kModeBlock && wi < 2) copy_quad<MODE>(sbase, s, BM + 64 * wi, rsb, voffS, sc_row);
}

// Raw 32-bit word holding a weight-block scale, through the scalar cache: the fp32 scale itself, or
// for E8M0 scales the aligned word holding the byte (decoded by block_scale_value).
template <bool E8>
__device__ __forceinline__ uint32_t block_scale_word(const void* base, int64_t i) {
    typedef __attribute__((address_space(4))) const uint32_t* cptr;
    const uint64_t a = reinterpret_cast<uint64_t>(base) + (uint64_t)(E8 ? i : 4 * i);
    const uint64_t u = (uint64_t)(uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)a) |
                       ((uint64_t)(uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)(a >> 32)) << 32);
    return *(cptr)(u & ~(uint64_t)3);
}
// The byte of an E8M0 scale sits at the low two bits of its own address within the aligned word
// (the scale array itself need not be 4-byte aligned).
template <bool E8>
__device__ __forceinline__ float block_scale_value(uint32_t w, const void* base, int64_t i) {
    if (E8) {
        const uint32_t sh = 8u * (uint32_t)((reinterpret_cast<uint64_t>(base) + (uint64_t)i) & 3u);
        return __builtin_amdgcn_ldexpf(1.0f, (int)((w >> sh) & 0xFFu) - 127);
    }
    return __uint_as_float(w);
}

// BLOCK only -- E8: the weight-block scales are E8M0 bytes (else fp32); AST: static activations (one
// per-tensor activation scale in Aglobal instead of the row scales).
template <int MODE, int AFMT, int BFMT, bool OUT_BF16, bool E8, bool AST>
__global__ __launch_bounds__(512, 1) void gemm_ppb_kernel(GemmArgs g) {
    constexpr bool BLOCKED = MODE == kModeBlock, SCALED = MODE == kModeMX || MODE == kModeMoss;
    constexpr bool RSC = BLOCKED && !AST;          // per-row activation scales in the quads
    constexpr int QB = quad_rows<MODE>() * 16;     // bytes of one scale quad
    extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
    const uint32_t sbase = g2::lds_addr(smem);    // LDS address of the dynamic allocation (copy targets)

    const int t = threadIdx.x, lane = t & 63;
    const int wave = __builtin_amdgcn_readfirstlane(t >> 6);
    const int grp = wave >> 2, wi = wave & 3;     // wave tile: rows 64 wi .. +64, cols 64 grp .. +64
    const int r16 = lane & 15, g4 = lane >> 4;
    const int64_t M = g.M, N = g.N;
    const int64_t ntm = (M + BM - 1) / BM, ntn = (N + BN - 1) / BN;

    // tile coordinates: undo the round-robin XCD dispatch, then walk groups of 8 tile-rows
    int64_t b = blockIdx.x;
    {
        const int64_t nb = ntm * ntn;
        if (nb % 8 == 0) b = (b % 8) * (nb / 8) + b / 8;
    }
    const int64_t per_group = 8 * ntn;
    const int64_t gi = b / per_group, first_m = gi * 8;
    const int64_t gm = min(ntm - first_m, (int64_t)8);
    const int64_t in_grp = b - gi * per_group;
    const int64_t m0 = (first_m + in_grp % gm) * BM, n0 = (in_grp / gm) * BN;
    const int nk = (int)(g.K / BK);

    // per-row scales: 4 bytes per K step (one fp32 block scale, or four E8M0 group scales)
    const uint32_t sc_row = (uint32_t)(4 * nk);
    const rsrc_t ra = make_rsrc(g.A + m0 * g.lda, (uint32_t)(max((int64_t)0, M - m0) * g.lda));
    const rsrc_t rb = make_rsrc(g.B + n0 * g.ldb, (uint32_t)(max((int64_t)0, N - n0) * g.ldb));
    // static activations: one tensor scale stands in for the row scales (whose copies then read an
    // empty range)
    const float s_static = AST ? g2::load_uniform_f32(g.Aglobal) : 0.0f;
    const rsrc_t rsa = make_rsrc(static_cast<const uint8_t*>(g.Ascale) + (RSC || SCALED ? m0 * (int64_t)sc_row : 0),
                                 RSC || SCALED ? (uint32_t)(max((int64_t)0, M - m0) * sc_row) : 0u);
    const rsrc_t rsb = make_rsrc(static_cast<const uint8_t*>(g.Bscale) + (SCALED ? n0 * (int64_t)sc_row : 0),
                                 SCALED ? (uint32_t)(max((int64_t)0, N - n0) * sc_row) : 0u);
    const int64_t wrow = (n0 / 128) * (int64_t)nk;  // BLOCK: this tile's row of weight-block scales
    // TENSOR / MOSS: the global factors, whose product scales the accumulators in the epilogue
    float ga = 1.0f, gb = 1.0f;
    if (MODE == kModeTensor || MODE == kModeMoss) {
        ga = g2::load_uniform_f32(g.Aglobal);
        gb = g2::load_uniform_f32(g.Bglobal);
    }

    const uint32_t ch = (uint32_t)(((lane & 7) ^ ((lane >> 3) & 7)) << 4);
    const uint32_t voffA = (uint32_t)((lane >> 3) * g.lda) + ch;
    const uint32_t voffB = (uint32_t)((lane >> 3) * g.ldb) + ch;
    const uint32_t voffS = (uint32_t)lane * sc_row;
    const uint32_t ulda = (uint32_t)g.lda, uldb = (uint32_t)g.ldb;

    const uint32_t cLo = (uint32_t)((g4 ^ (r16 & 7)) << 4), cHi = (uint32_t)(((4 + g4) ^ (r16 & 7)) << 4);
    const uint32_t rowA = (uint32_t)((wi * 64 + r16) * BK), rowB = (uint32_t)((grp * 64 + r16) * BK);
    // this lane's accumulator rows within the wave tile: 16 i + 4 g4 + e
    const int srow = wi * 64 + 4 * g4;

    v4f acc[4][4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = v4f{0.f, 0.f, 0.f, 0.f};

    // ---- prologue: both halves of steps 0 and 1, the first scale quad
#pragma unroll
    for (int j = 0; j < 6; ++j) copy_one(sbase, 0, 0, grp, wi, j, ra, rb, voffA, voffB, ulda, uldb);
    if (!(BLOCKED && AST)) issue_quad<MODE>(sbase, 0, grp, wi, rsa, rsb, voffS, sc_row);
    if (nk > 1) {
#pragma unroll
        for (int j = 0; j < 6; ++j) copy_one(sbase, 1, 1, grp, wi, j, ra, rb, voffA, voffB, ulda, uldb);
        wait_vm<6>();
    } else {
        wait_vm0();
    }
    barrier();
    if (grp == 1) barrier();                      // group 1 runs one phase behind

    // weight-block scale word of the current step; the next one is loaded at the end of each
    // compute phase and decoded in the next memory phase, so its latency is hidden
    uint32_t swraw = BLOCKED ? block_scale_word<E8>(g.Bscale, wrow) : 0u;
    for (int k = 0; k < nk; ++k) {
        // ---- memory phase for step k
        const int st = k % STAGES;
        const uint8_t* sa = smem + st * kStage;
        const uint8_t* sb = sa + kA;
        const bool cp = k + 2 < nk;
        const bool quad = !(BLOCKED && AST) && cp && ((k + 2) & 3) == 0 && wave_quads<MODE>(grp, wi) > 0;
        const uint8_t* sq = smem + kScBase + ((k >> 2) & 1) * QB;
        float sx[16];
        if (RSC) {
            const float* sqf = reinterpret_cast<const float*>(sq);
#pragma unroll
            for (int i = 0; i < 4; ++i)
#pragma unroll
                for (int e = 0; e < 4; ++e) sx[4 * i + e] = sqf[(srow + 16 * i + e) * 4 + (k & 3)];
        }
        // MX/MOSS: the E8M0 words of this lane's MFMA rows (A: row r16 of each row block; B: column
        // r16 of each column block); byte g4 is its 32-group's scale for this step
        uint32_t swa[4], swb[4];
        if (SCALED) {
            const uint32_t* sqw = reinterpret_cast<const uint32_t*>(sq);
#pragma unroll
            for (int i = 0; i < 4; ++i) swa[i] = sqw[(wi * 64 + i * 16 + r16) * 4 + (k & 3)];
#pragma unroll
            for (int j = 0; j < 4; ++j) swb[j] = sqw[(BM + grp * 64 + j * 16 + r16) * 4 + (k & 3)];
        }
        v8i fa[4], fb[4];
#pragma unroll
        for (int q = 0; q < 8; ++q) {
            if (q < 6) copy_one(sbase, k + 2, min(k + 2, nk - 1), grp, wi, q, ra, rb, voffA, voffB, ulda, uldb);
            if (q < 4) fa[q] = frag(sa + rowA + q * 16 * BK, cLo, cHi);
            else fb[q - 4] = frag(sb + rowB + (q - 4) * 16 * BK, cLo, cHi);
        }
        if (quad) issue_quad<MODE>(sbase, k + 2, grp, wi, rsa, rsb, voffS, sc_row);
        // BLOCK: the block-scale products of this step, fl(sx * sw)
        float rs[16];
        if (BLOCKED) {
            const float sw = block_scale_value<E8>(swraw, g.Bscale, wrow + k);
#pragma unroll
            for (int i = 0; i < 16; ++i) rs[i] = (AST ? s_static : sx[i]) * sw;
        }
        // MX/MOSS: four row blocks' scales per register, picked in the MFMA by its byte select
        int sca = 0, scb = 0;
        if (SCALED) {
            const uint32_t sel = pp::perm_selector(g4);
            sca = (int)pp::pack_scale_bytes(swa[0], swa[1], swa[2], swa[3], sel);
            scb = (int)pp::pack_scale_bytes(swb[0], swb[1], swb[2], swb[3], sel);
            asm volatile("" ::"v"(sca), "v"(scb));
        }
        // this wave's copies of step k+1 (sent one memory phase ago) land before the barrier; the
        // ones sent in this phase may stay in flight
        if (quad) wait_vm<7>();
        else wait_vm<6>();
        wait_lgkm0();
        barrier();
        // the next step's weight-scale word: nothing in the compute phase waits on it
        if (BLOCKED && k + 1 < nk) swraw = block_scale_word<E8>(g.Bscale, wrow + k + 1);
        if (BLOCKED) {
            // ---- compute phase: 16 MFMAs from zero; the promotion of row block i-1 (16 FMAs) is
            // interleaved with the MFMAs of row block i, so the VALU work runs while the matrix core
            // is busy instead of after it
            v4f pa[4], pb[4];
#pragma unroll
            for (int j = 0; j < 4; ++j)
                pa[j] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(fa[0], fb[j], v4f{0.f, 0.f, 0.f, 0.f}, AFMT, BFMT, 0,
                                                                         0, 0, 0);
#pragma unroll
            for (int i = 1; i <= 4; ++i) {
                v4f* const prev = (i & 1) ? pa : pb;
                v4f* const next = (i & 1) ? pb : pa;
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    // program order is kept (sched_barrier): MFMA (i, j), then the four FMAs of
                    // (i-1, j), whose partial sums were issued four MFMAs earlier
                    __builtin_amdgcn_sched_barrier(0);
                    if (i < 4)
                        next[j] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(fa[i], fb[j], v4f{0.f, 0.f, 0.f, 0.f},
                                                                                   AFMT, BFMT, 0, 0, 0, 0);
#pragma unroll
                    for (int e = 0; e < 4; ++e)
                        acc[i - 1][j][e] = __builtin_fmaf(rs[4 * (i - 1) + e], prev[j][e], acc[i - 1][j][e]);
                }
                __builtin_amdgcn_sched_barrier(0);
            }
        } else {
            // ---- compute phase: 16 MFMAs accumulating the whole K sum
#pragma unroll
            for (int i = 0; i < 4; ++i)
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    if (SCALED)
                        acc[i][j] = pp::mfma_sel<AFMT, BFMT>(fa[i], fb[j], acc[i][j], sca, scb, i, j);
                    else
                        acc[i][j] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(fa[i], fb[j], acc[i][j], AFMT, BFMT, 0,
                                                                                      0, 0, 0);
                }
        }
#pragma unroll
        for (int i = 0; i < 4; ++i)
            asm volatile("" ::"v"(acc[i][0]), "v"(acc[i][1]), "v"(acc[i][2]), "v"(acc[i][3]));
        barrier();
    }
    if (grp == 0) barrier();          // matches group 1's extra barrier at the start
    wait_vm0();                       // the last steps' repeated copies

    // ---- epilogue
    const float f = (MODE == kModeTensor || MODE == kModeMoss) ? ga * gb : 1.0f;
    if (OUT_BF16 && m0 + BM <= M && n0 + BN <= N) {
        // full tile: quad transposes and 8-byte stores (pp::quad_transpose_bf16)
        const int q = r16 & 3, c4 = r16 >> 2;
        const uint32_t modd = 0u - (uint32_t)(q & 1), mhi = 0u - (uint32_t)(q >> 1);
        uint16_t* const cw = static_cast<uint16_t*>(g.C) + (m0 + wi * 64) * g.ldc + n0 + grp * 64;
        const uint32_t loff = (uint32_t)((4 * g4 + q) * g.ldc + 4 * c4);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            uint16_t* const ci = cw + (int64_t)i * 16 * g.ldc;
#pragma unroll
            for (int j = 0; j < 4; ++j)
                *reinterpret_cast<uint2*>(ci + loff + j * 16) = pp::quad_transpose_bf16(acc[i][j] * f, modd, mhi);
        }
    } else {
        const int64_t row0 = m0 + wi * 64 + 4 * g4, col0 = n0 + grp * 64 + r16;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int64_t col = col0 + j * 16;
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int64_t row = row0 + i * 16 + e;
                    if (row < M && col < N) {
                        const float v = acc[i][j][e] * f;
                        if (OUT_BF16) static_cast<uint16_t*>(g.C)[row * g.ldc + col] = g2::f32_to_bf16_rne(v);
                        else static_cast<float*>(g.C)[row * g.ldc + col] = v;
                    }
                }
            }
        }
    }
}

}  // namespace ppb
}  // namespace fp8q
