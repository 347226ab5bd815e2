// Streaming persistent variant of the 256 x 256 ping-pong scaled FP8 GEMM (gemm_pp.cuh) for gfx950:
// the schedule of gemm_pp_kernel, with a workgroup's tiles run as one continuous stream of K steps.
//
// Same schemes as gemm_pp.cuh (TENSOR: fl(s_a*s_b) in the epilogue, page "Flax FP8 量化实战指南 ...",
// section 2.2; MX: E8M0 scales per 32-wide K group in v_mfma_scale_f32_16x16x128_f8f6f4, page
// "MOSS:高效、精确的 FP8 LLM 训练 ...", section 1; MOSS: as MX plus fl(S_A*S_B) in the epilogue,
// same page, section 4), bf16 output only.  It serves problems with more tiles than CUs (so that
// each workgroup loops over several tiles) and K steps nk with nk % 4 == 0 and nk >= kMinSteps.
//
// What differs from gemm_pp_kernel is what happens between two tiles of one workgroup:
//  * Look-ahead copies.  The copies of "step k+1" and "step k+2" that the last two K steps of a
//    tile issue carry the next tile's steps 0 and 1 (its lane offsets and K offsets 0, 1), and the
//    scale quad that would cover steps nk..nk+3 is the next tile's first quad.  Every wait and
//    barrier then works exactly as within a tile: the stream never drains, and no fill has to be
//    waited for at a tile start.  (The scale-quad ring entry runs on with a per-workgroup quad
//    counter, so the next tile's first quad never lands in the entry the last steps still read.)
//  * Stores behind the stream.  A tile's epilogue stores go out after the look-ahead copies of the
//    next tile's first steps, so the next tile's first waits allow them (32 per wave) to stay in
//    flight; vector-memory operations complete in issue order, so the second step's waits, which
//    target copies sent after the stores, hold until they have drained.  (Keeping the outputs in
//    registers and spreading their stores over later steps would need 64 registers per wave more
//    than the 256 two waves per SIMD leave.)
//  * No re-synchronisation.  Group 1 stays one phase behind group 0 across tiles, so a group's
//    tile-end work (scaling, packing) overlaps the other group's MFMAs.
// Partial tiles (at the right or bottom edge) are stored element by element, and those stores all
// complete before the next tile's counted waits, as in gemm_pp_kernel.
#pragma once
#include "gemm_pp.cuh"

namespace fp8q {
namespace pps {

using g2::rsrc_t;
using g2::v4f;
using g2::v8i;
using pp::barrier;
using pp::copy8;
using pp::fresh;
using pp::frag;
using pp::kargs_t;
using pp::kernel_args;
using pp::wait_lgkm0;
using pp::wait_vm;
using pp::wait_vm0;

constexpr int BM = pp::BM, BN = pp::BN, BK = pp::BK;
constexpr int kA = pp::kA, kStage = pp::kStage, kScBase = pp::kScBase, kScQuad = pp::kScQuad;
constexpr int kStores = 32;     // epilogue stores per wave of a full tile
constexpr int kMinSteps = 8;    // fewest K steps the stream schedule is used for

// At most n vector-memory operations of this wave outstanding, n one of the counts the schedule
// forms (a wave-uniform value, so the switch is a scalar branch); any other n waits for all.
__device__ __forceinline__ void wait_vm_n(int n) {
    switch (n) {
        case 8: wait_vm<8>(); break;
        case 10: wait_vm<10>(); break;
        case 12: wait_vm<12>(); break;
        case 14: wait_vm<14>(); break;
        case 16: wait_vm<16>(); break;
        case 18: wait_vm<18>(); break;
        case 40: wait_vm<40>(); break;
        case 42: wait_vm<42>(); break;
        default: wait_vm0(); break;
    }
}

// Group 1, wave wi: two instructions of the scale quad that covers four K steps starting at step
// kst of the operand rows behind voffS, into ring entry `entry`.
__device__ __forceinline__ void copy_quad(uint32_t sbase, int entry, int kst, int wi, rsrc_t rsa, rsrc_t rsb,
                                          uint32_t voffS, uint32_t sc_row) {
    const uint32_t sq = sbase + kScBase + (uint32_t)entry * kScQuad;
    const uint32_t voff = voffS + (uint32_t)kst * 4;
#pragma unroll
    for (int j = 0; j < 2; ++j) {
        const int inst = wi * 2 + j;              // 0..3: A rows, 4..7: B rows, 64 rows each
        const uint32_t r0 = (uint32_t)(inst & 3) * 64;
        copy8(sq + inst * 64 * 16, inst < 4 ? rsa : rsb, voff, r0 * sc_row, 0u);
    }
}

template <int MODE, int AFMT, int BFMT>
__global__ __launch_bounds__(512, 1) void gemm_pps_kernel(GemmArgs g) {
    constexpr bool SCALED = MODE == kModeMX || MODE == kModeMoss;
    static_assert(MODE != kModeBlock, "block scaling promotes per K step; it has its own kernel");
    extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
    typedef __attribute__((address_space(1))) uint16_t gu16;
    typedef __attribute__((address_space(1))) uint64_t gu64;

    const int t = threadIdx.x, lane = t & 63;
    const int wave = fresh(__builtin_amdgcn_readfirstlane(t >> 6));
    const int grp = wave >> 2;
    const int wm = wave & 3, wn = grp;            // wave tile: rows 64 wm .. +64, cols 128 wn .. +128
    const int r16 = lane & 15, g4 = lane >> 4;
    const int64_t M = g.M, N = g.N;
    const uint32_t ntm_ = (uint32_t)((M + BM - 1) / BM), ntn_ = (uint32_t)((N + BN - 1) / BN);
    const uint32_t ntiles = ntm_ * ntn_;
    // tile coordinates as in gemm_pp_kernel (XCD-compact groups of 8 tile-rows; workgroup w takes
    // tiles w, w + G, ..., G a multiple of 8)
    auto coords = [&](uint32_t tile, uint32_t& m0_, uint32_t& n0_) {
        kargs_t* gk = kernel_args();
        const uint32_t ntm = (uint32_t)((gk->M + BM - 1) / BM), ntn = (uint32_t)((gk->N + BN - 1) / BN);
        const uint32_t nt = ntm * ntn;
        uint32_t b = tile;
        if (nt % 8 == 0) b = (b % 8) * (nt / 8) + b / 8;
        const uint32_t per_group = 8 * ntn;
        const uint32_t gi = b / per_group, first_m = gi * 8;
        const uint32_t gm = min(ntm - first_m, 8u);
        const uint32_t in_grp = b - gi * per_group;
        m0_ = (uint32_t)__builtin_amdgcn_readfirstlane((int)((first_m + in_grp % gm) * BM));
        n0_ = (uint32_t)__builtin_amdgcn_readfirstlane((int)((in_grp / gm) * BN));
    };
    const int nk = (int)(g.K / BK);              // the launcher admits nk % 4 == 0, nk >= kMinSteps

    const int64_t sc_row = 4 * (int64_t)nk;
    const rsrc_t ra = g2::make_rsrc(g.A, (uint32_t)(M * g.lda));
    const rsrc_t rb = g2::make_rsrc(g.B, (uint32_t)(N * g.ldb));
    rsrc_t rsa = rsrc_t{0u, 0u, 0u, 0u}, rsb = rsrc_t{0u, 0u, 0u, 0u};
    if (SCALED) {
        rsa = g2::make_rsrc(g.Ascale, (uint32_t)(M * sc_row));
        rsb = g2::make_rsrc(g.Bscale, (uint32_t)(N * sc_row));
    }
    const uint32_t ch = (uint32_t)(((lane & 7) ^ ((lane >> 3) & 7)) << 4);
    const uint32_t ulda = (uint32_t)g.lda, uldb = (uint32_t)g.ldb, usc = (uint32_t)sc_row;
    const int wi = wave & 3;
    const uint32_t sbase = g2::lds_addr(smem);
    const uint32_t cLo = (uint32_t)((g4 ^ (r16 & 7)) << 4), cHi = (uint32_t)(((4 + g4) ^ (r16 & 7)) << 4);
    const uint32_t rowA = (uint32_t)((wm * 64 + r16) * BK), rowB = (uint32_t)((wn * 128 + r16) * BK);

    uint32_t tile = blockIdx.x, m0, n0;
    coords(tile, m0, n0);
    uint32_t voffA = (uint32_t)(lane >> 3) * ulda + ch + m0 * ulda;
    uint32_t voffB = (uint32_t)(lane >> 3) * uldb + ch + n0 * uldb;
    uint32_t voffS = (uint32_t)lane * usc + (wi < 2 ? m0 : n0) * usc;

    // ---- the stream's start: group 0 sends B1 of step 0 (it sends B0 and B1 of step k+1 in its
    // memory phase for step k); group 1 sends A and B0 of step 0, the first scale quad and A of
    // step 1, and waits for all but A of step 1
    if (grp == 0) {
        pp::copy_B(sbase, 0, 0, 128, wi, rb, voffB, uldb);
    } else {
        pp::copy_A(sbase, 0, 0, wi, ra, voffA, ulda);
        pp::copy_B(sbase, 0, 0, 0, wi, rb, voffB, uldb);
        if (SCALED) copy_quad(sbase, 0, 0, wi, rsa, rsb, voffS, usc);
        pp::copy_A(sbase, 1, 1, wi, ra, voffA, ulda);
        wait_vm<8>();
    }
    barrier();

    v8i fa[4], fb[8];
    v4f acc[4][8];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 8; ++j) acc[i][j] = v4f{0.f, 0.f, 0.f, 0.f};
    if (grp == 1) {
        // group 1 reads A of step 0 while group 0 has its first memory phase, and stays one phase
        // behind from here on
#pragma unroll
        for (int i = 0; i < 4; ++i) fa[i] = frag(smem + rowA + i * 16 * BK, cLo, cHi);
        barrier();
    }

    bool behind = false;           // the last tile's kStores stores are still queued behind the look-ahead
    int qb = 0;                    // ring entry of this tile's scale quad j: (qb + j) & 1

    for (;;) {
        const uint32_t tile_n = tile + fresh(gridDim.x);
        const bool more = tile_n < ntiles;
        uint32_t m0n = m0, n0n = n0;
        if (more) coords(tile_n, m0n, n0n);
        // the next tile's lane offsets (its steps 0 and 1 are steps nk and nk+1 of the stream) differ
        // from this tile's by wave-uniform amounts, kept in scalar registers
        const uint32_t dA = (uint32_t)__builtin_amdgcn_readfirstlane((int)((m0n - m0) * ulda));
        const uint32_t dB = (uint32_t)__builtin_amdgcn_readfirstlane((int)((n0n - n0) * uldb));
        const uint32_t dS = (uint32_t)__builtin_amdgcn_readfirstlane((int)((wi < 2 ? m0n - m0 : n0n - n0) * usc));

        int sca = 0, scb0 = 0, scb1 = 0;
        for (int k = 0; k < nk; ++k) {
            // in step 0 the copies waited for were sent before the last tile's stores
            const int st0 = (behind && k == 0) ? kStores : 0;
            const uint32_t sk = fresh(sbase + (k & 1) * kStage), sk1 = fresh(sbase + ((k + 1) & 1) * kStage);
            uint32_t sw[12];
            if (SCALED) {
                const uint32_t* sq =
                    reinterpret_cast<const uint32_t*>(smem + kScBase + ((qb + (k >> 2)) & 1) * kScQuad);
                const int qs = k & 3;
#pragma unroll
                for (int i = 0; i < 4; ++i) sw[i] = sq[(wm * 64 + i * 16 + r16) * 4 + qs];
#pragma unroll
                for (int j = 0; j < 8; ++j) sw[4 + j] = sq[(BM + wn * 128 + j * 16 + r16) * 4 + qs];
            }
            {
                const uint8_t* sa = smem + (k & 1) * kStage;
                const uint8_t* sb = sa + kA;
                if (grp == 0) {
                    // B0, then B1, of stream step k+1 (8 copies, one per fragment read): this
                    // tile's step, or after the last step the next tile's step 0 (past the last
                    // tile: the last step again, into a stage no step reads).  Both regions of that
                    // stage were last read one and two phases ago.
                    const int s = k + 1;
                    const uint32_t vB = voffB + ((s >= nk && more) ? dB : 0u);
                    const uint32_t koff = (uint32_t)(s < nk ? s : (more ? s - nk : nk - 1)) * BK;
                    uint32_t l = sk1 + kA + (uint32_t)(wi * 32) * BK, ro = (uint32_t)(wi * 32) * uldb;
#pragma unroll
                    for (int q = 0; q < 12; ++q) {
                        if (q < 8) {
                            if (q == 4) {
                                l = sk1 + kA + (uint32_t)(128 + wi * 32) * BK;
                                ro = (uint32_t)(128 + wi * 32) * uldb;
                            }
                            copy8(l, rb, vB, ro, koff);
                            l = fresh(l + 8 * BK);
                            ro = fresh(ro + 8 * uldb);
                        }
                        if (q < 4) fa[q] = frag(sa + rowA + q * 16 * BK, cLo, cHi);
                        else fb[q - 4] = frag(sb + rowB + (q - 4) * 16 * BK, cLo, cHi);
                    }
                    // B1 of step k (sent one memory phase ago) lands before group 1 reads it next
                    // phase; newer: this phase's 8 copies
                    wait_vm_n(8 + st0);
                } else {
                    // A of stream step k+2, and the scale quad that starts there
                    const int s = k + 2;
                    const uint32_t vA = voffA + ((s >= nk && more) ? dA : 0u);
                    const uint32_t koff = (uint32_t)(s < nk ? s : (more ? s - nk : nk - 1)) * BK;
                    uint32_t l = sk + (uint32_t)(wi * 64) * BK, ro = (uint32_t)(wi * 64) * ulda;
#pragma unroll
                    for (int q = 0; q < 8; ++q) {
                        copy8(l, ra, vA, ro, koff);
                        l = fresh(l + 8 * BK);
                        ro = fresh(ro + 8 * ulda);
                        fb[q] = frag(sb + rowB + q * 16 * BK, cLo, cHi);
                    }
                    // this tile's quad of steps s .. s+3, or the next tile's first (nk % 4 == 0, so
                    // ring entry (qb + s / 4) & 1 continues the count into the next tile)
                    const bool quad = SCALED && ((s < nk && (s & 3) == 0) || (s == nk && more));
                    if (quad) copy_quad(sbase, (qb + (s >> 2)) & 1, s < nk ? s : 0, wi, rsa, rsb, voffS + (s < nk ? 0u : dS), usc);
                    // A of step k+1 (and a quad sent with it) lands before group 0 reads it next
                    // phase; newer: this phase's copies
                    wait_vm_n(8 + (quad ? 2 : 0) + st0);
                }
            }
            if (SCALED) {
                const uint32_t sel = pp::perm_selector(g4);
                sca = (int)pp::pack_scale_bytes(sw[0], sw[1], sw[2], sw[3], sel);
                scb0 = (int)pp::pack_scale_bytes(sw[4], sw[5], sw[6], sw[7], sel);
                scb1 = (int)pp::pack_scale_bytes(sw[8], sw[9], sw[10], sw[11], sel);
                asm volatile("" ::"v"(sca), "v"(scb0), "v"(scb1));
            }
            wait_lgkm0();
            barrier();
            // ---- compute phase (group 1 also reads A of stream step k+1, row block by row block)
            const bool next_a = grp == 1;
            const uint8_t* sn = smem + ((k + 1) & 1) * kStage;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
#pragma unroll
                for (int j = 0; j < 8; ++j) {
                    if (SCALED)
                        acc[i][j] = pp::mfma_sel<AFMT, BFMT>(fa[i], fb[j], acc[i][j], sca, j < 4 ? scb0 : scb1, i, j & 3);
                    else
                        acc[i][j] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(fa[i], fb[j], acc[i][j], AFMT, BFMT,
                                                                                      0, 0, 0, 0);
                }
                if (next_a) {
                    asm volatile("" ::"v"(acc[i][0]), "v"(acc[i][1]), "v"(acc[i][2]), "v"(acc[i][3]), "v"(acc[i][4]),
                                 "v"(acc[i][5]), "v"(acc[i][6]), "v"(acc[i][7]));
                    fa[i] = frag(sn + rowA + i * 16 * BK, cLo, cHi);
                }
            }
#pragma unroll
            for (int i = 0; i < 4; ++i)
                asm volatile("" ::"v"(acc[i][0]), "v"(acc[i][1]), "v"(acc[i][2]), "v"(acc[i][3]), "v"(acc[i][4]),
                             "v"(acc[i][5]), "v"(acc[i][6]), "v"(acc[i][7]));
            // group 0: B0 of stream step k+1 (sent in the memory phase) lands before group 0 reads
            // it next phase; newer: the 4 B1 copies sent after it (at a tile's first step the last
            // tile's stores are older than these copies, so they complete first anyway)
            if (grp == 0) wait_vm<4>();
            barrier();
        }

        // ---- tile end (group 1 gets here one phase after group 0, while group 0 multiplies)
        kargs_t* ga_ = kernel_args();
        const int64_t ldc = ga_->ldc, Me = ga_->M, Ne = ga_->N;
        gu16* const C = (gu16*)ga_->C;
        float f = 1.0f;
        if (MODE == kModeTensor || MODE == kModeMoss) f = g2::load_uniform_f32(ga_->Aglobal) * g2::load_uniform_f32(ga_->Bglobal);
        const bool full = (int64_t)m0 + BM <= Me && (int64_t)n0 + BN <= Ne;
        if (!more) {
            if (grp == 0) barrier();     // matches group 1's extra barrier at the stream's start
            wait_vm0();                  // the repeated last-step copies
        }
        const int le = (int)__lane_id(), er16 = le & 15, eg4 = le >> 4;
        if (full) {
            // quad transposes and kStores 8-byte stores (pp::quad_transpose_bf16)
            const int q = er16 & 3, c4 = er16 >> 2;
            const uint32_t modd = 0u - (uint32_t)(q & 1), mhi = 0u - (uint32_t)(q >> 1);
            gu16* const cw = C + ((int64_t)m0 + wm * 64) * ldc + n0 + wn * 128;
            const int64_t loff = (int64_t)(4 * eg4 + q) * ldc + 4 * c4;
#pragma unroll
            for (int i = 0; i < 4; ++i)
#pragma unroll
                for (int j = 0; j < 8; ++j) {
                    const uint2 w = pp::quad_transpose_bf16(acc[i][j] * f, modd, mhi);
                    *reinterpret_cast<gu64*>(cw + (int64_t)i * 16 * ldc + loff + j * 16) =
                        (uint64_t)w.x | ((uint64_t)w.y << 32);
                }
        } else {
            // partial tile: element by element, masked; the varying number of stores all complete
            // before the next tile's counted waits
            const int64_t row0 = (int64_t)m0 + wm * 64 + 4 * eg4, col0 = (int64_t)n0 + wn * 128 + er16;
#pragma unroll
            for (int i = 0; i < 4; ++i)
#pragma unroll
                for (int j = 0; j < 8; ++j) {
                    const int64_t col = col0 + j * 16;
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        const int64_t row = row0 + i * 16 + e;
                        if (row < Me && col < Ne) C[row * ldc + col] = g2::f32_to_bf16_rne(acc[i][j][e] * f);
                    }
                }
            wait_vm0();
        }
        if (!more) break;
        behind = full;
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int j = 0; j < 8; ++j) acc[i][j] = v4f{0.f, 0.f, 0.f, 0.f};
        qb += nk >> 2;
        voffA += dA;
        voffB += dB;
        voffS += dS;
        m0 = m0n;
        n0 = n0n;
        tile = tile_n;
    }
}

}  // namespace pps
}  // namespace fp8q
