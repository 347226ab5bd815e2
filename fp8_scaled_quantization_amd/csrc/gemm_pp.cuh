// Ping-pong scaled FP8 GEMM for gfx950: 256 x 256 output tiles, 8 waves, two per SIMD.
//
// C = dequant(A) . dequant(B)^T with A: M x K and B: N x K, both K-contiguous FP8 bytes, for the
// schemes whose main loop stays on the matrix cores:
//   TENSOR  (sum qa*qb) * fl(s_a*s_b) in the epilogue (page "Flax FP8 量化实战指南 ...", section 2.2);
//   MX      E8M0 scales per 32-wide K group applied by v_mfma_scale_f32_16x16x128_f8f6f4 (page
//           "MOSS:高效、精确的 FP8 LLM 训练 ...", section 1);
//   MOSS    as MX, then fl(S_A*S_B) once in the epilogue (same page, section 4).
//
// Schedule.  Waves 0-3 (group 0) and waves 4-7 (group 1) each own half of the output tile; each
// SIMD runs one wave of each group.  A wave alternates a memory phase (issue its share of the
// global->LDS copies, read its operand fragments and scales from LDS into registers) and a compute
// phase (32 MFMAs on those fragments), with one workgroup barrier between phases.  Group 1 starts
// one phase late, so on every SIMD one wave multiplies while the other moves data: the LDS reads
// never sit between a wave's MFMAs, and the matrix core is fed from both waves in turn.
//
// LDS holds two K steps (2 x 64 KiB) and a two-entry ring of scale quads (16 bytes per row = four
// K steps of E8M0 bytes).  Group 0 reads all of A and B rows 0-127 (B0) of step k in its memory
// phase (phase 2k).  Group 1 reads B rows 128-255 (B1) of step k in its memory phase (phase 2k+1)
// but reads A of step k during its compute phase for step k-1 (also phase 2k), one 16-row A block
// right after the last MFMA that used the previous step's block, so it needs no extra registers.
// A and B0 of a stage are therefore free one phase after they are first read, B1 one phase later:
//   A of step k+2       group 1, memory phase for step k (phase 2k+1), waited at the end of 2k+3;
//   scale quad of steps s .. s+3
//                       group 1, memory phase for step s-2 after its A copies, waited with them;
//   B0 and B1 of step k+1
//                       group 0, memory phase for step k (phase 2k); B0 waited at the end of phase
//                       2k+1, B1 at the end of phase 2k+2.
// A copy instruction can hold its wave while the address unit is busy, so copies never sit between
// a wave's MFMAs: each group interleaves its eight copies with its fragment reads, and group 0's
// compute phase holds only its MFMAs and one wait.  (Measured with per-phase timestamps on a MOSS
// 16384x4096x4096 product: with all twelve A and B0 copies in group 1's memory phase a K step took
// ~3150 cycles; with B0 sent after group 0's MFMAs, ~2790; with both B halves in group 0's memory
// phase, ~2700, the memory phases (~1150 cycles each) now longer than the compute phases.)
//
// Global->LDS copies use buffer_load_dwordx4 ... lds (no VGPR staging; rows past M or N read zero
// through the buffer range), with each 16-byte chunk c of tile row r stored at chunk position
// c ^ (r & 7), which keeps both the copy writes and the fragment reads free of bank conflicts.
//
// Persistent grid.  With more tiles than CUs the grid has one workgroup per CU and each loops over
// its tiles.  At a tile's end the workgroup sends the next tile's pipeline fill first and only then
// the epilogue's 32 stores per wave, so the stores drain while the next tile's main loop starts
// instead of holding the CU until they complete (vector-memory operations complete in issue order,
// so the first waits of the next tile allow 32 more operations in flight).  Values that only the
// tile boundary needs (C, ldc, M, N, the global factors, the lane index) are read again there rather
// than kept in registers through the main loop, which uses nearly all of them.
#pragma once
#include "gemm_kernel.cuh"

namespace fp8q {
namespace pp {

using g2::dma16;
using g2::lds_addr;
using g2::make_rsrc;
using g2::rsrc_t;
using g2::v4f;
using g2::v8i;

constexpr int BM = 256, BN = 256, BK = 128;
constexpr int kA = BM * BK, kB = BN * BK, kStage = kA + kB;   // 64 KiB per K step
constexpr int kScBase = 2 * kStage;
constexpr int kScQuad = (BM + BN) * 16;                        // 8 KiB: 4 K steps of E8M0 bytes

template <int MODE>
constexpr size_t lds_bytes() {
    return (MODE == kModeMX || MODE == kModeMoss) ? (size_t)(kScBase + 2 * kScQuad) : (size_t)kScBase;
}

__device__ __forceinline__ void barrier() {
    __builtin_amdgcn_sched_barrier(0);
    asm volatile("s_barrier" ::: "memory");
    __builtin_amdgcn_sched_barrier(0);
}
__device__ __forceinline__ void wait_lgkm0() { asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory"); }
__device__ __forceinline__ void wait_vm0() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }
// all but the last N vector-memory instructions of this wave complete (they complete in order)
template <int N>
__device__ __forceinline__ void wait_vm() { g2::wait_vmcnt<N>(); }


// (a & m) | (b & ~m)
__device__ __forceinline__ uint32_t bitsel(uint32_t m, uint32_t a, uint32_t b) { return (a & m) | (b & ~m); }

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));
// two fp32 -> packed bf16 (round to nearest even; v_cvt_pk_bf16_f32), a in the low half
__device__ __forceinline__ uint32_t pack_bf16(float a, float b) {
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2_t{a, b}, bf16x2_t));
}

// Full-tile bf16 epilogue piece: a 4x4 transpose of bf16 values within each quad of lanes turns
// the MFMA layout (lane r16 holds one column, four rows of a 16 x 16 subtile) into one row and four
// columns per lane: lane (g4, r16 = 4 c4 + q) gets row 4 g4 + q, columns 4 c4 .. 4 c4 + 3, which it
// stores with one 8-byte write (each row's 32 bytes come from four lanes).  modd and mhi are the
// lane-constant masks 0 - (q & 1) and 0 - (q >> 1): the selections are bit selects, not branches.
// Input: the packed words w0 = bf16 rows (0, 1) and w1 = rows (2, 3) of the lane's column.
__device__ __forceinline__ uint2 quad_transpose_words(uint32_t w0, uint32_t w1, uint32_t modd, uint32_t mhi) {
    // swap with lane q^1: even lanes collect rows 0 and 2, odd lanes rows 1 and 3, of two adjacent
    // columns
    const uint32_t s1 = bitsel(modd, (w0 & 0xFFFFu) | (w1 << 16), (w0 >> 16) | (w1 & 0xFFFF0000u));
    const uint32_t r1 = (uint32_t)__builtin_amdgcn_mov_dpp((int)s1, 0xB1, 0xF, 0xF, false);   // [1,0,3,2]
    const uint32_t x0 = bitsel(modd, (r1 & 0xFFFFu) | (w0 & 0xFFFF0000u), (w0 & 0xFFFFu) | (r1 << 16));
    const uint32_t x1 = bitsel(modd, (r1 >> 16) | (w1 & 0xFFFF0000u), (w1 & 0xFFFFu) | (r1 & 0xFFFF0000u));
    // swap with lane q^2: lane q ends with row q, columns 0-1 and 2-3 of the quad
    const uint32_t r2 = (uint32_t)__builtin_amdgcn_mov_dpp((int)bitsel(mhi, x0, x1), 0x4E, 0xF, 0xF, false);   // [2,3,0,1]
    return make_uint2(bitsel(mhi, r2, x0), bitsel(mhi, x1, r2));
}
// The same from the four fp32 values of the lane's column (rounded to bf16 first).
__device__ __forceinline__ uint2 quad_transpose_bf16(v4f v, uint32_t modd, uint32_t mhi) {
    return quad_transpose_words(pack_bf16(v[0], v[1]), pack_bf16(v[2], v[3]), modd, mhi);
}

__device__ __forceinline__ v8i frag(const uint8_t* row, uint32_t lo, uint32_t hi) {
    const uint4 a = *reinterpret_cast<const uint4*>(row + lo);
    const uint4 b = *reinterpret_cast<const uint4*>(row + hi);
    return v8i{(int)a.x, (int)a.y, (int)a.z, (int)a.w, (int)b.x, (int)b.y, (int)b.z, (int)b.w};
}

// Byte g of each of four scale words w0..w3, packed as bytes 0..3 of one register.  v_perm_b32
// takes bytes 0-3 from its second operand and 4-7 from its first, and a selector byte 0x0C gives
// zero, so with sel = perm_selector(g) one permute puts byte g of w0 and of w1 in bytes 0 and 1;
// two permutes and a shift-or give the register (one selector register, as many as a shift count).
__device__ __forceinline__ uint32_t perm_selector(int g) {
    return (uint32_t)g | ((uint32_t)(4 + g) << 8) | 0x0C0C0000u;
}
__device__ __forceinline__ uint32_t pack_scale_bytes(uint32_t w0, uint32_t w1, uint32_t w2, uint32_t w3,
                                                     uint32_t sel) {
    return __builtin_amdgcn_perm(w1, w0, sel) | (__builtin_amdgcn_perm(w3, w2, sel) << 16);
}

// Block-scaled MFMA whose E8M0 scales sit in byte selA of sa and byte selB of sb (the byte
// selects must be literals; callers pass loop indices of fully unrolled loops, so the switch folds).
template <int AF, int BF>
__device__ __forceinline__ v4f mfma_sel(v8i a, v8i b, v4f c, int sa, int sb, int selA, int selB) {
#define FP8Q_MF(x, y) \
    case (x) * 4 + (y): return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, c, AF, BF, x, sa, y, sb);
    switch (selA * 4 + selB) {
        FP8Q_MF(0, 0) FP8Q_MF(0, 1) FP8Q_MF(0, 2) FP8Q_MF(0, 3)
        FP8Q_MF(1, 0) FP8Q_MF(1, 1) FP8Q_MF(1, 2) FP8Q_MF(1, 3)
        FP8Q_MF(2, 0) FP8Q_MF(2, 1) FP8Q_MF(2, 2) FP8Q_MF(2, 3)
        FP8Q_MF(3, 0) FP8Q_MF(3, 1) FP8Q_MF(3, 2)
        default: break;
    }
#undef FP8Q_MF
    return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, c, AF, BF, 3, sa, 3, sb);
}

// A wave-uniform value the compiler must treat as new at this point: what is derived from it is
// computed here, not hoisted out of the tile loop and kept live across the main loop.
template <class T>
__device__ __forceinline__ T fresh(T x) {
    asm volatile("" : "+s"(x));
    return x;
}

// The kernel's argument block, read through the scalar cache (constant address space) from a
// pointer the compiler must treat as new, so that an argument needed only at a tile's end is loaded
// there instead of occupying a scalar register through the main loop.
typedef __attribute__((address_space(4))) const GemmArgs kargs_t;
__device__ __forceinline__ kargs_t* kernel_args() {
    return reinterpret_cast<kargs_t*>(fresh(reinterpret_cast<uint64_t>(__builtin_amdgcn_kernarg_segment_ptr())));
}

// One copy instruction: 8 tile rows starting at row r0 (64 rows of scale bytes for a scale quad).
// The buffer descriptor's range ends at the operand's last row, and the row offset is part of the
// range-checked per-lane offset, so rows past M or N read zero; the K offset goes into the
// unchecked scalar offset.  The lane offset is formed by an asm add so that it is recomputed at
// each copy rather than kept in a register per instruction.
__device__ __forceinline__ void copy8(uint32_t lds, rsrc_t rs, uint32_t voff0, uint32_t row_off, uint32_t koff) {
    uint32_t voff;
    asm volatile("v_add_u32 %0, %1, %2" : "=v"(voff) : "s"(row_off), "v"(voff0));
    dma16(lds, rs, voff, koff);
}
// The same with the LDS destination as a pointer into the dynamic allocation.
__device__ __forceinline__ void copy8(uint8_t* lds, rsrc_t rs, uint32_t voff0, uint32_t row_off, uint32_t koff) {
    copy8(lds_addr(lds), rs, voff0, row_off, koff);
}

// Wave wi: A rows 64 wi .. +64 of step ks into the stage of step s (8 copies).  ks = s except past
// the last step, where the copies repeat the last step's data into a stage no step reads, so that
// the main loop has no branches and the same wait counts in every iteration.
__device__ __forceinline__ void copy_A(uint32_t sbase, int s, int ks, int wi, rsrc_t ra, uint32_t voffA, uint32_t lda) {
    const uint32_t st = sbase + (s & 1) * kStage;
    const uint32_t koff = (uint32_t)ks * BK;
    uint32_t l = st + (uint32_t)(wi * 64) * BK, ro = (uint32_t)(wi * 64) * lda;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
        copy8(l, ra, voffA, ro, koff);
        l = fresh(l + 8 * BK);
        ro = fresh(ro + 8 * lda);
    }
}
// Wave wi: B rows base + 32 wi .. +32 of step ks into the stage of step s (4 copies); base 0 (B0)
// or 128 (B1).
__device__ __forceinline__ void copy_B(uint32_t sbase, int s, int ks, int base, int wi, rsrc_t rb, uint32_t voffB,
                                       uint32_t ldb) {
    const uint32_t st = sbase + (s & 1) * kStage + kA;
    const uint32_t koff = (uint32_t)ks * BK;
    uint32_t l = st + (uint32_t)(base + wi * 32) * BK, ro = (uint32_t)(base + wi * 32) * ldb;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        copy8(l, rb, voffB, ro, koff);
        l = fresh(l + 8 * BK);
        ro = fresh(ro + 8 * ldb);
    }
}
// Group 1, wave wi, every fourth step: two instructions of the scale quad for steps s .. s+3.
// The K offset goes into the range-checked lane offset: when the K steps are not a multiple of 4
// the last quad of a row ends past the row, and on the array's last row past its end, where the
// buffer range turns the excess into zeros.
__device__ __forceinline__ void copy_quad(uint32_t sbase, int s, int wi, rsrc_t rsa, rsrc_t rsb, uint32_t voffS,
                                          uint32_t sc_row) {
    const uint32_t sq = sbase + kScBase + ((s >> 2) & 1) * kScQuad;
    const uint32_t voff = voffS + (uint32_t)s * 4;
#pragma unroll
    for (int j = 0; j < 2; ++j) {
        const int inst = wi * 2 + j;              // 0..3: A rows, 4..7: B rows, 64 rows each
        const uint32_t r0 = (uint32_t)(inst & 3) * 64;
        copy8(sq + inst * 64 * 16, inst < 4 ? rsa : rsb, voff, r0 * sc_row, 0u);
    }
}

template <int MODE, int AFMT, int BFMT, bool OUT_BF16>
__global__ __launch_bounds__(512, 1) void gemm_pp_kernel(GemmArgs g) {
    constexpr bool SCALED = MODE == kModeMX || MODE == kModeMoss;
    static_assert(MODE != kModeBlock, "block scaling promotes per K step; it has its own kernel");
    extern __shared__ __attribute__((aligned(16))) uint8_t smem[];

    const int t = threadIdx.x, lane = t & 63;
    const int wave = fresh(__builtin_amdgcn_readfirstlane(t >> 6));   // wave-uniform: kept in SGPRs
    const int grp = wave >> 2;
    const int wm = wave & 3, wn = grp;            // wave tile: rows 64 wm .. +64, cols 128 wn .. +128
    const int r16 = lane & 15, g4 = lane >> 4;
    const int64_t M = g.M, N = g.N;
    // the launcher admits operands of fewer than 2^32 bytes, so tile counts and byte offsets within
    // an operand fit 32 bits
    const uint32_t ntm_ = (uint32_t)((M + BM - 1) / BM), ntn_ = (uint32_t)((N + BN - 1) / BN);
    const uint32_t ntiles = ntm_ * ntn_;
    // Tile coordinates: undo the round-robin XCD dispatch, then walk groups of 8 tile-rows.  The
    // grid is a multiple of 8 workgroups (or one per tile) and workgroup w takes tiles w, w + G,
    // w + 2G, ... (G = gridDim.x), so tile % 8, the XCD, stays fixed and the tiles that one XCD
    // runs at the same time are neighbours in the walk.
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
        // the division runs on the vector unit: bring the results back to scalar registers
        m0_ = (uint32_t)__builtin_amdgcn_readfirstlane((int)((first_m + in_grp % gm) * BM));
        n0_ = (uint32_t)__builtin_amdgcn_readfirstlane((int)((in_grp / gm) * BN));
    };
    const int nk = (int)(g.K / BK);

    // Buffer descriptors over whole operands: their ranges end at the last row, so rows past M or N
    // read zero; a tile's row offset is part of the range-checked lane offset.
    const int64_t sc_row = 4 * (int64_t)nk;      // E8M0 bytes per row
    const rsrc_t ra = make_rsrc(g.A, (uint32_t)(M * g.lda));
    const rsrc_t rb = make_rsrc(g.B, (uint32_t)(N * g.ldb));
    rsrc_t rsa = rsrc_t{0u, 0u, 0u, 0u}, rsb = rsrc_t{0u, 0u, 0u, 0u};
    if (SCALED) {
        rsa = make_rsrc(g.Ascale, (uint32_t)(M * sc_row));
        rsb = make_rsrc(g.Bscale, (uint32_t)(N * sc_row));
    }
    // copy lanes: lane i of a copy instruction covers row r0 + i/8 at LDS chunk i%8, fetching global
    // chunk (i%8) ^ (row & 7) (r0 is a multiple of 8); scale quads take one row per lane (waves 0-1
    // of group 1 A rows, waves 2-3 B rows)
    const uint32_t ch = (uint32_t)(((lane & 7) ^ ((lane >> 3) & 7)) << 4);
    const uint32_t ulda = (uint32_t)g.lda, uldb = (uint32_t)g.ldb, usc = (uint32_t)sc_row;
    const int wi = wave & 3;
    const uint32_t sbase = lds_addr(smem);   // LDS address of the dynamic allocation

    // fragment read offsets (loop invariant): row base of each 16-row subtile, swizzled chunks
    const uint32_t cLo = (uint32_t)((g4 ^ (r16 & 7)) << 4), cHi = (uint32_t)(((4 + g4) ^ (r16 & 7)) << 4);
    const uint32_t rowA = (uint32_t)((wm * 64 + r16) * BK), rowB = (uint32_t)((wn * 128 + r16) * BK);

    uint32_t tile = blockIdx.x, m0, n0;
    coords(tile, m0, n0);
    uint32_t voffA, voffB, voffS;
    auto lane_offsets = [&](uint32_t tm, uint32_t tn) {
        voffA = (uint32_t)(lane >> 3) * ulda + ch + tm * ulda;
        voffB = (uint32_t)(lane >> 3) * uldb + ch + tn * uldb;
        voffS = (uint32_t)lane * usc + (wi < 2 ? tm : tn) * usc;
    };
    lane_offsets(m0, n0);

    // ---- a tile's pipeline fill: group 1 sends A and B0 of step 0 and A of step 1; group 0 sends
    // B1 of step 0 (afterwards it sends B0 and B1 of step k+1 in its memory phase for step k; group
    // 1 sends A of step k+2 in its memory phase).  For every tile but the first it goes out before
    // the previous tile's epilogue, whose stores then follow it in the wave's vector-memory queue.
    const int k1 = min(nk - 1, 1);   // (nk >= 1; a scalar min, not a select the compiler would keep in a VGPR)
    auto fill = [&]() {
        const uint32_t la = fresh(ulda), lb = fresh(uldb), ls = fresh(usc), sb0 = fresh(sbase);
        if (grp == 0) {
            copy_B(sb0, 0, 0, 128, wi, rb, voffB, lb);
        } else {
            copy_A(sb0, 0, 0, wi, ra, voffA, la);
            copy_B(sb0, 0, 0, 0, wi, rb, voffB, lb);
            if (SCALED) copy_quad(sb0, 0, wi, rsa, rsb, voffS, ls);
            copy_A(sb0, 1, k1, wi, ra, voffA, la);
        }
    };
    fill();
    // kStores stores of the previous tile sit behind the fill: vector-memory operations complete in
    // issue order, so a wait for the fill or older work must allow that many more in flight
    constexpr int kStores = 32;
    bool behind = false;
    v8i fa[4], fb[8];
    v4f acc[4][8];

    for (;;) {
        // next tile's coordinates, while the accumulators are dead
        const uint32_t tile_n = tile + fresh(gridDim.x);
        uint32_t m0n = 0, n0n = 0;
        if (tile_n < ntiles) coords(tile_n, m0n, n0n);

        // group 1's A and B0 of step 0 (and the scale quad) land before the barrier; group 0's
        // fill (B1 of step 0) is waited for in its first memory phase
        if (grp == 1) {
            if (behind) wait_vm<8 + kStores>();
            else wait_vm<8>();
        }
        barrier();
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int j = 0; j < 8; ++j) acc[i][j] = v4f{0.f, 0.f, 0.f, 0.f};
        if (grp == 1) {
            // group 1 reads A of step 0 while group 0 has its first memory phase
#pragma unroll
            for (int i = 0; i < 4; ++i) fa[i] = frag(smem + rowA + i * 16 * BK, cLo, cHi);
            barrier();
        }

        int sca = 0, scb0 = 0, scb1 = 0;
        for (int k = 0; k < nk; ++k) {
            // in step 0 the copies waited for are the fill's, which are older than the stores
            // (the test goes through fresh() so that the compiler does not peel the first step)
            const bool st0 = behind && fresh(k) == 0;
            // LDS bases of this step's stage and the other one, computed afresh in every step
            const uint32_t sk = fresh(sbase + (k & 1) * kStage), sk1 = fresh(sbase + ((k + 1) & 1) * kStage);
            // ---- memory phase: scale words first, then fragment reads interleaved with this phase's
            // copies (a copy may wait for the address unit; the LDS reads queued around it keep going)
            uint32_t sw[12];
            if (SCALED) {
                const uint32_t* sq = reinterpret_cast<const uint32_t*>(smem + kScBase + ((k >> 2) & 1) * kScQuad);
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
                    // A and B0 of step k; B0, then B1, of step k+1 (8 copies, one per fragment
                    // read; that stage's B0 was last read in the previous memory phase, its B1 one
                    // phase earlier)
                    const uint32_t st = sk1 + kA;
                    const uint32_t koff = (uint32_t)min(k + 1, nk - 1) * BK;
                    uint32_t l = st + (uint32_t)(wi * 32) * BK, ro = (uint32_t)(wi * 32) * uldb;
#pragma unroll
                    for (int q = 0; q < 12; ++q) {
                        if (q < 8) {
                            if (q == 4) {
                                l = st + (uint32_t)(128 + wi * 32) * BK;
                                ro = (uint32_t)(128 + wi * 32) * uldb;
                            }
                            copy8(l, rb, voffB, ro, koff);
                            l = fresh(l + 8 * BK);
                            ro = fresh(ro + 8 * uldb);
                        }
                        if (q < 4) fa[q] = frag(sa + rowA + q * 16 * BK, cLo, cHi);
                        else fb[q - 4] = frag(sb + rowB + (q - 4) * 16 * BK, cLo, cHi);
                    }
                    // B1 of step k (sent one memory phase ago, or the fill) lands before group 1
                    // reads it next phase; newer: this phase's 8 copies
                    if (st0) wait_vm<8 + kStores>();
                    else wait_vm<8>();
                } else {
                    // B1 of step k; A of step k+2 (8 copies, one per fragment read) and the scale quad
                    const uint32_t st = sk;
                    const uint32_t koff = (uint32_t)min(k + 2, nk - 1) * BK;
                    uint32_t l = st + (uint32_t)(wi * 64) * BK, ro = (uint32_t)(wi * 64) * ulda;
#pragma unroll
                    for (int q = 0; q < 8; ++q) {
                        copy8(l, ra, voffA, ro, koff);
                        l = fresh(l + 8 * BK);
                        ro = fresh(ro + 8 * ulda);
                        fb[q] = frag(sb + rowB + q * 16 * BK, cLo, cHi);
                    }
                    const bool quad = SCALED && k + 2 < nk && ((k + 2) & 3) == 0;
                    if (quad) copy_quad(sbase, k + 2, wi, rsa, rsb, voffS, usc);
                    // A of step k+1 (sent one memory phase ago, or in the fill) lands before group 0
                    // reads it next phase; this phase's copies may stay in flight
                    if (st0) {
                        if (quad) wait_vm<10 + kStores>();
                        else wait_vm<8 + kStores>();
                    } else {
                        if (quad) wait_vm<10>();
                        else wait_vm<8>();
                    }
                }
            }
            if (SCALED) {
                // byte g4 of a row's word = the E8M0 scale of (row, group g4) for this step; four
                // subtiles per register, picked in the MFMA by its byte select
                const uint32_t sel = perm_selector(g4);
                sca = (int)pack_scale_bytes(sw[0], sw[1], sw[2], sw[3], sel);
                scb0 = (int)pack_scale_bytes(sw[4], sw[5], sw[6], sw[7], sel);
                scb1 = (int)pack_scale_bytes(sw[8], sw[9], sw[10], sw[11], sel);
                // finish the packing here, in the memory phase, not after the barrier
                asm volatile("" ::"v"(sca), "v"(scb0), "v"(scb1));
            }
            wait_lgkm0();
            barrier();
            // ---- compute phase (group 1 also reads A of step k+1, row block by row block; past the
            // last step it reads a stage it does not use)
            const bool next_a = grp == 1;
            const uint8_t* sn = smem + ((k + 1) & 1) * kStage;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
#pragma unroll
                for (int j = 0; j < 8; ++j) {
                    if (SCALED)
                        acc[i][j] = mfma_sel<AFMT, BFMT>(fa[i], fb[j], acc[i][j], sca, j < 4 ? scb0 : scb1, i, j & 3);
                    else
                        acc[i][j] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(fa[i], fb[j], acc[i][j], AFMT, BFMT,
                                                                                      0, 0, 0, 0);
                }
                if (next_a) {
                    // the eight MFMAs above are issued before fa[i] is overwritten
                    asm volatile("" ::"v"(acc[i][0]), "v"(acc[i][1]), "v"(acc[i][2]), "v"(acc[i][3]), "v"(acc[i][4]),
                                 "v"(acc[i][5]), "v"(acc[i][6]), "v"(acc[i][7]));
                    fa[i] = frag(sn + rowA + i * 16 * BK, cLo, cHi);
                }
            }
            // every accumulator is read here, so all 32 MFMAs are issued before the barrier
#pragma unroll
            for (int i = 0; i < 4; ++i)
                asm volatile("" ::"v"(acc[i][0]), "v"(acc[i][1]), "v"(acc[i][2]), "v"(acc[i][3]), "v"(acc[i][4]),
                             "v"(acc[i][5]), "v"(acc[i][6]), "v"(acc[i][7]));
            // group 0: B0 of step k+1 (sent in the memory phase) lands before group 0 reads it next
            // phase; newer: the 4 B1 copies sent after it (at a tile's first step the previous
            // tile's stores are older than these copies and complete first anyway)
            if (grp == 0) wait_vm<4>();
            barrier();
        }
        if (grp == 0) barrier();          // matches group 1's extra barrier at the start
        // every wave's copies of this tile (the last steps repeat the last step's data) have landed
        // before any wave refills the stages
        wait_vm0();
        barrier();
        const bool more = tile_n < ntiles;
        if (more) {
            // move the lane offsets to the next tile (no lane index needs to stay live)
            voffA += (m0n - m0) * ulda;
            voffB += (n0n - n0) * uldb;
            voffS += (wi < 2 ? m0n - m0 : n0n - n0) * usc;
            fill();
        }
        // the epilogue's stores stay behind the fill
        __builtin_amdgcn_sched_barrier(0);

        // ---- epilogue
        // the epilogue's arguments are read again from the kernel argument segment, so that they
        // do not occupy scalar registers through the main loop
        kargs_t* ga_ = kernel_args();
        const int64_t ldc = ga_->ldc, Me = ga_->M, Ne = ga_->N;
        typedef __attribute__((address_space(1))) uint16_t gu16;
        typedef __attribute__((address_space(1))) uint64_t gu64;
        gu16* const C = (gu16*)ga_->C;
        // global dequantisation factors (TENSOR: s_a, s_b; MOSS: S_A, S_B) through the scalar cache;
        // their product fl(s_a * s_b) scales the accumulators
        float f = 1.0f;
        if (MODE == kModeTensor || MODE == kModeMoss) f = g2::load_uniform_f32(ga_->Aglobal) * g2::load_uniform_f32(ga_->Bglobal);
        const bool full = OUT_BF16 && (int64_t)m0 + BM <= Me && (int64_t)n0 + BN <= Ne;
        // lane index again from the hardware, rather than kept in a register through the main loop
        const int le = (int)__lane_id(), er16 = le & 15, eg4 = le >> 4;
        if (full) {
            // full tile: quad transposes and kStores 8-byte stores (quad_transpose_bf16)
            const int q = er16 & 3, c4 = er16 >> 2;
            const uint32_t modd = 0u - (uint32_t)(q & 1), mhi = 0u - (uint32_t)(q >> 1);
            gu16* const cw = C + ((int64_t)m0 + wm * 64) * ldc + n0 + wn * 128;
            const uint32_t loff = (uint32_t)((4 * eg4 + q) * ldc + 4 * c4);
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                gu16* const ci = cw + (int64_t)i * 16 * ldc;
#pragma unroll
                for (int j = 0; j < 8; ++j) {
                    const uint2 w = quad_transpose_bf16(acc[i][j] * f, modd, mhi);
                    *reinterpret_cast<gu64*>(ci + loff + j * 16) = (uint64_t)w.x | ((uint64_t)w.y << 32);
                }
            }
        } else {
            // partial tile or fp32 output: element by element, masked
            const int64_t row0 = (int64_t)m0 + wm * 64 + 4 * eg4, col0 = (int64_t)n0 + wn * 128 + er16;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
#pragma unroll
                for (int j = 0; j < 8; ++j) {
                    const int64_t col = col0 + j * 16;
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        const int64_t row = row0 + i * 16 + e;
                        if (row < Me && col < Ne) {
                            const float v = acc[i][j][e] * f;
                            if (OUT_BF16) C[row * ldc + col] = g2::f32_to_bf16_rne(v);
                            else ((__attribute__((address_space(1))) float*)C)[row * ldc + col] = v;
                        }
                    }
                }
            }
            // the masked path issues a varying number of stores: let them finish, so the next
            // tile's waits count only its own copies
            wait_vm0();
        }
        if (!more) break;
        behind = full;
        tile = tile_n;
        m0 = m0n;
        n0 = n0n;
    }
}

}  // namespace pp
}  // namespace fp8q
