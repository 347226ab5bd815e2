// FP8 cast kernels for the five scaling schemes.
//
// Every element is RNE8(clip(fl(x / scale))) (page "Flax FP8 量化实战指南 ...", sections 1 and 2.2),
// with the scale chosen per scheme:
//   TENSOR  one fp32 scale: current (amax/MAX of the whole tensor) or supplied (delayed / static);
//   BLOCK   one fp32 scale per 1x128 row group or 128x128 block (page "Transformers 中的细粒度 FP8
//           量化配置 ...", section 一);
//   MX      a power of two per 32 consecutive K values, chosen so that nothing clips (page "MOSS:
//           高效、精确的 FP8 LLM 训练 ...", section 1); the element is x * 2^-e, exact scaling;
//   MOSS    fp32 global S times a per-32 power-of-two local factor in (0, 1] (same page, section 4);
//           the element is fl(x / S) * 2^-e_i;
//   BLOCK_E8M0  one power-of-two (UE8M0) scale per block, chosen like MX so that nothing clips
//           (page "Transformers 中的细粒度 FP8 量化配置 ...", section 七); element x * 2^-e.
//
// Work layout.  A "lane chunk" is 32 consecutive values along the output's K axis, owned by one
// lane: an MX/MOSS group is exactly one lane (no cross-lane reduction) and a 1x128 group is four
// adjacent lanes (two xor-shuffles).  The division by a scale uses y = RN(1/s) and one Markstein
// correction, which equals IEEE division whenever the guards in common.cuh hold (exhaustively
// checked over all dividend significands for thousands of divisors); chunks outside the guards,
// and lanes holding NaN, use IEEE division and the NaN byte fix-up instead.
#include "common.cuh"
#include "kernels.h"

namespace fp8q {

// ------------------------------------------------------------------ per-chunk work
// Elements are cast N at a time (N = 32: one lane chunk; N = 8: one 16-byte bf16 load); out[i]
// packs the codes of v[4i .. 4i+3].
// max |x| bits of N values
template <int N>
__device__ __forceinline__ uint32_t chunk_max(const float* v) {
    uint32_t m = 0u;
#pragma unroll
    for (int j = 0; j < N; ++j) m = max(m, absbits(v[j]));
    return m;
}
// min (|x| bits - 1) of N values (zero wraps to 0xffffffff): the small-dividend guard of the
// one-correction division; only its paths compute it
template <int N>
__device__ __forceinline__ uint32_t chunk_min_m1(const float* v) {
    uint32_t m = 0xFFFFFFFFu;
#pragma unroll
    for (int j = 0; j < N; ++j) m = min(m, absbits(v[j]) - 1u);
    return m;
}

// element = clip(fl(v/s) * 2^shift); `fast` selects the one-correction division (its guards hold).
template <int FMT, bool SHIFT, int N>
__device__ __forceinline__ void cast_div(const float* v, float s, float y, int shift, bool fast, uint32_t* out) {
    if (fast) {
#pragma unroll
        for (int i = 0; i < N / 4; ++i) {
            float c[4];
#pragma unroll
            for (int k = 0; k < 4; ++k) {
                float q = div_fast(v[4 * i + k], s, y);
                if (SHIFT) q = __builtin_amdgcn_ldexpf(q, shift);
                c[k] = clip<FMT>(q);
            }
            out[i] = cvt4<FMT>(c[0], c[1], c[2], c[3]);
        }
    } else {
#pragma unroll
        for (int i = 0; i < N / 4; ++i) {
            uint32_t w = 0;
#pragma unroll
            for (int k = 0; k < 4; ++k) {
                float q = v[4 * i + k] / s;
                if (SHIFT) q = __builtin_amdgcn_ldexpf(q, shift);
                w |= code_slow<FMT>(q) << (8 * k);
            }
            out[i] = w;
        }
    }
}

// bf16 fast path: element = clip(RN(x / s)) computed as mul2 (valid when mul2_exact_bf16 held for
// s and the values are finite; see common.cuh).
template <int FMT, int N>
__device__ __forceinline__ void cast_mul2(const float* v, float yh, float yl, uint32_t* out) {
#pragma unroll
    for (int i = 0; i < N / 4; ++i) {
        float c[4];
#pragma unroll
        for (int k = 0; k < 4; ++k) c[k] = clip<FMT>(mul2(v[4 * i + k], yh, yl));
        out[i] = cvt4<FMT>(c[0], c[1], c[2], c[3]);
    }
}

// MX element: clip(x * 2^shift), exact scaling; only NaN needs the slow path.
template <int FMT, int N>
__device__ __forceinline__ void cast_mx(const float* v, int shift, bool has_nan, uint32_t* out) {
    if (!has_nan) {
#pragma unroll
        for (int i = 0; i < N / 4; ++i) {
            float c[4];
#pragma unroll
            for (int k = 0; k < 4; ++k) c[k] = clip<FMT>(__builtin_amdgcn_ldexpf(v[4 * i + k], shift));
            out[i] = cvt4<FMT>(c[0], c[1], c[2], c[3]);
        }
    } else {
#pragma unroll
        for (int i = 0; i < N / 4; ++i) {
            uint32_t w = 0;
#pragma unroll
            for (int k = 0; k < 4; ++k) w |= code_slow<FMT>(__builtin_amdgcn_ldexpf(v[4 * i + k], shift)) << (8 * k);
            out[i] = w;
        }
    }
}

// Tensor-uniform divisor state (TENSOR and MOSS).  y = RN(1/s) for the one-correction division
// (ok: s is in its range); two: bf16 inputs may use the two-term reciprocal (yh, yl).
struct UniformScale {
    float s, y, yh, yl;
    bool ok, two;
    SParts sp;        // MOSS: S as mantissa and exponent
};

// Called by every thread of the workgroup at kernel start (the bf16 check is a wave vote).
template <int FMT, int MODE, bool DERIVE, bool BF16>
__device__ __forceinline__ UniformScale uniform_scale(const CastArgs& a) {
    UniformScale u{1.0f, 1.0f, 1.0f, 0.0f, true, false, {0, 0u}};
    if (MODE == kModeTensor || MODE == kModeMoss) {
        float s = DERIVE ? scale_from_amax<FMT>(*a.amax_in, 1.0f) : *a.scale_in;
        u.s = s;
        u.y = recip_rn(s);
        u.ok = divisor_ok(s);
        if (BF16 && u.ok) {
            u.yh = recip_hi_rz(s);
            u.yl = recip_lo(s, u.yh);
            u.two = mul2_exact_bf16(s, u.yh, u.yl);
        }
        if (MODE == kModeMoss) u.sp = s_parts(s);
        if (DERIVE && blockIdx.x == 0 && blockIdx.y == 0 && threadIdx.x == 0) *a.scale_out = s;
    }
    return u;
}

// TENSOR / MX / MOSS cast of N values of one 32-group: gmx is the group's max |x| bits, lmx the
// max of these N values (the division path is chosen per lane; the result does not depend on it);
// lmn, when given, their min (|x| bits - 1) for the division guard (else computed from v -- the
// compiler evaluates it ahead of the per-lane branch, so callers holding packed words pass it).
// Returns the E8M0 byte (MX, MOSS) in sc.
template <int FMT, int MODE, bool BF16, int N>
__device__ __forceinline__ void cast_group(const float* v, uint32_t gmx, uint32_t lmx, const UniformScale& u,
                                           uint32_t* out, uint32_t& sc, const uint32_t* lmn = nullptr) {
    if (MODE == kModeTensor) {
        if (BF16 && u.two && lmx < 0x7F800000u) cast_mul2<FMT, N>(v, u.yh, u.yl, out);
        else cast_div<FMT, false, N>(v, u.s, u.y, 0, u.ok && dividends_ok(lmx, lmn ? *lmn : chunk_min_m1<N>(v)), out);
    } else if (MODE == kModeMX) {
        int e = mx_exponent<FMT>(__uint_as_float(gmx));
        cast_mx<FMT, N>(v, -e, lmx > 0x7F800000u, out);
        sc = (uint32_t)(e + 127);
    } else {  // MOSS
        const int e = moss_exponent_p(u.sp, div_by_max<FMT>(__uint_as_float(gmx)));
        // fl(x / S) * 2^-e equals fl(x / (S 2^e)) whenever fl(x / S) is normal; with e > -100 a
        // subnormal fl(x / S) is below 2^-26 after scaling, i.e. FP8 zero either way
        const float sg = __builtin_amdgcn_ldexpf(u.s, e);
        if (BF16 && u.two && e > -100 && divisor_ok(sg) && lmx < 0x7F800000u)
            cast_mul2<FMT, N>(v, __builtin_amdgcn_ldexpf(u.yh, -e), __builtin_amdgcn_ldexpf(u.yl, -e), out);
        else
            cast_div<FMT, true, N>(v, u.s, u.y, -e,
                                   u.ok && dividends_ok(lmx, lmn ? *lmn : chunk_min_m1<N>(v)) && e > -100, out);
        sc = (uint32_t)(e + 127);
    }
}

// Process one lane chunk v[32] (all 64 lanes of the wave call this together: BLOCK uses shuffles).
// Returns the per-lane scale value to store (BLOCK: fp32 bits; MX/MOSS: E8M0 byte) in `sc`.
// BLOCK 1x128: the four chunks of a group sit in lanes l, l ^ G, l ^ 2G, l ^ 3G.
// mx: the chunk's max |x| bits; mnm1: its min (|x| bits - 1), or nullptr to compute it from v (only
// BLOCK's division guard uses it).
template <int FMT, int MODE, bool BF16, int G = 1>
__device__ __forceinline__ void process_chunk_mm(const float* v, uint32_t mx, const uint32_t* mnm1, const UniformScale& u,
                                                 uint32_t* out, uint32_t& sc) {
    if (MODE == kModeBlock) {
        uint32_t gmx = mx;
        uint32_t o = (uint32_t)__shfl_xor((int)gmx, G, 64);
        gmx = max(gmx, o);
        o = (uint32_t)__shfl_xor((int)gmx, 2 * G, 64);
        gmx = max(gmx, o);
        float s = scale_from_amax<FMT>(__uint_as_float(gmx), 1.0f);
        float y = recip_rn(s);
        const uint32_t mn = mnm1 ? *mnm1 : chunk_min_m1<32>(v);
        cast_div<FMT, false, 32>(v, s, y, 0, divisor_ok(s) && dividends_ok(mx, mn), out);
        sc = __float_as_uint(s);
    } else {
        cast_group<FMT, MODE, BF16, 32>(v, mx, mx, u, out, sc, mnm1);
    }
}
template <int FMT, int MODE, bool BF16, int G = 1>
__device__ __forceinline__ void process_chunk(const float* v, const UniformScale& u, uint32_t* out,
                                              uint32_t& sc, uint32_t& chunk_max_out) {
    const uint32_t mx = chunk_max<32>(v);
    chunk_max_out = mx;
    process_chunk_mm<FMT, MODE, BF16, G>(v, mx, nullptr, u, out, sc);
}

__device__ __forceinline__ void store32(uint8_t* p, const uint32_t* w) {
    reinterpret_cast<uint4*>(p)[0] = make_uint4(w[0], w[1], w[2], w[3]);
    reinterpret_cast<uint4*>(p)[1] = make_uint4(w[4], w[5], w[6], w[7]);
}

// Workgroup max, then one atomic max into *out (same-address atomics serialize in L2, so callers keep
// the number of workgroups that do this small).
template <int THREADS>
__device__ __forceinline__ void block_reduce_atomic(uint32_t m, float* out) {
    constexpr int NW = THREADS / 64;
    __shared__ uint32_t red[NW];
    m = wave_max_u32(m);
    if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = m;
    __syncthreads();
    if (threadIdx.x == 0) {
        uint32_t b = red[0];
#pragma unroll
        for (int w = 1; w < NW; ++w) b = max(b, red[w]);
        atomicMax(reinterpret_cast<uint32_t*>(out), b);
    }
}

// ------------------------------------------------------------------ row kernel
// Output = input layout (rows x cols), cols % 32 == 0 (BLOCK: cols % 128 == 0).
template <int FMT, int MODE, bool BF16, bool FUSED_AMAX, bool DERIVE, int THREADS>
__global__ __launch_bounds__(THREADS) void cast_rows_kernel(CastArgs a) {
    const UniformScale u = uniform_scale<FMT, MODE, DERIVE, BF16>(a);
    const int64_t cpr = a.cols / 32;
    const int64_t total = a.rows * cpr;
    const size_t esz = BF16 ? 2 : 4;
    uint32_t tmax = 0;
    for (int64_t base = (int64_t)blockIdx.x * THREADS; base < total; base += (int64_t)gridDim.x * THREADS) {
        const int64_t g = base + threadIdx.x;
        const bool valid = g < total;
        const int64_t gg = valid ? g : total - 1;
        const int64_t r = gg / cpr, c = gg - r * cpr;
        const char* src = static_cast<const char*>(a.x) + (r * a.ld + c * 32) * esz;
        float v[32];
        uint32_t out[8], sc = 0, cm = 0;
        if constexpr (BF16) {
            // max and min of |x| from the packed words (one 16-bit op per two values)
            uint32_t w[16];
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const uint4 q = reinterpret_cast<const uint4*>(src)[j];
                w[4 * j] = q.x;
                w[4 * j + 1] = q.y;
                w[4 * j + 2] = q.z;
                w[4 * j + 3] = q.w;
            }
#pragma unroll
            for (int q = 0; q < 16; ++q) { v[2 * q] = bf16lo(w[q]); v[2 * q + 1] = bf16hi(w[q]); }
            cm = bf16w_absmax<16>(w);
            const uint32_t mn = bf16w_minm1<16>(w);
            process_chunk_mm<FMT, MODE, BF16>(v, cm, &mn, u, out, sc);
        } else {
#pragma unroll
            for (int j = 0; j < 4; ++j) load8<BF16>(src + j * 8 * esz, v + 8 * j);
            process_chunk<FMT, MODE, BF16>(v, u, out, sc, cm);
        }
        if (valid) {
            store32(a.q + r * a.ldq + c * 32, out);
            if (MODE == kModeBlock) {
                if ((threadIdx.x & 3) == 0) reinterpret_cast<uint32_t*>(a.scales)[r * (a.cols / 128) + c / 4] = sc;
            } else if (MODE == kModeMX || MODE == kModeMoss) {
                reinterpret_cast<uint8_t*>(a.scales)[r * cpr + c] = (uint8_t)sc;
            }
            tmax = max(tmax, cm);
        }
    }
    if (FUSED_AMAX) block_reduce_atomic<THREADS>(tmax, a.amax_out);
}

// ------------------------------------------------------------------ transposing kernel
// Tile of 128 input rows x 64 input columns through LDS, 256 threads; output row = input column.
// rows % 32 == 0 (BLOCK 1x128: rows % 128 == 0), cols % 8 == 0.  Thread t then owns output chunk
// (oc, seg): output row c0 + oc, K values r0 + 32 seg .. +31, so every output row gets 128
// contiguous bytes from one workgroup.  (A 128 x 128 tile with 512 threads, which also makes the
// dual cast's row-grouped stores whole lines, measured slower.)
//
// bf16 input: the tile is kept as raw bf16 pairs.  Word (c, m) holds rows 2m (low half) and 2m + 1
// (high half) of column c, at 4-byte index c * 64 + (m ^ 4 h(c)), h(c) = (c ^ c / 8) mod 8: an XOR
// of whole 16-byte groups, so a chunk is still four aligned 16-byte reads.  A load item is a row
// pair of one 8-column group; a half-wave covers 8 column groups x 4 row pairs, whose eight packed
// words per column land in 32 different banks, and the eight lanes of each 16-byte read pass hit
// eight different bank groups.
// fp32 input: word r * 69 + c + 4 (c / 32) + 8 (r / 32) for element (r, c); pitch 69 and the two
// offsets make both the row writes and the column reads conflict free.
constexpr int kTPitch = 69;
__device__ __forceinline__ int tile_word(int r, int c) { return r * kTPitch + c + ((c >> 5) << 2) + ((r >> 5) << 3); }
constexpr int kTileWords = 127 * kTPitch + 63 + 4 + 24 + 1;
__device__ __forceinline__ int pair_word(int c, int m) { return c * 64 + (m ^ (((c ^ (c >> 3)) & 7) << 2)); }
constexpr int kTileCols = 64, kTileThreads = 256;

// Row-grouped cast of 8 values of one row inside the transposed kernel's load phase (dual cast):
// the 32-group is the four lanes l ^ 0..3; all lanes call this together.
template <int FMT, int MODE, bool BF16>
__device__ __forceinline__ void dual_row8(const float* v8, int64_t row, int64_t c, const UniformScale& u, const CastArgs& a) {
    const uint32_t lmx = chunk_max<8>(v8);
    uint32_t g = lmx;
    g = max(g, (uint32_t)__shfl_xor((int)g, 1, 64));
    g = max(g, (uint32_t)__shfl_xor((int)g, 2, 64));
    uint32_t o[2], sc = 0;
    cast_group<FMT, MODE, BF16, 8>(v8, g, lmx, u, o, sc);
    if (row < a.rows && c < a.cols) {
        *reinterpret_cast<uint2*>(a.q2 + row * a.ldq2 + c) = make_uint2(o[0], o[1]);
        if ((MODE == kModeMX || MODE == kModeMoss) && (c & 31) == 0)
            reinterpret_cast<uint8_t*>(a.scales2)[row * (a.cols / 32) + c / 32] = (uint8_t)sc;
    }
}

template <int FMT, int MODE, bool BF16, bool FUSED_AMAX, bool DERIVE, bool DUAL>
__global__ __launch_bounds__(kTileThreads) void cast_transposed_kernel(CastArgs a) {
    constexpr int TC = kTileCols, NT = kTileThreads;
    __shared__ __attribute__((aligned(16))) uint32_t tile[BF16 ? TC * 64 : kTileWords];
    const UniformScale u = uniform_scale<FMT, MODE, DERIVE, BF16>(a);
    // Block order: groups of `tile_group` row bands; inside a group consecutive workgroups walk down
    // the bands of one column strip before moving to the next strip.
    const int64_t ntx = (a.cols + TC - 1) / TC, nty = (a.rows + 127) / 128;
    const int64_t gy = a.tile_group;
    const int64_t lin = blockIdx.x;
    const int64_t grp = lin / (gy * ntx), in = lin - grp * gy * ntx;
    const int64_t gh = min(gy, nty - grp * gy);
    const int64_t r0 = (grp * gy + in % gh) * 128, c0 = (in / gh) * TC;
    const int t = threadIdx.x;
    const int oc = ((t >> 5) << 3) | (t & 7), seg = (t >> 3) & 3;
    float v[32];
    if constexpr (BF16) {
        const uint16_t* x = static_cast<const uint16_t*>(a.x);
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            const int it = t + NT * j, cg = it & 7, m = it >> 3;
            const int64_t r = r0 + 2 * m, c = c0 + 8 * cg;
            uint4 lo = make_uint4(0u, 0u, 0u, 0u), hi = lo;
            if (c < a.cols) {
                if (r < a.rows) lo = *reinterpret_cast<const uint4*>(x + r * a.ld + c);
                if (r + 1 < a.rows) hi = *reinterpret_cast<const uint4*>(x + (r + 1) * a.ld + c);
            }
            const uint32_t wl[4] = {lo.x, lo.y, lo.z, lo.w}, wh[4] = {hi.x, hi.y, hi.z, hi.w};
            if constexpr (DUAL) {
                float v8[8];
#pragma unroll
                for (int k = 0; k < 4; ++k) { v8[2 * k] = bf16lo(wl[k]); v8[2 * k + 1] = bf16hi(wl[k]); }
                dual_row8<FMT, MODE, BF16>(v8, r, c, u, a);
#pragma unroll
                for (int k = 0; k < 4; ++k) { v8[2 * k] = bf16lo(wh[k]); v8[2 * k + 1] = bf16hi(wh[k]); }
                dual_row8<FMT, MODE, BF16>(v8, r + 1, c, u, a);
            }
#pragma unroll
            for (int k = 0; k < 4; ++k) {
                // column 8cg+2k: low halves of both rows; column 8cg+2k+1: high halves
                tile[pair_word(8 * cg + 2 * k, m)] = __builtin_amdgcn_perm(wh[k], wl[k], 0x05040100u);
                tile[pair_word(8 * cg + 2 * k + 1, m)] = __builtin_amdgcn_perm(wh[k], wl[k], 0x07060302u);
            }
        }
        __syncthreads();
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const uint4 w = *reinterpret_cast<const uint4*>(&tile[pair_word(oc, seg * 16 + 4 * i)]);
            const uint32_t ww[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
            for (int d = 0; d < 4; ++d) {
                v[8 * i + 2 * d] = bf16lo(ww[d]);
                v[8 * i + 2 * d + 1] = bf16hi(ww[d]);
            }
        }
    } else {
        float* tf = reinterpret_cast<float*>(tile);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int ch = t + 256 * i;
            const int rr = ch >> 3, cc = (ch & 7) * 8;
            float w[8];
            if (r0 + rr < a.rows && c0 + cc < a.cols) {
                load8<false>(static_cast<const float*>(a.x) + (r0 + rr) * a.ld + c0 + cc, w);
            } else {
#pragma unroll
                for (int k = 0; k < 8; ++k) w[k] = 0.0f;
            }
            if constexpr (DUAL) dual_row8<FMT, MODE, BF16>(w, r0 + rr, c0 + cc, u, a);
#pragma unroll
            for (int k = 0; k < 8; ++k) tf[tile_word(rr, cc + k)] = w[k];
        }
        __syncthreads();
#pragma unroll
        for (int j = 0; j < 32; ++j) v[j] = tf[tile_word(seg * 32 + j, oc)];
    }
    uint32_t out[8], sc = 0, cm = 0;
    process_chunk<FMT, MODE, BF16, 8>(v, u, out, sc, cm);
    const int64_t orow = c0 + oc, k0 = r0 + seg * 32;
    if (orow < a.cols && k0 < a.rows) {
        store32(a.q + orow * a.ldq + k0, out);
        if (MODE == kModeBlock) {
            if (seg == 0) reinterpret_cast<uint32_t*>(a.scales)[orow * (a.rows / 128) + r0 / 128] = sc;
        } else if (MODE == kModeMX || MODE == kModeMoss) {
            reinterpret_cast<uint8_t*>(a.scales)[orow * (a.rows / 32) + k0 / 32] = (uint8_t)sc;
        }
    }
    if (FUSED_AMAX) block_reduce_atomic<NT>(cm, a.amax_out);
}

// ------------------------------------------------------------------ dual cast over band runs
// Both copies of a bf16 tensor with rows % 128 == 0 and cols % 64 == 0, one pass.
//
// A workgroup walks NB consecutive 128-row bands of one 64-column strip and loads band b + 1 into
// registers while it casts band b (two LDS tiles, one barrier per band).  Lane t holds 32
// consecutive values of row t / 2 (columns 32 (t % 2) ..), so the row-grouped copy casts whole
// 32-groups from registers with no cross-lane work.  For the transposed copy the two rows of a
// pair are merged into bf16-pair words (the layout of the transposing kernel above): the lanes of
// rows 2m and 2m + 1 (t and t ^ 2) swap half of their words with one DPP move each and every lane
// writes 16 pair words.  Odd-row lanes load their two 16-column halves in swapped order, so that
// the words they keep and the words they send sit in the same registers as on even-row lanes.
//
// The transposed copy's E8M0 bytes of the strip's 64 output rows are collected in LDS and written
// once per run, 4 * NB contiguous bytes per output row: written band by band they are 4-byte
// pieces of lines that workgroups on other XCDs also write, and such partial lines reach HBM
// several times over.  Workgroup w runs on XCD w % 8 (round-robin dispatch); XCD x takes whole band
// runs x, x + 8, ... with all their strips, so the row-grouped copy's lines and its scale lines
// are completed inside one L2.
template <int FMT, int MODE, bool FUSED_AMAX, bool DERIVE, int NB>
__global__ __launch_bounds__(kTileThreads) void cast_dual_run_kernel(CastArgs a) {
    static_assert(MODE == kModeTensor || MODE == kModeMX || MODE == kModeMoss, "dual casts: TENSOR, MX, MOSS");
    constexpr int TC = kTileCols, NT = kTileThreads;
    __shared__ __attribute__((aligned(16))) uint32_t tile[2][TC * 64];
    __shared__ __attribute__((aligned(16))) uint8_t tsc[TC][4 * NB];
    const int64_t ntx = a.cols / TC, nty = a.rows / 128, nruns = (nty + NB - 1) / NB;
    const int64_t w = blockIdx.x, k = w / 8;
    const int64_t run = w % 8 + 8 * (k / ntx), strip = k % ntx;
    if (run >= nruns) return;                       // whole workgroup; no barrier reached yet
    const UniformScale u = uniform_scale<FMT, MODE, DERIVE, true>(a);
    const int64_t b0 = run * NB, b1 = min(nty, b0 + NB), c0 = strip * TC;
    const int t = threadIdx.x;
    const int rr = t >> 1, h = t & 1, odd = (t >> 1) & 1, m = t >> 2;
    const int oc = ((t >> 5) << 3) | (t & 7), seg = (t >> 3) & 3;
    // register slot i holds columns 32 h + 8 (i ^ 2 odd) .. + 7
    const uint16_t* xrow = static_cast<const uint16_t*>(a.x) + (int64_t)rr * a.ld + c0 + 32 * h;
    auto load = [&](int64_t band, uint4* v) {
        const uint16_t* p = xrow + band * 128 * a.ld;
#pragma unroll
        for (int i = 0; i < 4; ++i) v[i] = *reinterpret_cast<const uint4*>(p + 8 * (i ^ (2 * odd)));
    };
    // v_perm selectors: pair word = (even row value, odd row value) of one column
    const uint32_t sel_lo = odd ? 0x01000504u : 0x05040100u, sel_hi = odd ? 0x03020706u : 0x07060302u;
    // the 16 columns whose pair words this lane writes: 32 h + 16 odd + 0 .. 15
    const int cw = 32 * h + 16 * odd;
    uint4 cur[4], nxt[4];
    load(b0, cur);
    uint32_t tmax = 0;
    int buf = 0;
    for (int64_t band = b0; band < b1; ++band) {
        // unconditional (the last band reloads itself): a conditional prefetch makes the compiler
        // wait for every outstanding load at the top of the loop
        load(band + 1 < b1 ? band + 1 : band, nxt);
        uint32_t* tl = tile[buf];
        const uint32_t wv[16] = {cur[0].x, cur[0].y, cur[0].z, cur[0].w, cur[1].x, cur[1].y, cur[1].z, cur[1].w,
                                 cur[2].x, cur[2].y, cur[2].z, cur[2].w, cur[3].x, cur[3].y, cur[3].z, cur[3].w};
        // transposed copy: keep words 0..7, send words 8..15 to the partner row's lane
#pragma unroll
        for (int q = 0; q < 8; ++q) {
            const uint32_t got = (uint32_t)__builtin_amdgcn_mov_dpp((int)wv[8 + q], 0x4E, 0xF, 0xF, false);
            tl[pair_word(cw + 2 * q, m)] = __builtin_amdgcn_perm(got, wv[q], sel_lo);
            tl[pair_word(cw + 2 * q + 1, m)] = __builtin_amdgcn_perm(got, wv[q], sel_hi);
        }
        // row-grouped copy: one 32-group per lane
        {
            float v[32];
#pragma unroll
            for (int q = 0; q < 16; ++q) { v[2 * q] = bf16lo(wv[q]); v[2 * q + 1] = bf16hi(wv[q]); }
            uint32_t out[8], sc = 0;
            const uint32_t cm = bf16w_absmax<16>(wv), mn = bf16w_minm1<16>(wv);
            cast_group<FMT, MODE, true, 32>(v, cm, cm, u, out, sc, &mn);
            const int64_t r = band * 128 + rr;
            uint8_t* dst = a.q2 + r * a.ldq2 + c0 + 32 * h;
            *reinterpret_cast<uint4*>(dst + 16 * odd) = make_uint4(out[0], out[1], out[2], out[3]);
            *reinterpret_cast<uint4*>(dst + 16 - 16 * odd) = make_uint4(out[4], out[5], out[6], out[7]);
            if (MODE == kModeMX || MODE == kModeMoss)
                reinterpret_cast<uint8_t*>(a.scales2)[r * (a.cols / 32) + (c0 + 32 * h) / 32] = (uint8_t)sc;
            tmax = max(tmax, cm);
        }
        // one barrier per band: the other tile was last read before this barrier's previous instance
        __syncthreads();
        {
            float v[32];
            uint32_t pw[16];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const uint4 q4 = *reinterpret_cast<const uint4*>(&tl[pair_word(oc, seg * 16 + 4 * i)]);
                pw[4 * i] = q4.x;
                pw[4 * i + 1] = q4.y;
                pw[4 * i + 2] = q4.z;
                pw[4 * i + 3] = q4.w;
            }
#pragma unroll
            for (int q = 0; q < 16; ++q) { v[2 * q] = bf16lo(pw[q]); v[2 * q + 1] = bf16hi(pw[q]); }
            uint32_t out[8], sc = 0;
            const uint32_t cm = bf16w_absmax<16>(pw), mn = bf16w_minm1<16>(pw);
            cast_group<FMT, MODE, true, 32>(v, cm, cm, u, out, sc, &mn);
            store32(a.q + (c0 + oc) * a.ldq + band * 128 + seg * 32, out);
            if (MODE == kModeMX || MODE == kModeMoss) tsc[oc][4 * (band - b0) + seg] = (uint8_t)sc;
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) cur[i] = nxt[i];
        buf ^= 1;
    }
    if (MODE == kModeMX || MODE == kModeMoss) {
        __syncthreads();
        const int nb = (int)(b1 - b0);
        uint8_t* dst = reinterpret_cast<uint8_t*>(a.scales) + c0 * (a.rows / 32) + b0 * 4;
        for (int i = t; i < TC * nb; i += NT) {
            const int row = i / nb, pc = i - row * nb;
            *reinterpret_cast<uint32_t*>(dst + row * (a.rows / 32) + pc * 4) =
                *reinterpret_cast<const uint32_t*>(&tsc[row][pc * 4]);
        }
    }
    if (FUSED_AMAX) block_reduce_atomic<NT>(tmax, a.amax_out);
}

// ------------------------------------------------------------------ 128x128 weight blocks
// One workgroup per 128x128 block (non-transposed, rows % 128 == 0, cols % 128 == 0), the block in
// registers; block amax via LDS; one pass over HBM.  Sixteen consecutive lanes cover one row's 128
// values (8 each), so every load and store instruction reads or writes whole row segments; thread
// t holds columns 8 (t % 16) .. +8 of rows t / 16 + (NT / 16) j, j < 2048 / NT.
template <int FMT, bool BF16, bool E8, int NT = 512>
__global__ __launch_bounds__(NT) void cast_block128_kernel(CastArgs a) {
    constexpr int RPT = 128 * 16 / NT;            // rows per thread, NT / 16 rows apart
    constexpr int NW = NT / 64;
    const int64_t br = blockIdx.y, bc = blockIdx.x;
    const int t = threadIdx.x;
    const int64_t r0 = br * 128 + (t >> 4), c = bc * 128 + (t & 15) * 8;
    const size_t esz = BF16 ? 2 : 4;
    const char* src = static_cast<const char*>(a.x) + (r0 * a.ld + c) * esz;
    // bf16 input stays packed (two values per word) until its cast, which halves the registers the
    // block takes and lets every workgroup of a 2048 x 7168 weight be resident at once
    constexpr int VW = BF16 ? 4 : 8;              // registers per 8 values
    uint32_t raw[VW * RPT];
#pragma unroll
    for (int j = 0; j < RPT; ++j) {
        const uint4* p = reinterpret_cast<const uint4*>(src + (int64_t)j * (NT / 16) * a.ld * esz);
        const uint4 q0 = p[0];
        raw[VW * j] = q0.x;
        raw[VW * j + 1] = q0.y;
        raw[VW * j + 2] = q0.z;
        raw[VW * j + 3] = q0.w;
        if (!BF16) {
            const uint4 q1 = p[1];
            raw[VW * j + 4] = q1.x;
            raw[VW * j + 5] = q1.y;
            raw[VW * j + 6] = q1.z;
            raw[VW * j + 7] = q1.w;
        }
    }
    // the 8 values of row slot j as fp32
    auto unpack = [&](int j, float* v8) {
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            if (BF16) {
                v8[2 * q] = bf16lo(raw[VW * j + q]);
                v8[2 * q + 1] = bf16hi(raw[VW * j + q]);
            } else {
                v8[2 * q] = __uint_as_float(raw[VW * j + 2 * q]);
                v8[2 * q + 1] = __uint_as_float(raw[VW * j + 2 * q + 1]);
            }
        }
    };
    uint32_t mj[RPT];
#pragma unroll
    for (int j = 0; j < RPT; ++j) {
        if (BF16) {
            mj[j] = bf16w_absmax<4>(raw + VW * j);
        } else {
            float v8[8];
            unpack(j, v8);
            mj[j] = chunk_max<8>(v8);
        }
    }
    uint32_t m = 0;
#pragma unroll
    for (int j = 0; j < RPT; ++j) m = max(m, mj[j]);
    m = wave_max_u32(m);
    __shared__ uint32_t red[NW];
    if ((t & 63) == 0) red[t >> 6] = m;
    __syncthreads();
    uint32_t bm = red[0];
#pragma unroll
    for (int w = 1; w < NW; ++w) bm = max(bm, red[w]);
    uint32_t out[2 * RPT];
    if constexpr (E8) {
        // power-of-two block scale: the MX exponent rule over the whole block, exact scaling
        const int e = mx_exponent<FMT>(__uint_as_float(bm));
#pragma unroll
        for (int j = 0; j < RPT; ++j) {
            float v8[8];
            unpack(j, v8);
            cast_mx<FMT, 8>(v8, -e, mj[j] > 0x7F800000u, out + 2 * j);
        }
        if (t == 0) reinterpret_cast<uint8_t*>(a.scales)[br * (a.cols / 128) + bc] = (uint8_t)(e + 127);
    } else {
        const float s = scale_from_amax<FMT>(__uint_as_float(bm), 1.0f);
        const float y = recip_rn(s);
        const bool sok = divisor_ok(s);
#pragma unroll
        for (int j = 0; j < RPT; ++j) {
            float v8[8];
            unpack(j, v8);
            const uint32_t mn = BF16 ? bf16w_minm1<4>(raw + VW * j) : chunk_min_m1<8>(v8);
            cast_div<FMT, false, 8>(v8, s, y, 0, sok && dividends_ok(mj[j], mn), out + 2 * j);
        }
        if (t == 0) reinterpret_cast<float*>(a.scales)[br * (a.cols / 128) + bc] = s;
    }
    uint8_t* dst = a.q + r0 * a.ldq + c;
#pragma unroll
    for (int j = 0; j < RPT; ++j)
        *reinterpret_cast<uint2*>(dst + (int64_t)j * (NT / 16) * a.ldq) = make_uint2(out[2 * j], out[2 * j + 1]);
}

// ------------------------------------------------------------------ generic exact fallback
// One workgroup per output block (br x bc in output coordinates; TENSOR uses 1 x 256 tiles,
// MX/MOSS 1 x 32).  Scalar loads, IEEE division, ragged edges with ceil semantics.
template <int FMT, int MODE, bool BF16, bool FUSED_AMAX, bool DERIVE>
__global__ __launch_bounds__(256) void cast_generic_kernel(CastArgs a, int br, int bc) {
    const int64_t R = a.transpose ? a.cols : a.rows;   // output rows
    const int64_t K = a.transpose ? a.rows : a.cols;   // output cols
    const int64_t nbc = (K + bc - 1) / bc;
    const int64_t bi = blockIdx.y, bj = blockIdx.x;
    const int64_t rb = bi * br, kb = bj * bc;
    const int64_t rn = min((int64_t)br, R - rb), kn = min((int64_t)bc, K - kb);
    const int64_t n = rn * kn;
    auto load = [&](int64_t i) -> float {
        const int64_t orow = rb + i / kn, ok = kb + i % kn;
        const int64_t ir = a.transpose ? ok : orow, ic = a.transpose ? orow : ok;
        const int64_t idx = ir * a.ld + ic;
        if (BF16) return bf16lo(static_cast<const uint16_t*>(a.x)[idx]);
        return static_cast<const float*>(a.x)[idx];
    };
    __shared__ uint32_t red[4];
    uint32_t m = 0;
    for (int64_t i = threadIdx.x; i < n; i += 256) m = max(m, absbits(load(i)));
    m = wave_max_u32(m);
    if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = m;
    __syncthreads();
    const uint32_t bm = max(max(red[0], red[1]), max(red[2], red[3]));
    const float bamax = __uint_as_float(bm);
    float s = 1.0f;
    int shift = 0;
    if (MODE == kModeTensor) {
        s = DERIVE ? scale_from_amax<FMT>(*a.amax_in, 1.0f) : *a.scale_in;
        if (DERIVE && bi == 0 && bj == 0 && threadIdx.x == 0) *a.scale_out = s;
    } else if (MODE == kModeBlock) {
        s = scale_from_amax<FMT>(bamax, 1.0f);
        if (threadIdx.x == 0) reinterpret_cast<float*>(a.scales)[bi * nbc + bj] = s;
    } else if (MODE == kModeMX || MODE == kModeBlockE8) {
        int e = mx_exponent<FMT>(bamax);
        shift = -e;
        if (threadIdx.x == 0) reinterpret_cast<uint8_t*>(a.scales)[bi * nbc + bj] = (uint8_t)(e + 127);
    } else {
        s = DERIVE ? scale_from_amax<FMT>(*a.amax_in, 1.0f) : *a.scale_in;
        if (DERIVE && bi == 0 && bj == 0 && threadIdx.x == 0) *a.scale_out = s;
        int e = moss_exponent(s, bamax / fmt_max<FMT>());
        shift = -e;
        if (threadIdx.x == 0) reinterpret_cast<uint8_t*>(a.scales)[bi * nbc + bj] = (uint8_t)(e + 127);
    }
    for (int64_t i = threadIdx.x; i < n; i += 256) {
        float x = load(i);
        float v = (MODE == kModeMX || MODE == kModeBlockE8) ? x : x / s;
        v = __builtin_amdgcn_ldexpf(v, shift);
        a.q[(rb + i / kn) * a.ldq + kb + i % kn] = (uint8_t)code_slow<FMT>(v);
    }
    if (FUSED_AMAX && threadIdx.x == 0) atomicMax(reinterpret_cast<uint32_t*>(a.amax_out), bm);
}

// ------------------------------------------------------------------ small tensors, current scaling
// Per-tensor current scaling of a tensor of at most kSmallElems elements in one workgroup: the
// amax, the scale fl(amax / MAX) and the cast in one launch instead of three (zero, amax, cast),
// which is what such a tensor's time consists of.  IEEE division and the exact encoder, as in the
// generic kernel; either output layout, or both (dual cast, q2 set).
template <int FMT, bool BF16>
__global__ __launch_bounds__(1024) void cast_small_current_kernel(CastArgs a) {
    const int64_t n = a.rows * a.cols;
    auto load = [&](int64_t i) -> float {
        const int64_t r = i / a.cols, c = i - r * a.cols;
        if (BF16) return bf16lo(static_cast<const uint16_t*>(a.x)[r * a.ld + c]);
        return static_cast<const float*>(a.x)[r * a.ld + c];
    };
    uint32_t m = 0;
    for (int64_t i = threadIdx.x; i < n; i += 1024) m = max(m, absbits(load(i)));
    __shared__ uint32_t red[16];
    m = wave_max_u32(m);
    if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = m;
    __syncthreads();
    uint32_t bm = 0;
#pragma unroll
    for (int w = 0; w < 16; ++w) bm = max(bm, red[w]);
    const float s = scale_from_amax<FMT>(__uint_as_float(bm), 1.0f);
    if (threadIdx.x == 0) {
        reinterpret_cast<uint32_t*>(a.amax_out)[0] = bm;
        *a.scale_out = s;
    }
    for (int64_t i = threadIdx.x; i < n; i += 1024) {
        const int64_t r = i / a.cols, c = i - r * a.cols;
        const uint8_t code = (uint8_t)code_slow<FMT>(load(i) / s);
        if (a.transpose) a.q[c * a.ldq + r] = code;
        else a.q[r * a.ldq + c] = code;
        if (a.q2) a.q2[r * a.ldq2 + c] = code;     // dual cast: the row-layout copy as well
    }
}

int launch_cast_small_current(const CastArgs& a, hipStream_t st) {
    if (a.fmt == kE4M3) {
        if (a.bf16) hipLaunchKernelGGL((cast_small_current_kernel<kE4M3, true>), dim3(1), dim3(1024), 0, st, a);
        else hipLaunchKernelGGL((cast_small_current_kernel<kE4M3, false>), dim3(1), dim3(1024), 0, st, a);
    } else {
        if (a.bf16) hipLaunchKernelGGL((cast_small_current_kernel<kE5M2, true>), dim3(1), dim3(1024), 0, st, a);
        else hipLaunchKernelGGL((cast_small_current_kernel<kE5M2, false>), dim3(1), dim3(1024), 0, st, a);
    }
    return 0;
}

// ------------------------------------------------------------------ dispatch
template <int FMT, int MODE, bool BF16, bool FUSED, bool DERIVE>
static void dispatch_shape(const CastArgs& a, hipStream_t st) {
    const int64_t R = a.transpose ? a.cols : a.rows;
    const int64_t K = a.transpose ? a.rows : a.cols;
    if (R == 0 || K == 0) return;
    if (!a.vec_out) {
        int br = 1, bc = 32;
        if (MODE == kModeTensor) { br = 1; bc = 256; }
        if (MODE == kModeBlock || MODE == kModeBlockE8) { br = a.block_r; bc = a.block_c; }
        dim3 grid((unsigned)((K + bc - 1) / bc), (unsigned)((R + br - 1) / br));
        hipLaunchKernelGGL((cast_generic_kernel<FMT, MODE, BF16, FUSED, DERIVE>), grid, dim3(256), 0, st, a, br, bc);
        return;
    }
    const bool block128 = (MODE == kModeBlock || MODE == kModeBlockE8) && a.block_r == 128 && a.block_c == 128;
    if (!a.transpose && block128 && !FUSED && a.rows % 128 == 0 && a.cols % 128 == 0) {
        hipLaunchKernelGGL((cast_block128_kernel<FMT, BF16, MODE == kModeBlockE8, 512>),
                           dim3((unsigned)(a.cols / 128), (unsigned)(a.rows / 128)), dim3(512), 0, st, a);
        return;
    }
    if constexpr (MODE == kModeBlockE8) {
        // other UE8M0 block shapes and transposed outputs: the exact per-block kernel
        dim3 grid((unsigned)((K + a.block_c - 1) / a.block_c), (unsigned)((R + a.block_r - 1) / a.block_r));
        hipLaunchKernelGGL((cast_generic_kernel<FMT, MODE, BF16, FUSED, DERIVE>), grid, dim3(256), 0, st, a, a.block_r,
                           a.block_c);
        return;
    } else {
    const bool row_group_ok = MODE != kModeBlock || (a.block_r == 1 && a.block_c == 128);
    if (!a.transpose) {
        const int64_t kmod = MODE == kModeBlock ? 128 : 32;
        if (row_group_ok && a.cols % kmod == 0) {
            const int64_t total = a.rows * (a.cols / 32);
            if (FUSED) {
                // few large workgroups: each ends with one atomic on the same address
                int64_t blocks = (total + 1023) / 1024;
                if (blocks > kMaxReduceBlocks) blocks = kMaxReduceBlocks;
                hipLaunchKernelGGL((cast_rows_kernel<FMT, MODE, BF16, FUSED, DERIVE, 1024>), dim3((unsigned)blocks),
                                   dim3(1024), 0, st, a);
            } else {
                int64_t blocks = (total + 255) / 256;
                if (blocks > 8192) blocks = 8192;
                hipLaunchKernelGGL((cast_rows_kernel<FMT, MODE, BF16, FUSED, DERIVE, 256>), dim3((unsigned)blocks),
                                   dim3(256), 0, st, a);
            }
            return;
        }
    } else {
        const int64_t kmod = MODE == kModeBlock ? 128 : 32;
        if (row_group_ok && a.rows % kmod == 0 && a.cols % 8 == 0) {
            CastArgs b = a;
            if (b.tile_group <= 0) b.tile_group = 8;
            const int64_t tiles = ((a.cols + kTileCols - 1) / kTileCols) * ((a.rows + 127) / 128);
            hipLaunchKernelGGL((cast_transposed_kernel<FMT, MODE, BF16, FUSED, DERIVE, false>), dim3((unsigned)tiles),
                               dim3(kTileThreads), 0, st, b);
            return;
        }
    }
    int br = 1, bc = 32;
    if (MODE == kModeTensor) { br = 1; bc = 256; }
    if (MODE == kModeBlock) { br = a.block_r; bc = a.block_c; }
    dim3 grid((unsigned)((K + bc - 1) / bc), (unsigned)((R + br - 1) / br));
    hipLaunchKernelGGL((cast_generic_kernel<FMT, MODE, BF16, FUSED, DERIVE>), grid, dim3(256), 0, st, a, br, bc);
    }
}

template <int FMT, int MODE, bool BF16>
static void dispatch_flags(const CastArgs& a, hipStream_t st) {
    const bool derive = a.amax_in != nullptr;
    const bool fused = a.amax_out != nullptr && MODE == kModeTensor && !derive;
    if (MODE == kModeTensor || MODE == kModeMoss) {
        if (derive) dispatch_shape<FMT, MODE, BF16, false, true>(a, st);
        else if (fused) dispatch_shape<FMT, MODE, BF16, true, false>(a, st);
        else dispatch_shape<FMT, MODE, BF16, false, false>(a, st);
    } else {
        dispatch_shape<FMT, MODE, BF16, false, false>(a, st);
    }
}

template <int FMT, int MODE>
static void dispatch_in(const CastArgs& a, hipStream_t st) {
    if (a.bf16) dispatch_flags<FMT, MODE, true>(a, st);
    else dispatch_flags<FMT, MODE, false>(a, st);
}

template <int FMT>
static void dispatch_mode(const CastArgs& a, hipStream_t st) {
    switch (a.mode) {
        case kModeTensor: dispatch_in<FMT, kModeTensor>(a, st); break;
        case kModeBlock: dispatch_in<FMT, kModeBlock>(a, st); break;
        case kModeMX: dispatch_in<FMT, kModeMX>(a, st); break;
        case kModeBlockE8: dispatch_in<FMT, kModeBlockE8>(a, st); break;
        default: dispatch_in<FMT, kModeMoss>(a, st); break;
    }
}

// ------------------------------------------------------------------ dual cast dispatch
template <int FMT, int MODE, bool BF16>
static void dual_flags(const CastArgs& a, hipStream_t st) {
    CastArgs b = a;
    if (b.tile_group <= 0) b.tile_group = 8;
    const int64_t tiles = ((a.cols + kTileCols - 1) / kTileCols) * ((a.rows + 127) / 128);
    if (tiles == 0) return;
    const dim3 grid((unsigned)tiles), blk(kTileThreads);
    const bool derive = a.amax_in != nullptr;
    const bool fused = a.amax_out != nullptr && MODE == kModeTensor && !derive;
    const bool runs = BF16 && a.rows % 128 == 0 && a.cols % kTileCols == 0 && a.rows >= 32 * 128 &&
                      ((uintptr_t)a.scales & 3) == 0;
    if constexpr (BF16) {
        if (runs) {
            // runs of 16 bands from 16384 rows up, else of 4: at least 8 runs (one per XCD)
            const int64_t nty = a.rows / 128, ntx = a.cols / kTileCols;
            const int nb = nty >= 8 * 16 ? 16 : 4;
            const int64_t nruns = (nty + nb - 1) / nb;
            const dim3 g((unsigned)(((nruns + 7) / 8) * 8 * ntx));
#define FP8Q_RUN(NBV)                                                                                              \
            if (derive) hipLaunchKernelGGL((cast_dual_run_kernel<FMT, MODE, false, true, NBV>), g, blk, 0, st, b); \
            else if (fused) hipLaunchKernelGGL((cast_dual_run_kernel<FMT, MODE, true, false, NBV>), g, blk, 0, st, b); \
            else hipLaunchKernelGGL((cast_dual_run_kernel<FMT, MODE, false, false, NBV>), g, blk, 0, st, b);
            if (nb == 16) { FP8Q_RUN(16) } else { FP8Q_RUN(4) }
#undef FP8Q_RUN
            return;
        }
    }
    if (derive) hipLaunchKernelGGL((cast_transposed_kernel<FMT, MODE, BF16, false, true, true>), grid, blk, 0, st, b);
    else if (fused) hipLaunchKernelGGL((cast_transposed_kernel<FMT, MODE, BF16, true, false, true>), grid, blk, 0, st, b);
    else hipLaunchKernelGGL((cast_transposed_kernel<FMT, MODE, BF16, false, false, true>), grid, blk, 0, st, b);
}

template <int FMT, int MODE>
static void dual_in(const CastArgs& a, hipStream_t st) {
    if (a.bf16) dual_flags<FMT, MODE, true>(a, st);
    else dual_flags<FMT, MODE, false>(a, st);
}

template <int FMT>
static void dual_mode(const CastArgs& a, hipStream_t st) {
    switch (a.mode) {
        case kModeTensor: dual_in<FMT, kModeTensor>(a, st); break;
        case kModeMX: dual_in<FMT, kModeMX>(a, st); break;
        default: dual_in<FMT, kModeMoss>(a, st); break;
    }
}

int launch_cast_dual(const CastArgs& a, hipStream_t st) {
    if (a.fmt == kE4M3) dual_mode<kE4M3>(a, st);
    else dual_mode<kE5M2>(a, st);
    return 0;
}

int launch_cast(const CastArgs& a, hipStream_t st) {
    if (a.fmt == kE4M3) dispatch_mode<kE4M3>(a, st);
    else dispatch_mode<kE5M2>(a, st);
    return 0;
}

}  // namespace fp8q
