// Block-scaled FP8 GEMM for gfx950: dense, MoE contiguous and MoE masked.
//
// Method: "The Insider Secrets Of Deepseek Discovered", passages on limited
// Tensor Core accumulation and on promotion (Figure 7(b)): each 128-wide
// K-block is accumulated on its own and then promoted into an FP32
// accumulator, the product of the two group scales being applied at that
// moment:
//     acc += P_kb * (sA[kb][m] * sB[nb][kb])        (or sB[kb][n] for 1x128 B)
// Layouts (DeepGEMM launch article, "Principais caracteristicas": dense plus
// contiguous and masked MoE groupings): A codes [rows][K], B codes [N][K],
// both K-major; A scales [K/128][rows]; C [rows][N].
//
// Two engines compute P_kb:
//   exact   (default) -- each FP8 fragment is widened to BF16 in registers
//           (exact: BF16 holds every E4M3 value) and eight chained
//           v_mfma_f32_32x32x16_bf16 form P_kb.  This MFMA adds exact
//           products with IEEE FP32 round-to-nearest, so P_kb is an
//           FP32-accurate block sum, which is what the promotion assumes.
//   fp8mfma -- two chained v_mfma_f32_32x32x64_f8f6f4 per K-block straight
//           from the FP8 codes, at twice the MFMA rate.  gfx950's FP8 MFMAs
//           add their products in groups of eight consecutive K, truncating
//           each product to 13 fractional bits below the group's largest
//           exponent (about 14 significant bits: the kind of limited
//           accumulation the pages measured on H800, here inside a single
//           instruction), so promotion every 128 cannot restore FP32 accuracy
//           and this engine is held to a looser bound.  Chosen with
//           FP8FG_GEMM_ENGINE=fp8mfma.
//
// Kernels, by what they serve:
//   gemm_wide_*   exact engine, 128x128-scaled B, N % 256 == 0: dense,
//                 contiguous and long masked buffers (256 x 256 tiles), and
//                 decode-sized masked buffers (gemm_wdec_*, 64 x 256 tiles);
//                 the promotion is folded into the MFMA accumulator (below).
//   gemm_wdect_*  the decode tile on weights in the decode-tiled layout
//                 (written by tile_weights_decode): each half-block is one
//                 contiguous 16 KB block in the stage's LDS order.
//   gemm_wmix_*   dense grids planned as 256 x 256 tiles plus 256 x 192 tail
//                 tiles, so both kinds fill whole rounds of the device's CUs.
//   gemm_big_* / gemm_dec_*   the fold kernels described next: 1x128-scaled
//                 B (Wgrad), the fp8mfma engine, and N = 128 mod 256.
//   gemm_mx_*     the MX variant (E8M0 scales applied inside the MFMA).
//
// Fold kernels.  A 512-thread workgroup computes a
// 256 (m) x 128 (n) tile of C; each of its eight waves (two per SIMD) owns a
// 64 x 64 sub-tile = 2 x 2 MFMA tiles of 32 x 32.  K-blocks stream through a
// three-stage ring in LDS filled by direct-to-LDS loads
// (global_load_lds_dwordx4: the data never passes through registers), so two
// K-blocks are in flight while a third is multiplied.  A stage holds the FP8
// A tile (256 x 128 B), the FP8 B tile (128 x 128 B), the tile's 256 A
// scales and, for 1x128-scaled B, its 128 column scales.  Rows of 128 bytes
// are stored as eight 16-byte chunks, chunk c of row r at slot
// c ^ ((r >> 1) & 7), so the 16 rows read together by a fragment load hit 16
// distinct 16-byte bank groups.  One barrier per K-block: after it, the
// stage read in the previous iteration is refilled.
//
// MFMA operands: lane l of a 32x32 fragment holds row l%32 and, per 16-byte
// LDS chunk, 16 consecutive k; A and B use the same (lane, byte) -> k map, so
// the contraction pairs matching k whatever order the instruction gives to
// (lane, element).  B's fragment is the instruction's first operand, so lane
// l ends with m = l%32 and n = 8*(i/4) + 4*(l/32) + i%4 for result i: four
// runs of four consecutive n (one A scale per lane, 8- or 16-byte stores).
#include "device_common.hpp"
#include "launch.hpp"

#include <stddef.h>
#include <stdlib.h>
#include <string.h>

namespace fp8fg {

namespace gemm_detail {

constexpr int BK = 128;           // K-block = quantization group length
constexpr int kThreads = 512;     // eight waves

// Tile shape: WAVES_M x WAVES_N waves (8 in all), each owning FM x FN MFMA
// tiles of 32 x 32.  A workgroup tile is BM x BN.
template <int WAVES_M_, int WAVES_N_, int FM_, int FN_, int STAGES_ = 3>
struct Cfg {
    static constexpr int WAVES_M = WAVES_M_, WAVES_N = WAVES_N_, FM = FM_, FN = FN_, STAGES = STAGES_;
    static constexpr int BM = WAVES_M * FM * 32, BN = WAVES_N * FN * 32;
    static constexpr int A_PER_WAVE = BM * BK / 1024 / 8;   // 1 KB direct-to-LDS pieces per wave
    static constexpr int B_PER_WAVE = BN * BK / 1024 / 8;
    static constexpr int LOADS_PER_WAVE = A_PER_WAVE + B_PER_WAVE + 1;   // + one scale piece
    static_assert(WAVES_M * WAVES_N == 8, "eight waves");
    static_assert(A_PER_WAVE * 8 * 1024 == BM * BK && B_PER_WAVE * 8 * 1024 == BN * BK, "whole pieces per wave");
    static_assert(BM / 64 + BN / 64 <= 8, "scale pieces fit in eight waves");
    static_assert(STAGES >= 3 && STAGES <= 6, "ring depth");
};
// Dense and contiguous layouts: 256 x 128 tiles, waves 4 x 2 of 64 x 64.
typedef Cfg<4, 2, 2, 2> BigTile;

// Masked (decode) layout: 64 x 128 tiles, waves 2 x 4 of 32 x 32 -- few
// valid rows per expert, so the tile is short in m and the weights stream
// through with an eighth of the big tile's A traffic.
typedef Cfg<2, 4, 1, 1, 3> DecodeTile;

typedef __bf16 v8bf __attribute__((ext_vector_type(8)));
typedef float v16f __attribute__((ext_vector_type(16)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));

typedef __attribute__((address_space(3))) void* lds_ptr_t;

template <class C>
struct alignas(16) Stage {
    uint8_t a[C::BM * BK];   // FP8 A tile, swizzled rows
    uint8_t b[C::BN * BK];   // FP8 B tile, swizzled rows
    float sa[C::BM];         // A scales of this K-block for the tile's rows
    float sb[C::BN < 128 ? 128 : C::BN];   // B column scales (1x128 B), or per 128-wide n-block
                                           // 64 copies of its block scale (128x128 B)
    float dummy[64];         // target of the padding scale loads (never read)
};

__device__ __forceinline__ int swz(int row, int chunk) { return row * BK + ((chunk ^ ((row >> 1) & 7)) << 4); }

// ---------------------------------------------------------------------------
// Tile -> (group, rows, operand pointers)
struct Tile {
    int64_t m0;           // first row of the tile in its group's row space
    int64_t rows_valid;   // rows [0, rows_valid) of that row space are real
    int64_t lda_s;        // row count of the A scale array (stride between K-blocks)
    int64_t c_base;       // element offset of the group's C block
    const uint8_t* A;
    const float* SA;
    const uint8_t* B;
    const float* SB;
    int bn;
    bool live;
};

// Masked layout: the p-th (expert, m-tile) pair in order of decreasing work --
// the number of valid 32-row sub-tiles in the pair's m-range -- or -1 for a
// pair without valid rows (those come last).  Workgroups start in index
// order as CUs free up, so the longest ones start first and the short ones
// fill in behind them.  Every wave computes the same answer: one lane per
// pair, ballots count and locate.  Past 4096 pairs the natural order is kept.
template <int BM>
__device__ __forceinline__ int64_t masked_pair_by_work(const GemmArgs& args, int64_t p) {
    constexpr int NC = BM / 32 + 1;              // classes 0 (no valid rows) .. BM / 32
    const int lane = threadIdx.x & 63;
    const int64_t m_tiles = (args.M + BM - 1) / BM, pairs = args.G * m_tiles;
    auto cls = [&](int64_t pair) -> int {
        const int64_t g = pair / m_tiles, mt = pair - g * m_tiles;
        int64_t mm = args.aux[g];
        mm = mm < 0 ? 0 : (mm > args.M ? args.M : mm);
        const int64_t rows = mm - mt * BM;
        return rows <= 0 ? 0 : int(((rows < BM ? rows : BM) + 31) / 32);
    };
    if (pairs > 4096) return cls(p) > 0 ? p : -1;
    int64_t count[NC];
#pragma unroll
    for (int k = 0; k < NC; ++k) count[k] = 0;
    for (int64_t base = 0; base < pairs; base += 64) {
        const int64_t pair = base + lane;
        const int c = pair < pairs ? cls(pair) : -1;
#pragma unroll
        for (int k = 1; k < NC; ++k) count[k] += __builtin_popcountll(__builtin_amdgcn_ballot_w64(c == k));
    }
    int target = 0;
#pragma unroll
    for (int k = NC - 1; k >= 1; --k) {
        if (target == 0) {
            if (p < count[k]) target = k;
            else p -= count[k];
        }
    }
    if (target == 0) return -1;
    for (int64_t base = 0; base < pairs; base += 64) {
        const int64_t pair = base + lane;
        const int c = pair < pairs ? cls(pair) : -1;
        uint64_t m = __builtin_amdgcn_ballot_w64(c == target);
        const int64_t n = __builtin_popcountll(m);
        if (p < n) {
            for (int64_t i = 0; i < p; ++i) m &= m - 1;   // drop the p lowest set bits
            return base + __builtin_ctzll(m);
        }
        p -= n;
    }
    return -1;
}

// tile -> operands; n-tiles cover columns [0, n_ext) (n_ext < 0: all N)
template <class C, int MODE>
__device__ __forceinline__ Tile map_tile(const GemmArgs& args, int64_t tile, int64_t n_ext = -1) {
    constexpr int BM = C::BM, BN = C::BN;
    Tile t;
    const int n_tiles = int(((n_ext < 0 ? args.N : n_ext) + BN - 1) / BN);   // a last partial n-tile when N % BN != 0
    const int64_t kbs = (args.K + BK - 1) / BK;
    if (MODE == int(GemmMode::Masked) && args.xcds > 1) {
        // Workgroup w runs on XCD w mod xcds (round-robin dispatch).  Give each
        // XCD whole (expert, m-tile) pairs -- ranks x, x + xcds, ... -- so the
        // n-tiles sharing a pair's A rows share one L2; the host sets xcds only
        // when it divides the pair count, which keeps this a bijection.
        const int64_t x = tile % args.xcds, j = tile / args.xcds;
        tile = (x + args.xcds * (j / n_tiles)) * n_tiles + j % n_tiles;
    }
    t.bn = int(tile % n_tiles);
    tile /= n_tiles;
    t.A = args.a;
    t.SA = args.sa;
    t.B = args.b;
    t.SB = args.sb;
    t.c_base = 0;
    t.live = true;
    t.lda_s = args.M;
    int64_t g = 0;
    if (MODE == int(GemmMode::Dense)) {
        t.m0 = tile * BM;
        t.rows_valid = args.M;
    } else if (MODE == int(GemmMode::Contig)) {
        // walk the groups, counting ceil(rows / BM) tiles per group, until the
        // tile's index falls inside one; the grid is sized M_total/BM + G, an
        // upper bound of the total, and the surplus tiles find no group
        int64_t base = 0;
        t.live = false;
        t.m0 = 0;
        t.rows_valid = 0;
        for (int64_t gg = 0; gg < args.G; ++gg) {
            const int64_t lo = args.aux[gg], hi = args.aux[gg + 1];
            const int64_t n = hi > lo ? (hi - lo + BM - 1) / BM : 0;
            if (tile < base + n) {
                g = gg;
                t.m0 = lo + (tile - base) * BM;
                t.rows_valid = hi < args.M ? hi : args.M;
                t.live = lo >= 0;
                break;
            }
            base += n;
        }
    } else {
        const int64_t m_tiles = (args.M + BM - 1) / BM;
        const int64_t pair = masked_pair_by_work<BM>(args, tile);
        if (pair < 0) {
            t.live = false;
            return t;
        }
        g = pair / m_tiles;
        t.m0 = (pair - g * m_tiles) * BM;
        int64_t mm = args.aux[g];
        t.rows_valid = mm < 0 ? 0 : (mm > args.M ? args.M : mm);
        t.A += g * args.M * args.K;
        t.SA += g * kbs * args.M;
        t.c_base = g * args.M * args.N;
    }
    if (t.m0 >= t.rows_valid) t.live = false;
    if (MODE != int(GemmMode::Dense)) {
        t.B += g * args.N * args.K;
        t.SB += g * ((args.N + 127) / 128) * kbs;   // 128x128 scales [G][ceil(N/128)][ceil(K/128)]
    }
    return t;
}

// ---------------------------------------------------------------------------
// Direct-to-LDS copy of one K-block into a stage.  Every wave issues exactly
// C::LOADS_PER_WAVE load instructions per K-block (so one vmcnt value fits
// all waves): its 1 KB pieces of A and of B (8 rows each) and one 256-byte
// scale piece.  Scale pieces: the first BM/64 waves load the A scales; then,
// when B is 1x128-scaled, BN/64 waves its column scales, or, when it is
// 128x128-scaled, one wave per 128-wide n-block 64 copies of that block's
// scale; the remaining waves a padding load into Stage::dummy.  Keeping every
// scale on this path leaves vmcnt counting nothing but the ring.
template <class C>
struct Copier {
    const uint8_t* a_row[C::A_PER_WAVE];   // this lane's A row start per piece
    const uint8_t* b_row[C::B_PER_WAVE];
    int a_c16[C::A_PER_WAVE], b_c16[C::B_PER_WAVE];   // the lane's chunk offset within a K-block (bytes)
    int a_lds[C::A_PER_WAVE], b_lds[C::B_PER_WAVE];   // wave-uniform LDS byte offsets
    const float* s_src;        // this lane's scale source for K-block 0
    int64_t s_stride;          // scale source stride between K-blocks
    int s_lds;                 // wave-uniform LDS byte offset of the scale piece
    int64_t K;

    // issue this wave's loads of K-block kb into `stage`; a chunk past K (a
    // partial last K-block) reads the row's first chunk instead, never memory
    // past the row, and is zeroed in LDS by zero_tail
    __device__ __forceinline__ void copy(uint8_t* stage, int64_t kb) const {
        const int64_t koff = kb * BK;
#pragma unroll
        for (int i = 0; i < C::A_PER_WAVE; ++i) {
            const int64_t off = koff + a_c16[i];
            __builtin_amdgcn_global_load_lds(a_row[i] + (off < K ? off : 0), (lds_ptr_t)(stage + a_lds[i]), 16, 0, 0);
        }
#pragma unroll
        for (int i = 0; i < C::B_PER_WAVE; ++i) {
            const int64_t off = koff + b_c16[i];
            __builtin_amdgcn_global_load_lds(b_row[i] + (off < K ? off : 0), (lds_ptr_t)(stage + b_lds[i]), 16, 0, 0);
        }
        __builtin_amdgcn_global_load_lds(s_src + kb * s_stride, (lds_ptr_t)(stage + s_lds), 4, 0, 0);
    }

    // after this wave's loads of K-block kb have landed: zero its 16-byte
    // slots that lie past K, so those k contribute nothing
    __device__ __forceinline__ void zero_tail(uint8_t* stage, int64_t kb, int lane) const {
        const int64_t koff = kb * BK;
#pragma unroll
        for (int i = 0; i < C::A_PER_WAVE; ++i)
            if (koff + a_c16[i] >= K) st<u32x4>(stage + a_lds[i] + lane * 16, u32x4{0u, 0u, 0u, 0u});
#pragma unroll
        for (int i = 0; i < C::B_PER_WAVE; ++i)
            if (koff + b_c16[i] >= K) st<u32x4>(stage + b_lds[i] + lane * 16, u32x4{0u, 0u, 0u, 0u});
    }
};

template <class C, int BSCALE_1x128>
__device__ __forceinline__ Copier<C> make_copier(const Tile& t, int wave, int lane, int64_t K, int64_t N,
                                                 int64_t n0) {
    typedef Stage<C> S;
    Copier<C> c;
    c.K = K;
    const int sub = lane >> 3;            // row within an 8-row piece
    const int slot = lane & 7;            // 16-byte slot within the row (as stored)
#pragma unroll
    for (int i = 0; i < C::A_PER_WAVE; ++i) {
        const int r0 = (wave * C::A_PER_WAVE + i) * 8, r = r0 + sub;
        const int chunk = slot ^ ((r >> 1) & 7);
        int64_t row = t.m0 + r;
        if (row >= t.rows_valid) row = t.rows_valid - 1;      // clamp: loaded, never stored
        c.a_row[i] = t.A + row * K;
        c.a_c16[i] = chunk * 16;
        c.a_lds[i] = int(offsetof(S, a)) + r0 * BK;
    }
#pragma unroll
    for (int i = 0; i < C::B_PER_WAVE; ++i) {
        const int r0 = (wave * C::B_PER_WAVE + i) * 8, r = r0 + sub;
        const int chunk = slot ^ ((r >> 1) & 7);
        const int64_t brow = n0 + r < N ? n0 + r : N - 1;       // clamp: loaded, never stored
        c.b_row[i] = t.B + brow * K;
        c.b_c16[i] = chunk * 16;
        c.b_lds[i] = int(offsetof(S, b)) + r0 * BK;
    }
    constexpr int a_waves = C::BM / 64;
    constexpr int b_waves = BSCALE_1x128 ? C::BN / 64 : (C::BN + 127) / 128;
    if (wave < a_waves) {
        int64_t row = t.m0 + wave * 64 + lane;
        if (row >= t.rows_valid) row = t.rows_valid - 1;
        c.s_src = t.SA + row;
        c.s_stride = t.lda_s;
        c.s_lds = int(offsetof(S, sa)) + wave * 64 * 4;
    } else if (wave < a_waves + b_waves) {
        const int j = wave - a_waves;
        if (BSCALE_1x128) {
            const int64_t col = n0 + j * 64 + lane;
            c.s_src = t.SB + (col < N ? col : N - 1);
            c.s_stride = N;
        } else {
            c.s_src = t.SB + (n0 / 128 + j) * ((K + BK - 1) / BK);
            c.s_stride = 1;
        }
        c.s_lds = int(offsetof(S, sb)) + j * 64 * 4;
    } else {
        c.s_src = t.SA + (t.rows_valid - 1);
        c.s_stride = t.lda_s;
        c.s_lds = int(offsetof(S, dummy));
    }
    return c;
}

// ---------------------------------------------------------------------------
// bytes 0,1 (HI = false) or 2,3 (HI = true) of w -> two BF16 values, exactly
template <bool HI>
__device__ __forceinline__ uint32_t bf16x2_of_fp8(uint32_t w) {
    return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(int(w), 1.0f, HI));
}

// 8 FP8 codes (two words) -> 8 BF16 values, an MFMA operand
__device__ __forceinline__ v8bf widen8(uint32_t w0, uint32_t w1) {
    const u32x4 v{bf16x2_of_fp8<false>(w0), bf16x2_of_fp8<true>(w0), bf16x2_of_fp8<false>(w1),
                  bf16x2_of_fp8<true>(w1)};
    return __builtin_bit_cast(v8bf, v);
}

__device__ __forceinline__ u32x4 read_chunk(const uint8_t* tile, int row, int chunk) {
    return ld<u32x4>(tile + swz(row, chunk));
}

// P_kb for the wave's FM x FN MFMA tiles from one stage.  `mlive` = number of
// leading 32-row m-tiles that hold valid rows (the others are skipped).
template <int ENGINE, int FM, int FN>
__device__ __forceinline__ void kblock_partials(const uint8_t* ta, const uint8_t* tb, int lane, int mlive,
                                                v16f (&p)[FM][FN]) {
    const int r = lane & 31, h = lane >> 5;
#pragma unroll
    for (int mi = 0; mi < FM; ++mi)
#pragma unroll
        for (int ni = 0; ni < FN; ++ni)
#pragma unroll
            for (int i = 0; i < 16; ++i) p[mi][ni][i] = 0.f;
    if (ENGINE == 0) {
        // four chunk columns j: chunk 2j + h holds k = 32j + 16h .. +15; its
        // first 8 bytes feed k-step 2j, the last 8 bytes k-step 2j + 1
        u32x4 fa[FM], fb[FN];
#pragma unroll
        for (int mi = 0; mi < FM; ++mi) fa[mi] = read_chunk(ta, mi * 32 + r, h);
#pragma unroll
        for (int ni = 0; ni < FN; ++ni) fb[ni] = read_chunk(tb, ni * 32 + r, h);
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            u32x4 na[FM], nb[FN];
            if (j + 1 < 4) {
#pragma unroll
                for (int mi = 0; mi < FM; ++mi) na[mi] = read_chunk(ta, mi * 32 + r, 2 * (j + 1) + h);
#pragma unroll
                for (int ni = 0; ni < FN; ++ni) nb[ni] = read_chunk(tb, ni * 32 + r, 2 * (j + 1) + h);
            }
#pragma unroll
            for (int half = 0; half < 2; ++half) {
                v8bf a8[FM], b8[FN];
#pragma unroll
                for (int mi = 0; mi < FM; ++mi) a8[mi] = widen8(fa[mi][2 * half], fa[mi][2 * half + 1]);
#pragma unroll
                for (int ni = 0; ni < FN; ++ni) b8[ni] = widen8(fb[ni][2 * half], fb[ni][2 * half + 1]);
#pragma unroll
                for (int mi = 0; mi < FM; ++mi) {
                    if (mi >= mlive) break;
#pragma unroll
                    for (int ni = 0; ni < FN; ++ni)
                        p[mi][ni] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(b8[ni], a8[mi], p[mi][ni], 0, 0, 0);
                }
            }
            if (j + 1 < 4) {
#pragma unroll
                for (int mi = 0; mi < FM; ++mi) fa[mi] = na[mi];
#pragma unroll
                for (int ni = 0; ni < FN; ++ni) fb[ni] = nb[ni];
            }
        }
    } else {
        // two k-steps q of 64: lane supplies chunks 4q + 2h and 4q + 2h + 1
#pragma unroll
        for (int q = 0; q < 2; ++q) {
            v8i a8[FM], b8[FN];
#pragma unroll
            for (int mi = 0; mi < FM; ++mi) {
                const u32x4 lo = read_chunk(ta, mi * 32 + r, 4 * q + 2 * h);
                const u32x4 hi = read_chunk(ta, mi * 32 + r, 4 * q + 2 * h + 1);
                a8[mi] = v8i{int(lo[0]), int(lo[1]), int(lo[2]), int(lo[3]), int(hi[0]), int(hi[1]), int(hi[2]), int(hi[3])};
            }
#pragma unroll
            for (int ni = 0; ni < FN; ++ni) {
                const u32x4 lo = read_chunk(tb, ni * 32 + r, 4 * q + 2 * h);
                const u32x4 hi = read_chunk(tb, ni * 32 + r, 4 * q + 2 * h + 1);
                b8[ni] = v8i{int(lo[0]), int(lo[1]), int(lo[2]), int(lo[3]), int(hi[0]), int(hi[1]), int(hi[2]), int(hi[3])};
            }
#pragma unroll
            for (int mi = 0; mi < FM; ++mi) {
                if (mi >= mlive) break;
#pragma unroll
                for (int ni = 0; ni < FN; ++ni)
                    // formats 0/0 = E4M3 x E4M3; zero scale operands select the
                    // plain (unscaled) instruction
                    p[mi][ni] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(b8[ni], a8[mi], p[mi][ni], 0, 0, 0,
                                                                                0, 0, 0);
            }
        }
    }
}

// s_waitcnt vmcnt(N) with N an immediate
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
    asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

// wait until at most `later` K-blocks' worth of this wave's copies are outstanding
template <class C>
__device__ __forceinline__ void wait_copies(int later) {
    constexpr int L = C::LOADS_PER_WAVE;
    switch (later) {
        case 0: wait_vmcnt<0>(); break;
        case 1: wait_vmcnt<L>(); break;
        case 2: wait_vmcnt<2 * L>(); break;
        case 3: wait_vmcnt<3 * L>(); break;
        default: wait_vmcnt<4 * L>(); break;
    }
}

template <int WAVES_M, int WAVES_N, int FM_, int FN_, int STAGES_, int ENGINE, int BSCALE_1x128, int OUT_FP32, int MODE>
__device__ __forceinline__ void gemm_body(const GemmArgs& args) {
    typedef Cfg<WAVES_M, WAVES_N, FM_, FN_, STAGES_> C;
    constexpr int FM = C::FM, FN = C::FN;
    typedef Stage<C> S;
    constexpr int STAGES = C::STAGES;
    __shared__ __align__(16) uint8_t lds_raw[STAGES * sizeof(S)];
    S* ring = reinterpret_cast<S*>(lds_raw);

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int wm = wave / C::WAVES_N, wn = wave % C::WAVES_N;
    const int64_t N = args.N, K = args.K, kbs = (K + BK - 1) / BK;   // the last K-block may be partial
    const Tile t = map_tile<C, MODE>(args, blockIdx.x);
    if (!t.live) return;
    const int64_t n0 = int64_t(t.bn) * C::BN;
    const Copier<C> cp = make_copier<C, BSCALE_1x128>(t, wave, lane, K, N, n0);
    // 32-row m-tiles of this wave that hold valid rows (0 .. FM)
    const int64_t wrow0 = t.m0 + wm * FM * 32;
    const int64_t left = t.rows_valid - wrow0;
    const int mlive = left <= 0 ? 0 : (left >= FM * 32 ? FM : int((left + 31) / 32));
    const int n_lane = wn * FN * 32 + 4 * (lane >> 5);    // + ni*32 + 8*j: first n of each run of four

#pragma unroll
    for (int st = 0; st < STAGES - 1; ++st)
        if (st < kbs) cp.copy(reinterpret_cast<uint8_t*>(&ring[st]), st);

    v16f acc[FM][FN];
#pragma unroll
    for (int mi = 0; mi < FM; ++mi)
#pragma unroll
        for (int ni = 0; ni < FN; ++ni)
#pragma unroll
            for (int i = 0; i < 16; ++i) acc[mi][ni][i] = 0.f;

    int cur = 0;
    for (int64_t kb = 0; kb < kbs; ++kb) {
        // this wave's copy of K-block kb has landed once only the loads of the
        // K-blocks issued after it (up to STAGES-2 of them) are outstanding;
        // the barrier extends that to every wave and retires all reads of the
        // stage refilled below
        const int64_t later = kbs - 1 - kb;
        wait_copies<C>(int(later < STAGES - 2 ? later : STAGES - 2));
        if ((kb + 1) * BK > K) {                  // partial last K-block (uniform)
            cp.zero_tail(reinterpret_cast<uint8_t*>(&ring[cur]), kb, lane);
            asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
        }
        __builtin_amdgcn_s_barrier();
        if (kb + STAGES - 1 < kbs) {
            const int nxt = cur == 0 ? STAGES - 1 : cur - 1;        // (kb + STAGES - 1) % STAGES
            cp.copy(reinterpret_cast<uint8_t*>(&ring[nxt]), kb + STAGES - 1);
        }
        const S& sg = ring[cur];
        if (mlive > 0) {
            v16f p[FM][FN];
            kblock_partials<ENGINE, FM, FN>(sg.a + wm * FM * 32 * BK, sg.b + wn * FN * 32 * BK, lane, mlive, p);
            float sa[FM];
#pragma unroll
            for (int mi = 0; mi < FM; ++mi) sa[mi] = sg.sa[wm * FM * 32 + mi * 32 + (lane & 31)];
#pragma unroll
            for (int ni = 0; ni < FN; ++ni) {
                if (BSCALE_1x128) {
#pragma unroll
                    for (int j = 0; j < 4; ++j) {
                        const v4f sbv = ld<v4f>(&sg.sb[n_lane + ni * 32 + 8 * j]);
#pragma unroll
                        for (int mi = 0; mi < FM; ++mi)
#pragma unroll
                            for (int e = 0; e < 4; ++e)
                                acc[mi][ni][4 * j + e] =
                                    fmaf(p[mi][ni][4 * j + e], sa[mi] * sbv[e], acc[mi][ni][4 * j + e]);
                    }
                } else {
                    // the 128-wide n-block of this n-tile (tiles never straddle one)
                    const float sb = sg.sb[((wn * FN * 32 + ni * 32) / 128) * 64];
#pragma unroll
                    for (int mi = 0; mi < FM; ++mi) {
                        const float sc = sa[mi] * sb;
#pragma unroll
                        for (int i = 0; i < 16; ++i) acc[mi][ni][i] = fmaf(p[mi][ni][i], sc, acc[mi][ni][i]);
                    }
                }
            }
        }
        cur = cur == STAGES - 1 ? 0 : cur + 1;
    }
#pragma unroll
    for (int mi = 0; mi < FM; ++mi) {
        const int64_t m = wrow0 + mi * 32 + (lane & 31);
        if (m >= t.rows_valid) continue;
#pragma unroll
        for (int ni = 0; ni < FN; ++ni)
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                // a run of four columns starts on a multiple of 4 and N % 16 == 0:
                // the run lies wholly before N or wholly after it
                if (n0 + n_lane + ni * 32 + 8 * j >= N) continue;
                const int64_t idx = t.c_base + m * N + n0 + n_lane + ni * 32 + 8 * j;
                const v4f v = v4f{acc[mi][ni][4 * j], acc[mi][ni][4 * j + 1], acc[mi][ni][4 * j + 2],
                                  acc[mi][ni][4 * j + 3]};
                if (OUT_FP32) {
                    st<v4f>(static_cast<float*>(args.c) + idx, v);
                } else {
                    const uint32_t lo = bf16_bits(v[0]) | (bf16_bits(v[1]) << 16);
                    const uint32_t hi = bf16_bits(v[2]) | (bf16_bits(v[3]) << 16);
                    st<u32x2>(static_cast<uint16_t*>(args.c) + idx, u32x2{lo, hi});
                }
            }
    }
}

// ---------------------------------------------------------------------------
// Wide exact kernel (128x128-scaled B): the promotion folded into the MFMA
// accumulator.
//
// A 64 x 64 wave tile spends more VALU time widening FP8 to BF16 (one cvt per
// two codes of both operands) and folding P_kb into the accumulator (one FMA
// per output) than its MFMAs take, and a larger wave tile leaves no registers
// for a separate P_kb next to the accumulator.  So this kernel gives each wave
// a 64 x 128 tile (2 x 4 MFMA tiles; the workgroup tile is 256 x 256) and
// lets the MFMA add every block straight into the accumulator, which is kept
// in a unit that changes at each K-block:
//     s = sA[kb][m] * sB[nb][kb] = (ma * 2^ta) * (mb * 2^tb)
//     the widening cvt multiplies A codes by 2^ta and B codes by 2^tb
//     (its scale operand contributes only its exponent: exact), so the
//     MFMAs of K-block kb add  P_kb * 2^(ta + tb)  to the accumulator;
//     the accumulator holds  acc / u_kb  with  u_kb = ma * mb,  so before
//     K-block kb it is multiplied by u_(kb-1) / u_kb, and at the end by u.
// The per-element work is one multiply per K-block, as with the fold, and
// the cvts per MFMA drop by a third.  ta and tb are the scales' exponents,
// clamped only to the range where the cvt is exact, so the mantissa parts
// are at least 1 for every normal scale: the accumulator then never exceeds
// |C| and cannot overflow where C does not (subnormal scales give parts down
// to 2^-25).  Products of two widened codes are the true products times
// 2^-(log2 u): they fall below FP32's normal range only when the scale
// product itself is below about 2^-108, i.e. for blocks whose every
// contribution is smaller than 2^-80 in magnitude.
//
// Stages hold half a K-block (64 K: rows of 64 bytes, four 16-byte chunks,
// chunk c of row r at slot c ^ ((r >> 2) & 3)); four of them (135 KB) keep
// three half-blocks in flight.  The scales of K-block kb ride with both of
// its halves (masked layout: with the first only, on the waves that own a
// scale piece); the first half applies them.  Copies are buffer-to-LDS loads
// whose per-lane offsets are fixed for the whole tile, the K position riding
// in the scalar offset, and each half-block is one straight-line block of
// fragment reads, cvts and MFMAs.  A row whose A scale (or the block's B
// scale) is zero reads its codes from a zeroed 64-byte line after the ring,
// so its products are +0 whatever the codes hold.
//
// Measured on this kernel: a SIMD runs its two waves' MFMAs and VALU
// instructions essentially one after the other (only about two VALU
// instructions per 32x32x16 MFMA hide under it), so the loop costs MFMA time
// plus VALU time; the cvts (3 per MFMA) and the rescale (2 per MFMA) are most
// of the latter.
// Tile configurations of the kernel: WAVES_M x WAVES_N waves, each owning
// FM x FN MFMA tiles of 32 x 32, STAGES half-block stages.
template <int WAVES_M_, int WAVES_N_, int FM_, int FN_, int STAGES_>
struct WCfg {
    static constexpr int WAVES_M = WAVES_M_, WAVES_N = WAVES_N_, FM = FM_, FN = FN_, STAGES = STAGES_;
    static constexpr int NW = WAVES_M * WAVES_N, THREADS = NW * 64;
    static constexpr int BM = WAVES_M * FM * 32, BN = WAVES_N * FN * 32, KS = 64;
    static constexpr int ROWS_PER_PIECE = 1024 / KS;                   // 16 rows per 1 KB load
    static constexpr int A_PER_WAVE = BM / ROWS_PER_PIECE / NW;
    static constexpr int B_PER_WAVE = BN / ROWS_PER_PIECE / NW;
    static constexpr int A_SCALE_WAVES = BM / 64, B_SCALE_WAVES = BN / 128;
    static_assert(A_PER_WAVE * ROWS_PER_PIECE * NW == BM && B_PER_WAVE * ROWS_PER_PIECE * NW == BN,
                  "whole 1 KB pieces per wave");
    static_assert(A_SCALE_WAVES * 64 == BM && B_SCALE_WAVES * 128 == BN, "scale pieces");
    static_assert(A_SCALE_WAVES + B_SCALE_WAVES <= NW, "a scale piece per wave at most");
    static_assert(FN * 32 <= 128 && 128 % (FN * 32) == 0, "a wave's columns lie in one 128-wide n-block");
    static_assert(FM == 1 || FM == 2, "live m-tile paths exist for FM = 1, 2");
    static_assert(STAGES >= 3 && STAGES <= 5, "ring depth");
};
// dense / contiguous / long masked buffers: 256 x 256, waves 4 x 2 of 64 x 128
typedef WCfg<4, 2, 2, 4, 4> WideTile;
// decode-sized masked buffers: 64 x 256, waves 1 x 4 of 64 x 64, two
// workgroups per CU; every B code is widened once
typedef WCfg<1, 4, 2, 2, 3> WideDecodeTile;

template <class W>
struct alignas(16) WStage {
    uint8_t a[W::BM * W::KS];
    uint8_t b[W::BN * W::KS];
    float sa[W::BM];                    // A scales of the stage's K-block
    float sb[W::B_SCALE_WAVES * 64];    // 64 copies of each n-block's scale
    float dummy[64];
};

// how many of the n positions after one of parity e are even
constexpr int later_even(int n, int e) { return n % 2 == 0 ? n / 2 : (e == 1 ? (n + 1) / 2 : (n - 1) / 2); }

// Sparse copies: wait until at most the loads of the LATER later copies are
// outstanding -- DATA data loads each, plus a scale piece on the even ones
// when the wave has a scale role; e = the current copy's parity.
template <int LATER, int DATA>
__device__ __forceinline__ void wait_sparse(bool has_scale, int e) {
    if (!has_scale)
        wait_vmcnt<LATER * DATA>();
    else if (e == 0)
        wait_vmcnt<LATER * DATA + later_even(LATER, 0)>();
    else
        wait_vmcnt<LATER * DATA + later_even(LATER, 1)>();
}

// scale s -> (2^t with t = s's exponent clamped to [-124, 118], the range in
// which the widening cvt scales every code exactly; s / 2^t), with s == 0
// giving mantissa part 1 (its rows read the zero line instead).  The mantissa part
// is in [1, 2) for every normal s below 2^119 and never below 2^-25.
struct ScaleSplit {
    float pow2;
    float mant;
};
__device__ __forceinline__ ScaleSplit split_scale(float s) {
    const uint32_t e = (__builtin_bit_cast(uint32_t, s) >> 23) & 0xFF;
    const uint32_t ec = e < 3u ? 3u : (e > 245u ? 245u : e);
    ScaleSplit r;
    r.pow2 = __builtin_bit_cast(float, ec << 23);
    r.mant = s == 0.0f ? 1.0f : s * __builtin_bit_cast(float, (254u - ec) << 23);
    return r;
}

__device__ __forceinline__ float clamp_unit(float u) {
    return fminf(fmaxf(u, 0x1p-126f), 0x1p126f);
}

// 8 FP8 codes -> 8 BF16 values times 2^(exponent of p2)
__device__ __forceinline__ v8bf widen8_scaled(uint32_t w0, uint32_t w1, float p2) {
    const u32x4 v{__builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(int(w0), p2, false)),
                  __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(int(w0), p2, true)),
                  __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(int(w1), p2, false)),
                  __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(int(w1), p2, true))};
    return __builtin_bit_cast(v8bf, v);
}

typedef __amdgpu_buffer_rsrc_t rsrc_t;
constexpr int kRsrcFlags = 0x00020000;   // raw buffer, 32-bit dwords

__device__ __forceinline__ rsrc_t make_rsrc(const void* base, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, int(bytes), kRsrcFlags);
}

// TB: B is in the decode-tiled layout (fp8_tile_weights_decode): each
// half-block of a 256-row n-tile is one contiguous 16 KB block, already in
// the stage's LDS order, so the B pieces are plain contiguous copies.
template <class W, bool TB = false>
struct WideBufCopier {
    rsrc_t ra, rb, rs;
    uint32_t va[W::A_PER_WAVE], vb[W::B_PER_WAVE], vs;   // per-lane byte offsets
    uint32_t s_step;           // scale byte offset per K-block
    int a_lds[W::A_PER_WAVE], b_lds[W::B_PER_WAVE], s_lds;
    int a_c16[W::A_PER_WAVE], b_c16[W::B_PER_WAVE];       // the lane's chunk offset within a stage (bytes)
    int64_t K;
    bool has_scale;            // uniform: this wave copies a scale piece (not the dummy)
    bool skip_a;               // uniform: its one A piece holds only rows the compute never reads

    // After this wave's loads of half-block h have landed: zero its 16-byte
    // slots past K (a partial last K-block).  Those loads read whatever lies
    // there -- the next row, or zeros past the buffer's range -- never
    // outside the operand.
    __device__ __forceinline__ void zero_tail(uint8_t* stage, int h, int lane) const {
        const int64_t koff = int64_t(h) * W::KS;
#pragma unroll
        for (int i = 0; i < W::A_PER_WAVE; ++i)
            if (koff + a_c16[i] >= K) st<u32x4>(stage + a_lds[i] + lane * 16, u32x4{0u, 0u, 0u, 0u});
#pragma unroll
        for (int i = 0; i < W::B_PER_WAVE; ++i)
            if (koff + b_c16[i] >= K) st<u32x4>(stage + b_lds[i] + lane * 16, u32x4{0u, 0u, 0u, 0u});
    }

    // Half-block h into `stage`, as the pos-th copy of the sequence.  Dense:
    // every wave issues a scale piece with every half-block (waves without a
    // scale role load a dummy), so all waves wait alike.  `sparse` (the masked
    // layout, where the weight stream is the bound): scales change once per
    // K-block and only its first half reads them, so only the waves with a
    // scale role load one, with even positions only (h and pos have the same
    // parity except for the reloads past the end, which are never read).
    // Sparse also skips an A piece whose rows lie past every m-tile the tile
    // computes (decode tiles with at most 32 valid rows).
    __device__ __forceinline__ void copy(uint8_t* stage, int h, int pos, bool sparse) const {
        const uint32_t koff = uint32_t(h) * W::KS;
        if (!(sparse && skip_a)) {
#pragma unroll
            for (int i = 0; i < W::A_PER_WAVE; ++i)
                __builtin_amdgcn_raw_ptr_buffer_load_lds(ra, (lds_ptr_t)(stage + a_lds[i]), 16, va[i], koff, 0, 0);
        }
#pragma unroll
        for (int i = 0; i < W::B_PER_WAVE; ++i)
            __builtin_amdgcn_raw_ptr_buffer_load_lds(rb, (lds_ptr_t)(stage + b_lds[i]), 16, vb[i],
                                                     TB ? uint32_t(h) * uint32_t(W::BN * W::KS) : koff, 0, 0);
        if (!sparse || (has_scale && (pos & 1) == 0))
            __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_ptr_t)(stage + s_lds), 4, vs, uint32_t(h >> 1) * s_step,
                                                     0, 0);
    }
};

template <class W, bool TB = false>
__device__ __forceinline__ WideBufCopier<W, TB> make_wide_buf_copier(const Tile& t, int wave, int lane, int64_t K,
                                                                     int64_t n0) {
    typedef WStage<W> S;
    WideBufCopier<W, TB> c;
    c.K = K;
    c.has_scale = wave < W::A_SCALE_WAVES + W::B_SCALE_WAVES;
    const int sub = lane >> 2, slot = lane & 3;
    const int64_t tile_rows = t.rows_valid - t.m0 < W::BM ? t.rows_valid - t.m0 : W::BM;   // >= 1
    c.ra = make_rsrc(t.A + t.m0 * K, uint32_t(tile_rows * K));
    c.rb = make_rsrc(t.B + n0 * K, uint32_t(W::BN * K));
    // one m-row of waves: the compute reads the first ceil(tile_rows / 32) m-tiles
    c.skip_a = W::A_PER_WAVE == 1 && W::WAVES_M == 1 &&
               int64_t(wave) * W::ROWS_PER_PIECE >= (tile_rows + 31) / 32 * 32;
#pragma unroll
    for (int i = 0; i < W::A_PER_WAVE; ++i) {
        const int r0 = (wave * W::A_PER_WAVE + i) * W::ROWS_PER_PIECE, r = r0 + sub;
        const int chunk = slot ^ ((r >> 2) & 3);
        const int64_t row = r < tile_rows ? r : tile_rows - 1;      // clamp: loaded, never stored
        c.va[i] = uint32_t(row * K + chunk * 16);
        c.a_c16[i] = chunk * 16;
        c.a_lds[i] = int(offsetof(S, a)) + r0 * W::KS;
    }
#pragma unroll
    for (int i = 0; i < W::B_PER_WAVE; ++i) {
        const int r0 = (wave * W::B_PER_WAVE + i) * W::ROWS_PER_PIECE, r = r0 + sub;
        const int chunk = slot ^ ((r >> 2) & 3);
        // tiled: the lane's 16 bytes sit where the stage keeps them (row r,
        // position slot, holding K chunk `chunk` of the half-block)
        c.vb[i] = TB ? uint32_t(r0 * W::KS + lane * 16) : uint32_t(int64_t(r) * K + chunk * 16);
        c.b_c16[i] = chunk * 16;
        c.b_lds[i] = int(offsetof(S, b)) + r0 * W::KS;
    }
    const int64_t kbs = (K + BK - 1) / BK;
    if (wave < W::A_SCALE_WAVES) {        // A scales of rows 64 wave .. +63 (clamped)
        const int64_t rr = int64_t(wave) * 64 + lane;
        const int64_t row = rr < tile_rows ? rr : tile_rows - 1;
        c.rs = make_rsrc(t.SA + t.m0, uint32_t(((kbs - 1) * t.lda_s + tile_rows) * 4));
        c.vs = uint32_t(row * 4);
        c.s_step = uint32_t(t.lda_s * 4);
        c.s_lds = int(offsetof(S, sa)) + wave * 64 * 4;
    } else if (wave < W::A_SCALE_WAVES + W::B_SCALE_WAVES) {   // 64 copies of an n-block's scale
        const int j = wave - W::A_SCALE_WAVES;
        c.rs = make_rsrc(t.SB + (n0 / 128 + j) * kbs, uint32_t(kbs * 4));
        c.vs = 0;
        c.s_step = 4;
        c.s_lds = int(offsetof(S, sb)) + j * 64 * 4;
    } else {                              // padding: the tile's first A scale again
        c.rs = make_rsrc(t.SA + t.m0, uint32_t(((kbs - 1) * t.lda_s + 1) * 4));
        c.vs = 0;
        c.s_step = uint32_t(t.lda_s * 4);
        c.s_lds = int(offsetof(S, dummy));
    }
    return c;
}

// what a K-block's scales turn into for one wave
template <int FM>
struct WideScales {
    float pa[FM], pb;        // cvt scale operands (exponent parts)
    float unit[FM];          // mantissa-part products: the accumulator unit
    int zero[FM];            // 1 if the row's codes must read as +0 (its A scale or the B scale is 0)
};

template <class W>
__device__ __forceinline__ WideScales<W::FM> wide_scales(const WStage<W>& sg, int wm, int wn, int r) {
    WideScales<W::FM> w;
    const float sb = sg.sb[((wn * W::FN * 32) / 128) * 64];
    const ScaleSplit b = split_scale(sb);
    w.pb = b.pow2;
#pragma unroll
    for (int mi = 0; mi < W::FM; ++mi) {
        const float sa = sg.sa[wm * W::FM * 32 + mi * 32 + r];
        const ScaleSplit a = split_scale(sa);
        w.pa[mi] = a.pow2;
        w.unit[mi] = clamp_unit(a.mant * b.mant);
        w.zero[mi] = (sa == 0.0f || sb == 0.0f) ? 1 : 0;
    }
    return w;
}

template <int FM, int FN>
struct Frags {
    u32x4 a[FM], b[FN];
};

// this lane's fragments of chunk column j (32 K) of stage slot `slot`: A rows
// of the first ML m-tiles (or the zero line) and B rows of the FN n-tiles
template <class W, int ML>
__device__ __forceinline__ Frags<W::FM, W::FN> read_frags(const uint8_t* lds, int slot, int j, int wm, int wn,
                                                          int r, int h, const WideScales<W::FM>& w,
                                                          uint32_t zero_line) {
    Frags<W::FM, W::FN> x;
    const uint32_t base = uint32_t(slot) * uint32_t(sizeof(WStage<W>));
    const uint32_t chunk = uint32_t(((2 * j + h) ^ ((r >> 2) & 3)) << 4);
#pragma unroll
    for (int mi = 0; mi < ML; ++mi) {
        const uint32_t a = base + uint32_t(offsetof(WStage<W>, a)) +
                           uint32_t((wm * W::FM * 32 + mi * 32 + r) * W::KS) + chunk;
        x.a[mi] = ld<u32x4>(lds + (w.zero[mi] ? zero_line + chunk : a));
    }
    const uint32_t b = base + uint32_t(offsetof(WStage<W>, b)) + uint32_t((wn * W::FN * 32 + r) * W::KS) + chunk;
#pragma unroll
    for (int ni = 0; ni < W::FN; ++ni) x.b[ni] = ld<u32x4>(lds + b + ni * 32 * W::KS);
    return x;
}

// the two k-steps of one chunk column, first ML m-tiles
template <int FM, int FN, int ML>
__device__ __forceinline__ void mfma_column(const Frags<FM, FN>& x, const WideScales<FM>& w, v16f (&acc)[FM][FN]) {
#pragma unroll
    for (int half = 0; half < 2; ++half) {
        v8bf a8[FM], b8[FN];
#pragma unroll
        for (int mi = 0; mi < ML; ++mi) a8[mi] = widen8_scaled(x.a[mi][2 * half], x.a[mi][2 * half + 1], w.pa[mi]);
#pragma unroll
        for (int ni = 0; ni < FN; ++ni) b8[ni] = widen8_scaled(x.b[ni][2 * half], x.b[ni][2 * half + 1], w.pb);
#pragma unroll
        for (int mi = 0; mi < ML; ++mi)
#pragma unroll
            for (int ni = 0; ni < FN; ++ni)
                acc[mi][ni] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(b8[ni], a8[mi], acc[mi][ni], 0, 0, 0);
    }
}

// One half-block: both chunk columns' fragments, then their four k-steps.
template <class W, int ML>
__device__ __forceinline__ void wide_half_compute(const uint8_t* lds, int slot, int wm, int wn, int r, int h,
                                                  const WideScales<W::FM>& w, uint32_t zero_line,
                                                  v16f (&acc)[W::FM][W::FN]) {
    Frags<W::FM, W::FN> f[2];
#pragma unroll
    for (int j = 0; j < 2; ++j) f[j] = read_frags<W, ML>(lds, slot, j, wm, wn, r, h, w, zero_line);
#pragma unroll
    for (int j = 0; j < 2; ++j) mfma_column<W::FM, W::FN, ML>(f[j], w, acc);
}

// move the first ML m-tiles' accumulators from unit w to unit nw
template <int FM, int FN, int ML>
__device__ __forceinline__ void rescale(v16f (&acc)[FM][FN], const WideScales<FM>& w, const WideScales<FM>& nw) {
#pragma unroll
    for (int mi = 0; mi < ML; ++mi) {
        const float ratio = clamp_unit(w.unit[mi] * __builtin_amdgcn_rcpf(nw.unit[mi]));
#pragma unroll
        for (int ni = 0; ni < FN; ++ni)
#pragma unroll
            for (int i = 0; i < 16; ++i) acc[mi][ni][i] *= ratio;
    }
}

template <class W>
constexpr uint32_t wide_lds_bytes() { return uint32_t(W::STAGES * sizeof(WStage<W>) + 64); }

// OUT: 0 = BF16, 1 = FP32, 2 = FP8 codes + 1x128 scales along N (dense only).
// `lds_raw` holds wide_lds_bytes<W>(); the workgroup computes tile `tile` of
// the n-tiles covering columns [0, n_ext) (n_ext < 0: all N).
template <class W, int OUT, int MODE, bool TB = false>
__device__ __forceinline__ void gemm_wide_body(const GemmArgs& args, uint8_t* lds_raw, int64_t tile, int64_t n_ext) {
    typedef WStage<W> S;
    constexpr int FM = W::FM, FN = W::FN, STAGES = W::STAGES;
    constexpr uint32_t kZeroLine = STAGES * sizeof(S);
    S* ring = reinterpret_cast<S*>(lds_raw);

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // uniform: keeps wave-derived values scalar
    const int wm = wave / W::WAVES_N, wn = wave % W::WAVES_N;
    const int64_t N = args.N, K = args.K;
    const int halves = int(2 * ((K + BK - 1) / BK));   // the last K-block may be partial
    const Tile t = map_tile<W, MODE>(args, tile, n_ext);
    if (!t.live) return;
    const int64_t n0 = int64_t(t.bn) * W::BN;
    static_assert(!TB || (W::BN == 256 && W::KS == 64), "the decode-tiled layout has 256-row, 64-K blocks");
    const WideBufCopier<W, TB> cp = make_wide_buf_copier<W, TB>(t, wave, lane, K, n0);
    const int64_t wrow0 = t.m0 + wm * FM * 32;
    const int64_t left = t.rows_valid - wrow0;
    // m-tiles of this wave holding valid rows (uniform): 0, 1 or FM.  Only the
    // masked layout, whose tiles are mostly part-filled, takes the one-m-tile
    // path: elsewhere partial m-tiles occur at edges only, and a second path
    // would cost register copies where the two meet in every iteration.
    const int mlive = left <= 0 ? 0 : (left >= FM * 32 ? FM : int((left + 31) / 32));
    constexpr bool full = FM == 1 || MODE != int(GemmMode::Masked);
    const int r = lane & 31, h = lane >> 5;
    constexpr int L = W::A_PER_WAVE + W::B_PER_WAVE;   // data loads per half-block, + a scale piece
    constexpr bool SPARSE = MODE == int(GemmMode::Masked);

    if (tid < 4) st<u32x4>(lds_raw + kZeroLine + tid * 16, u32x4{0u, 0u, 0u, 0u});
    // half-blocks past the end reload the last one (into slots never read
    // again), so every iteration issues the same loads and waits the same
#pragma unroll
    for (int st = 0; st < STAGES - 1; ++st)
        cp.copy(reinterpret_cast<uint8_t*>(&ring[st]), st < halves ? st : halves - 1, st, SPARSE);
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");   // the zero line is written before the first barrier

    v16f acc[FM][FN];
#pragma unroll
    for (int mi = 0; mi < FM; ++mi)
#pragma unroll
        for (int ni = 0; ni < FN; ++ni)
#pragma unroll
            for (int i = 0; i < 16; ++i) acc[mi][ni][i] = 0.f;
    WideScales<FM> w;
    w.pb = 1.0f;
#pragma unroll
    for (int mi = 0; mi < FM; ++mi) {
        w.pa[mi] = 1.0f;
        w.unit[mi] = 1.0f;
        w.zero[mi] = 0;
    }

    int slot = 0, fill_slot = STAGES - 1;   // ring slots of half-blocks cur and cur + STAGES - 1
    for (int hb = 0; hb < halves; hb += 2) {
#pragma unroll
        for (int e = 0; e < 2; ++e) {
            const int cur = hb + e;
            // this wave's copy of half-block cur has landed: only the loads of
            // the STAGES - 2 later half-blocks may be outstanding
            // (sparse: per role -- a scale piece or not, the A piece skipped or not)
            if (!SPARSE)
                wait_vmcnt<(STAGES - 2) * (L + 1)>();
            else if (cp.skip_a)
                wait_sparse<(STAGES - 2), L - W::A_PER_WAVE>(cp.has_scale, e);
            else
                wait_sparse<(STAGES - 2), L>(cp.has_scale, e);
            if ((cur + 1) * W::KS > K) {      // partial last K-block (uniform)
                cp.zero_tail(reinterpret_cast<uint8_t*>(&ring[slot]), cur, lane);
                asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
            }
            __builtin_amdgcn_s_barrier();     // ... every wave's; the slot of cur - 1 is free
            const int fill = cur + STAGES - 1;
            cp.copy(reinterpret_cast<uint8_t*>(&ring[fill_slot]), fill < halves ? fill : halves - 1, fill, SPARSE);
            if (mlive > 0) {
                if (e == 0) {
                    const WideScales<FM> nw = wide_scales<W>(ring[slot], wm, wn, r);
                    if (full || mlive == FM)
                        rescale<FM, FN, FM>(acc, w, nw);
                    else
                        rescale<FM, FN, 1>(acc, w, nw);
                    w = nw;
                }
                if (full || mlive == FM)
                    wide_half_compute<W, FM>(lds_raw, slot, wm, wn, r, h, w, kZeroLine, acc);
                else
                    wide_half_compute<W, 1>(lds_raw, slot, wm, wn, r, h, w, kZeroLine, acc);
            }
            slot = slot == STAGES - 1 ? 0 : slot + 1;
            fill_slot = fill_slot == STAGES - 1 ? 0 : fill_slot + 1;
        }
    }
    wait_vmcnt<0>();   // no copy may land after the workgroup's LDS is handed on

    const int n_lane = wn * FN * 32 + 4 * h;
    if constexpr (OUT == 2) {
        // Fused 1x128 quantization of C along N for the next layer: the
        // wave's 128 columns are one group (they start on a multiple of 128),
        // and row m's 128 values sit in lanes r and r + 32.  The values are the
        // FP32 output's, bit for bit; the group is quantized exactly as the
        // 1x128 activation quantizer does (amax / 448, RN32(x / s), E4M3).
        static_assert(FN * 32 == 128, "one 128-column group per wave");
#pragma unroll
        for (int mi = 0; mi < FM; ++mi) {
            float amax = 0.0f;
#pragma unroll
            for (int ni = 0; ni < FN; ++ni)
#pragma unroll
                for (int i = 0; i < 16; ++i) amax = fmaxf(amax, fabsf(acc[mi][ni][i] * w.unit[mi]));
            amax = fmaxf(amax, __shfl_xor(amax, 32, 64));
            const float sc = amax / 448.0f;
            const float rc = 1.0f / sc;
            const int64_t m = wrow0 + mi * 32 + r;
            if (m >= t.rows_valid) continue;
#pragma unroll
            for (int ni = 0; ni < FN; ++ni)
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const v4f v = v4f{acc[mi][ni][4 * j], acc[mi][ni][4 * j + 1], acc[mi][ni][4 * j + 2],
                                      acc[mi][ni][4 * j + 3]} * w.unit[mi];
                    st<uint32_t>(static_cast<uint8_t*>(args.c) + m * N + n0 + n_lane + ni * 32 + 8 * j,
                                 encode4(v, sc, rc));
                }
            if (h == 0) args.cs[(n0 / 128 + wn) * args.M + m] = sc;
        }
        return;
    }
#pragma unroll
    for (int mi = 0; mi < FM; ++mi) {
        const int64_t m = wrow0 + mi * 32 + r;
        if (m >= t.rows_valid) continue;
#pragma unroll
        for (int ni = 0; ni < FN; ++ni)
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int64_t idx = t.c_base + m * N + n0 + n_lane + ni * 32 + 8 * j;
                const v4f v = v4f{acc[mi][ni][4 * j], acc[mi][ni][4 * j + 1], acc[mi][ni][4 * j + 2],
                                  acc[mi][ni][4 * j + 3]} * w.unit[mi];
                if (OUT == 1) {
                    st<v4f>(static_cast<float*>(args.c) + idx, v);
                } else {
                    const uint32_t lo = bf16_bits(v[0]) | (bf16_bits(v[1]) << 16);
                    const uint32_t hi = bf16_bits(v[2]) | (bf16_bits(v[3]) << 16);
                    st<u32x2>(static_cast<uint16_t*>(args.c) + idx, u32x2{lo, hi});
                }
            }
    }
}

// ---------------------------------------------------------------------------
// Tail tiles of a dense grid.  448 tiles of 256 x 256 (4096 x 7168) fill 256
// CUs 1.75 times, leaving a quarter of the chip idle for the second round.
// The planner (dispatch) then covers the last columns with 256 x 192 tiles,
// sized so that each kind fills whole rounds: 256 wide tiles, then 256 tail
// tiles of three quarters of the work, in one launch.  The tail tile is the
// wide kernel with waves 4 x 2 of 64 x 96 (FN = 3), so the VALU work per MFMA
// barely changes.  It starts on a multiple of 64 columns and spans two
// 128-wide n-blocks, and one wave column straddles them, so the B scale's
// exponent part, the zero test and the accumulator unit are per 32-column
// fragment.  12 B pieces per half-block: waves 0-3 copy two, waves 4-7 one.
struct TailCfg {
    static constexpr int WAVES_M = 4, WAVES_N = 2, FM = 2, FN = 3, STAGES = 4;
    static constexpr int NW = WAVES_M * WAVES_N, THREADS = NW * 64;
    static constexpr int BM = WAVES_M * FM * 32, BN = WAVES_N * FN * 32, KS = 64, ROWS_PER_PIECE = 16;
    static constexpr int A_PER_WAVE = BM / ROWS_PER_PIECE / NW;
    static constexpr int A_SCALE_WAVES = BM / 64, B_SCALE_WAVES = 2;   // the two n-blocks a tile touches
    static_assert(BN == 192 && BN / ROWS_PER_PIECE == 12 && A_PER_WAVE == 2, "piece split below");
};

struct alignas(16) TStage {
    uint8_t a[TailCfg::BM * TailCfg::KS];
    uint8_t b[TailCfg::BN * TailCfg::KS];
    float sa[TailCfg::BM];
    float sb[TailCfg::B_SCALE_WAVES * 64];   // 64 copies of each n-block's scale
    float dummy[64];
};
constexpr uint32_t tail_lds_bytes() { return uint32_t(TailCfg::STAGES * sizeof(TStage) + 64); }

struct TailCopier {
    rsrc_t ra, rb, rs;
    uint32_t va[2], vb[2], vs;
    uint32_t s_step;
    int a_lds[2], b_lds[2], s_lds;
    int a_c16[2], b_c16[2];
    bool two_b;              // uniform: this wave copies two B pieces (waves 0-3) or one
    int64_t K;

    // as WideBufCopier::zero_tail
    __device__ __forceinline__ void zero_tail(uint8_t* stage, int h, int lane) const {
        const int64_t koff = int64_t(h) * TailCfg::KS;
#pragma unroll
        for (int i = 0; i < 2; ++i)
            if (koff + a_c16[i] >= K) st<u32x4>(stage + a_lds[i] + lane * 16, u32x4{0u, 0u, 0u, 0u});
#pragma unroll
        for (int i = 0; i < 2; ++i)
            if ((i == 0 || two_b) && koff + b_c16[i] >= K)
                st<u32x4>(stage + b_lds[i] + lane * 16, u32x4{0u, 0u, 0u, 0u});
    }

    // half-block h into `stage`: A pieces, B pieces, one scale piece (a dummy
    // on waves 6 and 7) -- 5 loads on waves 0-3, 4 on waves 4-7
    __device__ __forceinline__ void copy(uint8_t* stage, int h) const {
        const uint32_t koff = uint32_t(h) * TailCfg::KS;
#pragma unroll
        for (int i = 0; i < 2; ++i)
            __builtin_amdgcn_raw_ptr_buffer_load_lds(ra, (lds_ptr_t)(stage + a_lds[i]), 16, va[i], koff, 0, 0);
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rb, (lds_ptr_t)(stage + b_lds[0]), 16, vb[0], koff, 0, 0);
        if (two_b) __builtin_amdgcn_raw_ptr_buffer_load_lds(rb, (lds_ptr_t)(stage + b_lds[1]), 16, vb[1], koff, 0, 0);
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_ptr_t)(stage + s_lds), 4, vs, uint32_t(h >> 1) * s_step, 0, 0);
    }
};

// t: dense tile (m0, rows_valid = M); n0: first column (a multiple of 64)
__device__ __forceinline__ TailCopier make_tail_copier(const Tile& t, int wave, int lane, int64_t K, int64_t N,
                                                       int64_t n0) {
    typedef TailCfg W;
    TailCopier c;
    c.K = K;
    c.two_b = wave < 4;
    const int sub = lane >> 2, slot = lane & 3;
    const int64_t tile_rows = t.rows_valid - t.m0 < W::BM ? t.rows_valid - t.m0 : W::BM;   // >= 1
    c.ra = make_rsrc(t.A + t.m0 * K, uint32_t(tile_rows * K));
    c.rb = make_rsrc(t.B + n0 * K, uint32_t(W::BN * K));
#pragma unroll
    for (int i = 0; i < 2; ++i) {
        const int r0 = (wave * 2 + i) * W::ROWS_PER_PIECE, r = r0 + sub;
        const int chunk = slot ^ ((r >> 2) & 3);
        const int64_t row = r < tile_rows ? r : tile_rows - 1;      // clamp: loaded, never stored
        c.va[i] = uint32_t(row * K + chunk * 16);
        c.a_c16[i] = chunk * 16;
        c.a_lds[i] = int(offsetof(TStage, a)) + r0 * W::KS;
    }
#pragma unroll
    for (int i = 0; i < 2; ++i) {
        const int piece = wave < 4 ? wave * 2 + i : 8 + (wave - 4);   // waves 4-7: one piece (i = 1 unused)
        const int r0 = piece * W::ROWS_PER_PIECE, r = r0 + sub;
        const int chunk = slot ^ ((r >> 2) & 3);
        c.vb[i] = uint32_t(int64_t(r) * K + chunk * 16);
        c.b_c16[i] = chunk * 16;
        c.b_lds[i] = int(offsetof(TStage, b)) + r0 * W::KS;
    }
    const int64_t kbs = (K + BK - 1) / BK, nbs = (N + 127) / 128;
    if (wave < W::A_SCALE_WAVES) {        // A scales of rows 64 wave .. +63 (clamped)
        const int64_t rr = int64_t(wave) * 64 + lane;
        const int64_t row = rr < tile_rows ? rr : tile_rows - 1;
        c.rs = make_rsrc(t.SA + t.m0, uint32_t(((kbs - 1) * t.lda_s + tile_rows) * 4));
        c.vs = uint32_t(row * 4);
        c.s_step = uint32_t(t.lda_s * 4);
        c.s_lds = int(offsetof(TStage, sa)) + wave * 64 * 4;
    } else if (wave < W::A_SCALE_WAVES + W::B_SCALE_WAVES) {   // 64 copies of n-block n0/128 + j
        const int j = wave - W::A_SCALE_WAVES;
        int64_t nb = n0 / 128 + j;
        nb = nb < nbs ? nb : nbs - 1;
        c.rs = make_rsrc(t.SB + nb * kbs, uint32_t(kbs * 4));
        c.vs = 0;
        c.s_step = 4;
        c.s_lds = int(offsetof(TStage, sb)) + j * 64 * 4;
    } else {                              // padding: the tile's first A scale again
        c.rs = make_rsrc(t.SA + t.m0, uint32_t(((kbs - 1) * t.lda_s + 1) * 4));
        c.vs = 0;
        c.s_step = uint32_t(t.lda_s * 4);
        c.s_lds = int(offsetof(TStage, dummy));
    }
    return c;
}

// a K-block's scales for one wave of a tail tile, per 32-column fragment
struct TailScales {
    float pa[TailCfg::FM], pb[TailCfg::FN];
    float unit[TailCfg::FM][TailCfg::FN];
    int za[TailCfg::FM], zb[TailCfg::FN];   // codes read as +0: A scale 0 (per row), B scale 0 (per fragment)
};

// nsel[ni]: which of the tile's two n-blocks fragment ni lies in (uniform)
__device__ __forceinline__ TailScales tail_scales(const TStage& sg, int wm, const int (&nsel)[TailCfg::FN], int r) {
    TailScales w;
    const float sb0 = sg.sb[0], sb1 = sg.sb[64];
    const ScaleSplit b0 = split_scale(sb0), b1 = split_scale(sb1);
    float bm[TailCfg::FN];
#pragma unroll
    for (int ni = 0; ni < TailCfg::FN; ++ni) {
        w.pb[ni] = nsel[ni] ? b1.pow2 : b0.pow2;
        bm[ni] = nsel[ni] ? b1.mant : b0.mant;
        w.zb[ni] = (nsel[ni] ? sb1 : sb0) == 0.0f ? 1 : 0;
    }
#pragma unroll
    for (int mi = 0; mi < TailCfg::FM; ++mi) {
        const float sa = sg.sa[wm * TailCfg::FM * 32 + mi * 32 + r];
        const ScaleSplit a = split_scale(sa);
        w.pa[mi] = a.pow2;
        w.za[mi] = sa == 0.0f ? 1 : 0;
#pragma unroll
        for (int ni = 0; ni < TailCfg::FN; ++ni) w.unit[mi][ni] = clamp_unit(a.mant * bm[ni]);
    }
    return w;
}

__device__ __forceinline__ void tail_rescale(v16f (&acc)[TailCfg::FM][TailCfg::FN], const TailScales& w,
                                             const TailScales& nw) {
#pragma unroll
    for (int mi = 0; mi < TailCfg::FM; ++mi)
#pragma unroll
        for (int ni = 0; ni < TailCfg::FN; ++ni) {
            const float ratio = clamp_unit(w.unit[mi][ni] * __builtin_amdgcn_rcpf(nw.unit[mi][ni]));
#pragma unroll
            for (int i = 0; i < 16; ++i) acc[mi][ni][i] *= ratio;
        }
}

// fragments of chunk column j (32 K) of stage slot `slot`, then its two k-steps
__device__ __forceinline__ void tail_column(const uint8_t* lds, int slot, int j, int wm, int wn, int r, int h,
                                            const TailScales& w, uint32_t zero_line,
                                            v16f (&acc)[TailCfg::FM][TailCfg::FN]) {
    typedef TailCfg W;
    const uint32_t base = uint32_t(slot) * uint32_t(sizeof(TStage));
    const uint32_t chunk = uint32_t(((2 * j + h) ^ ((r >> 2) & 3)) << 4);
    u32x4 a[W::FM], b[W::FN];
#pragma unroll
    for (int mi = 0; mi < W::FM; ++mi) {
        const uint32_t at = base + uint32_t(offsetof(TStage, a)) + uint32_t((wm * W::FM * 32 + mi * 32 + r) * W::KS) + chunk;
        a[mi] = ld<u32x4>(lds + (w.za[mi] ? zero_line + chunk : at));
    }
#pragma unroll
    for (int ni = 0; ni < W::FN; ++ni) {
        const uint32_t bt = base + uint32_t(offsetof(TStage, b)) + uint32_t((wn * W::FN * 32 + ni * 32 + r) * W::KS) + chunk;
        b[ni] = ld<u32x4>(lds + (w.zb[ni] ? zero_line + chunk : bt));
    }
#pragma unroll
    for (int half = 0; half < 2; ++half) {
        v8bf a8[W::FM], b8[W::FN];
#pragma unroll
        for (int mi = 0; mi < W::FM; ++mi) a8[mi] = widen8_scaled(a[mi][2 * half], a[mi][2 * half + 1], w.pa[mi]);
#pragma unroll
        for (int ni = 0; ni < W::FN; ++ni) b8[ni] = widen8_scaled(b[ni][2 * half], b[ni][2 * half + 1], w.pb[ni]);
#pragma unroll
        for (int mi = 0; mi < W::FM; ++mi)
#pragma unroll
            for (int ni = 0; ni < W::FN; ++ni)
                acc[mi][ni] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(b8[ni], a8[mi], acc[mi][ni], 0, 0, 0);
    }
}

// Dense tail tile `tile` of the 256 x 192 tiles covering columns [n_base, N)
// (N - n_base a multiple of 192, n_base of 64); `lds_raw` holds tail_lds_bytes().
// OUT: 0 = BF16, 1 = FP32.
template <int OUT>
__device__ __forceinline__ void gemm_tail_body(const GemmArgs& args, uint8_t* lds_raw, int64_t tile, int64_t n_base) {
    typedef TailCfg W;
    constexpr int FM = W::FM, FN = W::FN, STAGES = W::STAGES;
    constexpr uint32_t kZeroLine = STAGES * sizeof(TStage);
    TStage* ring = reinterpret_cast<TStage*>(lds_raw);

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm = wave / W::WAVES_N, wn = wave % W::WAVES_N;
    const int64_t N = args.N, K = args.K;
    const int halves = int(2 * ((K + BK - 1) / BK));
    const int64_t n_tiles = (N - n_base) / W::BN;
    Tile t;
    t.m0 = (tile / n_tiles) * W::BM;
    t.rows_valid = args.M;
    t.lda_s = args.M;
    t.c_base = 0;
    t.A = args.a;
    t.SA = args.sa;
    t.B = args.b;
    t.SB = args.sb;
    t.bn = int(tile % n_tiles);
    if (t.m0 >= t.rows_valid) return;
    const int64_t n0 = n_base + int64_t(t.bn) * W::BN;
    const TailCopier cp = make_tail_copier(t, wave, lane, K, N, n0);
    const int64_t wrow0 = t.m0 + wm * FM * 32;
    const bool live = wrow0 < t.rows_valid;   // uniform: this wave has valid rows
    const int r = lane & 31, h = lane >> 5;
    int nsel[FN];
#pragma unroll
    for (int ni = 0; ni < FN; ++ni) nsel[ni] = int(((n0 & 127) + wn * FN * 32 + ni * 32) >> 7);

    if (tid < 4) st<u32x4>(lds_raw + kZeroLine + tid * 16, u32x4{0u, 0u, 0u, 0u});
#pragma unroll
    for (int st_ = 0; st_ < STAGES - 1; ++st_)
        cp.copy(reinterpret_cast<uint8_t*>(&ring[st_]), st_ < halves ? st_ : halves - 1);
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");

    v16f acc[FM][FN];
#pragma unroll
    for (int mi = 0; mi < FM; ++mi)
#pragma unroll
        for (int ni = 0; ni < FN; ++ni)
#pragma unroll
            for (int i = 0; i < 16; ++i) acc[mi][ni][i] = 0.f;
    TailScales w;
#pragma unroll
    for (int mi = 0; mi < FM; ++mi) {
        w.pa[mi] = 1.0f;
        w.za[mi] = 0;
#pragma unroll
        for (int ni = 0; ni < FN; ++ni) w.unit[mi][ni] = 1.0f;
    }
#pragma unroll
    for (int ni = 0; ni < FN; ++ni) {
        w.pb[ni] = 1.0f;
        w.zb[ni] = 0;
    }

    int slot = 0, fill_slot = STAGES - 1;
    for (int hb = 0; hb < halves; hb += 2) {
#pragma unroll
        for (int e = 0; e < 2; ++e) {
            const int cur = hb + e;
            // this wave's copy of half-block cur has landed (5 or 4 loads per half-block)
            if (cp.two_b)
                wait_vmcnt<(STAGES - 2) * 5>();
            else
                wait_vmcnt<(STAGES - 2) * 4>();
            if ((cur + 1) * W::KS > K) {      // partial last K-block (uniform)
                cp.zero_tail(reinterpret_cast<uint8_t*>(&ring[slot]), cur, lane);
                asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
            }
            __builtin_amdgcn_s_barrier();
            const int fill = cur + STAGES - 1;
            cp.copy(reinterpret_cast<uint8_t*>(&ring[fill_slot]), fill < halves ? fill : halves - 1);
            if (live) {
                if (e == 0) {
                    const TailScales nw = tail_scales(ring[slot], wm, nsel, r);
                    tail_rescale(acc, w, nw);
                    w = nw;
                }
#pragma unroll
                for (int j = 0; j < 2; ++j) tail_column(lds_raw, slot, j, wm, wn, r, h, w, kZeroLine, acc);
            }
            slot = slot == STAGES - 1 ? 0 : slot + 1;
            fill_slot = fill_slot == STAGES - 1 ? 0 : fill_slot + 1;
        }
    }
    wait_vmcnt<0>();   // no copy may land after the workgroup's LDS is handed on

    const int n_lane = wn * FN * 32 + 4 * h;
#pragma unroll
    for (int mi = 0; mi < FM; ++mi) {
        const int64_t m = wrow0 + mi * 32 + r;
        if (m >= t.rows_valid) continue;
#pragma unroll
        for (int ni = 0; ni < FN; ++ni)
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int64_t idx = m * N + n0 + n_lane + ni * 32 + 8 * j;
                const v4f v = v4f{acc[mi][ni][4 * j], acc[mi][ni][4 * j + 1], acc[mi][ni][4 * j + 2],
                                  acc[mi][ni][4 * j + 3]} * w.unit[mi][ni];
                if (OUT == 1) {
                    st<v4f>(static_cast<float*>(args.c) + idx, v);
                } else {
                    const uint32_t lo = bf16_bits(v[0]) | (bf16_bits(v[1]) << 16);
                    const uint32_t hi = bf16_bits(v[2]) | (bf16_bits(v[3]) << 16);
                    st<u32x2>(static_cast<uint16_t*>(args.c) + idx, u32x2{lo, hi});
                }
            }
    }
}

// One launch of a planned dense grid: workgroups [0, tiles1) take the 256 x
// 256 tiles over columns [0, n_split), the rest the 256 x 192 tail tiles over
// [n_split, N).  Both bodies share one LDS array.
static_assert(tail_lds_bytes() <= wide_lds_bytes<WideTile>(), "the tail body fits the wide body's LDS");
template <int OUT>
__device__ __forceinline__ void gemm_wmix_body(const GemmArgs& args, int64_t tiles1, int64_t n_split) {
    __shared__ __align__(16) uint8_t lds[wide_lds_bytes<WideTile>()];
    if (int64_t(blockIdx.x) < tiles1)
        gemm_wide_body<WideTile, OUT, int(GemmMode::Dense)>(args, lds, blockIdx.x, n_split);
    else
        gemm_tail_body<OUT>(args, lds, int64_t(blockIdx.x) - tiles1, n_split);
}
__global__ __launch_bounds__(WideTile::THREADS) void gemm_wmix_o0_dense(GemmArgs args, int64_t tiles1,
                                                                        int64_t n_split) {
    gemm_wmix_body<0>(args, tiles1, n_split);
}
__global__ __launch_bounds__(WideTile::THREADS) void gemm_wmix_o1_dense(GemmArgs args, int64_t tiles1,
                                                                        int64_t n_split) {
    gemm_wmix_body<1>(args, tiles1, n_split);
}

// ---------------------------------------------------------------------------
// MX GEMM (microscaled operands: E4M3 codes with one power-of-two E8M0 scale
// per 32 consecutive K; the MX variant of the method, see quant.hip).
// C = A . B^T, A codes [M][K] with scale bytes [K/32][M], B codes [N][K] with
// [K/32][N].  gfx950's v_mfma_scale_f32_32x32x64_f8f6f4 applies both scales
// itself, so there is no promotion step and no VALU work per K: the K loop
// is fragment reads and MFMAs into one FP32 accumulator.  Like every FP8
// MFMA on gfx950 it sums each group of products with limited width, so the
// result is held to the FP8-MFMA engine's bound.
//
// Operand layout of the scaled instruction (measured): lane (r, h) of a
// 64-K step gives row r, K 16h .. 16h+15 in dwords 0-3 and K 32+16h .. +15 in
// dwords 4-7, and the scale of row r's 32-K block j is taken from lane
// r + 32 j; so lane (r, h) supplies the scale of block h of the step.
//
// Work decomposition as in the wide kernel: 256 x 256 tiles, 4 x 2 waves of
// 64 x 128, a four-stage ring of 64-K stages (rows of 64 bytes, chunk c at
// slot c ^ ((r >> 2) & 3)) filled by buffer-to-LDS loads; the scale bytes of
// a stage (two 256-byte runs for A and for B) ride with it.
struct MxTile {
    static constexpr int WAVES_M = 4, WAVES_N = 2, FM = 2, FN = 4, STAGES = 4;
    static constexpr int NW = 8, THREADS = 512, BM = 256, BN = 256, KS = 64;
    static constexpr int LOADS_PER_WAVE = 5;   // two A pieces, two B pieces, one scale run
};

struct alignas(16) MxStage {
    uint8_t a[MxTile::BM * MxTile::KS];
    uint8_t b[MxTile::BN * MxTile::KS];
    uint8_t sa[2][MxTile::BM];    // scale bytes of the stage's two 32-K blocks
    uint8_t sb[2][MxTile::BN];
    uint8_t dummy[256];
};

struct MxCopier {
    rsrc_t ra, rb, rs;
    uint32_t va[2], vb[2], vs, s_base, s_step;
    int a_lds[2], b_lds[2], s_lds;

    __device__ __forceinline__ void copy(uint8_t* stage, int st) const {
        const uint32_t koff = uint32_t(st) * MxTile::KS;
#pragma unroll
        for (int i = 0; i < 2; ++i)
            __builtin_amdgcn_raw_ptr_buffer_load_lds(ra, (lds_ptr_t)(stage + a_lds[i]), 16, va[i], koff, 0, 0);
#pragma unroll
        for (int i = 0; i < 2; ++i)
            __builtin_amdgcn_raw_ptr_buffer_load_lds(rb, (lds_ptr_t)(stage + b_lds[i]), 16, vb[i], koff, 0, 0);
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_ptr_t)(stage + s_lds), 4, vs,
                                                 s_base + uint32_t(2 * st) * s_step, 0, 0);
    }
};

// Waves 0-1 copy the A scale runs of blocks 2 st + w, waves 2-3 those of B,
// waves 4-7 repeat wave 0's run into the dummy line (equal load counts).
__device__ __forceinline__ MxCopier make_mx_copier(const GemmArgs& args, const Tile& t, int wave, int lane,
                                                   int64_t n0) {
    typedef MxTile W;
    const int64_t K = args.K, M = args.M, N = args.N;
    MxCopier c;
    const int sub = lane >> 2, slot = lane & 3;
    const int64_t tile_rows = t.rows_valid - t.m0 < W::BM ? t.rows_valid - t.m0 : W::BM;   // >= 1
    c.ra = make_rsrc(t.A + t.m0 * K, uint32_t(tile_rows * K));
    c.rb = make_rsrc(t.B + n0 * K, uint32_t(W::BN * K));
#pragma unroll
    for (int i = 0; i < 2; ++i) {
        const int r0 = (wave * 2 + i) * 16, r = r0 + sub;
        const int chunk = slot ^ ((r >> 2) & 3);
        const int64_t row = r < tile_rows ? r : tile_rows - 1;      // clamp: loaded, never stored
        c.va[i] = uint32_t(row * K + chunk * 16);
        c.vb[i] = uint32_t(int64_t(r) * K + chunk * 16);
        c.a_lds[i] = int(offsetof(MxStage, a)) + r0 * W::KS;
        c.b_lds[i] = int(offsetof(MxStage, b)) + r0 * W::KS;
    }
    const int64_t kblocks = K / 32;
    const uint8_t* ea = reinterpret_cast<const uint8_t*>(args.sa);
    const uint8_t* eb = reinterpret_cast<const uint8_t*>(args.sb);
    if (wave < 2) {           // A: bytes of rows m0 + 4 lane .. +3 in block 2 st + wave
        c.rs = make_rsrc(ea, uint32_t(kblocks * M));
        c.vs = uint32_t(t.m0 + 4 * lane);
        c.s_base = uint32_t(wave * M);
        c.s_step = uint32_t(M);
        c.s_lds = int(offsetof(MxStage, sa)) + wave * W::BM;
    } else if (wave < 4) {    // B: rows n0 + 4 lane .. +3 in block 2 st + wave - 2
        c.rs = make_rsrc(eb, uint32_t(kblocks * N));
        c.vs = uint32_t(n0 + 4 * lane);
        c.s_base = uint32_t((wave - 2) * N);
        c.s_step = uint32_t(N);
        c.s_lds = int(offsetof(MxStage, sb)) + (wave - 2) * W::BN;
    } else {
        c.rs = make_rsrc(ea, uint32_t(kblocks * M));
        c.vs = uint32_t(t.m0 + 4 * lane);
        c.s_base = 0;
        c.s_step = uint32_t(M);
        c.s_lds = int(offsetof(MxStage, dummy));
    }
    return c;
}

template <int OUT_FP32>
__device__ __forceinline__ void gemm_mx_body(const GemmArgs& args) {
    typedef MxTile W;
    constexpr int FM = W::FM, FN = W::FN, STAGES = W::STAGES, L = W::LOADS_PER_WAVE;
    __shared__ __align__(16) uint8_t lds_raw[STAGES * sizeof(MxStage)];
    MxStage* ring = reinterpret_cast<MxStage*>(lds_raw);

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm = wave / W::WAVES_N, wn = wave % W::WAVES_N;
    const int64_t N = args.N, K = args.K;
    const int stages = int(K / W::KS);
    const Tile t = map_tile<W, int(GemmMode::Dense)>(args, blockIdx.x);
    if (!t.live) return;
    const int64_t n0 = int64_t(t.bn) * W::BN;
    const MxCopier cp = make_mx_copier(args, t, wave, lane, n0);
    const int64_t wrow0 = t.m0 + wm * FM * 32;
    const bool live = wrow0 < t.rows_valid;
    const int r = lane & 31, h = lane >> 5;
    // per-lane LDS offsets within a stage: chunks h and 2 + h of the lane's rows
    uint32_t oa[FM][2], ob[FN][2], osa[FM], osb[FN];
#pragma unroll
    for (int mi = 0; mi < FM; ++mi) {
        const int row = wm * FM * 32 + mi * 32 + r;
#pragma unroll
        for (int c = 0; c < 2; ++c)
            oa[mi][c] = uint32_t(offsetof(MxStage, a)) + uint32_t(row * W::KS + (((2 * c + h) ^ ((row >> 2) & 3)) << 4));
        osa[mi] = uint32_t(offsetof(MxStage, sa)) + uint32_t(h * W::BM + row);
    }
#pragma unroll
    for (int ni = 0; ni < FN; ++ni) {
        const int row = wn * FN * 32 + ni * 32 + r;
#pragma unroll
        for (int c = 0; c < 2; ++c)
            ob[ni][c] = uint32_t(offsetof(MxStage, b)) + uint32_t(row * W::KS + (((2 * c + h) ^ ((row >> 2) & 3)) << 4));
        osb[ni] = uint32_t(offsetof(MxStage, sb)) + uint32_t(h * W::BN + row);
    }

#pragma unroll
    for (int st = 0; st < STAGES - 1; ++st)
        cp.copy(reinterpret_cast<uint8_t*>(&ring[st]), st < stages ? st : stages - 1);

    v16f acc[FM][FN];
#pragma unroll
    for (int mi = 0; mi < FM; ++mi)
#pragma unroll
        for (int ni = 0; ni < FN; ++ni)
#pragma unroll
            for (int i = 0; i < 16; ++i) acc[mi][ni][i] = 0.f;

    int slot = 0, fill_slot = STAGES - 1;
    for (int cur = 0; cur < stages; ++cur) {
        wait_vmcnt<(STAGES - 2) * L>();   // this wave's copy of stage cur has landed
        __builtin_amdgcn_s_barrier();     // ... every wave's; the slot of cur - 1 is free
        const int fill = cur + STAGES - 1;
        cp.copy(reinterpret_cast<uint8_t*>(&ring[fill_slot]), fill < stages ? fill : stages - 1);
        if (live) {
            const uint8_t* sg = lds_raw + uint32_t(slot) * uint32_t(sizeof(MxStage));
            v8i a8[FM], b8[FN];
            int ea[FM], eb[FN];
#pragma unroll
            for (int mi = 0; mi < FM; ++mi) {
                const u32x4 lo = ld<u32x4>(sg + oa[mi][0]), hi = ld<u32x4>(sg + oa[mi][1]);
                a8[mi] = v8i{int(lo[0]), int(lo[1]), int(lo[2]), int(lo[3]), int(hi[0]), int(hi[1]), int(hi[2]), int(hi[3])};
                ea[mi] = sg[osa[mi]];
            }
#pragma unroll
            for (int ni = 0; ni < FN; ++ni) {
                const u32x4 lo = ld<u32x4>(sg + ob[ni][0]), hi = ld<u32x4>(sg + ob[ni][1]);
                b8[ni] = v8i{int(lo[0]), int(lo[1]), int(lo[2]), int(lo[3]), int(hi[0]), int(hi[1]), int(hi[2]), int(hi[3])};
                eb[ni] = sg[osb[ni]];
            }
#pragma unroll
            for (int mi = 0; mi < FM; ++mi)
#pragma unroll
                for (int ni = 0; ni < FN; ++ni)
                    // formats 0/0 = E4M3 x E4M3; B is the instruction's first operand
                    acc[mi][ni] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(b8[ni], a8[mi], acc[mi][ni], 0, 0,
                                                                                  0, eb[ni], 0, ea[mi]);
        }
        slot = slot == STAGES - 1 ? 0 : slot + 1;
        fill_slot = fill_slot == STAGES - 1 ? 0 : fill_slot + 1;
    }
    wait_vmcnt<0>();   // no copy may land after the workgroup's LDS is handed on

    const int n_lane = wn * FN * 32 + 4 * h;
#pragma unroll
    for (int mi = 0; mi < FM; ++mi) {
        const int64_t m = wrow0 + mi * 32 + r;
        if (m >= t.rows_valid) continue;
#pragma unroll
        for (int ni = 0; ni < FN; ++ni)
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int64_t idx = m * N + n0 + n_lane + ni * 32 + 8 * j;
                const v4f v = v4f{acc[mi][ni][4 * j], acc[mi][ni][4 * j + 1], acc[mi][ni][4 * j + 2],
                                  acc[mi][ni][4 * j + 3]};
                if (OUT_FP32) {
                    st<v4f>(static_cast<float*>(args.c) + idx, v);
                } else {
                    const uint32_t lo = bf16_bits(v[0]) | (bf16_bits(v[1]) << 16);
                    const uint32_t hi = bf16_bits(v[2]) | (bf16_bits(v[3]) << 16);
                    st<u32x2>(static_cast<uint16_t*>(args.c) + idx, u32x2{lo, hi});
                }
            }
    }
}

__global__ __launch_bounds__(MxTile::THREADS) void gemm_mx_o0_dense(GemmArgs args) { gemm_mx_body<0>(args); }
__global__ __launch_bounds__(MxTile::THREADS) void gemm_mx_o1_dense(GemmArgs args) { gemm_mx_body<1>(args); }

// One plain __global__ function per instantiation (kernel templates whose
// instantiations differ only in the tile shape lost their host stubs).
// tile id: 0 = BigTile, 1 = DecodeTile
#define FP8FG_GEMM_KERNELS(X)                                              \
    X(big_e0_b0_o0_dense, 0, 4, 2, 2, 2, 3, 0, 0, 0, 0)                    \
    X(big_e0_b0_o1_dense, 0, 4, 2, 2, 2, 3, 0, 0, 1, 0)                    \
    X(big_e0_b1_o0_dense, 0, 4, 2, 2, 2, 3, 0, 1, 0, 0)                    \
    X(big_e0_b1_o1_dense, 0, 4, 2, 2, 2, 3, 0, 1, 1, 0)                    \
    X(big_e0_b0_o0_contig, 0, 4, 2, 2, 2, 3, 0, 0, 0, 1)                   \
    X(big_e0_b0_o1_contig, 0, 4, 2, 2, 2, 3, 0, 0, 1, 1)                   \
    X(big_e0_b0_o0_masked, 0, 4, 2, 2, 2, 3, 0, 0, 0, 2)                   \
    X(big_e0_b0_o1_masked, 0, 4, 2, 2, 2, 3, 0, 0, 1, 2)                   \
    X(dec_e0_b0_o0_masked, 1, 2, 4, 1, 1, 3, 0, 0, 0, 2)                   \
    X(dec_e0_b0_o1_masked, 1, 2, 4, 1, 1, 3, 0, 0, 1, 2)                   \
    X(big_e1_b0_o0_dense, 0, 4, 2, 2, 2, 3, 1, 0, 0, 0)                    \
    X(big_e1_b0_o1_dense, 0, 4, 2, 2, 2, 3, 1, 0, 1, 0)                    \
    X(big_e1_b1_o0_dense, 0, 4, 2, 2, 2, 3, 1, 1, 0, 0)                    \
    X(big_e1_b1_o1_dense, 0, 4, 2, 2, 2, 3, 1, 1, 1, 0)                    \
    X(big_e1_b0_o0_contig, 0, 4, 2, 2, 2, 3, 1, 0, 0, 1)                   \
    X(big_e1_b0_o1_contig, 0, 4, 2, 2, 2, 3, 1, 0, 1, 1)                   \
    X(big_e1_b0_o0_masked, 0, 4, 2, 2, 2, 3, 1, 0, 0, 2)                   \
    X(big_e1_b0_o1_masked, 0, 4, 2, 2, 2, 3, 1, 0, 1, 2)                   \
    X(dec_e1_b0_o0_masked, 1, 2, 4, 1, 1, 3, 1, 0, 0, 2)                   \
    X(dec_e1_b0_o1_masked, 1, 2, 4, 1, 1, 3, 1, 0, 1, 2)

#define FP8FG_DEFINE_KERNEL(NAME, TILE, WM, WN, FM, FN, ST, E, BS, OF, MODE)                  \
    __global__ __launch_bounds__(kThreads) void gemm_##NAME(GemmArgs args) {                  \
        gemm_body<WM, WN, FM, FN, ST, E, BS, OF, MODE>(args);                                 \
    }
FP8FG_GEMM_KERNELS(FP8FG_DEFINE_KERNEL)
#undef FP8FG_DEFINE_KERNEL

struct KernelEntry {
    void (*fn)(GemmArgs);
    int tile, engine, bscale, out_fp32, mode, threads;
};

#define FP8FG_ENTRY(NAME, TILE, WM, WN, FM, FN, ST, E, BS, OF, MODE) {gemm_##NAME, TILE, E, BS, OF, MODE, kThreads},
const KernelEntry kKernels[] = {FP8FG_GEMM_KERNELS(FP8FG_ENTRY)};
#undef FP8FG_ENTRY

// wide exact kernels, exact engine, 128x128 B scales, N a multiple of 256:
// tile id 2 = WideTile, 3 = WideDecodeTile
#define FP8FG_WIDE_KERNELS(X)                       \
    X(wide_o0_dense, WideTile, 2, 0, 0)             \
    X(wide_o1_dense, WideTile, 2, 1, 0)             \
    X(wide_o0_contig, WideTile, 2, 0, 1)            \
    X(wide_o1_contig, WideTile, 2, 1, 1)            \
    X(wide_o0_masked, WideTile, 2, 0, 2)            \
    X(wide_o1_masked, WideTile, 2, 1, 2)            \
    X(wdec_o0_masked, WideDecodeTile, 3, 0, 2)      \
    X(wdec_o1_masked, WideDecodeTile, 3, 1, 2)      \
    X(wide_o2_dense, WideTile, 2, 2, 0)
#define FP8FG_DEFINE_WIDE(NAME, CFG, TILE, OF, MODE)                                   \
    __global__ __launch_bounds__(CFG::THREADS) void gemm_##NAME(GemmArgs args) {       \
        __shared__ __align__(16) uint8_t lds[wide_lds_bytes<CFG>()];                   \
        gemm_wide_body<CFG, OF, MODE>(args, lds, blockIdx.x, -1);                     \
    }
FP8FG_WIDE_KERNELS(FP8FG_DEFINE_WIDE)
#undef FP8FG_DEFINE_WIDE
#define FP8FG_WIDE_ENTRY(NAME, CFG, TILE, OF, MODE) {gemm_##NAME, TILE, 0, 0, OF, MODE, CFG::THREADS},
const KernelEntry kWideKernels[] = {FP8FG_WIDE_KERNELS(FP8FG_WIDE_ENTRY)};
#undef FP8FG_WIDE_ENTRY

// the masked decode tile on decode-tiled B (fp8_grouped_gemm_masked_tiled)
__global__ __launch_bounds__(WideDecodeTile::THREADS) void gemm_wdect_o0_masked(GemmArgs args) {
    __shared__ __align__(16) uint8_t lds[wide_lds_bytes<WideDecodeTile>()];
    gemm_wide_body<WideDecodeTile, 0, int(GemmMode::Masked), true>(args, lds, blockIdx.x, -1);
}
__global__ __launch_bounds__(WideDecodeTile::THREADS) void gemm_wdect_o1_masked(GemmArgs args) {
    __shared__ __align__(16) uint8_t lds[wide_lds_bytes<WideDecodeTile>()];
    gemm_wide_body<WideDecodeTile, 1, int(GemmMode::Masked), true>(args, lds, blockIdx.x, -1);
}

// The decode-tiled weight layout, 16 bytes per thread in output order.  Output
// byte block blk (16 KB) = (g * N/256 + t) * (K/64) + h holds n-tile t of
// expert g (rows 256 t .. 256 t + 255) for K bytes 64 h .. 64 h + 63: row r of
// the n-tile at bytes 64 r .. 64 r + 63, whose 16-byte position s holds K chunk
// s ^ ((r >> 2) & 3) of the half-block -- the order the decode tile's stage
// keeps in LDS.
__global__ __launch_bounds__(256) void tile_weights_decode(const uint8_t* __restrict__ q, int64_t K, int64_t units,
                                                           uint8_t* __restrict__ out) {
    const int64_t halves = K / 64;
    for (int64_t u = int64_t(blockIdx.x) * 256 + threadIdx.x; u < units; u += int64_t(gridDim.x) * 256) {
        const int64_t blk = u >> 10;
        const int within = int(u & 1023), r = within >> 2, sl = within & 3;
        const int64_t gt = blk / halves, h = blk - gt * halves;
        const int c = sl ^ ((r >> 2) & 3);
        st<u32x4>(out + u * 16, ld<u32x4>(q + (gt * 256 + r) * K + h * 64 + c * 16));
    }
}

template <class C>
int64_t tile_count(GemmMode mode, const GemmArgs& args) {
    const int64_t n_tiles = (args.N + C::BN - 1) / C::BN;
    if (mode == GemmMode::Masked) return args.G * ((args.M + C::BM - 1) / C::BM) * n_tiles;
    if (mode == GemmMode::Contig) return (args.M / C::BM + args.G) * n_tiles;
    return ((args.M + C::BM - 1) / C::BM) * n_tiles;
}

// The wide kernel addresses its operands through buffer descriptors with
// 32-bit byte ranges: a 256-row slice of A or B (256 K bytes) and the A scale
// array ((K / 128) * rows * 4 bytes) must each stay below 4 GiB, and its n-tile
// is 256 wide.
bool wide_fits(const GemmArgs& args) {
    if (args.N % WideTile::BN != 0 || args.K >= (int64_t(1) << 24)) return false;
    return ((args.K + BK - 1) / BK) * args.M * 4 <= int64_t(0xFFFFFFFF);
}

// FP8FG_GEMM_WIDE=0 keeps the big tile for everything (comparison runs)
bool wide_enabled() {
    const char* e = getenv("FP8FG_GEMM_WIDE");
    return !(e && e[0] == '0');
}

// gfx950 (MI350 series): eight XCDs, each with its own L2
constexpr int kXcds = 8;
// FP8FG_GEMM_XCD=0 keeps the masked layout's tiles in plain rank order (comparison runs)
bool xcd_order_enabled() {
    const char* e = getenv("FP8FG_GEMM_XCD");
    return !(e && e[0] == '0');
}
// the masked layout's XCD grouping for tiles of bm rows: on when 8 divides the
// (expert, m-tile) pair count
int masked_xcds(const GemmArgs& args, int64_t bm) {
    return xcd_order_enabled() && (args.G * ((args.M + bm - 1) / bm)) % kXcds == 0 ? kXcds : 1;
}

// compute units of the current device (queried once per device)
int cu_count() {
    static int cache[64] = {0};
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 0;
    if (cache[dev] == 0) {
        int n = 0;
        if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return 0;
        cache[dev] = n;
    }
    return cache[dev];
}

// FP8FG_GEMM_TAIL: unset -> plan tail tiles when they fill whole rounds;
// "0" -> never; "force" -> whenever the columns split as 256 a + 192 b, b > 0
// (read at every call; "force" exists to exercise the tail tiles on small shapes)
int tail_mode() {
    const char* e = getenv("FP8FG_GEMM_TAIL");
    if (e && strcmp(e, "0") == 0) return 0;
    if (e && strcmp(e, "force") == 0) return 2;
    return 1;
}

// Split of a dense wide grid into 256 x 256 tiles over columns [0, n_split)
// and 256 x 192 tail tiles over [n_split, N).  Planned only when the 256 x 256
// grid leaves a partial last round and both kinds fill whole rounds on the
// device's CUs (a tail tile costs about 0.8 of a full one).
bool plan_tail(const GemmArgs& args, int64_t& tiles1, int64_t& tiles2, int64_t& n_split) {
    const int mode = tail_mode();
    if (mode == 0 || args.N % 256 != 0) return false;
    const int64_t mt = (args.M + WideTile::BM - 1) / WideTile::BM, nt = args.N / 256;
    bool found = false;
    if (mode == 2) {
        for (int64_t a = nt - 1; a >= 0 && !found; --a)
            if ((args.N - 256 * a) % TailCfg::BN == 0) {
                tiles1 = mt * a;
                tiles2 = mt * ((args.N - 256 * a) / TailCfg::BN);
                n_split = 256 * a;
                found = true;
            }
        return found;
    }
    const int64_t cus = cu_count();
    if (cus <= 0 || (mt * nt) % cus == 0) return false;
    double best = 0.97 * double((mt * nt + cus - 1) / cus);
    for (int64_t a = 0; a < nt; ++a) {
        const int64_t rem = args.N - 256 * a;
        if (rem % TailCfg::BN) continue;
        const int64_t t1 = mt * a, t2 = mt * (rem / TailCfg::BN);
        if (t1 % cus || t2 % cus) continue;
        const double cost = double(t1 / cus) + 0.8 * double(t2 / cus);
        if (cost < best) {
            best = cost;
            tiles1 = t1;
            tiles2 = t2;
            n_split = 256 * a;
            found = true;
        }
    }
    return found;
}

hipError_t dispatch(int engine, GemmMode mode, int bscale_1x128, int out_fp32, const GemmArgs& args,
                    hipStream_t stream) {
    // the exact engine on 128x128-scaled B with N a multiple of 256 runs the
    // wide kernel: 64 x 256 tiles for decode-sized masked buffers (at most
    // 128 rows), 256 x 256 tiles otherwise.  The rest (1x128 B scales, the
    // FP8-MFMA engine, N = 128 mod 256) runs the fold kernel: 64 x 128 tiles
    // for decode-sized masked buffers, 256 x 128 tiles otherwise.
    // the FP8 output mode exists only in the wide exact kernel (the entry point
    // checks that it fits)
    const bool wide = out_fp32 == 2 || (engine == 0 && !bscale_1x128 && wide_fits(args) && wide_enabled());
    if (out_fp32 == 2) engine = 0;
    int64_t tiles1 = 0, tiles2 = 0, n_split = 0;
    if (wide && mode == GemmMode::Dense && out_fp32 != 2 && args.M > 0 && plan_tail(args, tiles1, tiles2, n_split)) {
        hipLaunchKernelGGL(out_fp32 ? gemm_wmix_o1_dense : gemm_wmix_o0_dense, dim3(unsigned(tiles1 + tiles2)),
                           dim3(WideTile::THREADS), 0, stream, args, tiles1, n_split);
        return hipGetLastError();
    }
    int tile = 0;
    if (mode == GemmMode::Masked && args.M <= 128)
        tile = wide ? 3 : 1;
    else if (wide)
        tile = 2;
    const int64_t tiles = tile == 0   ? tile_count<BigTile>(mode, args)
                          : tile == 1 ? tile_count<DecodeTile>(mode, args)
                          : tile == 2 ? tile_count<WideTile>(mode, args)
                                      : tile_count<WideDecodeTile>(mode, args);
    if (tiles == 0) return hipSuccess;
    GemmArgs a = args;
    if (mode == GemmMode::Masked)
        a.xcds = masked_xcds(args, tile == 0   ? BigTile::BM
                                   : tile == 1 ? DecodeTile::BM
                                   : tile == 2 ? WideTile::BM
                                               : WideDecodeTile::BM);
    auto launch = [&](const KernelEntry& k) -> bool {
        if (k.tile == tile && k.engine == engine && k.bscale == bscale_1x128 && k.out_fp32 == out_fp32 &&
            k.mode == int(mode)) {
            hipLaunchKernelGGL(k.fn, dim3(unsigned(tiles)), dim3(k.threads), 0, stream, a);
            return true;
        }
        return false;
    };
    for (const KernelEntry& k : kKernels)
        if (launch(k)) return hipGetLastError();
    for (const KernelEntry& k : kWideKernels)
        if (launch(k)) return hipGetLastError();
    return hipErrorInvalidValue;
}

// FP8FG_GEMM_ENGINE: unset or "exact" -> 0, "fp8mfma" -> 1 (read at every call)
int engine_from_env() {
    const char* e = getenv("FP8FG_GEMM_ENGINE");
    return (e && strcmp(e, "fp8mfma") == 0) ? 1 : 0;
}

hipError_t launch_mx(int out_fp32, const GemmArgs& args, hipStream_t stream) {
    const int64_t tiles = ((args.M + MxTile::BM - 1) / MxTile::BM) * (args.N / MxTile::BN);
    if (tiles == 0) return hipSuccess;
    hipLaunchKernelGGL(out_fp32 ? gemm_mx_o1_dense : gemm_mx_o0_dense, dim3(unsigned(tiles)), dim3(MxTile::THREADS),
                       0, stream, args);
    return hipGetLastError();
}

hipError_t launch_masked_tiled(int out_fp32, const GemmArgs& args, hipStream_t stream) {
    const int64_t tiles = tile_count<WideDecodeTile>(GemmMode::Masked, args);
    if (tiles == 0) return hipSuccess;
    GemmArgs a = args;
    a.xcds = masked_xcds(args, WideDecodeTile::BM);
    hipLaunchKernelGGL(out_fp32 ? gemm_wdect_o1_masked : gemm_wdect_o0_masked, dim3(unsigned(tiles)),
                       dim3(WideDecodeTile::THREADS), 0, stream, a);
    return hipGetLastError();
}

hipError_t launch_tile_decode(const uint8_t* q, int64_t G, int64_t N, int64_t K, uint8_t* out, hipStream_t stream) {
    const int64_t units = G * N * (K / 16);
    if (units == 0) return hipSuccess;
    const int64_t blocks = (units + 255) / 256;
    hipLaunchKernelGGL(tile_weights_decode, dim3(unsigned(blocks < 65536 ? blocks : 65536)), dim3(256), 0, stream, q,
                       K, units, out);
    return hipGetLastError();
}

}  // namespace gemm_detail

hipError_t launch_gemm_masked_tiled(int out_fp32, const GemmArgs& args, hipStream_t stream) {
    return gemm_detail::launch_masked_tiled(out_fp32, args, stream);
}

hipError_t launch_tile_weights_decode(const uint8_t* q, int64_t G, int64_t N, int64_t K, uint8_t* out,
                                      hipStream_t stream) {
    return gemm_detail::launch_tile_decode(q, G, N, K, out, stream);
}

hipError_t launch_gemm_mx(int out_fp32, const GemmArgs& args, hipStream_t stream) {
    return gemm_detail::launch_mx(out_fp32, args, stream);
}

hipError_t launch_gemm(GemmMode mode, int bscale_1x128, int out_fp32, const GemmArgs& args,
                       hipStream_t stream) {
    return gemm_detail::dispatch(gemm_detail::engine_from_env(), mode, bscale_1x128, out_fp32, args, stream);
}

}  // namespace fp8fg
