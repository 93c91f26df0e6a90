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
//   exact   -- each FP8 fragment is widened to BF16 in registers (exact: BF16
//           holds every E4M3 value) and eight chained v_mfma_f32_32x32x16_bf16
//           form P_kb.  This MFMA adds exact products with IEEE FP32
//           round-to-nearest, so P_kb is an FP32-accurate block sum, which is
//           what the promotion assumes.  Every entry point but one.
//   fp8mfma -- two chained v_mfma_f32_32x32x64_f8f6f4 per K-block straight
//           from the FP8 codes, at twice the MFMA rate.  gfx950's FP8 MFMAs
//           add their products in groups of eight consecutive K, truncating
//           each product to 13 fractional bits below the group's largest
//           exponent (about 14 significant bits: the kind of limited
//           accumulation the pages measured on H800, here inside a single
//           instruction), so promotion every 128 cannot restore FP32 accuracy
//           and this engine is held to a looser bound.  Only the dense entry
//           point fp8_gemm_blockscaled_fp8mfma runs it.
//
// Kernels, by what they serve:
//   gemm_wide_*   exact engine, 128x128-scaled B, N % 256 == 0, at most 92
//                 K-blocks: dense and contiguous (256 x 256 tiles, the
//                 interleaved schedule), long masked buffers (256 x 256), and
//                 decode-sized masked buffers (gemm_wdec_*, 64 x 256 tiles);
//                 the promotion is folded into the MFMA accumulator (below).
//   gemm_dreg_*   persistent decode kernel on weights in the decode-tiled
//                 layout (written by tile_weights_decode): register-streamed
//                 weight fragments, the wide kernel's arithmetic; also with
//                 the fused FP8 output and with MX operands.
//   gemm_big_* / gemm_dec_*   the fold kernels described next: 1x128-scaled
//                 B (Wgrad), the fp8mfma engine, N = 128 mod 256, and K
//                 beyond the wide kernel's limit.
//   gemm_mx_*     the MX variant (E8M0 scales applied inside the MFMA), dense,
//                 contiguous and masked.
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
    int64_t g;            // the tile's expert (0 in the dense layout)
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
    if (MODE == int(GemmMode::Dense) && args.xcds > 1 && tile < ((args.M + BM - 1) / BM) * n_tiles) {
        // Workgroup w runs on XCD w mod xcds, and the workgroups of one XCD
        // start in order of w.  XCD x takes the x-th run of Q = T / xcds
        // consecutive tiles (T tiles in all; the last T mod xcds keep their
        // index) of an order that walks groups of GM m-tiles column by
        // column, so the tiles an XCD runs at once form a compact block
        // (4 x 8 for 32 CUs) whose A and B rows its L2 shares.  A bijection
        // on [0, T): the bits are those of the plain order.
        constexpr int64_t GM = 4;
        const int64_t m_tiles = (args.M + BM - 1) / BM, T = m_tiles * n_tiles, X = args.xcds, Q = T / X;
        const int64_t L = tile < Q * X ? (tile % X) * Q + tile / X : tile;
        const int64_t full = (m_tiles / GM) * GM * n_tiles;   // tiles in whole groups
        int64_t mt, bn;
        if (L < full) {
            const int64_t rem = L % (GM * n_tiles);
            bn = rem / GM;
            mt = (L / (GM * n_tiles)) * GM + rem % GM;
        } else {
            const int64_t h = m_tiles - (m_tiles / GM) * GM, rem = L - full;   // the last, shorter group
            bn = rem / h;
            mt = (m_tiles / GM) * GM + rem % h;
        }
        tile = mt * n_tiles + bn;
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
    t.g = g;
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

// C stores of one 32x32 MFMA tile row.  Lane l holds row l % 32 and, for
// j = 0..3, the run of four columns 8 j + 4 (l / 32) .. + 3, so lanes r and
// r + 32 hold the two halves of each run of eight columns 8 j .. 8 j + 7.  One
// swap across the wave's halves gives lane r both halves of runs 0 and 2 and
// lane r + 32 both halves of runs 1 and 3: each lane then writes two runs of
// eight columns (at 16 pr + 8 h) in place of four runs of four, half the
// store instructions, each twice as wide.  Both lanes of a pair hold the same
// row, so a per-row mask keeps the pair together; every lane of the wave that
// is still active must take part in the swap.  d[j] holds the lane's packed
// words of run j; p points at the tile's column 0 in the lane's row; runs at
// or past `cols` are not written (`cols` a multiple of 8).
template <int W>
__device__ __forceinline__ void pair_runs(uint32_t (&d)[4][W]) {
#pragma unroll
    for (int pr = 0; pr < 2; ++pr)
#pragma unroll
        for (int q = 0; q < W; ++q) {
            const auto sw = __builtin_amdgcn_permlane32_swap(d[2 * pr][q], d[2 * pr + 1][q], false, false);
            d[2 * pr][q] = sw[0];
            d[2 * pr + 1][q] = sw[1];
        }
}

__device__ __forceinline__ void store_bf16_runs(uint16_t* p, int h, uint32_t (&d)[4][2], int cols = 32) {
    pair_runs<2>(d);
#pragma unroll
    for (int pr = 0; pr < 2; ++pr)
        if (16 * pr + 8 * h < cols)
            st<u32x4>(p + 16 * pr + 8 * h, u32x4{d[2 * pr][0], d[2 * pr][1], d[2 * pr + 1][0], d[2 * pr + 1][1]});
}

__device__ __forceinline__ void store_fp8_runs(uint8_t* p, int h, uint32_t (&d)[4][1]) {
    pair_runs<1>(d);
#pragma unroll
    for (int pr = 0; pr < 2; ++pr) st<u32x2>(p + 16 * pr + 8 * h, u32x2{d[2 * pr][0], d[2 * pr + 1][0]});
}

// BF16 C of one 32x32 MFMA tile written as 64-byte row segments.  After
// pair_runs lane l holds, of tile row l % 32, the runs of eight columns
// 2 pr + h (pr = 0, 1); a swap of 16-lane rows then gives the lanes with
// l % 16 = i the four runs of tile row i in one chunk and those of row i + 16
// in the other.  Each store then writes 64 contiguous bytes of 16 rows, not
// 32 bytes of 32 rows: half the L2 write requests.  p points at the tile's
// row 0, column 0; `rows` of its rows exist (rows past them take part in
// the swaps and store nothing).  Every lane of the wave must take part.
__device__ __forceinline__ void store_bf16_rows64(uint16_t* p, int64_t ldc, int lane, int64_t rows,
                                                  uint32_t (&d)[4][2]) {
    pair_runs<2>(d);
    uint32_t c0[4] = {d[0][0], d[0][1], d[1][0], d[1][1]}, c1[4] = {d[2][0], d[2][1], d[3][0], d[3][1]};
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        const auto sw = __builtin_amdgcn_permlane16_swap(c0[q], c1[q], false, false);
        c0[q] = sw[0];
        c1[q] = sw[1];
    }
    const int i = lane & 15, col = 8 * (lane >> 5) + 16 * ((lane >> 4) & 1);
    if (i < rows) st<u32x4>(p + i * ldc + col, u32x4{c0[0], c0[1], c0[2], c0[3]});
    if (i + 16 < rows) st<u32x4>(p + (i + 16) * ldc + col, u32x4{c1[0], c1[1], c1[2], c1[3]});
}

// FP32 C of one 32x32 MFMA tile written as 64-byte row segments.  Lane l
// holds, of tile row l % 32, the four runs j of four columns 8 j + 4 (l / 32)
// .. + 3 (v[j]).  A swap of 16-lane rows between runs 2 p and 2 p + 1 gives
// the lanes with l % 16 = i columns 16 p .. 16 p + 15 of tile row i in one
// chunk and of row i + 16 in the other: each store writes 64 contiguous bytes
// of 16 rows, not 32 bytes of 32.  p points at the tile's row 0, column 0;
// `rows` of its rows exist.  Every lane of the wave must take part.
__device__ __forceinline__ void store_f32_rows64(float* p, int64_t ldc, int lane, int64_t rows, v4f (&v)[4]) {
    const int i = lane & 15, col = 4 * (lane >> 5) + 8 * ((lane >> 4) & 1);
#pragma unroll
    for (int pr = 0; pr < 2; ++pr) {
        const u32x4 a = __builtin_bit_cast(u32x4, v[2 * pr]), b = __builtin_bit_cast(u32x4, v[2 * pr + 1]);
        uint32_t x[4], y[4];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const auto sw = __builtin_amdgcn_permlane16_swap(a[q], b[q], false, false);
            x[q] = sw[0];
            y[q] = sw[1];
        }
        if (i < rows) st<u32x4>(p + i * ldc + 16 * pr + col, u32x4{x[0], x[1], x[2], x[3]});
        if (i + 16 < rows) st<u32x4>(p + (i + 16) * ldc + 16 * pr + col, u32x4{y[0], y[1], y[2], y[3]});
    }
}

// BF16 bits of four accumulator values, two to a word
__device__ __forceinline__ void bf16_words(v4f v, uint32_t (&w)[2]) {
    w[0] = bf16_bits(v[0]) | (bf16_bits(v[1]) << 16);
    w[1] = bf16_bits(v[2]) | (bf16_bits(v[3]) << 16);
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
        for (int ni = 0; ni < FN; ++ni) {
            // runs of four or eight columns start on multiples of 4 and N % 16 == 0:
            // a run lies wholly before N or wholly after it
            const int64_t col0 = n0 + wn * FN * 32 + ni * 32;   // the 32x32 tile's column 0
            const int64_t cols = N - col0;                      // the same on every lane
            if (cols <= 0) continue;
            const int hh = lane >> 5;
            uint32_t d[4][2];
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const v4f v = v4f{acc[mi][ni][4 * j], acc[mi][ni][4 * j + 1], acc[mi][ni][4 * j + 2],
                                  acc[mi][ni][4 * j + 3]};
                if (OUT_FP32) {
                    if (8 * j + 4 * hh < cols) st<v4f>(static_cast<float*>(args.c) + t.c_base + m * N + col0 + 8 * j + 4 * hh, v);
                } else {
                    bf16_words(v, d[j]);
                }
            }
            if (!OUT_FP32)
                store_bf16_runs(static_cast<uint16_t*>(args.c) + t.c_base + m * N + col0, hh, d,
                                cols < 32 ? int(cols) : 32);
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
// This loop serves the masked layout; the dense and contiguous layouts run
// the interleaved schedule below (gemm_wide_il_body), same arithmetic.
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
// decode-sized masked buffers on plain weights: 64 x 256, waves 1 x 4 of
// 64 x 64, two workgroups per CU; every B code is widened once
typedef WCfg<1, 4, 2, 2, 3> WideDecodeTile;

template <class W>
struct alignas(16) WStage {
    uint8_t a[W::BM * W::KS];
    uint8_t b[W::BN * W::KS];
    float sa[W::BM];                    // A scales of the stage's K-block
    float sb[W::BN];                    // 64 copies of each n-block's scale (128x128 B), or
                                        // one scale per column (1x128 B)
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

template <class W>
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
    // `ahead` (dense copies only): the scale piece of half-block h carries the
    // scales of the NEXT K-block, h / 2 + 1, so they sit in LDS a whole
    // K-block before they are applied (the first block's come another way).
    // The pieces of the last K-block then lie past the scale array and read
    // zeros (range-checked buffer loads); they are never used.
    // Piece i of copy(stage, h, pos, false, true): the A pieces, then the B
    // pieces, then the scale piece -- so that a copy can be spread over a
    // half-block's MFMAs instead of issued in one burst.
    __device__ __forceinline__ void copy_piece(uint8_t* stage, int h, int i) const {
        const uint32_t koff = uint32_t(h) * W::KS;
        if (i < W::A_PER_WAVE)
            __builtin_amdgcn_raw_ptr_buffer_load_lds(ra, (lds_ptr_t)(stage + a_lds[i]), 16, va[i], koff, 0, 0);
        else if (i < W::A_PER_WAVE + W::B_PER_WAVE)
            __builtin_amdgcn_raw_ptr_buffer_load_lds(rb, (lds_ptr_t)(stage + b_lds[i - W::A_PER_WAVE]), 16,
                                                     vb[i - W::A_PER_WAVE], koff, 0, 0);
        else
            __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_ptr_t)(stage + s_lds), 4, vs,
                                                     uint32_t((h >> 1) + 1) * s_step, 0, 0);
    }

    __device__ __forceinline__ void copy(uint8_t* stage, int h, int pos, bool sparse, bool ahead = false) const {
        const uint32_t koff = uint32_t(h) * W::KS;
        const uint32_t skb = uint32_t(ahead ? (h >> 1) + 1 : h >> 1);
        if (!(sparse && skip_a)) {
#pragma unroll
            for (int i = 0; i < W::A_PER_WAVE; ++i)
                __builtin_amdgcn_raw_ptr_buffer_load_lds(ra, (lds_ptr_t)(stage + a_lds[i]), 16, va[i], koff, 0, 0);
        }
#pragma unroll
        for (int i = 0; i < W::B_PER_WAVE; ++i)
            __builtin_amdgcn_raw_ptr_buffer_load_lds(rb, (lds_ptr_t)(stage + b_lds[i]), 16, vb[i], koff, 0, 0);
        if (!sparse || (has_scale && (pos & 1) == 0))
            __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_ptr_t)(stage + s_lds), 4, vs, skb * s_step, 0, 0);
    }
};

template <class W>
__device__ __forceinline__ WideBufCopier<W> make_wide_buf_copier(const Tile& t, int wave, int lane, int64_t K,
                                                                 int64_t n0) {
    typedef WStage<W> S;
    WideBufCopier<W> c;
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
        c.vb[i] = uint32_t(int64_t(r) * K + chunk * 16);
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
    bool zero[FM];           // the row's codes must read as +0 (its A scale or the B scale is 0); a
                             // lane mask, so it takes scalar registers, not vector ones
    // 1x128 B (one scale per column): the exponent part and zero flag of the
    // column each B fragment of the lane holds (n-tile g: column 32 g + r of
    // the wave's); `unit` is then the A part alone
    float pbn[4];
    int zbm;                 // bit g: that column's scale is 0 (its codes read as +0)
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

// (BS1: plus each wave's column arrays, 1536 bytes)
template <class W, bool BS1 = false>
constexpr uint32_t wide_lds_bytes() { return uint32_t(W::STAGES * sizeof(WStage<W>) + 64 + (BS1 ? W::NW * 1536 : 0)); }

// OUT: 0 = BF16, 1 = FP32, 2 = FP8 codes + 1x128 scales along N (dense only).
// `lds_raw` holds wide_lds_bytes<W>(); the workgroup computes tile `tile` of
// the n-tiles covering columns [0, n_ext) (n_ext < 0: all N).
template <class W, int OUT, int MODE>
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
    const WideBufCopier<W> cp = make_wide_buf_copier<W>(t, wave, lane, K, n0);
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
            for (int ni = 0; ni < FN; ++ni) {
                uint32_t d[4][1];
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const v4f v = v4f{acc[mi][ni][4 * j], acc[mi][ni][4 * j + 1], acc[mi][ni][4 * j + 2],
                                      acc[mi][ni][4 * j + 3]} * w.unit[mi];
                    d[j][0] = encode4(v, sc, rc);
                }
                store_fp8_runs(static_cast<uint8_t*>(args.c) + m * N + n0 + wn * FN * 32 + ni * 32, h, d);
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
        for (int ni = 0; ni < FN; ++ni) {
            uint32_t d[4][2];
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int64_t idx = t.c_base + m * N + n0 + n_lane + ni * 32 + 8 * j;
                const v4f v = v4f{acc[mi][ni][4 * j], acc[mi][ni][4 * j + 1], acc[mi][ni][4 * j + 2],
                                  acc[mi][ni][4 * j + 3]} * w.unit[mi];
                if (OUT == 1)
                    st<v4f>(static_cast<float*>(args.c) + idx, v);
                else
                    bf16_words(v, d[j]);
            }
            if (OUT == 0) store_bf16_runs(static_cast<uint16_t*>(args.c) + t.c_base + m * N + n0 + wn * FN * 32 + ni * 32, h, d);
        }
    }
}

// ---------------------------------------------------------------------------
// Copies of the interleaved schedule.  Only the first CW waves of the
// workgroup copy operand data (AP A pieces and BP B pieces of 1 KB each per
// half-block); every wave keeps its scale piece.  The first waves of a
// workgroup are the older ones on each SIMD, and the SIMD's issue arbiter
// favours them: measured, they finish a half-block's MFMAs far ahead of the
// younger waves and wait at the barrier, so a copy stalled on a full address
// queue costs them slack instead of costing the younger waves MFMA issue.
template <class W, int CW>
struct IlCopier {
    static constexpr int AP = W::BM / W::ROWS_PER_PIECE / CW, BP = W::BN / W::ROWS_PER_PIECE / CW;
    static_assert(AP * W::ROWS_PER_PIECE * CW == W::BM && BP * W::ROWS_PER_PIECE * CW == W::BN, "whole pieces");
    rsrc_t ra, rb, rs;
    // B pieces: every row lies in range, so piece i's offset is piece 0's
    // plus a uniform step, carried in the scalar offset (one VGPR, not BP)
    uint32_t va[AP], vb0, b_step, vs, s_step;
    int a_lds[AP], b_lds[BP], s_lds;
    int c16;   // the lane's 16-byte chunk within a row (the same in every piece: r0 % 16 == 0)
    int64_t K;
    bool copier;               // uniform: this wave copies operand data

    // piece i of half-block h: A pieces, then B pieces, then the scale piece,
    // which carries the NEXT K-block's scales (h / 2 + 1; past the end of the
    // scale array a range-checked load that reads zeros, never used)
    __device__ __forceinline__ void copy_piece(uint8_t* stage, int h, int i) const {
        const uint32_t koff = uint32_t(h) * W::KS;
        if (i < AP)
            __builtin_amdgcn_raw_ptr_buffer_load_lds(ra, (lds_ptr_t)(stage + a_lds[i]), 16, va[i], koff, 0, 0);
        else if (i < AP + BP)
            __builtin_amdgcn_raw_ptr_buffer_load_lds(rb, (lds_ptr_t)(stage + b_lds[i - AP]), 16, vb0,
                                                     koff + uint32_t(i - AP) * b_step, 0, 0);
        else
            __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_ptr_t)(stage + s_lds), 4, vs,
                                                     uint32_t((h >> 1) + 1) * s_step, 0, 0);
    }
    // the whole of this wave's share of half-block h
    __device__ __forceinline__ void copy(uint8_t* stage, int h) const {
        if (copier) {
#pragma unroll
            for (int i = 0; i < AP + BP; ++i) copy_piece(stage, h, i);
        }
        copy_piece(stage, h, AP + BP);
    }
    // after this wave's loads of half-block h have landed: zero its 16-byte
    // slots past K (a partial last K-block; the loads read whatever lies
    // there -- the next row, or zeros past the buffer's range)
    __device__ __forceinline__ void zero_tail(uint8_t* stage, int h, int lane) const {
        if (!copier) return;
        if (int64_t(h) * W::KS + c16 < K) return;
#pragma unroll
        for (int i = 0; i < AP; ++i) st<u32x4>(stage + a_lds[i] + lane * 16, u32x4{0u, 0u, 0u, 0u});
#pragma unroll
        for (int i = 0; i < BP; ++i) st<u32x4>(stage + b_lds[i] + lane * 16, u32x4{0u, 0u, 0u, 0u});
    }
};

template <class W, int CW, bool BS1 = false>
__device__ __forceinline__ IlCopier<W, CW> make_il_copier(const Tile& t, int wave, int lane, int64_t K, int64_t N,
                                                          int64_t n0) {
    typedef WStage<W> S;
    typedef IlCopier<W, CW> C;
    C c;
    c.K = K;
    c.copier = wave < CW;
    const int cw = c.copier ? wave : 0;     // non-copying waves set up (unused) offsets of wave 0
    const int sub = lane >> 2, slot = lane & 3;
    const int64_t tile_rows = t.rows_valid - t.m0 < W::BM ? t.rows_valid - t.m0 : W::BM;   // >= 1
    c.ra = make_rsrc(t.A + t.m0 * K, uint32_t(tile_rows * K));
    c.rb = make_rsrc(t.B + n0 * K, uint32_t(W::BN * K));
    // row r = r0 + sub of a piece holds the lane's chunk at slot ^ ((r >> 2) & 3),
    // and with r0 % 16 == 0 (sub < 16) that is slot ^ ((sub >> 2) & 3) in every piece
    static_assert(W::ROWS_PER_PIECE % 16 == 0, "one swizzle phase per piece");
    c.c16 = (slot ^ ((sub >> 2) & 3)) * 16;
#pragma unroll
    for (int i = 0; i < C::AP; ++i) {
        const int r0 = (cw * C::AP + i) * W::ROWS_PER_PIECE, r = r0 + sub;
        const int64_t row = r < tile_rows ? r : tile_rows - 1;      // clamp: loaded, never stored
        c.va[i] = uint32_t(row * K + c.c16);
        c.a_lds[i] = int(offsetof(S, a)) + r0 * W::KS;
    }
#pragma unroll
    for (int i = 0; i < C::BP; ++i) {
        const int r0 = (cw * C::BP + i) * W::ROWS_PER_PIECE, r = r0 + sub;
        if (i == 0) c.vb0 = uint32_t(int64_t(r) * K + c.c16);
        c.b_lds[i] = int(offsetof(S, b)) + r0 * W::KS;
    }
    c.b_step = uint32_t(W::ROWS_PER_PIECE * K);
    const int64_t kbs = (K + BK - 1) / BK;
    if (wave < W::A_SCALE_WAVES) {        // A scales of rows 64 wave .. +63 (clamped)
        const int64_t rr = int64_t(wave) * 64 + lane;
        const int64_t row = rr < tile_rows ? rr : tile_rows - 1;
        c.rs = make_rsrc(t.SA + t.m0, uint32_t(((kbs - 1) * t.lda_s + tile_rows) * 4));
        c.vs = uint32_t(row * 4);
        c.s_step = uint32_t(t.lda_s * 4);
        c.s_lds = int(offsetof(S, sa)) + wave * 64 * 4;
    } else if (BS1 && wave < W::A_SCALE_WAVES + W::BN / 64) {   // 64 column scales ([K/128][N], 1x128 B)
        static_assert(!BS1 || W::A_SCALE_WAVES + W::BN / 64 <= W::NW, "a scale piece per wave at most");
        const int j = wave - W::A_SCALE_WAVES;
        c.rs = make_rsrc(t.SB + n0 + 64 * j, uint32_t(((kbs - 1) * N + 64) * 4));
        c.vs = uint32_t(lane * 4);
        c.s_step = uint32_t(N * 4);
        c.s_lds = int(offsetof(S, sb)) + j * 64 * 4;
    } else if (!BS1 && wave < W::A_SCALE_WAVES + W::B_SCALE_WAVES) {   // 64 copies of an n-block's scale
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
constexpr int IL_COPY_WAVES = 4;

// ---------------------------------------------------------------------------
// Interleaved schedule of the wide exact kernel (dense and contiguous layouts).
//
// Measured on gfx950 (one 32x32x16 BF16 MFMA every 32 cycles per SIMD, with
// one or two waves): up to about six independent VALU instructions issue
// under each MFMA at no cost -- widening cvts and rescale multiplies alike --
// and eight cost a third more.  The exact engine needs about six per MFMA
// (three cvts, two rescale multiplies, scale and address arithmetic), so the
// schedule must spread them evenly; the loop above bunches them (the rescale
// multiplies of a whole K-block between a barrier and the first MFMA).  In a
// timestamped run of that loop on 4096 x 7168 x 2048, waves spent a third of
// each half-block in the barrier and in issuing the copies right after it.
// This schedule:
//   - one barrier per K-block: the ring's four half-block slots hold K-blocks
//     kb and kb + 1; kb + 1's copies are issued piece by piece between the
//     MFMAs of kb's even half-block (not in a burst after a barrier) into the
//     slots of kb - 1, so that each has at least a half-block to land;
//   - MFMAs run in groups of IL_GW n-tiles (all four k-steps of a half-block,
//     the group's FM x IL_GW tiles taking turns): the A fragments of a
//     half-block are used by every group, a group's B fragments only by it,
//     so each cvt runs just before its first use;
//   - a tile's rescale may run anywhere between its last MFMA of K-block kb-1
//     and its first of kb: the first half of the groups rescale in the odd
//     half-block of kb-1 (after their MFMAs), the others in the even
//     half-block of kb (before theirs), 64 multiplies per half-block;
//   - the scale piece of each stage carries the NEXT K-block's scales
//     (copy(ahead)), so the ratios and cvt exponents of K-block kb+1 are
//     computed in the last group of kb's even half-block; the first
//     K-block's scales are read from global memory before the loop;
//   - an odd half-block's A fragments and first group's B fragments are read
//     from LDS during the even half-block (into registers its first group has
//     finished with), so the odd half-block starts without an LDS burst;
//   - the K-block's barrier itself sits in the odd half-block before it, 14
//     MFMAs before its end, and each wave reads the new K-block's first
//     fragments right after it: the even half-block starts without an LDS
//     burst too (with 1x128 B only A's are read there: its loop has no
//     registers for B's);
//   - a compile-time plan (make_il_plan) gives every cvt and multiply a slot,
//     the gap after one MFMA: at most IL_CAP VALU instructions per slot, cvts
//     one MFMA before their first use, a tile's multiplies two MFMAs after its
//     last one; sched_barrier(0) fences keep the program order the plan sets.
// Same arithmetic in the same order per output element as gemm_wide_body:
// bit-identical results (tested).
constexpr int IL_CAP = 6;
constexpr int IL_GW = 2;   // n-tiles per group: FM x IL_GW accumulators in flight

// slot -1 = before the first MFMA; slot n = right after MFMA n.  MFMA n of a
// half-block is (group G, k-step k, m-tile mi, n-tile 2G + p) with
// n = G (4 FM GW) + k (FM GW) + mi GW + p: within a group the FM x GW tiles
// take turns, so consecutive MFMAs on one accumulator are FM x GW apart.
template <int FM, int FN>
struct IlPlan {
    static constexpr int NS = 4 * FM * FN;
    signed char a[FM][4][4];      // cvt q (one dword) of A fragment (mi, k)
    signed char b[FN][4][4];      // cvt q of B fragment (g, k)
    signed char m[FM][FN][16];    // rescale multiply of element i of tile (mi, g); -2: none in this half
    signed char rb[FN][4];        // 1x128 B: LDS read of the column ratios of elements 4q .. 4q + 3 of
                                  // n-tile g (two slots before their first multiply); -2: none
};

// mul_cost: VALU instructions per rescaled element (2 with 1x128 B: the row
// ratio and the column ratio)
template <int FM, int FN>
constexpr IlPlan<FM, FN> make_il_plan(bool odd, int scale_slot, int scale_ops, int mul_cost = 1,
                                       int slot_cap = IL_CAP) {
    constexpr int NS = IlPlan<FM, FN>::NS, GW = IL_GW, NG = FN / GW, PG = 4 * FM * GW;
    IlPlan<FM, FN> p{};
    int cap[NS] = {};
    for (int n = 0; n < NS; ++n) cap[n] = slot_cap;
    // the scale arithmetic of the next K-block (even half-blocks) takes room in
    // the slots from scale_slot on
    for (int n = scale_slot, left = scale_ops; n < NS && left > 0; ++n) {
        const int take = left < cap[n] ? left : cap[n];
        cap[n] -= take;
        left -= take;
    }
    // cvts first, each as late as possible but one MFMA before its first use
    // (latest use first); what finds no room runs before MFMA 0 (slot -1)
    auto late = [&](int hi) -> int {
        for (int n = hi; n >= 0; --n)
            if (cap[n] > 0) {
                --cap[n];
                return n;
            }
        return -1;
    };
    for (int n = NS - 1; n >= 0; --n) {
        const int G = n / PG, k = (n % PG) / (FM * GW), mi = (n % (FM * GW)) / GW, pp = n % GW;
        if (mi == 0)
            for (int q = 3; q >= 0; --q) p.b[G * GW + pp][k][q] = (signed char)late(n - 1);
        if (G == 0 && pp == 0)
            for (int q = 3; q >= 0; --q) p.a[mi][k][q] = (signed char)late(n - 1);
    }
    // then the multiplies, each tile's sixteen as early as its window allows
    // in the room left (a window that is full spills to its last slot): the
    // first NG/2 groups after their last MFMA of an odd half-block, the others
    // before their first MFMA of an even one
    auto early = [&](int lo, int hi) -> int {
        for (int n = lo < 0 ? 0 : lo; n <= hi; ++n)
            if (cap[n] >= mul_cost) {
                cap[n] -= mul_cost;
                return n;
            }
        return hi;
    };
    // (elements in runs of four columns, both m-tiles of a run together: with
    // 1x128 B a run shares one LDS read of its column ratios)
    for (int g = 0; g < FN; ++g)
        for (int qq = 0; qq < 16; qq += 4)
        for (int mi = 0; mi < FM; ++mi)
            for (int i = qq; i < qq + 4; ++i) {
                const int G = g / GW, first = G * PG + mi * GW + g % GW, last = first + 3 * FM * GW;
                if (odd && G < NG / 2)
                    p.m[mi][g][i] = (signed char)early(last + 2, NS - 1);
                else if (!odd && G >= NG / 2)
                    p.m[mi][g][i] = (signed char)early(0, first - 1);
                else
                    p.m[mi][g][i] = -2;
            }
    for (int g = 0; g < FN; ++g)
        for (int q = 0; q < 4; ++q) {
            int first = NS;
            for (int mi = 0; mi < FM; ++mi)
                for (int i = 4 * q; i < 4 * q + 4; ++i)
                    if (p.m[mi][g][i] != -2 && p.m[mi][g][i] < first) first = p.m[mi][g][i];
            p.rb[g][q] = (signed char)(first == NS ? -2 : (first - 2 < -1 ? -1 : first - 2));
        }
    return p;
}

// the first slot of any cvt of k-steps 2 and 3 (chunk column 1) of A or of
// the first group's B (the plan's)
template <int FM, int FN>
constexpr int il_first_k2_cvt(const IlPlan<FM, FN>& p) {
    int first = IlPlan<FM, FN>::NS;
    for (int k = 2; k < 4; ++k)
        for (int q = 0; q < 4; ++q) {
            for (int mi = 0; mi < FM; ++mi)
                if (p.a[mi][k][q] < first) first = p.a[mi][k][q];
            for (int g = 0; g < IL_GW; ++g)
                if (p.b[g][k][q] < first) first = p.b[g][k][q];
        }
    return first;
}

// the last slot of any rescale multiply (the plan's; -1 if none)
template <int FM, int FN>
constexpr int il_last_mul(const IlPlan<FM, FN>& p) {
    int last = -1;
    for (int mi = 0; mi < FM; ++mi)
        for (int g = 0; g < FN; ++g)
            for (int i = 0; i < 16; ++i)
                if (p.m[mi][g][i] > last) last = p.m[mi][g][i];
    return last;
}

// the first slot of any B cvt of n-tiles g0 and later (the plan's)
template <int FM, int FN>
constexpr int il_first_b_cvt(const IlPlan<FM, FN>& p, int g0) {
    int first = IlPlan<FM, FN>::NS;
    for (int g = g0; g < FN; ++g)
        for (int k = 0; k < 4; ++k)
            for (int q = 0; q < 4; ++q)
                if (p.b[g][k][q] < first) first = p.b[g][k][q];
    return first;
}

// one dword (two BF16 values) of a widened fragment: codes of bytes
// 2 (q & 1) .. +1 of word q >> 1 of the 8-byte half hh of a 16-byte chunk
__device__ __forceinline__ uint32_t widen_q(const u32x4& raw, int hh, int q, float p2) {
    const int wd = int(raw[2 * hh + (q >> 1)]);
    return __builtin_bit_cast(uint32_t, (q & 1) ? __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(wd, p2, true)
                                                : __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(wd, p2, false));
}

// The 16-byte chunk j (k-steps 2 j and 2 j + 1) of fragment row `row` (of
// the A part at `part` = offsetof(WStage, a), or of B) from LDS slot sl, as
// the lane reads it in a half-block; `zero`: the zero line instead.
template <class W>
__device__ __forceinline__ u32x4 il_frag(const uint8_t* lds, uint32_t sl, uint32_t part, int row, int r, int h,
                                         int j, bool zero, uint32_t zero_line) {
    const uint32_t ch = uint32_t(((2 * j + h) ^ ((r >> 2) & 3)) << 4);
    const uint32_t at = sl * uint32_t(sizeof(WStage<W>)) + part + uint32_t(row * W::KS) + ch;
    return ld<u32x4>(lds + (zero ? zero_line + ch : at));
}

// Even half-blocks also turn the stage's scale piece (the next K-block's
// scales) into `next`: its LDS reads go out with the fragment reads, its
// arithmetic runs in four slots of the last group, whose room the plan keeps.
// With 1x128 B (BS1) the accumulator unit is the A part alone and each
// column carries its own ratio: every rescaled element takes two multiplies,
// by its row's ratio and by its column's, read four at a time from this
// wave's private LDS arrays (`cl`: ratios of two transitions, by parity, then
// the columns' current mantissa parts); the column ratios of the next
// transition are computed here (even half-blocks), two columns per lane.  No
// fragments are read ahead for the odd half-block (no registers for them).
template <class W, int ODD, bool COPIER, bool BS1, class Sync>
__device__ __forceinline__ void wide_il_half(uint8_t* lds, int slot, int wm, int wn, int r, int h,
                                             const WideScales<W::FM>& w, float (&ratio)[W::FM],
                                             uint32_t zero_line, v16f (&acc)[W::FM][W::FN],
                                             WideScales<W::FM>& next, const IlCopier<W, IL_COPY_WAVES>& cp,
                                             int fill_slot, int fill_h, int fill2_slot, int fill2_h, int pf_slot,
                                             u32x4 (&pfa)[W::FM][2],
                                             u32x4 (&pfb)[IL_GW][2], uint32_t cl, int rpar, int wpar, bool more,
                                             int lane, u32x4 (&ea)[W::FM], u32x4 (&eb)[IL_GW], const Sync& sync) {
#if defined(__HIP_DEVICE_COMPILE__)   // device code only: the host pass never runs it
    constexpr int IL_SCALE_OPS = 32;
    constexpr int FM = W::FM, FN = W::FN, NS = 4 * FM * FN, SS = NS - 12;
    static_assert(FN % 2 == 0 && FM == 2 && FN <= 4, "plan shape");
    constexpr IlPlan<FM, FN> P = make_il_plan<FM, FN>(ODD != 0, SS, ODD ? 0 : IL_SCALE_OPS, BS1 ? 2 : 1,
                                                      BS1 ? 9 : IL_CAP);
    constexpr bool PREFETCH = !BS1;   // odd half-blocks' first fragments read during the even one
    // the even half-block turns `ratio` into the next transition's at slot
    // SS + 3, after its own multiplies (by the current one) are all done
    static_assert(ODD || il_last_mul(P) <= SS + 3, "ratio replaced before the even half-block's last multiply");
    // The K-block's barrier sits in the odd half-block before it, after MFMA
    // SYNC_AT: there each wave waits for its copies of the next K-block,
    // meets the others, and reads that K-block's first fragments (chunk
    // column 0 of A, into ea, and without 1x128 B of the first group's B, into
    // eb; the 1x128-B loop has no registers for eb) while the last MFMAs of
    // this one run on registers.  So no wave starts a K-block waiting on all
    // of its first reads.  Every read of this K-block's slots comes before
    // SYNC_AT (the odd half-block's own reads by RB_AT, the rest during the
    // even one), so the copies that follow the barrier may overwrite them.
    constexpr bool LOB_B = !BS1;
    constexpr int SYNC_AT = 4 * FM * FN - 14;
    const WStage<W>& sg = *reinterpret_cast<const WStage<W>*>(lds + uint32_t(slot) * uint32_t(sizeof(WStage<W>)));
    float nsa[FM], nsb = 0.0f;
    if (!ODD) {
        // (the wave's n-block scale: one value, kept in a scalar register)
        if (!BS1) nsb = __builtin_bit_cast(float, __builtin_amdgcn_readfirstlane(
                            __builtin_bit_cast(int, sg.sb[((wn * FN * 32) / 128) * 64])));
#pragma clang loop unroll(full)
        for (int mi = 0; mi < FM; ++mi) nsa[mi] = sg.sa[wm * FM * 32 + mi * 32 + r];
    }
    ScaleSplit nb{}, na[FM] = {};
    uint32_t ch[2];
#pragma clang loop unroll(full)
    for (int j = 0; j < 2; ++j) ch[j] = uint32_t(((2 * j + h) ^ ((r >> 2) & 3)) << 4);
    // fragment reads: the A rows and the B rows of n-tile g from LDS slot `sl`
    auto read_a = [&](uint32_t sl, int mi, int j) -> u32x4 {
        const uint32_t at = sl * uint32_t(sizeof(WStage<W>)) + uint32_t(offsetof(WStage<W>, a)) +
                            uint32_t((wm * FM * 32 + mi * 32 + r) * W::KS) + ch[j];
        return ld<u32x4>(lds + (w.zero[mi] ? zero_line + ch[j] : at));
    };
    auto read_b = [&](uint32_t sl, int g, int j) -> u32x4 {
        const uint32_t bt = sl * uint32_t(sizeof(WStage<W>)) + uint32_t(offsetof(WStage<W>, b)) +
                            uint32_t((wn * FN * 32 + g * 32 + r) * W::KS) + ch[j];
        // a column whose 1x128 scale is 0 reads as +0, like a zero-scaled A row
        return ld<u32x4>(lds + (BS1 && ((w.zbm >> g) & 1) ? zero_line + ch[j] : bt));
    };
    // An odd half-block's A fragments and its first group's B fragments were
    // read during the even half-block before it (the K-block's barrier covers
    // both slots); the rest is read here.  The even one reads all of its own.
    // The B fragments of the later groups are read only after MFMA RB_AT:
    // right after the K-block's barrier all eight waves read at once, and
    // fewer reads in that burst let every wave start its MFMAs sooner (the
    // plan's first cvt of a later group comes well after RB_AT).
    constexpr int RB_AT = 6;
    static_assert(il_first_b_cvt(P, IL_GW) > RB_AT, "later groups' B read before their first cvt");
    // Of the fragments read here, only chunk column 0 (k-steps 0 and 1, the
    // first eight MFMAs) is read before MFMA 0; chunk column 1 follows it (the
    // plan's first cvt of k-steps 2 and 3 comes later), which halves the
    // eight waves' read burst that every wave waits on after the barrier.
    constexpr bool READ_HERE = !(ODD && PREFETCH);
    static_assert(il_first_k2_cvt(P) > 0, "chunk column 1 read before its first cvt");
    u32x4 ra[FM][2], rb[FN][2];
#pragma clang loop unroll(full)
    for (int mi = 0; mi < FM; ++mi) {
        ra[mi][0] = READ_HERE ? (!ODD ? ea[mi] : read_a(uint32_t(slot), mi, 0)) : pfa[mi][0];
        if (!READ_HERE) ra[mi][1] = pfa[mi][1];
    }
#pragma clang loop unroll(full)
    for (int g = 0; g < IL_GW; ++g) {
        rb[g][0] = READ_HERE ? (LOB_B && !ODD ? eb[g] : read_b(uint32_t(slot), g, 0)) : pfb[g][0];
        if (!READ_HERE) rb[g][1] = pfb[g][1];
    }
    u32x4 ca[FM][4], cb[FN][4];
    v4f rbq[FN][4];   // 1x128 B: column ratios of elements 4q .. 4q + 3 of n-tile g
    // the VALU work planned for slot n
    auto valu = [&](int n) {
#pragma clang loop unroll(full)
        for (int mi = 0; mi < FM; ++mi)
#pragma clang loop unroll(full)
            for (int k = 0; k < 4; ++k)
#pragma clang loop unroll(full)
                for (int q = 0; q < 4; ++q)
                    if (P.a[mi][k][q] == n) ca[mi][k][q] = widen_q(ra[mi][k >> 1], k & 1, q, w.pa[mi]);
#pragma clang loop unroll(full)
        for (int g = 0; g < FN; ++g)
#pragma clang loop unroll(full)
            for (int k = 0; k < 4; ++k)
#pragma clang loop unroll(full)
                for (int q = 0; q < 4; ++q)
                    if (P.b[g][k][q] == n) cb[g][k][q] = widen_q(rb[g][k >> 1], k & 1, q, BS1 ? w.pbn[g] : w.pb);
        if (BS1) {
#pragma clang loop unroll(full)
            for (int g = 0; g < FN; ++g)
#pragma clang loop unroll(full)
                for (int q = 0; q < 4; ++q)
                    if (P.rb[g][q] == n)
                        rbq[g][q] = ld<v4f>(lds + cl + uint32_t(rpar) * 512u + uint32_t((g * 32 + 8 * q + 4 * h) * 4));
        }
#pragma clang loop unroll(full)
        for (int mi = 0; mi < FM; ++mi)
#pragma clang loop unroll(full)
            for (int g = 0; g < FN; ++g)
#pragma clang loop unroll(full)
                for (int i = 0; i < 16; ++i)
                    if (P.m[mi][g][i] == n) {
                        if (BS1)
                            acc[mi][g][i] *= ratio[mi] * rbq[g][i >> 2][i & 3];
                        else
                            acc[mi][g][i] *= ratio[mi];
                    }
    };
    // this wave's share of the copies of half-blocks fill_h and fill2_h (the
    // two halves of the next K-block, both in the even half-block so that the
    // last piece lands a whole half-block before the K-block's wait; the odd
    // half-block copies nothing): one piece of each every PSTRIDE MFMAs, the
    // last piece of each the scale piece, data only on copying waves
    typedef IlCopier<W, IL_COPY_WAVES> Cp;
    constexpr int PIECES = COPIER ? Cp::AP + Cp::BP + 1 : 1, PSTRIDE = NS / PIECES;
    static_assert(PSTRIDE >= 3, "two fills interleaved one MFMA apart");
    uint8_t* fill_stage = lds + uint32_t(fill_slot) * uint32_t(sizeof(WStage<W>));
    uint8_t* fill2_stage = lds + uint32_t(fill2_slot) * uint32_t(sizeof(WStage<W>));
    valu(-1);
    __builtin_amdgcn_sched_barrier(0);
#pragma clang loop unroll(full)
    for (int n = 0; n < NS; ++n) {
        constexpr int PG = 4 * FM * IL_GW;
        const int k = (n % PG) / (FM * IL_GW), mi = (n % (FM * IL_GW)) / IL_GW, g = (n / PG) * IL_GW + n % IL_GW;
        acc[mi][g] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(v8bf, cb[g][k]),
                                                             __builtin_bit_cast(v8bf, ca[mi][k]), acc[mi][g], 0, 0, 0);
        // The waves that do not copy are the younger ones on each SIMD, which
        // lose issue arbitration to the older.  In the even half-block, while
        // the older waves issue the next K-block's copies, they take the
        // higher wave priority (measured: Wgrad 2% and the dense GEMM 1%
        // faster; raising it in the odd half-block as well gains nothing for
        // Wgrad and costs the dense GEMM 1%, in the odd one only 3%).
        if (!COPIER && !ODD && n == 0) __builtin_amdgcn_s_setprio(1);
        if (!COPIER && !ODD && n == NS - 1) __builtin_amdgcn_s_setprio(0);
        if (ODD && n == SYNC_AT) {
            static_assert(SYNC_AT > RB_AT, "this K-block's slots read after the barrier");
            // (after the last K-block the reads still go out, of a slot no
            // one uses again: ea / eb are then dead once the even half-block
            // has taken them, not held through it)
            if (more) sync();
            const uint32_t nsl = uint32_t((slot + 1) & 3);   // the next K-block's even slot
#pragma clang loop unroll(full)
            for (int mi = 0; mi < FM; ++mi)
                ea[mi] = il_frag<W>(lds, nsl, uint32_t(offsetof(WStage<W>, a)), wm * FM * 32 + mi * 32 + r, r, h,
                                    0, next.zero[mi] != 0, zero_line);
#pragma clang loop unroll(full)
            for (int g = 0; g < (LOB_B ? IL_GW : 0); ++g)
                eb[g] = il_frag<W>(lds, nsl, uint32_t(offsetof(WStage<W>, b)), wn * FN * 32 + g * 32 + r, r, h, 0,
                                   false, zero_line);
        }
        if (READ_HERE && n == 0) {
#pragma clang loop unroll(full)
            for (int mi = 0; mi < FM; ++mi) ra[mi][1] = read_a(uint32_t(slot), mi, 1);
#pragma clang loop unroll(full)
            for (int g = 0; g < IL_GW; ++g) rb[g][1] = read_b(uint32_t(slot), g, 1);
        }
        if (n == RB_AT) {
#pragma clang loop unroll(full)
            for (int g = IL_GW; g < FN; ++g)
#pragma clang loop unroll(full)
                for (int j = 0; j < 2; ++j) rb[g][j] = read_b(uint32_t(slot), g, j);
        }
        if (!ODD && n % PSTRIDE == 1 && n / PSTRIDE < PIECES)
            cp.copy_piece(fill_stage, fill_h, COPIER ? n / PSTRIDE : Cp::AP + Cp::BP);
        if (!ODD && n % PSTRIDE == 2 && n / PSTRIDE < PIECES)
            cp.copy_piece(fill2_stage, fill2_h, COPIER ? n / PSTRIDE : Cp::AP + Cp::BP);
        if (PREFETCH && !ODD && n == NS / 2 + 2) {
            // the odd half-block's first fragments, into registers the first
            // group of this one no longer needs
#pragma clang loop unroll(full)
            for (int mi = 0; mi < FM; ++mi)
#pragma clang loop unroll(full)
                for (int j = 0; j < 2; ++j) pfa[mi][j] = read_a(uint32_t(pf_slot), mi, j);
#pragma clang loop unroll(full)
            for (int g = 0; g < IL_GW; ++g)
#pragma clang loop unroll(full)
                for (int j = 0; j < 2; ++j) pfb[g][j] = read_b(uint32_t(pf_slot), g, j);
        }
        valu(n);
        if (!ODD && !BS1) {
            // the next K-block's scales, split as wide_scales does
            if (n == SS) nb = split_scale(nsb);
            if (n == SS + 1) na[0] = split_scale(nsa[0]);
            if (n == SS + 2) na[1] = split_scale(nsa[1]);
            if (n == SS + 3) {
                next.pb = nb.pow2;
#pragma clang loop unroll(full)
                for (int q = 0; q < FM; ++q) {
                    next.pa[q] = na[q].pow2;
                    next.unit[q] = clamp_unit(na[q].mant * nb.mant);
                    next.zero[q] = (nsa[q] == 0.0f || nsb == 0.0f) ? 1 : 0;
                    ratio[q] = more ? clamp_unit(w.unit[q] * __builtin_amdgcn_rcpf(next.unit[q])) : 1.0f;
                }
            }
        }
        if (!ODD && BS1) {
            // the next K-block's row scales (its column scales are taken
            // between the half-blocks, by dreg_columns)
            if (n == SS + 1) na[0] = split_scale(nsa[0]);
            if (n == SS + 2) na[1] = split_scale(nsa[1]);
            if (n == SS + 3) {
#pragma clang loop unroll(full)
                for (int q = 0; q < FM; ++q) {
                    next.pa[q] = na[q].pow2;
                    next.unit[q] = clamp_unit(na[q].mant);
                    next.zero[q] = nsa[q] == 0.0f ? 1 : 0;
                    ratio[q] = more ? clamp_unit(w.unit[q] * __builtin_amdgcn_rcpf(next.unit[q])) : 1.0f;
                }
            }
        }
        __builtin_amdgcn_sched_barrier(0);
    }
#endif
}

// 1x128 B, between the two half-blocks of K-block kb: the next K-block's
// column scales (its scale piece sits in the even slot `sg`) -- the B
// exponents and zero mask of the lane's fragment columns into `nw`, and the
// ratios of the transition into it for this wave's private array of parity
// `wpar` (two columns per lane; 1 where no K-block follows), with the
// columns' new mantissa parts
template <class W>
__device__ __forceinline__ void il_columns(const uint8_t* lds, const WStage<W>& sg, uint32_t cl, int wpar, bool more,
                                           int wn, int r, int lane, WideScales<W::FM>& nw) {
    constexpr int FN = W::FN;
    nw.zbm = 0;
#pragma unroll
    for (int g = 0; g < FN; ++g) {
        const float sb = sg.sb[wn * FN * 32 + g * 32 + r];
        nw.pbn[g] = split_scale(sb).pow2;
        nw.zbm |= (sb == 0.0f ? 1 : 0) << g;
    }
#pragma unroll
    for (int j = 0; j < 2; ++j) {
        const uint32_t col = uint32_t((64 * j + lane) * 4);
        const float mn = split_scale(sg.sb[wn * FN * 32 + 64 * j + lane]).mant;
        const float mo = ld<float>(lds + cl + 1024u + col);
        st<float>(const_cast<uint8_t*>(lds) + cl + uint32_t(wpar) * 512u + col,
                  more ? clamp_unit(mo * __builtin_amdgcn_rcpf(mn)) : 1.0f);
        if (more) st<float>(const_cast<uint8_t*>(lds) + cl + 1024u + col, mn);
    }
}

// The K-loop of gemm_wide_il_body for one copy role (a template parameter, so
// each role's half-blocks are straight-line code with its own copy slots).
template <class W, bool COPIER, bool BS1>
__device__ __forceinline__ void il_kloop(uint8_t* lds_raw, WStage<W>* ring, const IlCopier<W, IL_COPY_WAVES>& cp,
                                         int halves, int64_t K, int wm, int wn, int r, int h, int lane, bool live,
                                         WideScales<W::FM>& w, WideScales<W::FM>& nw, float (&ratio)[W::FM],
                                         v16f (&acc)[W::FM][W::FN], uint32_t cl) {
    constexpr int FM = W::FM;
    constexpr uint32_t kZeroLine = W::STAGES * sizeof(WStage<W>);
    u32x4 pfa[FM][2], pfb[IL_GW][2];   // an odd half-block's first fragments, read ahead

    // Waves whose rows all lie past the tile's valid rows only copy.  Their
    // loop is separate (`live` is uniform per wave), so the computing loop
    // carries no values merged from a path that skips the compute.
    if (!live) {
        for (int hb = 0; hb < halves; hb += 2) {
            wait_vmcnt<0>();
            if ((hb + 2) * W::KS > K) {
                cp.zero_tail(reinterpret_cast<uint8_t*>(&ring[hb & 3]), hb, lane);
                cp.zero_tail(reinterpret_cast<uint8_t*>(&ring[(hb + 1) & 3]), hb + 1, lane);
                asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
            }
            __builtin_amdgcn_s_barrier();
            const int f0 = hb + 2 < halves ? hb + 2 : halves - 1, f1 = hb + 3 < halves ? hb + 3 : halves - 1;
            cp.copy(reinterpret_cast<uint8_t*>(&ring[(hb + 2) & 3]), f0);
            cp.copy(reinterpret_cast<uint8_t*>(&ring[(hb + 3) & 3]), f1);
        }
        return;
    }
    // Both halves of K-block kb have landed (this wave's copies: the only
    // loads in flight), then every wave's; a partial last K-block's slots
    // are zeroed past K first.  This runs in the odd half-block of kb - 1
    // (wide_il_half), and before the loop for kb = 0.
    auto kblock_sync = [&](int hbk) {
        wait_vmcnt<0>();
        const bool partial = (hbk + 2) * W::KS > K;   // partial last K-block (uniform)
        if (partial) {
            cp.zero_tail(reinterpret_cast<uint8_t*>(&ring[hbk & 3]), hbk, lane);
            cp.zero_tail(reinterpret_cast<uint8_t*>(&ring[(hbk + 1) & 3]), hbk + 1, lane);
        }
        // (mid-K-block, this wave's reads of the slots the copies after the
        // barrier refill are all done as well)
        asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
        __builtin_amdgcn_s_barrier();
    };
    u32x4 ea[FM], eb[IL_GW];   // the next K-block's first fragments, read at its barrier
    {
        kblock_sync(0);
#pragma unroll
        for (int mi = 0; mi < FM; ++mi)
            ea[mi] = il_frag<W>(lds_raw, 0u, uint32_t(offsetof(WStage<W>, a)), wm * FM * 32 + mi * 32 + r, r, h, 0,
                                nw.zero[mi] != 0, kZeroLine);
#pragma unroll
        for (int g = 0; g < (BS1 ? 0 : IL_GW); ++g)
            eb[g] = il_frag<W>(lds_raw, 0u, uint32_t(offsetof(WStage<W>, b)), wn * W::FN * 32 + g * 32 + r, r, h, 0,
                               false, kZeroLine);
    }
    for (int hb = 0; hb < halves; hb += 2) {
        // the next K-block's halves (past the end: the last half again, into
        // slots never read again)
        const int f0 = hb + 2 < halves ? hb + 2 : halves - 1, f1 = hb + 3 < halves ? hb + 3 : halves - 1;
        w = nw;
        // the even slot's scale piece holds the next K-block's scales
        const bool more = hb + 2 < halves;
        const int par = (hb >> 1) & 1;   // K-block parity: column ratios of the transition into it
        const auto no_sync = [] {};
        const auto next_sync = [&] { kblock_sync(hb + 2); };
        wide_il_half<W, 0, COPIER, BS1>(lds_raw, hb & 3, wm, wn, r, h, w, ratio, kZeroLine, acc, nw, cp, (hb + 2) & 3,
                                        f0, (hb + 3) & 3, f1, (hb + 1) & 3, pfa, pfb, cl, par, par ^ 1, more, lane,
                                        ea, eb, no_sync);
        if (BS1) il_columns<W>(lds_raw, ring[hb & 3], cl, par ^ 1, more, wn, r, lane, nw);
        wide_il_half<W, 1, COPIER, BS1>(lds_raw, (hb + 1) & 3, wm, wn, r, h, w, ratio, kZeroLine, acc, nw, cp,
                                        0, 0, 0, 0, 0, pfa, pfb, cl, par ^ 1, par ^ 1, more, lane, ea, eb, next_sync);
    }
}

// BS1: B is 1x128-scaled (one scale per column and K-block, [K/128][N]: the
// Wgrad operand); dense layout, BF16 / FP32 out.
template <class W, int OUT, int MODE, bool BS1 = false>
__device__ __forceinline__ void gemm_wide_il_body(const GemmArgs& args, uint8_t* lds_raw, int64_t tile, int64_t n_ext) {
    static_assert(MODE != int(GemmMode::Masked), "dense and contiguous layouts");
    static_assert(!BS1 || (OUT != 2 && MODE == int(GemmMode::Dense)), "1x128 B: dense, BF16 / FP32 out");
    typedef WStage<W> S;
    constexpr int FM = W::FM, FN = W::FN, STAGES = W::STAGES;
    constexpr uint32_t kZeroLine = STAGES * sizeof(S);
    S* ring = reinterpret_cast<S*>(lds_raw);

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm = wave / W::WAVES_N, wn = wave % W::WAVES_N;
    const int64_t N = args.N, K = args.K;
    const int halves = int(2 * ((K + BK - 1) / BK));
    const Tile t = map_tile<W, MODE>(args, tile, n_ext);
    if (!t.live) return;
    const int64_t n0 = int64_t(t.bn) * W::BN;
    const IlCopier<W, IL_COPY_WAVES> cp = make_il_copier<W, IL_COPY_WAVES, BS1>(t, wave, lane, K, N, n0);
    const int64_t wrow0 = t.m0 + wm * FM * 32;
    const bool live = wrow0 < t.rows_valid;   // uniform
    const int r = lane & 31, h = lane >> 5;

    // the first K-block's scales, straight from global memory (rows clamped
    // as the copier clamps them)
    float sa0[FM];
#pragma unroll
    for (int mi = 0; mi < FM; ++mi) {
        int64_t row = wrow0 + mi * 32 + r;
        row = row < t.rows_valid ? row : t.rows_valid - 1;
        sa0[mi] = t.SA[row];
    }
    const float sb0 = BS1 ? 1.0f : t.SB[((n0 + wn * FN * 32) / 128) * ((K + BK - 1) / BK)];
    // 1x128 B: the first K-block's column scales -- of the lane's B fragments
    // (column 32 g + r of the wave's) and of its two columns of the ratio
    // arrays (lane, 64 + lane); this wave's private arrays sit after the zero
    // line: two K-block parities of column ratios, then the columns' current
    // mantissa parts
    const uint32_t cl = kZeroLine + 64u + uint32_t(wave) * 1536u;
    float sbn0[4] = {};
    if (BS1) {
#pragma unroll
        for (int g = 0; g < FN; ++g) sbn0[g] = t.SB[n0 + wn * FN * 32 + g * 32 + r];
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            const float mb0 = split_scale(t.SB[n0 + wn * FN * 32 + 64 * j + lane]).mant;
            st<float>(lds_raw + cl + uint32_t((64 * j + lane) * 4), 1.0f);           // parity 0: no transition
            st<float>(lds_raw + cl + 1024u + uint32_t((64 * j + lane) * 4), mb0);
        }
    }

    if (tid < 4) st<u32x4>(lds_raw + kZeroLine + tid * 16, u32x4{0u, 0u, 0u, 0u});
    // the ring holds four half-blocks: K-block kb in slots 2kb % 4 and
    // 2kb % 4 + 1; the copies of K-block kb + 1 run during the MFMAs of kb's
    // even half-block, into the slots of kb - 1, which every wave has
    // finished by kb's barrier
    static_assert(STAGES == 4, "two K-blocks of half-block slots");
    cp.copy(reinterpret_cast<uint8_t*>(&ring[0]), 0);
    cp.copy(reinterpret_cast<uint8_t*>(&ring[1]), 1);
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");

    v16f acc[FM][FN];
#pragma unroll
    for (int mi = 0; mi < FM; ++mi)
#pragma unroll
        for (int ni = 0; ni < FN; ++ni)
#pragma unroll
            for (int i = 0; i < 16; ++i) acc[mi][ni][i] = 0.f;
    // w: scales of the current K-block; nw: of the next one.  ratio[mi] moves
    // a tile from the unit of one K-block to the next's (exactly 1 where no
    // block follows: multiplying by 1 is exact)
    WideScales<FM> w, nw;
    {
        const ScaleSplit b = split_scale(sb0);
        nw.pb = b.pow2;
#pragma unroll
        for (int mi = 0; mi < FM; ++mi) {
            const ScaleSplit a = split_scale(sa0[mi]);
            nw.pa[mi] = a.pow2;
            nw.unit[mi] = clamp_unit(BS1 ? a.mant : a.mant * b.mant);
            nw.zero[mi] = (sa0[mi] == 0.0f || sb0 == 0.0f) ? 1 : 0;
        }
        nw.zbm = 0;
#pragma unroll
        for (int g = 0; g < 4; ++g) {
            nw.pbn[g] = split_scale(sbn0[g]).pow2;
            nw.zbm |= (sbn0[g] == 0.0f ? 1 : 0) << g;
        }
    }
    float ratio[FM];
#pragma unroll
    for (int mi = 0; mi < FM; ++mi) ratio[mi] = 1.0f;
    if (cp.copier)
        il_kloop<W, true, BS1>(lds_raw, ring, cp, halves, K, wm, wn, r, h, lane, live, w, nw, ratio, acc, cl);
    else
        il_kloop<W, false, BS1>(lds_raw, ring, cp, halves, K, wm, wn, r, h, lane, live, w, nw, ratio, acc, cl);
    wait_vmcnt<0>();

    if constexpr (OUT == 2) {
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
            for (int ni = 0; ni < FN; ++ni) {
                uint32_t d[4][1];
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const v4f v = v4f{acc[mi][ni][4 * j], acc[mi][ni][4 * j + 1], acc[mi][ni][4 * j + 2],
                                      acc[mi][ni][4 * j + 3]} * w.unit[mi];
                    d[j][0] = encode4(v, sc, rc);
                }
                store_fp8_runs(static_cast<uint8_t*>(args.c) + m * N + n0 + wn * FN * 32 + ni * 32, h, d);
            }
            if (h == 0) args.cs[(n0 / 128 + wn) * args.M + m] = sc;
        }
        return;
    }
    if constexpr (OUT == 0) {   // BF16, in 64-byte row segments (measured: 0.7-1.1% on 4096 x 7168 x 2048)
#pragma unroll
        for (int mi = 0; mi < FM; ++mi) {
            const int64_t m0 = wrow0 + mi * 32;
            if (m0 >= t.rows_valid) continue;   // uniform
#pragma unroll
            for (int ni = 0; ni < FN; ++ni) {
                uint32_t d[4][2];   // the four runs of four columns, two dwords each
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    v4f v = v4f{acc[mi][ni][4 * j], acc[mi][ni][4 * j + 1], acc[mi][ni][4 * j + 2],
                                acc[mi][ni][4 * j + 3]} * w.unit[mi];
                    if (BS1)   // the columns' last mantissa parts
                        v = v * ld<v4f>(lds_raw + cl + 1024u + uint32_t((ni * 32 + 8 * j + 4 * h) * 4));
                    bf16_words(v, d[j]);
                }
                store_bf16_rows64(static_cast<uint16_t*>(args.c) + t.c_base + m0 * N + n0 + wn * FN * 32 + ni * 32, N,
                                  lane, t.rows_valid - m0, d);
            }
        }
    } else {   // FP32, in 64-byte row segments
#pragma unroll
        for (int mi = 0; mi < FM; ++mi) {
            const int64_t m0 = wrow0 + mi * 32;
            if (m0 >= t.rows_valid) continue;   // uniform
#pragma unroll
            for (int ni = 0; ni < FN; ++ni) {
                v4f v[4];
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    v[j] = v4f{acc[mi][ni][4 * j], acc[mi][ni][4 * j + 1], acc[mi][ni][4 * j + 2],
                               acc[mi][ni][4 * j + 3]} * w.unit[mi];
                    if (BS1)   // the columns' last mantissa parts
                        v[j] = v[j] * ld<v4f>(lds_raw + cl + 1024u + uint32_t((ni * 32 + 8 * j + 4 * h) * 4));
                }
                store_f32_rows64(static_cast<float*>(args.c) + t.c_base + m0 * N + n0 + wn * FN * 32 + ni * 32, N, lane,
                                 t.rows_valid - m0, v);
            }
        }
    }
}

// the wide kernel's body for a layout: the interleaved schedule for the dense
// and contiguous layouts, the half-block loop for the masked one (whose
// decode tiles are bound by the weight stream, not by the MFMAs)
template <class W, int OUT, int MODE>
__device__ __forceinline__ void gemm_wide_sel(const GemmArgs& args, uint8_t* lds_raw, int64_t tile, int64_t n_ext) {
    if constexpr (MODE != int(GemmMode::Masked))
        gemm_wide_il_body<W, OUT, MODE>(args, lds_raw, tile, n_ext);
    else
        gemm_wide_body<W, OUT, MODE>(args, lds_raw, tile, n_ext);
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

// The same ring on block-scaled operands (the FP8-MFMA engine of
// fp8_gemm_blockscaled_fp8mfma): each stage carries its K-block's FP32 A
// scales (256 rows) and the two 128-column B scales instead of E8M0 bytes.
struct alignas(16) MxbsStage {
    uint8_t a[MxTile::BM * MxTile::KS];
    uint8_t b[MxTile::BN * MxTile::KS];
    float sa[MxTile::BM];
    float sb[64];                  // lanes 0, 1 of one load: n-blocks 2 bn, 2 bn + 1
    uint8_t dummy[256];
};

struct MxCopier {
    rsrc_t ra, rb, rs;
    uint32_t va[2], vb[2], vs, s_base, s_step;
    int a_lds[2], b_lds[2], s_lds;

    // BS: the scale run of stage st is that of K-block st / 2 (two 64-K
    // stages per block); MX: of the 32-K blocks 2 st and 2 st + 1
    template <bool BS = false>
    __device__ __forceinline__ void copy(uint8_t* stage, int st) const {
        const uint32_t koff = uint32_t(st) * MxTile::KS;
#pragma unroll
        for (int i = 0; i < 2; ++i)
            __builtin_amdgcn_raw_ptr_buffer_load_lds(ra, (lds_ptr_t)(stage + a_lds[i]), 16, va[i], koff, 0, 0);
#pragma unroll
        for (int i = 0; i < 2; ++i)
            __builtin_amdgcn_raw_ptr_buffer_load_lds(rb, (lds_ptr_t)(stage + b_lds[i]), 16, vb[i], koff, 0, 0);
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_ptr_t)(stage + s_lds), 4, vs,
                                                 s_base + uint32_t(BS ? st >> 1 : 2 * st) * s_step, 0, 0);
    }
};

// Waves 0-1 copy the A scale runs of blocks 2 st + w, waves 2-3 those of B,
// waves 4-7 repeat wave 0's run into the dummy line (equal load counts).
// Grouped layouts: expert g's B codes (t.B) and scale bytes [K/32][N] follow
// one another; in the masked layout so do its A rows (t.A) and A scale bytes
// [K/32][M_max], while the contiguous layout's A rows and scales are shared.
template <int MODE, bool BS = false>
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
    if constexpr (BS) {   // dense: waves 0-3 the A scales of rows 64 w .., wave 4 the two B scales
        const int64_t kbs = (K + 127) / 128;
        if (wave < 4) {
            c.rs = make_rsrc(args.sa, uint32_t(kbs * M * 4));
            c.vs = uint32_t((t.m0 + 64 * wave + lane) * 4);
            c.s_step = uint32_t(M * 4);
            c.s_lds = int(offsetof(MxbsStage, sa)) + wave * 256;
        } else if (wave == 4) {
            c.rs = make_rsrc(args.sb, uint32_t((N / 128) * kbs * 4));
            c.vs = uint32_t(((n0 / 128) + (lane < 2 ? lane : 0)) * kbs * 4);
            c.s_step = 4u;
            c.s_lds = int(offsetof(MxbsStage, sb));
        } else {
            c.rs = make_rsrc(args.sa, uint32_t(kbs * M * 4));
            c.vs = uint32_t((t.m0 + lane) * 4);
            c.s_step = uint32_t(M * 4);
            c.s_lds = int(offsetof(MxbsStage, dummy));
        }
        c.s_base = 0;
        return c;
    }
    const int64_t kblocks = K / 32;
    const uint8_t* ea = reinterpret_cast<const uint8_t*>(args.sa) + (MODE == int(GemmMode::Masked) ? t.g * kblocks * M : 0);
    const uint8_t* eb = reinterpret_cast<const uint8_t*>(args.sb) + t.g * kblocks * N;
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

// BS: block-scaled operands (1x128 A, 128x128 B, FP32 scales) on the FP8
// MFMA, the FP8-MFMA engine.  As in the exact wide kernel, each scale splits
// into a power of two and a mantissa part: the powers of two go to the
// instruction as E8M0 scale bytes, and the accumulator is kept in the unit of
// the mantissa parts' product, moved to the next K-block's unit at every
// K-block (the promotion folded into the accumulator).  Rows whose A scale
// (or whose B scale) is 0 read a zero line.
template <int OUT_FP32, int MODE, bool BS = false>
__device__ __forceinline__ void gemm_mx_body(const GemmArgs& args) {
    typedef MxTile W;
    typedef typename std::conditional<BS, MxbsStage, MxStage>::type Stage;
    static_assert(offsetof(MxbsStage, a) == offsetof(MxStage, a) && offsetof(MxbsStage, b) == offsetof(MxStage, b),
                  "one copier layout for the codes");
    constexpr int FM = W::FM, FN = W::FN, STAGES = W::STAGES, L = W::LOADS_PER_WAVE;
    constexpr uint32_t kZeroLine = STAGES * sizeof(Stage);
    __shared__ __align__(16) uint8_t lds_raw[STAGES * sizeof(Stage) + (BS ? 64 : 0)];
    Stage* ring = reinterpret_cast<Stage*>(lds_raw);

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm = wave / W::WAVES_N, wn = wave % W::WAVES_N;
    const int64_t N = args.N, K = args.K;
    const int stages = int(K / W::KS);
    const Tile t = map_tile<W, MODE>(args, blockIdx.x);
    if (!t.live) return;
    const int64_t n0 = int64_t(t.bn) * W::BN;
    const MxCopier cp = make_mx_copier<MODE, BS>(args, t, wave, lane, n0);
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
            oa[mi][c] = uint32_t(offsetof(Stage, a)) + uint32_t(row * W::KS + (((2 * c + h) ^ ((row >> 2) & 3)) << 4));
        osa[mi] = BS ? uint32_t(offsetof(MxbsStage, sa)) + uint32_t(row * 4)
                     : uint32_t(offsetof(MxStage, sa)) + uint32_t(h * W::BM + row);
    }
#pragma unroll
    for (int ni = 0; ni < FN; ++ni) {
        const int row = wn * FN * 32 + ni * 32 + r;
#pragma unroll
        for (int c = 0; c < 2; ++c)
            ob[ni][c] = uint32_t(offsetof(Stage, b)) + uint32_t(row * W::KS + (((2 * c + h) ^ ((row >> 2) & 3)) << 4));
        osb[ni] = BS ? 0u : uint32_t(offsetof(MxStage, sb)) + uint32_t(h * W::BN + row);
    }
    if constexpr (BS) {   // the zero line, written before the first barrier
        if (tid < 4) st<u32x4>(lds_raw + kZeroLine + tid * 16, u32x4{0u, 0u, 0u, 0u});
        asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    }

#pragma unroll
    for (int st = 0; st < STAGES - 1; ++st)
        cp.template copy<BS>(reinterpret_cast<uint8_t*>(&ring[st]), st < stages ? st : stages - 1);
    WideScales<FM> w;   // BS: the current K-block's exponent parts and unit

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
        cp.template copy<BS>(reinterpret_cast<uint8_t*>(&ring[fill_slot]), fill < stages ? fill : stages - 1);
        if (live) {
            const uint8_t* sg = lds_raw + uint32_t(slot) * uint32_t(sizeof(Stage));
            v8i a8[FM], b8[FN];
            int ea[FM], eb[FN];
            if constexpr (BS) {
                if ((cur & 1) == 0) {   // a new K-block: its scales came with this stage
                    WideScales<FM> nw;
                    const float sb = ld<float>(sg + offsetof(MxbsStage, sb) + wn * 4);
                    const ScaleSplit b = split_scale(sb);
                    nw.pb = b.pow2;
#pragma unroll
                    for (int mi = 0; mi < FM; ++mi) {
                        const float sa = ld<float>(sg + osa[mi]);
                        const ScaleSplit a = split_scale(sa);
                        nw.pa[mi] = a.pow2;
                        nw.unit[mi] = clamp_unit(a.mant * b.mant);
                        nw.zero[mi] = (sa == 0.0f || sb == 0.0f) ? 1 : 0;
                    }
                    if (cur > 0) rescale<FM, FN, FM>(acc, w, nw);
                    w = nw;
                }
            }
#pragma unroll
            for (int mi = 0; mi < FM; ++mi) {
                uint32_t o0 = oa[mi][0], o1 = oa[mi][1];
                if (BS && w.zero[mi]) {   // the chunk offsets within the zero line
                    o0 = kZeroLine - uint32_t(slot) * uint32_t(sizeof(Stage)) + (o0 & 63u);
                    o1 = kZeroLine - uint32_t(slot) * uint32_t(sizeof(Stage)) + (o1 & 63u);
                }
                const u32x4 lo = ld<u32x4>(sg + o0), hi = ld<u32x4>(sg + o1);
                a8[mi] = v8i{int(lo[0]), int(lo[1]), int(lo[2]), int(lo[3]), int(hi[0]), int(hi[1]), int(hi[2]), int(hi[3])};
                ea[mi] = BS ? int((__builtin_bit_cast(uint32_t, w.pa[mi]) >> 23) & 0xFF) : int(sg[osa[mi]]);
            }
#pragma unroll
            for (int ni = 0; ni < FN; ++ni) {
                const u32x4 lo = ld<u32x4>(sg + ob[ni][0]), hi = ld<u32x4>(sg + ob[ni][1]);
                b8[ni] = v8i{int(lo[0]), int(lo[1]), int(lo[2]), int(lo[3]), int(hi[0]), int(hi[1]), int(hi[2]), int(hi[3])};
                eb[ni] = BS ? int((__builtin_bit_cast(uint32_t, w.pb) >> 23) & 0xFF) : int(sg[osb[ni]]);
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
        const int64_t m0 = wrow0 + mi * 32, m = m0 + r;
        if (m0 >= t.rows_valid) continue;   // uniform
#pragma unroll
        for (int ni = 0; ni < FN; ++ni) {
            uint32_t d[4][2];
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int64_t idx = t.c_base + m * N + n0 + n_lane + ni * 32 + 8 * j;
                v4f v = v4f{acc[mi][ni][4 * j], acc[mi][ni][4 * j + 1], acc[mi][ni][4 * j + 2],
                            acc[mi][ni][4 * j + 3]};
                if (BS) v = v * w.unit[mi];
                if (OUT_FP32) {
                    if (m < t.rows_valid) st<v4f>(static_cast<float*>(args.c) + idx, v);
                } else {
                    bf16_words(v, d[j]);
                }
            }
            if (!OUT_FP32)
                store_bf16_rows64(static_cast<uint16_t*>(args.c) + t.c_base + m0 * N + n0 + wn * FN * 32 + ni * 32, N,
                                  lane, t.rows_valid - m0, d);
        }
    }
}

#define FP8FG_MX_KERNEL(OUT, NAME, MODE)                                                                  \
    __global__ __launch_bounds__(MxTile::THREADS) void gemm_mx_o##OUT##_##NAME(GemmArgs args) {          \
        gemm_mx_body<OUT, int(GemmMode::MODE)>(args);                                                    \
    }
FP8FG_MX_KERNEL(0, dense, Dense)
FP8FG_MX_KERNEL(1, dense, Dense)
FP8FG_MX_KERNEL(0, contig, Contig)
FP8FG_MX_KERNEL(1, contig, Contig)
FP8FG_MX_KERNEL(0, masked, Masked)
FP8FG_MX_KERNEL(1, masked, Masked)
#undef FP8FG_MX_KERNEL
// the FP8-MFMA engine on 128x128-scaled B in this tiling (dense)
__global__ __launch_bounds__(MxTile::THREADS) void gemm_mxbs_o0_dense(GemmArgs args) {
    gemm_mx_body<0, int(GemmMode::Dense), true>(args);
}
__global__ __launch_bounds__(MxTile::THREADS) void gemm_mxbs_o1_dense(GemmArgs args) {
    gemm_mx_body<1, int(GemmMode::Dense), true>(args);
}

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
    X(big_e1_b1_o1_dense, 0, 4, 2, 2, 2, 3, 1, 1, 1, 0)

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
    X(wide_o2_dense, WideTile, 2, 2, 0)             \
    X(wide_o2_contig, WideTile, 2, 2, 1)
#define FP8FG_DEFINE_WIDE(NAME, CFG, TILE, OF, MODE)                                   \
    __global__ __launch_bounds__(CFG::THREADS) void gemm_##NAME(GemmArgs args) {       \
        __shared__ __align__(16) uint8_t lds[wide_lds_bytes<CFG>()];                   \
        gemm_wide_sel<CFG, OF, MODE>(args, lds, blockIdx.x, -1);                      \
    }
FP8FG_WIDE_KERNELS(FP8FG_DEFINE_WIDE)
#undef FP8FG_DEFINE_WIDE
#define FP8FG_WIDE_ENTRY(NAME, CFG, TILE, OF, MODE) {gemm_##NAME, TILE, 0, 0, OF, MODE, CFG::THREADS},
const KernelEntry kWideKernels[] = {FP8FG_WIDE_KERNELS(FP8FG_WIDE_ENTRY)};
#undef FP8FG_WIDE_ENTRY

// the interleaved schedule on 1x128-scaled B (dense, Wgrad)
__global__ __launch_bounds__(WideTile::THREADS) void gemm_wide_b1_o0_dense(GemmArgs args) {
    __shared__ __align__(16) uint8_t lds[wide_lds_bytes<WideTile, true>()];
    gemm_wide_il_body<WideTile, 0, int(GemmMode::Dense), true>(args, lds, blockIdx.x, -1);
}
__global__ __launch_bounds__(WideTile::THREADS) void gemm_wide_b1_o1_dense(GemmArgs args) {
    __shared__ __align__(16) uint8_t lds[wide_lds_bytes<WideTile, true>()];
    gemm_wide_il_body<WideTile, 1, int(GemmMode::Dense), true>(args, lds, blockIdx.x, -1);
}
const KernelEntry kWideB1Kernels[] = {{gemm_wide_b1_o0_dense, 2, 0, 1, 0, int(GemmMode::Dense), WideTile::THREADS},
                                      {gemm_wide_b1_o1_dense, 2, 0, 1, 1, int(GemmMode::Dense), WideTile::THREADS}};


// ---------------------------------------------------------------------------
// Persistent masked decode kernel on decode-tiled weights (gemm_dreg_*):
// masked buffers of at most 128 rows per expert, exact engine, 128x128-scaled
// B, N % 256 == 0.
//
// Decode is bound by the weight stream: every expert's N x K codes are read
// once per call and each meets at most 64 valid rows.  An item is 64 rows of
// one expert's buffer (an m-tile holding valid rows) times 64 NW columns; a
// workgroup of NW waves computes it, wave w owning columns 64 w .. 64 w + 63
// of all 64 rows (2 x 2 MFMA tiles of 32 x 32).  NW is 8 or 7 (one workgroup
// per CU; the host takes the one whose items fill more CUs: 7168 columns make
// 16 items of 448 per expert but 14 of 512) when N allows, else 4 (two per
// CU): two workgroups on one CU do not share it evenly -- the older one's
// waves win the SIMDs' issue arbitration and finish well ahead, leaving the
// younger to stream alone -- while the waves of one workgroup stay in step
// at every half-block's barrier.
// Workgroup b of P takes items b, b + P, b + 2P, ... and walks them as one
// flat sequence of half-blocks (64 K), so the weight stream runs on from one
// item into the next without a pause; the host sizes P so that the
// workgroups get equal item counts when the experts are about equally full.
// B never passes through LDS: each lane loads its own MFMA fragments (16
// bytes per 32 x 32 tile and 32-wide K step) straight into registers, NP - 1
// half-blocks ahead of the one being multiplied -- an NP-deep register ring,
// the loop unrolled NP times so that ring positions are fixed registers --
// with the non-temporal hint: each weight byte is read once, and the hint
// measurably raised the stream rate (it keeps the weights from displacing
// the A rows and scales that the items share).  A (64 rows x 64 K per
// half-block, shared by the waves) rides an NP-slot LDS ring of
// direct-to-LDS loads, each A byte copied by one wave; each K-block's scales
// ride into registers with its first half.  Items are the live (expert,
// m-tile) pairs ranked heaviest first (the ranking of masked_pair_by_work)
// times the n-tiles; when eight divides the live pair count, all n-tiles of
// a pair go to one XCD, whose L2 then serves the A rows they share.
// The arithmetic is the wide kernel's -- same fragments, same map of k to
// MFMA steps, same unit fold -- so the outputs are bit-identical to it.
//
// The decode-tiled layout (written by tile_weights_decode): the 16 KB block
// of (expert, 256-row n-tile, half-block) holds the fragments in load order,
// wave-major: bytes 4096 w + 1024 (2 ni + j) + 16 l are what lane l of wave
// w (of that n-tile's four) loads for MFMA tile ni and K step j, so every
// load instruction of the stream reads 1 KB of contiguous memory.
constexpr int kNonTemporal = 2;   // buffer-load cache policy: nt

// The ranking of the live (expert, 64-row m-tile) pairs, built once per
// workgroup into LDS before any weight is streamed: entry p = the p-th live
// pair, those with more valid 32-row sub-tiles first and then by index (the
// order of masked_pair_by_work), packed as pair | rows << 16 with rows the
// valid rows from the m-tile's first, at most 64; entry kDregMaxPairs = the
// live count.  One wave, two passes of ballots over the pairs.
constexpr int kDregMaxPairs = 4096;

__device__ __forceinline__ void dreg_rank_table(const GemmArgs& args, uint32_t* tab, int lane) {
    const int64_t m_tiles = (args.M + 63) / 64;
    const int pairs = int(args.G * m_tiles);
    int n2 = 0, n1 = 0;
    for (int pass = 0; pass < 2; ++pass) {
        int r2 = 0, r1 = n2;   // pass 1: next rank of each class
        for (int base = 0; base < pairs; base += 64) {
            const int pair = base + lane;
            int rows = 0;
            if (pair < pairs) {
                const int64_t g = pair / m_tiles, m0 = (pair - g * m_tiles) * 64;
                int64_t mm = args.aux[g];
                mm = mm < 0 ? 0 : (mm > args.M ? args.M : mm);
                rows = int(mm - m0 <= 0 ? 0 : (mm - m0 < 64 ? mm - m0 : 64));
            }
            const uint64_t b2 = __builtin_amdgcn_ballot_w64(rows > 32);
            const uint64_t b1 = __builtin_amdgcn_ballot_w64(rows > 0 && rows <= 32);
            if (pass == 0) {
                n2 += __builtin_popcountll(b2);
                n1 += __builtin_popcountll(b1);
            } else {
                const uint64_t below = (uint64_t(1) << lane) - 1;
                if (rows > 0) {
                    const int rank = rows > 32 ? r2 + __builtin_popcountll(b2 & below)
                                               : r1 + __builtin_popcountll(b1 & below);
                    tab[rank] = uint32_t(pair) | (uint32_t(rows) << 16);
                }
                r2 += __builtin_popcountll(b2);
                r1 += __builtin_popcountll(b1);
            }
        }
    }
    if (lane == 0) tab[kDregMaxPairs] = uint32_t(n2 + n1);
}

// One item's addressing for this lane: buffer resources over the item's A
// rows, its n-tile of B, its A scales and the wave's B scale row, and the
// lane's fixed offsets into them (the half-block or K-block position rides
// in the scalar offset).
struct DregSrc {
    rsrc_t ra, rb, rsa, rsb;
    uint32_t va, vb[4], vsa[2], vsb[2];
    uint32_t sa_step;      // bytes between K-blocks of the A scales (MX: between 32-K blocks)
    uint32_t sb_step;      // MX: bytes between 32-K blocks of the B scale bytes
    int64_t c_off;         // element offset of C at (row m0, column n0)
    int64_t s_off;         // FP8 output: offset of the scale of (row m0, 128-column group of n0)
    int rows;              // valid rows from m0, at most 64
};

// The A half-block (64 rows x 64 bytes) is copied by the first COPIERS
// waves, ROWS rows each (16: a whole wave of 16-byte pieces; 8: the lower
// half-wave, eight waves sharing it).  With seven waves the last three copy
// nothing; they issue the same direct-to-LDS load through an empty buffer
// range into a dummy LDS line, so every wave counts the same loads.
template <int NW>
struct DregA {
    static constexpr int ROWS = NW == 8 ? 8 : 16;
    static constexpr int COPIERS = 64 / ROWS;
};

template <int NW, bool MX = false>
__device__ __forceinline__ DregSrc dreg_src(const GemmArgs& args, const uint32_t* tab, int64_t item, int64_t n_tiles,
                                            bool xgroup, int wave, int lane) {
    constexpr int BN = 64 * NW;                  // columns of an item
    int64_t rank, bn;
    if (xgroup) {   // item i runs on XCD i % 8 (round-robin dispatch, P % 8 == 0): pairs x, x + 8, ...
        const int64_t x = item % 8, j = item / 8;
        rank = x + 8 * (j / n_tiles);
        bn = j % n_tiles;
    } else {
        rank = item / n_tiles;
        bn = item % n_tiles;
    }
    const int64_t M = args.M, N = args.N, K = args.K;
    const int64_t m_tiles = (M + 63) / 64, kbs = (K + BK - 1) / BK;
    const uint32_t e = __builtin_amdgcn_readfirstlane(tab[rank]);   // rank < live; uniform
    const int64_t pair = e & 0xFFFF;
    const int64_t g = pair / m_tiles, m0 = (pair - g * m_tiles) * 64;
    const int rows = int(e >> 16);                 // 1 .. 64
    DregSrc s;
    s.rows = rows;
    s.c_off = (g * M + m0) * N + bn * BN;
    s.s_off = (g * (N / 128) + bn * BN / 128) * M + m0;
    const int r = lane & 31, sub = lane >> 2, slot = lane & 3;
    // A piece of this wave: rows ROWS * wave .. of the m-tile, 16 bytes per
    // lane in the ring's order (chunk c of row rr at slot c ^ ((rr >> 2) & 3));
    // rows past the valid ones re-read the last valid row (never used)
    s.ra = wave < DregA<NW>::COPIERS ? make_rsrc(args.a + (g * M + m0) * K, uint32_t(rows * K))
                                     : make_rsrc(args.a, 0u);
    {
        const int rr = wave * DregA<NW>::ROWS + (DregA<NW>::ROWS == 8 ? (sub & 7) : sub);
        const int64_t row = rr < rows ? rr : rows - 1;
        s.va = uint32_t(row * K + ((slot ^ ((rr >> 2) & 3)) << 4));
    }
    {   // the wave's 64 columns: quarter q of 256-row n-tile t of the tiled layout
        const int64_t col = bn * BN + 64 * wave, t = col / 256, q = (col % 256) / 64;
        const int64_t halves_real = K / 64;
        s.rb = make_rsrc(args.b + (g * (N / 256) + t) * halves_real * 16384, uint32_t(halves_real * 16384));
#pragma unroll
        for (int u = 0; u < 4; ++u) s.vb[u] = uint32_t(q * 4096 + u * 1024 + lane * 16);
    }
    if constexpr (MX) {
        // E8M0 bytes: A [G][K/32][M], B [G][K/32][N]; lane (r, h) loads the
        // bytes of 32-K block 2 hb + h of its rows mi * 32 + r and of its
        // columns ni * 32 + r (the scaled MFMA takes block h from lanes
        // r + 32 h)
        const int64_t k32 = K / 32;
        const uint8_t* ea = reinterpret_cast<const uint8_t*>(args.sa);
        const uint8_t* eb = reinterpret_cast<const uint8_t*>(args.sb);
        s.rsa = make_rsrc(ea + g * k32 * M + m0, uint32_t((k32 - 1) * M + rows));
        s.sa_step = uint32_t(M);
        s.rsb = make_rsrc(eb + g * k32 * N, uint32_t(k32 * N));
        s.sb_step = uint32_t(N);
        const int h = lane >> 5;
#pragma unroll
        for (int mi = 0; mi < 2; ++mi) {
            const int rr = mi * 32 + r;
            s.vsa[mi] = uint32_t((rr < rows ? rr : rows - 1) + h * M);
            s.vsb[mi] = uint32_t(bn * BN + 64 * wave + mi * 32 + r + h * N);
        }
        return s;
    }
    s.rsa = make_rsrc(args.sa + g * kbs * M + m0, uint32_t(((kbs - 1) * M + rows) * 4));
    s.sa_step = uint32_t(M * 4);
#pragma unroll
    for (int mi = 0; mi < 2; ++mi) {
        const int rr = mi * 32 + r;
        s.vsa[mi] = uint32_t((rr < rows ? rr : rows - 1) * 4);
    }
    s.rsb = make_rsrc(args.sb + (g * (N / 128) + (bn * BN + 64 * wave) / 128) * kbs, uint32_t(kbs * 4));
    return s;
}

// loads of half-block hb of an item into ring position POS: B fragments,
// then the A piece, then (first half of a K-block) the scales
// The groups must leave in program order -- the vmcnt waits count whole
// groups, and the compiler's own waits on the ring registers are only as
// tight as the order it sees -- so the scheduler may not move loads across
// a group's ends.
// The scales in flight: FP32 scales of each K-block (loaded with its first
// half), or (MX) the E8M0 bytes of every half-block's two 32-K blocks.
template <int NP, bool MX>
struct DregScales {
    float qa[NP / 2][2], qb[NP / 2];
};
template <int NP>
struct DregScales<NP, true> {
    uint32_t ea[NP][2], eb[NP][2];
    v8i b8[NP][2];   // MX: the B ring itself, both K steps of tile ni as one operand
};

template <int NP, int NW, int POS, bool MX>
__device__ __forceinline__ void dreg_issue(const DregSrc& s, int hb, uint8_t* lds, int wave, int lane,
                                           u32x4 (&bq)[NP][4], DregScales<NP, MX>& sc) {
    constexpr int A_BYTES = DregA<NW>::ROWS * 64;   // a copying wave's share of the A half-block
    __builtin_amdgcn_sched_barrier(0);
    if constexpr (MX) {
#pragma unroll
        for (int ni = 0; ni < 2; ++ni) {
            const u32x4 lo = __builtin_amdgcn_raw_buffer_load_b128(s.rb, s.vb[2 * ni], uint32_t(hb) * 16384u,
                                                                   kNonTemporal);
            const u32x4 hi = __builtin_amdgcn_raw_buffer_load_b128(s.rb, s.vb[2 * ni + 1], uint32_t(hb) * 16384u,
                                                                   kNonTemporal);
            sc.b8[POS][ni] = __builtin_bit_cast(v8i, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
        }
    } else {
#pragma unroll
        for (int t = 0; t < 4; ++t)
            bq[POS][t] = __builtin_amdgcn_raw_buffer_load_b128(s.rb, s.vb[t], uint32_t(hb) * 16384u, kNonTemporal);
    }
    // (eight waves: the upper half-wave's lanes are off, so the copy is 512
    // bytes; waves past the copiers load nothing into the dummy line)
    uint8_t* dst = wave < DregA<NW>::COPIERS ? lds + POS * 4096 + wave * A_BYTES : lds + NP * 4096 + 64;
    if (DregA<NW>::ROWS == 16 || lane < 32)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(s.ra, (lds_ptr_t)dst, 16, s.va, uint32_t(hb) * 64u, 0, 0);
    if constexpr (MX) {
#pragma unroll
        for (int mi = 0; mi < 2; ++mi)
            sc.ea[POS][mi] = __builtin_amdgcn_raw_buffer_load_b8(s.rsa, s.vsa[mi], uint32_t(2 * hb) * s.sa_step, 0);
#pragma unroll
        for (int ni = 0; ni < 2; ++ni)
            sc.eb[POS][ni] = __builtin_amdgcn_raw_buffer_load_b8(s.rsb, s.vsb[ni], uint32_t(2 * hb) * s.sb_step, 0);
    } else if constexpr (POS % 2 == 0) {
        const uint32_t kb = uint32_t(hb >> 1);
#pragma unroll
        for (int mi = 0; mi < 2; ++mi)
            sc.qa[POS / 2][mi] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(s.rsa, s.vsa[mi],
                                                                                              kb * s.sa_step, 0));
        sc.qb[POS / 2] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(s.rsb, 0u, kb * 4u, 0));
    }
    __builtin_amdgcn_sched_barrier(0);
}

// LDS byte address of a pointer into the workgroup's LDS
__device__ __forceinline__ uint32_t lds_addr(const uint8_t* p) {
    return uint32_t(reinterpret_cast<uintptr_t>((const __attribute__((address_space(3))) uint8_t*)p));
}

// loads per half-block: 4 B fragments + 1 A piece, + 3 scales on even ones
// (MX: + 4 scale bytes on every one)
constexpr int dreg_loads(int q, bool mx) { return mx ? 9 : 5 + (q % 2 == 0 ? 3 : 0); }
// loads issued for the `ahead` half-blocks after one at ring position p
constexpr int dreg_later(int p, int ahead, bool mx) {
    int n = 0;
    for (int d = 1; d <= ahead; ++d) n += dreg_loads(p + d, mx);
    return n;
}

// OUT 2 (FP8 output): C's 1x128 quantization along N -- exactly the rowwise
// quantizer on the FP32 C that OUT 1 writes.  A 128-column group is the
// columns of waves 2p and 2p + 1 (items of 256 or 512 columns); each wave
// takes its rows' max-abs over its 64 columns, the pair meets in `xch`.
template <int OUT>
__device__ __forceinline__ void dreg_store(const GemmArgs& args, const DregSrc& c, int wave, int lane,
                                           const v16f (&acc)[2][2], const WideScales<2>& w, float* xch) {
    const int r = lane & 31, h = lane >> 5;
    const int64_t N = args.N;
    if constexpr (OUT == 2) {
        float am[2];
#pragma unroll
        for (int mi = 0; mi < 2; ++mi) {
            am[mi] = 0.0f;
#pragma unroll
            for (int ni = 0; ni < 2; ++ni)
#pragma unroll
                for (int i = 0; i < 16; ++i) am[mi] = fmaxf(am[mi], fabsf(acc[mi][ni][i] * w.unit[mi]));
            am[mi] = fmaxf(am[mi], __shfl_xor(am[mi], 32, 64));
            if (h == 0) xch[wave * 64 + mi * 32 + r] = am[mi];
        }
        // LDS only: the weight loads in flight for the next item keep going
        asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
        __builtin_amdgcn_s_barrier();
        asm volatile("" ::: "memory");   // the partner's maxima are read after the barrier
#pragma unroll
        for (int mi = 0; mi < 2; ++mi) {
            const float amax = fmaxf(am[mi], xch[(wave ^ 1) * 64 + mi * 32 + r]);
            const float sc = amax / 448.0f;
            const float rc = 1.0f / sc;
            const int m = mi * 32 + r;
            if (m >= c.rows) continue;
#pragma unroll
            for (int ni = 0; ni < 2; ++ni) {
                uint32_t d[4][1];
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const v4f v = v4f{acc[mi][ni][4 * j], acc[mi][ni][4 * j + 1], acc[mi][ni][4 * j + 2],
                                      acc[mi][ni][4 * j + 3]} * w.unit[mi];
                    d[j][0] = encode4(v, sc, rc);
                }
                store_fp8_runs(static_cast<uint8_t*>(args.c) + c.c_off + int64_t(m) * N + wave * 64 + ni * 32, h, d);
            }
            if (h == 0 && (wave & 1) == 0) args.cs[c.s_off + (wave >> 1) * args.M + m] = sc;
        }
        return;
    }
    const int n_lane = wave * 64 + 4 * h;
#pragma unroll
    for (int mi = 0; mi < 2; ++mi) {
        const int m = mi * 32 + r;
        if (m >= c.rows) continue;
#pragma unroll
        for (int ni = 0; ni < 2; ++ni) {
            uint32_t d[4][2];
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int64_t idx = c.c_off + int64_t(m) * N + n_lane + ni * 32 + 8 * j;
                const v4f v = v4f{acc[mi][ni][4 * j], acc[mi][ni][4 * j + 1], acc[mi][ni][4 * j + 2],
                                  acc[mi][ni][4 * j + 3]} * w.unit[mi];
                if (OUT == 1)
                    st<v4f>(static_cast<float*>(args.c) + idx, v);
                else
                    bf16_words(v, d[j]);
            }
            if (OUT == 0) store_bf16_runs(static_cast<uint16_t*>(args.c) + c.c_off + int64_t(m) * N + wave * 64 + ni * 32, h, d);
        }
    }
}

// One half-block at ring position P of the compute item: scales (first half
// of a K-block), then the two K steps of 32 from the A slot and the B
// registers.  `partial`: the K-block runs past K; fragments past K read as 0.
// MX: one scaled FP8 MFMA per 32 x 32 tile and half-block on the codes
// themselves (A chunks h and 2 + h, the two B pieces of the K steps), with
// the lane's scale bytes; no unit, no rescale.
template <int NP, int P, bool MX>
__device__ __forceinline__ void dreg_compute(const uint8_t* lds, int hb, int64_t K, bool partial, int r, int h,
                                             const u32x4 (&bq)[NP][4], const DregScales<NP, MX>& sc, WideScales<2>& w,
                                             v16f (&acc)[2][2]) {
    constexpr uint32_t kZero = NP * 4096;
    if constexpr (MX) {
        // K % 64 == 0: a half-block lies wholly inside K or wholly past it;
        // one past K contributes nothing (uniform branch)
        if (partial && int64_t(hb) * 64 >= K) return;
        const uint32_t base = lds_addr(lds) + uint32_t(P) * 4096u;
        uint32_t ad[2][2];
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            const uint32_t chunk = uint32_t(((2 * j + h) ^ ((r >> 2) & 3)) << 4);
#pragma unroll
            for (int mi = 0; mi < 2; ++mi) ad[j][mi] = base + uint32_t((mi * 32 + r) * 64) + chunk;
        }
        u32x4 fa[2][2];
        asm volatile(   // as below: waits for these reads only
            "ds_read_b128 %0, %4\n\t"
            "ds_read_b128 %1, %5\n\t"
            "ds_read_b128 %2, %6\n\t"
            "ds_read_b128 %3, %7\n\t"
            "s_waitcnt lgkmcnt(0)"
            : "=&v"(fa[0][0]), "=&v"(fa[0][1]), "=&v"(fa[1][0]), "=&v"(fa[1][1])
            : "v"(ad[0][0]), "v"(ad[0][1]), "v"(ad[1][0]), "v"(ad[1][1])
            : "memory");
#pragma unroll
        for (int ni = 0; ni < 2; ++ni) {
            const v8i b8 = sc.b8[P][ni];
#pragma unroll
            for (int mi = 0; mi < 2; ++mi) {
                const v8i a8 = v8i{int(fa[0][mi][0]), int(fa[0][mi][1]), int(fa[0][mi][2]), int(fa[0][mi][3]),
                                   int(fa[1][mi][0]), int(fa[1][mi][1]), int(fa[1][mi][2]), int(fa[1][mi][3])};
                // formats 0/0 = E4M3 x E4M3; B is the instruction's first operand
                acc[mi][ni] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(
                    b8, a8, acc[mi][ni], 0, 0, 0, int(sc.eb[P][ni]), 0, int(sc.ea[P][mi]));
            }
        }
        return;
    }
    if constexpr (!MX && P % 2 == 0) {
        WideScales<2> nw;
        const float sb = sc.qb[P / 2];
        const ScaleSplit b = split_scale(sb);
        nw.pb = b.pow2;
#pragma unroll
        for (int mi = 0; mi < 2; ++mi) {
            const float sa = sc.qa[P / 2][mi];
            const ScaleSplit a = split_scale(sa);
            nw.pa[mi] = a.pow2;
            nw.unit[mi] = clamp_unit(a.mant * b.mant);
            nw.zero[mi] = (sa == 0.0f || sb == 0.0f) ? 1 : 0;
        }
        rescale<2, 2, 2>(acc, w, nw);
        w = nw;
    }
    // The A fragments of both K steps, read in one block that also waits for
    // them.  The reads are written out so that the compiler's own wait
    // insertion does not see them: it cannot tell the slot read here from the
    // slot the direct-to-LDS copies are filling, and would wait for those
    // copies -- and, the counter being in order, for every prefetched B
    // fragment with them.  The slot's copies are complete: the vmcnt wait and
    // the barrier above cover every wave's.
    const uint32_t base = lds_addr(lds) + uint32_t(P) * 4096u;
    const uint32_t zero = lds_addr(lds) + kZero;
    uint32_t ad[2][2];
#pragma unroll
    for (int j = 0; j < 2; ++j) {
        const uint32_t chunk = uint32_t(((2 * j + h) ^ ((r >> 2) & 3)) << 4);
#pragma unroll
        for (int mi = 0; mi < 2; ++mi)
            ad[j][mi] = w.zero[mi] ? zero + chunk : base + uint32_t((mi * 32 + r) * 64) + chunk;
    }
    u32x4 fa[2][2];
    asm volatile(
        "ds_read_b128 %0, %4\n\t"
        "ds_read_b128 %1, %5\n\t"
        "ds_read_b128 %2, %6\n\t"
        "ds_read_b128 %3, %7\n\t"
        "s_waitcnt lgkmcnt(0)"
        : "=&v"(fa[0][0]), "=&v"(fa[0][1]), "=&v"(fa[1][0]), "=&v"(fa[1][1])
        : "v"(ad[0][0]), "v"(ad[0][1]), "v"(ad[1][0]), "v"(ad[1][1])
        : "memory");
#pragma unroll
    for (int j = 0; j < 2; ++j) {
        Frags<2, 2> x;
        x.a[0] = fa[j][0];
        x.a[1] = fa[j][1];
#pragma unroll
        for (int ni = 0; ni < 2; ++ni) {
            x.b[ni] = bq[P][2 * ni + j];
            if (partial && int64_t(hb) * 64 + 32 * j + 16 * h >= K) x.b[ni] = u32x4{0u, 0u, 0u, 0u};
        }
        mfma_column<2, 2, 2>(x, w, acc);
    }
}

// a new item: accumulators at 0, unit 1
__device__ __forceinline__ void dreg_reset(v16f (&acc)[2][2], WideScales<2>& w) {
#pragma unroll
    for (int mi = 0; mi < 2; ++mi) {
#pragma unroll
        for (int ni = 0; ni < 2; ++ni)
#pragma unroll
            for (int i = 0; i < 16; ++i) acc[mi][ni][i] = 0.f;
        w.pa[mi] = 1.0f;
        w.unit[mi] = 1.0f;
        w.zero[mi] = 0;
    }
    w.pb = 1.0f;
}

template <int OUT, int NP, int NW, bool MX>
__global__ __launch_bounds__(64 * NW, 2) void gemm_dreg(GemmArgs args) {
    static_assert(NP % 2 == 0 && NP >= 2 && NP <= 8, "whole K-blocks per ring turn");
    static_assert(NW == 4 || NW == 7 || NW == 8, "items of 256, 448 or 512 columns");
    static_assert(OUT != 2 || NW % 2 == 0, "FP8 output: 128-column groups are wave pairs");
    __shared__ float xch[OUT == 2 ? 64 * NW : 1];   // FP8 output: the waves' row maxima
    // the ring, the zero line and (seven waves) the dummy line of the non-copying waves
    __shared__ __align__(16) uint8_t lds[NP * 4096 + 64 + (NW == 7 ? 1024 : 0)];
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int r = lane & 31, h = lane >> 5, sub = lane >> 2, slot = lane & 3;
    const int64_t K = args.K;
    const int halves = int(2 * ((K + BK - 1) / BK));   // whole K-blocks; a multiple of NP (host)
    const int64_t n_tiles = args.N / (64 * NW);
    __shared__ uint32_t tab[kDregMaxPairs + 1];
    if (wave == 0) dreg_rank_table(args, tab, lane);
    __syncthreads();
    const int64_t live = __builtin_amdgcn_readfirstlane(tab[kDregMaxPairs]);
    const int64_t items = live * n_tiles, P = gridDim.x, b0 = blockIdx.x;
    if (b0 >= items) return;
    const int64_t my = (items - b0 + P - 1) / P;
    const int64_t F = my * halves;                     // this workgroup's half-blocks
    const bool xgroup = live % 8 == 0 && P % 8 == 0;

    if (tid < 4) st<u32x4>(lds + NP * 4096 + tid * 16, u32x4{0u, 0u, 0u, 0u});   // the zero line
    u32x4 bq[NP][4];
    DregScales<NP, MX> sc;
    // issue side: item of the next half-block to load; compute side: item being multiplied
    int64_t item_k = 0;
    DregSrc is = dreg_src<NW, MX>(args, tab, b0, n_tiles, xgroup, wave, lane);
    DregSrc cs = is;
    // the first NP - 1 half-blocks (F >= halves >= NP, all of the first item)
#pragma unroll
    for (int q = 0; q < NP - 1; ++q) {
        if (q == 0) dreg_issue<NP, NW, 0, MX>(is, 0, lds, wave, lane, bq, sc);
        if (q == 1) dreg_issue<NP, NW, 1 % NP, MX>(is, 1, lds, wave, lane, bq, sc);
        if (q == 2) dreg_issue<NP, NW, 2 % NP, MX>(is, 2, lds, wave, lane, bq, sc);
        if (q == 3) dreg_issue<NP, NW, 3 % NP, MX>(is, 3, lds, wave, lane, bq, sc);
        if (q == 4) dreg_issue<NP, NW, 4 % NP, MX>(is, 4, lds, wave, lane, bq, sc);
        if (q == 5) dreg_issue<NP, NW, 5 % NP, MX>(is, 5, lds, wave, lane, bq, sc);
        if (q == 6) dreg_issue<NP, NW, 6 % NP, MX>(is, 6, lds, wave, lane, bq, sc);
    }
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");   // the zero line is written before the first barrier

    v16f acc[2][2];
    WideScales<2> w;
    dreg_reset(acc, w);

    int hb0 = 0;                                         // compute side: half-block of position 0
    for (int64_t f = 0; f < F; f += NP, hb0 = hb0 + NP == halves ? 0 : hb0 + NP) {
        const bool item_ends = hb0 + NP == halves;       // the compute item's last half-block is at NP - 1
        const bool partial = (hb0 + NP) * 64 > K;        // this turn holds the K-block that runs past K
#define FP8FG_DREG_STEP(PP)                                                                                       \
        if constexpr ((PP) < NP) {                                                                                \
            constexpr int later = dreg_later((PP), NP - 2, MX);                                                   \
            wait_vmcnt<later>();                                                                                  \
            const int hbc = hb0 + (PP);                                                                           \
            if (partial && (hbc + 1) * 64 > K) {   /* this wave's A chunks past K read as 0 */                    \
                constexpr int ROWS = DregA<NW>::ROWS;                                                             \
                const int rr = wave * ROWS + (ROWS == 8 ? (sub & 7) : sub);                                       \
                if (wave < DregA<NW>::COPIERS && (ROWS == 16 || lane < 32) &&                                     \
                    int64_t(hbc) * 64 + ((slot ^ ((rr >> 2) & 3)) << 4) >= K)                                     \
                    st<u32x4>(lds + (PP) * 4096 + wave * (ROWS * 64) + lane * 16, u32x4{0u, 0u, 0u, 0u});         \
                asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");                                                \
            }                                                                                                     \
            __builtin_amdgcn_s_barrier();                                                                         \
            /* every step issues a group, so every path has the same loads in flight; past F the */              \
            /* group goes to ring positions never read again, through empty buffer ranges, so those */            \
            /* loads return zeros without touching memory */                                                      \
            if ((PP) == 1 && item_ends) {                                                                         \
                if (f + NP < F) {   /* the issue side moves to the next item */                                   \
                    ++item_k;                                                                                     \
                    is = dreg_src<NW, MX>(args, tab, b0 + item_k * P, n_tiles, xgroup, wave, lane);               \
                } else {                                                                                          \
                    is.ra = make_rsrc(args.a, 0u);                                                                \
                    is.rb = make_rsrc(args.b, 0u);                                                                \
                    is.rsa = make_rsrc(args.sa, 0u);                                                              \
                    is.rsb = make_rsrc(args.sb, 0u);                                                              \
                }                                                                                                 \
            }                                                                                                     \
            /* half-block hb0 + PP + NP - 1 of the compute item, or PP - 1 of the next one */                   \
            dreg_issue<NP, NW, ((PP) + NP - 1) % NP, MX>(is, item_ends && (PP) >= 1 ? (PP) - 1 : hb0 + (PP) + NP - 1, \
                                                         lds, wave, lane, bq, sc);                            \
            dreg_compute<NP, (PP), MX>(lds, hbc, K, partial, r, h, bq, sc, w, acc);                        \
        }
        FP8FG_DREG_STEP(0)
        FP8FG_DREG_STEP(1)
        FP8FG_DREG_STEP(2)
        FP8FG_DREG_STEP(3)
        FP8FG_DREG_STEP(4)
        FP8FG_DREG_STEP(5)
        FP8FG_DREG_STEP(6)
        FP8FG_DREG_STEP(7)
#undef FP8FG_DREG_STEP
        if (item_ends) {
            dreg_store<OUT>(args, cs, wave, lane, acc, w, xch);
            dreg_reset(acc, w);
            cs = is;
        }
    }
    wait_vmcnt<0>();   // no copy may land after the workgroup's LDS is handed on
}

#define FP8FG_DREG_KERNELS(X) \
    X(0, 4, 4, 0) X(0, 2, 4, 0) X(1, 4, 4, 0) X(1, 2, 4, 0) X(0, 4, 8, 0) X(0, 2, 8, 0) X(1, 4, 8, 0) X(1, 2, 8, 0) \
    X(0, 4, 7, 0) X(0, 2, 7, 0) X(1, 4, 7, 0) X(1, 2, 7, 0) X(2, 4, 4, 0) X(2, 2, 4, 0) X(2, 4, 8, 0) X(2, 2, 8, 0) \
    X(0, 4, 4, 1) X(0, 2, 4, 1) X(1, 4, 4, 1) X(1, 2, 4, 1) X(0, 4, 8, 1) X(0, 2, 8, 1) X(1, 4, 8, 1) X(1, 2, 8, 1) \
    X(0, 4, 7, 1) X(0, 2, 7, 1) X(1, 4, 7, 1) X(1, 2, 7, 1)
#define FP8FG_DREG_INST(OUT, NP, NW, MX) template __global__ void gemm_dreg<OUT, NP, NW, MX>(GemmArgs);
FP8FG_DREG_KERNELS(FP8FG_DREG_INST)
#undef FP8FG_DREG_INST

// The decode-tiled weight layout, 16 bytes per thread in output order: unit u
// (16 bytes) of block blk = (g * N/256 + t) * (K/64) + hb holds, at block
// offset 4096 w + 1024 (2 ni + j) + 16 l, bytes 64 hb + 32 j + 16 (l / 32)
// .. + 15 of row 256 t + 64 w + 32 ni + l % 32 of expert g -- the fragment
// that lane l of wave w of gemm_dreg loads for MFMA tile ni and K step j.
__global__ __launch_bounds__(256) void tile_weights_decode(const uint8_t* __restrict__ q, int64_t K, int64_t units,
                                                           uint8_t* __restrict__ out) {
    const int64_t halves = K / 64;
    for (int64_t u = int64_t(blockIdx.x) * 256 + threadIdx.x; u < units; u += int64_t(gridDim.x) * 256) {
        const int64_t blk = u >> 10;
        const int within = int(u & 1023);
        const int wv = within >> 8, t = (within >> 6) & 3, l = within & 63;
        const int64_t gt = blk / halves, hb = blk - gt * halves;
        const int64_t row = gt * 256 + wv * 64 + (t >> 1) * 32 + (l & 31);
        st<u32x4>(out + u * 16, ld<u32x4>(q + row * K + hb * 64 + (t & 1) * 32 + (l >> 5) * 16));
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
// is 256 wide.  It also keeps one FP32 accumulator over all of K, which takes
// about eleven roundings per K-block (the eight MFMAs' sums and the unit
// change, three), each at most 2^-24 of S, the running sum of |a b|: inside
// the 2^-14 S contract for at most 92 K-blocks (11 * 92 + 1 <= 1024).  Longer
// contractions run the fold kernel, whose block sums start from zero every
// K-block (8 roundings of the block's own S, plus one per promotion).
constexpr int64_t kWideMaxKBlocks = 92;
bool wide_fits(const GemmArgs& args) {
    if (args.N % WideTile::BN != 0 || (args.K + BK - 1) / BK > kWideMaxKBlocks) return false;
    return ((args.K + BK - 1) / BK) * args.M * 4 <= int64_t(0xFFFFFFFF);
}
// On 1x128-scaled B the unit change costs more roundings: the column ratio
// (reciprocal and multiply, about three) and its product with the row ratio
// (one) join the row ratio's three and the accumulator's multiply, about
// fifteen per K-block with the eight MFMA sums: inside the contract for at
// most 68 K-blocks (15 * 68 + 1 <= 1024); the column scale array's byte range
// must also fit 32 bits.
constexpr int64_t kWideB1MaxKBlocks = 68;
bool wide_b1_fits(const GemmArgs& args) {
    const int64_t kbs = (args.K + BK - 1) / BK;
    if (args.N % WideTile::BN != 0 || kbs > kWideB1MaxKBlocks) return false;
    return kbs * args.M * 4 <= int64_t(0xFFFFFFFF) && kbs * args.N * 4 <= int64_t(0xFFFFFFFF);
}

// gfx950 (MI350 series): eight XCDs, each with its own L2
constexpr int kXcds = 8;
// the masked layout's XCD grouping for tiles of bm rows: on when 8 divides the
// (expert, m-tile) pair count (the map is then a bijection)
int masked_xcds(const GemmArgs& args, int64_t bm) {
    return (args.G * ((args.M + bm - 1) / bm)) % kXcds == 0 ? kXcds : 1;
}

// The persistent decode kernel: grid P such that the items of fully live
// buffers split evenly over the workgroup slots (P a multiple of eight: the
// item -> XCD grouping assumes it); ring depth NP 4 when it divides the
// half-block count, else 2.  Items of 512 or 448 columns (one 8- or 7-wave
// workgroup per CU), whichever N allows and fills more slots, else 256 (two
// 4-wave workgroups per CU).  `pairs` (the FP8 output) leaves out 448: its
// 128-column groups must be wave pairs of one item.
struct DregGrid {
    int nw;
    int64_t P;
};
DregGrid dreg_grid(const GemmArgs& args, int cus, bool pairs) {
    DregGrid best{0, 0};
    double best_use = -1.0;
    for (const int nw : {8, 7, 4}) {
        if (args.N % (64 * nw) != 0 || (pairs && nw % 2 != 0)) continue;
        const int64_t items = args.G * ((args.M + 63) / 64) * (args.N / (64 * nw));
        if (items == 0) return DregGrid{nw, 0};
        const int64_t slots = (nw == 4 ? 2 : 1) * int64_t(cus > 0 ? cus : 1);
        const int64_t per = (items + slots - 1) / slots;
        int64_t P = (items + per - 1) / per;
        if (P >= 8) P -= P % 8;
        const double use = double(P) / double(slots);
        if (use > best_use) {
            best = DregGrid{nw, P};
            best_use = use;
        }
    }
    return best;
}

hipError_t launch_dreg(int out_fp32, bool mx, const GemmArgs& args, hipStream_t stream) {
    int dev = 0, cus = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
    if (e != hipSuccess) return e;
    const DregGrid grid = dreg_grid(args, cus, out_fp32 == 2);   // FP8 output: wave pairs own 128 columns
    const int nw = grid.nw;
    const int64_t P = grid.P;
    if (P == 0) return hipSuccess;
    const int64_t halves = 2 * ((args.K + BK - 1) / BK);
    const int np = halves % 4 == 0 ? 4 : 2;
    void (*k)(GemmArgs) = nullptr;
#define FP8FG_DREG_PICK(OUT, NP, NW, MX) \
    if (out_fp32 == OUT && np == NP && nw == NW && mx == bool(MX)) k = gemm_dreg<OUT, NP, NW, MX>;
    FP8FG_DREG_KERNELS(FP8FG_DREG_PICK)
#undef FP8FG_DREG_PICK
    if (!k) return hipErrorInvalidValue;
    return launch_kernel(k, dim3(unsigned(P)), dim3(unsigned(64 * nw)), stream, args);
}

// The FP8-MFMA engine on the MX kernel's tiling: dense, 128x128-scaled B,
// N % 256 == 0, K % 64 == 0, and byte ranges that fit the buffer descriptors
bool mxbs_fits(const GemmArgs& args) {
    const int64_t kbs = (args.K + 127) / 128;
    return args.N % MxTile::BN == 0 && args.K % MxTile::KS == 0 && args.K > 0 && args.K < (int64_t(1) << 24) &&
           kbs * args.M * 4 <= int64_t(0xFFFFFFFF) && (args.N / 128) * kbs * 4 <= int64_t(0xFFFFFFFF);
}

hipError_t dispatch(int engine, GemmMode mode, int bscale_1x128, int out_fp32, const GemmArgs& args,
                    hipStream_t stream) {
    if (engine == 1 && mode == GemmMode::Dense && !bscale_1x128 && out_fp32 != 2 && mxbs_fits(args)) {
        const int64_t tiles = ((args.M + MxTile::BM - 1) / MxTile::BM) * (args.N / MxTile::BN);
        if (tiles == 0) return hipSuccess;
        GemmArgs a = args;
        a.xcds = kXcds;
        return launch_kernel(out_fp32 ? gemm_mxbs_o1_dense : gemm_mxbs_o0_dense, dim3(unsigned(tiles)),
                             dim3(MxTile::THREADS), stream, a);
    }
    // The exact engine on 128x128-scaled B with N a multiple of 256 runs the
    // wide kernel: 64 x 256 tiles for decode-sized masked buffers (at most
    // 128 rows), 256 x 256 tiles otherwise.  The rest (1x128 B scales, the
    // FP8-MFMA engine, N = 128 mod 256, more than kWideMaxKBlocks K-blocks)
    // runs the fold kernel: 64 x 128 tiles for decode-sized masked buffers,
    // 256 x 128 tiles otherwise.  The FP8 output mode exists only in the wide
    // exact kernel (its entry point checks that it fits).
    const bool wide = out_fp32 == 2 ||
                      (engine == 0 && (bscale_1x128 ? mode == GemmMode::Dense && wide_b1_fits(args) : wide_fits(args)));
    if (out_fp32 == 2) engine = 0;
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
    else if (mode == GemmMode::Dense)
        a.xcds = kXcds;
    for (const KernelEntry* table : {kKernels, kWideKernels, kWideB1Kernels}) {
        const size_t count = table == kKernels       ? sizeof(kKernels) / sizeof(kKernels[0])
                             : table == kWideKernels ? sizeof(kWideKernels) / sizeof(kWideKernels[0])
                                                     : sizeof(kWideB1Kernels) / sizeof(kWideB1Kernels[0]);
        for (size_t i = 0; i < count; ++i) {
            const KernelEntry& k = table[i];
            if (k.tile == tile && k.engine == engine && k.bscale == bscale_1x128 && k.out_fp32 == out_fp32 &&
                k.mode == int(mode))
                return launch_kernel(k.fn, dim3(unsigned(tiles)), dim3(unsigned(k.threads)), stream, a);
        }
    }
    return hipErrorInvalidValue;
}

// The MX GEMM in any layout: 256 x 256 tiles; the dense layout in the
// XCD-grouped order, the masked one ranked heaviest first (one XCD per
// (expert, m-tile) pair when eight divides their count), the contiguous one
// walking the group offsets over a grid that bounds its tile count.
hipError_t launch_mx(int out_fp32, GemmMode mode, const GemmArgs& args, hipStream_t stream) {
    const int64_t tiles = tile_count<MxTile>(mode, args);
    if (tiles == 0) return hipSuccess;
    GemmArgs a = args;
    a.xcds = mode == GemmMode::Dense ? kXcds : mode == GemmMode::Masked ? masked_xcds(args, MxTile::BM) : 1;
    void (*k)(GemmArgs) = mode == GemmMode::Dense    ? (out_fp32 ? gemm_mx_o1_dense : gemm_mx_o0_dense)
                          : mode == GemmMode::Contig ? (out_fp32 ? gemm_mx_o1_contig : gemm_mx_o0_contig)
                                                     : (out_fp32 ? gemm_mx_o1_masked : gemm_mx_o0_masked);
    return launch_kernel(k, dim3(unsigned(tiles)), dim3(MxTile::THREADS), stream, a);
}

hipError_t launch_masked_tiled(int out_fp32, bool mx, const GemmArgs& args, hipStream_t stream) {
    return launch_dreg(out_fp32, mx, args, stream);
}

hipError_t launch_tile_decode(const uint8_t* q, int64_t G, int64_t N, int64_t K, uint8_t* out, hipStream_t stream) {
    const int64_t units = G * N * (K / 16);
    if (units == 0) return hipSuccess;
    const int64_t blocks = (units + 255) / 256;
    return launch_kernel(tile_weights_decode, dim3(unsigned(blocks < 65536 ? blocks : 65536)), dim3(256), stream, q, K,
                         units, out);
}

}  // namespace gemm_detail

hipError_t launch_gemm_masked_tiled(int out_fp32, const GemmArgs& args, hipStream_t stream, bool mx) {
    return gemm_detail::launch_masked_tiled(out_fp32, mx, args, stream);
}

hipError_t launch_tile_weights_decode(const uint8_t* q, int64_t G, int64_t N, int64_t K, uint8_t* out,
                                      hipStream_t stream) {
    return gemm_detail::launch_tile_decode(q, G, N, K, out, stream);
}

hipError_t launch_gemm_mx(int out_fp32, GemmMode mode, const GemmArgs& args, hipStream_t stream) {
    return gemm_detail::launch_mx(out_fp32, mode, args, stream);
}

hipError_t launch_gemm(int engine, GemmMode mode, int bscale_1x128, int out_fp32, const GemmArgs& args,
                       hipStream_t stream) {
    return gemm_detail::dispatch(engine, mode, bscale_1x128, out_fp32, args, stream);
}

}  // namespace fp8fg
