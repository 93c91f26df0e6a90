// Block-scaled FP8 GEMM for gfx950: dense, MoE contiguous and MoE masked.
//
// Method: "The Insider Secrets Of Deepseek Discovered", passages on limited
// Tensor Core accumulation and on promotion (Figure 7(b)): each 128-wide
// K-block is accumulated on its own, then promoted into an FP32 accumulator
// with the product of the two group scales applied at that moment.  On gfx950
// one v_mfma_f32_16x16x128_f8f6f4 covers exactly one K-block of a 16x16 output
// tile, so the per-K-block partial is the result of a single MFMA started from
// zero, and the promotion is one FP32 FMA per output element:
//     acc += P_kb * (sA[kb][m] * sB[nb][kb])        (or sB[kb][n] for 1x128 B)
// Layouts (DeepGEMM launch article, "Principais caracteristicas": dense plus
// contiguous and masked MoE groupings): A codes [rows][K], B codes [N][K],
// both K-major; A scales [K/128][rows]; C [rows][N].
//
// Tiling: a 256-thread workgroup computes a 128x128 tile of C; its four waves
// each own 64 (m) x 64 (n).  A and B K-block tiles (128 rows x 128 bytes each)
// are double-buffered in LDS; 16-byte chunks are XOR-swizzled by row so that
// the fragment reads of 16 consecutive rows spread over the banks.  The MFMA is
// issued with B's fragment as its first operand and A's as its second, so each
// lane ends up holding four consecutive n of one row m: one A scale per lane
// and fragment, and 8- or 16-byte output stores.
#include "device_common.hpp"
#include "launch.hpp"

namespace fp8fg {

namespace {

constexpr int BM = 128, BN = 128, BK = 128;
constexpr int kThreads = 256;
constexpr int kTileBytes = BM * BK;        // one operand tile per K-block (A and B alike)

// Byte offset of 16-byte chunk `chunk` (0..7) of tile row `row` in LDS.
__device__ __forceinline__ int lds_off(int row, int chunk) { return row * BK + ((chunk ^ (row & 7)) << 4); }

// One MFMA operand fragment: rows `row0 + lane%16`, 32 bytes starting at byte
// 32*(lane/16) of the K-block.  A and B fragments use the same byte mapping,
// so whatever K order the instruction assigns to (lane, byte) is shared by
// both operands and the contraction is over matching k.
__device__ __forceinline__ v8i read_frag(const uint8_t* tile, int row0, int lane) {
    const int row = row0 + (lane & 15);
    const int ch = (lane >> 4) * 2;
    const u32x4 lo = ld<u32x4>(tile + lds_off(row, ch));
    const u32x4 hi = ld<u32x4>(tile + lds_off(row, ch + 1));
    return v8i{int(lo[0]), int(lo[1]), int(lo[2]), int(lo[3]), int(hi[0]), int(hi[1]), int(hi[2]), int(hi[3])};
}

__device__ __forceinline__ v4f mfma_kblock(v8i bfrag, v8i afrag) {
    const v4f zero = {0.f, 0.f, 0.f, 0.f};
    // operand formats 0/0 = E4M3 x E4M3; zero scale operands select the plain
    // (unscaled) instruction
    return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(bfrag, afrag, zero, 0, 0, 0, 0, 0, 0);
}

template <int BSCALE_1x128, int OUT_FP32, int MODE>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(1, 1)))
void gemm_bs_kernel(GemmArgs args) {
    __shared__ __align__(16) uint8_t lds[2][2][kTileBytes];   // [buffer][A, B]

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int wm = wave >> 1, wn = wave & 1;
    const int64_t N = args.N, K = args.K;
    const int n_tiles = int(N / BN);
    const int64_t kbs = K / BK;

    // ---- tile -> (group, rows) ------------------------------------------
    int64_t tile = blockIdx.x;
    const int bn = int(tile % n_tiles);
    tile /= n_tiles;
    int64_t m0;               // first row of the tile within its group's row space
    int64_t rows_valid;       // rows [0, rows_valid) of that row space exist
    int64_t lda_s;            // row count of the scale array (stride between K-blocks)
    const uint8_t* A = args.a;
    const float* SA = args.sa;
    const uint8_t* B = args.b;
    const float* SB = args.sb;
    int64_t g = 0;
    if (MODE == int(GemmMode::Dense)) {
        m0 = tile * BM;
        rows_valid = args.M;
        lda_s = args.M;
    } else if (MODE == int(GemmMode::Contig)) {
        m0 = tile * BM;
        // largest g with offsets[g] <= m0
        int lo = 0, hi = int(args.G) - 1;
        while (lo < hi) {
            const int mid = (lo + hi + 1) >> 1;
            if (args.aux[mid] <= m0) lo = mid; else hi = mid - 1;
        }
        g = lo;
        const int64_t g_end = args.aux[g + 1];
        if (args.aux[g] > m0 || m0 >= g_end || g_end > args.M) return;
        rows_valid = g_end;
        lda_s = args.M;
    } else {
        const int64_t m_tiles = (args.M + BM - 1) / BM;
        g = tile / m_tiles;
        m0 = (tile - g * m_tiles) * BM;
        int64_t mm = args.aux[g];
        mm = mm < 0 ? 0 : (mm > args.M ? args.M : mm);
        rows_valid = mm;
        lda_s = args.M;
        A += g * args.M * K;
        SA += g * kbs * args.M;
    }
    if (m0 >= rows_valid) return;
    if (MODE != int(GemmMode::Dense)) {
        B += g * N * K;
        SB += g * (N / BN) * kbs;
    }
    const int64_t n0 = int64_t(bn) * BN;

    // ---- global -> LDS copy assignment: rows tid/8 + 32*i, chunk tid%8 -----
    const int ld_chunk = tid & 7;
    const int ld_row = tid >> 3;
    const uint8_t* a_src[4];
    const uint8_t* b_src[4];
    int st_off[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int r = ld_row + 32 * i;
        int64_t ar = m0 + r;
        if (ar >= rows_valid) ar = rows_valid - 1;     // clamp: loaded, never stored
        a_src[i] = A + ar * K + ld_chunk * 16;
        b_src[i] = B + (n0 + r) * K + ld_chunk * 16;
        st_off[i] = lds_off(r, ld_chunk);
    }

    // rows of this lane's A scales, one per 16-row fragment (clamped like the loads)
    int64_t sa_row[4];
#pragma unroll
    for (int mi = 0; mi < 4; ++mi) {
        int64_t r = m0 + wm * 64 + mi * 16 + (lane & 15);
        sa_row[mi] = r < rows_valid ? r : rows_valid - 1;
    }
    const int n_lane = wn * 64 + (lane >> 4) * 4;      // + ni*16: first of this lane's 4 columns

    u32x4 ra[4], rb[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        ra[i] = ld<u32x4>(a_src[i]);
        rb[i] = ld<u32x4>(b_src[i]);
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        st<u32x4>(&lds[0][0][st_off[i]], ra[i]);
        st<u32x4>(&lds[0][1][st_off[i]], rb[i]);
    }
    __syncthreads();

    v4f acc[4][4];
#pragma unroll
    for (int mi = 0; mi < 4; ++mi)
#pragma unroll
        for (int ni = 0; ni < 4; ++ni) acc[mi][ni] = v4f{0.f, 0.f, 0.f, 0.f};

    for (int64_t kb = 0; kb < kbs; ++kb) {
        const int cur = int(kb & 1);
        // prefetch the next K-block (the last iteration re-reads its own block;
        // the copy lands in the idle buffer and is never read)
        const int64_t koff = (kb + 1 < kbs ? kb + 1 : kb) * BK;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            ra[i] = ld<u32x4>(a_src[i] + koff);
            rb[i] = ld<u32x4>(b_src[i] + koff);
        }
        // scales of this K-block
        float sa[4];
#pragma unroll
        for (int mi = 0; mi < 4; ++mi) sa[mi] = SA[kb * lda_s + sa_row[mi]];
        float sb_blk = 0.f;
        v4f sb_col[4];
        if (BSCALE_1x128) {
#pragma unroll
            for (int ni = 0; ni < 4; ++ni) sb_col[ni] = ld<v4f>(SB + kb * N + n0 + n_lane + ni * 16);
        } else {
            sb_blk = SB[int64_t(bn) * kbs + kb];
        }

        const uint8_t* ta = lds[cur][0];
        const uint8_t* tb = lds[cur][1];
        v8i af[4], bf[4];
#pragma unroll
        for (int mi = 0; mi < 4; ++mi) af[mi] = read_frag(ta, wm * 64 + mi * 16, lane);
#pragma unroll
        for (int ni = 0; ni < 4; ++ni) bf[ni] = read_frag(tb, wn * 64 + ni * 16, lane);
        // all 16 partials of this K-block first (independent registers, so the
        // MFMA pipe never waits on the fold), then the promotion FMAs
        v4f p[4][4];
#pragma unroll
        for (int ni = 0; ni < 4; ++ni)
#pragma unroll
            for (int mi = 0; mi < 4; ++mi) p[mi][ni] = mfma_kblock(bf[ni], af[mi]);
#pragma unroll
        for (int mi = 0; mi < 4; ++mi) {
#pragma unroll
            for (int ni = 0; ni < 4; ++ni) {
                if (BSCALE_1x128) {
                    acc[mi][ni] = p[mi][ni] * (sa[mi] * sb_col[ni]) + acc[mi][ni];
                } else {
                    acc[mi][ni] = p[mi][ni] * (sa[mi] * sb_blk) + acc[mi][ni];
                }
            }
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            st<u32x4>(&lds[cur ^ 1][0][st_off[i]], ra[i]);
            st<u32x4>(&lds[cur ^ 1][1][st_off[i]], rb[i]);
        }
        __syncthreads();
    }

    // ---- epilogue: lane holds C[m][n .. n+3] for each (mi, ni) -------------
    int64_t c_base = 0;
    if (MODE == int(GemmMode::Masked)) c_base = g * args.M * N;
#pragma unroll
    for (int mi = 0; mi < 4; ++mi) {
        const int64_t m = m0 + wm * 64 + mi * 16 + (lane & 15);
        if (m >= rows_valid) continue;
#pragma unroll
        for (int ni = 0; ni < 4; ++ni) {
            const int64_t idx = c_base + m * N + n0 + n_lane + ni * 16;
            const v4f v = acc[mi][ni];
            if (OUT_FP32) {
                st<v4f>(static_cast<float*>(args.c) + idx, v);
            } else {
                typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));
                const uint32_t lo = bf16_bits(v[0]) | (bf16_bits(v[1]) << 16);
                const uint32_t hi = bf16_bits(v[2]) | (bf16_bits(v[3]) << 16);
                st<u32x2>(static_cast<uint16_t*>(args.c) + idx, u32x2{lo, hi});
            }
        }
    }
}

template <int BS, int OF, int MODE>
hipError_t launch_one(const GemmArgs& args, int64_t tiles, hipStream_t stream) {
    hipLaunchKernelGGL((gemm_bs_kernel<BS, OF, MODE>), dim3(unsigned(tiles)), dim3(kThreads), 0, stream, args);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_gemm(GemmMode mode, int bscale_1x128, int out_fp32, const GemmArgs& args,
                       hipStream_t stream) {
    const int64_t n_tiles = args.N / BN;
    int64_t tiles;
    if (mode == GemmMode::Masked) tiles = args.G * ((args.M + BM - 1) / BM) * n_tiles;
    else tiles = ((args.M + BM - 1) / BM) * n_tiles;
    if (tiles == 0) return hipSuccess;
    switch (mode) {
        case GemmMode::Dense:
            if (bscale_1x128) return out_fp32 ? launch_one<1, 1, 0>(args, tiles, stream) : launch_one<1, 0, 0>(args, tiles, stream);
            return out_fp32 ? launch_one<0, 1, 0>(args, tiles, stream) : launch_one<0, 0, 0>(args, tiles, stream);
        case GemmMode::Contig:
            return out_fp32 ? launch_one<0, 1, 1>(args, tiles, stream) : launch_one<0, 0, 1>(args, tiles, stream);
        case GemmMode::Masked:
            return out_fp32 ? launch_one<0, 1, 2>(args, tiles, stream) : launch_one<0, 0, 2>(args, tiles, stream);
    }
    return hipErrorInvalidValue;
}

}  // namespace fp8fg
