// Online fine-grained FP8 quantizers for gfx950.
//
// Method: "The Insider Secrets Of Deepseek Discovered", passage on Figure 7(a)
// (1x128 activation tiles, 128x128 weight blocks, scale from each group's
// max-abs); DeepSeek-V3 FP8 knowledge-base page (codingmall.com), section on
// online quantization (scales computed from the current data).  Per group:
//   amax = max|x|,  s = RN32(amax / 448),  code = E4M3_RNE_SAT(RN32(x / s)).
// The scale is an IEEE fp32 division; the per-element quotient RN32(x / s)
// is never formed in the common case: encode4() proves from x * RN32(1/s)
// which E4M3 code it rounds to and divides only when that cannot be decided,
// so every byte and scale is reproducible bit for bit.
//
// Kernels: rowwise 1x128 (quant_act_rows_*), token-wise 1x128 with
// transposed output (quant_act_tokens_*), 128x128 weights (quant_weight_*),
// both Fprop operands in one launch (quant_fprop_*), the FP8 activation cache
// to the token-wise layout (requant_act_tokens) and the MX variant
// (quant_mx_rows; quant_mx_tokens, blocks along M with transposed output).  All are HBM-bound: 4 bytes (fp32 input) or 2 bytes (bf16
// input, widened exactly) read and 1 byte written per element, plus 4 bytes of
// scale per group.
#include "device_common.hpp"
#include "launch.hpp"

namespace fp8fg {

// ---------------------------------------------------------------------------
// 1x128 tiles along K.  A workgroup of eight half-waves (32 lanes x float4
// each) owns eight rows and U consecutive K-blocks of them: workgroup (bx, by)
// of a grid with gy row groups gives half-wave h row by*8 + h (strided by
// gy*8 over the rows) and tiles kb0 .. kb0+U-1 with kb0 = bx*U, so U
// independent 16-byte loads per lane are in flight before the first reduction
// and no index needs a division.  Scales go to s[kb][m].
template <int U, class T, int NT = 256>
__device__ __forceinline__ void quant_act_rows_body(const T* __restrict__ x, int64_t M, int64_t K,
                                                    uint8_t* __restrict__ q, float* __restrict__ s, int64_t bx,
                                                    int64_t by, int64_t gy) {
    constexpr int RW = NT / 32;                        // rows (half-waves) per workgroup
    const int lane = threadIdx.x & 31;
    const int64_t kbs = (K + kBlock - 1) / kBlock;     // a last partial group holds K % 128 elements
    const int64_t kb0 = bx * U;
    for (int64_t m = by * RW + (threadIdx.x >> 5); m < M; m += gy * RW) {
        const T* xr = x + m * K + kb0 * kBlock + lane * 4;
        uint8_t* qr = q + m * K + kb0 * kBlock + lane * 4;
        v4f v[U];
#pragma unroll
        for (int u = 0; u < U; ++u)
            v[u] = (kb0 + u) * kBlock + lane * 4 < K ? load4(xr + u * kBlock) : v4f{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int u = 0; u < U; ++u) {
            if (kb0 + u >= kbs) break;
            const float amax = halfwave_max(abs_max4(v[u]));
            const float sc = amax / 448.0f;
            const float rc = 1.0f / sc;
            if ((kb0 + u) * kBlock + lane * 4 < K) st<uint32_t>(qr + u * kBlock, encode4(v[u], sc, rc));
            if (lane == 0) s[(kb0 + u) * M + m] = sc;
        }
    }
}

// bf16 rows: 16 lanes x 8 elements (one 16-byte load each) per group, so that
// every load moves as many bytes as the fp32 kernel's and the same number of
// loads keeps twice the elements in flight.  A workgroup of sixteen
// quarter-waves owns sixteen rows.
__device__ __forceinline__ float quarterwave_max(float v) {
#pragma unroll
    for (int off = 8; off >= 1; off >>= 1) v = fmaxf(v, __shfl_xor(v, off, 64));
    return v;
}

__device__ __forceinline__ v4f widen_bf16x4(uint32_t w0, uint32_t w1) {
    return v4f{__builtin_bit_cast(float, w0 << 16), __builtin_bit_cast(float, w0 & 0xFFFF0000u),
               __builtin_bit_cast(float, w1 << 16), __builtin_bit_cast(float, w1 & 0xFFFF0000u)};
}

template <int U, int NT = 256>
__device__ __forceinline__ void quant_act_rows_bf16_body(const uint16_t* __restrict__ x, int64_t M, int64_t K,
                                                         uint8_t* __restrict__ q, float* __restrict__ s, int64_t bx,
                                                         int64_t by, int64_t gy) {
    constexpr int RW = NT / 16;                        // rows (quarter-waves) per workgroup
    const int lane = threadIdx.x & 15;
    const int64_t kbs = (K + kBlock - 1) / kBlock;     // a last partial group holds K % 128 elements
    const int64_t kb0 = bx * U;
    for (int64_t m = by * RW + (threadIdx.x >> 4); m < M; m += gy * RW) {
        const uint16_t* xr = x + m * K + kb0 * kBlock + lane * 8;
        uint8_t* qr = q + m * K + kb0 * kBlock + lane * 8;
        u32x4 v[U];
#pragma unroll
        for (int u = 0; u < U; ++u)
            v[u] = (kb0 + u) * kBlock + lane * 8 < K ? ld_once<u32x4>(xr + u * kBlock) : u32x4{0u, 0u, 0u, 0u};
#pragma unroll
        for (int u = 0; u < U; ++u) {
            if (kb0 + u >= kbs) break;
            const v4f lo = widen_bf16x4(v[u][0], v[u][1]), hi = widen_bf16x4(v[u][2], v[u][3]);
            const float amax = quarterwave_max(fmaxf(abs_max4(lo), abs_max4(hi)));
            const float sc = amax / 448.0f;
            const float rc = 1.0f / sc;
            if ((kb0 + u) * kBlock + lane * 8 < K)
                st<u32x2_t>(qr + u * kBlock, u32x2_t{encode4(lo, sc, rc), encode4(hi, sc, rc)});
            if (lane == 0) s[(kb0 + u) * M + m] = sc;
        }
    }
}

// ---------------------------------------------------------------------------
// 1x128 tiles along M (tokens), codes written transposed: q [K][M],
// s [M/128][K].  A workgroup owns 128 tokens x 64 channels: it stages the
// fp32 block in LDS (row pitch 65 floats so that column walks do not collide
// on banks), each wave reduces one quarter of the tokens per channel, the
// four partial maxima meet in LDS, every lane encodes 32 consecutive tokens of
// its channel, and the codes return through LDS so that q^T is written in
// whole 128-byte row segments.  The fp32 values come from a source: a dense
// fp32 / bf16 tensor, or the rowwise FP8 cache (DenseSrc, CacheSrc).
constexpr int kTokCh = 64;

// E consecutive channels k .. k+E-1 of token m of a dense [M][K] tensor
// (channels past K read as 0): four per 16-byte load for fp32, eight for bf16
template <class T>
struct DenseSrc {
    static constexpr int E = sizeof(T) == 4 ? 4 : 8;
    const T* x;
    int64_t K;
    // every channel of the workgroup's block exists and rows are 16-byte aligned
    __device__ __forceinline__ bool full(int64_t k0) const { return (K & (E - 1)) == 0 && k0 + kTokCh <= K; }
    __device__ __forceinline__ void load_fast(int64_t m, int64_t k, float (&e)[E]) const {
        const T* p = x + m * K + k;
        {
            if constexpr (E == 4) {
                const v4f v = ld_once<v4f>(p);
#pragma unroll
                for (int j = 0; j < 4; ++j) e[j] = v[j];
            } else {
                // (a bit_cast of a vector element would read element 0: shift
                // and mask work on values)
                const u32x4 w = ld_once<u32x4>(p);
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    e[2 * j] = __builtin_bit_cast(float, w[j] << 16);
                    e[2 * j + 1] = __builtin_bit_cast(float, w[j] & 0xFFFF0000u);
                }
            }
        }
    }
    __device__ __forceinline__ void load(int64_t m, int64_t k, float (&e)[E]) const {
        const T* p = x + m * K + k;
        if ((K & (E - 1)) == 0 && k + E <= K) {
            load_fast(m, k, e);
        } else {
#pragma unroll
            for (int j = 0; j < E; ++j) e[j] = (k + j < K) ? f32_of(p[j]) : 0.0f;
        }
    }
};

// The rowwise FP8 cache of a tensor (codes q [M][K], scales s [K/128][M]),
// dequantized element by element as RN32(decode(code) * s): the decode is
// exact (every E4M3 value is an fp32), the product rounds once.  Eight codes
// per load.
struct CacheSrc {
    static constexpr int E = 8;
    const uint8_t* q;
    const float* s;
    int64_t M, K;
    __device__ __forceinline__ bool full(int64_t k0) const { return k0 + kTokCh <= K; }
    __device__ __forceinline__ void load(int64_t m, int64_t k, float (&e)[E]) const {
        if (k < K) {                        // K % 8 == 0: the eight channels exist together
            load_fast(m, k, e);
        } else {
#pragma unroll
            for (int j = 0; j < E; ++j) e[j] = 0.0f;
        }
    }
    __device__ __forceinline__ void load_fast(int64_t m, int64_t k, float (&e)[E]) const {
        const u32x2_t w = ld<u32x2_t>(q + m * K + k);
        const float sc = s[(k / kBlock) * M + m];
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            const v2f lo = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(w[j], 1.0f, false);
            const v2f hi = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(w[j], 1.0f, true);
            e[4 * j] = lo[0] * sc;
            e[4 * j + 1] = lo[1] * sc;
            e[4 * j + 2] = hi[0] * sc;
            e[4 * j + 3] = hi[1] * sc;
        }
    }
};

// MX = true: the MX rule instead (blocks of 32 tokens, E8M0 scale bytes
// e [M/32][K]; see quant_mx_rows): each lane's 32 tokens of its channel are
// one whole block, so no partial maxima are exchanged.
template <class Src, bool MX = false, class S = float>
__device__ __forceinline__ void quant_tokens_core(const Src& src, int64_t M, int64_t K, uint8_t* __restrict__ q,
                                                  S* __restrict__ s) {
    __shared__ __align__(16) float tile[kBlock][kTokCh + 1];
    __shared__ float part[4][kTokCh];
    // the codes reuse the tile's memory: every read of the tile precedes the
    // barrier after the partial maxima
    typedef uint8_t CodeRow[kBlock + 16];
    CodeRow* codes = reinterpret_cast<CodeRow*>(&tile[0][0]);
    static_assert(sizeof(tile) >= kTokCh * sizeof(CodeRow), "codes fit in the tile");
    const int t = threadIdx.x;
    const int64_t mb = blockIdx.x;
    const int64_t k0 = int64_t(blockIdx.y) * kTokCh;
    // thread t loads E channels of rows t / (64 / E) + i * (256 E / 64)
    constexpr int E = Src::E, TPR = kTokCh / E, RSTEP = 256 / TPR;
    constexpr int NI = kBlock / RSTEP;
    const int ce = (t % TPR) * E;
    if (src.full(k0) && (mb + 1) * kBlock <= M) {   // uniform: all loads in flight before the first use
        float e[NI][E];
#pragma unroll
        for (int i = 0; i < NI; ++i) src.load_fast(mb * kBlock + t / TPR + RSTEP * i, k0 + ce, e[i]);
#pragma unroll
        for (int i = 0; i < NI; ++i)
#pragma unroll
            for (int j = 0; j < E; ++j) tile[t / TPR + RSTEP * i][ce + j] = e[i][j];
    } else {
#pragma unroll
        for (int i = 0; i < NI; ++i) {
            const int r = t / TPR + RSTEP * i;
            float e[E];
            if (mb * kBlock + r < M) {      // a last partial tile of M % 128 tokens
                src.load(mb * kBlock + r, k0 + ce, e);
            } else {
#pragma unroll
                for (int j = 0; j < E; ++j) e[j] = 0.0f;
            }
#pragma unroll
            for (int j = 0; j < E; ++j) tile[r][ce + j] = e[j];
        }
    }
    __syncthreads();

    const int c = t & 63;           // channel within the block
    const int quarter = t >> 6;     // tokens quarter*32 .. +32
    float v[32];
    float amax = 0.0f;
#pragma unroll
    for (int i = 0; i < 32; ++i) {
        v[i] = tile[quarter * 32 + i][c];
        amax = fmaxf(amax, fabsf(v[i]));
    }
    const int64_t k = k0 + c;
    uint32_t w[8];
    if constexpr (MX) {
        const int field = int((__float_as_uint(amax) >> 23) & 0xFF);
        const int sh = field - 135 < -127 ? -127 : field - 135;
        const float mul = __uint_as_float(uint32_t(127 - sh) << 23);   // 2^-s, a normal float
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            float y[4];
#pragma unroll
            for (int j = 0; j < 4; ++j) y[j] = fmaxf(fminf(v[4 * i + j] * mul, 448.0f), -448.0f);
            w[i] = cvt4(y[0], y[1], y[2], y[3]);
        }
        if (k < K && mb * kBlock + quarter * 32 < M) s[(mb * 4 + quarter) * K + k] = S(sh + 127);
        __syncthreads();   // every read of the tile is done before the codes overwrite it
    } else {
        part[quarter][c] = amax;
        __syncthreads();
        amax = fmaxf(fmaxf(part[0][c], part[1][c]), fmaxf(part[2][c], part[3][c]));
        const float sc = amax / 448.0f;
        const float rc = 1.0f / sc;
#pragma unroll
        for (int i = 0; i < 8; ++i) w[i] = encode4(v4f{v[4 * i], v[4 * i + 1], v[4 * i + 2], v[4 * i + 3]}, sc, rc);
        if (quarter == 0 && k < K) s[mb * K + k] = sc;
    }
    // the codes go through LDS as [channel][token], so that each store
    // instruction below writes eight whole 128-byte row segments of q^T
    // instead of 64 scattered 16-byte pieces
    st<u32x4>(&codes[c][quarter * 32], u32x4{w[0], w[1], w[2], w[3]});
    st<u32x4>(&codes[c][quarter * 32 + 16], u32x4{w[4], w[5], w[6], w[7]});
    __syncthreads();
#pragma unroll
    for (int i = 0; i < 2; ++i) {
        const int piece = t + 256 * i;             // 64 rows x 8 pieces of 16 bytes
        const int row = piece >> 3, off = (piece & 7) * 16;
        if (k0 + row < K && mb * kBlock + off < M)   // M % 16 == 0: whole 16-byte pieces
            st<u32x4>(q + (k0 + row) * M + mb * kBlock + off, ld<u32x4>(&codes[row][off]));
    }
}

// ---------------------------------------------------------------------------
// 128x128 weight blocks: one workgroup per block.  Thread t holds 16
// float4: rows 16*(t/32) .. +15, columns 4*(t%32) .. +3.  The block max-abs is
// reduced across the wave and then across the four waves in LDS.  The
// transposed variant turns each 4x4 group of codes around in registers
// (byte permutes) and stages the block in LDS as [column][row], 16-byte
// column groups XOR-swizzled by row, then writes whole 16-byte pieces of the
// rows of q^T.
__device__ __forceinline__ int qt_off(int row, int col) {
    return row * (kBlock + 16) + ((((col >> 4) ^ (row & 7))) << 4) + (col & 15);
}

// in[i] holds codes of row i (byte j = column j); out[j] the codes of column
// j (byte i = row i)
__device__ __forceinline__ void transpose4x4(const uint32_t (&in)[4], uint32_t (&out)[4]) {
    const uint32_t a = __builtin_amdgcn_perm(in[1], in[0], 0x05010400u);   // r0c0 r1c0 r0c1 r1c1
    const uint32_t b = __builtin_amdgcn_perm(in[1], in[0], 0x07030602u);   // r0c2 r1c2 r0c3 r1c3
    const uint32_t c = __builtin_amdgcn_perm(in[3], in[2], 0x05010400u);   // r2c0 r3c0 r2c1 r3c1
    const uint32_t d = __builtin_amdgcn_perm(in[3], in[2], 0x07030602u);   // r2c2 r3c2 r2c3 r3c3
    out[0] = __builtin_amdgcn_perm(c, a, 0x05040100u);
    out[1] = __builtin_amdgcn_perm(c, a, 0x07060302u);
    out[2] = __builtin_amdgcn_perm(d, b, 0x05040100u);
    out[3] = __builtin_amdgcn_perm(d, b, 0x07060302u);
}

// bf16 weights: 16 lanes x 8 elements (one 16-byte load) per 128-column row
// and 8 consecutive rows per thread, so a load moves as many bytes as the fp32
// body's; the block's codes, scale and transposed layout are the fp32 body's.
template <int NT = 256>
__device__ __forceinline__ void quant_weight_bf16_body(const uint16_t* __restrict__ w, int64_t N, int64_t K,
                                                       int transpose_out, uint8_t* __restrict__ q,
                                                       float* __restrict__ s, int64_t kb, int64_t nb) {
    constexpr int RPT = 2048 / NT;                 // rows per thread: 8 (256 threads) or 4 (512)
    constexpr int NWV = NT / 64;
    __shared__ float red[NWV];
    __shared__ __align__(16) uint8_t qt[kBlock * (kBlock + 16)];
    const int t = threadIdx.x;
    const int c8 = (t & 15) * 8;
    const int r8 = (t >> 4) * RPT;
    const int64_t nbs = (N + kBlock - 1) / kBlock;
    const uint16_t* wb = w + nb * kBlock * K + kb * kBlock + c8;
    const bool cvalid = kb * kBlock + c8 < K;     // K % 16 == 0: eight columns lie wholly inside or past K
    const int64_t kbs = (K + kBlock - 1) / kBlock;
    v4f lo[RPT], hi[RPT];
    float amax = 0.0f;
#pragma unroll
    for (int i = 0; i < RPT; ++i) {
        const u32x4 raw = cvalid && nb * kBlock + r8 + i < N ? ld_once<u32x4>(wb + int64_t(r8 + i) * K)
                                                              : u32x4{0u, 0u, 0u, 0u};
        lo[i] = widen_bf16x4(raw[0], raw[1]);
        hi[i] = widen_bf16x4(raw[2], raw[3]);
        amax = fmaxf(amax, fmaxf(abs_max4(lo[i]), abs_max4(hi[i])));
    }
    amax = wave_max(amax);
    if ((t & 63) == 0) red[t >> 6] = amax;
    __syncthreads();
    amax = red[0];
#pragma unroll
    for (int i = 1; i < NWV; ++i) amax = fmaxf(amax, red[i]);
    const float sc = amax / 448.0f;
    const float rc = 1.0f / sc;
    if (!transpose_out) {
#pragma unroll
        for (int i = 0; i < RPT; ++i) {
            const int64_t row = nb * kBlock + r8 + i;
            if (cvalid && row < N)
                st<u32x2_t>(q + row * K + kb * kBlock + c8, u32x2_t{encode4(lo[i], sc, rc), encode4(hi[i], sc, rc)});
        }
        if (t == 0) s[nb * kbs + kb] = sc;
        return;
    }
    // 4x4 groups of codes (rows r8 + 4g .., columns c8 + 4hh ..) turned around
    // in registers, staged as [column][row]
#pragma unroll
    for (int g = 0; g < RPT / 4; ++g)
#pragma unroll
        for (int hh = 0; hh < 2; ++hh) {
            uint32_t in[4], out[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) in[i] = encode4(hh ? hi[4 * g + i] : lo[4 * g + i], sc, rc);
            transpose4x4(in, out);
#pragma unroll
            for (int j = 0; j < 4; ++j) st<uint32_t>(&qt[qt_off(c8 + 4 * hh + j, r8 + 4 * g)], out[j]);
        }
    __syncthreads();
#pragma unroll
    for (int i = 0; i < 1024 / NT; ++i) {
        const int piece = t + NT * i;           // 1024 pieces of 16 B
        const int kr = piece >> 3, off = (piece & 7) * 16;
        if (kb * kBlock + kr < K && nb * kBlock + off < N)
            st<u32x4>(q + (kb * kBlock + kr) * N + nb * kBlock + off, ld<u32x4>(&qt[qt_off(kr, off)]));
    }
    if (t == 0) s[kb * nbs + nb] = sc;
}

// fp32 weights: 32 lanes x 4 elements per 128-column row, 16 rows per thread
template <int NT = 256>
__device__ __forceinline__ void quant_weight_f32_body(const float* __restrict__ w, int64_t N, int64_t K,
                                                      int transpose_out, uint8_t* __restrict__ q,
                                                      float* __restrict__ s, int64_t kb, int64_t nb) {
    constexpr int RPT = 4096 / NT;                 // rows per thread: 16 (256 threads) or 8 (512)
    constexpr int NWV = NT / 64;
    __shared__ float red[NWV];
    __shared__ __align__(16) uint8_t qt[kBlock * (kBlock + 16)];
    const int t = threadIdx.x;
    const int c4 = (t & 31) * 4;
    const int r0 = (t >> 5) * RPT;
    const int64_t nbs = (N + kBlock - 1) / kBlock;    // N % 16 == 0: a last partial block of N % 128 rows
    const float* wb = w + nb * kBlock * K + kb * kBlock + c4;
    const bool cvalid = kb * kBlock + c4 < K;     // K % 16 == 0: a last partial block of K % 128 columns
    const int64_t kbs = (K + kBlock - 1) / kBlock;
    v4f v[RPT];
    float amax = 0.0f;
#pragma unroll
    for (int i = 0; i < RPT; ++i) {
        v[i] = cvalid && nb * kBlock + r0 + i < N ? load4(wb + int64_t(r0 + i) * K) : v4f{0.f, 0.f, 0.f, 0.f};
        amax = fmaxf(amax, abs_max4(v[i]));
    }
    amax = wave_max(amax);
    if ((t & 63) == 0) red[t >> 6] = amax;
    __syncthreads();
    amax = red[0];
#pragma unroll
    for (int i = 1; i < NWV; ++i) amax = fmaxf(amax, red[i]);
    const float sc = amax / 448.0f;
    const float rc = 1.0f / sc;
    if (!transpose_out) {
#pragma unroll
        for (int i = 0; i < RPT; ++i) {
            const int64_t row = nb * kBlock + r0 + i;
            if (cvalid && row < N)
                *reinterpret_cast<uint32_t*>(q + row * K + kb * kBlock + c4) = encode4(v[i], sc, rc);
        }
        if (t == 0) s[nb * kbs + kb] = sc;
        return;
    }
#pragma unroll
    for (int g = 0; g < RPT / 4; ++g) {
        uint32_t in[4], out[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) in[i] = encode4(v[4 * g + i], sc, rc);
        transpose4x4(in, out);
#pragma unroll
        for (int j = 0; j < 4; ++j) st<uint32_t>(&qt[qt_off(c4 + j, r0 + 4 * g)], out[j]);
    }
    __syncthreads();
    // row kr of the transposed block: 128 bytes, written by 8 threads x 16 B
#pragma unroll
    for (int i = 0; i < 1024 / NT; ++i) {
        const int piece = t + NT * i;           // 1024 pieces of 16 B
        const int kr = piece >> 3, off = (piece & 7) * 16;
        if (kb * kBlock + kr < K && nb * kBlock + off < N)
            st<u32x4>(q + (kb * kBlock + kr) * N + nb * kBlock + off, ld<u32x4>(&qt[qt_off(kr, off)]));
    }
    if (t == 0) s[kb * nbs + nb] = sc;
}

// the 128x128 block (nb, kb), by a workgroup of NT threads
template <int NT = 256>
__device__ __forceinline__ void quant_weight_body(const float* w, int64_t N, int64_t K, int transpose_out, uint8_t* q,
                                                  float* s, int64_t kb, int64_t nb) {
    quant_weight_f32_body<NT>(w, N, K, transpose_out, q, s, kb, nb);
}
template <int NT = 256>
__device__ __forceinline__ void quant_weight_body(const uint16_t* w, int64_t N, int64_t K, int transpose_out,
                                                  uint8_t* q, float* s, int64_t kb, int64_t nb) {
    quant_weight_bf16_body<NT>(w, N, K, transpose_out, q, s, kb, nb);
}

// workgroup (bx, by) of NT threads in a grid with gy row groups
template <int U, int NT = 256>
__device__ __forceinline__ void quant_act_rows_dispatch(const float* x, int64_t M, int64_t K, uint8_t* q, float* s,
                                                        int64_t bx, int64_t by, int64_t gy) {
    quant_act_rows_body<U, float, NT>(x, M, K, q, s, bx, by, gy);
}
template <int U, int NT = 256>
__device__ __forceinline__ void quant_act_rows_dispatch(const uint16_t* x, int64_t M, int64_t K, uint8_t* q,
                                                        float* s, int64_t bx, int64_t by, int64_t gy) {
    quant_act_rows_bf16_body<U, NT>(x, M, K, q, s, bx, by, gy);
}
// rowwise grid of an [M][K] activation for NT-thread workgroups: (K-block
// chunks of U, row groups)
template <class T, int NT = 256>
inline void act_rows_grid(int64_t M, int64_t K, int64_t& chunks, int64_t& row_groups) {
    constexpr int U = 4;
    constexpr int rows_per_group = sizeof(T) == 4 ? NT / 32 : NT / 16;   // half-waves (fp32) or quarter-waves (bf16)
    chunks = ((K + kBlock - 1) / kBlock + U - 1) / U;
    row_groups = (M + rows_per_group - 1) / rows_per_group;
    if (row_groups > 65535) row_groups = 65535;      // the kernel strides over the rest
}

// ---------------------------------------------------------------------------
// MX quantization (microscaling: blocks of 32 along K, power-of-two E8M0
// scale).  "The Insider Secrets Of Deepseek Discovered", passage after
// Figure 7, relates the method to microscaling formats; the block rule is the
// OCP MX one for E4M3 elements:
//   s = clamp(floor(log2(amax)) - 8, -127, 127),  code = E4M3_RNE_SAT(x * 2^-s),
//   scale byte = s + 127  (amax = 0 gives s = -127).
// For a normal amax floor(log2) is its exponent field minus 127, and every
// amax below 2^-119 (subnormals and zero included) clamps to s = -127, so
// s = max(field - 135, -127).  x * 2^-s rounds once (only when it falls below
// fp32's normal range) and |x * 2^-s| < 512; clamping to +-448 before the
// conversion is the saturation.  A half-wave holds eight blocks of one row,
// 4 lanes x 8 elements each; codes q [R][K], scale bytes e [K/32][R].
constexpr int kMxBlock = 32;

__global__ __launch_bounds__(256) void quant_mx_rows(const float* __restrict__ x, int64_t R, int64_t K,
                                                     uint8_t* __restrict__ q, uint8_t* __restrict__ e) {
    const int lane = threadIdx.x & 31;
    const int64_t k = int64_t(blockIdx.x) * 256 + lane * 8;      // first of this lane's 8 elements
    const bool valid = k < K;                                      // K % 32 == 0: whole blocks
    for (int64_t m = int64_t(blockIdx.y) * 8 + (threadIdx.x >> 5); m < R; m += int64_t(gridDim.y) * 8) {
        v4f v0 = v4f{0.f, 0.f, 0.f, 0.f}, v1 = v0;
        if (valid) {
            v0 = ld_once<v4f>(x + m * K + k);
            v1 = ld_once<v4f>(x + m * K + k + 4);
        }
        float amax = fmaxf(abs_max4(v0), abs_max4(v1));
        amax = fmaxf(amax, __shfl_xor(amax, 1, 64));
        amax = fmaxf(amax, __shfl_xor(amax, 2, 64));
        const int field = int((__float_as_uint(amax) >> 23) & 0xFF);
        const int sh = field - 135 < -127 ? -127 : field - 135;   // at most 254 - 135 = 119
        const float mul = __uint_as_float(uint32_t(127 - sh) << 23);   // 2^-s, a normal float
        v4f y0 = v0 * mul, y1 = v1 * mul;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            y0[j] = fmaxf(fminf(y0[j], 448.0f), -448.0f);
            y1[j] = fmaxf(fminf(y1[j], 448.0f), -448.0f);
        }
        if (valid) {
            st<u32x2_t>(q + m * K + k, u32x2_t{cvt4(y0[0], y0[1], y0[2], y0[3]), cvt4(y1[0], y1[1], y1[2], y1[3])});
            if ((lane & 3) == 0) e[(k / kMxBlock) * R + m] = uint8_t(sh + 127);
        }
    }
}

// MX blocks of 32 tokens, codes written transposed: q [K][M], e [M/32][K]
// (exactly quant_mx_rows of x^T), through the token-wise kernel's staging
__global__ __launch_bounds__(256) void quant_mx_tokens(const float* __restrict__ x, int64_t M, int64_t K,
                                                       uint8_t* __restrict__ q, uint8_t* __restrict__ e) {
    quant_tokens_core<DenseSrc<float>, true>(DenseSrc<float>{x, K}, M, K, q, e);
}

hipError_t launch_quant_mx_tokens(const float* x, int64_t M, int64_t K, uint8_t* q, uint8_t* e, hipStream_t stream) {
    const dim3 grid(unsigned((M + kBlock - 1) / kBlock), unsigned((K + kTokCh - 1) / kTokCh));
    return launch_kernel(quant_mx_tokens, grid, dim3(256), stream, x, M, K, q, e);
}

hipError_t launch_quant_mx(const float* x, int64_t R, int64_t K, uint8_t* q, uint8_t* e, hipStream_t stream) {
    const int64_t chunks = (K + 255) / 256;
    int64_t row_groups = (R + 7) / 8;
    if (row_groups > 65535) row_groups = 65535;      // the kernel strides over the rest
    return launch_kernel(quant_mx_rows, dim3(unsigned(chunks), unsigned(row_groups)), dim3(256), stream, x, R, K, q,
                         e);
}

// ---------------------------------------------------------------------------
// One plain kernel per element type (fp32, bf16 bits).
#define FP8FG_QUANT_KERNELS(T, SUFFIX)                                                                     \
    __global__ __launch_bounds__(256) void quant_act_rows_##SUFFIX(const T* __restrict__ x, int64_t M,      \
                                                                   int64_t K, uint8_t* __restrict__ q,     \
                                                                   float* __restrict__ s) {                \
        quant_act_rows_dispatch<4>(x, M, K, q, s, blockIdx.x, blockIdx.y, gridDim.y);                      \
    }                                                                                                      \
    __global__ __launch_bounds__(256) void quant_act_tokens_##SUFFIX(const T* __restrict__ x, int64_t M,    \
                                                                     int64_t K, uint8_t* __restrict__ q,   \
                                                                     float* __restrict__ s) {              \
        quant_tokens_core(DenseSrc<T>{x, K}, M, K, q, s);                                                  \
    }                                                                                                      \
    __global__ __launch_bounds__(256) void quant_weight_##SUFFIX(const T* __restrict__ w, int64_t N,        \
                                                                 int64_t K, int transpose_out,             \
                                                                 uint8_t* __restrict__ q,                  \
                                                                 float* __restrict__ s) {                  \
        quant_weight_body(w, N, K, transpose_out, q, s, blockIdx.x, blockIdx.y);                           \
    }
FP8FG_QUANT_KERNELS(float, f32)
FP8FG_QUANT_KERNELS(uint16_t, bf16)
#undef FP8FG_QUANT_KERNELS

// ---------------------------------------------------------------------------
// Both Fprop operands in one launch: the 128x128 weight blocks (the longer
// workgroups) first, then the rowwise activation workgroups, each running the
// body of its own kernel, so every byte is what the two separate launches
// write.  One launch lets the two small grids overlap instead of each paying
// its own ramp-up and drain.
constexpr int kFpropThreads = 512;   // eight waves: half the registers per weight thread of a 256-thread block
#define FP8FG_FPROP_KERNEL(TX, TW, SUFFIX)                                                                   \
    __global__ __launch_bounds__(kFpropThreads) void quant_fprop_##SUFFIX(                                   \
        const TX* __restrict__ x, int64_t M, const TW* __restrict__ w, int64_t N, int64_t K,                 \
        uint8_t* __restrict__ qa, float* __restrict__ sa, uint8_t* __restrict__ qb, float* __restrict__ sb,  \
        int64_t act_chunks, int64_t act_groups) {                                                            \
        const int64_t kbs = (K + kBlock - 1) / kBlock, w_blocks = kbs * ((N + kBlock - 1) / kBlock);         \
        const int64_t b = blockIdx.x;                                                                        \
        if (b < w_blocks) {                                                                                  \
            quant_weight_body<kFpropThreads>(w, N, K, 0, qb, sb, b % kbs, b / kbs);                          \
        } else {                                                                                             \
            const int64_t a = b - w_blocks;                                                                  \
            quant_act_rows_dispatch<4, kFpropThreads>(x, M, K, qa, sa, a % act_chunks, a / act_chunks,       \
                                                      act_groups);                                           \
        }                                                                                                    \
    }
FP8FG_FPROP_KERNEL(float, float, f32_f32)
FP8FG_FPROP_KERNEL(uint16_t, float, bf16_f32)
FP8FG_FPROP_KERNEL(float, uint16_t, f32_bf16)
FP8FG_FPROP_KERNEL(uint16_t, uint16_t, bf16_bf16)
#undef FP8FG_FPROP_KERNEL

// FP8 activation cache -> token-wise Wgrad operand
__global__ __launch_bounds__(256) void requant_act_tokens(const uint8_t* __restrict__ qr, const float* __restrict__ sr,
                                                          int64_t M, int64_t K, uint8_t* __restrict__ q,
                                                          float* __restrict__ s) {
    quant_tokens_core(CacheSrc{qr, sr, M, K}, M, K, q, s);
}

template <class T>
static hipError_t launch_act(const T* x, int64_t M, int64_t K, int transpose_out, uint8_t* q, float* s,
                             hipStream_t stream, void (*rows)(const T*, int64_t, int64_t, uint8_t*, float*),
                             void (*tokens)(const T*, int64_t, int64_t, uint8_t*, float*)) {
    if (!transpose_out) {
        int64_t chunks = 0, row_groups = 0;
        act_rows_grid<T>(M, K, chunks, row_groups);
        return launch_kernel(rows, dim3(unsigned(chunks), unsigned(row_groups)), dim3(256), stream, x, M, K, q, s);
    }
    const dim3 grid(unsigned((M + kBlock - 1) / kBlock), unsigned((K + kTokCh - 1) / kTokCh));
    return launch_kernel(tokens, grid, dim3(256), stream, x, M, K, q, s);
}

hipError_t launch_quant_act(const void* x, int bf16, int64_t M, int64_t K, int transpose_out, uint8_t* q,
                            float* s, hipStream_t stream) {
    if (bf16)
        return launch_act(static_cast<const uint16_t*>(x), M, K, transpose_out, q, s, stream, quant_act_rows_bf16,
                          quant_act_tokens_bf16);
    return launch_act(static_cast<const float*>(x), M, K, transpose_out, q, s, stream, quant_act_rows_f32,
                      quant_act_tokens_f32);
}

hipError_t launch_requant_act_tokens(const uint8_t* qr, const float* sr, int64_t M, int64_t K, uint8_t* q, float* s,
                                     hipStream_t stream) {
    const dim3 grid(unsigned((M + kBlock - 1) / kBlock), unsigned((K + kTokCh - 1) / kTokCh));
    return launch_kernel(requant_act_tokens, grid, dim3(256), stream, qr, sr, M, K, q, s);
}

template <class TX, class TW>
static hipError_t launch_fprop(const TX* x, int64_t M, const TW* w, int64_t N, int64_t K, uint8_t* qa, float* sa,
                               uint8_t* qb, float* sb, hipStream_t stream,
                               void (*kern)(const TX*, int64_t, const TW*, int64_t, int64_t, uint8_t*, float*,
                                            uint8_t*, float*, int64_t, int64_t)) {
    int64_t chunks = 0, row_groups = 0;
    act_rows_grid<TX, kFpropThreads>(M, K, chunks, row_groups);
    const int64_t w_blocks = ((K + kBlock - 1) / kBlock) * ((N + kBlock - 1) / kBlock);
    const int64_t blocks = w_blocks + chunks * row_groups;
    return launch_kernel(kern, dim3(unsigned(blocks)), dim3(kFpropThreads), stream, x, M, w, N, K, qa, sa, qb, sb,
                         chunks, row_groups);
}

hipError_t launch_quant_fprop(const void* x, int x_bf16, int64_t M, const void* w, int w_bf16, int64_t N, int64_t K,
                              uint8_t* qa, float* sa, uint8_t* qb, float* sb, hipStream_t stream) {
    const float* xf = static_cast<const float*>(x);
    const uint16_t* xh = static_cast<const uint16_t*>(x);
    const float* wf = static_cast<const float*>(w);
    const uint16_t* wh = static_cast<const uint16_t*>(w);
    if (!x_bf16 && !w_bf16) return launch_fprop(xf, M, wf, N, K, qa, sa, qb, sb, stream, quant_fprop_f32_f32);
    if (x_bf16 && !w_bf16) return launch_fprop(xh, M, wf, N, K, qa, sa, qb, sb, stream, quant_fprop_bf16_f32);
    if (!x_bf16) return launch_fprop(xf, M, wh, N, K, qa, sa, qb, sb, stream, quant_fprop_f32_bf16);
    return launch_fprop(xh, M, wh, N, K, qa, sa, qb, sb, stream, quant_fprop_bf16_bf16);
}

hipError_t launch_quant_weight(const void* w, int bf16, int64_t N, int64_t K, int transpose_out, uint8_t* q,
                               float* s, hipStream_t stream) {
    const dim3 grid(unsigned((K + kBlock - 1) / kBlock), unsigned((N + kBlock - 1) / kBlock));
    if (bf16)
        return launch_kernel(quant_weight_bf16, grid, dim3(256), stream, static_cast<const uint16_t*>(w), N, K,
                             transpose_out, q, s);
    return launch_kernel(quant_weight_f32, grid, dim3(256), stream, static_cast<const float*>(w), N, K, transpose_out,
                         q, s);
}

}  // namespace fp8fg
