/*
 * fp8fg.h -- fine-grained FP8 quantization and block-scaled FP8 GEMM on AMD
 * Instinct MI355X (gfx950).  C ABI of libfp8fg.so.
 *
 * The method (DeepSeek-V3's FP8 recipe, as retold by the pages this library
 * follows):
 *   - "The Insider Secrets Of Deepseek Discovered", passage on Figure 7(a):
 *     activations are scaled per 1x128 tile (one token, 128 channels) and
 *     weights per 128x128 block; passage on Figure 7(b): partial GEMM sums are
 *     promoted to FP32 at a fixed K interval and the scales are applied there;
 *     passage on Figure 6: Fprop, Dgrad and Wgrad of a Linear all run in FP8.
 *   - DeepSeek-V3 FP8 knowledge-base page (codingmall.com), sections on
 *     fine-grained quantization, online quantization (scales from the current
 *     tile's max-abs), increased accumulation precision and unified E4M3.
 *   - DeepGEMM launch article (itstec.com.br), "Principais caracteristicas":
 *     dense GEMMs plus two MoE grouped layouts, contiguous and masked.
 *
 * Conventions shared by every entry point
 *   - Every pointer is a DEVICE pointer owned by the caller, 16-byte aligned.
 *     The library allocates, frees and synchronizes nothing; it keeps no state
 *     between calls and is reentrant.
 *   - `stream` is a hipStream_t passed as void* (NULL = the null stream).  Work
 *     is enqueued asynchronously on it; the call returns before it runs.
 *   - Codes are OCP E4M3 bytes ("E4M3FN": bias 7, max 448, NaN = 0x7F/0xFF,
 *     no infinities).  Scales are FP32 DEQUANTIZATION multipliers:
 *     value ~= decode(code) * scale, with scale = RN32(amax / 448) and the
 *     code = E4M3 round-to-nearest-even-saturating of RN32(x / scale), IEEE
 *     division throughout.  A group whose amax is 0 gets scale 0 and signed
 *     zero codes.  Inputs must be finite (NaN/Inf: unspecified output).
 *   - Return value: FP8FG_OK, or a negative fp8fg_status.  Argument errors are
 *     detected on the host BEFORE anything is enqueued (no partial work);
 *     FP8FG_ERR_HIP means the kernel launch itself failed.  A zero-sized
 *     problem (M == 0, G == 0, ...) is a successful no-op.  The quantizers
 *     also accept NULL for the pointers of an operand with no elements.
 *   - Scale layouts.  A 1x128-scaled operand of logical shape [R][K] (K = the
 *     axis the 128-element groups run along) stores codes u8 [R][K] row-major
 *     and scales f32 [K/128][R] ("kb-major").  A 128x128-scaled [N][K] operand
 *     stores codes u8 [N][K] and scales f32 [N/128][K/128].
 *   - Partial groups.  The grouped axis (K, or the token axis of the
 *     token-wise layout) need only be a multiple of 16: the last group then
 *     holds fewer than 128 elements and is quantized as that group padded
 *     with zeros (its max-abs runs over the elements that exist).  Every
 *     count "K/128" in this header means ceil(K/128).  Likewise N, the
 *     output channels (rows of B), need only be a multiple of 16 where stated:
 *     "N/128" then means ceil(N/128).
 *   - GEMM: C[M][N] = A[M][K] . B[N][K]^T, both operands K-major (a Linear
 *     layer y = x . W^T with W [out][in]).  C is the sum over k of
 *     decode(a) * sA * decode(b) * sB, the scales of each 128-wide K-block
 *     applied once per block in FP32 (promotion at a fixed K interval).
 *     Output row-major [M][N], BF16 (round-to-nearest-even) or FP32.
 *     Accuracy contract, element by element, against the exact real-number
 *     result C*:  |C - C*| <= 2^-14 * S  (FP32 out), with
 *     S = sum_k |decode(a) sA decode(b) sB|, plus one BF16 rounding of C*
 *     for BF16 out.  The codes are widened exactly to BF16 and multiplied on
 *     the BF16 matrix cores (exact products, FP32 sums).  One call,
 *     fp8_gemm_blockscaled_fp8mfma, runs the FP8 matrix cores instead and
 *     has its own, looser contract (see there).  Results are deterministic
 *     (no atomics, no split-K).  The library reads no environment variables.
 *   - The 2^-14 * S contract is a worst-case bound: it counts at most 1024
 *     FP32 roundings of quantities no larger than S.  The calls that take any
 *     K keep it for K <= 114688 (896 K-blocks: fresh FP32 sums per K-block,
 *     one rounding per promotion); beyond that it holds for the typical
 *     (random-sign) accumulation, not in the worst case.
 */
#ifndef FP8FG_H
#define FP8FG_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define FP8FG_ABI_VERSION 14

enum fp8fg_status {
    FP8FG_OK = 0,
    FP8FG_ERR_NULL = -1,         /* a required pointer is NULL                 */
    FP8FG_ERR_SHAPE = -2,        /* negative size, or a size rule of the call  */
    FP8FG_ERR_ALIGN = -3,        /* a pointer is not 16-byte aligned           */
    FP8FG_ERR_UNSUPPORTED = -4,  /* unknown enum value or size beyond limits   */
    FP8FG_ERR_HIP = -5           /* the HIP runtime refused the launch         */
};

enum fp8fg_out { FP8FG_OUT_BF16 = 0, FP8FG_OUT_FP32 = 1 };

enum fp8fg_bscale {
    FP8FG_BSCALE_128x128 = 0,    /* sb f32 [N/128][K/128]   (weights: Fprop, Dgrad) */
    FP8FG_BSCALE_1x128 = 1       /* sb f32 [K/128][N]       (token-wise operand: Wgrad) */
};

/*
 * Online 1x128 activation quantization.
 * x: f32 [M][K] row-major (M tokens, K channels).
 * transpose_out = 0: tiles run along K (one token x 128 channels).
 *     q: u8 [M][K], s: f32 [K/128][M].          Requires K % 16 == 0.
 * transpose_out = 1: tiles run along M (128 tokens x one channel), the
 *     operand layout of the Wgrad GEMM, whose contraction runs over tokens.
 *     q: u8 [K][M] (transposed), s: f32 [M/128][K].  Requires M % 16 == 0.
 * Sizes: M, K >= 0 and M * K < 2^40.
 */
int fp8_quant_act_1x128(const float* x, int64_t M, int64_t K, int transpose_out,
                        uint8_t* q, float* s, void* stream);

/*
 * Online 128x128 weight quantization.
 * w: f32 [N][K] row-major (N output channels, K input channels).
 * transpose_out = 0: q u8 [N][K], s f32 [N/128][K/128].
 * transpose_out = 1: q u8 [K][N] = the codes of w, transposed, with
 *     s f32 [K/128][N/128]: the B operand of the Dgrad GEMM.  Square blocks
 *     make this identical to quantizing w^T.
 * Requires N % 16 == 0 and K % 16 == 0 (partial blocks at either end);
 * N * K < 2^40.
 */
int fp8_quant_weight_128x128(const float* w, int64_t N, int64_t K, int transpose_out,
                             uint8_t* q, float* s, void* stream);

/*
 * The same two quantizations with BF16 inputs: x / w hold bf16 bit patterns
 * (u16, same shapes and layouts as above).  The tensors around the FP8 GEMMs
 * stay in a wider format (DeepSeek-V3 FP8 knowledge-base page, section on
 * the mixed-precision framework), and BF16 is the one named beside FP8 ("The
 * Insider Secrets Of Deepseek Discovered", passage on FP8 and BF16 modes).
 * Each bf16 value widens to fp32 exactly, so codes and scales are identical to
 * those of the fp32 entry points on the widened tensor; the reads are half as
 * many bytes.  Sizes, alignment (16 bytes for every pointer), errors and
 * layouts as for the fp32 calls.
 */
int fp8_quant_act_1x128_bf16(const uint16_t* x, int64_t M, int64_t K, int transpose_out,
                             uint8_t* q, float* s, void* stream);
int fp8_quant_weight_128x128_bf16(const uint16_t* w, int64_t N, int64_t K, int transpose_out,
                                  uint8_t* q, float* s, void* stream);

/*
 * Both operands of a Linear layer's Fprop GEMM in one launch (both are
 * quantized online each step: "The Insider Secrets Of Deepseek Discovered",
 * passages on Figure 7(a) and on online quantization): exactly
 *   fp8_quant_act_1x128(x, M, K, 0, qa, sa)        (or _bf16 when x_bf16 = 1)
 *   fp8_quant_weight_128x128(w, N, K, 0, qb, sb)   (or _bf16 when w_bf16 = 1)
 * byte for byte, with the same layouts (qa u8 [M][K], sa f32 [K/128][M],
 * qb u8 [N][K], sb f32 [N/128][K/128]).  x / w are f32, or bf16 bit patterns
 * when x_bf16 / w_bf16 is 1.  The two small grids share one launch, so they
 * overlap instead of each paying its own ramp-up and drain.  Requires
 * K % 16 == 0, N % 16 == 0, M, N, K >= 0, M * K < 2^40 and N * K < 2^40;
 * 16-byte aligned pointers; x_bf16 and w_bf16 in {0, 1}.  M = 0 or N = 0
 * skips that operand only, as the separate call would, and that operand's
 * pointers may then be NULL; K = 0, or M = N = 0, is a successful no-op.
 * Errors as for the separate calls.
 */
int fp8_quant_fprop_operands(const void* x, int x_bf16, int64_t M, const void* w, int w_bf16, int64_t N,
                             int64_t K, uint8_t* qa, float* sa, uint8_t* qb, float* sb, void* stream);

/*
 * FP8 activation cache for backward ("The Insider Secrets Of Deepseek
 * Discovered", passage on Figure 6: with Wgrad in FP8, the input of a Linear
 * can be kept in FP8 for the backward pass).  Builds the Wgrad operand from
 * the cached Fprop operand without its fp32 source:
 *   q: u8 [M][K] with s: f32 [K/128][M]  -- 1x128 codes along K (the output
 *      of fp8_quant_act_1x128 with transpose_out = 0);
 *   x'[m][k] = RN32(decode(q[m][k]) * s[k/128][m])  (fp32, one rounding);
 *   qt: u8 [K][M], st: f32 [M/128][K]  -- 1x128 codes of x' along tokens,
 *      transposed: exactly fp8_quant_act_1x128(x', transpose_out = 1).
 * Requires M % 16 == 0 and K % 16 == 0; M * K < 2^40.  Codes 0x7F / 0xFF
 * (NaN) in q give unspecified output.
 */
int fp8_requant_act_tokenwise(const uint8_t* q, const float* s, int64_t M, int64_t K,
                              uint8_t* qt, float* st, void* stream);

/*
 * MX variant (microscaling).  "The Insider Secrets Of Deepseek Discovered",
 * passage after Figure 7: the method is consistent with microscaling
 * formats.  Reading (the pages define no MX rule): the OCP MX rule for E4M3
 * elements, one power-of-two scale per block of 32 consecutive K, stored as
 * an E8M0 byte.  This is a different numeric contract from the calls above
 * (power-of-two scales, 32-element blocks, no FP32 scale), offered beside
 * them for comparison; gfx950 applies these scales inside the MFMA.
 *
 * fp8_quant_mx_1x32: x f32 [R][K] -> codes q u8 [R][K] and scale bytes
 *   e u8 [K/32][R]:  s = clamp(floor(log2(amax)) - 8, -127, 127) per block
 *   (amax = 0 gives -127), code = E4M3_RNE_SAT(RN32(x * 2^-s)), e = s + 127.
 *   Requires K % 32 == 0; R * K < 2^40.
 * fp8_quant_mx_1x32_transposed: the same rule on blocks of 32 consecutive
 *   rows (tokens) of one column, codes written transposed -- exactly
 *   fp8_quant_mx_1x32 applied to x^T: x f32 [M][K] -> q u8 [K][M], e u8
 *   [M/32][K].  The operands of the MX Wgrad (X and dY, contraction over
 *   tokens) and the MX Dgrad weight (W [N][K] -> W^T blocked along N; "The
 *   Insider Secrets Of Deepseek Discovered", Figure 6: all three GEMMs of a
 *   Linear in FP8).  Requires M % 32 == 0 (any K); M * K < 2^40,
 *   ceil(K / 64) <= 65535.  Empty arrays may be NULL.
 * fp8_gemm_mx: C[M][N] = sum_k decode(a) 2^(ea-127) decode(b) 2^(eb-127) with
 *   a u8 [M][K], ea u8 [K/32][M], b u8 [N][K], eb u8 [K/32][N]; c BF16 or FP32
 *   [M][N].  Accuracy: |C - C*| <= 2^-9 * S (S = sum_k |a_k b_k| of the
 *   dequantized operands) plus the BF16 rounding: gfx950's FP8 MFMA sums its
 *   products with limited width.  Requires M % 4 == 0, N % 256 == 0,
 *   K % 64 == 0, K > 0 when M * N > 0, K < 2^24, (K / 32) * max(M, N) < 2^32.
 */
int fp8_quant_mx_1x32(const float* x, int64_t R, int64_t K, uint8_t* q, uint8_t* e, void* stream);
int fp8_quant_mx_1x32_transposed(const float* x, int64_t M, int64_t K, uint8_t* q, uint8_t* e, void* stream);
int fp8_gemm_mx(const uint8_t* a, const uint8_t* ea, const uint8_t* b, const uint8_t* eb,
                void* c, int out_dtype, int64_t M, int64_t N, int64_t K, void* stream);

/*
 * The MX GEMM in the two MoE layouts ("Deepgemm lançado no dia 4 da semana de
 * código aberto Deepseek", section "Principais características": dense plus a
 * contiguous and a masked grouped layout), with fp8_gemm_mx's arithmetic and
 * accuracy contract for each expert's rows:
 *   b u8 [G][N][K] with eb u8 [G][K/32][N] (each expert's weight quantized by
 *   fp8_quant_mx_1x32).
 * fp8_grouped_gemm_contiguous_mx: a u8 [M_total][K] with ea u8 [K/32][M_total]
 *   (all rows quantized together), group_offsets as for
 *   fp8_grouped_gemm_contiguous (DEVICE int32 [G+1], non-decreasing, from 0 to
 *   M_total, multiples of 128); c [M_total][N].  Rows in no expert's range are
 *   not written.  Requires M_total % 128 == 0, N % 256 == 0, K % 64 == 0,
 *   K > 0 when there is work, K < 2^24, (K / 32) * max(M_total, N) < 2^32.
 * fp8_grouped_gemm_masked_mx: a u8 [G][M_max][K] with ea u8 [G][K/32][M_max],
 *   masked_m as for fp8_grouped_gemm_masked (DEVICE int32 [G], clamped to
 *   [0, M_max] on the device); c [G][M_max][N], rows at or beyond masked_m[g]
 *   NOT written.  Requires M_max % 4 == 0, N % 256 == 0, K % 64 == 0, K > 0
 *   when there is work, K < 2^24, (K / 32) * max(M_max, N) < 2^32.
 * Each expert's rows come out bit for bit as fp8_gemm_mx gives them for that
 * expert's operands.
 */
int fp8_grouped_gemm_contiguous_mx(const uint8_t* a, const uint8_t* ea, const uint8_t* b, const uint8_t* eb,
                                   const int32_t* group_offsets, int64_t G, int64_t M_total,
                                   int64_t N, int64_t K, void* c, int out_dtype, void* stream);
int fp8_grouped_gemm_masked_mx(const uint8_t* a, const uint8_t* ea, const uint8_t* b, const uint8_t* eb,
                               const int32_t* masked_m, int64_t G, int64_t M_max,
                               int64_t N, int64_t K, void* c, int out_dtype, void* stream);

/*
 * Dense block-scaled FP8 GEMM: C[M][N] = A[M][K] . B[N][K]^T.
 * a: u8 [M][K] with sa f32 [K/128][M] (1x128 along K).
 * b: u8 [N][K] with sb laid out per bscale_kind (fp8fg_bscale).
 * c: [M][N], BF16 (uint16 bit patterns) or FP32 per out_dtype (fp8fg_out).
 * Requires M >= 0 (any value, ragged tails allowed), N % 16 == 0,
 * K % 16 == 0 (a last partial K-block is allowed), K > 0 when M*N > 0;
 * M, N, K < 2^31.
 */
int fp8_gemm_blockscaled(const uint8_t* a, const float* sa, const uint8_t* b, const float* sb,
                         int bscale_kind, void* c, int out_dtype,
                         int64_t M, int64_t N, int64_t K, void* stream);

/*
 * fp8_gemm_blockscaled on the FP8 matrix cores: the same arguments, layouts,
 * rules and errors, and the same per-K-block promotion with the scale
 * product applied at it ("The Insider Secrets Of Deepseek Discovered",
 * passage on Figure 7(b)), but each K-block's partial sum P_kb comes from
 * gfx950's FP8 MFMA (two 64-deep instructions per block) on the codes
 * themselves, at twice the rate of the BF16 matrix cores.  That instruction
 * adds its products in groups of eight consecutive K and keeps about 14
 * significant bits of each group (every product truncated toward zero to
 * 13 fractional bits below the group's largest exponent): the limited
 * accumulation the same passage measures on H800 Tensor Cores, here inside
 * one instruction, so promoting every 128 cannot remove it.
 * Accuracy contract: |C - C*| <= 2^-9 * S (FP32 out), plus one BF16
 * rounding of C* for BF16 out; the 2^-14 contract of every other call does
 * not hold here.  Deterministic.
 */
int fp8_gemm_blockscaled_fp8mfma(const uint8_t* a, const float* sa, const uint8_t* b, const float* sb,
                                 int bscale_kind, void* c, int out_dtype,
                                 int64_t M, int64_t N, int64_t K, void* stream);

/*
 * Dense GEMM with the next layer's quantization fused into the epilogue
 * ("The Insider Secrets Of Deepseek Discovered", passage on Figure 6: with
 * every Linear in FP8, a layer's output is quantized again before it feeds
 * the next one).  Computes the FP32 C of fp8_gemm_blockscaled (128x128 B
 * scales) and writes, instead of C, its 1x128 quantization along N:
 *   q: u8 [M][N], s: f32 [N/128][M] -- exactly fp8_quant_act_1x128 applied to
 *   the FP32 C that out_dtype = FP8FG_OUT_FP32 would write (same values, bit
 *   for bit), i.e. the A operand layout of a following GEMM with K = N.
 * Requires N % 256 == 0, K % 16 == 0, K > 0 when M * N > 0, K <= 11776
 * (92 K-blocks: this kernel keeps one FP32 accumulator over all of K, about
 * eleven roundings per K-block, within the 2^-14 contract up to there; else
 * FP8FG_ERR_UNSUPPORTED), ceil(K/128) * M * 4 < 2^32.
 */
int fp8_gemm_blockscaled_fp8out(const uint8_t* a, const float* sa, const uint8_t* b, const float* sb,
                                uint8_t* q, float* s, int64_t M, int64_t N, int64_t K, void* stream);

/*
 * MoE grouped GEMM, contiguous layout (training / prefill).
 * The rows of all G local experts are concatenated: expert g owns rows
 * [group_offsets[g], group_offsets[g+1]) of a / c.
 * group_offsets: DEVICE int32 [G+1], non-decreasing, group_offsets[0] = 0,
 *     group_offsets[G] = M_total, every entry a multiple of 128 (each expert's
 *     rows padded to whole 128-row tiles).  Read only on the device, so the
 *     host never waits for routing results.  A 128-row tile of a that lies
 *     outside [0, group_offsets[G]) is not computed and its rows of c are not
 *     written.  Padding rows are computed like any other row.
 * a: u8 [M_total][K], sa f32 [K/128][M_total];
 * b: u8 [G][N][K], sb f32 [G][N/128][K/128] (128x128 blocks per expert);
 * c: [M_total][N] BF16 or FP32.
 * Requires M_total % 128 == 0, N % 16 == 0, K % 16 == 0, K > 0, G >= 0.
 */
int fp8_grouped_gemm_contiguous(const uint8_t* a, const float* sa, const uint8_t* b, const float* sb,
                                const int32_t* group_offsets, int64_t G, int64_t M_total,
                                int64_t N, int64_t K, void* c, int out_dtype, void* stream);

/*
 * fp8_grouped_gemm_contiguous with the next layer's quantization fused into
 * the epilogue ("The Insider Secrets Of Deepseek Discovered", passage on
 * Figure 6: with every Linear in FP8, a layer's output is quantized again
 * before it feeds the next one -- for a MoE layer, the gate+up output that
 * feeds the down projection).  Computes the FP32 C of
 * fp8_grouped_gemm_contiguous and writes, instead of C, its 1x128
 * quantization along N:
 *   q: u8 [M_total][N], s: f32 [N/128][M_total] -- exactly
 *   fp8_quant_act_1x128 applied to the FP32 C that out_dtype = FP8FG_OUT_FP32
 *   would write (same values, bit for bit); rows in no expert's range are not
 *   written (neither q nor s).
 * Same arguments and rules as fp8_grouped_gemm_contiguous, and in addition
 * N % 256 == 0, K <= 11776 (92 K-blocks, as for fp8_gemm_blockscaled_fp8out:
 * else FP8FG_ERR_UNSUPPORTED), ceil(K/128) * M_total * 4 < 2^32.
 */
int fp8_grouped_gemm_contiguous_fp8out(const uint8_t* a, const float* sa, const uint8_t* b, const float* sb,
                                       const int32_t* group_offsets, int64_t G, int64_t M_total,
                                       int64_t N, int64_t K, uint8_t* q, float* s, void* stream);

/*
 * MoE grouped GEMM, masked layout (decode).
 * Expert g has a padded buffer of M_max rows of which the first masked_m[g]
 * are valid.
 * masked_m: DEVICE int32 [G]; each value is clamped to [0, M_max] on the
 *     device.  Rows at or beyond masked_m[g] of c are NOT written.
 * a: u8 [G][M_max][K], sa f32 [G][K/128][M_max];
 * b: u8 [G][N][K], sb f32 [G][N/128][K/128];
 * c: [G][M_max][N] BF16 or FP32.
 * Requires M_max >= 0, N % 16 == 0, K % 16 == 0, K > 0, G >= 0.
 */
int fp8_grouped_gemm_masked(const uint8_t* a, const float* sa, const uint8_t* b, const float* sb,
                            const int32_t* masked_m, int64_t G, int64_t M_max,
                            int64_t N, int64_t K, void* c, int out_dtype, void* stream);

/*
 * Decode-tiled weight layout for the masked GEMM (this library's own format;
 * the pages define the masked layout's operation -- "Deepgemm lançado no dia 4
 * da semana de código aberto Deepseek", section "Principais características"
 * -- not a storage order).  Decode streams every expert's weights once per
 * step, so a storage order in which each step of the kernel reads one
 * contiguous block raises the HBM rate; weights are static, so the
 * rearrangement is made once, when they are loaded.
 * q: u8 [G][N][K] codes, as written by fp8_quant_weight_128x128 per expert.
 * q_tiled: u8, G*N*K bytes (caller-owned, must not overlap q).  Block
 *   blk = (g * N/256 + t) * (K/64) + h (16384 bytes at offset 16384 * blk)
 *   holds rows 256 t .. 256 t + 255 of expert g, K bytes 64 h .. 64 h + 63,
 *   as sixteen 1024-byte units u = 4 w + 2 n + j (w 0..3, n 0..1, j 0..1):
 *   bytes 16 l .. 16 l + 15 of unit u (l = 0..63) are K bytes
 *   64 h + 32 j + 16 (l / 32) .. + 15 of row 256 t + 64 w + 32 n + l % 32 --
 *   the 16-byte MFMA fragments of the decode kernel in the order its lanes
 *   load them.  A pure byte permutation; the scales are not touched (sb stays
 *   [G][N/128][K/128]).
 * Requires N % 256 == 0, K % 64 == 0, K < 2^24, G >= 0 (empty arrays may be
 * NULL).
 */
int fp8_tile_weights_decode(const uint8_t* q, int64_t G, int64_t N, int64_t K, uint8_t* q_tiled, void* stream);

/*
 * fp8_grouped_gemm_masked on decode-tiled weights: the same operation, the
 * same arguments and the same result bit for bit, except that b_tiled holds
 * the experts' codes in the layout written by fp8_tile_weights_decode.
 * Requires M_max <= 128, N % 256 == 0, K % 64 == 0, K > 0, K <= 11776 (92
 * K-blocks, as for fp8_gemm_blockscaled_fp8out), G >= 0, and
 * G * ceil(M_max / 64) <= 4096 (FP8FG_ERR_UNSUPPORTED beyond).
 */
int fp8_grouped_gemm_masked_tiled(const uint8_t* a, const float* sa, const uint8_t* b_tiled, const float* sb,
                                  const int32_t* masked_m, int64_t G, int64_t M_max,
                                  int64_t N, int64_t K, void* c, int out_dtype, void* stream);

/*
 * fp8_grouped_gemm_masked_mx on decode-tiled weights: the same operation,
 * arguments and result bit for bit (each expert's valid rows as
 * fp8_gemm_mx gives them), with the experts' codes in the layout written by
 * fp8_tile_weights_decode (which the scaled FP8 MFMA reads as it stands: a
 * lane's two 16-byte pieces of a 64-K step are one operand).
 * a u8 [G][M_max][K], ea u8 [G][K/32][M_max], b_tiled (decode-tiled [G][N][K]
 * codes), eb u8 [G][K/32][N], masked_m DEVICE int32 [G] (clamped to
 * [0, M_max]); c [G][M_max][N] BF16 or FP32, rows past masked_m[g] NOT
 * written.  Requires M_max <= 128, M_max % 4 == 0, N % 256 == 0, K % 64 == 0,
 * K > 0 when there is work, K < 2^24, (K / 32) * N < 2^32,
 * G * ceil(M_max / 64) <= 4096 (FP8FG_ERR_UNSUPPORTED beyond).
 */
int fp8_grouped_gemm_masked_tiled_mx(const uint8_t* a, const uint8_t* ea, const uint8_t* b_tiled, const uint8_t* eb,
                                     const int32_t* masked_m, int64_t G, int64_t M_max,
                                     int64_t N, int64_t K, void* c, int out_dtype, void* stream);

/*
 * fp8_grouped_gemm_masked_tiled with the next layer's quantization fused into
 * the epilogue ("The Insider Secrets Of Deepseek Discovered", passage on
 * Figure 6: every Linear runs in FP8, so a layer's output is quantized again
 * before the next GEMM reads it), the decode counterpart of
 * fp8_grouped_gemm_contiguous_fp8out.  Computes the FP32 C of
 * fp8_grouped_gemm_masked_tiled and writes, instead of C, its 1x128
 * quantization along N, in the masked A operand's own layout:
 *   q: u8 [G][M_max][N], s: f32 [G][N/128][M_max] -- for every valid row,
 *   exactly fp8_quant_act_1x128 applied to the FP32 C that out_dtype =
 *   FP8FG_OUT_FP32 would write (same values, bit for bit); rows at or beyond
 *   masked_m[g] are not written (neither q nor s).
 * Same arguments and rules as fp8_grouped_gemm_masked_tiled.
 */
int fp8_grouped_gemm_masked_tiled_fp8out(const uint8_t* a, const float* sa, const uint8_t* b_tiled, const float* sb,
                                         const int32_t* masked_m, int64_t G, int64_t M_max,
                                         int64_t N, int64_t K, uint8_t* q, float* s, void* stream);

/* Human-readable name of a status code (static string, never NULL). */
const char* fp8fg_status_string(int status);

/* FP8FG_ABI_VERSION of the loaded library. */
int fp8fg_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* FP8FG_H */
