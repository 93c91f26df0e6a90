// C entry points of libfp8fg.so (declared in include/fp8fg.h).
//
// Every argument is checked on the host before anything is enqueued, in this
// order: NULL pointers, sizes and each call's multiple-of rules, 16-byte
// alignment, enum values.  A zero-sized problem returns FP8FG_OK without touching the
// HIP runtime, so these checks can be exercised on a machine without a GPU.
#include "fp8fg.h"
#include "launch.hpp"

#include <stdint.h>

namespace {

constexpr int64_t kMaxDim = (int64_t(1) << 31) - 1;
constexpr int64_t kMaxElems = int64_t(1) << 40;
// K-blocks of the calls that always run the wide exact kernel, whose single
// FP32 accumulator keeps the 2^-14 S contract up to this many (gemm.hip)
constexpr int64_t kWideMaxKBlocks = 92;

inline bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

inline int hip_status(hipError_t e) { return e == hipSuccess ? FP8FG_OK : FP8FG_ERR_HIP; }

inline bool valid_out(int out_dtype) { return out_dtype == FP8FG_OUT_BF16 || out_dtype == FP8FG_OUT_FP32; }

}  // namespace

extern "C" {

int fp8fg_abi_version(void) { return FP8FG_ABI_VERSION; }

const char* fp8fg_status_string(int status) {
    switch (status) {
        case FP8FG_OK: return "ok";
        case FP8FG_ERR_NULL: return "null pointer argument";
        case FP8FG_ERR_SHAPE: return "invalid shape (negative size, or a size that breaks the call's multiple-of rule)";
        case FP8FG_ERR_ALIGN: return "pointer not 16-byte aligned";
        case FP8FG_ERR_UNSUPPORTED: return "unsupported argument value or size";
        case FP8FG_ERR_HIP: return "HIP runtime error at launch";
        default: return "unknown status";
    }
}

// the quantizers' checks, shared by the fp32 and bf16 entry points
static int quant_act(const void* x, int bf16, int64_t M, int64_t K, int transpose_out, uint8_t* q, float* s,
                     void* stream) {
    if (M > 0 && K > 0 && (!x || !q || !s)) return FP8FG_ERR_NULL;   // empty arrays may be NULL
    if (M < 0 || K < 0) return FP8FG_ERR_SHAPE;
    if (transpose_out != 0 && transpose_out != 1) return FP8FG_ERR_UNSUPPORTED;
    // the grouped axis: a multiple of 16 (a last partial group is allowed)
    if (transpose_out == 0 && K % 16 != 0) return FP8FG_ERR_SHAPE;
    if (transpose_out == 1 && M % 16 != 0) return FP8FG_ERR_SHAPE;
    if (!aligned16(x) || !aligned16(q) || !aligned16(s)) return FP8FG_ERR_ALIGN;
    if (M > kMaxDim || K > kMaxDim || (M > 0 && K > kMaxElems / M)) return FP8FG_ERR_UNSUPPORTED;
    if (transpose_out == 1 && ((K + 63) / 64 > 65535)) return FP8FG_ERR_UNSUPPORTED;
    if (M == 0 || K == 0) return FP8FG_OK;
    return hip_status(fp8fg::launch_quant_act(x, bf16, M, K, transpose_out, q, s, static_cast<hipStream_t>(stream)));
}

static int quant_weight(const void* w, int bf16, int64_t N, int64_t K, int transpose_out, uint8_t* q, float* s,
                        void* stream) {
    if (N > 0 && K > 0 && (!w || !q || !s)) return FP8FG_ERR_NULL;   // empty arrays may be NULL
    if (N < 0 || K < 0 || N % 16 != 0 || K % 16 != 0) return FP8FG_ERR_SHAPE;
    if (transpose_out != 0 && transpose_out != 1) return FP8FG_ERR_UNSUPPORTED;
    if (!aligned16(w) || !aligned16(q) || !aligned16(s)) return FP8FG_ERR_ALIGN;
    if (N > kMaxDim || K > kMaxDim || (N > 0 && K > kMaxElems / N)) return FP8FG_ERR_UNSUPPORTED;
    if ((N + 127) / 128 > 65535) return FP8FG_ERR_UNSUPPORTED;
    if (N == 0 || K == 0) return FP8FG_OK;
    return hip_status(
        fp8fg::launch_quant_weight(w, bf16, N, K, transpose_out, q, s, static_cast<hipStream_t>(stream)));
}

int fp8_quant_act_1x128(const float* x, int64_t M, int64_t K, int transpose_out, uint8_t* q, float* s,
                        void* stream) {
    return quant_act(x, 0, M, K, transpose_out, q, s, stream);
}

int fp8_quant_act_1x128_bf16(const uint16_t* x, int64_t M, int64_t K, int transpose_out, uint8_t* q, float* s,
                             void* stream) {
    return quant_act(x, 1, M, K, transpose_out, q, s, stream);
}

int fp8_quant_weight_128x128(const float* w, int64_t N, int64_t K, int transpose_out, uint8_t* q, float* s,
                             void* stream) {
    return quant_weight(w, 0, N, K, transpose_out, q, s, stream);
}

int fp8_quant_weight_128x128_bf16(const uint16_t* w, int64_t N, int64_t K, int transpose_out, uint8_t* q, float* s,
                                  void* stream) {
    return quant_weight(w, 1, N, K, transpose_out, q, s, stream);
}

int fp8_quant_fprop_operands(const void* x, int x_bf16, int64_t M, const void* w, int w_bf16, int64_t N, int64_t K,
                             uint8_t* qa, float* sa, uint8_t* qb, float* sb, void* stream) {
    // an operand with no elements may come with NULL pointers (never touched)
    if (M > 0 && K > 0 && (!x || !qa || !sa)) return FP8FG_ERR_NULL;
    if (N > 0 && K > 0 && (!w || !qb || !sb)) return FP8FG_ERR_NULL;
    if (M < 0 || N < 0 || K < 0 || K % 16 != 0 || N % 16 != 0) return FP8FG_ERR_SHAPE;
    if ((x_bf16 != 0 && x_bf16 != 1) || (w_bf16 != 0 && w_bf16 != 1)) return FP8FG_ERR_UNSUPPORTED;
    if (!aligned16(x) || !aligned16(w) || !aligned16(qa) || !aligned16(sa) || !aligned16(qb) || !aligned16(sb))
        return FP8FG_ERR_ALIGN;
    if (M > kMaxDim || N > kMaxDim || K > kMaxDim || (M > 0 && K > kMaxElems / M) || (N > 0 && K > kMaxElems / N))
        return FP8FG_ERR_UNSUPPORTED;
    // one 1-D grid: weight blocks plus rowwise workgroups (at most 65535 row groups)
    const int64_t kbs = (K + 127) / 128;
    if (kbs * ((N + 127) / 128) + ((kbs + 3) / 4) * 65535 > 0x7FFFFFFF) return FP8FG_ERR_UNSUPPORTED;
    if (K == 0 || (M == 0 && N == 0)) return FP8FG_OK;
    return hip_status(fp8fg::launch_quant_fprop(x, x_bf16, M, w, w_bf16, N, K, qa, sa, qb, sb,
                                                static_cast<hipStream_t>(stream)));
}

int fp8_requant_act_tokenwise(const uint8_t* q, const float* s, int64_t M, int64_t K, uint8_t* qt, float* st,
                              void* stream) {
    if (!q || !s || !qt || !st) return FP8FG_ERR_NULL;
    if (M < 0 || K < 0 || M % 16 != 0 || K % 16 != 0) return FP8FG_ERR_SHAPE;
    if (!aligned16(q) || !aligned16(s) || !aligned16(qt) || !aligned16(st)) return FP8FG_ERR_ALIGN;
    if (M > kMaxDim || K > kMaxDim || (M > 0 && K > kMaxElems / M)) return FP8FG_ERR_UNSUPPORTED;
    if (K / 64 > 65535 || M / 128 > 0x7FFFFFFF) return FP8FG_ERR_UNSUPPORTED;
    if (M == 0 || K == 0) return FP8FG_OK;
    return hip_status(fp8fg::launch_requant_act_tokens(q, s, M, K, qt, st, static_cast<hipStream_t>(stream)));
}

int fp8_quant_mx_1x32(const float* x, int64_t R, int64_t K, uint8_t* q, uint8_t* e, void* stream) {
    if (!x || !q || !e) return FP8FG_ERR_NULL;
    if (R < 0 || K < 0 || K % 32 != 0) return FP8FG_ERR_SHAPE;
    if (!aligned16(x) || !aligned16(q) || !aligned16(e)) return FP8FG_ERR_ALIGN;
    if (R > kMaxDim || K > kMaxDim || (R > 0 && K > kMaxElems / R)) return FP8FG_ERR_UNSUPPORTED;
    if (R == 0 || K == 0) return FP8FG_OK;
    return hip_status(fp8fg::launch_quant_mx(x, R, K, q, e, static_cast<hipStream_t>(stream)));
}

int fp8_quant_mx_1x32_transposed(const float* x, int64_t M, int64_t K, uint8_t* q, uint8_t* e, void* stream) {
    if (M > 0 && K > 0 && (!x || !q || !e)) return FP8FG_ERR_NULL;   // empty arrays may be NULL
    if (M < 0 || K < 0 || M % 32 != 0) return FP8FG_ERR_SHAPE;
    if (!aligned16(x) || !aligned16(q) || !aligned16(e)) return FP8FG_ERR_ALIGN;
    if (M > kMaxDim || K > kMaxDim || (M > 0 && K > kMaxElems / M)) return FP8FG_ERR_UNSUPPORTED;
    if ((K + 63) / 64 > 65535) return FP8FG_ERR_UNSUPPORTED;
    if (M == 0 || K == 0) return FP8FG_OK;
    return hip_status(fp8fg::launch_quant_mx_tokens(x, M, K, q, e, static_cast<hipStream_t>(stream)));
}

int fp8_gemm_mx(const uint8_t* a, const uint8_t* ea, const uint8_t* b, const uint8_t* eb, void* c, int out_dtype,
                int64_t M, int64_t N, int64_t K, void* stream) {
    if (!a || !ea || !b || !eb || !c) return FP8FG_ERR_NULL;
    if (M < 0 || N < 0 || K < 0 || M % 4 != 0 || N % 256 != 0 || K % 64 != 0) return FP8FG_ERR_SHAPE;
    if (K == 0 && M > 0 && N > 0) return FP8FG_ERR_SHAPE;
    if (!aligned16(a) || !aligned16(ea) || !aligned16(b) || !aligned16(eb) || !aligned16(c)) return FP8FG_ERR_ALIGN;
    if (!valid_out(out_dtype)) return FP8FG_ERR_UNSUPPORTED;
    if (M > kMaxDim || N > kMaxDim || K >= (int64_t(1) << 24)) return FP8FG_ERR_UNSUPPORTED;
    if ((K / 32) * M > int64_t(0xFFFFFF00) || (K / 32) * N > int64_t(0xFFFFFF00)) return FP8FG_ERR_UNSUPPORTED;
    if (((M + 255) / 256) * (N / 256) > kMaxDim) return FP8FG_ERR_UNSUPPORTED;
    if (M == 0 || N == 0) return FP8FG_OK;
    fp8fg::GemmArgs args{a, reinterpret_cast<const float*>(ea), b, reinterpret_cast<const float*>(eb), c,
                         nullptr, M, N, K, 1};
    return hip_status(fp8fg::launch_gemm_mx(out_dtype == FP8FG_OUT_FP32, fp8fg::GemmMode::Dense, args,
                                            static_cast<hipStream_t>(stream)));
}

int fp8_grouped_gemm_contiguous_mx(const uint8_t* a, const uint8_t* ea, const uint8_t* b, const uint8_t* eb,
                                   const int32_t* group_offsets, int64_t G, int64_t M_total, int64_t N, int64_t K,
                                   void* c, int out_dtype, void* stream) {
    if (!a || !ea || !b || !eb || !group_offsets || !c) return FP8FG_ERR_NULL;
    if (G < 0 || M_total < 0 || N < 0 || K < 0 || M_total % 128 != 0 || N % 256 != 0 || K % 64 != 0)
        return FP8FG_ERR_SHAPE;
    if (K == 0 && M_total > 0 && N > 0 && G > 0) return FP8FG_ERR_SHAPE;
    if (!aligned16(a) || !aligned16(ea) || !aligned16(b) || !aligned16(eb) || !aligned16(c) ||
        !aligned16(group_offsets))
        return FP8FG_ERR_ALIGN;
    if (!valid_out(out_dtype)) return FP8FG_ERR_UNSUPPORTED;
    if (M_total > kMaxDim || N > kMaxDim || K >= (int64_t(1) << 24) || G > kMaxDim - 1) return FP8FG_ERR_UNSUPPORTED;
    if ((K / 32) * M_total > int64_t(0xFFFFFF00) || (K / 32) * N > int64_t(0xFFFFFF00)) return FP8FG_ERR_UNSUPPORTED;
    if ((M_total / 256 + G) * (N / 256) > kMaxDim) return FP8FG_ERR_UNSUPPORTED;
    if (G == 0 || M_total == 0 || N == 0) return FP8FG_OK;
    fp8fg::GemmArgs args{a, reinterpret_cast<const float*>(ea), b, reinterpret_cast<const float*>(eb), c,
                         group_offsets, M_total, N, K, G};
    return hip_status(fp8fg::launch_gemm_mx(out_dtype == FP8FG_OUT_FP32, fp8fg::GemmMode::Contig, args,
                                            static_cast<hipStream_t>(stream)));
}

int fp8_grouped_gemm_masked_mx(const uint8_t* a, const uint8_t* ea, const uint8_t* b, const uint8_t* eb,
                               const int32_t* masked_m, int64_t G, int64_t M_max, int64_t N, int64_t K, void* c,
                               int out_dtype, void* stream) {
    if (!a || !ea || !b || !eb || !masked_m || !c) return FP8FG_ERR_NULL;
    if (G < 0 || M_max < 0 || N < 0 || K < 0 || M_max % 4 != 0 || N % 256 != 0 || K % 64 != 0)
        return FP8FG_ERR_SHAPE;
    if (K == 0 && M_max > 0 && N > 0 && G > 0) return FP8FG_ERR_SHAPE;
    if (!aligned16(a) || !aligned16(ea) || !aligned16(b) || !aligned16(eb) || !aligned16(c) || !aligned16(masked_m))
        return FP8FG_ERR_ALIGN;
    if (!valid_out(out_dtype)) return FP8FG_ERR_UNSUPPORTED;
    if (M_max > kMaxDim || N > kMaxDim || K >= (int64_t(1) << 24) || G > kMaxDim) return FP8FG_ERR_UNSUPPORTED;
    if ((K / 32) * M_max > int64_t(0xFFFFFF00) || (K / 32) * N > int64_t(0xFFFFFF00)) return FP8FG_ERR_UNSUPPORTED;
    const int64_t tiles_per_group = ((M_max + 255) / 256) * (N / 256);
    if (tiles_per_group > 0 && G > kMaxDim / tiles_per_group) return FP8FG_ERR_UNSUPPORTED;
    if (G == 0 || M_max == 0 || N == 0) return FP8FG_OK;
    fp8fg::GemmArgs args{a, reinterpret_cast<const float*>(ea), b, reinterpret_cast<const float*>(eb), c, masked_m,
                         M_max, N, K, G};
    return hip_status(fp8fg::launch_gemm_mx(out_dtype == FP8FG_OUT_FP32, fp8fg::GemmMode::Masked, args,
                                            static_cast<hipStream_t>(stream)));
}

// the dense call's checks; engine 0 = exact, 1 = FP8 MFMA
static int gemm_dense(const uint8_t* a, const float* sa, const uint8_t* b, const float* sb, int bscale_kind, void* c,
                      int out_dtype, int64_t M, int64_t N, int64_t K, void* stream, int engine) {
    if (!a || !sa || !b || !sb || !c) return FP8FG_ERR_NULL;
    if (M < 0 || N < 0 || K < 0 || N % 16 != 0 || K % 16 != 0) return FP8FG_ERR_SHAPE;
    if (K == 0 && M > 0 && N > 0) return FP8FG_ERR_SHAPE;
    if (!aligned16(a) || !aligned16(sa) || !aligned16(b) || !aligned16(sb) || !aligned16(c)) return FP8FG_ERR_ALIGN;
    if (bscale_kind != FP8FG_BSCALE_128x128 && bscale_kind != FP8FG_BSCALE_1x128) return FP8FG_ERR_UNSUPPORTED;
    if (!valid_out(out_dtype)) return FP8FG_ERR_UNSUPPORTED;
    if (M > kMaxDim || N > kMaxDim || K > kMaxDim) return FP8FG_ERR_UNSUPPORTED;
    if (((M + 127) / 128) * ((N + 127) / 128) > kMaxDim) return FP8FG_ERR_UNSUPPORTED;
    if (M == 0 || N == 0) return FP8FG_OK;
    fp8fg::GemmArgs args{a, sa, b, sb, c, nullptr, M, N, K, 1};
    return hip_status(fp8fg::launch_gemm(engine, fp8fg::GemmMode::Dense, bscale_kind == FP8FG_BSCALE_1x128,
                                         out_dtype == FP8FG_OUT_FP32, args, static_cast<hipStream_t>(stream)));
}

int fp8_gemm_blockscaled(const uint8_t* a, const float* sa, const uint8_t* b, const float* sb, int bscale_kind,
                         void* c, int out_dtype, int64_t M, int64_t N, int64_t K, void* stream) {
    return gemm_dense(a, sa, b, sb, bscale_kind, c, out_dtype, M, N, K, stream, 0);
}

int fp8_gemm_blockscaled_fp8mfma(const uint8_t* a, const float* sa, const uint8_t* b, const float* sb,
                                 int bscale_kind, void* c, int out_dtype, int64_t M, int64_t N, int64_t K,
                                 void* stream) {
    return gemm_dense(a, sa, b, sb, bscale_kind, c, out_dtype, M, N, K, stream, 1);
}

int fp8_gemm_blockscaled_fp8out(const uint8_t* a, const float* sa, const uint8_t* b, const float* sb, uint8_t* q,
                                float* s, int64_t M, int64_t N, int64_t K, void* stream) {
    if (!a || !sa || !b || !sb || !q || !s) return FP8FG_ERR_NULL;
    if (M < 0 || N < 0 || K < 0 || N % 256 != 0 || K % 16 != 0) return FP8FG_ERR_SHAPE;
    if (K == 0 && M > 0 && N > 0) return FP8FG_ERR_SHAPE;
    if (!aligned16(a) || !aligned16(sa) || !aligned16(b) || !aligned16(sb) || !aligned16(q) || !aligned16(s))
        return FP8FG_ERR_ALIGN;
    if (M > kMaxDim || N > kMaxDim || (K + 127) / 128 > kWideMaxKBlocks) return FP8FG_ERR_UNSUPPORTED;
    if (((K + 127) / 128) * M * 4 > int64_t(0xFFFFFFFF)) return FP8FG_ERR_UNSUPPORTED;
    if (((M + 255) / 256) * (N / 256) > kMaxDim) return FP8FG_ERR_UNSUPPORTED;
    if (M == 0 || N == 0) return FP8FG_OK;
    fp8fg::GemmArgs args{a, sa, b, sb, q, nullptr, M, N, K, 1, s};
    return hip_status(fp8fg::launch_gemm(0, fp8fg::GemmMode::Dense, 0, 2, args, static_cast<hipStream_t>(stream)));
}

int fp8_grouped_gemm_contiguous(const uint8_t* a, const float* sa, const uint8_t* b, const float* sb,
                                const int32_t* group_offsets, int64_t G, int64_t M_total, int64_t N, int64_t K,
                                void* c, int out_dtype, void* stream) {
    if (!a || !sa || !b || !sb || !group_offsets || !c) return FP8FG_ERR_NULL;
    if (G < 0 || M_total < 0 || N < 0 || K < 0 || M_total % 128 != 0 || N % 16 != 0 || K % 16 != 0)
        return FP8FG_ERR_SHAPE;
    if (K == 0 && M_total > 0 && N > 0 && G > 0) return FP8FG_ERR_SHAPE;
    if (!aligned16(a) || !aligned16(sa) || !aligned16(b) || !aligned16(sb) || !aligned16(c) ||
        !aligned16(group_offsets))
        return FP8FG_ERR_ALIGN;
    if (!valid_out(out_dtype)) return FP8FG_ERR_UNSUPPORTED;
    if (M_total > kMaxDim || N > kMaxDim || K > kMaxDim || G > kMaxDim - 1) return FP8FG_ERR_UNSUPPORTED;
    if ((M_total / 128) * ((N + 127) / 128) > kMaxDim) return FP8FG_ERR_UNSUPPORTED;
    if (G == 0 || M_total == 0 || N == 0) return FP8FG_OK;
    fp8fg::GemmArgs args{a, sa, b, sb, c, group_offsets, M_total, N, K, G};
    return hip_status(fp8fg::launch_gemm(0, fp8fg::GemmMode::Contig, 0, out_dtype == FP8FG_OUT_FP32, args,
                                         static_cast<hipStream_t>(stream)));
}

int fp8_grouped_gemm_contiguous_fp8out(const uint8_t* a, const float* sa, const uint8_t* b, const float* sb,
                                       const int32_t* group_offsets, int64_t G, int64_t M_total, int64_t N,
                                       int64_t K, uint8_t* q, float* s, void* stream) {
    if (!a || !sa || !b || !sb || !group_offsets || !q || !s) return FP8FG_ERR_NULL;
    if (G < 0 || M_total < 0 || N < 0 || K < 0 || M_total % 128 != 0 || N % 256 != 0 || K % 16 != 0)
        return FP8FG_ERR_SHAPE;
    if (K == 0 && M_total > 0 && N > 0 && G > 0) return FP8FG_ERR_SHAPE;
    if (!aligned16(a) || !aligned16(sa) || !aligned16(b) || !aligned16(sb) || !aligned16(q) || !aligned16(s) ||
        !aligned16(group_offsets))
        return FP8FG_ERR_ALIGN;
    if (M_total > kMaxDim || N > kMaxDim || G > kMaxDim - 1 || (K + 127) / 128 > kWideMaxKBlocks)
        return FP8FG_ERR_UNSUPPORTED;
    if (((K + 127) / 128) * M_total * 4 > int64_t(0xFFFFFFFF)) return FP8FG_ERR_UNSUPPORTED;
    if ((M_total / 128) * ((N + 127) / 128) > kMaxDim) return FP8FG_ERR_UNSUPPORTED;
    if (G == 0 || M_total == 0 || N == 0) return FP8FG_OK;
    fp8fg::GemmArgs args{a, sa, b, sb, q, group_offsets, M_total, N, K, G, s};
    return hip_status(fp8fg::launch_gemm(0, fp8fg::GemmMode::Contig, 0, 2, args, static_cast<hipStream_t>(stream)));
}

int fp8_grouped_gemm_masked(const uint8_t* a, const float* sa, const uint8_t* b, const float* sb,
                            const int32_t* masked_m, int64_t G, int64_t M_max, int64_t N, int64_t K, void* c,
                            int out_dtype, void* stream) {
    if (!a || !sa || !b || !sb || !masked_m || !c) return FP8FG_ERR_NULL;
    if (G < 0 || M_max < 0 || N < 0 || K < 0 || N % 16 != 0 || K % 16 != 0) return FP8FG_ERR_SHAPE;
    if (K == 0 && M_max > 0 && N > 0 && G > 0) return FP8FG_ERR_SHAPE;
    if (!aligned16(a) || !aligned16(sa) || !aligned16(b) || !aligned16(sb) || !aligned16(c) || !aligned16(masked_m))
        return FP8FG_ERR_ALIGN;
    if (!valid_out(out_dtype)) return FP8FG_ERR_UNSUPPORTED;
    if (M_max > kMaxDim || N > kMaxDim || K > kMaxDim || G > kMaxDim) return FP8FG_ERR_UNSUPPORTED;
    const int64_t tiles_per_group = ((M_max + 127) / 128) * ((N + 127) / 128);
    if (tiles_per_group > 0 && G > kMaxDim / tiles_per_group) return FP8FG_ERR_UNSUPPORTED;
    if (G == 0 || M_max == 0 || N == 0) return FP8FG_OK;
    fp8fg::GemmArgs args{a, sa, b, sb, c, masked_m, M_max, N, K, G};
    return hip_status(fp8fg::launch_gemm(0, fp8fg::GemmMode::Masked, 0, out_dtype == FP8FG_OUT_FP32, args,
                                         static_cast<hipStream_t>(stream)));
}

int fp8_tile_weights_decode(const uint8_t* q, int64_t G, int64_t N, int64_t K, uint8_t* q_tiled, void* stream) {
    if (G > 0 && N > 0 && K > 0 && (!q || !q_tiled)) return FP8FG_ERR_NULL;   // empty arrays may be NULL
    if (G < 0 || N < 0 || K < 0 || N % 256 != 0 || K % 64 != 0) return FP8FG_ERR_SHAPE;
    if (!aligned16(q) || !aligned16(q_tiled)) return FP8FG_ERR_ALIGN;
    if (G > kMaxDim || N > kMaxDim || K >= (int64_t(1) << 24)) return FP8FG_ERR_UNSUPPORTED;
    if (G == 0 || N == 0 || K == 0) return FP8FG_OK;
    if (G * N > kMaxElems / K) return FP8FG_ERR_UNSUPPORTED;
    return hip_status(fp8fg::launch_tile_weights_decode(q, G, N, K, q_tiled, static_cast<hipStream_t>(stream)));
}

int fp8_grouped_gemm_masked_tiled_mx(const uint8_t* a, const uint8_t* ea, const uint8_t* b_tiled, const uint8_t* eb,
                                     const int32_t* masked_m, int64_t G, int64_t M_max, int64_t N, int64_t K, void* c,
                                     int out_dtype, void* stream) {
    if (!a || !ea || !b_tiled || !eb || !masked_m || !c) return FP8FG_ERR_NULL;
    if (G < 0 || M_max < 0 || N < 0 || K < 0 || M_max % 4 != 0 || N % 256 != 0 || K % 64 != 0) return FP8FG_ERR_SHAPE;
    if (K == 0 && M_max > 0 && N > 0 && G > 0) return FP8FG_ERR_SHAPE;
    if (!aligned16(a) || !aligned16(ea) || !aligned16(b_tiled) || !aligned16(eb) || !aligned16(c) ||
        !aligned16(masked_m))
        return FP8FG_ERR_ALIGN;
    if (!valid_out(out_dtype)) return FP8FG_ERR_UNSUPPORTED;
    if (M_max > 128 || N > kMaxDim || K >= (int64_t(1) << 24) || G > kMaxDim) return FP8FG_ERR_UNSUPPORTED;
    if ((K / 32) * N > int64_t(0xFFFFFF00)) return FP8FG_ERR_UNSUPPORTED;
    if (N > 0 && G > kMaxDim / (2 * (N / 256))) return FP8FG_ERR_UNSUPPORTED;
    if (G * ((M_max + 63) / 64) > 4096) return FP8FG_ERR_UNSUPPORTED;
    if (G == 0 || M_max == 0 || N == 0) return FP8FG_OK;
    fp8fg::GemmArgs args{a, reinterpret_cast<const float*>(ea), b_tiled, reinterpret_cast<const float*>(eb), c,
                         masked_m, M_max, N, K, G};
    return hip_status(fp8fg::launch_gemm_masked_tiled(out_dtype == FP8FG_OUT_FP32, args,
                                                      static_cast<hipStream_t>(stream), true));
}

int fp8_grouped_gemm_masked_tiled_fp8out(const uint8_t* a, const float* sa, const uint8_t* b_tiled, const float* sb,
                                         const int32_t* masked_m, int64_t G, int64_t M_max, int64_t N, int64_t K,
                                         uint8_t* q, float* s, void* stream) {
    if (!a || !sa || !b_tiled || !sb || !masked_m || !q || !s) return FP8FG_ERR_NULL;
    if (G < 0 || M_max < 0 || N < 0 || K < 0 || N % 256 != 0 || K % 64 != 0) return FP8FG_ERR_SHAPE;
    if (K == 0 && M_max > 0 && N > 0 && G > 0) return FP8FG_ERR_SHAPE;
    if (!aligned16(a) || !aligned16(sa) || !aligned16(b_tiled) || !aligned16(sb) || !aligned16(q) || !aligned16(s) ||
        !aligned16(masked_m))
        return FP8FG_ERR_ALIGN;
    if (M_max > 128 || N > kMaxDim || (K + 127) / 128 > kWideMaxKBlocks || G > kMaxDim) return FP8FG_ERR_UNSUPPORTED;
    if (N > 0 && G > kMaxDim / (2 * (N / 256))) return FP8FG_ERR_UNSUPPORTED;
    if (G * ((M_max + 63) / 64) > 4096) return FP8FG_ERR_UNSUPPORTED;
    if (G == 0 || M_max == 0 || N == 0) return FP8FG_OK;
    fp8fg::GemmArgs args{a, sa, b_tiled, sb, q, masked_m, M_max, N, K, G, s};
    return hip_status(fp8fg::launch_gemm_masked_tiled(2, args, static_cast<hipStream_t>(stream)));
}

int fp8_grouped_gemm_masked_tiled(const uint8_t* a, const float* sa, const uint8_t* b_tiled, const float* sb,
                                  const int32_t* masked_m, int64_t G, int64_t M_max, int64_t N, int64_t K, void* c,
                                  int out_dtype, void* stream) {
    if (!a || !sa || !b_tiled || !sb || !masked_m || !c) return FP8FG_ERR_NULL;
    if (G < 0 || M_max < 0 || N < 0 || K < 0 || N % 256 != 0 || K % 64 != 0) return FP8FG_ERR_SHAPE;
    if (K == 0 && M_max > 0 && N > 0 && G > 0) return FP8FG_ERR_SHAPE;
    if (!aligned16(a) || !aligned16(sa) || !aligned16(b_tiled) || !aligned16(sb) || !aligned16(c) ||
        !aligned16(masked_m))
        return FP8FG_ERR_ALIGN;
    if (!valid_out(out_dtype)) return FP8FG_ERR_UNSUPPORTED;
    // the decode tile: buffers of at most 128 rows; 256 K bytes per n-tile stay below 4 GiB
    if (M_max > 128 || N > kMaxDim || (K + 127) / 128 > kWideMaxKBlocks || G > kMaxDim) return FP8FG_ERR_UNSUPPORTED;
    if (N > 0 && G > kMaxDim / (2 * (N / 256))) return FP8FG_ERR_UNSUPPORTED;
    // the decode kernel ranks at most 4096 (expert, 64-row m-tile) pairs
    if (G * ((M_max + 63) / 64) > 4096) return FP8FG_ERR_UNSUPPORTED;
    if (G == 0 || M_max == 0 || N == 0) return FP8FG_OK;
    fp8fg::GemmArgs args{a, sa, b_tiled, sb, c, masked_m, M_max, N, K, G};
    return hip_status(fp8fg::launch_gemm_masked_tiled(out_dtype == FP8FG_OUT_FP32, args,
                                                      static_cast<hipStream_t>(stream)));
}

}  // extern "C"
