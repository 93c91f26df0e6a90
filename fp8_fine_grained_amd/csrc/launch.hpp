// Internal launchers (host side).  Arguments are validated by the C entry
// points before any of these is called.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

namespace fp8fg {

// Launch `kernel` on `stream` and return the status of this launch itself.
// (hipGetLastError() after a <<<>>> launch would also report an earlier,
// unrelated error left in the runtime's last-error slot as this call's.)
// The arguments are converted to the kernel's parameter types.
template <typename... P>
hipError_t launch_kernel(void (*kernel)(P...), dim3 grid, dim3 block, hipStream_t stream,
                         typename std::common_type<P>::type... args) {
    void* ptrs[] = {static_cast<void*>(&args)...};
    return hipLaunchKernel(reinterpret_cast<const void*>(kernel), grid, block, ptrs, 0, stream);
}

// x / w: fp32, or bf16 bit patterns when bf16 != 0
hipError_t launch_quant_act(const void* x, int bf16, int64_t M, int64_t K, int transpose_out, uint8_t* q,
                            float* s, hipStream_t stream);
hipError_t launch_requant_act_tokens(const uint8_t* qr, const float* sr, int64_t M, int64_t K, uint8_t* q, float* s,
                                     hipStream_t stream);
hipError_t launch_quant_mx(const float* x, int64_t R, int64_t K, uint8_t* q, uint8_t* e, hipStream_t stream);
// MX blocks of 32 along M, codes transposed: q [K][M], e [M/32][K]
hipError_t launch_quant_mx_tokens(const float* x, int64_t M, int64_t K, uint8_t* q, uint8_t* e, hipStream_t stream);
// both Fprop operands (rowwise activation, 128x128 weight, no transpose) in one launch
hipError_t launch_quant_fprop(const void* x, int x_bf16, int64_t M, const void* w, int w_bf16, int64_t N, int64_t K,
                              uint8_t* qa, float* sa, uint8_t* qb, float* sb, hipStream_t stream);
hipError_t launch_quant_weight(const void* w, int bf16, int64_t N, int64_t K, int transpose_out, uint8_t* q,
                               float* s, hipStream_t stream);

enum class GemmMode : int { Dense = 0, Contig = 1, Masked = 2 };

struct GemmArgs {
    const uint8_t* a;       // A codes (group 0)
    const float* sa;        // A scales, kb-major
    const uint8_t* b;       // B codes (group 0)
    const float* sb;        // B scales
    void* c;                // output (group 0)
    const int32_t* aux;     // group_offsets (contiguous) or masked_m (masked)
    int64_t M;              // rows: dense M, contiguous M_total, masked M_max (per group)
    int64_t N, K;
    int64_t G;              // groups (1 for dense)
    float* cs;              // output scales [N/128][M] of the FP8 output mode (else unused)
    int xcds = 1;           // XCDs whose L2s the tile order groups tiles for (1: the plain order)
};

// MX GEMM: args.sa / args.sb carry the E8M0 scale bytes ([K/32][M], [K/32][N];
// per expert in the grouped layouts: A's [G][K/32][M_max] when masked, B's
// [G][K/32][N])
hipError_t launch_gemm_mx(int out_fp32, GemmMode mode, const GemmArgs& args, hipStream_t stream);
// engine 0: exact (FP8 codes widened to BF16, BF16 MFMA); 1: FP8 MFMA on the codes
hipError_t launch_gemm(int engine, GemmMode mode, int bscale_1x128, int out_fp32, const GemmArgs& args,
                       hipStream_t stream);
// the masked layout on decode-tiled B (M <= 128, N % 256 == 0, K % 64 == 0);
// out_fp32 2: FP8 codes to args.c with their 1x128 scales to args.cs;
// mx: MX operands (args.sa / args.sb carry E8M0 bytes [G][K/32][M], [G][K/32][N])
hipError_t launch_gemm_masked_tiled(int out_fp32, const GemmArgs& args, hipStream_t stream, bool mx = false);
// [G][N][K] codes -> the decode-tiled layout (N % 256 == 0, K % 64 == 0)
hipError_t launch_tile_weights_decode(const uint8_t* q, int64_t G, int64_t N, int64_t K, uint8_t* out,
                                      hipStream_t stream);

}  // namespace fp8fg
