// Block-scaled FP8 GEMM with power-of-two (E8M0) 32x32 tile scales for
// gfx950: the 32x32 microscaling of "FP8 GEMM in JAX with Triton for
// Blackwell" (parameter paragraph) with the scales applied by the matrix
// cores (the scaled FP8 MFMA multiplies each 32-deep K block of a lane by
// 2^(e - 127)), so no vector-ALU promotion step is needed.  Tile loop of
// gemm_kernel.h in MODE_E8M0; the accumulators stay in the accumulation
// registers.
#include "gemm_dispatch.h"

namespace fp8k {

hipError_t launch_gemm_blockscaled_e8m0(const uint8_t* A, const uint8_t* B, const uint8_t* e8_a, const uint8_t* e8_b,
                                        void* C, int64_t M, int64_t N, int64_t K, int32_t out, hipStream_t s) {
    GemmProblem g{};
    g.A = A;
    g.B = B;
    g.C = C;
    g.scale_a = nullptr;
    g.scale_b = nullptr;
    g.offsets = nullptr;
    g.experts = 0;
    g.M = M;
    g.N = N;
    g.K = K;
    g.out_bf16 = out != 0;
    g.out_f16 = out == 2;
    g.fast_acc = 1;
    g.fmt = 0;
    g.e8_a = e8_a;
    g.e8_b = e8_b;
    if (K == 0) return fill_zero(C, M * N * (out == 0 ? 4 : 2), s);  // empty sums: C = 0
    // 256 x 256 tiles when they fill the GPU (as for the per-tensor GEMM),
    // else 128 x 128
    if (fills_with_256(M, N)) return launch_mode<256, 256, 2, 2, 1, 4, 8, MODE_E8M0>(g, s);
    return launch_mode<128, 128, 2, 2, 1, 4, 8, MODE_E8M0>(g, s);
}

}  // namespace fp8k
