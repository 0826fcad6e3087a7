// Block-scaled FP8 GEMM (32x32 or 64x64 tile scales) for gfx950, over the
// tile loop of gemm_kernel.h in MODE_BLOCK / MODE_BLOCK64.  This file is
// compiled with the MFMA results forced into the architectural VGPRs: the
// partial products feed the vector FMAs that fold them into the
// accumulators, which cannot read the accumulation registers directly.
#include "gemm_kernel.h"

namespace fp8k {

// Block-scaled GEMM (block: 32 or 64): 128 x 128 tiles of 4 waves of
// 64 x 64, whose FP32 accumulators and partial products both live in the
// vector registers the scale folding works on (two workgroups per CU).
hipError_t launch_gemm_blockscaled(const uint8_t* A, const uint8_t* B, const float* s_a, const float* s_b, void* C,
                                   int64_t M, int64_t N, int64_t K, int32_t out, int32_t block, hipStream_t s) {
    GemmProblem g{};
    g.A = A;
    g.B = B;
    g.C = C;
    g.scale_a = s_a;
    g.scale_b = s_b;
    g.offsets = nullptr;
    g.experts = 0;
    g.M = M;
    g.N = N;
    g.K = K;
    g.out_bf16 = out != 0;
    g.out_f16 = out == 2;
    g.fast_acc = 0;
    g.fmt = 0;
    if (K == 0) return fill_zero(C, M * N * (out == 0 ? 4 : 2), s);  // empty sums: C = 0
    if (block == 64) return launch_mode<128, 128, 2, 2, 1, 4, 8, MODE_BLOCK64>(g, s);
    return launch_mode<128, 128, 2, 2, 1, 4, 8, MODE_BLOCK>(g, s);
}

}  // namespace fp8k
