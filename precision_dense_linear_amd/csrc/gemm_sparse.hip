// FP8 GEMM with a 2:4-sparse weight matrix on the sparse FP8 matrix cores
// of gfx950 ("FP8 GEMM in JAX with Triton for Blackwell", opening section:
// the matrix cores' sparsity support, about twice the efficiency at 50%
// weight sparsity).  B is stored compressed -- the two kept values of every
// group of 4 along K, [K/2][N], and their 2-bit positions, one word per
// column and 32-deep K block, [K/32][N] -- and fed to
// v_smfmac_f32_32x32x64_fp8_fp8, which multiplies 64 K per instruction at
// twice the dense rate.  Tile loop of gemm_kernel.h in MODE_SPARSE.
#include "gemm_dispatch.h"

namespace fp8k {

hipError_t launch_gemm_sparse24(const uint8_t* A, const uint8_t* Bv, const uint32_t* Bi, const float* scale_a,
                                const float* scale_b, void* C, int64_t M, int64_t N, int64_t K, int32_t out,
                                hipStream_t s) {
    if (K == 0) return fill_zero(C, M * N * (out == 0 ? 4 : 2), s);  // empty sums: C = 0
    GemmProblem g{};
    g.A = A;
    g.B = Bv;
    g.C = C;
    g.scale_a = scale_a;
    g.scale_b = scale_b;
    g.offsets = nullptr;
    g.experts = 0;
    g.M = M;
    g.N = N;
    g.K = K;
    g.out_bf16 = out != 0;
    g.out_f16 = out == 2;
    g.fast_acc = 1;
    g.fmt = 0;
    g.sp_idx = Bi;
    // 256 x 256 tiles when they fill the GPU (as for the per-tensor GEMM),
    // else 128 x 128
    if (fills_with_256(M, N)) return launch_mode<256, 256, 2, 2, 1, 4, 8, MODE_SPARSE>(g, s);
    return launch_mode<128, 128, 2, 2, 1, 4, 8, MODE_SPARSE>(g, s);
}

}  // namespace fp8k
