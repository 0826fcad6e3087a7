// The per-tensor and grouped FP8 GEMM for E5M2 A x E5M2 B operands ("FP8 GEMM in
// JAX with Triton for Blackwell", opening section: the E4M3 and E5M2
// formats on the matrix cores), compiled on its own.
#include "gemm_dispatch.h"

namespace fp8k {

hipError_t launch_gemm_fmt3(const GemmProblem& g, hipStream_t s) { return launch_gemm_t<3>(g, s); }

}  // namespace fp8k
