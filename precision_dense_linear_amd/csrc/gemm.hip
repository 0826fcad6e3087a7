// Per-tensor scaled FP8 GEMM and its MoE grouped form, for gfx950: the
// E4M3 x E4M3 tile-class dispatch (gemm_dispatch.h), the choice between the
// operand-format pairs, and the split choice of plain GEMMs with fewer tiles
// than the GPU has workgroup slots (their partial sums meet in a workspace
// the caller provides; the library allocates nothing).
#include "gemm_dispatch.h"

namespace fp8k {

namespace {

int cu_count() {
    static const int cus = [] {
        int dev = 0, n = 0;
        if (hipGetDevice(&dev) == hipSuccess &&
            hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess && n > 0)
            return n;
        return 256;
    }();
    return cus;
}

}  // namespace

int64_t split_slots() { return 2 * (int64_t)cu_count(); }

// Splits for a plain GEMM of `tiles` tiles, `per_cu` workgroups resident per
// CU: fill the workgroup slots, at most 8 ways, each split at least 512
// bytes of K (so at least two 256-byte K stages each, never an empty one),
// and tiles * splits within the `capacity` split tiles of the workspace.
int choose_splits(int64_t tiles, int64_t K, int per_cu, int64_t capacity) {
    const int64_t slots = split_slots() / 2 * per_cu;
    if (tiles <= 0 || tiles * 2 > slots || tiles * 2 > capacity) return 1;
    int64_t sp = slots / tiles < 8 ? slots / tiles : 8;
    if (sp > capacity / tiles) sp = capacity / tiles;
    while (sp > 1 && K / sp < 512) --sp;
    return (int)sp;
}

hipError_t launch_gemm_fmt0(const GemmProblem& g, hipStream_t s) { return launch_gemm_t<0>(g, s); }

hipError_t launch_gemm(const GemmProblem& g, hipStream_t s) {
    switch (g.fmt & 3) {
        case 1: return launch_gemm_fmt1(g, s);
        case 2: return launch_gemm_fmt2(g, s);
        case 3: return launch_gemm_fmt3(g, s);
        default: return launch_gemm_fmt0(g, s);
    }
}

}  // namespace fp8k
