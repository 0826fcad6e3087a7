// Per-tensor scaled FP8 GEMM and its MoE grouped form, for gfx950: tile
// configuration by shape class over the tile loop of gemm_kernel.h.
#include "gemm_kernel.h"

namespace fp8k {

namespace {

template <int BM, int BN, int WM, int WN, int KS, int NB, int GROUP_M>
hipError_t launch_cfg(const GemmProblem& g, hipStream_t s) {
    return g.fast_acc ? launch_mode<BM, BN, WM, WN, KS, NB, GROUP_M, MODE_FAST>(g, s)
                      : launch_mode<BM, BN, WM, WN, KS, NB, GROUP_M, MODE_EXACT>(g, s);
}

}  // namespace

// Tile configuration by shape class (a static table, no runtime tuning):
//  * M (rows per expert when grouped) <= 64: 32 x 64 tiles with each K step
//    split over two wave groups -- many workgroups to stream B, HBM bound;
//  * M <= 1024: 128 x 128 tiles, 4 waves of 64 x 64 per K half, the K range
//    split over two wave groups (more loads in flight per tile);
//  * larger M: 256 x 256 tiles, 4 waves of 128 x 128 -- MFMA bound.
hipError_t launch_gemm(const GemmProblem& g, hipStream_t s) {
    const int64_t rows_per_problem = g.experts ? (g.M + g.experts - 1) / g.experts : g.M;
    if (rows_per_problem <= 64) return launch_cfg<32, 64, 1, 2, 2, 4, 8>(g, s);
    if (rows_per_problem <= 1024) return launch_cfg<128, 128, 2, 2, 2, 4, 8>(g, s);
    return launch_cfg<256, 256, 2, 2, 1, 4, 8>(g, s);
}

}  // namespace fp8k
