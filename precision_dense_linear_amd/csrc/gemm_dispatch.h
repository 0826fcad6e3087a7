// Tile-class dispatch of the per-tensor and grouped FP8 GEMM, for one
// operand-format pair FMT (bit 0: A holds E5M2 codes, bit 1: B; else E4M3).
// Each format pair is instantiated in a translation unit of its own
// (gemm.hip, gemm_fmt1.hip, gemm_fmt2.hip, gemm_fmt3.hip).
#pragma once

#include "gemm_kernel.h"

namespace fp8k {

// Split choice (gemm.hip).  A split tile of the workspace holds the FP32
// partial sums of one 32 x 64 tile (SPLIT_TILE_FLOATS floats).
constexpr int64_t SPLIT_TILE_FLOATS = 32 * 64;
int64_t split_slots();
int choose_splits(int64_t tiles, int64_t K, int per_cu, int64_t capacity);

inline int64_t tiles_of(int64_t M, int64_t N, int BM, int BN) { return ((M + BM - 1) / BM) * ((N + BN - 1) / BN); }

// Whether the 256 x 256 class takes a plain M x N GEMM: M > 64 and its
// tiles fill at least 7/8 of the CUs with at most 1/8 of their rows padding.
inline bool fills_with_256(int64_t M, int64_t N) {
    const int64_t cus = split_slots() / 2;   // split_slots() is twice the CU count
    const int64_t padded = (M + 255) / 256 * 256;
    return M > 64 && tiles_of(M, N, 256, 256) * 8 >= 7 * cus && 8 * (padded - M) <= M;
}

// Plain GEMM with M <= 16 (gemm_skinny.hip): the split count it would use
// (0 when the skinny class does not take the problem), and the launch.
int skinny_splits(const GemmProblem& g);
template <int FMT>
hipError_t launch_skinny(const GemmProblem& g, hipStream_t s, int splits);

template <int FMT, int BM, int BN, int WM, int WN, int KS, int NB, int GROUP_M>
hipError_t launch_cfg(const GemmProblem& g, hipStream_t s) {
    return g.fast_acc ? launch_mode<BM, BN, WM, WN, KS, NB, GROUP_M, MODE_FAST, false, FMT>(g, s)
                      : launch_mode<BM, BN, WM, WN, KS, NB, GROUP_M, MODE_EXACT, false, FMT>(g, s);
}

// The same tile class with K split `splits` ways across workgroups, their
// partials in the caller's workspace (tiles * splits <= its split tiles).
template <int FMT, int BM, int BN, int WM, int WN, int KS, int NB, int GROUP_M>
hipError_t launch_cfg_splitk(const GemmProblem& g, hipStream_t s, int32_t splits) {
    static_assert(BM * BN == SPLIT_TILE_FLOATS, "workspace sized for this tile");
    if (tiles_of(g.M, g.N, BM, BN) * splits > g.ws_tiles || !g.ws || !g.counters) return hipErrorInvalidValue;
    float* ws = g.ws;
    uint32_t* counters = g.counters;
    return g.fast_acc
               ? launch_mode<BM, BN, WM, WN, KS, NB, GROUP_M, MODE_FAST, true, FMT>(g, s, splits, ws, counters)
               : launch_mode<BM, BN, WM, WN, KS, NB, GROUP_M, MODE_EXACT, true, FMT>(g, s, splits, ws, counters);
}

// Tile configuration by shape class (a static table, no runtime tuning).
// Grouped GEMMs go by the rows per expert: <= 64 the 32 x 64 class, <= 1024
// 128 x 128, else 256 x 256.  A plain GEMM takes the largest class whose
// tiles fill the GPU:
//  * M <= 16 whose K the caller's workspace lets the skinny streaming kernel
//    split (or with at least half as many 256-column tiles as CUs): that
//    kernel (gemm_skinny.hip), in either accumulation mode -- reading B
//    bounds it, so the exact products cost nothing over the FP8 rate;
//  * 256 x 256 tiles (4 waves of 128 x 128; MFMA bound) when M > 64 and
//    they fill at least 7/8 of the CUs with at most 1/8 of their rows
//    padding;
//  * else 128 x 128 tiles (4 waves of 64 x 64 per K half, the K range split
//    over two wave groups) when M > 64 and they fill at least half of the
//    CUs;
//  * else (few tiles, or M <= 64) 32 x 64 tiles with each K step split over
//    two wave groups, K split across workgroups too when the caller gave a
//    workspace and there are fewer such tiles than half the GPU's
//    workgroup slots (measured on M = 16/32, N = 8192, K = 8192 with B out
//    of HBM: 36.5 -> 26 us) -- or, for M > 64 with more 64 x 64 tiles than
//    half the CUs, 64 x 64 tiles (2 waves of 64 x 32 per K half).
// Measured against the class each shape had before (event-timed, exact
// [FP8_ACC_FAST]): 256 x 256 instead of 128 x 128 for 1024 x 28672 x 8192
// 439 -> 392 us [319 -> 198], 512 x 28672 x 8192 251 -> 212 [139 -> 96]
// (but 1024 x 8192 x 8192, 128 tiles, 142 -> 169, and 384 x 28672 x 8192,
// a third of its rows padding, 189 -> 196); 128 x 128 instead of 256 x 256
// for 4096 x 1024 x 8192 155 -> 68 us [81 -> 37], 2048 x 2048 x 8192 155
// -> 70, 4096 x 2048 x 8192 166 -> 145 [82 -> 69], 1536 x 4096 x 8192 161
// -> 122 (but 2048 x 8192 x 8192, 256 tiles, 217 -> 263); 64 x 64 instead
// of 32 x 64 for 1024^3 10.4 -> 9.8 us, 512 x 2048 x 4096 20.4 -> 18.9
// [18.3 -> 14.0], 1024 x 1024 x 8192 36.1 -> 31.2 [32.0 -> 24.9] (these
// shapes are bound by each CU's L2 request rate, and a 64-row tile reads
// half of B's bytes per output that a 32-row one does), while with at most
// half as many 64 x 64 tiles as CUs the 32 x 64 class's twice as many
// workgroups win (512 x 1024 x 4096 14.8 against 17.3 us, 128 x 2048 x
// 8192 21.9 against 26.8) and for M <= 64 it wastes fewer rows (40 x 4096
// x 4096 13.7 against 16.6).  (The 32 x 64 class replaced 128 x 128 tiles
// there earlier: 1024^3 11.8 -> 8.6 us, 512 x 2048 x 4096 27.0 -> 18.6,
// 1024 x 1024 x 8192 47.6 -> 32.8, kernel time.)
template <int FMT>
hipError_t launch_gemm_t(const GemmProblem& g, hipStream_t s) {
    if (g.experts > 0) {
        const int64_t rows_per_expert = (g.M + g.experts - 1) / g.experts;
        if (rows_per_expert <= 64) return launch_cfg<FMT, 32, 64, 1, 2, 2, 4, 8>(g, s);
        if (rows_per_expert <= 1024) return launch_cfg<FMT, 128, 128, 2, 2, 2, 4, 8>(g, s);
        return launch_cfg<FMT, 256, 256, 2, 2, 1, 4, 8>(g, s);
    }
    if (g.M <= 16) {
        const int sk = skinny_splits(g);
        if (sk > 0) return launch_skinny<FMT>(g, s, sk);
    }
    const int64_t cus = split_slots() / 2;
    if (fills_with_256(g.M, g.N)) return launch_cfg<FMT, 256, 256, 2, 2, 1, 4, 8>(g, s);
    if (g.M > 64 && tiles_of(g.M, g.N, 128, 128) * 2 >= cus) return launch_cfg<FMT, 128, 128, 2, 2, 2, 4, 8>(g, s);
    const int sp = g.ws_tiles > 0 ? choose_splits(tiles_of(g.M, g.N, 32, 64), g.K, 2, g.ws_tiles) : 1;
    if (sp > 1) return launch_cfg_splitk<FMT, 32, 64, 1, 2, 2, 4, 8>(g, s, sp);
    if (g.M > 64 && tiles_of(g.M, g.N, 64, 64) * 2 > cus) return launch_cfg<FMT, 64, 64, 1, 2, 2, 4, 8>(g, s);
    return launch_cfg<FMT, 32, 64, 1, 2, 2, 4, 8>(g, s);
}

}  // namespace fp8k
