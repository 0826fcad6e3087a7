// Per-tensor scaled FP8 GEMM and its MoE grouped form, for gfx950: tile
// configuration by shape class over the tile loop of gemm_kernel.h, and
// split-K across workgroups for plain GEMMs with fewer tiles than the GPU
// has workgroup slots.
#include <map>
#include <mutex>
#include <utility>

#include "gemm_kernel.h"

namespace fp8k {

namespace {

__global__ void zero_u32(uint32_t* p, int n) {
    const int i = blockIdx.x * blockDim.x + threadIdx.x;
    if (i < n) p[i] = 0u;
}

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

// Split-K workspace, one per (device, stream): calls on one stream run in
// order, so they never use it concurrently.  Allocated at its fixed maximum
// (FP32 partials for 2 * CUs split tiles of 32 x 64, plus one arrival counter
// per tile: 4 MiB at 256 CUs) by the first split-K call on the stream, and
// kept until the process ends.  The counters are zeroed once, on the stream,
// when allocated; every launch leaves them at zero again.
constexpr int64_t SPLIT_TILE_FLOATS = 32 * 64;
struct SplitWorkspace {
    float* ws = nullptr;
    uint32_t* counters = nullptr;
};
std::mutex g_ws_mutex;
std::map<std::pair<int, hipStream_t>, SplitWorkspace> g_ws;

int64_t split_slots() { return 2 * (int64_t)cu_count(); }

hipError_t get_workspace(hipStream_t s, float** ws, uint32_t** counters) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    std::lock_guard<std::mutex> lock(g_ws_mutex);
    SplitWorkspace& w = g_ws[std::make_pair(dev, s)];
    if (!w.ws) {
        const int64_t slots = split_slots();
        void* mem = nullptr;
        e = hipMalloc(&mem, (size_t)slots * SPLIT_TILE_FLOATS * sizeof(float) + (size_t)slots * sizeof(uint32_t));
        if (e != hipSuccess) return e;
        float* f = static_cast<float*>(mem);
        uint32_t* c = reinterpret_cast<uint32_t*>(f + slots * SPLIT_TILE_FLOATS);
        hipLaunchKernelGGL(zero_u32, dim3((unsigned)((slots + 255) / 256)), dim3(256), 0, s, c, (int)slots);
        e = hipGetLastError();
        if (e != hipSuccess) {
            (void)hipFree(mem);
            return e;
        }
        w.ws = f;
        w.counters = c;
    }
    *ws = w.ws;
    *counters = w.counters;
    return hipSuccess;
}

// Splits for a plain GEMM of `tiles` tiles, `per_cu` workgroups resident per
// CU: fill the workgroup slots, at most 8 ways, each split at least 512
// bytes of K (so at least two 256-byte K stages each, never an empty one).
// tiles * splits <= 2 * CUs bounds the workspace (4 MiB at 256 CUs).
int choose_splits(int64_t tiles, int64_t K, int per_cu) {
    const int64_t slots = split_slots() / 2 * per_cu;
    if (tiles <= 0 || tiles * 2 > slots) return 1;
    int sp = (int)(slots / tiles < 8 ? slots / tiles : 8);
    while (sp > 1 && K / sp < 512) --sp;
    return sp;
}

int64_t tiles_of(int64_t M, int64_t N, int BM, int BN) { return ((M + BM - 1) / BM) * ((N + BN - 1) / BN); }

template <int BM, int BN, int WM, int WN, int KS, int NB, int GROUP_M>
hipError_t launch_cfg(const GemmProblem& g, hipStream_t s) {
    return g.fast_acc ? launch_mode<BM, BN, WM, WN, KS, NB, GROUP_M, MODE_FAST>(g, s)
                      : launch_mode<BM, BN, WM, WN, KS, NB, GROUP_M, MODE_EXACT>(g, s);
}

// The same tile class with K split `splits` ways across workgroups
// (tiles * splits <= the workspace's split tiles).
template <int BM, int BN, int WM, int WN, int KS, int NB, int GROUP_M>
hipError_t launch_cfg_splitk(const GemmProblem& g, hipStream_t s, int32_t splits) {
    static_assert(BM * BN == SPLIT_TILE_FLOATS, "workspace sized for this tile");
    if (tiles_of(g.M, g.N, BM, BN) * splits > split_slots()) return hipErrorInvalidValue;
    float* ws = nullptr;
    uint32_t* counters = nullptr;
    const hipError_t e = get_workspace(s, &ws, &counters);
    if (e != hipSuccess) return e;
    return g.fast_acc ? launch_mode<BM, BN, WM, WN, KS, NB, GROUP_M, MODE_FAST, true>(g, s, splits, ws, counters)
                      : launch_mode<BM, BN, WM, WN, KS, NB, GROUP_M, MODE_EXACT, true>(g, s, splits, ws, counters);
}

}  // namespace

// Tile configuration by shape class (a static table, no runtime tuning):
//  * M (rows per expert when grouped) <= 64: 32 x 64 tiles with each K step
//    split over two wave groups -- many workgroups to stream B, HBM bound; a
//    plain GEMM with fewer such tiles than half the GPU's workgroup slots
//    also splits K across workgroups (measured on M = 16/32, N = 8192,
//    K = 8192 with B out of HBM: 36.5 -> 26 us);
//  * M <= 1024: 128 x 128 tiles, 4 waves of 64 x 64 per K half, the K range
//    split over two wave groups (more loads in flight per tile);
//  * larger M: 256 x 256 tiles, 4 waves of 128 x 128 -- MFMA bound.
hipError_t launch_gemm(const GemmProblem& g, hipStream_t s) {
    const bool plain = g.experts == 0;
    const int64_t rows_per_problem = plain ? g.M : (g.M + g.experts - 1) / g.experts;
    if (rows_per_problem <= 64) {
        const int sp = plain ? choose_splits(tiles_of(g.M, g.N, 32, 64), g.K, 2) : 1;
        if (sp > 1) return launch_cfg_splitk<32, 64, 1, 2, 2, 4, 8>(g, s, sp);
        return launch_cfg<32, 64, 1, 2, 2, 4, 8>(g, s);
    }
    if (rows_per_problem <= 1024) return launch_cfg<128, 128, 2, 2, 2, 4, 8>(g, s);
    return launch_cfg<256, 256, 2, 2, 1, 4, 8>(g, s);
}

}  // namespace fp8k
