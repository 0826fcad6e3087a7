// Per-tensor scaled FP8 GEMM and its MoE grouped form, for gfx950: the
// E4M3 x E4M3 tile-class dispatch (gemm_dispatch.h), the choice between the
// operand-format pairs, and the split-K workspace that plain GEMMs with fewer
// tiles than the GPU has workgroup slots use.
#include <map>
#include <mutex>
#include <utility>

#include "gemm_dispatch.h"

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
struct SplitWorkspace {
    float* ws = nullptr;
    uint32_t* counters = nullptr;
};
std::mutex g_ws_mutex;
std::map<std::pair<int, hipStream_t>, SplitWorkspace> g_ws;

}  // namespace

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
