// C ABI (include/fp8gemm.h): argument validation on the host, then the
// launchers.  Nothing here allocates, synchronises or touches the GPU before
// every check has passed, so the error paths run without a device.
#include <stdarg.h>
#include <stdio.h>
#include <stdint.h>

#include <mutex>

#include "../../include/fp8gemm.h"
#include "launch.h"

namespace {

thread_local char g_err[512] = "";

fp8_status fail(fp8_status st, const char* fmt, ...) {
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_err, sizeof(g_err), fmt, ap);
    va_end(ap);
    return st;
}

fp8_status ok() {
    g_err[0] = '\0';
    return FP8_OK;
}

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

fp8_status from_hip(hipError_t e, const char* what) {
    if (e == hipSuccess) return ok();
    return fail(FP8_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

constexpr int64_t kMaxK = int64_t(1) << 23;  // 256 rows x K stays below 2^31 bytes per tile
constexpr int64_t kMaxN = int64_t(1) << 20;  // 256 K-rows x N stays below 2^31 bytes per step
// Split-K workspace: per split tile, the FP32 partial sums of a 32 x 64 tile
// and a 4-byte arrival counter (FP8_GEMM_WS_TILE_BYTES in all).
constexpr int64_t kSplitTileFloatBytes = 32 * 64 * 4;
static_assert(kSplitTileFloatBytes + 4 == FP8_GEMM_WS_TILE_BYTES, "workspace tile size");

fp8_status check_gemm_common(const void* A, const void* B, const void* C, int64_t M, int64_t N, int64_t K,
                             int32_t out_dtype, int32_t allowed_flags) {
    if (M < 0 || N < 0 || K < 0) return fail(FP8_ERR_INVALID_ARG, "negative size (M=%lld N=%lld K=%lld)",
                                             (long long)M, (long long)N, (long long)K);
    // size limits first: past them M * K, K * N or M * N could overflow below
    if (K > kMaxK) return fail(FP8_ERR_UNSUPPORTED_SHAPE, "K=%lld exceeds 2^23", (long long)K);
    if (N > kMaxN) return fail(FP8_ERR_UNSUPPORTED_SHAPE, "N=%lld exceeds 2^20", (long long)N);
    if (M > (int64_t(1) << 31) - 1) return fail(FP8_ERR_UNSUPPORTED_SHAPE, "M=%lld exceeds 2^31-1", (long long)M);
    // an operand with no elements may be null
    if ((!A && M * K > 0) || (!B && K * N > 0) || (!C && M * N > 0))
        return fail(FP8_ERR_INVALID_ARG, "null matrix pointer");
    const int32_t base = out_dtype & 0xFF;
    if (out_dtype & ~(0xFF | allowed_flags))
        return fail(FP8_ERR_INVALID_ARG, "out_dtype %#x has flag bits this call does not take (%#x)", out_dtype,
                    out_dtype & ~(0xFF | allowed_flags));
    if (base != FP8_OUT_F32 && base != FP8_OUT_BF16 && base != FP8_OUT_F16)
        return fail(FP8_ERR_INVALID_ARG,
                    "out_dtype %#x is not FP8_OUT_F32, FP8_OUT_BF16 or FP8_OUT_F16 (| FP8_ACC_FAST, FP8_A_E5M2, "
                    "FP8_B_E5M2)",
                    out_dtype);
    if (!aligned16(A) || !aligned16(B) || !aligned16(C)) return fail(FP8_ERR_INVALID_ARG, "A, B and C must be 16-byte aligned");
    return FP8_OK;
}

// The launcher's view of out_dtype: output kind, accumulation mode, formats.
void decode_out(int32_t out_dtype, fp8k::GemmProblem& g) {
    const int32_t base = out_dtype & 0xFF;
    g.out_bf16 = base != FP8_OUT_F32;
    g.out_f16 = base == FP8_OUT_F16;
    g.fast_acc = (out_dtype & FP8_ACC_FAST) != 0;
    g.fmt = ((out_dtype & FP8_A_E5M2) ? 1 : 0) | ((out_dtype & FP8_B_E5M2) ? 2 : 0);
}

fp8_status quantize_pertensor(const float* x, int64_t n, uint8_t* q, float* scale, float* amax, int fmt, void* stream,
                              const char* what) {
    if (n < 0) return fail(FP8_ERR_INVALID_ARG, "negative n=%lld", (long long)n);
    if (!scale || !amax || (n > 0 && (!x || !q))) return fail(FP8_ERR_INVALID_ARG, "null pointer argument");
    if (!aligned16(x) || !aligned16(q)) return fail(FP8_ERR_INVALID_ARG, "x and q must be 16-byte aligned");
    if (scale == amax) return fail(FP8_ERR_INVALID_ARG, "scale and amax must be distinct");
    return from_hip(fp8k::launch_quantize_pertensor(x, n, q, scale, amax, fmt, (hipStream_t)stream), what);
}

fp8_status quantize_blocked(const float* x, int64_t rows, int64_t cols, int T, uint8_t* q, float* tile_scales,
                            void* stream, const char* what) {
    if (!x || !q || !tile_scales) return fail(FP8_ERR_INVALID_ARG, "null pointer argument");
    if (rows < 0 || cols < 0) return fail(FP8_ERR_INVALID_ARG, "negative size");
    if (rows % T || cols % T)
        return fail(FP8_ERR_UNSUPPORTED_SHAPE, "rows=%lld and cols=%lld must be multiples of %d", (long long)rows,
                    (long long)cols, T);
    if (!aligned16(x) || !aligned16(q)) return fail(FP8_ERR_INVALID_ARG, "x and q must be 16-byte aligned");
    if ((rows / T) * (cols / T) > (int64_t(1) << 34)) return fail(FP8_ERR_UNSUPPORTED_SHAPE, "too many tiles");
    return from_hip(fp8k::launch_quantize_blocked(x, rows, cols, T, q, tile_scales, (hipStream_t)stream), what);
}

fp8_status quantize_grouped(const float* x, int64_t rows, int64_t cols, const int32_t* offsets, int32_t groups,
                            uint8_t* q, float* scales, float* amax, int fmt, void* stream, const char* what) {
    if (!x || !q || !scales || !amax || !offsets) return fail(FP8_ERR_INVALID_ARG, "null pointer argument");
    if (rows < 0 || cols < 0) return fail(FP8_ERR_INVALID_ARG, "negative size");
    if (groups < 1 || groups > 1024) return fail(FP8_ERR_INVALID_ARG, "groups=%d outside [1, 1024]", groups);
    if (cols % 4) return fail(FP8_ERR_UNSUPPORTED_SHAPE, "cols=%lld must be a multiple of 4", (long long)cols);
    if (rows > (int64_t(1) << 31) - 1) return fail(FP8_ERR_UNSUPPORTED_SHAPE, "rows exceed 2^31-1");
    if (!aligned16(x) || !aligned16(q)) return fail(FP8_ERR_INVALID_ARG, "x and q must be 16-byte aligned");
    if (scales == amax) return fail(FP8_ERR_INVALID_ARG, "scales and amax must be distinct");
    return from_hip(
        fp8k::launch_quantize_grouped(x, rows, cols, offsets, groups, q, scales, amax, fmt, (hipStream_t)stream),
        what);
}

// Argument checks of the per-tensor GEMM (fp8_gemm and its variants).
fp8_status check_pertensor(const uint8_t* A, const uint8_t* B, const float* scale_a, const float* scale_b,
                           const void* C, int64_t M, int64_t N, int64_t K, int32_t out_dtype) {
    fp8_status st = check_gemm_common(A, B, C, M, N, K, out_dtype, FP8_ACC_FAST | FP8_A_E5M2 | FP8_B_E5M2);
    if (st != FP8_OK) return st;
    if (!scale_a || !scale_b) return fail(FP8_ERR_INVALID_ARG, "null scale pointer");
    if (K % 16 || N % 16)
        return fail(FP8_ERR_UNSUPPORTED_SHAPE, "K=%lld and N=%lld must be multiples of 16", (long long)K, (long long)N);
    return FP8_OK;
}

// The per-tensor GEMM with an optional split-K workspace (ws_tiles split
// tiles: FP32 partial sums first, then one arrival counter per split tile).
// Arguments already checked.
fp8_status launch_pertensor(const uint8_t* A, const uint8_t* B, const float* scale_a, const float* scale_b, void* C,
                            int64_t M, int64_t N, int64_t K, int32_t out_dtype, void* ws, int64_t ws_tiles,
                            void* stream, const char* what) {
    if (M == 0 || N == 0) return ok();
    fp8k::GemmProblem g{A, B, C, scale_a, scale_b, nullptr, 0, M, N, K, 0, 0, 0, 0};
    decode_out(out_dtype, g);
    if (ws && ws_tiles > 0) {
        g.ws = static_cast<float*>(ws);
        g.counters = reinterpret_cast<uint32_t*>(static_cast<uint8_t*>(ws) + ws_tiles * kSplitTileFloatBytes);
        g.ws_tiles = ws_tiles;
    }
    return from_hip(fp8k::launch_gemm(g, (hipStream_t)stream), what);
}

fp8_status gemm_pertensor(const uint8_t* A, const uint8_t* B, const float* scale_a, const float* scale_b, void* C,
                          int64_t M, int64_t N, int64_t K, int32_t out_dtype, void* ws, int64_t ws_tiles,
                          void* stream, const char* what) {
    const fp8_status st = check_pertensor(A, B, scale_a, scale_b, C, M, N, K, out_dtype);
    if (st != FP8_OK) return st;
    return launch_pertensor(A, B, scale_a, scale_b, C, M, N, K, out_dtype, ws, ws_tiles, stream, what);
}

// fp8_gemm_noalloc's split-K workspace: one array per GPU, in the library's
// own device memory, for callers that cannot allocate.  Host code never uses
// the array's name as an address: at the first call on a device its address
// there is looked up with hipGetSymbolAddress (with that device current) and
// kept in scratch_ptr[device].
constexpr int kMaxDevices = 64;
static __device__ __align__(256) uint8_t scratch[FP8_GEMM_WORKSPACE_BYTES];
std::mutex scratch_mutex;
void* scratch_ptr[kMaxDevices] = {};

__global__ void zero_words(uint32_t* p, int n) {
    const int i = blockIdx.x * blockDim.x + threadIdx.x;
    if (i < n) p[i] = 0u;
}

// The device address of the current device's scratch array (set up on the
// first call there: the symbol lookup, then a fill kernel on `s` that clears
// the arrival counters, which every completed call leaves at zero again).
fp8_status scratch_for_current_device(hipStream_t s, void** out) {
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return fail(FP8_ERR_HIP, "fp8_gemm_noalloc: hipGetDevice: %s", hipGetErrorString(e));
    if (dev < 0 || dev >= kMaxDevices) return fail(FP8_ERR_INVALID_ARG, "fp8_gemm_noalloc: device %d out of range", dev);
    std::lock_guard<std::mutex> lock(scratch_mutex);
    if (!scratch_ptr[dev]) {
        void* ptr = nullptr;
        e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
        if (e != hipSuccess || !ptr)
            return fail(FP8_ERR_HIP, "fp8_gemm_noalloc: hipGetSymbolAddress: %s", hipGetErrorString(e));
        constexpr int tiles = FP8_GEMM_WORKSPACE_BYTES / FP8_GEMM_WS_TILE_BYTES;
        uint32_t* counters = reinterpret_cast<uint32_t*>(static_cast<uint8_t*>(ptr) + tiles * kSplitTileFloatBytes);
        hipLaunchKernelGGL(zero_words, dim3((tiles + 255) / 256), dim3(256), 0, s, counters, tiles);
        e = hipGetLastError();
        if (e != hipSuccess) return fail(FP8_ERR_HIP, "fp8_gemm_noalloc: clearing the counters: %s", hipGetErrorString(e));
        scratch_ptr[dev] = ptr;
    }
    *out = scratch_ptr[dev];
    return FP8_OK;
}

}  // namespace

extern "C" {

const char* fp8_status_string(int32_t status) {
    switch (status) {
        case FP8_OK: return "FP8_OK";
        case FP8_ERR_INVALID_ARG: return "FP8_ERR_INVALID_ARG";
        case FP8_ERR_UNSUPPORTED_SHAPE: return "FP8_ERR_UNSUPPORTED_SHAPE";
        case FP8_ERR_HIP: return "FP8_ERR_HIP";
        default: return "FP8_ERR_UNKNOWN";
    }
}

const char* fp8_last_error(void) { return g_err; }

fp8_status fp8_quantize(const float* x, int64_t n, uint8_t* q, float* scale, float* amax, void* stream) {
    return quantize_pertensor(x, n, q, scale, amax, 0, stream, "fp8_quantize");
}

fp8_status fp8_quantize_e5m2(const float* x, int64_t n, uint8_t* q, float* scale, float* amax, void* stream) {
    return quantize_pertensor(x, n, q, scale, amax, 1, stream, "fp8_quantize_e5m2");
}

fp8_status fp8_quantize_blocked(const float* x, int64_t rows, int64_t cols, uint8_t* q, float* tile_scales,
                                void* stream) {
    return quantize_blocked(x, rows, cols, 32, q, tile_scales, stream, "fp8_quantize_blocked");
}

fp8_status fp8_quantize_blocked64(const float* x, int64_t rows, int64_t cols, uint8_t* q, float* tile_scales,
                                  void* stream) {
    return quantize_blocked(x, rows, cols, 64, q, tile_scales, stream, "fp8_quantize_blocked64");
}

fp8_status fp8_quantize_blocked_e8m0(const float* x, int64_t rows, int64_t cols, int32_t k_major, uint8_t* q,
                                     uint8_t* tile_exps, void* stream) {
    if (!x || !q || !tile_exps) return fail(FP8_ERR_INVALID_ARG, "null pointer argument");
    if (k_major != 0 && k_major != 1) return fail(FP8_ERR_INVALID_ARG, "k_major=%d is neither 0 nor 1", k_major);
    if ((uintptr_t)tile_exps & 3) return fail(FP8_ERR_INVALID_ARG, "tile_exps must be 4-byte aligned");
    if (rows < 0 || cols < 0) return fail(FP8_ERR_INVALID_ARG, "negative size");
    if (rows % 32 || cols % 32)
        return fail(FP8_ERR_UNSUPPORTED_SHAPE, "rows=%lld and cols=%lld must be multiples of 32", (long long)rows,
                    (long long)cols);
    if (!aligned16(x) || !aligned16(q)) return fail(FP8_ERR_INVALID_ARG, "x and q must be 16-byte aligned");
    if ((rows / 32) * (cols / 32) > (int64_t(1) << 34)) return fail(FP8_ERR_UNSUPPORTED_SHAPE, "too many tiles");
    return from_hip(fp8k::launch_quantize_blocked_e8m0(x, rows, cols, q, tile_exps, k_major, (hipStream_t)stream),
                    "fp8_quantize_blocked_e8m0");
}

fp8_status fp8_quantize_grouped(const float* x, int64_t rows, int64_t cols, const int32_t* offsets, int32_t groups,
                                uint8_t* q, float* scales, float* amax, void* stream) {
    return quantize_grouped(x, rows, cols, offsets, groups, q, scales, amax, 0, stream, "fp8_quantize_grouped");
}

fp8_status fp8_quantize_grouped_e5m2(const float* x, int64_t rows, int64_t cols, const int32_t* offsets,
                                     int32_t groups, uint8_t* q, float* scales, float* amax, void* stream) {
    return quantize_grouped(x, rows, cols, offsets, groups, q, scales, amax, 1, stream, "fp8_quantize_grouped_e5m2");
}

fp8_status fp8_gemm(const uint8_t* A, const uint8_t* B, const float* scale_a, const float* scale_b, void* C,
                    int64_t M, int64_t N, int64_t K, int32_t out_dtype, void* stream) {
    return gemm_pertensor(A, B, scale_a, scale_b, C, M, N, K, out_dtype, nullptr, 0, stream, "fp8_gemm");
}

fp8_status fp8_gemm_ws(const uint8_t* A, const uint8_t* B, const float* scale_a, const float* scale_b, void* C,
                       int64_t M, int64_t N, int64_t K, int32_t out_dtype, void* workspace, int64_t workspace_bytes,
                       void* stream) {
    if (workspace_bytes < 0) return fail(FP8_ERR_INVALID_ARG, "negative workspace_bytes=%lld", (long long)workspace_bytes);
    if (!workspace && workspace_bytes > 0) return fail(FP8_ERR_INVALID_ARG, "null workspace with workspace_bytes > 0");
    if (!aligned16(workspace)) return fail(FP8_ERR_INVALID_ARG, "the workspace must be 16-byte aligned");
    return gemm_pertensor(A, B, scale_a, scale_b, C, M, N, K, out_dtype, workspace,
                          workspace_bytes / FP8_GEMM_WS_TILE_BYTES, stream, "fp8_gemm_ws");
}

fp8_status fp8_gemm_noalloc(const uint8_t* A, const uint8_t* B, const float* scale_a, const float* scale_b, void* C,
                            int64_t M, int64_t N, int64_t K, int32_t out_dtype, void* stream) {
    // argument checks first (no device work for a rejected or empty call),
    // then the scratch array of the current device
    fp8_status st = check_pertensor(A, B, scale_a, scale_b, C, M, N, K, out_dtype);
    if (st != FP8_OK) return st;
    if (M == 0 || N == 0) return ok();
    void* ws = nullptr;
    st = scratch_for_current_device((hipStream_t)stream, &ws);
    if (st != FP8_OK) return st;
    return launch_pertensor(A, B, scale_a, scale_b, C, M, N, K, out_dtype, ws,
                            FP8_GEMM_WORKSPACE_BYTES / FP8_GEMM_WS_TILE_BYTES, stream, "fp8_gemm_noalloc");
}

fp8_status fp8_gemm_blockscaled(const uint8_t* A, const uint8_t* B, const float* s_a, const float* s_b, void* C,
                                int64_t M, int64_t N, int64_t K, int32_t out_dtype, void* stream) {
    if (out_dtype & FP8_ACC_FAST)
        return fail(FP8_ERR_INVALID_ARG, "FP8_ACC_FAST is not available for the block-scaled GEMM");
    if (out_dtype & (FP8_A_E5M2 | FP8_B_E5M2))
        return fail(FP8_ERR_INVALID_ARG, "the block-scaled GEMM takes E4M3 operands only");
    fp8_status st = check_gemm_common(A, B, C, M, N, K, out_dtype, FP8_BLOCK64);
    if (st != FP8_OK) return st;
    if (!s_a || !s_b) return fail(FP8_ERR_INVALID_ARG, "null scale pointer");
    const int32_t T = (out_dtype & FP8_BLOCK64) ? 64 : 32;
    if (M % T || N % T || K % T)
        return fail(FP8_ERR_UNSUPPORTED_SHAPE, "M=%lld N=%lld K=%lld must be multiples of %d", (long long)M,
                    (long long)N, (long long)K, T);
    if (M == 0 || N == 0) return ok();
    return from_hip(fp8k::launch_gemm_blockscaled(A, B, s_a, s_b, C, M, N, K, out_dtype & 0xFF, T, (hipStream_t)stream),
                    "fp8_gemm_blockscaled");
}

fp8_status fp8_gemm_blockscaled_e8m0(const uint8_t* A, const uint8_t* B, const uint8_t* e_a, const uint8_t* e_b,
                                     void* C, int64_t M, int64_t N, int64_t K, int32_t out_dtype, void* stream) {
    fp8_status st = check_gemm_common(A, B, C, M, N, K, out_dtype, 0);
    if (st != FP8_OK) return st;
    if ((!e_a || !e_b) && K > 0) return fail(FP8_ERR_INVALID_ARG, "null exponent pointer");  // empty when K == 0
    if (((uintptr_t)e_a & 3) || ((uintptr_t)e_b & 3))
        return fail(FP8_ERR_INVALID_ARG, "the exponent arrays must be 4-byte aligned");
    if (M % 32 || N % 32 || K % 32)
        return fail(FP8_ERR_UNSUPPORTED_SHAPE, "M=%lld N=%lld K=%lld must be multiples of 32", (long long)M,
                    (long long)N, (long long)K);
    if (M == 0 || N == 0) return ok();
    return from_hip(
        fp8k::launch_gemm_blockscaled_e8m0(A, B, e_a, e_b, C, M, N, K, out_dtype & 0xFF, (hipStream_t)stream),
        "fp8_gemm_blockscaled_e8m0");
}

fp8_status fp8_quantize_2of4(const float* w, int64_t K, int64_t N, uint8_t* vals, uint32_t* idx, float* scale,
                             float* amax, void* stream) {
    if (K < 0 || N < 0) return fail(FP8_ERR_INVALID_ARG, "negative size");
    if (!scale || !amax || (K * N > 0 && (!w || !vals || !idx))) return fail(FP8_ERR_INVALID_ARG, "null pointer argument");
    if (K % 32) return fail(FP8_ERR_UNSUPPORTED_SHAPE, "K=%lld must be a multiple of 32", (long long)K);
    if (!aligned16(w) || ((uintptr_t)idx & 3)) return fail(FP8_ERR_INVALID_ARG, "w must be 16-byte and idx 4-byte aligned");
    if (scale == amax) return fail(FP8_ERR_INVALID_ARG, "scale and amax must be distinct");
    if (K > kMaxK || N > kMaxN) return fail(FP8_ERR_UNSUPPORTED_SHAPE, "K or N too large");
    return from_hip(fp8k::launch_quantize_2of4(w, K, N, vals, idx, scale, amax, (hipStream_t)stream),
                    "fp8_quantize_2of4");
}

fp8_status fp8_gemm_sparse24(const uint8_t* A, const uint8_t* Bv, const uint32_t* Bi, const float* scale_a,
                             const float* scale_b, void* C, int64_t M, int64_t N, int64_t K, int32_t out_dtype,
                             void* stream) {
    fp8_status st = check_gemm_common(A, Bv, C, M, N, K, out_dtype, 0);
    if (st != FP8_OK) return st;
    if (!scale_a || !scale_b) return fail(FP8_ERR_INVALID_ARG, "null scale pointer");
    if (!Bi && K * N > 0) return fail(FP8_ERR_INVALID_ARG, "null index pointer");
    if (!aligned16(Bi)) return fail(FP8_ERR_INVALID_ARG, "the index words must be 16-byte aligned");
    if (K % 32 || N % 16)
        return fail(FP8_ERR_UNSUPPORTED_SHAPE, "K=%lld must be a multiple of 32 and N=%lld of 16", (long long)K,
                    (long long)N);
    if (M == 0 || N == 0) return ok();
    return from_hip(fp8k::launch_gemm_sparse24(A, Bv, Bi, scale_a, scale_b, C, M, N, K, out_dtype & 0xFF,
                                               (hipStream_t)stream),
                    "fp8_gemm_sparse24");
}

fp8_status fp8_attention(const uint8_t* Q, const uint8_t* K, const uint8_t* V, const float* scale_q,
                         const float* scale_k, const float* scale_v, void* O, int64_t batch_heads, int64_t seq_q,
                         int64_t seq_kv, int64_t head_dim, float softmax_scale, int32_t causal, int32_t out_dtype,
                         void* stream) {
    if (batch_heads < 0 || seq_q < 0 || seq_kv < 0)
        return fail(FP8_ERR_INVALID_ARG, "negative size (batch_heads=%lld seq_q=%lld seq_kv=%lld)",
                    (long long)batch_heads, (long long)seq_q, (long long)seq_kv);
    if (head_dim != 64 && head_dim != 128)
        return fail(FP8_ERR_UNSUPPORTED_SHAPE, "head_dim=%lld is neither 64 nor 128", (long long)head_dim);
    const bool fast_qk = (out_dtype & FP8_ACC_FAST) != 0;
    const int32_t out_kind = out_dtype & ~FP8_ACC_FAST;
    if (out_kind != FP8_OUT_F32 && out_kind != FP8_OUT_BF16 && out_kind != FP8_OUT_F16)
        return fail(FP8_ERR_INVALID_ARG,
                    "out_dtype %#x is not FP8_OUT_F32, FP8_OUT_BF16 or FP8_OUT_F16 (optionally with FP8_ACC_FAST)",
                    out_dtype);
    if (causal != 0 && causal != 1) return fail(FP8_ERR_INVALID_ARG, "causal=%d is neither 0 nor 1", causal);
    if (!(softmax_scale > 0.0f) || softmax_scale > 3.0e38f)
        return fail(FP8_ERR_INVALID_ARG, "softmax_scale must be positive and finite");
    // one head's Q, K or V stays below 2^31 bytes (32-bit buffer offsets)
    if (seq_q > (int64_t(1) << 31) / head_dim - 1 || seq_kv > (int64_t(1) << 31) / head_dim - 1)
        return fail(FP8_ERR_UNSUPPORTED_SHAPE, "seq_q=%lld or seq_kv=%lld exceeds 2^31 / head_dim - 1",
                    (long long)seq_q, (long long)seq_kv);
    if (batch_heads * ((seq_q + 127) / 128) > (int64_t(1) << 31) - 1)
        return fail(FP8_ERR_UNSUPPORTED_SHAPE, "too many query blocks");
    const int64_t nq = batch_heads * seq_q;
    const int64_t nkv = batch_heads * seq_kv;
    if ((!Q && nq > 0) || ((!K || !V) && nkv > 0) || (!O && nq > 0))
        return fail(FP8_ERR_INVALID_ARG, "null tensor pointer");
    if (!scale_q || !scale_k || !scale_v) return fail(FP8_ERR_INVALID_ARG, "null scale pointer");
    if (!aligned16(Q) || !aligned16(K) || !aligned16(V) || !aligned16(O))
        return fail(FP8_ERR_INVALID_ARG, "Q, K, V and O must be 16-byte aligned");
    if (nq == 0) return ok();
    fp8k::AttnProblem g{Q, K, V, scale_q, scale_k, scale_v, O, batch_heads, seq_q, seq_kv, head_dim,
                        softmax_scale, causal, out_kind, fast_qk};
    return from_hip(fp8k::launch_attention(g, (hipStream_t)stream), "fp8_attention");
}

fp8_status fp8_grouped_gemm(const uint8_t* A, const uint8_t* B, const int32_t* offsets, int32_t experts,
                            const float* scale_a, const float* scale_b, void* C, int64_t T, int64_t N, int64_t K,
                            int32_t out_dtype, void* stream) {
    fp8_status st = check_gemm_common(A, B, C, T, N, K, out_dtype, FP8_ACC_FAST | FP8_A_E5M2 | FP8_B_E5M2);
    if (st != FP8_OK) return st;
    if (!scale_a || !scale_b || !offsets) return fail(FP8_ERR_INVALID_ARG, "null scale or offsets pointer");
    if (experts < 1 || experts > 1024) return fail(FP8_ERR_INVALID_ARG, "experts=%d outside [1, 1024]", experts);
    if (K % 16 || N % 16)
        return fail(FP8_ERR_UNSUPPORTED_SHAPE, "K=%lld and N=%lld must be multiples of 16", (long long)K, (long long)N);
    if (T == 0 || N == 0) return ok();
    fp8k::GemmProblem g{A, B, C, scale_a, scale_b, offsets, experts, T, N, K, 0, 0, 0, 0};
    decode_out(out_dtype, g);
    return from_hip(fp8k::launch_gemm(g, (hipStream_t)stream), "fp8_grouped_gemm");
}

}  // extern "C"
