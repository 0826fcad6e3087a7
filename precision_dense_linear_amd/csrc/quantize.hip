// Input side of the scaled FP8 GEMM: amax reduction and E4M3 quantization.
//
// Per-tensor scaling keeps values inside the E4M3 range +-448 ("Triton FP8
// GEMM via CUTLASS naming", risk paragraph and the scale_max 448 item of its
// parameter list); 32x32 block scales follow the parameter paragraph of "FP8
// GEMM in JAX with Triton for Blackwell".  In every mode:
//     scale = amax / 448 (IEEE binary32 division, 1 for amax == 0)
//     code  = E4M3_RNE(clamp(fl32(x / scale), -448, 448))
// All kernels are HBM-bound streams: 16-byte loads, 16-byte code stores.
#include "device_utils.h"
#include "launch.h"

namespace fp8k {

namespace {

constexpr int kThreads = 256;

__global__ void fill_f32(float* p, int n, float v) {
    int i = blockIdx.x * blockDim.x + threadIdx.x;
    if (i < n) p[i] = v;
}

// Block-level max of non-negative values, then one atomicMax on the float's
// bit pattern (order-preserving for non-negative floats).
__device__ __forceinline__ void block_max_to(float m, float* dst) {
    __shared__ float red[kThreads / 64];
    m = wave_max(m);
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    if (lane == 0) red[wave] = m;
    __syncthreads();
    if (threadIdx.x == 0) {
        float r = red[0];
#pragma unroll
        for (int w = 1; w < kThreads / 64; ++w) r = fmaxf(r, red[w]);
        atomicMax(reinterpret_cast<unsigned int*>(dst), __float_as_uint(r));
    }
}

// amax over n floats (x 16-byte aligned).  Grid-stride over groups of U
// float4s per thread (U independent 16-byte loads in flight per thread).
constexpr int AMAX_U = 8;
__global__ void __launch_bounds__(kThreads) amax_kernel(const float* __restrict__ x, int64_t n, float* amax) {
    const int64_t n4 = n >> 2;
    const v4f* x4 = reinterpret_cast<const v4f*>(x);
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    const int64_t tid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    float m = 0.0f;
    int64_t i = tid;
    for (; i + (AMAX_U - 1) * stride < n4; i += AMAX_U * stride) {
        v4f v[AMAX_U];
#pragma unroll
        for (int u = 0; u < AMAX_U; ++u) v[u] = x4[i + u * stride];
#pragma unroll
        for (int u = 0; u < AMAX_U; ++u)
            m = fmaxf(m, fmaxf(fmaxf(fabsf(v[u].x), fabsf(v[u].y)), fmaxf(fabsf(v[u].z), fabsf(v[u].w))));
    }
    for (; i < n4; i += stride) {
        const v4f v = x4[i];
        m = fmaxf(m, fmaxf(fmaxf(fabsf(v.x), fabsf(v.y)), fmaxf(fabsf(v.z), fabsf(v.w))));
    }
    for (int64_t j = (n4 << 2) + tid; j < n; j += stride) m = fmaxf(m, fabsf(x[j]));
    block_max_to(m, amax);
}

// Codes for n floats with the scale derived from *amax.  Each thread takes
// QUANT_U groups of 16 consecutive elements per iteration (4 x QUANT_U
// independent 16-byte loads in flight), one 16-byte code store per group.
constexpr int QUANT_U = 2;
__device__ __forceinline__ uint4 quant16(const v4f* src, float s) {
    v4f v[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) v[j] = __builtin_nontemporal_load(&src[j]);
    uint4 o;
    o.x = e4m3x4_sat(__fdiv_rn(v[0].x, s), __fdiv_rn(v[0].y, s), __fdiv_rn(v[0].z, s), __fdiv_rn(v[0].w, s));
    o.y = e4m3x4_sat(__fdiv_rn(v[1].x, s), __fdiv_rn(v[1].y, s), __fdiv_rn(v[1].z, s), __fdiv_rn(v[1].w, s));
    o.z = e4m3x4_sat(__fdiv_rn(v[2].x, s), __fdiv_rn(v[2].y, s), __fdiv_rn(v[2].z, s), __fdiv_rn(v[2].w, s));
    o.w = e4m3x4_sat(__fdiv_rn(v[3].x, s), __fdiv_rn(v[3].y, s), __fdiv_rn(v[3].z, s), __fdiv_rn(v[3].w, s));
    return o;
}

__global__ void __launch_bounds__(kThreads) quantize_kernel(const float* __restrict__ x, int64_t n,
                                                            const float* __restrict__ amax, uint8_t* __restrict__ q,
                                                            float* scale_out) {
    const float s = scale_from_amax(*amax);
    if (blockIdx.x == 0 && threadIdx.x == 0) *scale_out = s;
    const int64_t n16 = n >> 4;
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    const int64_t tid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    const v4f* x4 = reinterpret_cast<const v4f*>(x);
    uint4* q16 = reinterpret_cast<uint4*>(q);
    int64_t i = tid;
    for (; i + (QUANT_U - 1) * stride < n16; i += QUANT_U * stride) {
        uint4 o[QUANT_U];
#pragma unroll
        for (int u = 0; u < QUANT_U; ++u) o[u] = quant16(x4 + 4 * (i + u * stride), s);
#pragma unroll
        for (int u = 0; u < QUANT_U; ++u) q16[i + u * stride] = o[u];
    }
    for (; i < n16; i += stride) q16[i] = quant16(x4 + 4 * i, s);
    for (int64_t j = (n16 << 4) + tid; j < n; j += stride) q[j] = e4m3_sat(__fdiv_rn(x[j], s));
}

// 32x32 tiles: one wave per tile.  Lane l covers row l/2 of the tile, columns
// 16*(l%2) .. +15: amax over the tile by a wave reduction, then the codes.
__global__ void __launch_bounds__(kThreads) quantize_blocked_kernel(const float* __restrict__ x, int64_t rows,
                                                                    int64_t cols, uint8_t* __restrict__ q,
                                                                    float* __restrict__ tile_scales) {
    const int64_t tiles_c = cols >> 5;
    const int64_t ntiles = (rows >> 5) * tiles_c;
    const int lane = threadIdx.x & 63;
    const int64_t tile = (int64_t)blockIdx.x * (kThreads / 64) + (threadIdx.x >> 6);
    if (tile >= ntiles) return;
    const int64_t ti = tile / tiles_c, tj = tile % tiles_c;
    const int64_t r = ti * 32 + (lane >> 1);
    const int64_t c = tj * 32 + (lane & 1) * 16;
    const v4f* src = reinterpret_cast<const v4f*>(x + r * cols + c);
    v4f v[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) v[j] = __builtin_nontemporal_load(&src[j]);
    float m = 0.0f;
#pragma unroll
    for (int j = 0; j < 4; ++j) m = fmaxf(m, fmaxf(fmaxf(fabsf(v[j].x), fabsf(v[j].y)), fmaxf(fabsf(v[j].z), fabsf(v[j].w))));
    m = wave_max(m);
    const float s = scale_from_amax(m);
    if (lane == 0) tile_scales[tile] = s;
    uint4 o;
    o.x = e4m3x4_sat(__fdiv_rn(v[0].x, s), __fdiv_rn(v[0].y, s), __fdiv_rn(v[0].z, s), __fdiv_rn(v[0].w, s));
    o.y = e4m3x4_sat(__fdiv_rn(v[1].x, s), __fdiv_rn(v[1].y, s), __fdiv_rn(v[1].z, s), __fdiv_rn(v[1].w, s));
    o.z = e4m3x4_sat(__fdiv_rn(v[2].x, s), __fdiv_rn(v[2].y, s), __fdiv_rn(v[2].z, s), __fdiv_rn(v[2].w, s));
    o.w = e4m3x4_sat(__fdiv_rn(v[3].x, s), __fdiv_rn(v[3].y, s), __fdiv_rn(v[3].z, s), __fdiv_rn(v[3].w, s));
    *reinterpret_cast<uint4*>(q + r * cols + c) = o;
}

// Group of row r by binary search over the (already clamped) boundaries held
// in LDS; returns -1 for rows outside every group.
__device__ __forceinline__ int find_group(const int64_t* bnd, int groups, int64_t r) {
    if (r < bnd[0] || r >= bnd[groups]) return -1;
    int lo = 0, hi = groups;  // bnd[lo] <= r < bnd[hi]
    while (hi - lo > 1) {
        int mid = (lo + hi) >> 1;
        if (bnd[mid] <= r) lo = mid; else hi = mid;
    }
    return lo;
}

__device__ __forceinline__ void load_bounds(const int32_t* off, int groups, int64_t rows, int64_t* bnd) {
    // Clamp sequentially in thread 0 (groups <= 1024: negligible).
    if (threadIdx.x == 0) {
        int64_t lo = 0;
        for (int g = 0; g <= groups; ++g) {
            int64_t v = off[g];
            v = v < lo ? lo : (v > rows ? rows : v);
            bnd[g] = v;
            lo = v;
        }
    }
    __syncthreads();
}

// Grouped kernels: workgroup b owns the contiguous rows [b*rpb, (b+1)*rpb)
// (rpb = rows per block), its waves take them in turn, and a row is streamed
// with GQ_U independent 16-byte loads in flight per lane (cols % 4 == 0).
constexpr int GQ_U = 8;

__device__ __forceinline__ float row_absmax(const v4f* src, int64_t c4, int lane) {
    float m = 0.0f;
    for (int64_t j0 = lane; j0 < c4; j0 += 64 * GQ_U) {
        v4f v[GQ_U];
#pragma unroll
        for (int u = 0; u < GQ_U; ++u) {
            const int64_t j = j0 + u * 64;
            v[u] = j < c4 ? __builtin_nontemporal_load(&src[j]) : (v4f){0.0f, 0.0f, 0.0f, 0.0f};
        }
#pragma unroll
        for (int u = 0; u < GQ_U; ++u)
            m = fmaxf(m, fmaxf(fmaxf(fabsf(v[u].x), fabsf(v[u].y)), fmaxf(fabsf(v[u].z), fabsf(v[u].w))));
    }
    return m;
}

// Grouped amax: the row maxima of a workgroup meet in a per-group LDS max,
// and the workgroup then folds each group it touched into the global amax
// with one atomicMax (on the bit pattern, order-preserving for non-negative
// floats).
__global__ void __launch_bounds__(kThreads) amax_grouped_kernel(const float* __restrict__ x, int64_t rows, int64_t cols,
                                                                const int32_t* __restrict__ off, int groups, int64_t rpb,
                                                                float* amax) {
    __shared__ int64_t bnd[1025];
    __shared__ unsigned int gmax[1024];
    for (int g = threadIdx.x; g < groups; g += blockDim.x) gmax[g] = 0u;
    load_bounds(off, groups, rows, bnd);  // ends with a barrier
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int64_t r0 = (int64_t)blockIdx.x * rpb;
    const int64_t r1 = min(r0 + rpb, rows);
    const int64_t c4 = cols >> 2;
    for (int64_t r = r0 + wave; r < r1; r += kThreads / 64) {
        const int g = find_group(bnd, groups, r);
        if (g < 0) continue;
        const float m = wave_max(row_absmax(reinterpret_cast<const v4f*>(x + r * cols), c4, lane));
        if (lane == 0) atomicMax(&gmax[g], __float_as_uint(m));
    }
    __syncthreads();
    // only the groups this workgroup's rows belong to can be non-zero (a zero
    // needs no atomic: amax starts at zero)
    for (int g = threadIdx.x; g < groups; g += blockDim.x)
        if (gmax[g] != 0u) atomicMax(reinterpret_cast<unsigned int*>(amax + g), gmax[g]);
}

// Grouped quantize: same row partition; each row uses its group's scale.
// Block 0 also writes the scales.
__global__ void __launch_bounds__(kThreads) quantize_grouped_kernel(const float* __restrict__ x, int64_t rows,
                                                                    int64_t cols, const int32_t* __restrict__ off,
                                                                    int groups, int64_t rpb,
                                                                    const float* __restrict__ amax,
                                                                    uint8_t* __restrict__ q, float* scales) {
    __shared__ int64_t bnd[1025];
    load_bounds(off, groups, rows, bnd);
    if (blockIdx.x == 0)
        for (int g = threadIdx.x; g < groups; g += blockDim.x) scales[g] = scale_from_amax(amax[g]);
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int64_t r0 = (int64_t)blockIdx.x * rpb;
    const int64_t r1 = min(r0 + rpb, rows);
    const int64_t c4 = cols >> 2;
    for (int64_t r = r0 + wave; r < r1; r += kThreads / 64) {
        const int g = find_group(bnd, groups, r);
        if (g < 0) continue;
        const float s = scale_from_amax(amax[g]);
        const v4f* src = reinterpret_cast<const v4f*>(x + r * cols);
        uint32_t* dst = reinterpret_cast<uint32_t*>(q + r * cols);
        for (int64_t j0 = lane; j0 < c4; j0 += 64 * GQ_U) {
            v4f v[GQ_U];
#pragma unroll
            for (int u = 0; u < GQ_U; ++u) {
                const int64_t j = j0 + u * 64;
                v[u] = j < c4 ? __builtin_nontemporal_load(&src[j]) : (v4f){0.0f, 0.0f, 0.0f, 0.0f};
            }
#pragma unroll
            for (int u = 0; u < GQ_U; ++u) {
                const int64_t j = j0 + u * 64;
                if (j < c4)
                    dst[j] = e4m3x4_sat(__fdiv_rn(v[u].x, s), __fdiv_rn(v[u].y, s), __fdiv_rn(v[u].z, s),
                                        __fdiv_rn(v[u].w, s));
            }
        }
    }
}

int stream_blocks(int64_t work_items, int per_block) {
    int64_t b = (work_items + per_block - 1) / per_block;
    if (b < 1) b = 1;
    if (b > 256 * 16) b = 256 * 16;  // 16 blocks per CU on 256 CUs; grid-stride beyond
    return (int)b;
}

}  // namespace

hipError_t launch_quantize_pertensor(const float* x, int64_t n, uint8_t* q, float* scale, float* amax, hipStream_t s) {
    hipLaunchKernelGGL(fill_f32, dim3(1), dim3(64), 0, s, amax, 1, 0.0f);
    if (n > 0)
        hipLaunchKernelGGL(amax_kernel, dim3(stream_blocks(n / (4 * AMAX_U) + 1, kThreads)), dim3(kThreads), 0, s, x, n,
                           amax);
    hipLaunchKernelGGL(quantize_kernel, dim3(stream_blocks(n / (16 * QUANT_U) + 1, kThreads)), dim3(kThreads), 0, s, x,
                       n, (const float*)amax, q, scale);
    return hipGetLastError();
}

hipError_t launch_quantize_blocked(const float* x, int64_t rows, int64_t cols, uint8_t* q, float* tile_scales,
                                   hipStream_t s) {
    const int64_t ntiles = (rows / 32) * (cols / 32);
    if (ntiles == 0) return hipSuccess;
    const int64_t blocks = (ntiles + kThreads / 64 - 1) / (kThreads / 64);
    hipLaunchKernelGGL(quantize_blocked_kernel, dim3((unsigned)blocks), dim3(kThreads), 0, s, x, rows, cols, q,
                       tile_scales);
    return hipGetLastError();
}

hipError_t launch_quantize_grouped(const float* x, int64_t rows, int64_t cols, const int32_t* offsets, int32_t groups,
                                   uint8_t* q, float* scales, float* amax, hipStream_t s) {
    hipLaunchKernelGGL(fill_f32, dim3((groups + 255) / 256), dim3(256), 0, s, amax, groups, 0.0f);
    // contiguous row runs: up to 2048 workgroups, at least one row each
    const int64_t nblk = rows < 1 ? 1 : (rows < 2048 ? rows : 2048);
    const int64_t rpb = rows < 1 ? 1 : (rows + nblk - 1) / nblk;
    const int blocks = (int)((rows + rpb - 1) / rpb > 0 ? (rows + rpb - 1) / rpb : 1);
    if (rows > 0 && cols > 0)
        hipLaunchKernelGGL(amax_grouped_kernel, dim3(blocks), dim3(kThreads), 0, s, x, rows, cols, offsets, groups,
                           rpb, amax);
    hipLaunchKernelGGL(quantize_grouped_kernel, dim3(blocks), dim3(kThreads), 0, s, x, rows, cols, offsets, groups,
                       rpb, (const float*)amax, q, scales);
    return hipGetLastError();
}

}  // namespace fp8k
