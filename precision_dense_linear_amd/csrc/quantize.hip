// Input side of the scaled FP8 GEMM: amax reduction and E4M3 / E5M2
// quantization.
//
// Per-tensor scaling keeps values inside the E4M3 range +-448 ("Triton FP8
// GEMM via CUTLASS naming", risk paragraph and the scale_max 448 item of its
// parameter list); 32x32 block scales follow the parameter paragraph of "FP8
// GEMM in JAX with Triton for Blackwell", whose opening section also names
// the E5M2 format.  In every mode, with FMAX = 448 (E4M3) or 57344 (E5M2,
// per-tensor and row-group quantization only; block scales of 32x32 or 64x64
// tiles, the latter the coarser granularity of that page's monitoring
// paragraph, are E4M3):
//     scale = amax / FMAX (IEEE binary32 division, 1 for amax == 0)
//     code  = RNE(clamp(fl32(x / scale), -FMAX, FMAX))
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
template <int NT = kThreads>
__device__ __forceinline__ void block_max_to(float m, float* dst) {
    __shared__ float red[NT / 64];
    m = wave_max(m);
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    if (lane == 0) red[wave] = m;
    __syncthreads();
    if (threadIdx.x == 0) {
        float r = red[0];
#pragma unroll
        for (int w = 1; w < NT / 64; ++w) r = fmaxf(r, red[w]);
        atomicMax(reinterpret_cast<unsigned int*>(dst), __float_as_uint(r));
    }
}

// Per-tensor kernels over n floats (x 16-byte aligned).  The n/4 full
// float4s form chunks of CHUNK4 = 64 * PT_U; workgroup b owns the contiguous
// chunks [b*cpb, (b+1)*cpb), its waves take them in turn, and a wave streams a
// chunk with PT_U independent, fully coalesced 16-byte loads per lane in
// flight.  Workgroup 0 also takes the n % 4 trailing floats.
constexpr int PT_U = 8;
constexpr int64_t CHUNK4 = 64 * PT_U;

// amax runs 16-wave workgroups over 4x the chunks of a quantize workgroup:
// the same waves in flight, a quarter of the atomics on the one amax word
// (2048 of them, all landing within a few microseconds on a 64 MB tensor,
// serialise to ~13 us).
constexpr int kAmaxThreads = 1024;
__global__ void __launch_bounds__(kAmaxThreads) amax_kernel(const float* __restrict__ x, int64_t n, int64_t cpb,
                                                        float* amax) {
    const int64_t n4 = n >> 2;
    const v4f* x4 = reinterpret_cast<const v4f*>(x);
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int64_t c0 = (int64_t)blockIdx.x * cpb;
    const int64_t c1 = min(c0 + cpb, (n4 + CHUNK4 - 1) / CHUNK4);
    float m = 0.0f;
    for (int64_t c = c0 + wave; c < c1; c += kAmaxThreads / 64) {
        v4f v[PT_U];
#pragma unroll
        for (int u = 0; u < PT_U; ++u) {
            const int64_t j = c * CHUNK4 + u * 64 + lane;
            v[u] = j < n4 ? x4[j] : (v4f){0.0f, 0.0f, 0.0f, 0.0f};
        }
#pragma unroll
        for (int u = 0; u < PT_U; ++u)
            m = fmaxf(m, fmaxf(fmaxf(fabsf(v[u].x), fabsf(v[u].y)), fmaxf(fabsf(v[u].z), fabsf(v[u].w))));
    }
    if (blockIdx.x == 0)
        for (int64_t j = (n4 << 2) + threadIdx.x; j < n; j += blockDim.x) m = fmaxf(m, fabsf(x[j]));
    block_max_to<kAmaxThreads>(m, amax);
}

// Codes for n floats with the scale derived from *amax: the chunk partition
// of amax_kernel, four codes (one 32-bit store) per float4.  amax_kernel
// reads with ordinary (cache-allocating) loads and this pass walks each
// workgroup's chunks backwards, so it starts on the lines the first pass
// touched last, the likeliest to still be in the last-level cache.
template <int F>
__global__ void __launch_bounds__(kThreads) quantize_kernel(const float* __restrict__ x, int64_t n, int64_t cpb,
                                                            const float* __restrict__ amax, uint8_t* __restrict__ q,
                                                            float* scale_out) {
    const float s = scale_from_amax_fmt<F>(*amax);
    if (blockIdx.x == 0 && threadIdx.x == 0) *scale_out = s;
    const int64_t n4 = n >> 2;
    const v4f* x4 = reinterpret_cast<const v4f*>(x);
    uint32_t* q4 = reinterpret_cast<uint32_t*>(q);
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int64_t c0 = (int64_t)blockIdx.x * cpb;
    const int64_t c1 = min(c0 + cpb, (n4 + CHUNK4 - 1) / CHUNK4);
    for (int64_t c = c1 - 1 - wave; c >= c0; c -= kThreads / 64) {
        v4f v[PT_U];
#pragma unroll
        for (int u = 0; u < PT_U; ++u) {
            const int64_t j = c * CHUNK4 + u * 64 + lane;
            v[u] = j < n4 ? __builtin_nontemporal_load(&x4[j]) : (v4f){0.0f, 0.0f, 0.0f, 0.0f};
        }
#pragma unroll
        for (int u = 0; u < PT_U; ++u) {
            const int64_t j = c * CHUNK4 + u * 64 + lane;
            if (j < n4)
                q4[j] = fp8x4_sat<F>(__fdiv_rn(v[u].x, s), __fdiv_rn(v[u].y, s), __fdiv_rn(v[u].z, s),
                                     __fdiv_rn(v[u].w, s));
        }
    }
    if (blockIdx.x == 0)
        for (int64_t j = (n4 << 2) + threadIdx.x; j < n; j += blockDim.x) q[j] = fp8_sat<F>(__fdiv_rn(x[j], s));
}

// T x T tiles (T = 32 or 64): one wave per tile.  A row of the tile is T/4
// lanes of four floats (LPR lanes); load j of lane l covers tile row
// (64/LPR) j + l/LPR, columns 4(l%LPR) .. +3, so each load instruction reads
// whole 4T-byte row segments.  amax over the tile by a wave reduction, then
// the codes (a T-byte run per row and instruction).  E8: the tile's scale is
// the power of two 2^e, e = floor(log2(amax)) - 8 clamped to [-127, 127]
// (0 for an all-zero tile), stored as the byte e + 127 (E8M0) -- the OCP
// microscaling conversion for E4M3 elements.
template <int T, bool E8>
__global__ void __launch_bounds__(kThreads) quantize_blocked_kernel(const float* __restrict__ x, int64_t rows,
                                                                    int64_t cols, uint8_t* __restrict__ q,
                                                                    void* __restrict__ tile_scales, int kmajor) {
    constexpr int LPR = T / 4;        // lanes per tile row
    constexpr int RPI = 64 / LPR;     // tile rows per load instruction
    constexpr int NL = T / RPI;       // loads per lane
    const int64_t tiles_c = cols / T;
    const int64_t ntiles = (rows / T) * tiles_c;
    const int lane = threadIdx.x & 63;
    const int64_t tile = (int64_t)blockIdx.x * (kThreads / 64) + (threadIdx.x >> 6);
    if (tile >= ntiles) return;
    const int64_t ti = tile / tiles_c, tj = tile % tiles_c;
    const int64_t r = ti * T + lane / LPR;
    const int64_t c = tj * T + (lane % LPR) * 4;
    v4f v[NL];
#pragma unroll
    for (int j = 0; j < NL; ++j)
        v[j] = __builtin_nontemporal_load(reinterpret_cast<const v4f*>(x + (r + RPI * j) * cols + c));
    float m = 0.0f;
#pragma unroll
    for (int j = 0; j < NL; ++j) m = fmaxf(m, fmaxf(fmaxf(fabsf(v[j].x), fabsf(v[j].y)), fmaxf(fabsf(v[j].z), fabsf(v[j].w))));
    m = wave_max(m);
    float s;
    if constexpr (E8) {
        int e = m == 0.0f ? 0 : __builtin_amdgcn_frexp_expf(m) - 1 - 8;  // m = f * 2^ex, f in [0.5, 1)
        e = e < -127 ? -127 : (e > 127 ? 127 : e);
        s = __builtin_amdgcn_ldexpf(1.0f, e);
        // [rows/32][pitch(cols/32)], or [cols/32][pitch(rows/32)] (kmajor),
        // pitch(n) = n rounded up to a multiple of 4; the last tile of each
        // row also writes that row's padding bytes (127)
        uint8_t* ex = reinterpret_cast<uint8_t*>(tile_scales);
        const int64_t inner = kmajor ? rows / T : tiles_c;
        const int64_t pitch = (inner + 3) & ~int64_t(3);
        const int64_t outer_i = kmajor ? tj : ti, inner_i = kmajor ? ti : tj;
        if (lane == 0) ex[outer_i * pitch + inner_i] = (uint8_t)(e + 127);
        if (inner_i == inner - 1 && lane >= 1 && lane < 1 + pitch - inner) ex[outer_i * pitch + inner + lane - 1] = 127;
    } else {
        s = scale_from_amax(m);
        if (lane == 0) reinterpret_cast<float*>(tile_scales)[tile] = s;
    }
#pragma unroll
    for (int j = 0; j < NL; ++j)
        *reinterpret_cast<uint32_t*>(q + (r + RPI * j) * cols + c) =
            e4m3x4_sat(__fdiv_rn(v[j].x, s), __fdiv_rn(v[j].y, s), __fdiv_rn(v[j].z, s), __fdiv_rn(v[j].w, s));
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
template <int F>
__global__ void __launch_bounds__(kThreads) quantize_grouped_kernel(const float* __restrict__ x, int64_t rows,
                                                                    int64_t cols, const int32_t* __restrict__ off,
                                                                    int groups, int64_t rpb,
                                                                    const float* __restrict__ amax,
                                                                    uint8_t* __restrict__ q, float* scales) {
    __shared__ int64_t bnd[1025];
    load_bounds(off, groups, rows, bnd);
    if (blockIdx.x == 0)
        for (int g = threadIdx.x; g < groups; g += blockDim.x) scales[g] = scale_from_amax_fmt<F>(amax[g]);
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int64_t r0 = (int64_t)blockIdx.x * rpb;
    const int64_t r1 = min(r0 + rpb, rows);
    const int64_t c4 = cols >> 2;
    for (int64_t r = r0 + wave; r < r1; r += kThreads / 64) {
        const int g = find_group(bnd, groups, r);
        if (g < 0) continue;
        const float s = scale_from_amax_fmt<F>(amax[g]);
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
                    dst[j] = fp8x4_sat<F>(__fdiv_rn(v[u].x, s), __fdiv_rn(v[u].y, s), __fdiv_rn(v[u].z, s),
                                          __fdiv_rn(v[u].w, s));
            }
        }
    }
}

// 2:4 pruning, per-tensor E4M3 quantization and compression of a K x N
// weight matrix (K % 32 == 0), the scale taken from *amax (the largest |w|
// always survives the pruning).  One wave per 64 columns and one 32-deep K
// block; lane = column, so each load and store instruction touches one
// 64-column run of a row.  Per group of 4 along K: keep the two largest |w|
// (the first maximum on ties), quantize them (the other two become code
// 0x00), then store the group's two entries that are nonzero codes (a kept
// value may round to zero), completed by its lowest-k zero entries, in
// ascending k, with their 2-bit positions.
__global__ void __launch_bounds__(kThreads) quantize_2of4_kernel(const float* __restrict__ w, int64_t K, int64_t N,
                                                                 const float* __restrict__ amax,
                                                                 uint8_t* __restrict__ vals, uint32_t* __restrict__ idx,
                                                                 float* scale_out) {
    const float s = scale_from_amax(*amax);
    if (blockIdx.x == 0 && threadIdx.x == 0) *scale_out = s;
    const int lane = threadIdx.x & 63;
    const int64_t wv = (int64_t)blockIdx.x * (kThreads / 64) + (threadIdx.x >> 6);
    const int64_t colblocks = (N + 63) / 64;
    const int64_t kb = wv / colblocks, n = (wv % colblocks) * 64 + lane;
    if (kb >= K / 32 || n >= N) return;
    uint32_t word = 0;
#pragma unroll
    for (int gg = 0; gg < 8; ++gg) {
        float v[4];
#pragma unroll
        for (int q = 0; q < 4; ++q) v[q] = w[(kb * 32 + gg * 4 + q) * N + n];
        int best = 0;
#pragma unroll
        for (int q = 1; q < 4; ++q) if (fabsf(v[q]) > fabsf(v[best])) best = q;
        int second = best == 0 ? 1 : 0;
#pragma unroll
        for (int q = 0; q < 4; ++q) if (q != best && fabsf(v[q]) > fabsf(v[second])) second = q;
        uint8_t c[4];
#pragma unroll
        for (int q = 0; q < 4; ++q) c[q] = (q == best || q == second) ? e4m3_sat(__fdiv_rn(v[q], s)) : (uint8_t)0;
        int pos[2] = {0, 0}, np = 0;
#pragma unroll
        for (int q = 0; q < 4; ++q)
            if (np < 2 && (c[q] & 0x7F) != 0) pos[np++] = q;
#pragma unroll
        for (int q = 0; q < 4; ++q)
            if (np < 2 && (c[q] & 0x7F) == 0 && !(np == 1 && pos[0] == q)) pos[np++] = q;
        if (pos[0] > pos[1]) { const int t = pos[0]; pos[0] = pos[1]; pos[1] = t; }
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            vals[(kb * 16 + gg * 2 + j) * N + n] = c[pos[j]];
            word |= (uint32_t)pos[j] << (2 * (2 * gg + j));
        }
    }
    idx[kb * N + n] = word;
}

}  // namespace

hipError_t launch_quantize_2of4(const float* w, int64_t K, int64_t N, uint8_t* vals, uint32_t* idx, float* scale,
                                float* amax, hipStream_t s) {
    hipLaunchKernelGGL(fill_f32, dim3(1), dim3(64), 0, s, amax, 1, 0.0f);
    const int64_t n = K * N;
    const int64_t nchunks = ((n >> 2) + CHUNK4 - 1) / CHUNK4;
    const int64_t cpb = nchunks < 2048 ? 1 : (nchunks + 2047) / 2048;
    const int64_t blocks = nchunks < 1 ? 1 : (nchunks + cpb - 1) / cpb;
    const int64_t acpb = cpb * (kAmaxThreads / kThreads), ablocks = nchunks < 1 ? 1 : (nchunks + acpb - 1) / acpb;
    if (n > 0) hipLaunchKernelGGL(amax_kernel, dim3((unsigned)ablocks), dim3(kAmaxThreads), 0, s, w, n, acpb, amax);
    const int64_t waves = (K / 32) * ((N + 63) / 64);
    const int64_t qblocks = waves < 1 ? 1 : (waves + kThreads / 64 - 1) / (kThreads / 64);
    hipLaunchKernelGGL(quantize_2of4_kernel, dim3((unsigned)qblocks), dim3(kThreads), 0, s, w, K, N,
                       (const float*)amax, vals, idx, scale);
    return hipGetLastError();
}

hipError_t launch_quantize_pertensor(const float* x, int64_t n, uint8_t* q, float* scale, float* amax, int fmt,
                                     hipStream_t s) {
    hipLaunchKernelGGL(fill_f32, dim3(1), dim3(64), 0, s, amax, 1, 0.0f);
    // up to 2048 workgroups of contiguous chunks (at least one workgroup)
    const int64_t nchunks = ((n >> 2) + CHUNK4 - 1) / CHUNK4;
    const int64_t cpb = nchunks < 2048 ? 1 : (nchunks + 2047) / 2048;
    const int64_t blocks = nchunks < 1 ? 1 : (nchunks + cpb - 1) / cpb;
    const int64_t acpb = cpb * (kAmaxThreads / kThreads), ablocks = nchunks < 1 ? 1 : (nchunks + acpb - 1) / acpb;
    if (n > 0)
        hipLaunchKernelGGL(amax_kernel, dim3((unsigned)ablocks), dim3(kAmaxThreads), 0, s, x, n, acpb, amax);
    if (fmt == 0)
        hipLaunchKernelGGL(quantize_kernel<0>, dim3((unsigned)blocks), dim3(kThreads), 0, s, x, n, cpb,
                           (const float*)amax, q, scale);
    else
        hipLaunchKernelGGL(quantize_kernel<1>, dim3((unsigned)blocks), dim3(kThreads), 0, s, x, n, cpb,
                           (const float*)amax, q, scale);
    return hipGetLastError();
}

hipError_t launch_quantize_blocked(const float* x, int64_t rows, int64_t cols, int T, uint8_t* q, float* tile_scales,
                                   hipStream_t s) {
    const int64_t ntiles = (rows / T) * (cols / T);
    if (ntiles == 0) return hipSuccess;
    const int64_t blocks = (ntiles + kThreads / 64 - 1) / (kThreads / 64);
    if (T == 64)
        hipLaunchKernelGGL((quantize_blocked_kernel<64, false>), dim3((unsigned)blocks), dim3(kThreads), 0, s, x, rows,
                           cols, q, (void*)tile_scales, 0);
    else
        hipLaunchKernelGGL((quantize_blocked_kernel<32, false>), dim3((unsigned)blocks), dim3(kThreads), 0, s, x, rows,
                           cols, q, (void*)tile_scales, 0);
    return hipGetLastError();
}

hipError_t launch_quantize_blocked_e8m0(const float* x, int64_t rows, int64_t cols, uint8_t* q, uint8_t* e8,
                                        int kmajor, hipStream_t s) {
    const int64_t ntiles = (rows / 32) * (cols / 32);
    if (ntiles == 0) return hipSuccess;
    const int64_t blocks = (ntiles + kThreads / 64 - 1) / (kThreads / 64);
    hipLaunchKernelGGL((quantize_blocked_kernel<32, true>), dim3((unsigned)blocks), dim3(kThreads), 0, s, x, rows,
                       cols, q, (void*)e8, kmajor);
    return hipGetLastError();
}

hipError_t launch_quantize_grouped(const float* x, int64_t rows, int64_t cols, const int32_t* offsets, int32_t groups,
                                   uint8_t* q, float* scales, float* amax, int fmt, hipStream_t s) {
    hipLaunchKernelGGL(fill_f32, dim3((groups + 255) / 256), dim3(256), 0, s, amax, groups, 0.0f);
    // contiguous row runs: up to 2048 workgroups, at least one row each
    const int64_t nblk = rows < 1 ? 1 : (rows < 2048 ? rows : 2048);
    const int64_t rpb = rows < 1 ? 1 : (rows + nblk - 1) / nblk;
    const int blocks = (int)((rows + rpb - 1) / rpb > 0 ? (rows + rpb - 1) / rpb : 1);
    if (rows > 0 && cols > 0)
        hipLaunchKernelGGL(amax_grouped_kernel, dim3(blocks), dim3(kThreads), 0, s, x, rows, cols, offsets, groups,
                           rpb, amax);
    if (fmt == 0)
        hipLaunchKernelGGL(quantize_grouped_kernel<0>, dim3(blocks), dim3(kThreads), 0, s, x, rows, cols, offsets,
                           groups, rpb, (const float*)amax, q, scales);
    else
        hipLaunchKernelGGL(quantize_grouped_kernel<1>, dim3(blocks), dim3(kThreads), 0, s, x, rows, cols, offsets,
                           groups, rpb, (const float*)amax, q, scales);
    return hipGetLastError();
}

}  // namespace fp8k
