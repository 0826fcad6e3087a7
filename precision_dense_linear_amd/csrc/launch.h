// Host-side launchers behind the C ABI (fp8gemm.h).  Arguments have already
// been validated by the entry points; each launcher only enqueues kernels on
// `s` and returns the first HIP error it sees.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fp8k {

// fmt: 0 = E4M3, 1 = E5M2
hipError_t launch_quantize_pertensor(const float* x, int64_t n, uint8_t* q, float* scale, float* amax, int fmt,
                                     hipStream_t s);
// T x T tiles, T = 32 or 64
hipError_t launch_quantize_blocked(const float* x, int64_t rows, int64_t cols, int T, uint8_t* q, float* tile_scales,
                                   hipStream_t s);
// 32x32 tiles with E8M0 exponents (one byte per tile), stored
// [rows/32][cols/32], or [cols/32][rows/32] when kmajor
hipError_t launch_quantize_blocked_e8m0(const float* x, int64_t rows, int64_t cols, uint8_t* q, uint8_t* e8,
                                        int kmajor, hipStream_t s);
hipError_t launch_quantize_grouped(const float* x, int64_t rows, int64_t cols, const int32_t* offsets, int32_t groups,
                                   uint8_t* q, float* scales, float* amax, int fmt, hipStream_t s);

// Dense GEMM on FP8 codes; `experts` > 0 selects the grouped (MoE) problem,
// where M is the total row count T and B holds `experts` K x N matrices.
struct GemmProblem {
    const uint8_t* A;
    const uint8_t* B;
    void* C;
    const float* scale_a;
    const float* scale_b;
    const int32_t* offsets;  // grouped only
    int32_t experts;         // 0 for the plain GEMM
    int64_t M, N, K;
    int32_t out_bf16;  // 2-byte output (BF16, or FP16 when out_f16)
    int32_t fast_acc;  // 1: native FP8 MFMA accumulation; 0: exact products (BF16 MFMA)
    int32_t out_f16;   // 2-byte output is IEEE binary16
    int32_t fmt;       // operand formats: bit 0 set = A holds E5M2 codes, bit 1 = B (else E4M3)
    const uint8_t* e8_a = nullptr;  // E8M0 tile exponents (block-scaled E8M0 GEMM only)
    const uint8_t* e8_b = nullptr;
    const uint32_t* sp_idx = nullptr;  // 2:4-sparse B (B then holds the compressed values)
    // Split-K workspace (plain GEMM only; none: K is never split across
    // workgroups): ws_tiles split tiles of FP32 partial sums at ws and one
    // arrival counter per split tile at counters, zero between launches.
    float* ws = nullptr;
    uint32_t* counters = nullptr;
    int64_t ws_tiles = 0;
};
hipError_t launch_gemm(const GemmProblem& p, hipStream_t s);

// The four operand-format pairs of launch_gemm, each compiled on its own.
hipError_t launch_gemm_fmt0(const GemmProblem& p, hipStream_t s);
hipError_t launch_gemm_fmt1(const GemmProblem& p, hipStream_t s);
hipError_t launch_gemm_fmt2(const GemmProblem& p, hipStream_t s);
hipError_t launch_gemm_fmt3(const GemmProblem& p, hipStream_t s);

// 32x32 tiles with E8M0 exponents e8_a [K/32][M/32], e8_b [K/32][N/32]
// (M, N, K multiples of 32); out: 0 FP32, 1 BF16, 2 FP16
hipError_t launch_gemm_blockscaled_e8m0(const uint8_t* A, const uint8_t* B, const uint8_t* e8_a, const uint8_t* e8_b,
                                        void* C, int64_t M, int64_t N, int64_t K, int32_t out, hipStream_t s);

// 2:4-sparse B: values [K/2][N], positions idx [K/32][N] (K % 32 == 0)
hipError_t launch_gemm_sparse24(const uint8_t* A, const uint8_t* Bv, const uint32_t* Bi, const float* scale_a,
                                const float* scale_b, void* C, int64_t M, int64_t N, int64_t K, int32_t out,
                                hipStream_t s);
// prune (2 of every 4 along K), quantize per tensor and compress a K x N weight matrix
hipError_t launch_quantize_2of4(const float* w, int64_t K, int64_t N, uint8_t* vals, uint32_t* idx, float* scale,
                                float* amax, hipStream_t s);

// out: 0 FP32, 1 BF16, 2 FP16; block: edge of the scale tiles, 32 or 64
hipError_t launch_gemm_blockscaled(const uint8_t* A, const uint8_t* B, const float* s_a, const float* s_b, void* C,
                                   int64_t M, int64_t N, int64_t K, int32_t out, int32_t block, hipStream_t s);

// Multi-head attention on E4M3 Q, K, V (per-tensor scales): Q [heads][seq_q]
// [head_dim], K and V [heads][seq_kv][head_dim], O [heads][seq_q][head_dim];
// head_dim 64 or 128; out: 0 FP32, 1 BF16, 2 FP16.
struct AttnProblem {
    const uint8_t* Q;
    const uint8_t* K;
    const uint8_t* V;
    const float* scale_q;
    const float* scale_k;
    const float* scale_v;
    void* O;
    int64_t heads, seq_q, seq_kv, head_dim;
    float softmax_scale;
    int32_t causal;
    int32_t out;
    bool fast_qk;   // Q K^T on the FP8 matrix cores (FP8_ACC_FAST)
};
hipError_t launch_attention(const AttnProblem& p, hipStream_t s);

}  // namespace fp8k
