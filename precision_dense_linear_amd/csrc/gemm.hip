// Per-tensor scaled FP8 GEMM and its MoE grouped form, for gfx950.
//
//   C[m, n] = (scale_a * scale_b) * sum_k A[m, k] * B[k, n]
//
// E4M3 operands, FP32 accumulation, the scales applied once to the finished
// sum, FP32 or BF16 (RNE) output ("Triton FP8 GEMM via CUTLASS naming": kernel
// section, the paragraph after it and the parameter list).  A is M x K with K
// contiguous and B is K x N with N contiguous, as in the kernel sketch of
// "FP8 GEMM in JAX with Triton for Blackwell"; the grouped form runs the same
// tile loop over expert row ranges with per-expert scales (that page's MoE
// paragraph).
//
// Operand feed per 64-byte K slice (v_mfma_f32_32x32x64_f8f6f4):
//  * A: lane l reads row l%32 of its 32-row block, K bytes 32*(l/32)..+31,
//    as two ds_read_b128 from the swizzled A stage;
//  * B: lane l needs column l%32 with the same 32 K bytes; four
//    ds_read_b64_tr_b8 reads each gather 8 K-consecutive bytes of one column
//    from the N-contiguous B stage (the 16 lanes of a group address 8 K-rows
//    x two 8-byte column halves; lane 8h+c receives column c of half h).
#include "gemm_common.h"
#include "launch.h"

namespace fp8k {

namespace {

template <int BM, int BN, int WM, int WN, int KS, int GROUP_M, bool BF16, bool EXACT>
__global__ void __launch_bounds__(64 * WM * WN * KS) gemm_kernel(GemmArgs p) {
    using C = TileCfg<BM, BN, WM, WN, KS>;
    __shared__ __attribute__((aligned(1024))) uint8_t smem[C::LDS];

    const TileSlice t = resolve_tile<BM, BN, GROUP_M>(p);
    if (!t.valid) return;

    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int ks = wave / (WM * WN);
    const int wm = (wave % (WM * WN)) / WN;
    const int wn = wave % WN;
    const int64_t K = p.K, N = p.N;
    const int nsteps = (int)((K + KS * BK - 1) / (KS * BK));
    lds_u8* lds = (lds_u8*)smem;

    v16f acc[C::TM][C::TN];
#pragma unroll
    for (int i = 0; i < C::TM; ++i)
#pragma unroll
        for (int j = 0; j < C::TN; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;

    const int a_row0 = wm * C::WTM + (lane & 31);
    const int a_c0 = (lane >> 5) * 2;
    const int b_krow0 = (lane >> 5) * 32 + ((lane & 15) >> 1);
    const int b_col0 = wn * C::WTN + 16 * ((lane >> 4) & 1) + 8 * (lane & 1);

    if (nsteps > 0) load_stage<BM, BN, WM, WN, KS>(t, N, K, 0, lds, wave, lane);
    for (int step = 0; step < nsteps; ++step) {
        __builtin_amdgcn_s_waitcnt(0);  // this wave's stage loads have landed in LDS
        __syncthreads();                // ... and every wave's; the other buffer is free
        if (step + 1 < nsteps)
            load_stage<BM, BN, WM, WN, KS>(t, N, K, (int64_t)(step + 1) * (KS * BK), lds + ((step + 1) & 1) * C::STAGE,
                                           wave, lane);

        const lds_u8* As = lds + (step & 1) * C::STAGE + ks * BM * BK;
        const lds_u8* Bs = lds + (step & 1) * C::STAGE + C::A_STAGE + ks * BK * BN;
#pragma unroll
        for (int s = 0; s < 2; ++s) {
            v8i a[C::TM], b[C::TN];
#pragma unroll
            for (int mi = 0; mi < C::TM; ++mi) {
                const int row = a_row0 + mi * 32;
                const int c = s * 4 + a_c0;
                const v4i lo = lds_read16(As + row * BK + swz_a(row, c) * 16);
                const v4i hi = lds_read16(As + row * BK + swz_a(row, c + 1) * 16);
                a[mi] = (v8i){lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
            }
#pragma unroll
            for (int ni = 0; ni < C::TN; ++ni) {
                const int col = b_col0 + ni * 32;
                v2i part[4];
#pragma unroll
                for (int tq = 0; tq < 4; ++tq) {
                    const int kr = s * 64 + b_krow0 + 8 * tq;
                    part[tq] = lds_read_tr8(Bs + kr * BN + swz_b<BN>(kr, col >> 4) * 16 + (col & 15));
                }
                b[ni] = (v8i){part[0][0], part[0][1], part[1][0], part[1][1],
                              part[2][0], part[2][1], part[3][0], part[3][1]};
            }
            if constexpr (EXACT) {
                // four K=16 BF16 MFMAs per 64-byte slice; chunk c of each lane's
                // 32 bytes (K 32*(l/32) + 8c .. +7) feeds the c-th one, for A and B alike
#pragma unroll
                for (int c = 0; c < 4; ++c) {
                    v8bf ab[C::TM], bb[C::TN];
#pragma unroll
                    for (int mi = 0; mi < C::TM; ++mi) ab[mi] = e4m3x8_to_bf16(a[mi][2 * c], a[mi][2 * c + 1]);
#pragma unroll
                    for (int ni = 0; ni < C::TN; ++ni) bb[ni] = e4m3x8_to_bf16(b[ni][2 * c], b[ni][2 * c + 1]);
#pragma unroll
                    for (int mi = 0; mi < C::TM; ++mi)
#pragma unroll
                        for (int ni = 0; ni < C::TN; ++ni) acc[mi][ni] = mfma_32x32x16_bf16(ab[mi], bb[ni], acc[mi][ni]);
                }
            } else {
#pragma unroll
                for (int mi = 0; mi < C::TM; ++mi)
#pragma unroll
                    for (int ni = 0; ni < C::TN; ++ni) acc[mi][ni] = mfma_32x32x64_e4m3(a[mi], b[ni], acc[mi][ni]);
            }
        }
    }

    // Split-K: wave groups 1..KS-1 hand their partial sums to group 0 via LDS.
    if constexpr (KS > 1) {
        __syncthreads();
        float* red = (float*)smem;
        const int wslot = wm * WN + wn;
        constexpr int PER = C::TM * C::TN * 16 * 64;
        if (ks > 0) {
            float* dst = red + ((ks - 1) * WM * WN + wslot) * PER;
#pragma unroll
            for (int mi = 0; mi < C::TM; ++mi)
#pragma unroll
                for (int ni = 0; ni < C::TN; ++ni)
#pragma unroll
                    for (int r = 0; r < 16; ++r) dst[((mi * C::TN + ni) * 16 + r) * 64 + lane] = acc[mi][ni][r];
        }
        __syncthreads();
        if (ks > 0) return;
#pragma unroll
        for (int g = 0; g < KS - 1; ++g) {
            const float* src = red + (g * WM * WN + wslot) * PER;
#pragma unroll
            for (int mi = 0; mi < C::TM; ++mi)
#pragma unroll
                for (int ni = 0; ni < C::TN; ++ni)
#pragma unroll
                    for (int r = 0; r < 16; ++r) acc[mi][ni][r] += src[((mi * C::TN + ni) * 16 + r) * 64 + lane];
        }
    }

    // Epilogue: the per-tensor (or per-expert) scale applied once to the sum.
    const float scale = p.scale_a[t.expert] * p.scale_b[t.expert];
#pragma unroll
    for (int mi = 0; mi < C::TM; ++mi)
#pragma unroll
        for (int ni = 0; ni < C::TN; ++ni)
            store_block<BF16>(p.C, acc[mi][ni], scale, t.m0 + wm * C::WTM + mi * 32, t.n0 + wn * C::WTN + ni * 32,
                              t.M, N, t.c_row0, lane);
}

template <int BM, int BN, int WM, int WN, int KS, int GROUP_M>
hipError_t launch_cfg(const GemmProblem& g, hipStream_t s) {
    GemmArgs a;
    a.A = g.A;
    a.B = g.B;
    a.C = g.C;
    a.scale_a = g.scale_a;
    a.scale_b = g.scale_b;
    a.offsets = g.offsets;
    a.experts = g.experts;
    a.M = g.M;
    a.N = g.N;
    a.K = g.K;
    a.tiles_n = (int32_t)((g.N + BN - 1) / BN);
    // grouped: an upper bound of sum_e ceil(rows_e / BM); surplus workgroups exit at once
    a.tiles_m = g.experts == 0 ? (int32_t)((g.M + BM - 1) / BM)
                               : (int32_t)((g.M + (int64_t)g.experts * (BM - 1)) / BM);
    const int64_t blocks = (int64_t)a.tiles_m * a.tiles_n;
    if (blocks == 0) return hipSuccess;
    constexpr int NT = 64 * WM * WN * KS;
    const dim3 grid((unsigned)blocks), block(NT);
    if (g.fast_acc) {
        if (g.out_bf16) hipLaunchKernelGGL((gemm_kernel<BM, BN, WM, WN, KS, GROUP_M, true, false>), grid, block, 0, s, a);
        else hipLaunchKernelGGL((gemm_kernel<BM, BN, WM, WN, KS, GROUP_M, false, false>), grid, block, 0, s, a);
    } else {
        if (g.out_bf16) hipLaunchKernelGGL((gemm_kernel<BM, BN, WM, WN, KS, GROUP_M, true, true>), grid, block, 0, s, a);
        else hipLaunchKernelGGL((gemm_kernel<BM, BN, WM, WN, KS, GROUP_M, false, true>), grid, block, 0, s, a);
    }
    return hipGetLastError();
}

}  // namespace

// Tile configuration by shape class (a static table, no runtime tuning):
//  * M (rows per expert when grouped) <= 64: 32 x 64 tiles with each K step
//    split over two wave groups -- many workgroups to stream B, HBM bound;
//  * M <= 1024: 128 x 128 tiles, 4 waves of 64 x 64;
//  * larger M: 256 x 256 tiles, 4 waves of 128 x 128 -- MFMA bound.
hipError_t launch_gemm(const GemmProblem& g, hipStream_t s) {
    const int64_t rows_per_problem = g.experts ? (g.M + g.experts - 1) / g.experts : g.M;
    if (rows_per_problem <= 64) return launch_cfg<32, 64, 1, 2, 2, 8>(g, s);
    if (rows_per_problem <= 1024) return launch_cfg<128, 128, 2, 2, 1, 8>(g, s);
    return launch_cfg<256, 256, 2, 2, 1, 8>(g, s);
}

}  // namespace fp8k
