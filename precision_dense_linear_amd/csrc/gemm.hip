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

// Operand fragments of one 64-byte K slice for a wave: TM A blocks, TN B blocks.
template <int TM, int TN>
struct Frags {
    v8i a[TM];
    v8i b[TN];
};

template <int BM, int BN, int WM, int WN, int KS, int NBUF, int GROUP_M, bool BF16, bool EXACT>
__global__ void __launch_bounds__(64 * WM * WN * KS) gemm_kernel(GemmArgs p) {
    using C = PipeCfg<BM, BN, WM, WN, KS, NBUF>;
    constexpr int TM = C::TM, TN = C::TN;
    constexpr int EPI = (KS > 1 ? C::RED : 0) + WM * WN * TileStore<BF16, TM, TN>::LDS_BYTES;
    static_assert(EPI <= 160 * 1024, "epilogue LDS budget");
    __shared__ __attribute__((aligned(1024))) uint8_t smem[C::LDS > EPI ? C::LDS : EPI];

    const TileSlice t = resolve_tile<BM, BN, GROUP_M>(p);
    if (!t.valid) return;

    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int ks = wave / (WM * WN);
    const int wm = (wave % (WM * WN)) / WN;
    const int wn = wave % WN;
    const int64_t K = p.K, N = p.N;
    const int nsteps = (int)((K + KS * BKP - 1) / (KS * BKP));
    lds_u8* lds = (lds_u8*)smem;
    const PipeLoader<BM, BN, WM, WN, KS, NBUF> loader(t, N, K, wave, lane, (uint32_t)(uintptr_t)lds);

    v16f acc[TM][TN];
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;

    // Per-lane LDS byte offsets of this wave's operands inside a stage.
    int a_off[TM];
    int b_off[TN][4];
#pragma unroll
    for (int mi = 0; mi < TM; ++mi) {
        const int row = wm * C::WTM + mi * 32 + (lane & 31);
        a_off[mi] = ks * BM * BKP + row * BKP + swz_a64(row, (lane >> 5) * 2) * 16;
    }
    // the second chunk of the pair: (2h+1) ^ f = (2h ^ f) ^ 1, i.e. +-16 bytes
    const int a_pair = (((lane & 31) >> 2) & 1) ? -16 : 16;
#pragma unroll
    for (int ni = 0; ni < TN; ++ni) {
        const int col = wn * C::WTN + ni * 32 + 16 * ((lane >> 4) & 1) + 8 * (lane & 1);
#pragma unroll
        for (int tq = 0; tq < 4; ++tq) {
            const int kr = (lane >> 5) * 32 + ((lane & 15) >> 1) + 8 * tq;
            b_off[ni][tq] = C::A_STAGE + ks * BKP * BN + kr * BN + swz_b<BN>(kr, col >> 4) * 16 + (col & 15);
        }
    }

    auto read_frags = [&](int st, Frags<TM, TN>& f) {
        const lds_u8* stage = lds + (st % NBUF) * C::STAGE;
#pragma unroll
        for (int mi = 0; mi < TM; ++mi) {
            const v4i lo = lds_read16(stage + a_off[mi]);
            const v4i hi = lds_read16(stage + a_off[mi] + a_pair);
            f.a[mi] = (v8i){lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
        }
#pragma unroll
        for (int ni = 0; ni < TN; ++ni) {
            v2i q[4];
#pragma unroll
            for (int tq = 0; tq < 4; ++tq) q[tq] = lds_read_tr8(stage + b_off[ni][tq]);
            f.b[ni] = (v8i){q[0][0], q[0][1], q[1][0], q[1][1], q[2][0], q[2][1], q[3][0], q[3][1]};
        }
    };

    // All MFMAs of one 64-byte slice.  The B fragment is the first operand, so
    // accumulator block (mi, ni) holds C^T (see TileStore).
    auto mma = [&](const Frags<TM, TN>& f) {
        if constexpr (EXACT) {
            // four K=16 BF16 MFMAs per block; chunk c of each lane's 32 bytes
            // (K 32*(l/32) + 8c .. +7) feeds the c-th, for A and B alike.  The
            // chunk loop is outermost, so consecutive MFMAs update different
            // accumulators and the conversions of chunk c+1 can overlap the
            // MFMAs of chunk c.
#pragma unroll
            for (int c = 0; c < 4; ++c) {
                v8bf ab[TM], bb[TN];
#pragma unroll
                for (int mi = 0; mi < TM; ++mi) ab[mi] = e4m3x8_to_bf16(f.a[mi][2 * c], f.a[mi][2 * c + 1]);
#pragma unroll
                for (int ni = 0; ni < TN; ++ni) bb[ni] = e4m3x8_to_bf16(f.b[ni][2 * c], f.b[ni][2 * c + 1]);
#pragma unroll
                for (int mi = 0; mi < TM; ++mi)
#pragma unroll
                    for (int ni = 0; ni < TN; ++ni) acc[mi][ni] = mfma_32x32x16_bf16(bb[ni], ab[mi], acc[mi][ni]);
            }
        } else {
#pragma unroll
            for (int mi = 0; mi < TM; ++mi)
#pragma unroll
                for (int ni = 0; ni < TN; ++ni) acc[mi][ni] = mfma_32x32x64_e4m3(f.b[ni], f.a[mi], acc[mi][ni]);
        }
    };

    // Pipeline: stage s lives in LDS buffer s % NBUF; D = NBUF-1 stages are in
    // flight.  Iteration s (fragments of slice s already requested):
    //   wait until stage s+1 has landed (the D-2 newer stages may still be in
    //   flight), barrier -- stage s+1 is visible to all waves, and every wave
    //   has finished its MFMAs of slice s-1, hence its reads of buffer
    //   (s-1) % NBUF = (s+D) % NBUF;
    //   issue stage s+D into that buffer;
    //   read the slice s+1 fragments while the slice s MFMAs run.
    // Loads past the end of K are empty (they read zero), so the body is
    // branch-free and the in-flight load count is the same every iteration.
    constexpr int D = NBUF - 1;
    constexpr int MF = TM * TN * (EXACT ? 4 : 1);  // MFMA instructions per slice
    constexpr int RD = 2 * TM + 4 * TN;             // LDS reads per slice
    Frags<TM, TN> f0, f1;
#pragma unroll
    for (int st = 0; st < D; ++st) loader.issue(st);
    wait_vmcnt<(D - 1) * C::LPS>();
    __syncthreads();
    read_frags(0, f0);

    auto iteration = [&](int s, Frags<TM, TN>& cur, Frags<TM, TN>& next) {
        wait_vmcnt<(D - 2) * C::LPS>();
        __syncthreads();
        loader.issue(s + D);
        read_frags(s + 1, next);
        mma(cur);
        // interleave: the next fragment's LDS reads spread over the MFMAs
        constexpr int RPM = (RD + MF - 1) / MF;
#pragma unroll
        for (int i = 0; i < (RD + RPM - 1) / RPM; ++i) {
            __builtin_amdgcn_sched_group_barrier(0x100, RPM, 0);  // DS read
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);    // MFMA
        }
        __builtin_amdgcn_sched_barrier(0);
    };
    int s = 0;
    for (; s + 1 < nsteps; s += 2) {
        iteration(s, f0, f1);
        iteration(s + 1, f1, f0);
    }
    if (s < nsteps) iteration(s, f0, f1);

    // Drain: the empty tail loads must land before the LDS is reused.
    wait_vmcnt<0>();

    // Split-K: wave groups 1..KS-1 hand their partial sums to group 0 via LDS.
    if constexpr (KS > 1) {
        __syncthreads();
        float* red = (float*)smem;
        const int wslot = wm * WN + wn;
        constexpr int PER = TM * TN * 16 * 64;
        if (ks > 0) {
            float* dst = red + ((ks - 1) * WM * WN + wslot) * PER;
#pragma unroll
            for (int mi = 0; mi < TM; ++mi)
#pragma unroll
                for (int ni = 0; ni < TN; ++ni)
#pragma unroll
                    for (int r = 0; r < 16; ++r) dst[((mi * TN + ni) * 16 + r) * 64 + lane] = acc[mi][ni][r];
        }
        __syncthreads();
        if (ks > 0) return;
#pragma unroll
        for (int g = 0; g < KS - 1; ++g) {
            const float* src = red + (g * WM * WN + wslot) * PER;
#pragma unroll
            for (int mi = 0; mi < TM; ++mi)
#pragma unroll
                for (int ni = 0; ni < TN; ++ni)
#pragma unroll
                    for (int r = 0; r < 16; ++r) acc[mi][ni][r] += src[((mi * TN + ni) * 16 + r) * 64 + lane];
        }
    }

    // Epilogue: the per-tensor (or per-expert) scale applied once to the sum.
    // With KS > 1 the LDS scratch sits after the reduction buffer; otherwise
    // every wave must first be done with the stage buffers.
    if constexpr (KS == 1) __syncthreads();
    using Store = TileStore<BF16, TM, TN>;
    lds_u8* scratch = lds + (KS > 1 ? C::RED : 0) + (wm * WN + wn) * Store::LDS_BYTES;
    const float scale = p.scale_a[t.expert] * p.scale_b[t.expert];
    Store::run(p.C, acc, scale, t.m0 + wm * C::WTM, t.n0 + wn * C::WTN, t.M, N, t.c_row0, lane, scratch);
}

template <int BM, int BN, int WM, int WN, int KS, int NBUF, int GROUP_M>
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
        if (g.out_bf16) hipLaunchKernelGGL((gemm_kernel<BM, BN, WM, WN, KS, NBUF, GROUP_M, true, false>), grid, block, 0, s, a);
        else hipLaunchKernelGGL((gemm_kernel<BM, BN, WM, WN, KS, NBUF, GROUP_M, false, false>), grid, block, 0, s, a);
    } else {
        if (g.out_bf16) hipLaunchKernelGGL((gemm_kernel<BM, BN, WM, WN, KS, NBUF, GROUP_M, true, true>), grid, block, 0, s, a);
        else hipLaunchKernelGGL((gemm_kernel<BM, BN, WM, WN, KS, NBUF, GROUP_M, false, true>), grid, block, 0, s, a);
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
    if (rows_per_problem <= 64) return launch_cfg<32, 64, 1, 2, 2, 4, 8>(g, s);
    if (rows_per_problem <= 1024) return launch_cfg<128, 128, 2, 2, 1, 4, 8>(g, s);
    return launch_cfg<256, 256, 2, 2, 1, 4, 8>(g, s);
}

}  // namespace fp8k
