// Tiling, tile scheduling and the global -> LDS stage loader shared by the
// FP8 GEMM kernels (per-tensor, grouped and block-scaled).
//
// A workgroup owns a BM x BN tile of C.  Its waves form a WM x WN grid of
// (BM/WM) x (BN/WN) wave tiles made of 32x32 MFMA blocks; KS > 1 splits each
// K step over KS wave groups.  The K loop moves KS*128 bytes of K per step.
// Stages go from global memory straight into LDS (buffer_load_dwordx4 ...
// lds: no VGPR staging), double buffered.  Ragged M/N/K edges use
// out-of-range buffer offsets, which read as zero without touching memory.
//
// LDS layouts, XOR-swizzled at 16-byte granularity:
//  * A stage: KS sub-tiles of [BM rows][128 bytes of K]; chunk c of row r sits
//    at position c ^ ((r >> 1) & 7): the 16 rows one ds_read_b128 phase
//    touches (two rows per 256-byte bank window) land on 16 distinct chunks.
//  * B stage: KS sub-tiles of [128 K-rows][BN bytes]; rows sharing a 256-byte
//    window get distinct even XOR masks, so the 8 rows x 2 chunks that one
//    32-lane phase of ds_read_b64_tr_b8 touches are distinct.
#pragma once

#include "device_utils.h"

namespace fp8k {

constexpr int BK = 128;  // bytes of K per wave group per step

struct GemmArgs {
    const uint8_t* A;
    const uint8_t* B;
    void* C;
    const float* scale_a;   // per-tensor: [1]; grouped: [experts]; block-scaled: [M/32][K/32]
    const float* scale_b;   // per-tensor: [1]; grouped: [experts]; block-scaled: [K/32][N/32]
    const int32_t* offsets; // grouped only: experts+1 row boundaries
    int32_t experts;        // 0 unless grouped
    int64_t M, N, K;
    int32_t tiles_m, tiles_n;
};

__device__ __forceinline__ int swz_a(int row, int c) { return c ^ ((row >> 1) & 7); }

template <int BN>
__device__ __forceinline__ int swz_b(int r, int c) {
    constexpr int CPR = BN / 16;                   // chunks per row
    constexpr int RPW = BN >= 256 ? 1 : 256 / BN;  // rows per 256-byte window
    return c ^ (((r / RPW) % (CPR / 2)) * 2);
}

template <int BM, int BN, int WM, int WN, int KS>
struct TileCfg {
    static constexpr int NW = WM * WN * KS;
    static constexpr int NT = 64 * NW;
    static constexpr int WTM = BM / WM, WTN = BN / WN;
    static constexpr int TM = WTM / 32, TN = WTN / 32;
    static constexpr int A_STAGE = KS * BM * BK;
    static constexpr int B_STAGE = KS * BK * BN;
    static constexpr int STAGE = A_STAGE + B_STAGE;
    static constexpr int A_INSTR = A_STAGE / 1024;  // wave-wide 1 KiB loads per stage
    static constexpr int B_INSTR = B_STAGE / 1024;
    static constexpr int RED = (KS > 1) ? (KS - 1) * BM * BN * 4 : 0;
    static constexpr int LDS = (2 * STAGE > RED) ? 2 * STAGE : RED;
    static_assert(WTM % 32 == 0 && WTN % 32 == 0, "wave tile must be whole 32x32 blocks");
    static_assert(A_INSTR % NW == 0 && B_INSTR % NW == 0, "stage loads must split evenly over waves");
    static_assert(BN >= 64 && BN <= 256 && (BN & (BN - 1)) == 0, "BN must be 64, 128 or 256");
    static_assert(LDS <= 160 * 1024, "LDS budget");
};

// The part of the problem one workgroup works on.
struct TileSlice {
    const uint8_t* A;   // row 0 of this problem (an expert's first row when grouped)
    const uint8_t* B;   // this problem's K x N matrix
    int64_t M;          // rows in this problem
    int64_t m0, n0;     // tile origin inside the problem
    int64_t c_row0;     // row of C that problem row 0 maps to
    int32_t expert;
    bool valid;
};

// Workgroup id -> tile.  Ids are dealt round-robin over the 8 XCDs, so they
// are first remapped to give each XCD a contiguous run; runs are then laid
// out in column bands of GROUP_M tile rows, so that the tiles one XCD works
// on at the same time share A and B panels in its L2.
template <int BM, int BN, int GROUP_M>
__device__ __forceinline__ TileSlice resolve_tile(const GemmArgs& p) {
    TileSlice s;
    int bid = blockIdx.x;
    const int nblk = gridDim.x;
    if ((nblk & 7) == 0) bid = (bid & 7) * (nblk >> 3) + (bid >> 3);
    const int per_group = GROUP_M * p.tiles_n;
    const int group = bid / per_group;
    const int first_m = group * GROUP_M;
    const int gm = min(p.tiles_m - first_m, GROUP_M);
    const int in_group = bid - group * per_group;
    const int tm = first_m + in_group % gm;
    const int tn = in_group / gm;
    s.n0 = (int64_t)tn * BN;
    s.valid = true;
    s.expert = 0;
    if (p.experts == 0) {
        s.A = p.A;
        s.B = p.B;
        s.M = p.M;
        s.m0 = (int64_t)tm * BM;
        s.c_row0 = 0;
        return s;
    }
    // Grouped: walk the experts' row ranges (clamped into [0, M] and made
    // non-decreasing) to find which expert owns global m tile tm.
    int64_t lo = 0;
    int rem = tm;
    for (int e = 0; e < p.experts; ++e) {
        int64_t b0 = p.offsets[e], b1 = p.offsets[e + 1];
        b0 = b0 < lo ? lo : (b0 > p.M ? p.M : b0);
        b1 = b1 < b0 ? b0 : (b1 > p.M ? p.M : b1);
        lo = b0;
        const int64_t cnt = b1 - b0;
        const int tiles = (int)((cnt + BM - 1) / BM);
        if (rem < tiles) {
            s.A = p.A + b0 * p.K;
            s.B = p.B + (int64_t)e * p.K * p.N;
            s.M = cnt;
            s.m0 = (int64_t)rem * BM;
            s.c_row0 = b0;
            s.expert = e;
            return s;
        }
        rem -= tiles;
    }
    s.valid = false;
    return s;
}

// Enqueue one stage (KS*128 bytes of K starting at k0) into LDS buffer `dst`.
// Called by every wave of the workgroup with its wave index; each wave issues
// A_INSTR/NW + B_INSTR/NW wave-wide 1 KiB loads.
template <int BM, int BN, int WM, int WN, int KS>
__device__ __forceinline__ void load_stage(const TileSlice& t, int64_t N, int64_t K, int64_t k0, lds_u8* dst,
                                           int wave, int lane) {
    using C = TileCfg<BM, BN, WM, WN, KS>;
    lds_u8* As = dst;
    lds_u8* Bs = dst + C::A_STAGE;
    const int64_t rows_here = t.M - t.m0;
    const __amdgpu_buffer_rsrc_t ra = make_rsrc(t.A + t.m0 * K + k0, clamp_records(rows_here * K - k0));
#pragma unroll
    for (int i = 0; i < C::A_INSTR / C::NW; ++i) {
        const int q = i * C::NW + wave;
        const int slot = q * 64 + lane;
        const int sub = slot / (BM * 8);
        const int s2 = slot % (BM * 8);
        const int row = s2 >> 3;
        const int c = swz_a(row, s2 & 7);
        const int64_t kk = (int64_t)sub * BK + c * 16;
        const bool ok = (row < rows_here) && (k0 + kk < K);
        load16_to_lds(ra, As + q * 1024, ok ? (uint32_t)(row * K + kk) : OOB);
    }
    const __amdgpu_buffer_rsrc_t rb = make_rsrc(t.B + k0 * N + t.n0, clamp_records((K - k0) * N - t.n0));
#pragma unroll
    for (int i = 0; i < C::B_INSTR / C::NW; ++i) {
        const int q = i * C::NW + wave;
        const int slot = q * 64 + lane;
        const int sub = slot / (BK * BN / 16);
        const int s2 = slot % (BK * BN / 16);
        const int r = s2 / (BN / 16);
        const int c = swz_b<BN>(r, s2 % (BN / 16));
        const int64_t kr = (int64_t)sub * BK + r;
        const bool ok = (k0 + kr < K) && (t.n0 + c * 16 < N);
        load16_to_lds(rb, Bs + q * 1024, ok ? (uint32_t)(kr * N + c * 16) : OOB);
    }
}

// Store one 32x32 accumulator block (rows m_base.., columns n_base.. of the
// problem), multiplied by `scale`, masking rows >= M and columns >= N.
template <bool BF16>
__device__ __forceinline__ void store_block(void* C, const v16f& acc, float scale, int64_t m_base, int64_t n_base,
                                            int64_t M, int64_t N, int64_t c_row0, int lane) {
    const int64_t col = n_base + (lane & 31);
    if (col >= N) return;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
        const int64_t row = m_base + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
        if (row >= M) continue;
        const float v = acc[r] * scale;
        const int64_t idx = (c_row0 + row) * N + col;
        if constexpr (BF16) reinterpret_cast<uint16_t*>(C)[idx] = f32_to_bf16_rne(v);
        else reinterpret_cast<float*>(C)[idx] = v;
    }
}

}  // namespace fp8k
