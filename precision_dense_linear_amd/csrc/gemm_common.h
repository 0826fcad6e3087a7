// Tiling, tile scheduling and the global -> LDS stage loader shared by the
// FP8 GEMM kernels (per-tensor, grouped and block-scaled).
//
// A workgroup owns a BM x BN tile of C.  Its waves form a WM x WN grid of
// (BM/WM) x (BN/WN) wave tiles made of 32x32 MFMA blocks; KS > 1 splits the
// K range over KS wave groups.  Stages go from global memory straight into
// LDS (buffer_load_dwordx4 ... lds: no VGPR staging).  Ragged M/N/K edges use
// out-of-range buffer offsets, which read as zero without touching memory.
#pragma once

#include "device_utils.h"

namespace fp8k {

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
    // split-K across workgroups (plain GEMM only): `splits` workgroups share a
    // tile, each over its own K range; their FP32 partials meet in `ws` and
    // the last to finish (per-tile arrival counters, zero between launches)
    // sums them in split order and writes C
    int32_t splits;
    float* ws;
    uint32_t* counters;
    int32_t out_f16;  // 2-byte output is IEEE binary16 rather than BF16
    const uint8_t* e8_a;  // E8M0 tile exponents of A [K/32][M/32] (MODE_E8M0 only)
    const uint8_t* e8_b;  // E8M0 tile exponents of B [K/32][N/32]
    const uint32_t* sp_idx;  // 2:4-sparse B: 2-bit positions [K/32][N] (B then holds the values [K/2][N])
};

// B stage layout [K-rows][BN bytes], XOR-swizzled at 16-byte granularity:
// rows sharing a 256-byte bank window get distinct even XOR masks, so the 8
// rows x 2 chunks that one phase of ds_read_b64_tr_b8 touches are distinct.
template <int BN>
__device__ __forceinline__ int swz_b(int r, int c) {
    constexpr int CPR = BN / 16;                   // chunks per row
    constexpr int RPW = BN >= 256 ? 1 : 256 / BN;  // rows per 256-byte window
    return c ^ (((r / RPW) % (CPR / 2)) * 2);
}

// The part of the problem one workgroup works on.
struct TileSlice {
    const uint8_t* A;   // row 0 of this problem (an expert's first row when grouped)
    const uint8_t* B;   // this problem's K x N matrix
    int64_t M;          // rows in this problem
    int64_t m0, n0;     // tile origin inside the problem
    int64_t c_row0;     // row of C that problem row 0 maps to
    int32_t expert;
    int32_t tile;       // linear tile index (split-K bookkeeping)
    int32_t split;      // which of the splits of this tile
    bool valid;
};

// Workgroup id -> tile.  Ids are dealt round-robin over the 8 XCDs, so they
// are first remapped to give each XCD a contiguous run; runs are then laid
// out in column bands of GROUP_M tile rows, so that the tiles one XCD works
// on at the same time share A and B panels in its L2.  With split-K the
// `splits` consecutive remapped ids of a tile are its splits.
template <int BM, int BN, int GROUP_M>
__device__ __forceinline__ TileSlice resolve_tile(const GemmArgs& p) {
    TileSlice s;
    int bid = blockIdx.x;
    const int nblk = gridDim.x;
    if ((nblk & 7) == 0) bid = (bid & 7) * (nblk >> 3) + (bid >> 3);
    s.split = bid % p.splits;
    bid /= p.splits;
    s.tile = bid;
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

// ---------------------------------------------------------------------------
// Deep pipeline (per-tensor and grouped GEMM).  The MFMA loop walks slices of
// 64 bytes of K per wave group.  A is staged 128 bytes of K (two slices) at a
// time, so every A row of a stage is one whole 128-byte line and each A load
// is a full-line L2 request; B is staged one slice (64 K-rows of BN bytes,
// two whole lines per row for BN = 256) at a time.  LDS holds NBUF_A A stages
// and then NB B stages; a deeper pipeline (larger NB) keeps more bytes in
// flight per workgroup where LDS allows it.
//  * A stage: KS sub-tiles of [BM rows][128 bytes]; chunk c of row r sits at
//    position c ^ ((r >> 1) & 7), so the 16 rows of one ds_read_b128 phase
//    (two rows per 256-byte bank window) hit 16 distinct 16-byte bank groups.
//    Wave group ks takes bytes [128 ks, 128 ks + 128) of each A stage.
//  * B stage j: KS sub-tiles of [64 K-rows][BN bytes], swizzled as swz_b;
//    sub-tile ks holds the K-rows that wave group ks multiplies in slice j.
// ---------------------------------------------------------------------------
constexpr int BKP = 64;   // bytes of K per slice (one K step of the MFMA loop)
constexpr int BKA = 128;  // bytes of K per wave group per A stage

__device__ __forceinline__ int swz_a128(int row, int c) { return c ^ ((row >> 1) & 7); }

template <int BM, int BN, int WM, int WN, int KS, int NB_, bool SP = false>
struct PipeCfg {
    static constexpr int NBUF_B = NB_;               // B stage buffers: NB-1 slices of look-ahead
    static constexpr int NBUF_A = (NB_ + 2) / 2;     // A stage buffers (two slices each)
    static constexpr int NW = WM * WN * KS;
    static constexpr int WTM = BM / WM, WTN = BN / WN;
    static constexpr int TM = WTM / 32, TN = WTN / 32;
    static constexpr int A_STAGE = KS * BM * BKA;
    // B stage: the slice's B rows; for a 2:4-sparse B (SP) its 32 compressed
    // value rows, then the index words of its two 32-deep K blocks for the
    // tile's BN columns ([2][BN] x 4 bytes), padded to whole loads per wave.
    static constexpr int B_VAL = KS * (SP ? BKP / 2 : BKP) * BN;
    static constexpr int B_IDX = SP ? 2 * BN * 4 : 0;
    static constexpr int B_STAGE = (B_VAL + B_IDX + 1024 * NW - 1) / (1024 * NW) * (1024 * NW);
    static constexpr int NB_VAL = B_VAL / 1024, NB_IDX = B_IDX / 1024;  // 1 KiB load slots of values, of index
    static constexpr int B_BASE = NBUF_A * A_STAGE;  // LDS offset of the B stages
    static constexpr int NA = A_STAGE / 1024 / NW;   // loads per wave per A stage
    static constexpr int NB = B_STAGE / 1024 / NW;   // loads per wave per B stage
    static constexpr int LPS = NB + NA / 2;          // loads per wave per slice
    static constexpr int RED = (KS > 1) ? (KS - 1) * BM * BN * 4 : 0;
    static constexpr int LDS = B_BASE + NBUF_B * B_STAGE;
    static_assert(WTM % 32 == 0 && WTN % 32 == 0, "wave tile must be whole 32x32 blocks");
    static_assert(A_STAGE % (1024 * NW) == 0 && B_STAGE % (1024 * NW) == 0, "stage loads must split evenly over waves");
    static_assert(NA % 2 == 0, "an A stage is issued in two halves");
    static_assert(BN >= 64 && BN <= 256 && (BN & (BN - 1)) == 0, "BN must be 64, 128 or 256");
    static_assert(NB_ >= 4 && NB_ % 2 == 0, "B buffers: even, at least 4");
    static_assert((NB_ - 1) * LPS <= 63, "in-flight loads must fit the vmcnt counter");
    static_assert(LDS <= 160 * 1024, "LDS budget");
    static_assert(!SP || (KS == 1 && B_IDX % 1024 == 0), "sparse B: one wave group, whole index loads");
};

// One wave-wide global->LDS load, written as inline assembly: M0 holds the
// wave's LDS destination, lane l's 16 bytes land at M0 + 16*l.  The compiler
// does not see these as LDS writes, so it neither serialises later LDS reads
// behind them nor counts them; the kernel waits for them explicitly with
// s_waitcnt vmcnt(n), n = loads issued after the stage it needs.  (The
// compiler's own form, __builtin_amdgcn_raw_ptr_buffer_load_lds, makes it
// wait for every such load before the next LDS read: 30 vmcnt(0) waits
// instead of 2 in the 256 x 256 exact tile loop, which drains the pipeline.)
// M0 is listed as clobbered, which the compiler does not promise to honour
// for a reserved register; that is safe only while no other code in these
// kernels keeps a value in M0.  tests/test_isa_invariants.py checks it on
// every build: in the disassembly, each instruction naming M0 is this
// s_mov_b32 directly followed by its LDS-direct load.
__device__ __forceinline__ void dma16(__amdgpu_buffer_rsrc_t r, uint32_t lds_addr, uint32_t voff) {
    asm volatile("s_mov_b32 m0, %0\n\tbuffer_load_dwordx4 %1, %2, 0 offen lds"
                 :
                 : "s"(lds_addr), "v"(voff), "s"(r)
                 : "memory", "m0");
}

// s_waitcnt vmcnt(n) with the other counters left alone (gfx9 encoding:
// vmcnt[3:0] in bits 3:0 and vmcnt[5:4] in bits 15:14, expcnt 6:4 = 7,
// lgkmcnt 11:8 = 15).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
    static_assert(N >= 0 && N <= 63, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

// s_waitcnt vmcnt(n) lgkmcnt(0): also every LDS read this wave has issued is
// complete (its data is in registers), so after a following barrier no wave
// still reads the buffers whose fragments are already loaded.
template <int N>
__device__ __forceinline__ void wait_vmcnt_lds() {
    static_assert(N >= 0 && N <= 63, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4));
}

// Load schedule (NB = NBUF_B): slice s issues B stage s+NB and one half of A
// stage (s+NB+1)/2 (half (s+1)&1), LPS loads per wave in all.  Stage data is
// thus issued NB-1 slices before the slice whose fragment reads need it.  A
// buffer is refilled only after the barrier that follows the reads of its
// last fragments: B stage s+NB goes to the buffer of stage s, whose
// fragments are in registers by slice s; A stage a is issued from slice
// 2a-NB-1 into the buffer of stage a-NBUF_A, last read in slice
// 2(a-NBUF_A) <= 2a-NB-2 because 2*NBUF_A >= NB+2.
template <int BM, int BN, int WM, int WN, int KS, int NB, bool SP = false>
struct PipeLoader {
    using C = PipeCfg<BM, BN, WM, WN, KS, NB, SP>;
    uint32_t a_off[C::NA], a_kk[C::NA], b_off[C::NB];
    bool b_idx[C::NB];  // SP: load slot i of this wave fetches index words (else values)
    const uint8_t* a_base;
    const uint8_t* b_base;
    const uint8_t* i_base;  // SP: index words of the tile's first column
    int64_t a_bytes, b_bytes, i_bytes, K, N;
    uint32_t lds_wave;  // LDS byte address of this wave's first 1 KiB slot

    // Loads K bytes [k_begin, k_end) of the tile's A rows and B columns (the
    // whole K unless split-K gives this workgroup a part).
    __device__ __forceinline__ PipeLoader(const TileSlice& t, int64_t N_, int64_t K_, int64_t k_begin, int64_t k_end,
                                          int wave, int lane, uint32_t lds_base, const uint32_t* sp_idx = nullptr) {
        K = k_end - k_begin;  // K range this loader covers (A rows keep the full stride K_)
        N = N_;
        const int64_t rows_here = t.M - t.m0;
        a_base = t.A + t.m0 * K_ + k_begin;
        a_bytes = rows_here * K_ - k_begin;
        if constexpr (SP) {  // values [K/2][N], index words [K/32][N] (whole K: no split-K here)
            b_base = t.B + t.n0;
            b_bytes = (K / 2) * N - t.n0;
            i_base = reinterpret_cast<const uint8_t*>(sp_idx) + t.n0 * 4;
            i_bytes = ((K + 31) / 32) * N * 4 - t.n0 * 4;
        } else {
            b_base = t.B + t.n0 + k_begin * N;
            b_bytes = K * N - t.n0;
            i_base = nullptr;
            i_bytes = 0;
        }
        lds_wave = lds_base + wave * 1024;
#pragma unroll
        for (int i = 0; i < C::NA; ++i) {
            const int slot = (i * C::NW + wave) * 64 + lane;
            const int sub = slot / (BM * 8);
            const int s2 = slot % (BM * 8);
            const int row = s2 >> 3;
            const int kk = sub * BKA + swz_a128(row, s2 & 7) * 16;
            a_kk[i] = kk;
            a_off[i] = row < rows_here ? (uint32_t)(row * K_ + kk) : OOB;
        }
#pragma unroll
        for (int i = 0; i < C::NB; ++i) {
            if constexpr (SP) {
                const int ld = i * C::NW + wave;  // 1 KiB slot of the stage
                b_idx[i] = ld >= C::NB_VAL;
                if (ld < C::NB_VAL) {  // value rows, swizzled as B
                    const int s2 = ld * 64 + lane;
                    const int r = s2 / (BN / 16);
                    const int c = swz_b<BN>(r, s2 % (BN / 16));
                    b_off[i] = (t.n0 + c * 16 < N) ? (uint32_t)(r * N + c * 16) : OOB;
                } else if (ld < C::NB_VAL + C::NB_IDX) {  // index words: K block o / (4 BN), 4 columns per lane
                    const int o = (ld - C::NB_VAL) * 1024 + lane * 16;
                    const int kb = o / (BN * 4), w = o % (BN * 4);
                    b_off[i] = (t.n0 + w / 4 < N) ? (uint32_t)(kb * N * 4 + w) : OOB;
                } else {
                    b_off[i] = OOB;  // padding of the stage
                }
            } else {
                const int slot = (i * C::NW + wave) * 64 + lane;
                const int sub = slot / (BKP * BN / 16);
                const int s2 = slot % (BKP * BN / 16);
                const int r = s2 / (BN / 16);
                const int c = swz_b<BN>(r, s2 % (BN / 16));
                b_off[i] = (t.n0 + c * 16 < N) ? (uint32_t)((sub * BKA + r) * N + c * 16) : OOB;
                b_idx[i] = false;
            }
        }
    }

    // The loads of slice s (see above): resources and LDS destinations.  Past
    // the end of K the resources are empty, so every load reads zero.
    struct Stage {
        __amdgpu_buffer_rsrc_t ra, rb, ri;
        int64_t krem;
        uint32_t dst_a, dst_b;
    };
    __device__ __forceinline__ Stage prepare(int s) const {
        Stage g;
        const int jb = s + NB;             // B stage
        const int ja = (s + NB + 1) >> 1;  // A stage
        const int64_t kb0 = (int64_t)(jb >> 1) * (KS * BKA) + (jb & 1) * BKP;
        const int64_t ka0 = (int64_t)ja * (KS * BKA);
        g.ra = make_rsrc(a_base + ka0, clamp_records(a_bytes - ka0));
        if constexpr (SP) {  // compressed rows kb0/2 .., index row kb0/32 ..
            g.rb = make_rsrc(b_base + (kb0 / 2) * N, clamp_records(b_bytes - (kb0 / 2) * N));
            g.ri = make_rsrc(i_base + (kb0 / 32) * N * 4, clamp_records(i_bytes - (kb0 / 32) * N * 4));
        } else {
            g.rb = make_rsrc(b_base + kb0 * N, clamp_records(b_bytes - kb0 * N));
            g.ri = g.rb;
        }
        g.krem = K - ka0;
        g.dst_a = __builtin_amdgcn_readfirstlane(lds_wave + (uint32_t)(ja % C::NBUF_A) * C::A_STAGE);
        g.dst_b = __builtin_amdgcn_readfirstlane(lds_wave + C::B_BASE + (uint32_t)(jb % NB) * C::B_STAGE);
        return g;
    }
    // Load r (0 <= r < LPS) of a slice whose A half is `half`: the NB B loads
    // first, then the A stage's loads [half * NA/2, half * NA/2 + NA/2).
    __device__ __forceinline__ void issue_one(const Stage& g, int r, int half) const {
        if (r < C::NB) {
            dma16((SP && b_idx[r]) ? g.ri : g.rb, g.dst_b + r * C::NW * 1024, b_off[r]);
        } else {
            const int i = half * (C::NA / 2) + (r - C::NB);
            dma16(g.ra, g.dst_a + i * C::NW * 1024, (int64_t)a_kk[i] < g.krem ? a_off[i] : OOB);
        }
    }
    // A slice's loads all at once (the pipeline prologue).
    __device__ __forceinline__ void issue_slice(int s) const {
        const Stage g = prepare(s);
        const int half = (s + 1) & 1;
#pragma unroll
        for (int r = 0; r < C::LPS; ++r) issue_one(g, r, half);
    }
    // Only the A half of slice s (the first load of the prologue).
    __device__ __forceinline__ void issue_a_half(int s) const {
        const Stage g = prepare(s);
        const int half = (s + 1) & 1;
#pragma unroll
        for (int r = C::NB; r < C::LPS; ++r) issue_one(g, r, half);
    }
};

// Epilogue: store the wave's TM x TN accumulator blocks, each sum
// multiplied by `sa` and then by `sb` (two roundings; the product sa * sb
// itself could fall below the normal binary32 range where C does not).  The kernels issue each MFMA with the B fragment as the first
// operand, so accumulator block (mi, ni) holds C^T: element r of lane l is
// row 32mi + (l & 31), column 32ni + 8(r >> 2) + 4(l >> 5) + (r & 3) of the
// wave tile -- four consecutive columns of one row per r/4 group.  Those go
// to a wave-private LDS region as 8-byte (BF16) or 16-byte (FP32) writes,
// row-major with the 16-byte chunks XOR-swizzled by row, and come back as
// 16-byte row chunks that are stored to C fully coalesced (one 1 KiB
// contiguous run per 64 lanes and instruction).  Rows are done in passes of
// at most 32 KiB of LDS.  Rows >= M and columns >= N (N % 16 == 0, so a
// chunk is either inside or outside) are masked only at the edges.
template <bool BF16, int TM, int TN>
struct TileStore {
    static constexpr int OSZ = BF16 ? 2 : 4;
    static constexpr int ROWB = 32 * TN * OSZ;  // bytes per wave-tile row
    static constexpr int CHUNKS = ROWB / 16;
    static constexpr int PASS_MI = (32768 / (32 * ROWB)) < TM ? (32768 / (32 * ROWB)) : TM;
    static constexpr int LDS_BYTES = PASS_MI * 32 * ROWB;  // per wave
    static_assert(PASS_MI >= 1 && TM % PASS_MI == 0, "epilogue pass size");

    __device__ static __forceinline__ int swz(int row, int ch) { return ch ^ (row & (CHUNKS - 1)); }

    __device__ static __forceinline__ void run(void* C, const v16f (&acc)[TM][TN], float sa, float sb, int64_t m_base,
                                               int64_t n_base, int64_t M, int64_t N, int64_t c_row0, int lane,
                                               lds_u8* scratch, bool f16) {
        const bool full = (m_base + 32 * TM <= M) && (n_base + 32 * TN <= N);
        const int rows_left = (int)(M - m_base < 32 * TM ? M - m_base : 32 * TM);
        const int cols_left = (int)(N - n_base < 32 * TN ? N - n_base : 32 * TN);
        uint8_t* base = reinterpret_cast<uint8_t*>(C) + ((c_row0 + m_base) * N + n_base) * OSZ;
        const int ldc = (int)N * OSZ;
#pragma unroll
        for (int p0 = 0; p0 < TM; p0 += PASS_MI) {
#pragma unroll
            for (int mi = 0; mi < PASS_MI; ++mi) {
                const int row = mi * 32 + (lane & 31);
#pragma unroll
                for (int ni = 0; ni < TN; ++ni)
#pragma unroll
                    for (int q = 0; q < 4; ++q) {
                        const v16f& a = acc[p0 + mi][ni];
                        const int cb = (ni * 32 + 8 * q + 4 * (lane >> 5)) * OSZ;  // byte column in the row
                        lds_u8* dst = scratch + row * ROWB + swz(row, cb >> 4) * 16 + (cb & 15);
                        const float c0 = (a[4 * q] * sa) * sb, c1 = (a[4 * q + 1] * sa) * sb;
                        const float c2 = (a[4 * q + 2] * sa) * sb, c3 = (a[4 * q + 3] * sa) * sb;
                        if constexpr (BF16) {
                            if (f16) {
                                typedef _Float16 v4h __attribute__((ext_vector_type(4)));
                                const v4h v = {(_Float16)c0, (_Float16)c1, (_Float16)c2, (_Float16)c3};
                                *(__attribute__((address_space(3))) v4h*)dst = v;
                            } else {
                                typedef __bf16 v4bf __attribute__((ext_vector_type(4)));
                                const v4bf v = {(__bf16)c0, (__bf16)c1, (__bf16)c2, (__bf16)c3};
                                *(__attribute__((address_space(3))) v4bf*)dst = v;
                            }
                        } else {
                            const v4f v = {c0, c1, c2, c3};
                            *(__attribute__((address_space(3))) v4f*)dst = v;
                        }
                    }
            }
            constexpr int ITER = PASS_MI * 32 * CHUNKS / 64;
#pragma unroll
            for (int it = 0; it < ITER; ++it) {
                const int idx = it * 64 + lane;
                const int row = idx / CHUNKS, ch = idx % CHUNKS;
                const v4i v = lds_read16(scratch + row * ROWB + swz(row, ch) * 16);
                const int grow = p0 * 32 + row, gcolb = ch * 16;
                if (full || (grow < rows_left && gcolb < cols_left * OSZ))
                    *reinterpret_cast<v4i*>(base + grow * ldc + gcolb) = v;
            }
        }
    }
};

}  // namespace fp8k
