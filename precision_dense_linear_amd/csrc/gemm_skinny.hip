// Skinny per-tensor FP8 GEMM for M <= 16 rows (a few tokens times a large
// weight: the decode-time linear layers of "Triton FP8 GEMM via CUTLASS
// naming", whose opening section has GEMMs carrying the bulk of inference),
// default (exact-product) accumulation, K split across workgroups through
// the caller's workspace:
//
//   C[m, n] = (scale_a * scale_b) * sum_k A[m, k] * B[k, n]
//
// Such a GEMM streams B once from memory, so the kernel is built around how
// B is read.  A workgroup owns 256 columns and a range of K, which it walks
// in stages of 32 K-rows: every stage is 32 whole 256-byte row segments of B
// (8 KiB, one 1 KiB load per wave) and A's 16 rows x 32 bytes, loaded
// straight from global memory into a ring of R stages in LDS, R - 1 stages
// in flight.  Workgroup ids are laid out K-range-major, so the workgroups
// that run together read one band of whole B rows (reading 64-byte-wide
// strips down many rows instead measured ~23 us for a 64 MiB B, 256-byte
// segments ~12.5 us).  Each of the 8 waves owns 32 of the columns, so the
// stages are shared but no sums are: the codes are widened exactly to BF16
// and multiplied on v_mfma_f32_16x16x32_bf16 (16 rows: nothing padded at
// M = 16) into C^T blocks, and the splits' partial sums meet through the
// workspace, added in split order.
#include "gemm_dispatch.h"

namespace fp8k {

namespace {

constexpr int SK_BN = 256;                // columns per workgroup
constexpr int SK_KS = 32;                 // K bytes per stage
constexpr int SK_W = 8;                   // waves per workgroup
constexpr int SK_NI = SK_BN / SK_W / 16;  // 16-column MFMA blocks per wave
constexpr int SK_T = SK_KS / 32;          // 32-deep MFMA steps per stage
constexpr int SK_CA = SK_KS / 16;         // 16-byte chunks per A row of a stage
constexpr int SK_A = 1024;                // A part of a stage: 16 rows x SK_KS bytes (the rest zero)
constexpr int SK_STAGE = SK_A + SK_KS * SK_BN;
constexpr int SK_CHUNK = 8;               // partials read at a time by the last split
constexpr int SK_SLOTS = SK_BN * 16 / SPLIT_TILE_FLOATS;  // workspace split tiles per partial
constexpr int SK_LPW = SK_KS * SK_BN / 1024 / SK_W;  // B loads per wave per stage
static_assert(SK_LPW * SK_W * 1024 == SK_KS * SK_BN, "a stage's B loads split evenly over the waves");

typedef float v4f_t __attribute__((ext_vector_type(4)));

__device__ __forceinline__ v4f_t mfma_16x16x32_bf16(v8bf a, v8bf b, v4f_t c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// A part layout: row m's 16-byte chunk c (of SK_CA) at position
// c ^ ((m / (16 / SK_CA)) % SK_CA), so the 8-byte reads of rows 0..15 at one
// chunk fall in distinct banks.
__device__ __forceinline__ int swz_sa(int m, int c) { return c ^ ((m / (16 / SK_CA)) % SK_CA); }

template <int R, bool BF16, bool SPLITK, int FMT>
__global__ void __launch_bounds__(64 * SK_W) skinny_kernel(GemmArgs p) {
    constexpr int FA = FMT & 1, FB = (FMT >> 1) & 1;
    __shared__ __attribute__((aligned(1024))) uint8_t smem[R * SK_STAGE];

    int bid = blockIdx.x;
    const int nblk = gridDim.x;
    if ((nblk & 7) == 0) bid = (bid & 7) * (nblk >> 3) + (bid >> 3);  // a contiguous run of ids per XCD
    const int tile = bid % p.tiles_n;        // K-range-major: an XCD's run covers neighbouring columns
    const int split = bid / p.tiles_n;
    const int64_t n0 = (int64_t)tile * SK_BN;
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int g = lane >> 4, i16 = lane & 15;
    const int64_t M = p.M, N = p.N, K = p.K;
    const float sa = p.scale_a[0], sb = p.scale_b[0];

    // this workgroup's stages [s0, s1) of 32 bytes of K (stages past the end
    // of K read zero)
    const int64_t nsl = (K + SK_KS - 1) / SK_KS;
    const int64_t s0 = split * nsl / p.splits, s1 = (split + 1) * nsl / p.splits;
    const int ns = (int)(s1 - s0);

    // per-lane load offsets: wave w's load i fetches B rows 4 q .. 4 q + 3
    // of a stage, q = SK_LPW w + i (lane L: row 4 q + L/16, chunk position
    // L%16; swz_b is its own inverse); wave 0 also A (lanes 0..31: row L/2,
    // chunk position L%2)
    uint32_t b_off[SK_LPW];
#pragma unroll
    for (int i = 0; i < SK_LPW; ++i) {
        const int br = 4 * (SK_LPW * wave + i) + (lane >> 4), bc = swz_b<SK_BN>(br, lane & 15);
        b_off[i] = n0 + bc * 16 < N ? (uint32_t)(br * N + bc * 16) : OOB;
    }
    const int am = lane / SK_CA, ac = swz_sa(am, lane % SK_CA);
    const bool a_lane_ok = lane < 16 * SK_CA && am < M;
    const uint32_t lds0 = (uint32_t)(uintptr_t)smem;
    const __amdgpu_buffer_rsrc_t ra = make_rsrc(p.A, clamp_records(M * K));
    auto issue = [&](int j) {
        const int64_t st = s0 + j;
        const bool live = st < s1;
        const int64_t k0 = st * SK_KS;
        const uint32_t e = lds0 + (j % R) * SK_STAGE;
        const __amdgpu_buffer_rsrc_t rb =
            make_rsrc(p.B + (live ? k0 * N : 0) + n0, live ? clamp_records((K - k0) * N - n0) : 0u);
#pragma unroll
        for (int i = 0; i < SK_LPW; ++i)
            dma16(rb, __builtin_amdgcn_readfirstlane(e + SK_A + (SK_LPW * wave + i) * 1024), b_off[i]);
        if (wave == 0) {
            const bool a_ok = live && a_lane_ok && k0 + ac * 16 < K;
            dma16(ra, __builtin_amdgcn_readfirstlane(e), a_ok ? (uint32_t)(am * K + k0 + ac * 16) : OOB);
        }
    };

    // LDS read offsets within a stage, per 32-deep step t: A -- lane (g,
    // m = l%16) reads K 32 t + 8 g .. +7 of row m; B -- this wave's
    // 16-column block h: rows 32 t + 8 g + (l%16)/2, columns 32 w + 16 h +
    // 8 (l&1) (transposed on read: lane (g, i) gets column 32 w + 16 h + i,
    // K rows 32 t + 8 g .. +7)
    int a_rd[SK_T], b_rd[SK_T][SK_NI];
#pragma unroll
    for (int t = 0; t < SK_T; ++t) {
        a_rd[t] = i16 * SK_KS + swz_sa(i16, 2 * t + (g >> 1)) * 16 + 8 * (g & 1);
#pragma unroll
        for (int h = 0; h < SK_NI; ++h) {
            const int r = 32 * t + 8 * g + (i16 >> 1);
            const int col = SK_NI * 16 * wave + 16 * h + 8 * (i16 & 1);
            b_rd[t][h] = SK_A + r * SK_BN + swz_b<SK_BN>(r, col >> 4) * 16 + (col & 15);
        }
    }

    v4f_t acc[SK_NI];
#pragma unroll
    for (int h = 0; h < SK_NI; ++h) acc[h] = (v4f_t){0.0f, 0.0f, 0.0f, 0.0f};

    // Stage j: wait for this wave's loads of stage j (wave 0 issues one more
    // per stage, A's); barrier -- every wave's loads of stage j have landed and every
    // wave is done reading stage j - 1, whose slot stage j + R - 1 refills.
#pragma unroll
    for (int j = 0; j < R - 1; ++j) issue(j);
    for (int j = 0; j < ns; ++j) {
        if (wave == 0) wait_vmcnt_lds<(SK_LPW + 1) * (R - 2)>();
        else wait_vmcnt_lds<SK_LPW * (R - 2)>();
        __syncthreads();
        issue(j + R - 1);
        const lds_u8* e = (const lds_u8*)smem + (j % R) * SK_STAGE;
#pragma unroll
        for (int t = 0; t < SK_T; ++t) {
            const v2i av = *(const __attribute__((address_space(3))) v2i*)(e + a_rd[t]);
            const v8bf af = fp8x8_to_bf16<FA>(av[0], av[1]);
#pragma unroll
            for (int h = 0; h < SK_NI; ++h) {
                const v2i bv = lds_read_tr8(e + b_rd[t][h]);
                acc[h] = mfma_16x16x32_bf16(fp8x8_to_bf16<FB>(bv[0], bv[1]), af, acc[h]);
            }
        }
    }
    wait_vmcnt<0>();                        // (the empty loads past the last stage)

    // split-K across workgroups: every wave writes its blocks of the partial
    // (rows < M) to the caller's workspace (through to memory); once all have, one
    // arrival is counted per workgroup; the waves of the last of the splits
    // to arrive read the partials of their blocks (bypassing their caches)
    // and add them in split order.  Counters are zero between launches: the
    // last arrival resets its own.
    if constexpr (SPLITK) {
        constexpr int SC1 = 16;             // cache policy: coherent at device scope
        constexpr uint32_t PART = SK_SLOTS * SPLIT_TILE_FLOATS * 4;  // bytes per partial
        const __amdgpu_buffer_rsrc_t rw =
            make_rsrc(p.ws + (int64_t)tile * p.splits * SK_SLOTS * SPLIT_TILE_FLOATS, (uint32_t)p.splits * PART);
        const uint32_t mine = (uint32_t)((SK_NI * wave * 64 + lane) * 16);
        const bool row_ok = i16 < M;
        if (row_ok)
#pragma unroll
            for (int h = 0; h < SK_NI; ++h)
                __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(v4i, acc[h]), rw,
                                                       split * PART + mine + h * 1024, 0, SC1);
        wait_vmcnt<0>();                    // this wave's stores have reached memory
        __syncthreads();                    // ... and every wave's
        int* flag = reinterpret_cast<int*>(smem);
        if (threadIdx.x == 0)
            *flag = __hip_atomic_fetch_add(p.counters + tile, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) ==
                    (uint32_t)(p.splits - 1);
        __syncthreads();
        if (!*flag) return;
#pragma unroll
        for (int h = 0; h < SK_NI; ++h) acc[h] = (v4f_t){0.0f, 0.0f, 0.0f, 0.0f};
        for (int sp0 = 0; sp0 < p.splits; sp0 += SK_CHUNK) {
            v4i part[SK_CHUNK][SK_NI];
#pragma unroll
            for (int u = 0; u < SK_CHUNK; ++u)
#pragma unroll
                for (int h = 0; h < SK_NI; ++h)
                    part[u][h] = row_ok && sp0 + u < p.splits ? __builtin_amdgcn_raw_buffer_load_b128(
                                                          rw, (sp0 + u) * PART + mine + h * 1024, 0, SC1)
                                                    : (v4i){0, 0, 0, 0};
#pragma unroll
            for (int u = 0; u < SK_CHUNK; ++u)
                if (sp0 + u < p.splits)
#pragma unroll
                    for (int h = 0; h < SK_NI; ++h) acc[h] += __builtin_bit_cast(v4f_t, part[u][h]);
        }
        if (threadIdx.x == 0) __hip_atomic_store(p.counters + tile, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }

    // epilogue: lane (g, m) holds row m, columns n0 + 32 w + 16 h + 4 g .. +3
    // (C^T blocks); scales applied one after the other
    const int m = i16;
    if (m >= M) return;
    const bool f16 = p.out_f16 != 0;
#pragma unroll
    for (int h = 0; h < SK_NI; ++h) {
        const int64_t col = n0 + 16 * (SK_NI * wave + h) + 4 * g;
        if (col >= N) continue;
        const v4f_t c = acc[h];
        const float c0 = (c[0] * sa) * sb, c1 = (c[1] * sa) * sb;
        const float c2 = (c[2] * sa) * sb, c3 = (c[3] * sa) * sb;
        if constexpr (BF16) {
            uint16_t* dst = reinterpret_cast<uint16_t*>(p.C) + m * N + col;
            if (f16) {
                typedef _Float16 v4h __attribute__((ext_vector_type(4)));
                *reinterpret_cast<v4h*>(dst) = (v4h){(_Float16)c0, (_Float16)c1, (_Float16)c2, (_Float16)c3};
            } else {
                typedef __bf16 v4bf __attribute__((ext_vector_type(4)));
                *reinterpret_cast<v4bf*>(dst) = (v4bf){(__bf16)c0, (__bf16)c1, (__bf16)c2, (__bf16)c3};
            }
        } else {
            *reinterpret_cast<v4f*>(reinterpret_cast<float*>(p.C) + m * N + col) = (v4f){c0, c1, c2, c3};
        }
    }
}

template <int R, bool SPLITK, int FMT>
hipError_t launch_r(const GemmProblem& g, hipStream_t s, int splits) {
    GemmArgs a{};
    a.A = g.A;
    a.B = g.B;
    a.C = g.C;
    a.scale_a = g.scale_a;
    a.scale_b = g.scale_b;
    a.M = g.M;
    a.N = g.N;
    a.K = g.K;
    a.tiles_n = (int32_t)((g.N + SK_BN - 1) / SK_BN);
    a.tiles_m = 1;
    a.splits = splits;
    a.ws = g.ws;
    a.counters = g.counters;
    a.out_f16 = g.out_f16;
    const int64_t blocks = (int64_t)a.tiles_n * splits;
    if (blocks == 0) return hipSuccess;
    if (g.out_bf16) hipLaunchKernelGGL((skinny_kernel<R, true, SPLITK, FMT>), dim3((unsigned)blocks), dim3(64 * SK_W), 0, s, a);
    else hipLaunchKernelGGL((skinny_kernel<R, false, SPLITK, FMT>), dim3((unsigned)blocks), dim3(64 * SK_W), 0, s, a);
    return hipGetLastError();
}

}  // namespace

// M <= 16.  Splits (with a workspace): one workgroup per CU, at most 16 per
// tile, each over at least 16 stages, SK_SLOTS workspace split tiles each.
// Without a split the class takes only problems with at least half as many
// tiles as CUs.
int skinny_splits(const GemmProblem& g) {
    const int64_t tiles = (g.N + SK_BN - 1) / SK_BN;
    const int64_t nsl = (g.K + SK_KS - 1) / SK_KS;
    const int64_t cus = split_slots() / 2;
    int64_t sp = 1;
    if (g.ws && g.counters && g.ws_tiles >= tiles * SK_SLOTS * 2) {
        sp = cus / tiles;
        if (sp > 16) sp = 16;
        if (sp > g.ws_tiles / (tiles * SK_SLOTS)) sp = g.ws_tiles / (tiles * SK_SLOTS);
        while (sp > 1 && nsl / sp < 16) --sp;
        if (sp < 1) sp = 1;
    }
    return sp > 1 || tiles * 2 >= cus ? (int)sp : 0;
}

template <int FMT>
hipError_t launch_skinny(const GemmProblem& g, hipStream_t s, int splits) {
    constexpr int R = 4;
    return splits > 1 ? launch_r<R, true, FMT>(g, s, splits) : launch_r<R, false, FMT>(g, s, 1);
}

template hipError_t launch_skinny<0>(const GemmProblem&, hipStream_t, int);
template hipError_t launch_skinny<1>(const GemmProblem&, hipStream_t, int);
template hipError_t launch_skinny<2>(const GemmProblem&, hipStream_t, int);
template hipError_t launch_skinny<3>(const GemmProblem&, hipStream_t, int);

}  // namespace fp8k
