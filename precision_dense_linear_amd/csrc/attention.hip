// FP8 multi-head attention for gfx950 ("Leveraging CUTLASS kernel naming in
// Triton for a 100 TFLOPS FP8 tensor-core speed-up in multi-head attention":
// the fp8_mha_kernel sketch -- Q K^T as an FP8 dot product, the softmax and
// the accumulation of V fused behind it -- with BLOCK_M = 128 query rows and
// BLOCK_N = 64 keys per step, its parameter list's values for a 4096-token,
// 32-head LLM).  Per head h and query i:
//
//   S[i, j] = (scale_q * scale_k * softmax_scale) * sum_d Q[i, d] K[j, d]
//   O[i, :] = scale_v * sum_j softmax_j(S[i, :]) V[j, :]
//
// over the visible keys (all, or causal: j <= i + seq_kv - seq_q).  Q, K, V
// are E4M3 codes widened exactly to BF16 for the matrix cores, so both
// products are exact and accumulate in FP32.  The softmax runs online over
// 64-key blocks in FP32: base-2 exponentials of the scaled score minus an
// offset (one FMA each), where the offset is the running max as of the last
// rescale.  A block is first computed with the current offsets and no block
// max; only when a lane's share of the block's row sum exceeds ATT_PMAX (or
// overflowed) -- or a query has no offset yet -- does it take the block
// max, move the offsets to the new maxima, rescale accumulator and row sum,
// and compute the block again.  Most blocks thus skip both the max and the
// rescale, and every unnormalised probability kept is at most ATT_PMAX.
// Each unnormalised probability is rounded to BF16 for the second product
// and the row sum adds the same rounded values; the output is divided by it
// at the end.
//
// Layout: Q [BH][seq_q][D], K and V [BH][seq_kv][D], O [BH][seq_q][D], D
// contiguous, D = 64 or 128.  A workgroup of 4 waves takes 128 queries of
// one head; wave w owns queries 32w .. 32w+31 and walks every key block:
//  * S^T = mfma(K fragment, Q fragment): lane l holds query l%32 and, per
//    32-key block, the 16 keys 8(r/4) + 4(l/32) + r%4 (r = 0..15), so the
//    row max and row sum of a query live in lanes l and l^32;
//  * O^T = mfma(V fragment, P fragment): P comes straight from the S^T
//    registers -- 16-key MFMA m of a 32-key block takes elements r = 8m ..
//    8m+7, i.e. keys 16m + {0..3, 8..11} + 4(l/32) -- and V is staged in LDS
//    with bits 2 and 3 of the key index swapped within each 16 rows, so the
//    transposing LDS read (8 consecutive rows of one column) hands lane group
//    g exactly those keys in that order;
//  * O^T's register layout is the GEMM epilogue's (a lane owns one query and
//    four consecutive d per group of four), so TileStore writes it.
// K and V stages go from global memory straight into LDS (3 buffers, two
// blocks of look-ahead).
#include "gemm_common.h"
#include "launch.h"

namespace fp8k {

namespace {

constexpr int ATT_BM = 128;   // queries per workgroup
constexpr int ATT_BN = 64;    // keys per step
constexpr int ATT_NBUF = 3;   // K/V stage buffers
constexpr float LOG2E = 1.4426950408889634f;
constexpr float ATT_PMAX = 65536.0f;   // bound on a lane's share of a block's row sum (so on each probability kept)

struct AttnArgs {
    const uint8_t* Q;
    const uint8_t* K;
    const uint8_t* V;
    const float* scale_q;
    const float* scale_k;
    const float* scale_v;
    void* O;
    int64_t seq_q, seq_kv;
    float softmax_scale;
    int32_t q_blocks;   // ceil(seq_q / 128)
    int32_t causal;
    int32_t out_f16;
};

// Chunk position of 16-byte chunk c of K-tile row r: rows sharing a 256-byte
// bank window get distinct masks, so the 16 rows one ds_read_b128 phase reads
// hit 16 distinct bank groups.
template <int D>
__device__ __forceinline__ int swz_k(int r, int c) {
    constexpr int RPW = 256 / D, CPR = D / 16;
    return c ^ ((r / RPW) % CPR);
}

// V-tile row of key k (and key of row k): bits 2 and 3 swapped.
__device__ __forceinline__ int v_row(int k) { return (k & ~12) | ((k & 4) << 1) | ((k & 8) >> 1); }

template <int D, bool BF16, bool CAUSAL, bool FASTQK>
__global__ void __launch_bounds__(256, 2) attention_kernel(AttnArgs p) {
    constexpr int TILE = ATT_BN * D;                // bytes of a K or V tile
    constexpr int STAGE = 2 * TILE;
    constexpr int DC = D / 32;                      // 32-wide d blocks; 16-byte chunks per lane group half
    constexpr int LOADS = TILE / 1024 / 4;          // loads per wave per tile
    using Store = TileStore<BF16, 1, DC>;
    constexpr int EPI = 4 * Store::LDS_BYTES;
    __shared__ __attribute__((aligned(1024))) uint8_t smem[ATT_NBUF * STAGE > EPI ? ATT_NBUF * STAGE : EPI];

    int bid = blockIdx.x;
    const int nblk = gridDim.x;
    if ((nblk & 7) == 0) bid = (bid & 7) * (nblk >> 3) + (bid >> 3);  // a head's query blocks on one XCD
    const int head = bid / p.q_blocks;
    // causal: a query block's work grows with its index, so the heaviest
    // blocks of a head are issued first and the light ones fill in behind
    const int qb = CAUSAL ? p.q_blocks - 1 - bid % p.q_blocks : bid % p.q_blocks;
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int h = lane >> 5;
    const int64_t Sq = p.seq_q, Skv = p.seq_kv;
    const int64_t q0 = (int64_t)qb * ATT_BM + wave * 32;      // this wave's first query
    const int64_t my_q = q0 + (lane & 31);
    const int64_t offs = Skv - Sq;                             // causal: key j visible to query i iff j <= i + offs

    // key blocks this workgroup visits (causal: up to its last query's keys)
    int64_t kv_end = Skv;
    if constexpr (CAUSAL) {
        const int64_t q_last = min<int64_t>((int64_t)qb * ATT_BM + ATT_BM - 1, Sq - 1);
        kv_end = max<int64_t>(0, min<int64_t>(Skv, q_last + offs + 1));
    }
    const int nkb = (int)((kv_end + ATT_BN - 1) / ATT_BN);

    const uint8_t* Kh = p.K + (int64_t)head * Skv * D;
    const uint8_t* Vh = p.V + (int64_t)head * Skv * D;

    // Q fragments: lane group g of the MFMA K slots takes d = (D/2) g + 8t ..
    // +7 at step t (the d order is the contraction's own; K is read the same
    // way), so a lane holds the D/2 contiguous bytes of its half of its row.
    // FASTQK: instruction m (K = 64) of a 32-key block takes d = 64 m + 32 g
    // .. +31 from lane group g, as raw codes (K read the same way).
    v8bf qf[FASTQK ? 1 : D / 16];
    v8i q8[D / 64];
    if constexpr (FASTQK) {
        const __amdgpu_buffer_rsrc_t rq = make_rsrc(p.Q + (int64_t)head * Sq * D, clamp_records(Sq * D));
#pragma unroll
        for (int m = 0; m < D / 64; ++m) {
            const uint32_t o = (uint32_t)(my_q * D + 64 * m + 32 * h);
            const v4i lo = __builtin_bit_cast(v4i, __builtin_amdgcn_raw_buffer_load_b128(rq, my_q < Sq ? o : OOB, 0, 0));
            const v4i hi = __builtin_bit_cast(v4i, __builtin_amdgcn_raw_buffer_load_b128(rq, my_q < Sq ? o + 16 : OOB, 0, 0));
            q8[m] = (v8i){lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
        }
    } else {
        v4i raw[DC];
        const __amdgpu_buffer_rsrc_t rq = make_rsrc(p.Q + (int64_t)head * Sq * D, clamp_records(Sq * D));
        const uint32_t qoff = (uint32_t)(my_q * D + (D / 2) * h);
#pragma unroll
        for (int u = 0; u < DC; ++u)
            raw[u] = __builtin_bit_cast(v4i, __builtin_amdgcn_raw_buffer_load_b128(rq, my_q < Sq ? qoff + 16 * u : OOB, 0, 0));
#pragma unroll
        for (int u = 0; u < DC; ++u) {
            qf[2 * u] = e4m3x8_to_bf16(raw[u][0], raw[u][1]);
            qf[2 * u + 1] = e4m3x8_to_bf16(raw[u][2], raw[u][3]);
        }
    }

    // Per-lane global offsets (within a 64-key block) and LDS slots of this
    // wave's stage loads: load i of K / V fills the 1 KiB slot (i*4 + wave).
    uint32_t koff[LOADS], voff[LOADS];
#pragma unroll
    for (int i = 0; i < LOADS; ++i) {
        const int o = (i * 4 + wave) * 1024 + lane * 16;
        const int r = o / D, pos = (o % D) / 16;
        koff[i] = (uint32_t)(r * D + (pos ^ (swz_k<D>(r, 0))) * 16);           // chunk c at position c ^ mask
        const int vr = v_row(r);                                                 // key held by V-tile row r
        voff[i] = (uint32_t)(vr * D + swz_b<D>(r, pos) * 16);                    // swz_b is its own inverse
    }
    const uint32_t lds0 = (uint32_t)(uintptr_t)smem;
    auto issue = [&](int kb) {
        const int64_t key0 = (int64_t)kb * ATT_BN;
        const int buf = kb % ATT_NBUF;
        const __amdgpu_buffer_rsrc_t rk = make_rsrc(Kh + key0 * D, clamp_records((Skv - key0) * D));
        const __amdgpu_buffer_rsrc_t rv = make_rsrc(Vh + key0 * D, clamp_records((Skv - key0) * D));
        const uint32_t base = lds0 + buf * STAGE;
#pragma unroll
        for (int i = 0; i < LOADS; ++i) {
            dma16(rk, __builtin_amdgcn_readfirstlane(base + (i * 4 + wave) * 1024), koff[i]);
            dma16(rv, __builtin_amdgcn_readfirstlane(base + TILE + (i * 4 + wave) * 1024), voff[i]);
        }
    };

    // LDS read offsets: K rows 32 kb + (l%32), chunk (D/32) g + u; V (mirror
    // of the GEMM's B operand) rows 32 kb + 16 m + 8 g + (l%16)/2, column
    // 32 ni + l%32 after the transpose.
    // (FASTQK: K rows 32 kb + (l%32), chunks 4 m + 2 g and 4 m + 2 g + 1 for
    // instruction m, the same d as the lane's Q bytes)
    int k_rd[2][DC];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int u = 0; u < DC; ++u) {
            const int r = kb * 32 + (lane & 31);
            const int c = FASTQK ? 4 * (u / 2) + 2 * h + (u % 2) : DC * h + u;
            k_rd[kb][u] = r * D + swz_k<D>(r, c) * 16;
        }
    int v_rd[2][2][DC];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int m = 0; m < 2; ++m)
#pragma unroll
            for (int ni = 0; ni < DC; ++ni) {
                const int col = ni * 32 + 16 * ((lane >> 4) & 1) + 8 * (lane & 1);
                const int kr = kb * 32 + 16 * m + 8 * h + ((lane & 15) >> 1);
                v_rd[kb][m][ni] = TILE + kr * D + swz_b<D>(kr, col >> 4) * 16 + (col & 15);
            }

    // score -> log2 units, kept positive so that a masked raw score of -inf
    // stays -inf: a negative product of scales is moved onto Q (an exact
    // sign flip of its codes), and one that underflowed to 0 becomes the
    // least normal float (every |score| is then below 2^-100, so each
    // exponential still rounds to 1)
    float c2 = (p.scale_q[0] * p.scale_k[0]) * (p.softmax_scale * LOG2E);
    if (c2 == 0.0f) c2 = 1.17549435e-38f;
    if (c2 < 0.0f) {
        c2 = -c2;
        if constexpr (FASTQK) {
#pragma unroll
            for (int m = 0; m < D / 64; ++m) q8[m] ^= (int)0x80808080;
        } else {
#pragma unroll
            for (int t = 0; t < D / 16; ++t) qf[t] = __builtin_bit_cast(v8bf, __builtin_bit_cast(v4i, qf[t]) ^ (int)0x80008000);
        }
    }
    v16f acc[1][DC];
#pragma unroll
    for (int ni = 0; ni < DC; ++ni)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[0][ni][r] = 0.0f;
    float m_off = -__builtin_inff();   // exponent offset (log2 units; -inf: no visible key yet)
    float l_run = 0.0f;   // this lane's share of the row sum (its 32 of every 64 keys)

#pragma unroll
    for (int kb = 0; kb < ATT_NBUF - 1; ++kb)
        if (kb < nkb) issue(kb);

    // One key block; its stage buffer BUF = kb % ATT_NBUF is a compile-time
    // constant, so every LDS read address is a per-lane register plus an
    // immediate offset.
    auto step = [&](const int kb, auto buf_c) {
        constexpr int BUF = decltype(buf_c)::value;
        // the loads of block kb have landed (block kb+1's may still fly),
        // and every wave is done with the buffer block kb+2 refills
        if (kb + 1 < nkb) wait_vmcnt_lds<2 * LOADS>();
        else wait_vmcnt_lds<0>();
        __syncthreads();
        if (kb + ATT_NBUF - 1 < nkb) issue(kb + ATT_NBUF - 1);
        const lds_u8* st = (const lds_u8*)smem + BUF * STAGE;
        // the block's V fragments, read ahead of the first product and the
        // softmax so that the LDS latency hides behind them
        v2i vf[2][2][DC];
#pragma unroll
        for (int hb = 0; hb < 2; ++hb)
#pragma unroll
            for (int mm = 0; mm < 2; ++mm)
#pragma unroll
                for (int ni = 0; ni < DC; ++ni) vf[hb][mm][ni] = lds_read_tr8(st + v_rd[hb][mm][ni]);

        // S^T for the block's two 32-key halves
        v16f s[2];
#pragma unroll
        for (int hb = 0; hb < 2; ++hb) {
#pragma unroll
            for (int r = 0; r < 16; ++r) s[hb][r] = 0.0f;
            if constexpr (FASTQK) {
#pragma unroll
                for (int m = 0; m < D / 64; ++m) {
                    const v4i lo = lds_read16(st + k_rd[hb][2 * m]), hi = lds_read16(st + k_rd[hb][2 * m + 1]);
                    const v8i k8 = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
                    s[hb] = mfma_32x32x64_f8<0, 0>(k8, q8[m], s[hb]);
                }
            } else {
#pragma unroll
                for (int u = 0; u < DC; ++u) {
                    const v4i kr = lds_read16(st + k_rd[hb][u]);
                    s[hb] = mfma_32x32x16_bf16(e4m3x8_to_bf16(kr[0], kr[1]), qf[2 * u], s[hb]);
                    s[hb] = mfma_32x32x16_bf16(e4m3x8_to_bf16(kr[2], kr[3]), qf[2 * u + 1], s[hb]);
                }
            }
        }
        // Keys past seq_kv (zero-filled) and, causal, past the query's last
        // visible key get the raw score -inf (c2 > 0 keeps it -inf in the
        // exponent); only edge blocks evaluate the mask.
        const int64_t key0 = (int64_t)kb * ATT_BN;
        if (key0 + ATT_BN > Skv || (CAUSAL && key0 + ATT_BN - 1 > q0 + offs)) {
            // keys 0 .. lim-1 of the block are visible to this lane's query;
            // element r of half hb holds key 32 hb + 8 (r/4) + 4 h + r%4
            int64_t l = Skv - key0;
            if constexpr (CAUSAL) l = min<int64_t>(l, my_q + offs + 1 - key0);
            const int lim = (int)max<int64_t>(0, min<int64_t>(ATT_BN, l)) - 4 * h;
#pragma unroll
            for (int hb = 0; hb < 2; ++hb)
#pragma unroll
                for (int r = 0; r < 16; ++r)
                    if (hb * 32 + 8 * (r >> 2) + (r & 3) >= lim) s[hb][r] = -__builtin_inff();
        }
        // probabilities exp2(c2 s - m_off), rounded to BF16 in pairs for the
        // second product, and this lane's share of the row sum over the same
        // rounded values (v_dot2c_f32_bf16 against ones)
        const v2bf ones = {(__bf16)1.0f, (__bf16)1.0f};
        v8bf pf[2][2];
        auto probs = [&](const float nb) {
            float ls[4] = {0.0f, 0.0f, 0.0f, 0.0f};   // four independent partial sums
#pragma unroll
            for (int hb = 0; hb < 2; ++hb)
#pragma unroll
                for (int mm = 0; mm < 2; ++mm)
#pragma unroll
                    for (int e = 0; e < 8; e += 2) {
                        const int r = 8 * mm + e;
                        const v2bf pr = {(__bf16)__builtin_amdgcn_exp2f(fmaf(s[hb][r], c2, nb)),
                                         (__bf16)__builtin_amdgcn_exp2f(fmaf(s[hb][r + 1], c2, nb))};
                        pf[hb][mm][e] = pr[0];
                        pf[hb][mm][e + 1] = pr[1];
                        ls[e / 2] = __builtin_amdgcn_fdot2_f32_bf16(pr, ones, ls[e / 2], false);
                    }
            return (ls[0] + ls[1]) + (ls[2] + ls[3]);
        };
        // First with the current offsets and no block max: kept when every
        // lane's share of the sum is at most ATT_PMAX, so that no
        // probability exceeds it (an overflow to inf fails the test too).
        bool remax = __ballot(m_off == -__builtin_inff()) != 0;
        float lsum = 0.0f;
        if (!remax) {
            lsum = probs(-m_off);
            remax = __ballot(!(lsum <= ATT_PMAX)) != 0;
        }
        if (remax) {
            // block max of the raw scores (c2 > 0: the max of the scaled
            // ones), as four independent chains; every query's offset moves
            // to its max so far, and the block is computed again
            float m4[4] = {-__builtin_inff(), -__builtin_inff(), -__builtin_inff(), -__builtin_inff()};
#pragma unroll
            for (int hb = 0; hb < 2; ++hb)
#pragma unroll
                for (int r = 0; r < 16; ++r) m4[r & 3] = fmaxf(m4[r & 3], s[hb][r]);
            float mx = fmaxf(fmaxf(m4[0], m4[1]), fmaxf(m4[2], m4[3]));
            mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
            const float mxs = mx == -__builtin_inff() ? mx : mx * c2;   // log2 units
            const float m_new = fmaxf(m_off, mxs);
            // (v_exp_f32 itself: results below 2^-126, far under any weight
            // that matters, flush to zero)
            const float alpha = m_off == -__builtin_inff() ? 0.0f : __builtin_amdgcn_exp2f(m_off - m_new);
            m_off = m_new;
            l_run *= alpha;
#pragma unroll
            for (int ni = 0; ni < DC; ++ni)
#pragma unroll
                for (int r = 0; r < 16; ++r) acc[0][ni][r] *= alpha;
            lsum = probs(m_off == -__builtin_inff() ? 0.0f : -m_off);
        }
        l_run += lsum;
        // O^T += V^T P^T over the block's four 16-key groups
#pragma unroll
        for (int hb = 0; hb < 2; ++hb)
#pragma unroll
            for (int mm = 0; mm < 2; ++mm)
#pragma unroll
                for (int ni = 0; ni < DC; ++ni) {
                    const v2i vr = vf[hb][mm][ni];
                    acc[0][ni] = mfma_32x32x16_bf16(e4m3x8_to_bf16(vr[0], vr[1]), pf[hb][mm], acc[0][ni]);
                }
    };
    static_assert(ATT_NBUF == 3, "the key-block loop is unrolled over the stage buffers");
    for (int kb = 0; kb < nkb; kb += ATT_NBUF) {
        step(kb, std::integral_constant<int, 0>{});
        if (kb + 1 < nkb) step(kb + 1, std::integral_constant<int, 1>{});
        if (kb + 2 < nkb) step(kb + 2, std::integral_constant<int, 2>{});
    }
    wait_vmcnt<0>();

    // O = scale_v * acc / l (0 for a query that saw no key)
    const float l = l_run + __shfl_xor(l_run, 32, 64);
    const float inv = l > 0.0f ? 1.0f / l : 0.0f;
    __syncthreads();   // every wave is done with the stage buffers
    lds_u8* scratch = (lds_u8*)smem + wave * Store::LDS_BYTES;
    Store::run(p.O, acc, inv, p.scale_v[0], q0, 0, Sq, D, (int64_t)head * Sq, lane, scratch, p.out_f16 != 0);
}

template <int D, bool BF16, bool FASTQK>
hipError_t launch_d(const AttnArgs& a, int64_t heads, hipStream_t s) {
    const int64_t blocks = heads * a.q_blocks;
    if (blocks == 0) return hipSuccess;
    if (a.causal)
        hipLaunchKernelGGL((attention_kernel<D, BF16, true, FASTQK>), dim3((unsigned)blocks), dim3(256), 0, s, a);
    else hipLaunchKernelGGL((attention_kernel<D, BF16, false, FASTQK>), dim3((unsigned)blocks), dim3(256), 0, s, a);
    return hipGetLastError();
}

template <bool FASTQK>
hipError_t launch_fast(const AttnArgs& a, int64_t heads, int64_t head_dim, bool two_byte, hipStream_t s) {
    if (head_dim == 64)
        return two_byte ? launch_d<64, true, FASTQK>(a, heads, s) : launch_d<64, false, FASTQK>(a, heads, s);
    return two_byte ? launch_d<128, true, FASTQK>(a, heads, s) : launch_d<128, false, FASTQK>(a, heads, s);
}

}  // namespace

hipError_t launch_attention(const AttnProblem& g, hipStream_t s) {
    AttnArgs a;
    a.Q = g.Q;
    a.K = g.K;
    a.V = g.V;
    a.scale_q = g.scale_q;
    a.scale_k = g.scale_k;
    a.scale_v = g.scale_v;
    a.O = g.O;
    a.seq_q = g.seq_q;
    a.seq_kv = g.seq_kv;
    a.softmax_scale = g.softmax_scale;
    a.q_blocks = (int32_t)((g.seq_q + ATT_BM - 1) / ATT_BM);
    a.causal = g.causal;
    a.out_f16 = g.out == 2;
    const bool two_byte = g.out != 0;
    return g.fast_qk ? launch_fast<true>(a, g.heads, g.head_dim, two_byte, s)
                     : launch_fast<false>(a, g.heads, g.head_dim, two_byte, s);
}

}  // namespace fp8k
