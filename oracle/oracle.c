/*
 * CPU oracle for the scaled FP8 (OCP E4M3) GEMM.  TEST INFRASTRUCTURE ONLY:
 * nothing in the product library links, includes or calls this file; only the
 * tests, the smoke check and the benchmark's CPU-baseline leg load it.
 *
 * It computes, slowly and exactly, what the pages define:
 *   "Triton FP8 GEMM via CUTLASS naming" page (blog.hotdry.top, 2025-10-03),
 *   kernel section and its parameter list: FP8 e4m3fn inputs with range +-448,
 *   an FP32 accumulator, per-tensor scales applied as acc*scale_a*scale_b,
 *   output dequantised to FP32 or BF16; the risk paragraph asks for per-tensor
 *   scaling so that values stay inside +-448.
 *   "FP8 GEMM in JAX with Triton for Blackwell" page (2025-10-07), parameter
 *   paragraph: 32x32-block scale granularity ("microscaling"); MoE paragraph:
 *   the grouped GEMM over experts; opening section and kernel sketch: the
 *   E5M2 format beside E4M3, and a float16 store of the accumulator (the
 *   operand-format and FP16-output variants at the end of this file).
 * Readings where the pages are silent (scale = amax/448, round-to-nearest-even
 * with saturation, division rather than reciprocal, scale applied once after
 * the sum) are listed in the design notes; each function states the one it
 * uses.
 *
 * Exactness argument used throughout: every finite E4M3 value is an integer
 * multiple of 2^-9 with magnitude <= 448 = 229376 * 2^-9.  A product of two
 * codes is an integer multiple of 2^-18 below 2^36 * 2^-18, so any sum of up
 * to 171196 such products is an integer multiple of 2^-18 below 2^53 * 2^-18:
 * FP64 represents every partial sum exactly and the order of summation does
 * not matter.  The per-tensor results below are therefore the exact sums,
 * rounded once.
 *
 * Build: gcc -O2 -fopenmp -ffp-contract=off -shared -fPIC oracle.c -o liboracle.so
 * (no -ffast-math: the quantizer relies on IEEE binary32 division).
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

/* ------------------------------------------------------------------------ */
/* E4M3 decode by table.                                                     */
/* Magnitude of each code 0x00..0x7E in units of 2^-9 (OCP FP8 E4M3 "fn":    */
/* exponent bias 7, three mantissa bits, exponent field 0 holds subnormals,  */
/* exponent and mantissa all ones (0x7F) is NaN, no infinities).  Codes with */
/* bit 7 set are the negatives.  Typed out as a table, one row per exponent  */
/* field value; the tests check it against the closed form and against       */
/* torch's float8_e4m3fn decode.                                              */
/* ------------------------------------------------------------------------ */
static const int32_t E4M3_MAG_X512[127] = {
    0,      1,      2,      3,      4,      5,      6,      7,       /* e=0  */
    8,      9,      10,     11,     12,     13,     14,     15,      /* e=1  */
    16,     18,     20,     22,     24,     26,     28,     30,      /* e=2  */
    32,     36,     40,     44,     48,     52,     56,     60,      /* e=3  */
    64,     72,     80,     88,     96,     104,    112,    120,     /* e=4  */
    128,    144,    160,    176,    192,    208,    224,    240,     /* e=5  */
    256,    288,    320,    352,    384,    416,    448,    480,     /* e=6  */
    512,    576,    640,    704,    768,    832,    896,    960,     /* e=7  */
    1024,   1152,   1280,   1408,   1536,   1664,   1792,   1920,    /* e=8  */
    2048,   2304,   2560,   2816,   3072,   3328,   3584,   3840,    /* e=9  */
    4096,   4608,   5120,   5632,   6144,   6656,   7168,   7680,    /* e=10 */
    8192,   9216,   10240,  11264,  12288,  13312,  14336,  15360,   /* e=11 */
    16384,  18432,  20480,  22528,  24576,  26624,  28672,  30720,   /* e=12 */
    32768,  36864,  40960,  45056,  49152,  53248,  57344,  61440,   /* e=13 */
    65536,  73728,  81920,  90112,  98304,  106496, 114688, 122880,  /* e=14 */
    131072, 147456, 163840, 180224, 196608, 212992, 229376           /* e=15 */
};

/* Signed value of a code in units of 2^-9; NaN codes report 0 and *is_nan. */
static int32_t e4m3_x512(uint8_t c, int* is_nan) {
    uint8_t m = c & 0x7F;
    if (m == 0x7F) { if (is_nan) *is_nan = 1; return 0; }
    if (is_nan) *is_nan = 0;
    return (c & 0x80) ? -E4M3_MAG_X512[m] : E4M3_MAG_X512[m];
}

/* Decoded value as double (exact); NaN codes decode to NaN. */
double orc_e4m3_decode(uint8_t c) {
    int nan_;
    int32_t v = e4m3_x512(c, &nan_);
    if (nan_) return NAN;
    if (v == 0) return (c & 0x80) ? -0.0 : 0.0;
    return (double)v / 512.0;
}

void orc_e4m3_table(double* out256) {
    for (int c = 0; c < 256; c++) out256[c] = orc_e4m3_decode((uint8_t)c);
}

/* ------------------------------------------------------------------------ */
/* FP32 -> E4M3, round to nearest (ties to the even code), saturating.       */
/* The plain definition: pick the finite E4M3 value nearest to v; where two  */
/* are equally near, the one whose code is even (mantissa LSB 0); anything   */
/* above 448 in magnitude becomes +-448 (saturation, as the pages ask for    */
/* values to stay within +-448).  Search is a binary search over the sorted  */
/* magnitude table, comparisons done exactly in double.  The sign is kept,   */
/* also for results that round to zero.  NaN maps to the NaN code.           */
/* ------------------------------------------------------------------------ */
uint8_t orc_e4m3_rne_sat(float v) {
    if (isnan(v)) return signbit(v) ? 0xFF : 0x7F;
    uint8_t sign = signbit(v) ? 0x80 : 0x00;
    double a = fabs((double)v) * 512.0;  /* magnitude in units of 2^-9, exact */
    if (a >= (double)E4M3_MAG_X512[126]) return sign | 0x7E;
    /* largest code lo with mag[lo] <= a (mag[0] = 0 <= a always) */
    int lo = 0, hi = 126;
    while (hi - lo > 1) {
        int mid = (lo + hi) / 2;
        if ((double)E4M3_MAG_X512[mid] <= a) lo = mid; else hi = mid;
    }
    if ((double)E4M3_MAG_X512[hi] <= a) lo = hi; /* only when a == mag[126], handled above */
    int up = lo + 1;
    double dlo = a - (double)E4M3_MAG_X512[lo];
    double dup = (double)E4M3_MAG_X512[up] - a;
    int pick;
    if (dlo < dup) pick = lo;
    else if (dup < dlo) pick = up;
    else pick = (lo % 2 == 0) ? lo : up;
    return sign | (uint8_t)pick;
}

/* amax = max |x_i|, exact comparisons; NaN inputs are outside the contract. */
float orc_amax(const float* x, int64_t n) {
    float m = 0.0f;
    for (int64_t i = 0; i < n; i++) {
        float a = fabsf(x[i]);
        if (a > m) m = a;
    }
    return m;
}

/* scale = amax / 448 as one IEEE binary32 division; an all-zero group gets 1. */
float orc_scale_from_amax(float amax) {
    if (amax == 0.0f) return 1.0f;
    volatile float d = 448.0f;   /* keep it a real binary32 division */
    return amax / d;
}

/* q_i = E4M3_RNE_SAT(fl32(x_i / scale)): the quotient is rounded to binary32
 * first (what a binary32 value handed to an FP8 convert is), then to E4M3. */
void orc_quantize_with_scale(const float* x, int64_t n, float scale, uint8_t* q) {
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < n; i++) {
        volatile float quot = x[i] / scale;
        q[i] = orc_e4m3_rne_sat(quot);
    }
}

/* Per-tensor quantization: amax over all of x, scale, codes. */
void orc_quantize_pertensor(const float* x, int64_t n, uint8_t* q, float* scale_out, float* amax_out) {
    float amax = orc_amax(x, n);
    float s = orc_scale_from_amax(amax);
    orc_quantize_with_scale(x, n, s, q);
    *scale_out = s;
    *amax_out = amax;
}

/* 32x32-tile quantization of a rows x cols row-major matrix (rows, cols
 * multiples of 32): each tile gets its own amax and scale; scales are stored
 * row-major as [rows/32][cols/32]. */
void orc_quantize_blocked(const float* x, int64_t rows, int64_t cols, uint8_t* q, float* tile_scales) {
    int64_t tr = rows / 32, tc = cols / 32;
#pragma omp parallel for schedule(static)
    for (int64_t t = 0; t < tr * tc; t++) {
        int64_t bi = t / tc, bj = t % tc;
        float amax = 0.0f;
        for (int64_t i = 0; i < 32; i++)
            for (int64_t j = 0; j < 32; j++) {
                float a = fabsf(x[(bi * 32 + i) * cols + bj * 32 + j]);
                if (a > amax) amax = a;
            }
        float s = orc_scale_from_amax(amax);
        tile_scales[t] = s;
        for (int64_t i = 0; i < 32; i++)
            for (int64_t j = 0; j < 32; j++) {
                int64_t idx = (bi * 32 + i) * cols + bj * 32 + j;
                volatile float quot = x[idx] / s;
                q[idx] = orc_e4m3_rne_sat(quot);
            }
    }
}

/* Row-group quantization: group g is rows [off[g], off[g+1]) of a rows x cols
 * matrix; each group gets its own amax and scale (empty group: amax 0, scale 1). */
void orc_quantize_grouped(const float* x, int64_t rows, int64_t cols, const int32_t* off, int32_t G,
                          uint8_t* q, float* scales, float* amaxes) {
    (void)rows;
    for (int32_t g = 0; g < G; g++) {
        int64_t r0 = off[g], r1 = off[g + 1];
        float amax = (r1 > r0) ? orc_amax(x + r0 * cols, (r1 - r0) * cols) : 0.0f;
        float s = orc_scale_from_amax(amax);
        scales[g] = s;
        amaxes[g] = amax;
        if (r1 > r0) orc_quantize_with_scale(x + r0 * cols, (r1 - r0) * cols, s, q + r0 * cols);
    }
}

/* ------------------------------------------------------------------------ */
/* Exact rounding.  value = v * 2^e with v a signed 128-bit integer, rounded  */
/* once to nearest-even into a binary format with p significand bits and the */
/* binary32 exponent range (emin -126, emax 127): p = 24 gives FP32 bits,     */
/* p = 8 gives BF16 bits.  Overflow gives infinity, tiny values subnormals.   */
/* ------------------------------------------------------------------------ */
typedef __int128 i128;
typedef unsigned __int128 u128;

static int bitlen_u128(u128 u) {
    int n = 0;
    while (u) { n++; u >>= 1; }
    return n;
}

static uint32_t round_exact_bits(i128 v, int e, int p) {
    int signshift = 8 + p - 1;
    uint32_t sign = (v < 0) ? (1u << signshift) : 0u;
    u128 u = (v < 0) ? (u128)(-v) : (u128)v;
    if (u == 0) return sign;
    int nb = bitlen_u128(u);
    int E = nb - 1 + e;                       /* unbiased exponent of the leading bit */
    int lsb = (E < -126 ? -126 : E) - (p - 1); /* weight of the last kept bit */
    int shift = lsb - e;                      /* low bits of u to drop */
    u128 mant;
    if (shift <= 0) {
        mant = u << (-shift);                 /* exact, fewer than p bits in use */
    } else if (shift > nb) {
        mant = 0;                             /* below half of the smallest step */
    } else {
        u128 rem, half;
        if (shift == 128) { mant = 0; rem = u; half = (u128)1 << 127; }
        else { mant = u >> shift; rem = u & ((((u128)1) << shift) - 1); half = ((u128)1) << (shift - 1); }
        if (rem > half || (rem == half && (mant & 1))) mant += 1;
    }
    if (mant == ((u128)1 << p)) { mant >>= 1; lsb += 1; }
    if (mant >= ((u128)1 << (p - 1))) {
        int Ex = lsb + p - 1;
        int biased = Ex + 127;
        if (biased >= 255) return sign | (0xFFu << (p - 1));  /* infinity */
        return sign | ((uint32_t)biased << (p - 1)) | (uint32_t)(mant - ((u128)1 << (p - 1)));
    }
    return sign | (uint32_t)mant;             /* subnormal (biased exponent 0) */
}

/* Split a finite float into an integer significand and a power of two. */
static void split_f32(float f, int64_t* m, int* e) {
    uint32_t b;
    memcpy(&b, &f, 4);
    int be = (b >> 23) & 0xFF;
    int64_t frac = b & 0x7FFFFF;
    if (be == 0) { *m = frac; *e = -149; }
    else { *m = frac | 0x800000; *e = be - 150; }
    if (b >> 31) *m = -*m;
}

/* Exact value sa*sb*d*2^-18, rounded once; kind 0 -> FP32 bits, 1 -> BF16 bits. */
uint32_t orc_round_scaled(int64_t d, float sa, float sb, int kind) {
    int64_t ma, mb;
    int ea, eb;
    split_f32(sa, &ma, &ea);
    split_f32(sb, &mb, &eb);
    i128 v = (i128)ma * (i128)mb * (i128)d;
    return round_exact_bits(v, ea + eb - 18, kind == 0 ? 24 : 8);
}

/* A double rounded once to FP32 (kind 0) or BF16 (kind 1). */
uint32_t orc_round_f64(double x, int kind) {
    if (x == 0.0) return signbit(x) ? (kind == 0 ? 0x80000000u : 0x8000u) : 0u;
    int ex;
    double fr = frexp(x, &ex);                /* x = fr * 2^ex, 0.5 <= |fr| < 1 */
    int64_t m = (int64_t)ldexp(fr, 53);       /* exact: 53-bit integer significand */
    return round_exact_bits((i128)m, ex - 53, kind == 0 ? 24 : 8);
}

/* ------------------------------------------------------------------------ */
/* GEMMs.  A is M x K and B is K x N, both row-major E4M3 codes.             */
/* ------------------------------------------------------------------------ */

/* Exact D[i,j] = sum_k a[i,k]*b[k,j] in units of 2^-18, via the integer codes.
 * Plain triple loop; the reference for the faster FP64 path below. */
void orc_gemm_dot_i64(const uint8_t* A, const uint8_t* B, int64_t M, int64_t N, int64_t K, int64_t* D) {
    for (int64_t i = 0; i < M; i++)
        for (int64_t j = 0; j < N; j++) {
            int64_t s = 0;
            for (int64_t k = 0; k < K; k++)
                s += (int64_t)e4m3_x512(A[i * K + k], 0) * (int64_t)e4m3_x512(B[k * N + j], 0);
            D[i * N + j] = s;
        }
}

/* Exact sums for a set of rows of A (row indices rows[0..nr)), in FP64:
 * dot[r*N + j] = sum_k a*b and sabs[r*N + j] = sum_k |a*b| (both exact, see
 * the exactness argument at the top).  OpenMP over the selected rows; within a
 * row the k loop is the outer loop so that B is read row by row. */
void orc_gemm_rows_f64(const uint8_t* A, const uint8_t* B, int64_t N, int64_t K,
                       const int64_t* rows, int64_t nr, double* dot, double* sabs) {
    double tab[256];
    orc_e4m3_table(tab);
    for (int c = 0; c < 256; c++) if (isnan(tab[c])) tab[c] = 0.0;
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t r = 0; r < nr; r++) {
        const uint8_t* arow = A + rows[r] * K;
        double* drow = dot + r * N;
        double* srow = sabs ? sabs + r * N : 0;
        for (int64_t j = 0; j < N; j++) { drow[j] = 0.0; if (srow) srow[j] = 0.0; }
        for (int64_t k = 0; k < K; k++) {
            double a = tab[arow[k]];
            if (a == 0.0) continue;
            const uint8_t* brow = B + k * N;
            for (int64_t j = 0; j < N; j++) drow[j] += a * tab[brow[j]];
            if (srow) {
                double aa = fabs(a);
                for (int64_t j = 0; j < N; j++) srow[j] += aa * fabs(tab[brow[j]]);
            }
        }
    }
}

/* Per-tensor scaled GEMM on a set of rows: C[r, j] = round(sa*sb*sum_k a*b),
 * rounded once from the exact value (kind 0: FP32 bits in out32; kind 1: BF16
 * bits in out16).  Optionally also returns the exact value in FP64 (one
 * rounding of an exact number, relative error <= 2^-53) and sum_k |a*b|. */
void orc_gemm_rows(const uint8_t* A, const uint8_t* B, float sa, float sb, int64_t N, int64_t K,
                   const int64_t* rows, int64_t nr, int kind, uint32_t* out32, uint16_t* out16,
                   double* exact, double* sabs) {
    double* dot = exact;  /* caller buffer of nr*N doubles (required) */
    orc_gemm_rows_f64(A, B, N, K, rows, nr, dot, sabs);
#pragma omp parallel for schedule(static)
    for (int64_t t = 0; t < nr * N; t++) {
        int64_t d = (int64_t)ldexp(dot[t], 18);  /* exact integer in units of 2^-18 */
        uint32_t bits = orc_round_scaled(d, sa, sb, kind);
        if (kind == 0) out32[t] = bits; else out16[t] = (uint16_t)bits;
        dot[t] = (double)sa * (double)sb * dot[t];  /* sa*sb exact in FP64, one rounding */
    }
}

/* Sampled entries of the per-tensor GEMM: C[ii[s], jj[s]] for s < ns, each
 * computed one by one from its row of A and column of B. */
void orc_gemm_sampled(const uint8_t* A, const uint8_t* B, float sa, float sb, int64_t N, int64_t K,
                      const int64_t* ii, const int64_t* jj, int64_t ns, int kind,
                      uint32_t* out_bits, double* exact, double* sabs) {
    double tab[256];
    orc_e4m3_table(tab);
    for (int c = 0; c < 256; c++) if (isnan(tab[c])) tab[c] = 0.0;
#pragma omp parallel for schedule(static)
    for (int64_t s = 0; s < ns; s++) {
        double acc = 0.0, aacc = 0.0;
        for (int64_t k = 0; k < K; k++) {
            double p = tab[A[ii[s] * K + k]] * tab[B[k * N + jj[s]]];
            acc += p;
            aacc += fabs(p);
        }
        out_bits[s] = orc_round_scaled((int64_t)ldexp(acc, 18), sa, sb, kind);
        exact[s] = (double)sa * (double)sb * acc;
        sabs[s] = aacc;
    }
}

/* Block-scaled GEMM (32x32 tile scales), on a set of rows:
 *   P_kb[i,j] = sum_{k in [32kb, 32kb+32)} a[i,k]*b[k,j]          (exact)
 *   C[i,j]    = sum_kb s_a[i/32, kb] * s_b[kb, j/32] * P_kb[i,j]   (FP64)
 * then one rounding of the FP64 sum to FP32/BF16.  s_a is [M/32][K/32] and
 * s_b is [K/32][N/32], both row-major.  sabs gets sum_kb s_a*s_b*sum_k|a*b|.
 * exact (required, nr*N) receives the FP64 sum. */
void orc_gemm_blockscaled_rows(const uint8_t* A, const uint8_t* B, const float* s_a, const float* s_b,
                               int64_t N, int64_t K, const int64_t* rows, int64_t nr, int kind,
                               uint32_t* out32, uint16_t* out16, double* exact, double* sabs) {
    double tab[256];
    orc_e4m3_table(tab);
    for (int c = 0; c < 256; c++) if (isnan(tab[c])) tab[c] = 0.0;
    int64_t KB = K / 32, NB = N / 32;
#pragma omp parallel
    {
        double* part = (double*)malloc(sizeof(double) * (size_t)N);
        double* apart = (double*)malloc(sizeof(double) * (size_t)N);
#pragma omp for schedule(dynamic, 1)
        for (int64_t r = 0; r < nr; r++) {
            int64_t i = rows[r];
            double* crow = exact + r * N;
            double* srow = sabs ? sabs + r * N : 0;
            for (int64_t j = 0; j < N; j++) { crow[j] = 0.0; if (srow) srow[j] = 0.0; }
            for (int64_t kb = 0; kb < KB; kb++) {
                for (int64_t j = 0; j < N; j++) { part[j] = 0.0; apart[j] = 0.0; }
                for (int64_t k = kb * 32; k < kb * 32 + 32; k++) {
                    double a = tab[A[i * K + k]];
                    if (a == 0.0) continue;
                    const uint8_t* brow = B + k * N;
                    for (int64_t j = 0; j < N; j++) {
                        double p = a * tab[brow[j]];
                        part[j] += p;
                        apart[j] += fabs(p);
                    }
                }
                double sa = (double)s_a[(i / 32) * KB + kb];
                for (int64_t j = 0; j < N; j++) {
                    double sab = sa * (double)s_b[kb * NB + j / 32];  /* exact: 24+24 bits */
                    crow[j] += sab * part[j];
                    if (srow) srow[j] += sab * apart[j];
                }
            }
            for (int64_t j = 0; j < N; j++) {
                uint32_t bits = orc_round_f64(crow[j], kind);
                if (kind == 0) out32[r * N + j] = bits; else out16[r * N + j] = (uint16_t)bits;
            }
        }
        free(part);
        free(apart);
    }
}

/* Number of OpenMP threads the oracle's parallel loops use. */
int orc_num_threads(void) {
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

/* ======================================================================== */
/* Operand-format and output variants: OCP E5M2 codes, mixed E4M3 x E5M2     */
/* operands, FP16 output.  "FP8 GEMM in JAX with Triton for Blackwell" page:  */
/* its opening section names both FP8 formats (E4M3 and E5M2) for the matrix  */
/* cores, and its kernel sketch stores the FP32 accumulator as float16.       */
/* Readings (the page gives no more than that): an E5M2 tensor is scaled      */
/* exactly as an E4M3 one, with E5M2's largest finite value 57344 in place of */
/* 448 (scale = fl32(amax / 57344), RNE, saturating at +-57344); FP16 output  */
/* is the IEEE binary16 rounding of the exact scaled sum (nearest-even,       */
/* subnormals kept, overflow to infinity, as a plain cast does).              */
/* ======================================================================== */

/* E5M2 ("OCP FP8 E5M2"): sign bit, five exponent bits with bias 15, two
 * mantissa bits; exponent field 0 holds the subnormals f * 2^-16, field 31
 * holds +-Inf (mantissa 0) and NaN (mantissa 1..3).  Every finite value is an
 * integer multiple of 2^-16 no larger than 7 * 2^13 = 57344.  Magnitude of
 * code m (0 <= m <= 0x7B) in units of 2^-16, straight from the fields:
 * subnormal f, normal (4 + f) * 2^(e - 1). */
static int64_t e5m2_mag_x65536(int m) {
    int e = m >> 2, f = m & 3;
    return e == 0 ? (int64_t)f : (int64_t)(4 + f) << (e - 1);
}

/* Signed value of a code in units of 2^-16; Inf and NaN codes report 0 and
 * *special = 1 (Inf) or 2 (NaN). */
static int64_t e5m2_x65536(uint8_t c, int* special) {
    int m = c & 0x7F;
    if (m >= 0x7C) { if (special) *special = (m == 0x7C) ? 1 : 2; return 0; }
    if (special) *special = 0;
    int64_t v = e5m2_mag_x65536(m);
    return (c & 0x80) ? -v : v;
}

double orc_e5m2_decode(uint8_t c) {
    int sp;
    int64_t v = e5m2_x65536(c, &sp);
    if (sp == 1) return (c & 0x80) ? -INFINITY : INFINITY;
    if (sp == 2) return NAN;
    if (v == 0) return (c & 0x80) ? -0.0 : 0.0;
    return ldexp((double)v, -16);
}

void orc_e5m2_table(double* out256) {
    for (int c = 0; c < 256; c++) out256[c] = orc_e5m2_decode((uint8_t)c);
}

/* FP32 -> E5M2, round to nearest (ties to the even code), saturating at
 * +-57344 (Inf included); the sign is kept also when the result is zero; NaN
 * maps to a NaN code.  The nearest finite value is found by binary search
 * over the magnitudes of codes 0..0x7B, compared exactly in double. */
uint8_t orc_e5m2_rne_sat(float v) {
    if (isnan(v)) return signbit(v) ? 0xFF : 0x7F;
    uint8_t sign = signbit(v) ? 0x80 : 0x00;
    double a = ldexp(fabs((double)v), 16);      /* magnitude in units of 2^-16, exact */
    const int top = 0x7B;
    if (a >= (double)e5m2_mag_x65536(top)) return sign | (uint8_t)top;
    int lo = 0, hi = top;                          /* mag[lo] <= a < mag[hi] */
    while (hi - lo > 1) {
        int mid = (lo + hi) / 2;
        if ((double)e5m2_mag_x65536(mid) <= a) lo = mid; else hi = mid;
    }
    double dlo = a - (double)e5m2_mag_x65536(lo);
    double dup = (double)e5m2_mag_x65536(hi) - a;
    int pick;
    if (dlo < dup) pick = lo;
    else if (dup < dlo) pick = hi;
    else pick = (lo % 2 == 0) ? lo : hi;
    return sign | (uint8_t)pick;
}

/* Format codes: 0 = E4M3, 1 = E5M2. */
static uint8_t rne_sat_fmt(float v, int fmt) { return fmt ? orc_e5m2_rne_sat(v) : orc_e4m3_rne_sat(v); }
static float fmt_max(int fmt) { return fmt ? 57344.0f : 448.0f; }

/* scale = amax / (largest finite value of the format), one binary32
 * division; an all-zero group gets 1. */
float orc_scale_from_amax_fmt(float amax, int fmt) {
    if (amax == 0.0f) return 1.0f;
    volatile float d = fmt_max(fmt);
    return amax / d;
}

/* q_i = RNE_SAT_fmt(fl32(x_i / scale)). */
void orc_quantize_with_scale_fmt(const float* x, int64_t n, float scale, int fmt, uint8_t* q) {
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < n; i++) {
        volatile float quot = x[i] / scale;
        q[i] = rne_sat_fmt(quot, fmt);
    }
}

void orc_quantize_pertensor_fmt(const float* x, int64_t n, int fmt, uint8_t* q, float* scale_out, float* amax_out) {
    float amax = orc_amax(x, n);
    float s = orc_scale_from_amax_fmt(amax, fmt);
    orc_quantize_with_scale_fmt(x, n, s, fmt, q);
    *scale_out = s;
    *amax_out = amax;
}

void orc_quantize_grouped_fmt(const float* x, int64_t cols, const int32_t* off, int32_t G, int fmt,
                              uint8_t* q, float* scales, float* amaxes) {
    for (int32_t g = 0; g < G; g++) {
        int64_t r0 = off[g], r1 = off[g + 1];
        float amax = (r1 > r0) ? orc_amax(x + r0 * cols, (r1 - r0) * cols) : 0.0f;
        float s = orc_scale_from_amax_fmt(amax, fmt);
        scales[g] = s;
        amaxes[g] = amax;
        if (r1 > r0) orc_quantize_with_scale_fmt(x + r0 * cols, (r1 - r0) * cols, s, fmt, q + r0 * cols);
    }
}

/* ------------------------------------------------------------------------ */
/* Exact rounding to an IEEE binary format with p significand bits (hidden   */
/* bit included) and an exponent field of `ebits` bits: value = v * 2^e,     */
/* v a signed 128-bit integer, rounded once to nearest-even; exponent bias   */
/* 2^(ebits-1) - 1, subnormals below 2^(1 - bias), infinity on overflow.     */
/* kind 0: binary32 (p 24, 8 bits), 1: bfloat16 (p 8, 8 bits), 2: binary16  */
/* (p 11, 5 bits).  Returns the bit pattern.                                 */
/* ------------------------------------------------------------------------ */
static uint32_t round_ieee(i128 v, int e, int p, int ebits) {
    const int bias = (1 << (ebits - 1)) - 1;
    const int emin = 1 - bias;
    const uint32_t sign = (v < 0) ? (1u << (ebits + p - 1)) : 0u;
    u128 u = (v < 0) ? (u128)(-v) : (u128)v;
    if (u == 0) return sign;
    const int nb = bitlen_u128(u);
    const int E = nb - 1 + e;                          /* exponent of the leading bit */
    int lsb = (E < emin ? emin : E) - (p - 1);         /* weight of the last kept bit */
    const int drop = lsb - e;                          /* low bits of u to drop */
    u128 mant;
    if (drop <= 0) {
        mant = u << (-drop);
    } else if (drop > nb) {
        mant = 0;                                      /* below half the smallest step */
    } else {
        u128 half = (u128)1 << (drop - 1);
        u128 rem = (drop == 128) ? u : (u & (((u128)1 << drop) - 1));
        mant = (drop == 128) ? 0 : (u >> drop);
        if (rem > half || (rem == half && (mant & 1))) mant += 1;
    }
    if (mant == ((u128)1 << p)) { mant >>= 1; lsb += 1; }
    if (mant >= ((u128)1 << (p - 1))) {                /* normal */
        const int biased = lsb + p - 1 + bias;
        if (biased >= (1 << ebits) - 1) return sign | (((1u << ebits) - 1) << (p - 1));
        return sign | ((uint32_t)biased << (p - 1)) | (uint32_t)(mant - ((u128)1 << (p - 1)));
    }
    return sign | (uint32_t)mant;                      /* subnormal */
}

static void kind_format(int kind, int* p, int* ebits) {
    if (kind == 0) { *p = 24; *ebits = 8; }
    else if (kind == 1) { *p = 8; *ebits = 8; }
    else { *p = 11; *ebits = 5; }
}

/* A double rounded once to binary32 / bfloat16 / binary16 (kind 0 / 1 / 2). */
uint32_t orc_round_ieee_f64(double x, int kind) {
    int p, eb;
    kind_format(kind, &p, &eb);
    if (x == 0.0) return signbit(x) ? (1u << (eb + p - 1)) : 0u;
    int ex;
    double fr = frexp(x, &ex);
    int64_t m = (int64_t)ldexp(fr, 53);
    return round_ieee((i128)m, ex - 53, p, eb);
}

/* Value of a code in units of 2^-unit (unit 9 for E4M3, 16 for E5M2). */
static int64_t code_units(uint8_t c, int fmt) {
    return fmt ? e5m2_x65536(c, 0) : (int64_t)e4m3_x512(c, 0);
}

/* Per-tensor scaled GEMM with operand formats fa, fb (0 E4M3, 1 E5M2) on a
 * set of rows of A:
 *     D[r, j] = sum_k a[rows[r], k] * b[k, j]        exact, as a 128-bit
 *               integer in units of 2^-(ua + ub) (ua, ub = 9 or 16)
 *     C[r, j] = round_kind(sa * sb * D[r, j])        one rounding
 * out receives the bits (kind 0 FP32, 1 BF16, 2 FP16; one uint32 each),
 * exact the value sa*sb*D in FP64 and sabs sum_k |a*b| (unscaled, FP64).
 * Returns 0, or -1 if a sum is too large for the 128-bit scaled product (the
 * products and K at which that can happen are far beyond the workloads). */
int orc_gemm_rows_fmt(const uint8_t* A, const uint8_t* B, int fa, int fb, float sa, float sb,
                      int64_t N, int64_t K, const int64_t* rows, int64_t nr, int kind,
                      uint32_t* out, double* exact, double* sabs) {
    const int ua = fa ? 16 : 9, ub = fb ? 16 : 9;
    int64_t ma, mb;
    int ea, eb;
    split_f32(sa, &ma, &ea);
    split_f32(sb, &mb, &eb);
    const int mbits = bitlen_u128((u128)(ma < 0 ? -ma : ma)) + bitlen_u128((u128)(mb < 0 ? -mb : mb));
    const double sab_scale = ldexp(1.0, -(ua + ub));
    int p, ebits;
    kind_format(kind, &p, &ebits);
    int status = 0;
#pragma omp parallel
    {
        i128* acc = (i128*)malloc(sizeof(i128) * (size_t)(N > 0 ? N : 1));
        double* aacc = (double*)malloc(sizeof(double) * (size_t)(N > 0 ? N : 1));
#pragma omp for schedule(dynamic, 1)
        for (int64_t r = 0; r < nr; r++) {
            const uint8_t* arow = A + rows[r] * K;
            for (int64_t j = 0; j < N; j++) { acc[j] = 0; aacc[j] = 0.0; }
            for (int64_t k = 0; k < K; k++) {
                const int64_t a = code_units(arow[k], fa);
                if (a == 0) continue;
                const uint8_t* brow = B + k * N;
                for (int64_t j = 0; j < N; j++) {
                    const i128 prod = (i128)a * (i128)code_units(brow[j], fb);
                    acc[j] += prod;
                    aacc[j] += fabs((double)prod);
                }
            }
            for (int64_t j = 0; j < N; j++) {
                const i128 d = acc[j];
                const int dbits = bitlen_u128((u128)(d < 0 ? -d : d));
                if (dbits + mbits > 126) {
#pragma omp atomic write
                    status = -1;
                    out[r * N + j] = 0;
                } else {
                    out[r * N + j] = round_ieee((i128)ma * (i128)mb * d, ea + eb - (ua + ub), p, ebits);
                }
                exact[r * N + j] = (double)sa * (double)sb * ((double)d * sab_scale);
                sabs[r * N + j] = aacc[j] * sab_scale;
            }
        }
        free(acc);
        free(aacc);
    }
    return status;
}

/* ======================================================================== */
/* Block-scale granularity as a parameter.  "FP8 GEMM in JAX with Triton for  */
/* Blackwell": the parameter paragraph sets the scale granularity to 32x32    */
/* blocks; its monitoring paragraph names 64x64 as the coarser granularity to */
/* move to when accuracy suffers.  Both are T x T tiles of A (rows x K) and   */
/* of B (K x columns), T = 32 or 64, each quantized with its own              */
/* fl32(tile_amax / 448).                                                      */
/* ======================================================================== */

/* T x T tile quantization (rows, cols multiples of T); scales row-major as
 * [rows/T][cols/T]. */
void orc_quantize_blocked_t(const float* x, int64_t rows, int64_t cols, int T, uint8_t* q, float* tile_scales) {
    int64_t tr = rows / T, tc = cols / T;
#pragma omp parallel for schedule(static)
    for (int64_t t = 0; t < tr * tc; t++) {
        int64_t bi = t / tc, bj = t % tc;
        float amax = 0.0f;
        for (int64_t i = 0; i < T; i++)
            for (int64_t j = 0; j < T; j++) {
                float a = fabsf(x[(bi * T + i) * cols + bj * T + j]);
                if (a > amax) amax = a;
            }
        float s = orc_scale_from_amax(amax);
        tile_scales[t] = s;
        for (int64_t i = 0; i < T; i++)
            for (int64_t j = 0; j < T; j++) {
                int64_t idx = (bi * T + i) * cols + bj * T + j;
                volatile float quot = x[idx] / s;
                q[idx] = orc_e4m3_rne_sat(quot);
            }
    }
}

/* Block-scaled GEMM with T-deep K blocks and T x T scale tiles:
 *   P_kb[i,j] = sum_{k in [T*kb, T*kb + T)} a[i,k]*b[k,j]          (exact)
 *   C[i,j]    = sum_kb s_a[i/T, kb] * s_b[kb, j/T] * P_kb[i,j]     (FP64)
 * rounded once to FP32 / BF16 / FP16 (kind 0 / 1 / 2; one uint32 of bits per
 * output).  exact receives the FP64 sum, sabs sum_kb s_a*s_b*sum_k |a*b|. */
void orc_gemm_blockscaled_rows_t(const uint8_t* A, const uint8_t* B, const float* s_a, const float* s_b,
                                 int64_t N, int64_t K, int T, const int64_t* rows, int64_t nr, int kind,
                                 uint32_t* out, double* exact, double* sabs) {
    double tab[256];
    orc_e4m3_table(tab);
    for (int c = 0; c < 256; c++) if (isnan(tab[c])) tab[c] = 0.0;
    int64_t KB = K / T, NBT = N / T;
#pragma omp parallel
    {
        double* part = (double*)malloc(sizeof(double) * (size_t)(N > 0 ? N : 1));
        double* apart = (double*)malloc(sizeof(double) * (size_t)(N > 0 ? N : 1));
#pragma omp for schedule(dynamic, 1)
        for (int64_t r = 0; r < nr; r++) {
            int64_t i = rows[r];
            double* crow = exact + r * N;
            double* srow = sabs + r * N;
            for (int64_t j = 0; j < N; j++) { crow[j] = 0.0; srow[j] = 0.0; }
            for (int64_t kb = 0; kb < KB; kb++) {
                for (int64_t j = 0; j < N; j++) { part[j] = 0.0; apart[j] = 0.0; }
                for (int64_t k = kb * T; k < kb * T + T; k++) {
                    double a = tab[A[i * K + k]];
                    if (a == 0.0) continue;
                    const uint8_t* brow = B + k * N;
                    for (int64_t j = 0; j < N; j++) {
                        double p = a * tab[brow[j]];
                        part[j] += p;
                        apart[j] += fabs(p);
                    }
                }
                double sa = (double)s_a[(i / T) * KB + kb];
                for (int64_t j = 0; j < N; j++) {
                    double sab = sa * (double)s_b[kb * NBT + j / T];
                    crow[j] += sab * part[j];
                    srow[j] += sab * apart[j];
                }
            }
            for (int64_t j = 0; j < N; j++) out[r * N + j] = orc_round_ieee_f64(crow[j], kind);
        }
        free(part);
        free(apart);
    }
}

/* ======================================================================== */
/* 32x32 block scales as powers of two (E8M0), applied by the matrix cores:  */
/* the microscaling of "FP8 GEMM in JAX with Triton for Blackwell"           */
/* (parameter paragraph: 32x32 scale blocks) with each scale an 8-bit        */
/* exponent, as the OCP microscaling formats store it.  Reading (the page    */
/* gives only the granularity): the shared exponent of a tile follows the    */
/* OCP MX conversion for an E4M3 element type -- e = floor(log2(amax)) - 8  */
/* (8: the largest E4M3 exponent), clamped to [-127, 127], stored as the     */
/* byte e + 127; the codes are RNE_SAT(fl32(x / 2^e)), saturating at +-448   */
/* (amax / 2^e lies in [256, 512)).  An all-zero tile stores e = 0 (127).    */
/* ======================================================================== */

/* Shared exponent of a tile from its amax (finite, >= 0). */
int orc_e8m0_exponent(float amax) {
    if (amax == 0.0f) return 0;
    int ex;
    frexp((double)amax, &ex);          /* amax = f * 2^ex, 0.5 <= f < 1: floor(log2 amax) = ex - 1 */
    int e = (ex - 1) - 8;
    if (e < -127) e = -127;
    if (e > 127) e = 127;
    return e;
}

/* 32x32 tiles (rows, cols multiples of 32): codes and one E8M0 byte per tile,
 * row-major [rows/32][cols/32]. */
void orc_quantize_blocked_e8m0(const float* x, int64_t rows, int64_t cols, uint8_t* q, uint8_t* scales) {
    int64_t tr = rows / 32, tc = cols / 32;
#pragma omp parallel for schedule(static)
    for (int64_t t = 0; t < tr * tc; t++) {
        int64_t bi = t / tc, bj = t % tc;
        float amax = 0.0f;
        for (int64_t i = 0; i < 32; i++)
            for (int64_t j = 0; j < 32; j++) {
                float a = fabsf(x[(bi * 32 + i) * cols + bj * 32 + j]);
                if (a > amax) amax = a;
            }
        int e = orc_e8m0_exponent(amax);
        scales[t] = (uint8_t)(e + 127);
        float X = ldexpf(1.0f, e);   /* 2^e: 2^-127 is a binary32 subnormal, still exact */
        for (int64_t i = 0; i < 32; i++)
            for (int64_t j = 0; j < 32; j++) {
                int64_t idx = (bi * 32 + i) * cols + bj * 32 + j;
                volatile float quot = x[idx] / X;
                q[idx] = orc_e4m3_rne_sat(quot);
            }
    }
}

/* GEMM with E8M0 tile scales on a set of rows:
 *   C[i,j] = sum_kb 2^(ea[i/32,kb] + eb[kb,j/32]) * sum_{k in block kb} a[i,k]*b[k,j]
 * (ea, eb = byte - 127); each block sum is exact and scaling by a power of two
 * is exact, the sum over blocks is taken in FP64, rounded once (kind 0 / 1 /
 * 2: FP32 / BF16 / FP16; one uint32 of bits per output).  exact receives the
 * FP64 sum, sabs sum_kb 2^(ea+eb) * sum_k |a*b|. */
void orc_gemm_blockscaled_e8m0_rows(const uint8_t* A, const uint8_t* B, const uint8_t* s_a, const uint8_t* s_b,
                                    int64_t N, int64_t K, const int64_t* rows, int64_t nr, int kind,
                                    uint32_t* out, double* exact, double* sabs) {
    double tab[256];
    orc_e4m3_table(tab);
    for (int c = 0; c < 256; c++) if (isnan(tab[c])) tab[c] = 0.0;
    int64_t KB = K / 32, NBT = N / 32;
#pragma omp parallel
    {
        double* part = (double*)malloc(sizeof(double) * (size_t)(N > 0 ? N : 1));
        double* apart = (double*)malloc(sizeof(double) * (size_t)(N > 0 ? N : 1));
#pragma omp for schedule(dynamic, 1)
        for (int64_t r = 0; r < nr; r++) {
            int64_t i = rows[r];
            double* crow = exact + r * N;
            double* srow = sabs + r * N;
            for (int64_t j = 0; j < N; j++) { crow[j] = 0.0; srow[j] = 0.0; }
            for (int64_t kb = 0; kb < KB; kb++) {
                for (int64_t j = 0; j < N; j++) { part[j] = 0.0; apart[j] = 0.0; }
                for (int64_t k = kb * 32; k < kb * 32 + 32; k++) {
                    double a = tab[A[i * K + k]];
                    if (a == 0.0) continue;
                    const uint8_t* brow = B + k * N;
                    for (int64_t j = 0; j < N; j++) {
                        double p = a * tab[brow[j]];
                        part[j] += p;
                        apart[j] += fabs(p);
                    }
                }
                int ea = (int)s_a[(i / 32) * KB + kb] - 127;
                for (int64_t j = 0; j < N; j++) {
                    int e = ea + (int)s_b[kb * NBT + j / 32] - 127;
                    crow[j] += ldexp(part[j], e);
                    srow[j] += ldexp(apart[j], e);
                }
            }
            for (int64_t j = 0; j < N; j++) out[r * N + j] = orc_round_ieee_f64(crow[j], kind);
        }
        free(part);
        free(apart);
    }
}

/* ======================================================================== */
/* 50% structured sparsity of the weights.  "FP8 GEMM in JAX with Triton    */
/* for Blackwell", opening section: the matrix cores' sparsity support and   */
/* about twice the efficiency at 50% weight sparsity.  Reading: the 2:4      */
/* pattern the matrix cores take -- in every group of 4 consecutive K of a   */
/* column of the weight matrix B (K x N) at most two entries are nonzero --  */
/* obtained by magnitude pruning before quantization: the two entries of     */
/* largest |w| are kept (ties: the lower k), the other two set to zero.  The */
/* pruned matrix is then quantized per tensor as any other, and the GEMM is  */
/* the plain GEMM with the pruned B (orc_gemm_rows).                          */
/* ======================================================================== */

/* The two kept positions (ascending) of one group of 4 values. */
static void keep_two(const float* g, int stride, int* p0, int* p1) {
    int best = 0;
    for (int q = 1; q < 4; q++) if (fabsf(g[q * stride]) > fabsf(g[best * stride])) best = q;
    int second = best == 0 ? 1 : 0;
    for (int q = 0; q < 4; q++)
        if (q != best && fabsf(g[q * stride]) > fabsf(g[second * stride])) second = q;
    /* ties: the lower index wins (strict comparisons keep the first maximum) */
    *p0 = best < second ? best : second;
    *p1 = best < second ? second : best;
}

/* out = w with the two smaller-magnitude entries of each group of 4 along K
 * set to zero (w: K x N row-major, K % 4 == 0). */
void orc_prune_2of4(const float* w, int64_t K, int64_t N, float* out) {
#pragma omp parallel for schedule(static)
    for (int64_t n = 0; n < N; n++)
        for (int64_t g = 0; g < K / 4; g++) {
            int p0, p1;
            keep_two(w + (4 * g) * N + n, (int)N, &p0, &p1);
            for (int q = 0; q < 4; q++) {
                float v = w[(4 * g + q) * N + n];
                out[(4 * g + q) * N + n] = (q == p0 || q == p1) ? v : 0.0f;
            }
        }
}

/* Compressed form of 2:4-sparse codes q (K x N, K % 32 == 0) for the sparse
 * matrix cores:
 *   vals[(2g + j) * N + n] = code of the j-th kept entry (ascending k) of
 *                            group g of column n;
 *   idx[kb * N + n]        = 32-bit word of K block kb (32 K, 8 groups,
 *                            16 kept entries): bits 2e .. 2e+1 hold the
 *                            position (0..3) within its group of entry e
 *                            (e = 2 * (g - 8 kb) + j).
 * Which two entries a group keeps: its nonzero codes, completed (when it has
 * fewer than two) by its lowest-k zero entries. */
void orc_compress_2of4(const uint8_t* q, int64_t K, int64_t N, uint8_t* vals, uint32_t* idx) {
#pragma omp parallel for schedule(static)
    for (int64_t n = 0; n < N; n++)
        for (int64_t kb = 0; kb < K / 32; kb++) {
            uint32_t word = 0;
            for (int gg = 0; gg < 8; gg++) {
                int64_t g = 8 * kb + gg;
                int pos[2], np = 0;
                for (int s = 0; s < 4 && np < 2; s++)
                    if ((q[(4 * g + s) * N + n] & 0x7F) != 0) pos[np++] = s;
                for (int s = 0; s < 4 && np < 2; s++) {
                    int taken = 0;
                    for (int t = 0; t < np; t++) taken |= pos[t] == s;
                    if (!taken && (q[(4 * g + s) * N + n] & 0x7F) == 0) pos[np++] = s;
                }
                if (pos[0] > pos[1]) { int t = pos[0]; pos[0] = pos[1]; pos[1] = t; }
                for (int j = 0; j < 2; j++) {
                    vals[(2 * g + j) * N + n] = q[(4 * g + pos[j]) * N + n];
                    word |= (uint32_t)pos[j] << (2 * (2 * gg + j));
                }
            }
            idx[kb * N + n] = word;
        }
}
