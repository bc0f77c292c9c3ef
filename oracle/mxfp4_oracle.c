/*
 * CPU oracle for the MXFP4 (bf16 A quantized on the fly) x MXFP4 B GEMM.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product path may link, load or
 * call this file; only the tests, the smoke check and the CPU-baseline leg of
 * the benchmark do.  It shares no source with the HIP library.
 *
 * It is deliberately plain and slow: every quantity is computed from its
 * definition with exact integer arithmetic where the definition is integer,
 * and in fp64 where it is real-valued (the GEMM also in the fp32 group
 * accumulation of the matrix unit).  Rows and output elements are
 * independent and are computed in parallel (OpenMP); no result depends on
 * the number of threads.
 *
 * Sources (three web pages, each a diff between two versions of a submission
 * to the "amd-mxfp4-mm" leaderboard; cited by submission number):
 *   [608632]  submission 608632 (hardware FP4 convert, "v7")
 *   [610679]  submission 610679 (constexpr-specialized kernels, "v13")
 *   [711914]  submission 711914 (three-path dispatch)
 *
 * Readings taken where the pages are silent or disagree are listed in the
 * repository's design notes; each function below names the one it uses.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

#define ORACLE_API __attribute__((visibility("default")))

/* ------------------------------------------------------------------------ */
/* e2m1 code -> value.                                                       */
/* Code layout [711914, _mxfp4_quant_tile: sign restored at bit 3; exponent  */
/* rebias from f32 to a 2-bit field with bias 1; one mantissa bit; largest   */
/* magnitude 6].  value = (-1)^s * (e == 0 ? m/2 : (1 + m/2) * 2^(e-1)).     */
/* ------------------------------------------------------------------------ */
ORACLE_API double oracle_e2m1_value(int code)
{
    int s = (code >> 3) & 1;
    int e = (code >> 1) & 3;
    int m = code & 1;
    double mag = (e == 0) ? 0.5 * m : (1.0 + 0.5 * m) * ldexp(1.0, e - 1);
    return s ? -mag : mag;
}

/* e8m0 byte -> value 2^(b-127).  Byte 255 is the NaN encoding and never
 * produced by the quantizer (see oracle_scale_byte). */
ORACLE_API double oracle_e8m0_value(int b)
{
    if (b == 255) return NAN;
    return ldexp(1.0, b - 127);
}

/* ------------------------------------------------------------------------ */
/* Block scale of one 32-element group.                                      */
/* [608632, _hw_mxfp4_quant_op, step 1] and [610679, same function]:         */
/*   amax = max |x| as f32; R = (bits(amax) + 0x200000) & 0xFF800000;        */
/*   E = biased exponent of R; scale byte = clamp(E - 2, 0, 254).            */
/* Reading: the integer path, not the log2 path of [711914] (they differ     */
/* for an all-zero group and depend on a cast there).                        */
/* Inputs are bf16 bits; |x| as f32 has bits (h & 0x7fff) << 16, and for     */
/* non-negative finite floats the bit pattern orders like the value.         */
/* ------------------------------------------------------------------------ */
ORACLE_API int oracle_scale_byte(const uint16_t *x, int n)
{
    uint32_t amax_bits = 0;
    for (int i = 0; i < n; i++) {
        uint32_t a = (uint32_t)(x[i] & 0x7FFF) << 16;
        if (a > amax_bits) amax_bits = a;
    }
    uint32_t r = (amax_bits + 0x00200000u) & 0xFF800000u;
    int E = (int)((r >> 23) & 0xFF);
    int s = E - 2;
    if (s < 0) s = 0;
    if (s > 254) s = 254;
    return s;
}

/* ------------------------------------------------------------------------ */
/* Element encoder, exact integer form.                                      */
/* The element x (bf16) is divided by the group scale 2^(s-127) and rounded  */
/* to the nearest e2m1 magnitude {0, .5, 1, 1.5, 2, 3, 4, 6}; a tie goes to   */
/* the even code; anything at or above 6 (after rounding) gives code 7; the  */
/* sign goes to bit 3 even when the magnitude rounds to zero.               */
/* [711914, _mxfp4_quant_tile: saturate / denormal / normal branches, RNE    */
/* correction, sign OR].  Reading: the division is exact (x is bf16 and the  */
/* scale a power of two), so the comparison below is exact.                  */
/*                                                                           */
/* |x| = S * 2^q with integer S < 256, so 4v = S * 2^(q + 129 - s) and the   */
/* decision midpoints between consecutive magnitudes, times 4, are           */
/* {1, 3, 5, 7, 10, 14, 20}.                                                 */
/* ------------------------------------------------------------------------ */
static int cmp_4v(uint32_t S, int sh, int64_t T)
{
    /* sign of S*2^sh - T, T >= 1 */
    if (S == 0) return -1;
    if (sh >= 0) {
        if (sh > 30) return 1;
        int64_t v = (int64_t)S << sh;
        return (v > T) - (v < T);
    }
    if (-sh > 40) return -1; /* S < 2^8, so S*2^sh < 2^-32 < 1 <= T */
    int64_t t = T << (-sh);
    int64_t v = (int64_t)S;
    return (v > t) - (v < t);
}

ORACLE_API int oracle_encode(uint16_t x, int s)
{
    static const int64_t mid4[7] = {1, 3, 5, 7, 10, 14, 20};
    int sign = (x >> 15) & 1;
    int e = (x >> 7) & 0xFF;
    uint32_t m = x & 0x7F;
    uint32_t S;
    int q;
    if (e == 0) { S = m; q = -133; }
    else { S = 128 + m; q = e - 134; }
    int sh = q + 129 - s;
    int mag = 0;
    for (int c = 0; c < 7; c++) {
        int d = cmp_4v(S, sh, mid4[c]);
        if (d > 0) { mag = c + 1; continue; }
        if (d == 0) mag = (c % 2 == 0) ? c : c + 1; /* tie -> even code */
        break;
    }
    return (sign << 3) | mag;
}

/* ------------------------------------------------------------------------ */
/* Element encoder, second formulation: a nearest-value search.              */
/* The same rule as oracle_encode, taken literally: v = |x| * 2^(127-s) in   */
/* fp64 (exact: a bf16 value times a power of two within fp64's range),      */
/* then the e2m1 magnitude at the least distance from v; when two are at the */
/* same distance the even code wins; the sign goes to bit 3.  v is first     */
/* capped at 8: every v >= 7 is nearest to 6 (code 7), and the cap keeps the */
/* distances exact for huge v (where v - 4 and v - 6 would round to one      */
/* double and fake a tie).  It shares nothing with oracle_encode but the     */
/* magnitude table, and the tests require the two to agree on every input.   */
/* ------------------------------------------------------------------------ */
ORACLE_API int oracle_encode_nearest(uint16_t x, int s)
{
    static const double mags[8] = {0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0};
    int sign = (x >> 15) & 1;
    int e = (x >> 7) & 0xFF;
    int m = x & 0x7F;
    double ax = (e == 0) ? ldexp((double)m, -133) : ldexp((double)(128 + m), e - 134);
    double v = ldexp(ax, 127 - s);
    if (v > 8.0) v = 8.0;
    int best = 0;
    double best_d = fabs(v - mags[0]);
    for (int c = 1; c < 8; c++) {
        double d = fabs(v - mags[c]);
        if (d < best_d || (d == best_d && c % 2 == 0)) {
            best = c;
            best_d = d;
        }
    }
    return (sign << 3) | best;
}

/* Vector forms for exhaustive sweeps. */
ORACLE_API void oracle_encode_many(const uint16_t *x, const uint8_t *s, int64_t n, uint8_t *out)
{
    for (int64_t i = 0; i < n; i++) out[i] = (uint8_t)oracle_encode(x[i], s[i]);
}

ORACLE_API void oracle_encode_nearest_many(const uint16_t *x, const uint8_t *s, int64_t n, uint8_t *out)
{
    for (int64_t i = 0; i < n; i++) out[i] = (uint8_t)oracle_encode_nearest(x[i], s[i]);
}

/* ------------------------------------------------------------------------ */
/* Quantize rows of bf16 [rows, K] (K % 32 == 0) to                          */
/*   q      uint8 [rows, K/2]   element 2i in the low nibble of byte i,      */
/*                              element 2i+1 in the high nibble              */
/*                              [608632, _hw_mxfp4_quant_op step 3 split]    */
/*   scales uint8 [rows, K/32]  raw (natural) e8m0 bytes                     */
/* Returns 0, or -1 if an input is not finite (outside the method).          */
/* ------------------------------------------------------------------------ */
ORACLE_API int oracle_quantize(const uint16_t *x, int64_t rows, int64_t K, uint8_t *q, uint8_t *scales)
{
    if (K % 32 != 0) return -1;
    for (int64_t i = 0; i < rows * K; i++)
        if (((x[i] >> 7) & 0xFF) == 0xFF) return -1;
    int64_t G = K / 32;
    /* rows are independent */
#pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < rows; r++) {
        for (int64_t g = 0; g < G; g++) {
            const uint16_t *grp = x + r * K + g * 32;
            int s = oracle_scale_byte(grp, 32);
            scales[r * G + g] = (uint8_t)s;
            for (int j = 0; j < 32; j += 2) {
                int lo = oracle_encode(grp[j], s);
                int hi = oracle_encode(grp[j + 1], s);
                q[r * (K / 2) + g * 16 + j / 2] = (uint8_t)(lo | (hi << 4));
            }
        }
    }
    return 0;
}

/* Dequantize q/raw scales back to fp64 [rows, K]: value(code) * 2^(s-127). */
ORACLE_API void oracle_dequantize(const uint8_t *q, const uint8_t *scales, int64_t rows, int64_t K, double *out)
{
    int64_t G = K / 32;
#pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < rows; r++)
        for (int64_t k = 0; k < K; k++) {
            uint8_t byte = q[r * (K / 2) + k / 2];
            int code = (k % 2 == 0) ? (byte & 0xF) : (byte >> 4);
            out[r * K + k] = oracle_e2m1_value(code) * oracle_e8m0_value(scales[r * G + k / 32]);
        }
}

/* ------------------------------------------------------------------------ */
/* Scale shuffle.  [608632, _shuffle_scales: view (rows/32, 2, 16, G/8, 2,   */
/* 4), permute (0, 3, 5, 2, 4, 1)] and, equivalently, the address            */
/* arithmetic of [711914, _standalone_quant_kernel].  Written here in the    */
/* address form:                                                             */
/*   row = 32*r0 + 16*r1 + r2,  group = 8*k0 + 4*k1 + k2                      */
/*   byte = r1 + 2*k1 + 4*r2 + 64*k2 + 256*k0 + r0 * 32 * Gp                  */
/* with the buffer padded to pad256(rows) x Gp, Gp = pad8(K/32)              */
/* [608632, bypass launchers: s0, s1 padding].  Reading: padding bytes are   */
/* 127 (the A-scale buffer of [711914] is pre-filled with 127).              */
/* ------------------------------------------------------------------------ */
static int64_t pad_to(int64_t v, int64_t m) { return (v + m - 1) / m * m; }

ORACLE_API int64_t oracle_shuffled_scale_bytes(int64_t rows, int64_t K)
{
    return pad_to(rows, 256) * pad_to(K / 32, 8);
}

ORACLE_API int64_t oracle_shuffled_scale_index(int64_t row, int64_t g, int64_t Gp)
{
    int64_t r0 = row / 32, r1 = (row % 32) / 16, r2 = row % 16;
    int64_t k0 = g / 8, k1 = (g % 8) / 4, k2 = g % 4;
    return r1 + 2 * k1 + 4 * r2 + 64 * k2 + 256 * k0 + r0 * 32 * Gp;
}

ORACLE_API void oracle_shuffle_scales(const uint8_t *raw, int64_t rows, int64_t K, uint8_t *out)
{
    int64_t G = K / 32;
    int64_t Gp = pad_to(G, 8);
    int64_t total = oracle_shuffled_scale_bytes(rows, K);
    memset(out, 127, (size_t)total);
    for (int64_t r = 0; r < rows; r++)
        for (int64_t g = 0; g < G; g++)
            out[oracle_shuffled_scale_index(r, g, Gp)] = raw[r * G + g];
}

ORACLE_API void oracle_unshuffle_scales(const uint8_t *sh, int64_t rows, int64_t K, uint8_t *raw)
{
    int64_t G = K / 32;
    int64_t Gp = pad_to(G, 8);
    for (int64_t r = 0; r < rows; r++)
        for (int64_t g = 0; g < G; g++)
            raw[r * G + g] = sh[oracle_shuffled_scale_index(r, g, Gp)];
}

/* ------------------------------------------------------------------------ */
/* B weight preshuffle, 16 rows x 16 bytes tiles.  The pages print only its  */
/* inverse ([608632, _gemm_a16wfp4_preshuffle_kernel_v7: reshape (1, BN/16,  */
/* BK/64, 2, 16, 16), permute (0, 1, 4, 2, 3, 5)] and [711914,               */
/* _unshuffle_b_preshuffle]); both say: row group g of 16 rows is stored     */
/* contiguously, as (K/2)/16 tiles of 16 rows x 16 bytes, each tile          */
/* row-major.  Hence                                                         */
/*   out[g*(K/2)*16 + t*256 + n*16 + j] = bq[(16g + n)*(K/2) + 16t + j].      */
/* Requires rows % 16 == 0 and K % 32 == 0.                                  */
/* ------------------------------------------------------------------------ */
ORACLE_API void oracle_preshuffle_b(const uint8_t *bq, int64_t N, int64_t K, uint8_t *out)
{
    int64_t KB = K / 2;
    for (int64_t g = 0; g < N / 16; g++)
        for (int64_t t = 0; t < KB / 16; t++)
            for (int64_t n = 0; n < 16; n++)
                for (int64_t j = 0; j < 16; j++)
                    out[g * KB * 16 + t * 256 + n * 16 + j] = bq[(16 * g + n) * KB + 16 * t + j];
}

ORACLE_API void oracle_unpreshuffle_b(const uint8_t *sh, int64_t N, int64_t K, uint8_t *bq)
{
    int64_t KB = K / 2;
    for (int64_t g = 0; g < N / 16; g++)
        for (int64_t t = 0; t < KB / 16; t++)
            for (int64_t n = 0; n < 16; n++)
                for (int64_t j = 0; j < 16; j++)
                    bq[(16 * g + n) * KB + 16 * t + j] = sh[g * KB * 16 + t * 256 + n * 16 + j];
}

/* ------------------------------------------------------------------------ */
/* GEMM on quantized operands in natural layouts:                            */
/*   C[m][n] = sum_k deq(A)[m][k] * deq(B)[n][k]                             */
/* where deq() is value(code) * 2^(scale-127) per 32-group.                  */
/* [608632, kernel v7: the scaled dot of two e2m1 operands with e8m0 scales  */
/* into an accumulator].  Two accumulations are provided:                    */
/*   oracle_gemm_f64  fp64, k ascending.  Each product is exact and the sum  */
/*                    rounds at ~1e-16 relative: the exact product for all   */
/*                    practical purposes (exact on small shapes).            */
/*   oracle_gemm_f32  the matrix unit's own precision: per 32-group the      */
/*                    integer dot of the codes (exact), times both scales,   */
/*                    converted to fp32, then the groups summed in fp32 in   */
/*                    ascending group order [608632, kernel v7: an f32       */
/*                    accumulator over the K loop].                          */
/* Output elements are independent, so they are computed in parallel        */
/* (OpenMP over (m, n)); each one's arithmetic is the plain loop below.      */
/* ------------------------------------------------------------------------ */
ORACLE_API int oracle_num_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

ORACLE_API void oracle_gemm_f64(const uint8_t *qa, const uint8_t *sa, const uint8_t *qb, const uint8_t *sb,
                                int64_t M, int64_t N, int64_t K, double *C)
{
    double *da = (double *)malloc(sizeof(double) * (size_t)(M * K));
    double *db = (double *)malloc(sizeof(double) * (size_t)(N * K));
    oracle_dequantize(qa, sa, M, K, da);
    oracle_dequantize(qb, sb, N, K, db);
#pragma omp parallel for collapse(2) schedule(static)
    for (int64_t m = 0; m < M; m++)
        for (int64_t n = 0; n < N; n++) {
            double acc = 0.0;
            for (int64_t k = 0; k < K; k++) acc += da[m * K + k] * db[n * K + k];
            C[m * N + n] = acc;
        }
    free(da);
    free(db);
}

/* Twice the e2m1 value of a code: an integer in {0, 1, 2, 3, 4, 6, 8, 12},  */
/* signed (the table of oracle_e2m1_value, doubled).                         */
static int e2m1_twice(int code)
{
    static const int mag2[8] = {0, 1, 2, 3, 4, 6, 8, 12};
    return (code & 8) ? -mag2[code & 7] : mag2[code & 7];
}

ORACLE_API void oracle_gemm_f32(const uint8_t *qa, const uint8_t *sa, const uint8_t *qb, const uint8_t *sb,
                                int64_t M, int64_t N, int64_t K, float *C)
{
    int64_t G = K / 32;
#pragma omp parallel for collapse(2) schedule(static)
    for (int64_t m = 0; m < M; m++)
        for (int64_t n = 0; n < N; n++) {
            float acc = 0.0f;
            for (int64_t g = 0; g < G; g++) {
                /* integer dot in units of 1/4: sum of (2 a)(2 b) over the group */
                int64_t dot4 = 0;
                for (int64_t j = 0; j < 32; j++) {
                    int64_t k = 32 * g + j;
                    uint8_t ba = qa[m * (K / 2) + k / 2], bb = qb[n * (K / 2) + k / 2];
                    int ca = (k % 2 == 0) ? (ba & 0xF) : (ba >> 4);
                    int cb = (k % 2 == 0) ? (bb & 0xF) : (bb >> 4);
                    dot4 += (int64_t)e2m1_twice(ca) * e2m1_twice(cb);
                }
                /* exact in fp64 (|dot4| <= 4608); one rounding to fp32 */
                double term = ldexp((double)dot4, (int)sa[m * G + g] + (int)sb[n * G + g] - 254 - 2);
                acc = acc + (float)term;
            }
            C[m * N + n] = acc;
        }
}

/* Same fp64 sum for selected output elements only (for full-size parity
 * sampling): C_out[i] = C[ms[i]][ns[i]]. */
ORACLE_API void oracle_gemm_f64_sampled(const uint8_t *qa, const uint8_t *sa, const uint8_t *qb, const uint8_t *sb,
                                        int64_t M, int64_t N, int64_t K, const int64_t *ms, const int64_t *ns,
                                        int64_t count, double *out)
{
    (void)M;
    (void)N;
    int64_t G = K / 32;
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < count; i++) {
        int64_t m = ms[i], n = ns[i];
        double acc = 0.0;
        for (int64_t k = 0; k < K; k++) {
            uint8_t ba = qa[m * (K / 2) + k / 2], bb = qb[n * (K / 2) + k / 2];
            int ca = (k % 2 == 0) ? (ba & 0xF) : (ba >> 4);
            int cb = (k % 2 == 0) ? (bb & 0xF) : (bb >> 4);
            acc += oracle_e2m1_value(ca) * oracle_e8m0_value(sa[m * G + k / 32]) * oracle_e2m1_value(cb) *
                   oracle_e8m0_value(sb[n * G + k / 32]);
        }
        out[i] = acc;
    }
}

/* ------------------------------------------------------------------------ */
/* fp64 -> bf16 bits, round to nearest, ties to even, directly from the      */
/* double (no intermediate f32 rounding).  Reading: the pages cast the f32   */
/* accumulator to bf16 without naming a mode; nearest-even is taken.  An     */
/* fp32 accumulator converts to fp64 exactly, so this also rounds the fp32   */
/* mode's results.                                                           */
/* ------------------------------------------------------------------------ */
static uint32_t f2u(float f) { uint32_t u; memcpy(&u, &f, 4); return u; }

ORACLE_API uint16_t oracle_bf16_from_f64(double d)
{
    if (isnan(d)) return 0x7FC0;
    uint16_t sign = signbit(d) ? 0x8000 : 0;
    double a = fabs(d);
    if (a == 0.0) return sign;
    int e;
    (void)frexp(a, &e); /* a = f * 2^e, f in [0.5, 1): leading bit weight 2^(e-1) */
    int lead = e - 1;
    int quantum_exp = (lead < -126) ? -133 : lead - 7; /* bf16 ulp */
    double r = nearbyint(ldexp(a, -quantum_exp));      /* RNE in the default mode */
    double v = ldexp(r, quantum_exp);
    if (v >= ldexp(1.0, 128)) return sign | 0x7F80;
    float f = (float)v; /* exact: v has <= 8 significant bits and is in f32 range */
    return sign | (uint16_t)(f2u(f) >> 16);
}

ORACLE_API void oracle_bf16_from_f64_many(const double *d, int64_t n, uint16_t *out)
{
    for (int64_t i = 0; i < n; i++) out[i] = oracle_bf16_from_f64(d[i]);
}

/* ------------------------------------------------------------------------ */
/* The whole per-call path from bf16 A: quantize A, GEMM against quantized   */
/* B given in natural layout (fp32 group accumulation when f32acc != 0, else */
/* fp64), round to bf16.  Used for the CPU baseline.                         */
/* ------------------------------------------------------------------------ */
ORACLE_API int oracle_mxfp4_gemm_bf16(const uint16_t *A, const uint8_t *qb, const uint8_t *sb, int64_t M, int64_t N,
                                      int64_t K, uint16_t *C, int f32acc)
{
    uint8_t *qa = (uint8_t *)malloc((size_t)(M * K / 2));
    uint8_t *sa = (uint8_t *)malloc((size_t)(M * K / 32));
    double *c64 = (double *)malloc(sizeof(double) * (size_t)(M * N));
    float *c32 = f32acc ? (float *)malloc(sizeof(float) * (size_t)(M * N)) : NULL;
    int rc = oracle_quantize(A, M, K, qa, sa);
    if (rc == 0) {
        if (f32acc) {
            oracle_gemm_f32(qa, sa, qb, sb, M, N, K, c32);
            for (int64_t i = 0; i < M * N; i++) c64[i] = (double)c32[i];
        } else {
            oracle_gemm_f64(qa, sa, qb, sb, M, N, K, c64);
        }
        oracle_bf16_from_f64_many(c64, M * N, C);
    }
    free(qa);
    free(sa);
    free(c64);
    free(c32);
    return rc;
}
