/*
 * mx_oracle.c -- plain, slow CPU reference for the MX block-scaled NT GEMM.
 *
 * TEST INFRASTRUCTURE ONLY.  The test-suite, the smoke check and the CPU
 * baseline leg of the benchmark load this file's library; the GPU library
 * never links it, includes it or calls it, and the two share no code.
 *
 * What is computed.  The FlyDSL summary pages (yuxiaoba.github.io, "FlyDSL"
 * article, section "API compatibility is not universal input coverage")
 * define the MX scaled GEMM's input contract: operands in a fixed row/column
 * layout, one E8M0 scale per 32 consecutive values along K, K a multiple of
 * 128.  The AI-compiler digest of 2026-10-22 (item 1, "Accelerating PyTorch on
 * AMD GPUs with FlyDSL") adds "BlockWise1x32, E8M0 scale, FP32 accumulation"
 * and names the element formats MXFP4 and MXFP8.  The element encodings are
 * those of the OCP Microscaling (MX) v1.0 specification: MXFP4 = E2M1,
 * MXFP8 = E4M3 (no infinities, S.1111.111 is NaN), scale = E8M0.
 *
 * With A (M x K) and B (N x K) both stored K-contiguous, scale bytes
 * sA[m][b], sB[n][b] for block b = K-values 32b .. 32b+31, and dec() the
 * element decode:
 *
 *   C[m][n] = sum_b 2^(sA[m][b] + sB[n][b] - 254) * P(m,n,b)
 *   P(m,n,b) = sum_{j<32} dec(A[m][32b+j]) * dec(B[n][32b+j])
 *   T[m][n]  = sum_b 2^(sA+sB-254) * sum_{j<32} |dec(A) * dec(B)|
 *
 * T is the magnitude sum used as the tolerance denominator.
 *
 * E (optional) bounds what a dot-product unit loses when it adds each group
 * of 8 consecutive K-values by aligning every product to the group's largest
 * one on a grid of 2^(floor(log2 max|p|) - 12) and dropping the bits below
 * it: E = sum over groups of 2^(sA+sB-254) * sum_k (|p_k| mod grid).  This is
 * a tolerance term, not part of C: gfx950's block-scaled MFMA reduces E4M3
 * products this way (measured grid 2^(e_max-13); one bit of slack here).
 * For E2M1 every product is a multiple of 1/4 no smaller than the grid, so
 * E is zero.
 *
 * Mixed formats.  A and B may hold different element formats (A E4M3 with
 * B E2M1, "W4A8", or the reverse): the scaled MFMA takes a format selector
 * per operand, and the OCP MX definition of a block dot product does not
 * require equal formats.  dec() is then each operand's own decode.
 *
 * E5M2 (MXFP8's other encoding, both operands) has a wider range: values are
 * multiples of 2^-16 up to 57344, so a product is a multiple of 2^-32 below
 * 2^32 and a 32-term sum can need about 69 significant bits.  Its block sums
 * are therefore taken exactly in 128-bit integers (units of 2^-32) and
 * rounded to double once (block_exact); a block holding an infinity or a
 * NaN keeps IEEE double arithmetic instead.
 *
 * Precision.  P is exact in double: E2M1 values are multiples of 1/2 with
 * |v| <= 6, so a block sum is a multiple of 1/4 below 2^11; E4M3 values are
 * multiples of 2^-9 with |v| <= 448, so a product is a multiple of 2^-18
 * below 2^18 and a 32-term sum needs at most 41 significant bits; a mixed
 * E4M3 x E2M1 product is a multiple of 2^-10 below 2^12 (27 bits per sum).  Scaling by
 * a power of two in [2^-254, 2^254] is exact.  The only rounding is the final
 * double-precision sum over the K/32 blocks, taken in increasing b.
 *
 * Storage.  MXFP8 rows are K bytes, element k in byte k.  MXFP4 rows are K/2
 * bytes, element 2i in the low nibble of byte i and element 2i+1 in the high
 * nibble.  Scale rows are K/32 bytes.  Everything is row-major and dense.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#include <omp.h>

#define MXO_FMT_E2M1 1
#define MXO_FMT_E4M3 2
#define MXO_FMT_E5M2 3
#define MXO_FMT_E2M3 4
#define MXO_FMT_E3M2 5

/* E2M1: sign bit 3, exponent bits 2..1 (bias 1), mantissa bit 0.  Exponent
 * field 0 is subnormal: m * 2^-1.  No Inf, no NaN (OCP MX v1.0, FP4). */
double mxo_e2m1_value(unsigned code)
{
    unsigned s = (code >> 3) & 1u, e = (code >> 1) & 3u, m = code & 1u;
    double mag = (e == 0) ? 0.5 * (double)m : ldexp(1.0 + 0.5 * (double)m, (int)e - 1);
    return s ? -mag : mag;
}

/* E4M3 ("FN"): sign bit 7, exponent bits 6..3 (bias 7), mantissa bits 2..0.
 * Exponent field 0 is subnormal: m/8 * 2^-6.  S.1111.111 is NaN, no Inf
 * (OCP MX v1.0, FP8 E4M3). */
double mxo_e4m3_value(unsigned code)
{
    unsigned s = (code >> 7) & 1u, e = (code >> 3) & 15u, m = code & 7u;
    if (e == 15 && m == 7) return NAN;
    double mag = (e == 0) ? ldexp((double)m / 8.0, -6) : ldexp(1.0 + (double)m / 8.0, (int)e - 7);
    return s ? -mag : mag;
}

/* E5M2: sign bit 7, exponent bits 6..2 (bias 15), mantissa bits 1..0.
 * Exponent field 0 is subnormal: m/4 * 2^-14.  Exponent field 31 is
 * infinity (m = 0) or NaN (OCP MX v1.0, FP8 E5M2, IEEE-like). */
double mxo_e5m2_value(unsigned code)
{
    unsigned s = (code >> 7) & 1u, e = (code >> 2) & 31u, m = code & 3u;
    double mag;
    if (e == 31) mag = (m == 0) ? INFINITY : NAN;
    else mag = (e == 0) ? ldexp((double)m / 4.0, -14) : ldexp(1.0 + (double)m / 4.0, (int)e - 15);
    return s ? -mag : mag;
}

/* FP6 E2M3: sign bit 5, exponent bits 4..3 (bias 1), mantissa bits 2..0.
 * Exponent field 0 is subnormal: m/8.  No Inf, no NaN; largest 7.5 (OCP MX
 * v1.0, FP6 E2M3). */
double mxo_e2m3_value(unsigned code)
{
    unsigned s = (code >> 5) & 1u, e = (code >> 3) & 3u, m = code & 7u;
    double mag = (e == 0) ? (double)m / 8.0 : ldexp(1.0 + (double)m / 8.0, (int)e - 1);
    return s ? -mag : mag;
}

/* FP6 E3M2: sign bit 5, exponent bits 4..2 (bias 3), mantissa bits 1..0.
 * Exponent field 0 is subnormal: m/4 * 2^-2.  No Inf, no NaN; largest 28
 * (OCP MX v1.0, FP6 E3M2). */
double mxo_e3m2_value(unsigned code)
{
    unsigned s = (code >> 5) & 1u, e = (code >> 2) & 7u, m = code & 3u;
    double mag = (e == 0) ? ldexp((double)m / 4.0, -2) : ldexp(1.0 + (double)m / 4.0, (int)e - 3);
    return s ? -mag : mag;
}

/* E8M0 scale: 2^(byte - 127); byte 255 is NaN (OCP MX v1.0, E8M0). */
double mxo_e8m0_value(unsigned byte)
{
    if (byte == 255) return NAN;
    return ldexp(1.0, (int)byte - 127);
}

/* Decode element k of one packed row into a double.  FP6 rows are a
 * little-endian bit string with element k in bits 6k .. 6k+5 (bit b is bit
 * b % 8 of byte b / 8), four elements per three bytes. */
static double decode_elem(int fmt, const uint8_t *row, int64_t k,
                          const double *t4, const double *t8)
{
    if (fmt == MXO_FMT_E4M3) return t8[row[k]];
    if (fmt == MXO_FMT_E5M2) return mxo_e5m2_value(row[k]);
    if (fmt == MXO_FMT_E2M3 || fmt == MXO_FMT_E3M2) {
        const int64_t bit = 6 * k;
        unsigned v = row[bit >> 3];
        if ((bit & 7) > 2) v |= (unsigned)row[(bit >> 3) + 1] << 8;
        const unsigned code = (v >> (bit & 7)) & 63u;
        return fmt == MXO_FMT_E2M3 ? mxo_e2m3_value(code) : mxo_e3m2_value(code);
    }
    uint8_t byte = row[k >> 1];
    return t4[(k & 1) ? (byte >> 4) : (byte & 15u)];
}

static void make_tables(double t4[16], double t8[256], double pow2[509])
{
    for (unsigned c = 0; c < 16; ++c) t4[c] = mxo_e2m1_value(c);
    for (unsigned c = 0; c < 256; ++c) t8[c] = mxo_e4m3_value(c);
    /* pow2[i] = 2^(i - 254), i = sA + sB in 0..508: every entry is an exact
     * double (normal range reaches 2^-1022). */
    for (int i = 0; i < 509; ++i) pow2[i] = ldexp(1.0, i - 254);
}

static int64_t row_bytes(int fmt, int64_t K)
{
    if (fmt == MXO_FMT_E2M1) return K / 2;
    if (fmt == MXO_FMT_E2M3 || fmt == MXO_FMT_E3M2) return K / 4 * 3;
    return K;
}

/* Exact block sums with an E5M2 operand: every finite E5M2, E4M3 or E2M1
 * value is an integer multiple of 2^-16 below 2^32 in those units, so each
 * product is an exact
 * 64-bit-magnitude integer in units of 2^-32 and 32 of them sum exactly in
 * 128 bits.  Writes sum p and magnitude sum q rounded once to double;
 * returns 0 if a value is not finite (the caller keeps its IEEE sums). */
static int block_exact(const double *x, const double *y, double *p, double *q)
{
    __int128 sp = 0, sq = 0;
    for (int j = 0; j < 32; ++j) {
        if (!isfinite(x[j]) || !isfinite(y[j])) return 0;
        __int128 a = (__int128)(int64_t)ldexp(x[j], 16), b = (__int128)(int64_t)ldexp(y[j], 16);
        __int128 t = a * b;
        sp += t;
        sq += t < 0 ? -t : t;
    }
    *p = ldexp((double)sp, -32);
    *q = ldexp((double)sq, -32);
    return 1;
}

/* Sub-grid loss of one group of 8 products: sum of |p| mod grid, with grid =
 * 2^(floor(log2 max|p|) - 12).  Products are exact doubles. */
static double group_loss(const double *prod)
{
    double mx = 0.0;
    for (int i = 0; i < 8; ++i) mx = fmax(mx, fabs(prod[i]));
    if (!(mx > 0.0)) return 0.0;
    int e;
    frexp(mx, &e);                      /* mx = f * 2^e, f in [0.5, 1) */
    double grid = ldexp(1.0, (e - 1) - 12);
    double loss = 0.0;
    for (int i = 0; i < 8; ++i) loss += fmod(fabs(prod[i]), grid);
    return loss;
}

/* Fill the caller's 16- and 256-entry arrays with the element decode tables. */
void mxo_tables(double *e2m1_out16, double *e4m3_out256)
{
    double pow2[509];
    make_tables(e2m1_out16, e4m3_out256, pow2);
}

/*
 * One block's contribution 2^(sA[m][b]+sB[n][b]-254) * P(m,n,b), with its
 * magnitude counterpart written to *t_out (may be NULL).  Returns NaN if
 * either scale byte is 255 or an element decodes to NaN.
 */
double mxo_block_contrib(int fmt, int64_t K,
                         const uint8_t *A, const uint8_t *A_scale,
                         const uint8_t *B, const uint8_t *B_scale,
                         int64_t m, int64_t n, int64_t b, double *t_out)
{
    double t4[16], t8[256], pow2[509];
    make_tables(t4, t8, pow2);
    const int64_t nb = K / 32, rb = row_bytes(fmt, K);
    const uint8_t *arow = A + m * rb, *brow = B + n * rb;
    unsigned sa = A_scale[m * nb + b], sb = B_scale[n * nb + b];
    double p = 0.0, t = 0.0;
    for (int64_t j = 0; j < 32; ++j) {
        double x = decode_elem(fmt, arow, 32 * b + j, t4, t8);
        double y = decode_elem(fmt, brow, 32 * b + j, t4, t8);
        p += x * y;
        t += fabs(x * y);
    }
    double w = (sa == 255 || sb == 255) ? NAN : pow2[sa + sb];
    if (t_out) *t_out = t * w;
    return p * w;
}

/*
 * C[i][n], T[i][n] and E[i][n] for the rows m = rows[i] (i < nrows), all
 * n < N, with A's elements in fmt_a and B's in fmt_b.  rows may be NULL, meaning rows 0..nrows-1.  C, T and E are
 * nrows x N doubles, row-major; T and E may be NULL.  nthreads <= 0 uses
 * OpenMP's default.  Returns 0, or -1 on an argument the definition does
 * not cover.
 */
int mxo_gemm_ab(int fmt_a, int fmt_b, int64_t M, int64_t N, int64_t K,
                const uint8_t *A, const uint8_t *A_scale,
                const uint8_t *B, const uint8_t *B_scale,
                const int64_t *rows, int64_t nrows,
                double *C, double *T, double *E, int nthreads)
{
    if (fmt_a < MXO_FMT_E2M1 || fmt_a > MXO_FMT_E3M2 || fmt_b < MXO_FMT_E2M1 || fmt_b > MXO_FMT_E3M2)
        return -1;
    /* With an E5M2 operand a block sum can need more than 53 bits (E5M2 x
     * E4M3 products span 50 binades, E5M2 x E5M2 64), so it is taken in
     * 128-bit integers; every value of the three formats is a whole multiple
     * of 2^-16. */
    const int exact128 = fmt_a == MXO_FMT_E5M2 || fmt_b == MXO_FMT_E5M2;
    if (M < 0 || N < 0 || K <= 0 || K % 32 != 0 || nrows < 0) return -1;
    for (int64_t i = 0; rows && i < nrows; ++i)
        if (rows[i] < 0 || rows[i] >= M) return -1;
    if (!rows && nrows > M) return -1;

    double t4[16], t8[256], pow2[509];
    make_tables(t4, t8, pow2);
    const int64_t nb = K / 32, rba = row_bytes(fmt_a, K), rbb = row_bytes(fmt_b, K);
    const int64_t chunk = 128;      /* decoded A rows held at once */
    double *adec = (double *)malloc(sizeof(double) * (size_t)(chunk * K));
    if (!adec) return -1;
    if (nthreads <= 0) nthreads = omp_get_max_threads();

    for (int64_t i0 = 0; i0 < nrows; i0 += chunk) {
        const int64_t ni = (nrows - i0 < chunk) ? nrows - i0 : chunk;
        /* Step 1: decode the chunk's A rows by table. */
        for (int64_t i = 0; i < ni; ++i) {
            int64_t m = rows ? rows[i0 + i] : i0 + i;
            for (int64_t k = 0; k < K; ++k)
                adec[i * K + k] = decode_elem(fmt_a, A + m * rba, k, t4, t8);
        }
        int failed = 0;
#pragma omp parallel num_threads(nthreads)
        {
            double *bdec = (double *)malloc(sizeof(double) * (size_t)K);
            if (!bdec) {
#pragma omp atomic write
                failed = 1;
            }
#pragma omp for schedule(dynamic, 4)
            for (int64_t n = 0; n < N; ++n) {
                if (!bdec) continue;
                /* Step 1 (B side): decode row n of B by table. */
                for (int64_t k = 0; k < K; ++k)
                    bdec[k] = decode_elem(fmt_b, B + n * rbb, k, t4, t8);
                const uint8_t *sbrow = B_scale + n * nb;
                for (int64_t i = 0; i < ni; ++i) {
                    int64_t m = rows ? rows[i0 + i] : i0 + i;
                    const uint8_t *sarow = A_scale + m * nb;
                    const double *a = adec + i * K;
                    double c = 0.0, t = 0.0, el = 0.0;
                    for (int64_t b = 0; b < nb; ++b) {
                        /* Step 2: the exact block dot product P(m,n,b). */
                        double p = 0.0, q = 0.0, loss = 0.0, prod[32];
                        for (int64_t j = 32 * b; j < 32 * b + 32; ++j) {
                            prod[j - 32 * b] = a[j] * bdec[j];
                            p += prod[j - 32 * b];
                            q += fabs(prod[j - 32 * b]);
                        }
                        if (exact128) block_exact(a + 32 * b, bdec + 32 * b, &p, &q);
                        if (E)
                            for (int gi = 0; gi < 4; ++gi) loss += group_loss(prod + 8 * gi);
                        /* Step 3: the block's power-of-two scale. */
                        unsigned sa = sarow[b], sb = sbrow[b];
                        double w = (sa == 255 || sb == 255) ? NAN : pow2[sa + sb];
                        /* Step 4: accumulate blocks in increasing b. */
                        c += p * w;
                        t += q * w;
                        el += loss * w;
                    }
                    C[(i0 + i) * N + n] = c;
                    if (T) T[(i0 + i) * N + n] = t;
                    if (E) E[(i0 + i) * N + n] = el;
                }
            }
            free(bdec);
        }
        if (failed) { free(adec); return -1; }
    }
    free(adec);
    return 0;
}

/* Both operands in one format. */
int mxo_gemm(int fmt, int64_t M, int64_t N, int64_t K,
             const uint8_t *A, const uint8_t *A_scale,
             const uint8_t *B, const uint8_t *B_scale,
             const int64_t *rows, int64_t nrows,
             double *C, double *T, double *E, int nthreads)
{
    return mxo_gemm_ab(fmt, fmt, M, N, K, A, A_scale, B, B_scale, rows, nrows, C, T, E,
                       nthreads);
}

/* ------------------------------------------------------------------------
 * MX quantization (the step before the GEMM): conversion of a matrix of
 * wider values to MX elements and E8M0 scales by the OCP Microscaling v1.0
 * rule, for checking a GPU quantizer.  The FlyDSL article times its scaled
 * GEMMs from operands already in this form (section "Performance numbers
 * need their baselines"); the rule itself is the OCP one:
 *
 * per block of 32 consecutive values x_j along K,
 *   amax = max_j |x_j|
 *   X    = floor(log2 amax) - emax   (emax: exponent of the element format's
 *                                     largest normal: 2 for E2M1 and E2M3,
 *                                     8 for E4M3, 15 for E5M2, 4 for E3M2)
 *   s    = X + 127 clamped to [0, 254]   (the E8M0 byte; s = 0 if amax = 0)
 *   P_j  = x_j * 2^(127 - s) rounded to the nearest element value, ties to
 *          the even code (even last mantissa bit), magnitudes above the
 *          format's largest (6, 448, 57344, 7.5, 28) saturating to it; the sign bit is x_j's
 *          sign, also when the magnitude rounds to zero.
 * A block holding a NaN or an infinity gets s = 255 (E8M0 NaN) and every
 * element code 0.
 */

/* Magnitude a >= 0 (finite) -> element code without its sign bit, for a
 * format with `man` mantissa bits, exponent bias `bias`, smallest normal
 * exponent 1 - bias and largest magnitude `maxv`. */
static unsigned encode_magnitude(double a, int man, int bias, double maxv)
{
    const int emin = 1 - bias;
    if (a > maxv) a = maxv;
    int e2;
    frexp(a, &e2);                                   /* a = f * 2^e2, f in [0.5, 1) */
    const int e = (a > 0.0) ? e2 - 1 : emin;         /* floor(log2 a) */
    const double quantum = ldexp(1.0, (e < emin ? emin : e) - man);
    const double v = nearbyint(a / quantum) * quantum;   /* ties to even */
    if (v < ldexp(1.0, emin))                        /* subnormal or zero */
        return (unsigned)(v / ldexp(1.0, emin - man));
    frexp(v, &e2);
    const int ev = e2 - 1;
    const unsigned mant = (unsigned)((v / ldexp(1.0, ev) - 1.0) * (double)(1 << man));
    return ((unsigned)(ev + bias) << man) | mant;
}

/* Quantize X (rows x K doubles, each an exact FP32 or BF16 value; K a
 * multiple of 32) to Q (rows x K bytes for E4M3 / E5M2, rows x K/2 for E2M1, element
 * 2i in the low nibble, rows x 3K/4 for E2M3 / E3M2, element k at bits
 * 6k .. 6k+5) and S (rows x K/32 E8M0 bytes).  Returns 0, or -1 on
 * an argument the rule does not cover. */
int mxo_quantize(int fmt, int64_t rows, int64_t K, const double *X, uint8_t *Q, uint8_t *S)
{
    if (fmt < MXO_FMT_E2M1 || fmt > MXO_FMT_E3M2) return -1;
    if (rows < 0 || K <= 0 || K % 32 != 0) return -1;
    /* Per format (OCP MX v1.0 element formats): emax = exponent of the
     * largest normal value (6 = 1.5 * 2^2, 448 = 1.75 * 2^8, 57344 =
     * 1.75 * 2^15, 7.5 = 1.875 * 2^2, 28 = 1.75 * 2^4), mantissa bits,
     * exponent bias, largest magnitude and the sign bit of a code. */
    static const int emax_of[6] = {0, 2, 8, 15, 2, 4};
    static const int man_of[6] = {0, 1, 3, 2, 3, 2};
    static const int bias_of[6] = {0, 1, 7, 15, 1, 3};
    static const double maxv_of[6] = {0, 6.0, 448.0, 57344.0, 7.5, 28.0};
    static const unsigned sign_of[6] = {0, 8u, 128u, 128u, 32u, 32u};
    const int e2m1 = fmt == MXO_FMT_E2M1;
    const int fp6 = fmt == MXO_FMT_E2M3 || fmt == MXO_FMT_E3M2;
    const int emax = emax_of[fmt], man = man_of[fmt], bias = bias_of[fmt];
    const double maxv = maxv_of[fmt];
    const unsigned sign_bit = sign_of[fmt];
    const int64_t nb = K / 32, rb = row_bytes(fmt, K);
#pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < rows; ++r) {
        for (int64_t b = 0; b < nb; ++b) {
            const double *x = X + r * K + 32 * b;
            double amax = 0.0;
            int finite = 1;
            for (int j = 0; j < 32; ++j) {
                if (!isfinite(x[j])) finite = 0;
                else if (fabs(x[j]) > amax) amax = fabs(x[j]);
            }
            int s;
            if (!finite) {
                s = 255;
            } else if (amax == 0.0) {
                s = 0;
            } else {
                int e2;
                frexp(amax, &e2);
                s = (e2 - 1) - emax + 127;
                s = s < 0 ? 0 : (s > 254 ? 254 : s);
            }
            S[r * nb + b] = (uint8_t)s;
            for (int j = 0; j < 32; ++j) {
                unsigned code = 0;
                if (finite) {
                    code = encode_magnitude(fabs(x[j]) * ldexp(1.0, 127 - s), man, bias, maxv);
                    if (signbit(x[j])) code |= sign_bit;
                }
                const int64_t k = 32 * b + j;
                if (fp6) {
                    /* element k is bits 6k .. 6k+5 of the row's little-endian
                     * bit string: set each bit on its own */
                    for (int i = 0; i < 6; ++i) {
                        const int64_t bit = 6 * k + i;
                        uint8_t *byte = &Q[r * rb + (bit >> 3)];
                        const uint8_t m = (uint8_t)(1u << (bit & 7));
                        *byte = (uint8_t)(((code >> i) & 1u) ? (*byte | m) : (*byte & ~m));
                    }
                } else if (!e2m1) {
                    Q[r * rb + k] = (uint8_t)code;
                } else {
                    uint8_t *byte = &Q[r * rb + (k >> 1)];
                    if (k & 1) *byte = (uint8_t)((*byte & 0x0fu) | (code << 4));
                    else *byte = (uint8_t)((*byte & 0xf0u) | code);
                }
            }
        }
    }
    return 0;
}

/* ------------------------------------------------------------------------
 * BF16 dense NT GEMM (the pages' second GEMM workload: BF16 dense GEMMs,
 * FlyDSL article, "Performance numbers need their baselines"; no scales):
 *   C[m][n] = sum_k a[m][k] * b[n][k],  T[m][n] = sum_k |a[m][k] * b[n][k]|
 * with a, b BF16 values given as their 16-bit patterns (the upper half of
 * the IEEE binary32 pattern).  A product of two BF16 values (8-bit
 * significands) is exact in double; the K-term sum, taken in increasing k,
 * is the only rounding (at most K * 2^-53 * T).
 */
double mxo_bf16_value(unsigned bits)
{
    union { uint32_t u; float f; } v;
    v.u = (uint32_t)(bits & 0xffffu) << 16;
    return (double)v.f;
}

int mxo_gemm_bf16(int64_t M, int64_t N, int64_t K, const uint16_t *A, const uint16_t *B,
                  const int64_t *rows, int64_t nrows, double *C, double *T, int nthreads)
{
    if (M < 0 || N < 0 || K <= 0 || nrows < 0) return -1;
    for (int64_t i = 0; rows && i < nrows; ++i)
        if (rows[i] < 0 || rows[i] >= M) return -1;
    if (!rows && nrows > M) return -1;
    if (nthreads <= 0) nthreads = omp_get_max_threads();
    double *bdec = (double *)malloc(sizeof(double) * (size_t)(N * K));
    double *adec = (double *)malloc(sizeof(double) * (size_t)(nrows * K));
    if (!bdec || !adec) { free(bdec); free(adec); return -1; }
    for (int64_t i = 0; i < N * K; ++i) bdec[i] = mxo_bf16_value(B[i]);
    for (int64_t i = 0; i < nrows; ++i) {
        const int64_t m = rows ? rows[i] : i;
        for (int64_t k = 0; k < K; ++k) adec[i * K + k] = mxo_bf16_value(A[m * K + k]);
    }
#pragma omp parallel for num_threads(nthreads) schedule(dynamic, 4)
    for (int64_t i = 0; i < nrows; ++i) {
        const double *a = adec + i * K;
        for (int64_t n = 0; n < N; ++n) {
            const double *b = bdec + n * K;
            double c = 0.0, t = 0.0;
            for (int64_t k = 0; k < K; ++k) {
                c += a[k] * b[k];
                t += fabs(a[k] * b[k]);
            }
            C[i * N + n] = c;
            if (T) T[i * N + n] = t;
        }
    }
    free(bdec);
    free(adec);
    return 0;
}
