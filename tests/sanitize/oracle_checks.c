/*
 * The CPU oracle under AddressSanitizer and UndefinedBehaviorSanitizer.
 * Test infrastructure: built with gcc by tests/test_sanitize_cpu.py, which
 * includes the oracle's source in this one translation unit.  Every entry
 * point runs on small ragged shapes with arbitrary bytes (NaN codes, scale
 * bytes 0 and 255, every FP6 bit pattern), non-finite and subnormal
 * quantizer inputs, row subsets and the argument errors; the sanitizers
 * abort on the first out-of-bounds access, use of freed memory or undefined
 * operation.  Prints "oracle checks passed" and exits 0 otherwise.
 */
#include "../../oracle/mx_oracle.c"

#include <stdio.h>

static int fails;
#define CHECK(c) do { if (!(c)) { fprintf(stderr, "check failed, line %d: %s\n", __LINE__, #c); ++fails; } } while (0)

static uint64_t state = 0x9E3779B97F4A7C15ull;
static uint64_t next(void)
{
    state ^= state << 13;
    state ^= state >> 7;
    state ^= state << 17;
    return state;
}

static uint8_t *bytes(int64_t n)
{
    uint8_t *p = (uint8_t *)malloc((size_t)(n > 0 ? n : 1));
    for (int64_t i = 0; i < n; ++i) p[i] = (uint8_t)next();
    return p;
}

static int64_t rowb(int fmt, int64_t K)
{
    return fmt == MXO_FMT_E2M1 ? K / 2 : (fmt == MXO_FMT_E2M3 || fmt == MXO_FMT_E3M2) ? K / 4 * 3 : K;
}

int main(void)
{
    double t4[16], t8[256];
    mxo_tables(t4, t8);
    for (unsigned c = 0; c < 512; ++c) {
        (void)mxo_e2m1_value(c); (void)mxo_e4m3_value(c); (void)mxo_e5m2_value(c);
        (void)mxo_e2m3_value(c); (void)mxo_e3m2_value(c); (void)mxo_e8m0_value(c);
        (void)mxo_bf16_value(c * 257u);
    }

    const int64_t ms[] = {1, 3, 17};
    const int64_t ks[] = {32, 128, 384};
    for (int fa = MXO_FMT_E2M1; fa <= MXO_FMT_E3M2; ++fa)
        for (int fb = MXO_FMT_E2M1; fb <= MXO_FMT_E3M2; ++fb)
            for (int im = 0; im < 3; ++im)
                for (int ik = 0; ik < 3; ++ik) {
                    const int64_t M = ms[im], N = ms[2 - im], K = ks[ik];
                    if ((fa == MXO_FMT_E2M3 || fa == MXO_FMT_E3M2 || fb == MXO_FMT_E2M3 ||
                         fb == MXO_FMT_E3M2) && K % 128 != 0)
                        continue;   /* FP6 rows hold whole 4-element groups of 3 bytes */
                    uint8_t *A = bytes(M * rowb(fa, K)), *B = bytes(N * rowb(fb, K));
                    uint8_t *As = bytes(M * K / 32), *Bs = bytes(N * K / 32);
                    double *C = malloc(sizeof(double) * (size_t)(M * N));
                    double *T = malloc(sizeof(double) * (size_t)(M * N));
                    double *E = malloc(sizeof(double) * (size_t)(M * N));
                    CHECK(mxo_gemm_ab(fa, fb, M, N, K, A, As, B, Bs, NULL, M, C, T, E, 1) == 0);
                    const int64_t rows[2] = {M - 1, 0};
                    CHECK(mxo_gemm_ab(fa, fb, M, N, K, A, As, B, Bs, rows, 2 < M ? 2 : M, C, T,
                                      NULL, 1) == 0);
                    if (fa == fb) {
                        CHECK(mxo_gemm(fa, M, N, K, A, As, B, Bs, NULL, M, C, NULL, NULL, 1) == 0);
                        double t;
                        (void)mxo_block_contrib(fa, K, A, As, B, Bs, M - 1, N - 1, K / 32 - 1, &t);
                    }
                    const int64_t bad[1] = {M};
                    CHECK(mxo_gemm_ab(fa, fb, M, N, K, A, As, B, Bs, bad, 1, C, T, E, 1) == -1);
                    CHECK(mxo_gemm_ab(fa, fb, M, N, K, A, As, B, Bs, NULL, M + 1, C, T, E, 1) == -1);
                    free(A); free(B); free(As); free(Bs); free(C); free(T); free(E);
                }
    CHECK(mxo_gemm_ab(0, 1, 1, 1, 32, NULL, NULL, NULL, NULL, NULL, 0, NULL, NULL, NULL, 1) == -1);
    CHECK(mxo_gemm(1, 1, 1, 33, NULL, NULL, NULL, NULL, NULL, 0, NULL, NULL, NULL, 1) == -1);

    /* quantizer: finite values of every magnitude, FP32 subnormals, zeros,
     * infinities and NaNs, in blocks of their own and mixed */
    for (int fmt = MXO_FMT_E2M1; fmt <= MXO_FMT_E3M2; ++fmt) {
        const int64_t rows = 5, K = 128;
        double *X = malloc(sizeof(double) * (size_t)(rows * K));
        for (int64_t i = 0; i < rows * K; ++i) {
            const uint64_t r = next();
            const int e = (int)(r % 300) - 150;
            X[i] = ldexp((double)(int32_t)(r >> 40) / 8388608.0, e);
            X[i] = (double)(float)X[i];
        }
        for (int64_t i = 32; i < 64; ++i) X[i] = 0.0;
        X[70] = INFINITY; X[100] = -INFINITY; X[130] = NAN; X[200] = 1e-45; X[201] = -0.0;
        uint8_t *Q = malloc((size_t)(rows * rowb(fmt, K))), *S = malloc((size_t)(rows * K / 32));
        CHECK(mxo_quantize(fmt, rows, K, X, Q, S) == 0);
        CHECK(mxo_quantize(fmt, rows, 48, X, Q, S) == -1);
        free(X); free(Q); free(S);
    }
    CHECK(mxo_quantize(0, 1, 32, NULL, NULL, NULL) == -1);

    /* dense BF16 */
    {
        const int64_t M = 3, N = 5, K = 48;
        uint16_t *A = malloc(sizeof(uint16_t) * M * K), *B = malloc(sizeof(uint16_t) * N * K);
        for (int64_t i = 0; i < M * K; ++i) A[i] = (uint16_t)next();
        for (int64_t i = 0; i < N * K; ++i) B[i] = (uint16_t)next();
        double *C = malloc(sizeof(double) * M * N), *T = malloc(sizeof(double) * M * N);
        CHECK(mxo_gemm_bf16(M, N, K, A, B, NULL, M, C, T, 1) == 0);
        const int64_t rows[1] = {2};
        CHECK(mxo_gemm_bf16(M, N, K, A, B, rows, 1, C, NULL, 1) == 0);
        CHECK(mxo_gemm_bf16(M, N, K, A, B, NULL, M + 1, C, T, 1) == -1);
        free(A); free(B); free(C); free(T);
    }
    if (fails) return 1;
    printf("oracle checks passed\n");
    return 0;
}
