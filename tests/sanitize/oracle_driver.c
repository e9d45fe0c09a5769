/*
 * The C oracle under AddressSanitizer and UBSan, on the CPU: every routine on
 * small inputs of many shapes (lengths 1 .. 1024, images, volumes, products of
 * unequal lengths), the routines checked against one another (the radix-2
 * FFT against the direct DFT, the FFT product against the schoolbook sum) so
 * that an out-of-bounds index that happens to read plausible values still
 * fails, and every bad-argument return.  oracle.c is included whole.
 *
 * Built and run by tests/test_host_sanitizers.py.  Exit status 0 = all checks
 * passed and the sanitizers reported nothing.
 */
#include "oracle.c"

#include <stdio.h>

static int g_fail = 0;
#define CHECK(c)                                                        \
    do {                                                                \
        if (!(c)) {                                                     \
            fprintf(stderr, "check failed: %s (line %d)\n", #c, __LINE__); \
            ++g_fail;                                                   \
        }                                                               \
    } while (0)

static double frand(uint64_t* s)
{
    *s = *s * 6364136223846793005ULL + 1442695040888963407ULL;
    return (double)(*s >> 11) / 9007199254740992.0 * 2.0 - 1.0;
}

static double max_diff(const double* a, const double* b, int64_t n)
{
    double m = 0;
    for (int64_t i = 0; i < n; ++i) m = fmax(m, fabs(a[i] - b[i]));
    return m;
}

static void check_1d(void)
{
    uint64_t s = 1;
    for (int64_t n = 1; n <= 1024; n *= 2)
        for (int64_t batch = 1; batch <= 3; ++batch)
            for (int inv = 0; inv < 2; ++inv) {
                const int64_t len = 2 * n * batch;
                double* x = malloc(len * sizeof(double));
                double* X = malloc(len * sizeof(double));
                double* D = malloc(len * sizeof(double));
                for (int64_t i = 0; i < len; ++i) x[i] = frand(&s);
                CHECK(oracle_fft(x, X, n, batch, inv) == 0);
                CHECK(oracle_dft_direct(x, D, n, batch, inv) == 0);
                CHECK(max_diff(X, D, len) < 1e-10 * (double)n);
                int64_t ks[3] = {0, n / 2, n - 1};
                double S[3 * 2 * 3];
                CHECK(oracle_dft_sample(x, n, batch, ks, 3, S, inv) == 0);
                for (int64_t b = 0; b < batch; ++b)
                    for (int j = 0; j < 3; ++j) {
                        CHECK(fabs(S[2 * (b * 3 + j)] - D[2 * (b * n + ks[j])]) < 1e-9 * (double)n);
                        CHECK(fabs(S[2 * (b * 3 + j) + 1] - D[2 * (b * n + ks[j]) + 1]) < 1e-9 * (double)n);
                    }
                free(x);
                free(X);
                free(D);
            }
    for (int64_t n = 1; n <= 40; ++n) {  /* the direct DFT at lengths that are not powers of two */
        double* x = malloc(4 * n * sizeof(double));
        double* X = malloc(4 * n * sizeof(double));
        double* Y = malloc(4 * n * sizeof(double));
        for (int64_t i = 0; i < 4 * n; ++i) x[i] = frand(&s);
        CHECK(oracle_dft_direct(x, X, n, 2, 0) == 0);
        CHECK(oracle_dft_direct(X, Y, n, 2, 1) == 0);
        CHECK(max_diff(x, Y, 4 * n) < 1e-12 * (double)n);
        free(x);
        free(X);
        free(Y);
    }
    double z[2] = {0, 0};
    int64_t k0 = 0;
    CHECK(oracle_fft(z, z, 3, 1, 0) < 0);
    CHECK(oracle_fft(z, z, 0, 1, 0) < 0);
    CHECK(oracle_dft_direct(z, z, 0, 1, 0) < 0);
    CHECK(oracle_dft_sample(z, 1, -1, &k0, 1, z, 0) < 0);
}

static void check_nd(void)
{
    uint64_t s = 7;
    for (int64_t h = 1; h <= 16; h *= 2)
        for (int64_t w = 1; w <= 32; w *= 4) {
            const int64_t len = 2 * h * w * 2;
            double* x = malloc(len * sizeof(double));
            double* X = malloc(len * sizeof(double));
            double* Y = malloc(len * sizeof(double));
            for (int64_t i = 0; i < len; ++i) x[i] = frand(&s);
            CHECK(oracle_fft2(x, X, h, w, 2, 0) == 0);
            CHECK(oracle_fft2(X, Y, h, w, 2, 1) == 0);
            CHECK(max_diff(x, Y, len) < 1e-12 * (double)(h * w));
            CHECK(oracle_fft3(x, X, 2, h, w, 1, 0) == 0);
            CHECK(oracle_fft3(X, Y, 2, h, w, 1, 1) == 0);
            CHECK(max_diff(x, Y, len) < 1e-12 * (double)(h * w));
            free(x);
            free(X);
            free(Y);
        }
    double z[2] = {0, 0};
    CHECK(oracle_fft2(z, z, 3, 2, 1, 0) < 0);
    CHECK(oracle_fft3(z, z, 2, 3, 2, 1, 0) < 0);
}

static void check_poly(void)
{
    uint64_t s = 11;
    for (int64_t la = 1; la <= 70; la += 3)
        for (int64_t lb = 1; lb <= 70; lb += 7) {
            const int64_t batch = 2, lc = la + lb - 1;
            int64_t n = 1;
            while (n < lc) n *= 2;
            int64_t* a = malloc(batch * la * sizeof(int64_t));
            int64_t* b = malloc(batch * lb * sizeof(int64_t));
            int64_t* c = malloc(batch * lc * sizeof(int64_t));
            int64_t* d = malloc(batch * lc * sizeof(int64_t));
            for (int64_t i = 0; i < batch * la; ++i) a[i] = (int64_t)(frand(&s) * 1000);
            for (int64_t i = 0; i < batch * lb; ++i) b[i] = (int64_t)(frand(&s) * 1000);
            double resid = -1;
            CHECK(oracle_polymul_fft(a, la, b, lb, c, n, batch, &resid) == 0);
            CHECK(oracle_schoolbook(a, la, b, lb, d, batch) == 0);
            CHECK(resid >= 0 && resid < 0.1);
            CHECK(memcmp(c, d, batch * lc * sizeof(int64_t)) == 0);
            int64_t ks[2] = {0, lc - 1}, cs[4];
            CHECK(oracle_schoolbook_sample(a, la, b, lb, batch, ks, 2, cs) == 0);
            CHECK(cs[0] == d[0] && cs[1] == d[lc - 1] && cs[2] == d[lc] && cs[3] == d[2 * lc - 1]);
            CHECK(oracle_polymul_fft(a, la, b, lb, c, n / 2 >= lc ? n / 2 : n - 1, batch, &resid) < 0 ||
                  n / 2 >= lc);
            free(a);
            free(b);
            free(c);
            free(d);
        }
    int64_t one = 1, k = 5, out = 0;
    CHECK(oracle_schoolbook_sample(&one, 1, &one, 1, 1, &k, 1, &out) < 0);
    CHECK(oracle_schoolbook(&one, 0, &one, 1, &out, 1) < 0);
}

int main(void)
{
    oracle_set_threads(2);
    check_1d();
    check_nd();
    check_poly();
    printf("oracle checks: %d failed\n", g_fail);
    return g_fail ? 1 : 0;
}
