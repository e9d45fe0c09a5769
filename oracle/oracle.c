/*
 * oracle.c -- plain fp64 CPU reference for the FFT library.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product path may include, link or
 * call this file; only the tests, the smoke check and the benchmark's CPU
 * baseline use it.  It shares no code, header, table or constant with the HIP
 * library: every twiddle here is computed from libm cos/sin on the spot.
 *
 * Every routine follows a passage of the pages:
 *   - "FFT on GPU" (elwhyjay.github.io/post/fft), section "Discrete Fourier
 *     Transform": X_k = sum_n x_n e^{-i 2 pi k n / N}          -> oracle_dft_direct
 *   - same page, section "Fast Fourier Transform": even/odd split,
 *     X_k = E_k + w^k O_k, X_{k+N/2} = E_k - w^k O_k            -> oracle_fft (recursive)
 *   - same page, section on why roots of unity are chosen: inverse is
 *     w -> w^{-1} and a factor 1/N                              -> inverse flag
 *   - same page, section on polynomial multiplication: c_k = sum_i a_i b_{k-i};
 *     forward both, pointwise product, inverse                  -> oracle_polymul_*,
 *                                                                  oracle_schoolbook_*
 *   - "Stockham FFT Butterfly Algorithm in Parallel GLSL", section
 *     "Multi-Dimensional Transforms and Separability": rows, then columns
 *     (2D), and one axis after another for 3D data       -> oracle_fft2, oracle_fft3
 *
 * The ORACLE_PLANT_* macros exist only so that a test can build a throw-away
 * copy with one plausible mistake planted and check that the pins catch it;
 * the oracle proper is always built with none of them defined.
 *
 * Complex data are interleaved (re, im) doubles.  All routines return 0 on
 * success and a negative value on bad arguments.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#include <omp.h>

static const double TWO_PI = 6.283185307179586476925286766559;

static int is_pow2(int64_t n) { return n > 0 && (n & (n - 1)) == 0; }

void oracle_set_threads(int n) { if (n > 0) omp_set_num_threads(n); }
int oracle_get_threads(void) { return omp_get_max_threads(); }

/* ------------------------------------------------------------------------ */
/* Direct DFT, O(N^2) ("FFT on GPU", Discrete Fourier Transform).  The       */
/* product k*n is reduced mod N in integers first, so the angle 2 pi m / N   */
/* never carries the rounding of a large k*n.  Works for any N >= 1.         */
/* ------------------------------------------------------------------------ */
static void dft_direct_row(const double* x, double* X, int64_t n, int inverse)
{
    const double sgn = inverse ? 1.0 : -1.0;
    for (int64_t k = 0; k < n; ++k) {
        double sr = 0.0, si = 0.0;
        for (int64_t t = 0; t < n; ++t) {
            int64_t m = (k * t) % n;
            double ang = TWO_PI * ((double)m / (double)n);
            double wr = cos(ang), wi = sgn * sin(ang);
            double xr = x[2 * t], xi = x[2 * t + 1];
            sr += xr * wr - xi * wi;
            si += xr * wi + xi * wr;
        }
        if (inverse) { sr /= (double)n; si /= (double)n; }
        X[2 * k] = sr;
        X[2 * k + 1] = si;
    }
}

int oracle_dft_direct(const double* x, double* X, int64_t n, int64_t batch, int inverse)
{
    if (n < 1 || batch < 0 || !x || !X || x == X) return -1;
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t b = 0; b < batch; ++b)
        dft_direct_row(x + 2 * n * b, X + 2 * n * b, n, inverse);
    return 0;
}

/* Selected outputs of the direct DFT: X[b][j] = X_{ks[j]} of row b (any N),
 * each one by the definition in O(N). */
int oracle_dft_sample(const double* x, int64_t n, int64_t batch, const int64_t* ks, int64_t nk,
                      double* X, int inverse)
{
    if (n < 1 || batch < 0 || nk < 0 || !x || !ks || !X) return -1;
    for (int64_t j = 0; j < nk; ++j)
        if (ks[j] < 0 || ks[j] >= n) return -1;
    const double sgn = inverse ? 1.0 : -1.0;
#pragma omp parallel for collapse(2) schedule(dynamic, 4)
    for (int64_t b = 0; b < batch; ++b)
        for (int64_t j = 0; j < nk; ++j) {
            const int64_t k = ks[j];
            const double* xr = x + 2 * n * b;
            double sr = 0.0, si = 0.0;
            for (int64_t t = 0; t < n; ++t) {
                const int64_t m = (int64_t)(((unsigned __int128)k * (unsigned __int128)t) % (unsigned __int128)n);
                const double ang = TWO_PI * ((double)m / (double)n);
                const double wr = cos(ang), wi = sgn * sin(ang);
                sr += xr[2 * t] * wr - xr[2 * t + 1] * wi;
                si += xr[2 * t] * wi + xr[2 * t + 1] * wr;
            }
            if (inverse) { sr /= (double)n; si /= (double)n; }
            X[2 * (b * nk + j)] = sr;
            X[2 * (b * nk + j) + 1] = si;
        }
    return 0;
}

/* ------------------------------------------------------------------------ */
/* Recursive radix-2 decimation in time ("FFT on GPU", Fast Fourier          */
/* Transform).  The transform of x[0], x[s], x[2s], ... (n points) is built  */
/* from the transforms of its even-indexed and odd-indexed halves:           */
/*   E = DFT_{n/2}(x[0], x[2s], ...),  O = DFT_{n/2}(x[s], x[3s], ...)       */
/*   X_k = E_k + w_n^k O_k,  X_{k+n/2} = E_k - w_n^k O_k,  w_n = e^{-2 pi i/n} */
/* E is written to out[0, n/2) and O to out[n/2, n); the combine for index k */
/* reads only out[k] and out[k+n/2], so it is done in place.                 */
/*                                                                          */
/* tw[2*q] + i tw[2*q+1] = e^{sgn 2 pi i q / N} for q < N/2 (N = top size).  */
/* For a sub-transform of size n, w_n^k = w_N^{k N/n}: k/n and (kN/n)/N are  */
/* the same dyadic rational, so the table entry is exactly the value that    */
/* cos/sin of 2 pi k / n would give.                                          */
/* ------------------------------------------------------------------------ */
static void fft_rec(const double* x, int64_t stride, double* out, int64_t n,
                    const double* tw, int64_t tw_step, int par_depth)
{
    if (n == 1) {
        out[0] = x[0];
        out[1] = x[1];
        return;
    }
    const int64_t h = n / 2;
    if (par_depth > 0) {
#pragma omp task
        fft_rec(x, 2 * stride, out, h, tw, 2 * tw_step, par_depth - 1);
#pragma omp task
        fft_rec(x + 2 * stride, 2 * stride, out + 2 * h, h, tw, 2 * tw_step, par_depth - 1);
#pragma omp taskwait
    } else {
#ifdef ORACLE_PLANT_TWIDDLE_STEP
        /* planted mistake: sub-transforms keep the parent's twiddle step */
        fft_rec(x, 2 * stride, out, h, tw, tw_step, 0);
        fft_rec(x + 2 * stride, 2 * stride, out + 2 * h, h, tw, tw_step, 0);
#else
        fft_rec(x, 2 * stride, out, h, tw, 2 * tw_step, 0);
        fft_rec(x + 2 * stride, 2 * stride, out + 2 * h, h, tw, 2 * tw_step, 0);
#endif
    }
    for (int64_t k = 0; k < h; ++k) {
        const double wr = tw[2 * k * tw_step], wi = tw[2 * k * tw_step + 1];
        const double er = out[2 * k], ei = out[2 * k + 1];
        const double or_ = out[2 * (k + h)], oi = out[2 * (k + h) + 1];
#ifdef ORACLE_PLANT_CONJ_PRODUCT
        const double tr = wr * or_ + wi * oi;   /* planted mistake: w* o */
        const double ti = wr * oi - wi * or_;
#else
        const double tr = wr * or_ - wi * oi;
        const double ti = wr * oi + wi * or_;
#endif
        out[2 * k] = er + tr;
        out[2 * k + 1] = ei + ti;
        out[2 * (k + h)] = er - tr;
        out[2 * (k + h) + 1] = ei - ti;
    }
}

/* e^{sgn 2 pi i q / n}, q < n/2, from libm in fp64. */
static double* make_roots(int64_t n, int inverse)
{
    const int64_t h = n / 2 > 0 ? n / 2 : 1;
    double* tw = (double*)malloc(sizeof(double) * 2 * h);
    if (!tw) return NULL;
    double sgn = inverse ? 1.0 : -1.0;
#ifdef ORACLE_PLANT_TWIDDLE_SIGN
    sgn = -sgn;   /* planted mistake, only in a test's throw-away build */
#endif
    for (int64_t q = 0; q < h; ++q) {
        double ang = TWO_PI * ((double)q / (double)n);
        tw[2 * q] = cos(ang);
        tw[2 * q + 1] = sgn * sin(ang);
    }
    return tw;
}

static void fft_one(const double* x, double* X, int64_t n, const double* tw,
                    int inverse, int par_depth)
{
    if (par_depth > 0) {
#pragma omp parallel
#pragma omp single
        fft_rec(x, 1, X, n, tw, 1, par_depth);
    } else {
        fft_rec(x, 1, X, n, tw, 1, 0);
    }
#ifndef ORACLE_PLANT_NO_INVERSE_SCALE
    if (inverse) {
        const double s = 1.0 / (double)n;
        for (int64_t i = 0; i < 2 * n; ++i) X[i] *= s;
    }
#endif
}

/* Batched 1D transform of `batch` contiguous rows of n points (n a power of
 * two).  Forward uses e^{-i}, inverse e^{+i} and 1/n.  Rows are independent,
 * so they are spread over threads; a single row is split over threads at the
 * top recursion levels instead. */
int oracle_fft(const double* x, double* X, int64_t n, int64_t batch, int inverse)
{
    if (!is_pow2(n) || batch < 0 || !x || !X || x == X) return -1;
    double* tw = make_roots(n, inverse);
    if (!tw) return -2;
    if (batch == 1 && n >= (1 << 16)) {
        fft_one(x, X, n, tw, inverse, 6);
    } else {
#pragma omp parallel for schedule(dynamic, 1)
        for (int64_t b = 0; b < batch; ++b)
            fft_one(x + 2 * n * b, X + 2 * n * b, n, tw, inverse, 0);
    }
    free(tw);
    return 0;
}

/* ------------------------------------------------------------------------ */
/* Separable 2D transform ("Stockham FFT ... in Parallel GLSL",              */
/* Multi-Dimensional Transforms and Separability): the 1D transform along    */
/* each row (length W), then along each column (length H).  x is            */
/* [batch][H][W] row-major.  The inverse applies 1/W in the row pass and     */
/* 1/H in the column pass, i.e. 1/(H W) overall.                             */
/* ------------------------------------------------------------------------ */
int oracle_fft2(const double* x, double* X, int64_t h, int64_t w, int64_t batch, int inverse)
{
    if (!is_pow2(h) || !is_pow2(w) || batch < 0 || !x || !X || x == X) return -1;
    double* twr = make_roots(w, inverse);
    double* twc = make_roots(h, inverse);
    if (!twr || !twc) { free(twr); free(twc); return -2; }
    for (int64_t b = 0; b < batch; ++b) {
        const double* xi = x + 2 * h * w * b;
        double* Xi = X + 2 * h * w * b;
#pragma omp parallel for schedule(static)
        for (int64_t y = 0; y < h; ++y)
            fft_one(xi + 2 * w * y, Xi + 2 * w * y, w, twr, inverse, 0);
#pragma omp parallel
        {
            double* col = (double*)malloc(sizeof(double) * 2 * h);
            double* res = (double*)malloc(sizeof(double) * 2 * h);
#pragma omp for schedule(static)
            for (int64_t c = 0; c < w; ++c) {
                for (int64_t y = 0; y < h; ++y) {
                    col[2 * y] = Xi[2 * (y * w + c)];
                    col[2 * y + 1] = Xi[2 * (y * w + c) + 1];
                }
                fft_one(col, res, h, twc, inverse, 0);
                for (int64_t y = 0; y < h; ++y) {
                    Xi[2 * (y * w + c)] = res[2 * y];
                    Xi[2 * (y * w + c) + 1] = res[2 * y + 1];
                }
            }
            free(col);
            free(res);
        }
    }
    free(twr);
    free(twc);
    return 0;
}

/* ------------------------------------------------------------------------ */
/* Separable 3D transform: the same separability ("Stockham FFT ... in      */
/* Parallel GLSL" names 2D and 3D data), one axis after another: the 2D      */
/* transform of every depth slice [h][w], then the 1D transform along the    */
/* depth axis of every (y, x).  x is [batch][d][h][w]; the inverse scales by  */
/* 1/(d h w) (1/d here, 1/(h w) inside the 2D step).                          */
/* ------------------------------------------------------------------------ */
int oracle_fft3(const double* x, double* X, int64_t d, int64_t h, int64_t w, int64_t batch, int inverse)
{
    if (!is_pow2(d) || !is_pow2(h) || !is_pow2(w) || batch < 0 || !x || !X || x == X) return -1;
    int rc = oracle_fft2(x, X, h, w, batch * d, inverse);
    if (rc) return rc;
    double* twd = make_roots(d, inverse);
    if (!twd) return -2;
    const int64_t plane = h * w;
    for (int64_t b = 0; b < batch; ++b) {
        double* Xi = X + 2 * d * plane * b;
#pragma omp parallel
        {
            double* col = (double*)malloc(sizeof(double) * 2 * d);
            double* res = (double*)malloc(sizeof(double) * 2 * d);
#pragma omp for schedule(static)
            for (int64_t p = 0; p < plane; ++p) {
                for (int64_t z = 0; z < d; ++z) {
                    col[2 * z] = Xi[2 * (z * plane + p)];
                    col[2 * z + 1] = Xi[2 * (z * plane + p) + 1];
                }
                fft_one(col, res, d, twd, inverse, 0);
                for (int64_t z = 0; z < d; ++z) {
                    Xi[2 * (z * plane + p)] = res[2 * z];
                    Xi[2 * (z * plane + p) + 1] = res[2 * z + 1];
                }
            }
            free(col);
            free(res);
        }
    }
    free(twd);
    return 0;
}

/* ------------------------------------------------------------------------ */
/* Polynomial multiplication ("FFT on GPU", polynomial multiplication and    */
/* whole-process sections).                                                  */
/* ------------------------------------------------------------------------ */

/* Exact coefficient c_k = sum_i a_i b_{k-i} (schoolbook), int64 arithmetic. */
int64_t oracle_schoolbook_coeff(const int64_t* a, int64_t la, const int64_t* b, int64_t lb, int64_t k)
{
    int64_t lo = k - (lb - 1);
    if (lo < 0) lo = 0;
    int64_t hi = k < la - 1 ? k : la - 1;
    int64_t s = 0;
    for (int64_t i = lo; i <= hi; ++i) s += a[i] * b[k - i];
    return s;
}

/* Full schoolbook product of `batch` pairs: c[batch][la+lb-1]. */
int oracle_schoolbook(const int64_t* a, int64_t la, const int64_t* b, int64_t lb,
                      int64_t* c, int64_t batch)
{
    if (la < 1 || lb < 1 || batch < 0 || !a || !b || !c) return -1;
    const int64_t lc = la + lb - 1;
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t p = 0; p < batch; ++p)
        for (int64_t k = 0; k < lc; ++k)
            c[p * lc + k] = oracle_schoolbook_coeff(a + p * la, la, b + p * lb, lb, k);
    return 0;
}

/* Sampled schoolbook: c_out[p*nk + j] = c_{ks[j]} of pair p. */
int oracle_schoolbook_sample(const int64_t* a, int64_t la, const int64_t* b, int64_t lb,
                             int64_t batch, const int64_t* ks, int64_t nk, int64_t* c_out)
{
    if (la < 1 || lb < 1 || batch < 0 || nk < 0 || !a || !b || !ks || !c_out) return -1;
    for (int64_t j = 0; j < nk; ++j)
        if (ks[j] < 0 || ks[j] > la + lb - 2) return -1;
#pragma omp parallel for collapse(2) schedule(dynamic, 16)
    for (int64_t p = 0; p < batch; ++p)
        for (int64_t j = 0; j < nk; ++j)
            c_out[p * nk + j] = oracle_schoolbook_coeff(a + p * la, la, b + p * lb, lb, ks[j]);
    return 0;
}

/* FFT route: zero-pad a and b to n >= la+lb-1, forward both (fp64), multiply
 * pointwise, inverse (which scales by 1/n), round the real part to the
 * nearest integer (ties to even, rint).  max_resid (nullable) receives the
 * largest |Re - rint(Re)| over all outputs. */
int oracle_polymul_fft(const int64_t* a, int64_t la, const int64_t* b, int64_t lb,
                       int64_t* c, int64_t n, int64_t batch, double* max_resid)
{
    if (la < 1 || lb < 1 || batch < 0 || !a || !b || !c) return -1;
    if (!is_pow2(n) || la + lb - 1 > n) return -1;
    const int64_t lc = la + lb - 1;
    double* twf = make_roots(n, 0);
    double* twi = make_roots(n, 1);
    if (!twf || !twi) { free(twf); free(twi); return -2; }
    double worst = 0.0;
#pragma omp parallel reduction(max : worst)
    {
        double* xa = (double*)calloc(2 * n, sizeof(double));
        double* xb = (double*)calloc(2 * n, sizeof(double));
        double* A = (double*)malloc(sizeof(double) * 2 * n);
        double* B = (double*)malloc(sizeof(double) * 2 * n);
#pragma omp for schedule(dynamic, 1)
        for (int64_t p = 0; p < batch; ++p) {
            memset(xa, 0, sizeof(double) * 2 * n);
            memset(xb, 0, sizeof(double) * 2 * n);
            for (int64_t i = 0; i < la; ++i) xa[2 * i] = (double)a[p * la + i];
            for (int64_t i = 0; i < lb; ++i) xb[2 * i] = (double)b[p * lb + i];
            fft_one(xa, A, n, twf, 0, 0);
            fft_one(xb, B, n, twf, 0, 0);
            for (int64_t k = 0; k < n; ++k) {
                const double ar = A[2 * k], ai = A[2 * k + 1];
                const double br = B[2 * k], bi = B[2 * k + 1];
                xa[2 * k] = ar * br - ai * bi;
                xa[2 * k + 1] = ar * bi + ai * br;
            }
            fft_one(xa, A, n, twi, 1, 0);
#ifdef ORACLE_PLANT_POLY_SHIFT
            for (int64_t k = 0; k < lc; ++k) {   /* planted mistake: off by one */
                const double v = A[2 * ((k + 1) % n)];
#else
            for (int64_t k = 0; k < lc; ++k) {
                const double v = A[2 * k];
#endif
                const double r = rint(v);
                c[p * lc + k] = (int64_t)r;
                const double d = fabs(v - r);
                if (d > worst) worst = d;
            }
        }
        free(xa);
        free(xb);
        free(A);
        free(B);
    }
    free(twf);
    free(twi);
    if (max_resid) *max_resid = worst;
    return 0;
}
