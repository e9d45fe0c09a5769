// Host-side checks of the library under AddressSanitizer and UBSan, on the
// CPU: the planner (every path's layout for many shapes), the fp64 twiddle
// and schedule generators, and the argument validation of every entry point,
// none of which needs a GPU.  The library source is included whole so that
// its internal generators can be called; the kernel launchers come from the
// .hip files built host-only (they are never reached here).
//
// Built and run by tests/test_host_sanitizers.py.  Exit status 0 = all
// checks passed and the sanitizers reported nothing.
#include "api.cpp"

#include <cstdio>

static int g_fail = 0;
#define CHECK(c)                                                          \
    do {                                                                  \
        if (!(c)) {                                                       \
            std::fprintf(stderr, "check failed: %s (line %d)\n", #c, __LINE__); \
            ++g_fail;                                                     \
        }                                                                 \
    } while (0)

// w = e^{-2 pi i m / M}: |w| = 1, and w agrees with cos / sin of the angle
// formed directly (the generators reduce it first, so they may differ by a
// rounding or two of a value of size 1).
static void check_roots()
{
    for (int64_t M : {1, 2, 3, 4, 5, 7, 8, 12, 16, 1000, 1024, 4096, 1 << 20, 1 << 26})
        for (int64_t m = -3; m < std::min<int64_t>(M + 3, 5000); ++m) {
            double re, im, ra, ia;
            root_of_unity_any(m, M, &ra, &ia);
            const double th = -2.0 * M_PI * (double)(((m % M) + M) % M) / (double)M;
            CHECK(std::fabs(ra - std::cos(th)) < 1e-14 && std::fabs(ia - std::sin(th)) < 1e-14);
            CHECK(std::fabs(ra * ra + ia * ia - 1.0) < 1e-15);
            if ((M & (M - 1)) == 0) {
                root_of_unity(m, M, &re, &im);
                CHECK(std::fabs(re - ra) < 1e-15 && std::fabs(im - ia) < 1e-15);
            }
        }
    for (int64_t n : {1, 2, 3, 97, 1009, 100003})
        for (int64_t j = 0; j < std::min<int64_t>(2 * n, 3000); ++j) {
            double re, im;
            chirp_value(j, n, &re, &im);
            const double th = -M_PI * std::fmod((double)j * (double)j, 2.0 * (double)n) / (double)n;
            CHECK(std::fabs(re - std::cos(th)) < 1e-12 && std::fabs(im - std::sin(th)) < 1e-12);
        }
}

// Stage tables of every power-of-two length: entry [l][k] of stage s is
// w_{Ns R}^{k 2^l}.
static void check_stage_tables()
{
    for (int prec = 0; prec < 2; ++prec)
        for (int logn = 1; logn <= 13; ++logn) {
            const std::vector<double> t = stage_table(logn, prec);
            const int lem = plan_lem(prec);
            CHECK(t.size() == 2 * (size_t)plan_tw_entries(logn, lem));
            for (int s = 1; s < plan_nstages(logn, lem); ++s) {
                const int lr = plan_stage_logr(logn, lem, s);
                const int64_t ns = int64_t(1) << plan_stage_lns(logn, lem, s);
                for (int l = 0; l < lr; ++l)
                    for (int64_t k = 0; k < ns; ++k) {
                        const size_t e = 2 * (size_t)(plan_tw_offset(logn, lem, s) + l * ns + k);
                        double re, im, ra, ia;
                        root_of_unity(k << l, ns << lr, &re, &im);
                        root_of_unity_any(k << l, ns << lr, &ra, &ia);
                        CHECK(e + 1 < t.size() && t[e] == re && t[e + 1] == im);
                        CHECK(std::fabs(re - ra) < 1e-15 && std::fabs(im - ia) < 1e-15);
                    }
            }
        }
}

// Mixed-radix schedules and their twiddle tables for every 13-smooth length
// up to 20000, and the pass splits beyond.
static void check_mixed()
{
    for (int64_t n = 2; n <= 20000; ++n) {
        MixedSchedule ms{};
        if (!mixed_factor(n, &ms)) continue;
        int64_t prod = 1;
        for (int s = 0; s < ms.nst; ++s) {
            CHECK(ms.ns[s] == prod);
            prod *= ms.radix[s];
            CHECK(ms.stride[s] == n / ms.radix[s]);
        }
        CHECK(prod == n);
        const std::vector<double> tab = mixed_table(ms);
        CHECK(tab.size() == 2 * (size_t)std::max<int64_t>(1, mixed_table_entries(ms)));  // one unused entry if none
        for (double v : tab) CHECK(std::fabs(v) <= 1.0 + 1e-15);
        if (n > 8192) {
            int r[3] = {0, 0, 0};
            const int np = mixed_split(n, r);
            CHECK(np >= 0 && np <= 3);
            if (np) {
                int64_t p = 1;
                for (int q = 0; q < np; ++q) p *= r[q];
                CHECK(p == n);
            }
        }
    }
}

// The planner through the public host-only query, for every path.
static void check_query()
{
    char buf[512];
    int ok = 0;
    for (int prec = 0; prec < 2; ++prec) {
        for (int64_t n = 1; n <= 5000; ++n) {
            const int st = fft_plan_query(1, &n, prec, buf, sizeof buf);
            CHECK(st == FFT_OK || st == FFT_ERR_UNSUPPORTED_SIZE);
            ok += st == FFT_OK;
        }
        for (int l = 13; l <= 27; ++l) {
            const int64_t n = int64_t(1) << l;
            const int st = fft_plan_query(1, &n, prec, buf, sizeof buf);
            CHECK(st == (n <= max_n(prec) ? FFT_OK : FFT_ERR_UNSUPPORTED_SIZE));
        }
        for (int64_t n : {int64_t(1) << 23, (int64_t(1) << 23) - 1, int64_t(1000000), int64_t(8000000), int64_t(100003)}) {
            const int st = fft_plan_query(1, &n, prec, buf, sizeof buf);
            CHECK(st == FFT_OK || st == FFT_ERR_UNSUPPORTED_SIZE);
        }
        for (int64_t h = 1; h <= 8192; h *= 2)
            for (int64_t w = 1; w <= 8192; w *= 2) {
                const int64_t d2[2] = {h, w};
                const int st = fft_plan_query(2, d2, prec, buf, sizeof buf);
                CHECK(st == FFT_OK || st == FFT_ERR_UNSUPPORTED_SIZE);
            }
        for (int64_t h : {3, 12, 100, 720, 1000, 1080})
            for (int64_t w : {5, 20, 97, 1280, 1920}) {
                const int64_t d2[2] = {h, w};
                const int st = fft_plan_query(2, d2, prec, buf, sizeof buf);
                CHECK(st == FFT_OK || st == FFT_ERR_UNSUPPORTED_SIZE);
                const int64_t d3[3] = {h % 64 + 1, h, w};
                const int st3 = fft_plan_query(3, d3, prec, buf, sizeof buf);
                CHECK(st3 == FFT_OK || st3 == FFT_ERR_UNSUPPORTED_SIZE);
            }
        const int64_t bad[3] = {0, -1, 5};
        CHECK(fft_plan_query(1, bad, prec, buf, sizeof buf) == FFT_ERR_INVALID_ARG);
        CHECK(fft_plan_query(4, bad + 2, prec, buf, sizeof buf) == FFT_ERR_INVALID_ARG);
        CHECK(fft_plan_query(1, nullptr, prec, buf, sizeof buf) == FFT_ERR_INVALID_ARG);
        const int64_t tiny = 64;
        CHECK(fft_plan_query(1, &tiny, prec, buf, 4) == FFT_OK && std::strlen(buf) < 4);  // truncated
    }
    CHECK(ok > 1000);
}

// Validation of the exec calls on a plan built by the planner alone (no
// device tables): every error comes back before any HIP call.
static void check_validation()
{
    fft_plan p;
    const int64_t n = 1 << 20;
    CHECK(plan_prepare(&p, 1, &n, FFT_C32) == FFT_OK);
    void* in = (void*)(uintptr_t)(1 << 20);
    void* out = (void*)((uintptr_t)1 << 40);
    void* ws = (void*)((uintptr_t)1 << 44);
    CHECK(fft_exec_c2c(&p, 2, in, out, 1, ws, nullptr) == FFT_ERR_INVALID_ARG);
    CHECK(fft_exec_c2c(&p, 0, in, out, -1, ws, nullptr) == FFT_ERR_INVALID_ARG);
    CHECK(fft_exec_c2c(&p, 0, nullptr, out, 1, ws, nullptr) == FFT_ERR_INVALID_ARG);
    CHECK(fft_exec_c2c(&p, 0, (char*)in + 4, out, 1, ws, nullptr) == FFT_ERR_ALIGN);
    CHECK(fft_exec_c2c(&p, 0, in, (char*)in + 8, 1, ws, nullptr) == FFT_ERR_OVERLAP);
    CHECK(fft_exec_c2c(&p, 0, in, out, 1, nullptr, nullptr) == FFT_ERR_WORKSPACE);
    CHECK(fft_exec_c2c(&p, 0, in, out, 1, in, nullptr) == FFT_ERR_WORKSPACE);
    CHECK(fft_exec_c2c(&p, 0, in, out, 0, nullptr, nullptr) == FFT_OK);
    CHECK(fft_exec_2d(&p, 0, in, out, 1, ws, nullptr) == FFT_ERR_RANK);
    CHECK(fft_exec_c2c_noalloc(&p, 0, in, out, 17 << 4, nullptr) == FFT_ERR_WORKSPACE);
    size_t bytes = 0;
    CHECK(fft_workspace_size(&p, 3, &bytes) == FFT_OK && bytes == 3 * (size_t)n * 8);
    CHECK(fft_workspace_size(&p, INT64_MAX, &bytes) == FFT_ERR_INVALID_ARG);
    CHECK(fft_poly_mul(&p, (const int64_t*)in, 10, (const int64_t*)in, 10, (int64_t*)out, 1, ws, nullptr,
                       nullptr) == FFT_ERR_PRECISION);
    CHECK(fft_stream_copy(in, out, 12, nullptr) == FFT_ERR_ALIGN);
    for (int st = -10; st <= 1; ++st) CHECK(fft_status_string(st) != nullptr);
    CHECK(std::strlen(fft_last_error()) > 0);
}

int main()
{
    check_roots();
    check_stage_tables();
    check_mixed();
    check_query();
    check_validation();
    // A valid plan on a host without a GPU: FFT_ERR_DEVICE, not a crash.
    fft_plan* plan = nullptr;
    const int64_t n = 4096;
    const int st = fft_plan_create(&plan, 1, &n, FFT_C32);
    CHECK(st == FFT_ERR_DEVICE || st == FFT_OK);
    if (plan) fft_plan_destroy(plan);
    std::printf("host checks: %d failed\n", g_fail);
    return g_fail ? 1 : 0;
}
