// api.cpp -- the C ABI of include/fftmi.h: argument validation, plans and
// their twiddle tables, and dispatch to the kernels.
//
// Every argument is validated before the first HIP call, so validation
// errors are reported the same way with or without a GPU.
#include "fftmi.h"

#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <mutex>
#include <new>
#include <string>
#include <vector>

#include "launch.hpp"
#include "radix_plan.hpp"

using namespace fftmi;

namespace {

thread_local std::string g_last_error;

int fail(int status, const char* fmt, ...) __attribute__((format(printf, 2, 3)));
int fail(int status, const char* fmt, ...)
{
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof buf, fmt, ap);
    va_end(ap);
    g_last_error = buf;
    return status;
}

int hip_fail(hipError_t e, const char* what)
{
    return fail(FFT_ERR_DEVICE, "%s: %s (%d)", what, hipGetErrorString(e), (int)e);
}

int ilog2(int64_t n)
{
    int l = 0;
    while ((int64_t(1) << l) < n) ++l;
    return l;
}

bool is_pow2(int64_t n) { return n > 0 && (n & (n - 1)) == 0; }

// e^{-2 pi i m / M} in fp64 for a power-of-two M, with the angle reduced to
// [0, pi/4] by the symmetries of the unit circle before calling libm, so the
// value carries one rounding of a small angle instead of the rounding of
// 2 pi m / M for large m.
void root_of_unity(int64_t m, int64_t M, double* re, double* im)
{
    m %= M;
    if (m < 0) m += M;
    double c, s;  // cos, sin of 2 pi m / M
    if (M < 8) {
        // multiples of an eighth of a turn
        const int q = (int)(m * (8 / M));
        static const double h = 0.70710678118654752440084436210485;
        static const double cs[8][2] = {{1, 0}, {h, h}, {0, 1}, {-h, h}, {-1, 0}, {-h, -h}, {0, -1}, {h, -h}};
        c = cs[q][0];
        s = cs[q][1];
    } else {
        const int64_t quarter = M / 4, eighth = M / 8;
        const int64_t quad = m / quarter, x = m % quarter;
        double cx, sx;
        if (x <= eighth) {
            const double th = 2.0 * M_PI * ((double)x / (double)M);
            cx = std::cos(th);
            sx = std::sin(th);
        } else {
            const double th = 2.0 * M_PI * ((double)(quarter - x) / (double)M);
            cx = std::sin(th);
            sx = std::cos(th);
        }
        switch (quad) {
            case 0: c = cx; s = sx; break;
            case 1: c = -sx; s = cx; break;
            case 2: c = -cx; s = -sx; break;
            default: c = sx; s = -cx; break;
        }
    }
    *re = c;
    *im = -s;
}

// e^{-2 pi i m / M} for any M >= 1: the angle, as p/q of a turn with q = 8M,
// is folded into [0, 1/8] of a turn with integer arithmetic before libm.
void root_of_unity_any(int64_t m, int64_t M, double* re, double* im)
{
    m %= M;
    if (m < 0) m += M;
    const int64_t q = 8 * M;
    int64_t p = 8 * m;
    double sin_sign = 1.0, cos_sign = 1.0;
    bool swap = false;
    if (2 * p > q) {  // theta in (pi, 2 pi): sin(2 pi - x) = -sin x
        p = q - p;
        sin_sign = -1.0;
    }
    if (4 * p > q) {  // theta in (pi/2, pi]: cos(pi - x) = -cos x
        p = q / 2 - p;
        cos_sign = -1.0;
    }
    if (8 * p > q) {  // theta in (pi/4, pi/2]: swap cos and sin
        p = q / 4 - p;
        swap = true;
    }
    const double th = 2.0 * M_PI * ((double)p / (double)q);
    const double c = swap ? std::sin(th) : std::cos(th);
    const double sn = swap ? std::cos(th) : std::sin(th);
    *re = cos_sign * c;
    *im = -sin_sign * sn;
}

// Radices of a mixed-radix plan: 8s, then 4, 2, then 9s, 3, 5s, 7s, 11s, 13s, and the
// per-stage span, stride, quotient magic and twiddle-table offset; false if N
// has another prime factor or needs more stages than the schedule holds.
bool mixed_factor(int64_t n, MixedSchedule* ms)
{
    ms->nst = 0;
    int64_t rest = n;
    const int order[9] = {8, 4, 2, 9, 3, 5, 7, 11, 13};
    for (int r : order) {
        while (rest % r == 0) {
            if (ms->nst == kMixedMaxStages) return false;
            ms->radix[ms->nst++] = r;
            rest /= r;
        }
    }
    if (rest != 1) return false;
    int64_t ns = 1, off = 0;
    for (int q = 0; q < ms->nst; ++q) {
        const int r = ms->radix[q];
        ms->ns[q] = (int)ns;
        ms->stride[q] = (int)(n / r);
        ms->magic[q] = ns > 1 ? (unsigned)(((uint64_t(1) << 32) + ns - 1) / ns) : 0u;
        ms->twoff[q] = (int)off;
        if (q > 0) off += ns * mixed_tw_slots(r);
        ns *= r;
    }
    return true;
}

// Entries of a mixed-radix twiddle table (see MixedSchedule).
int64_t mixed_table_entries(const MixedSchedule& ms)
{
    int64_t e = 0;
    for (int q = 1; q < ms.nst; ++q) e += (int64_t)ms.ns[q] * mixed_tw_slots(ms.radix[q]);
    return e;
}

// A mixed-radix twiddle table (see MixedSchedule), interleaved fp64: rows
// w_{ns R}^{r k}, r = 1 .. R-1, for k < ns, per stage s >= 1; pad entries 0
// (N = R alone has no table: one entry, unused).
std::vector<double> mixed_table(const MixedSchedule& ms)
{
    std::vector<double> t(2 * (size_t)std::max<int64_t>(1, mixed_table_entries(ms)), 0.0);
    for (int q = 1; q < ms.nst; ++q) {
        const int r = ms.radix[q];
        const int64_t ns = ms.ns[q];
        for (int64_t k = 0; k < ns; ++k)
            for (int j = 1; j < r; ++j) {
                const size_t e = (size_t)(ms.twoff[q] + k * mixed_tw_slots(r) + (j - 1));
                root_of_unity_any(j * k, ns * r, &t[2 * e], &t[2 * e + 1]);
            }
    }
    return t;
}

// Radices of a multi-pass mixed-radix plan: N = r[0] r[1] (r[2]), as few
// passes as possible, then as even as possible (the largest smallest factor),
// larger first; each radix at most kMixPassMax, or up to kMixPassWide where
// that saves a pass (two passes instead of three; one pass for an axis) and
// the radix has no factor 11 or 13 (whose wide-pass kernels would spill).
// Returns the pass count, 0 if none.
constexpr int kMixPassMax = 512;
constexpr int kMixPassWide = 1024;
static bool pass_radix_ok(int64_t r, int cap)
{
    return r <= kMixPassMax || (r <= cap && r % 11 != 0 && r % 13 != 0);
}
static int mixed_split_cap(int64_t n, int cap, int np_max, int* r)
{
    std::vector<int64_t> divs;
    for (int64_t d = 2; d <= cap && d < n; ++d)
        if (n % d == 0 && pass_radix_ok(d, cap)) divs.push_back(d);
    for (int np = 2; np <= np_max; ++np) {
        int64_t best[3] = {0, 0, 0}, best_min = 0;
        for (int64_t a : divs) {
            if (np == 2) {
                const int64_t b = n / a;
                if (b >= 2 && pass_radix_ok(b, cap) && std::min(a, b) > best_min) {
                    best_min = std::min(a, b);
                    best[0] = a;
                    best[1] = b;
                }
                continue;
            }
            for (int64_t b : divs) {
                if ((n / a) % b) continue;
                const int64_t c = n / a / b;
                if (c < 2 || !pass_radix_ok(c, cap)) continue;
                const int64_t m = std::min(a, std::min(b, c));
                if (m > best_min) {
                    best_min = m;
                    best[0] = a;
                    best[1] = b;
                    best[2] = c;
                }
            }
        }
        if (best_min > 0) {
            std::sort(best, best + np, [](int64_t x, int64_t y) { return x > y; });
            for (int q = 0; q < np; ++q) r[q] = (int)best[q];
            return np;
        }
    }
    return 0;
}

int mixed_split(int64_t n, int* r)
{
    if (mixed_split_cap(n, kMixPassMax, 2, r)) return 2;
    if (mixed_split_cap(n, kMixPassWide, 2, r)) return 2;
    return mixed_split_cap(n, kMixPassMax, 3, r);
}

// Passes of an axis of len points (len > 1): one up to kMixPassWide.
static int axis_split(int64_t len, int* r)
{
    if (pass_radix_ok(len, kMixPassWide)) {
        r[0] = (int)len;
        return 1;
    }
    return mixed_split(len, r);
}

// Host copy of the stage tables of radix_plan.hpp for N = 2^logn, as
// interleaved doubles: stage s >= 1 holds [l][k] = w_{Ns R}^{k 2^l}.
std::vector<double> stage_table(int logn, int prec)
{
    const int lem = plan_lem(prec);
    std::vector<double> t(2 * (size_t)plan_tw_entries(logn, lem));
    for (int s = 1; s < plan_nstages(logn, lem); ++s) {
        const int lr = plan_stage_logr(logn, lem, s);
        const int64_t ns = int64_t(1) << plan_stage_lns(logn, lem, s);
        const long off = plan_tw_offset(logn, lem, s);
        for (int l = 0; l < lr; ++l)
            for (int64_t k = 0; k < ns; ++k) {
                const size_t e = (size_t)(off + l * ns + k);
                root_of_unity(k << l, ns << lr, &t[2 * e], &t[2 * e + 1]);
            }
    }
    return t;
}

}  // namespace

enum PlanPath {
    PATH_COPY = 0,
    PATH_ROWS = 1,
    PATH_MULTIPASS = 2,
    PATH_ND = 3,
    PATH_BLUESTEIN = 4,
    PATH_REAL = 5,
    PATH_MIXED = 6,
    PATH_MIXPASS = 7,
    PATH_NDX = 8
};

// One super-stage pass of a multi-pass plan.
struct PassPlan {
    int logr = 0, logns = 0, kind = 0;
    // mixed-radix passes: radix r (its stage schedule ms), span ns
    int r = 0, ns = 0;
    MixedSchedule ms{};
    const void* tw = nullptr;  // stage table for 2^logr (owned by the plan's table list)
    void* big_hi = nullptr;    // tables for w_M, M = 2^(logns + logr) (owned)
    void* big_lo = nullptr;
    int big_lbits = 0;
};

struct fft_plan {
    int rank = 0;
    int64_t dims[3] = {1, 1, 1};
    int prec = 0;
    int device = 0;
    int path = PATH_COPY;
    int64_t n = 1;          // points per transform (H*W for 2D)
    int logn = 0;
    // rank 1, rows:      tw_a = stage table for N
    // rank 1, multipass: passes[], poly-mul four-step: tw_a = rows (N1), tw_b = columns (N2), big_* = w_N,
    //                    tw_c = rows of N1/2 (the half-length inverse)
    // rank 2:            tw_a = rows (W), tw_b = columns (Lc = H / F), big_* = w_H (F > 1)
    int log_a = 0, log_b = 0;
    void* tw_a = nullptr;
    void* tw_b = nullptr;
    void* big_hi = nullptr;
    void* big_lo = nullptr;
    int big_lbits = 0;
    // rank 2 / 3: the axes longer than 1, outer to inner (nd_k of them), and
    // tw_a = innermost axis, tw_b = next axis (length 2^log_b after the fold),
    // tw_c = outermost axis of three, big_* = w of the folded axis.
    int nd_k = 0;
    int eff_log[3] = {0, 0, 0};
    void* tw_c = nullptr;
    int logf = 0;  // log2 of the column super-stage folded into the row pass
    // the radix-2^logf column super-stage runs as a pass of its own (rows too
    // wide for F of them in LDS): rows, column stage, column pass
    bool col_split = false;
    // rank 1, any N (Bluestein): chirp c_j (N entries), B = F_M(b) (M entries),
    // the power-of-two plan of length M = 2^logm it runs on.
    int logm = 0;
    // set before the layout is chosen: a power-of-two plan beyond the LDS range
    // stays in super-stage passes (the chirp-z passes read its pass layout)
    bool passes_only = false;
    // mixed radix: the stage schedule; tw_a = its twiddle table
    MixedSchedule mixed{};
    // real rows of N = 2H points: inner = the complex plan of length H,
    // big_* = w_N, log_a = log2 H; real_fused: H within the rows kernel's range.
    bool real_fused = false;
    // real rows of odd N: inner = the complex plan of length N (any route);
    // rows are widened to complex in the workspace, transformed in place there
    // and the bins 0 .. (N - 1) / 2 copied out (C2R: the Hermitian extension,
    // the inverse, the real parts).
    bool real_odd = false;
    // real images [H][W] (rank 2): the W-point rows as above, then the H-point
    // columns over W/2 + 1 columns: tw_b = stage table for 2^log_b, logf > 0:
    // a radix-2^logf column stage first, col_* = tables for w_H.
    void* col_hi = nullptr;
    void* col_lo = nullptr;
    int col_lbits = 0;
    void* chirp = nullptr;
    void* bspec = nullptr;
    fft_plan* inner = nullptr;
    int npass = 0;
    PassPlan passes[8];
    void* pass_tw[8] = {nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr};
    // rank 2 / 3 with a dimension that is not a power of two: inner = the
    // rank-1 plan of the innermost axis (any length); then the other axes
    // longer than 1, inner to outer (nx_k of them): axis a of length nx_len[a]
    // and stride nx_stride[a] runs nx_np[a] super-stage passes,
    // passes[3a .. 3a + nx_np[a]) (span = stride x the axis's own span).
    int nx_k = 0;
    int64_t nx_len[2] = {1, 1}, nx_stride[2] = {1, 1};
    int nx_np[2] = {0, 0};
    // an axis whose length has a prime factor above 13 (nx_np = 0): brought
    // innermost by a transpose, transformed as rows by the rank-1 plan of its
    // length (chirp-z or any other route), and transposed back
    fft_plan* nx_plan[2] = {nullptr, nullptr};
    // real images outside the power-of-two route: inner = the real-row plan
    // of length W, then the column axis as above over the W/2 + 1 columns of
    // the half spectrum (nx_stride[0] = W/2 + 1)
    bool real_nd = false;
    size_t elem = 8;
};

// plan creation with the layout choice open to the library's own sub-plans
static int plan_create(fft_plan** out_plan, int rank, const int64_t* dims, int prec, bool passes_only);

namespace {

size_t elem_bytes(int prec) { return prec == FFT_C32 ? 8 : 16; }

int64_t max_lds_n(int prec) { return prec == FFT_C32 ? FFT_MAX_LDS_N_C32 : FFT_MAX_LDS_N_C64; }
// Rows of twice the LDS range (2^14 complex64 / 2^13 complex128 points) still
// run as one kernel: one 1024-thread workgroup holds a row in LDS (128 KiB +
// pad) -- rank-1 plans and the chirp-z rows only
int64_t big_row_n(int prec) { return prec == FFT_C32 ? int64_t(1) << 14 : int64_t(1) << 13; }
// the chirp-z route in one kernel per row (else on the M-point passes)
bool bluestein_fused(const fft_plan* p) { return (int64_t(1) << p->logm) <= big_row_n(p->prec); }
int64_t max_n(int prec) { return prec == FFT_C32 ? FFT_MAX_N_C32 : FFT_MAX_N_C64; }

// Upload interleaved fp64 values rounded to the plan precision.
int upload(const std::vector<double>& host, int prec, void** dev)
{
    *dev = nullptr;
    if (host.empty()) return FFT_OK;
    const size_t count = host.size();
    const size_t bytes = prec == FFT_C32 ? count * sizeof(float) : count * sizeof(double);
    std::vector<float> f;
    const void* src = host.data();
    if (prec == FFT_C32) {
        f.resize(count);
        for (size_t i = 0; i < count; ++i) f[i] = (float)host[i];
        src = f.data();
    }
    hipError_t e = hipMalloc(dev, bytes);
    if (e != hipSuccess) {
        *dev = nullptr;
        return hip_fail(e, "hipMalloc(twiddles)");
    }
    e = hipMemcpy(*dev, src, bytes, hipMemcpyHostToDevice);
    if (e != hipSuccess) {
        (void)hipFree(*dev);
        *dev = nullptr;
        return hip_fail(e, "hipMemcpy(twiddles)");
    }
    return FFT_OK;
}

void free_plan(fft_plan* p)
{
    if (!p) return;
    void* ptrs[] = {p->tw_a, p->tw_b, p->tw_c, p->big_hi, p->big_lo, p->chirp, p->bspec, p->col_hi, p->col_lo};
    for (void* q : ptrs)
        if (q) (void)hipFree(q);  // teardown: nothing to report a failure to
    for (int i = 0; i < 8; ++i) {
        if (p->pass_tw[i]) (void)hipFree(p->pass_tw[i]);
        if (p->passes[i].big_hi) (void)hipFree(p->passes[i].big_hi);
        if (p->passes[i].big_lo) (void)hipFree(p->passes[i].big_lo);
    }
    if (p->inner) free_plan(p->inner);
    for (fft_plan* q : p->nx_plan)
        if (q) free_plan(q);
    delete p;
}

// Tables for w_M^m = hi[m >> L] lo[m & (2^L - 1)], M = 2^logm, L = ceil(logm / 2)
// unless `want_lbits` >= 0 gives L.
int upload_big(int logm, int prec, void** hi_dev, void** lo_dev, int* lbits, int want_lbits = -1)
{
    *lbits = want_lbits >= 0 ? want_lbits : (logm + 1) / 2;
    const int64_t m = int64_t(1) << logm;
    const int64_t nlo = int64_t(1) << *lbits, nhi = m >> *lbits;
    std::vector<double> lo(2 * nlo), hi(2 * nhi);
    for (int64_t q = 0; q < nlo; ++q) root_of_unity(q, m, &lo[2 * q], &lo[2 * q + 1]);
    for (int64_t q = 0; q < nhi; ++q) root_of_unity(q << *lbits, m, &hi[2 * q], &hi[2 * q + 1]);
    int st = upload(lo, prec, lo_dev);
    if (st == FFT_OK) st = upload(hi, prec, hi_dev);
    return st;
}

// Two-level table for w_M^m, any M: lo[q] = w_M^q (q < 2^lbits), hi[q] =
// w_M^{q 2^lbits} (q < ceil(M / 2^lbits)).
int upload_big_any(int64_t m, int prec, void** hi_dev, void** lo_dev, int* lbits)
{
    int lm = 0;
    while ((int64_t(1) << lm) < m) ++lm;
    *lbits = (lm + 1) / 2;
    const int64_t nlo = int64_t(1) << *lbits, nhi = (m + nlo - 1) / nlo;
    std::vector<double> lo(2 * nlo), hi(2 * nhi);
    for (int64_t q = 0; q < nlo; ++q) root_of_unity_any(q, m, &lo[2 * q], &lo[2 * q + 1]);
    for (int64_t q = 0; q < nhi; ++q) root_of_unity_any(q * nlo, m, &hi[2 * q], &hi[2 * q + 1]);
    int st = upload(lo, prec, lo_dev);
    if (st == FFT_OK) st = upload(hi, prec, hi_dev);
    return st;
}

bool ranges_overlap(const void* a, size_t na, const void* b, size_t nb)
{
    const uintptr_t x = (uintptr_t)a, y = (uintptr_t)b;
    return x < y + nb && y < x + na;
}

// Common checks of an exec call; returns FFT_OK or an error, sets *noop.
int check_exec(const fft_plan* plan, int dir, int rank, const void* in, void* out, int64_t batch,
               void* workspace, size_t ws_needed, bool* noop)
{
    *noop = false;
    if (!plan) return fail(FFT_ERR_INVALID_ARG, "plan is NULL");
    if (dir != FFT_FORWARD && dir != FFT_INVERSE) return fail(FFT_ERR_INVALID_ARG, "dir %d is not FFT_FORWARD/FFT_INVERSE", dir);
    if (batch < 0) return fail(FFT_ERR_INVALID_ARG, "batch %lld < 0", (long long)batch);
    if (plan->path == PATH_REAL)
        return fail(FFT_ERR_RANK, "plan is for real rows: use fft_exec_r2c / fft_exec_c2r");
    if (plan->rank != rank)
        return fail(FFT_ERR_RANK, "plan has rank %d, this call needs rank %d", plan->rank, rank);
    if (batch == 0) {
        *noop = true;
        return FFT_OK;
    }
    if (!in || !out) return fail(FFT_ERR_INVALID_ARG, "in or out is NULL");
    if (batch > INT64_MAX / (int64_t)(plan->n * plan->elem))
        return fail(FFT_ERR_INVALID_ARG, "batch %lld overflows the buffer size", (long long)batch);
    if (((uintptr_t)in | (uintptr_t)out) % plan->elem)
        return fail(FFT_ERR_ALIGN, "in/out must be aligned to %zu bytes", plan->elem);
    const size_t bytes = (size_t)batch * (size_t)plan->n * plan->elem;
    if (in != out && ranges_overlap(in, bytes, out, bytes))
        return fail(FFT_ERR_OVERLAP, "in and out overlap partially");
    if (ws_needed) {
        if (!workspace) return fail(FFT_ERR_WORKSPACE, "workspace of %zu bytes required", ws_needed);
        if ((uintptr_t)workspace % plan->elem) return fail(FFT_ERR_ALIGN, "workspace misaligned");
        if (ranges_overlap(workspace, ws_needed, in, bytes) || ranges_overlap(workspace, ws_needed, out, bytes))
            return fail(FFT_ERR_WORKSPACE, "workspace overlaps in or out");
    }
    return FFT_OK;
}

int check_device(const fft_plan* plan)
{
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
    if (dev != plan->device)
        return fail(FFT_ERR_DEVICE, "plan was created on device %d, current device is %d", plan->device, dev);
    return FFT_OK;
}

// Workspace of an exec call: the multi-pass transform ping-pongs through one
// signal-sized buffer; the folded 2D transform needs one only in place.
size_t c2c_workspace(const fft_plan* p, int64_t batch);
size_t planar_ws(const fft_plan* p, int64_t batch);

// Rank 2 / 3, some dimension not a power of two: buffers for the axis passes
// (one signal-sized buffer when an axis takes two or more passes; planar
// calls a second one when it takes three), then the rows' own workspace.
size_t ndx_axis_buffers(const fft_plan* p, bool planar)
{
    int most = 0;
    for (int a = 0; a < p->nx_k; ++a) most = std::max(most, p->nx_np[a]);
    return most >= 3 && planar ? 2 : most >= 2 ? 1 : 0;
}
// Workspace of the axes transformed as rank-1 rows: the transposed signal,
// then the largest such axis plan's own workspace.
size_t ndx_transposed_ws(const fft_plan* p, int64_t batch)
{
    size_t most = 0;
    bool any = false;
    for (int a = 0; a < p->nx_k; ++a)
        if (p->nx_np[a] == 0 && p->nx_plan[a]) {
            any = true;
            most = std::max(most, c2c_workspace(p->nx_plan[a], batch * (p->n / p->nx_len[a])));
        }
    return any ? (size_t)batch * (size_t)p->n * p->elem + most : 0;
}

// [axis pass buffers][rows' workspace][transposed axes' workspace]
size_t ndx_workspace(const fft_plan* p, int64_t batch, bool planar)
{
    const size_t sig = (size_t)batch * (size_t)p->n * p->elem;
    const int64_t rows = batch * (p->n / p->dims[p->rank - 1]);
    const size_t rws = p->dims[p->rank - 1] == 1 ? 0 : planar ? planar_ws(p->inner, rows) : c2c_workspace(p->inner, rows);
    return ndx_axis_buffers(p, planar) * sig + rws + ndx_transposed_ws(p, batch);
}

size_t c2c_workspace(const fft_plan* p, int64_t batch)
{
    if (p->path == PATH_NDX) return ndx_workspace(p, batch, false);
    if (p->path == PATH_BLUESTEIN)  // none when M is within one workgroup (one kernel)
        return bluestein_fused(p)
                   ? 0
                   : ((size_t)batch << p->logm) * p->elem + c2c_workspace(p->inner, batch);
    if (p->path == PATH_REAL && p->rank == 2 && p->real_nd) {
        // [Z: the half spectrum (C2R)][Y: an axis of two or more passes, or
        // the transposed half spectrum][the rows' own][the transposed
        // columns' plan's own]
        const int64_t wc = p->dims[1] / 2 + 1;
        const size_t half = (size_t)batch * (size_t)p->dims[0] * (size_t)wc * p->elem;
        const bool tr = p->nx_k && p->nx_np[0] == 0;
        const size_t zy = p->nx_k ? half * (p->nx_np[0] == 1 ? 1 : 2) : 0;
        return zy + c2c_workspace(p->inner, batch * p->dims[0]) + (tr ? c2c_workspace(p->nx_plan[0], batch * wc) : 0);
    }
    if (p->path == PATH_REAL && p->rank == 2)  // the half spectrum of every image (C2R; R2C with a column stage)
        return p->dims[0] > 1 ? (size_t)batch * (size_t)p->dims[0] * (size_t)(p->dims[1] / 2 + 1) * p->elem : 0;
    if (p->path == PATH_REAL) {  // the H-point spectrum of every row, beyond the one-kernel range
        if (p->real_fused || p->n == 1) return 0;
        if (p->real_odd)  // the rows as complex signals, then the N-point plan's own workspace
            return (size_t)batch * (size_t)p->n * p->elem + c2c_workspace(p->inner, batch);
        const size_t z = (size_t)batch * (size_t)(p->n / 2) * p->elem;
        // lengths that are not powers of two: the H-point plan's own workspace after it
        return is_pow2(p->n) ? z : z + c2c_workspace(p->inner, batch);
    }
    const bool need = p->path == PATH_MULTIPASS || p->path == PATH_MIXPASS || (p->path == PATH_ND && p->logf > 0);
    return need ? (size_t)batch * (size_t)p->n * p->elem : 0;
}

// Workspace a rank-2/3 interleaved call needs: the folded layout only in
// place, the split layout always.
size_t nd_workspace(const fft_plan* p, int64_t batch, bool in_place)
{
    return p->col_split || in_place ? c2c_workspace(p, batch) : 0;
}

// Largest radix per super-stage pass, and the preferred / largest column
// length of the 2D column pass (LDS: lines of 128 bytes x length must fit).
// Columns of 512 points, the rest of the column transform folded into the
// row pass (F up to 8), measured fastest on MI355X for complex64 2048^2 x 8:
// 189 us against 209 us with 1024-point columns and 207 us with 256-point ones.
constexpr int kMaxPassLog = 9;
constexpr int kPolyMaxLog = 22;  // largest poly-mul transform, 2^22 points
constexpr int kPolyRowsMaxLog = 13;  // the fused poly-mul row kernels: N <= 8192
constexpr int64_t kBluesteinMax = FFT_MAX_BLUESTEIN_N;  // largest length that is not a power of two
int col_pref_log(int) { return 9; }
int col_cap_log(int prec) { return prec == FFT_C32 ? 11 : 10; }

// Rank 2 / 3 with a dimension that is not a power of two: the innermost axis
// as rank-1 rows, every other axis longer than 1 as super-stage passes over
// signals of (its length x its stride) points.
int ndx_layout(fft_plan* p, int rank, const int64_t* dims)
{
    p->path = PATH_NDX;
    p->nx_k = 0;
    int64_t stride = dims[rank - 1];
    for (int d = rank - 2; d >= 0; --d) {
        const int64_t len = dims[d];
        if (len > 1) {
            const int a = p->nx_k++;
            p->nx_len[a] = len;
            p->nx_stride[a] = stride;
            int rs[3] = {(int)len, 0, 0};
            MixedSchedule chk;
            const int np = mixed_factor(len, &chk) ? axis_split(len, rs) : 0;
            p->nx_np[a] = np;  // 0: transposed, the rank-1 plan of its length
            int64_t ns = 1;
            for (int q = 0; q < np; ++q) {
                PassPlan& pp = p->passes[3 * a + q];
                pp.r = rs[q];
                pp.ns = (int)(ns * stride);
                if (!mixed_factor(pp.r, &pp.ms))
                    return fail(FFT_ERR_UNSUPPORTED_SIZE, "no schedule for radix %d", pp.r);
                ns *= rs[q];
            }
        }
        stride *= len;
    }
    return FFT_OK;
}

// Chooses the kernel path and its sizes; host only.
int plan_layout(fft_plan* p, int rank, const int64_t* dims, int prec)
{
    if (rank > 1) {
        bool all_pow2 = true;
        for (int d = 0; d < rank; ++d) all_pow2 = all_pow2 && is_pow2(dims[d]);
        if (!all_pow2) return ndx_layout(p, rank, dims);
    }
    if (rank == 1) {
        const int64_t n = dims[0];
        if (!is_pow2(n)) {
            // lengths of 2, 3, 5, 7, 11 and 13 only: mixed radix, in one kernel
            // within one workgroup's LDS, else in 2-3 super-stage passes; any
            // other length: Bluestein
            int rs[3];
            int np = 0;
            if (n <= mixed_max_n(prec) && mixed_factor(n, &p->mixed)) {
                p->path = PATH_MIXED;
            } else if (n > mixed_max_n(prec) && mixed_factor(n, &p->mixed) && (np = mixed_split(n, rs)) > 0) {
                p->path = PATH_MIXPASS;
                p->npass = np;
                int64_t ns = 1;
                for (int q = 0; q < np; ++q) {
                    PassPlan& pp = p->passes[q];
                    pp.r = rs[q];
                    pp.ns = (int)ns;
                    if (!mixed_factor(pp.r, &pp.ms))
                        return fail(FFT_ERR_UNSUPPORTED_SIZE, "no pass schedule for n = %lld", (long long)n);
                    ns *= rs[q];
                }
            } else {
                p->path = PATH_BLUESTEIN;
                while ((int64_t(1) << p->logm) < 2 * n - 1) ++p->logm;
            }
        } else if (n == 1) {
            p->path = PATH_COPY;
        } else if (n <= max_lds_n(prec) || (n == big_row_n(prec) && !p->passes_only)) {
            p->path = PATH_ROWS;
            p->log_a = p->logn;
        } else {
            p->path = PATH_MULTIPASS;
            // Super-stages of at most 2^9 points, as even as possible, larger first.
            const int np = (p->logn + kMaxPassLog - 1) / kMaxPassLog;
            int logns = 0;
            for (int q = 0; q < np; ++q) {
                PassPlan& pp = p->passes[q];
                pp.logr = p->logn / np + (q < p->logn % np ? 1 : 0);
                pp.logns = logns;
                pp.kind = q == 0 ? 0 : (q == np - 1 ? 2 : 1);
                logns += pp.logr;
                const int c = tile_lines_2d(prec, pp.logr);
                const int64_t bfly = int64_t(1) << (p->logn - pp.logr);
                if (c <= 0 || bfly % c || (pp.kind == 1 && (int64_t(1) << pp.logns) % c))
                    return fail(FFT_ERR_UNSUPPORTED_SIZE, "no pass layout for n = %lld", (long long)p->n);
            }
            p->npass = np;
            // The poly-mul split N = N1 N2 (fp64 only): columns of at most 512
            // (1024 beyond 2^21) points, rows of at most 4096.
            if (prec == FFT_C64 && p->logn <= kPolyMaxLog) {
                p->log_b = std::min(9, (p->logn + 1) / 2);  // N2, the column length
                if (p->logn - p->log_b > 12) p->log_b = p->logn - 12;
                p->log_a = p->logn - p->log_b;               // N1, the row length
            }
        }
        return FFT_OK;
    }
    // Separable transform over rank 2 or 3 axes ("Stockham FFT ... in Parallel
    // GLSL", Multi-Dimensional Transforms and Separability).  Axes of length 1
    // drop out; the innermost remaining axis is contiguous.
    p->path = PATH_ND;
    for (int d = 0; d < rank; ++d)
        if (dims[d] > 1) p->eff_log[p->nd_k++] = ilog2(dims[d]);
    const int k = p->nd_k;
    if (k >= 1) p->log_a = p->eff_log[k - 1];
    if (k >= 2) {
        const int logh = p->eff_log[k - 2];
        if (logh > col_pref_log(prec)) {
            // Fold the radix-F column super-stage into the row pass: the column
            // pass then runs on H / F points.
            int lf = logh - col_pref_log(prec);
            while (lf > 0 && (lf > 3 || !fold_supported(prec, p->log_a, lf))) --lf;
            p->logf = lf;
        }
        p->log_b = logh - p->logf;
        if (p->log_b > col_cap_log(prec)) {
            // the fold cannot shorten the columns enough: the column
            // super-stage of radix up to 16 as a separate pass
            p->col_split = true;
            p->logf = std::min(4, logh - col_pref_log(prec));
            p->log_b = logh - p->logf;
        }
        if (p->log_b > col_cap_log(prec))
            return fail(FFT_ERR_UNSUPPORTED_SIZE, "no layout for a %lld-point axis over %lld-point rows",
                        1LL << logh, 1LL << p->log_a);
    }
    if (k == 3 && p->eff_log[0] > col_cap_log(prec))
        return fail(FFT_ERR_UNSUPPORTED_SIZE, "outer axis of %lld points exceeds %lld", 1LL << p->eff_log[0],
                    1LL << col_cap_log(prec));
    return FFT_OK;
}

// c_j = e^{-i pi j^2 / N} in fp64: j^2 is reduced mod 2N in integers and the
// angle folded into [0, pi/2] before libm is called.
void chirp_value(int64_t j, int64_t n, double* re, double* im)
{
    int64_t q = (int64_t)(((unsigned __int128)j * (unsigned __int128)j) % (unsigned __int128)(2 * n));
    double sign = 1.0;
    if (q >= n) {  // e^{-i pi (q - n)/N} e^{-i pi}
        q -= n;
        sign = -1.0;
    }
    double c, sn;  // cos, sin of pi q / N, q in [0, N)
    if (2 * q <= n) {
        const double th = M_PI * ((double)q / (double)n);
        c = std::cos(th);
        sn = std::sin(th);
    } else {
        const double th = M_PI * ((double)(n - q) / (double)n);
        c = -std::cos(th);
        sn = std::sin(th);
    }
    *re = sign * c;
    *im = -sign * sn;
}

// Bluestein tables: the chirp, and B = F_M(b) computed on the device with an
// fp64 power-of-two plan, rounded to the plan precision; plus the plan of
// length M the transforms run on.
int bluestein_tables(fft_plan* p)
{
    const int64_t n = p->n, m = int64_t(1) << p->logm;
    std::vector<double> c(2 * n), b(2 * m, 0.0);
    for (int64_t j = 0; j < n; ++j) chirp_value(j, n, &c[2 * j], &c[2 * j + 1]);
    for (int64_t j = 0; j < n; ++j) {
        b[2 * j] = c[2 * j];
        b[2 * j + 1] = -c[2 * j + 1];
        if (j > 0) {
            b[2 * (m - j)] = c[2 * j];
            b[2 * (m - j) + 1] = -c[2 * j + 1];
        }
    }
    int st = upload(c, p->prec, &p->chirp);
    if (st != FFT_OK) return st;
    void* bdev = nullptr;
    st = upload(b, FFT_C64, &bdev);
    if (st != FFT_OK) return st;
    fft_plan* sub = nullptr;
    const int64_t mdim = m;
    st = plan_create(&sub, 1, &mdim, FFT_C64, false);
    void* ws = nullptr;
    const size_t wsb = st == FFT_OK ? c2c_workspace(sub, 1) : 0;
    if (st == FFT_OK && wsb) {
        hipError_t e = hipMalloc(&ws, wsb);
        if (e != hipSuccess) st = hip_fail(e, "hipMalloc(plan workspace)");
    }
    if (st == FFT_OK) st = fft_exec_c2c(sub, FFT_FORWARD, bdev, bdev, 1, ws, nullptr);
    if (st == FFT_OK) {
        if (p->prec == FFT_C32) {
            hipError_t e = hipMalloc(&p->bspec, (size_t)m * 8);
            if (e != hipSuccess) st = hip_fail(e, "hipMalloc(bluestein table)");
            if (st == FFT_OK) {
                e = launch_narrow(bdev, p->bspec, m, nullptr);
                if (e != hipSuccess) st = hip_fail(e, "narrow");
            }
        } else {
            p->bspec = bdev;
            bdev = nullptr;
        }
    }
    if (st == FFT_OK) {
        hipError_t e = hipStreamSynchronize(nullptr);
        if (e != hipSuccess) st = hip_fail(e, "hipStreamSynchronize(plan)");
    }
    if (ws) (void)hipFree(ws);
    if (bdev) (void)hipFree(bdev);
    if (sub) fft_plan_destroy(sub);
    // beyond one workgroup the chirp-z route runs on the M-point passes
    if (st == FFT_OK) st = plan_create(&p->inner, 1, &mdim, p->prec, !bluestein_fused(p));
    return st;
}

// Builds and uploads the twiddle tables the layout needs.
int upload_tables(fft_plan* p)
{
    const int prec = p->prec;
    int st = FFT_OK;
    switch (p->path) {
        case PATH_COPY:
            break;
        case PATH_BLUESTEIN:
            st = bluestein_tables(p);
            break;
        case PATH_MIXED:
            st = upload(mixed_table(p->mixed), prec, &p->tw_a);
            break;
        case PATH_MIXPASS:
            for (int q = 0; q < p->npass && st == FFT_OK; ++q) {
                PassPlan& pp = p->passes[q];
                st = upload(mixed_table(pp.ms), prec, &p->pass_tw[q]);
                pp.tw = p->pass_tw[q];
                if (st == FFT_OK && q > 0)
                    st = upload_big_any((int64_t)pp.ns * pp.r, prec, &pp.big_hi, &pp.big_lo, &pp.big_lbits);
            }
            break;
        case PATH_NDX: {
            // the rows' plan, then each axis pass's tables: w_M with M = the
            // axis's own span x radix (the span over the stride)
            const int64_t w = p->dims[p->rank - 1];
            if (w > 1) st = fft_plan_create(&p->inner, 1, &w, prec);
            for (int a = 0; a < p->nx_k && st == FFT_OK; ++a)
                if (p->nx_np[a] == 0) st = fft_plan_create(&p->nx_plan[a], 1, &p->nx_len[a], prec);
            for (int a = 0; a < p->nx_k && st == FFT_OK; ++a)
                for (int q = 0; q < p->nx_np[a] && st == FFT_OK; ++q) {
                    PassPlan& pp = p->passes[3 * a + q];
                    st = upload(mixed_table(pp.ms), prec, &p->pass_tw[3 * a + q]);
                    pp.tw = p->pass_tw[3 * a + q];
                    if (st == FFT_OK && q > 0)
                        st = upload_big_any(pp.ns / p->nx_stride[a] * pp.r, prec, &pp.big_hi, &pp.big_lo,
                                            &pp.big_lbits);
                }
            break;
        }
        case PATH_ROWS:
            st = upload(stage_table(p->log_a, prec), prec, &p->tw_a);
            break;
        case PATH_MULTIPASS:
            for (int q = 0; q < p->npass && st == FFT_OK; ++q) {
                PassPlan& pp = p->passes[q];
                st = upload(stage_table(pp.logr, prec), prec, &p->pass_tw[q]);
                pp.tw = p->pass_tw[q];
                if (st == FFT_OK && q > 0) st = upload_big(pp.logns + pp.logr, prec, &pp.big_hi, &pp.big_lo, &pp.big_lbits);
            }
            if (st == FFT_OK && p->log_a > 0) {
                st = upload(stage_table(p->log_a, prec), prec, &p->tw_a);
                if (st == FFT_OK) st = upload(stage_table(p->log_b, prec), prec, &p->tw_b);
                if (st == FFT_OK) st = upload_big(p->logn, prec, &p->big_hi, &p->big_lo, &p->big_lbits);
                // rows of N1/2 points: the half-length inverse of the real product
                if (st == FFT_OK) st = upload(stage_table(p->log_a - 1, prec), prec, &p->tw_c);
            }
            break;
        default:
            if (p->nd_k >= 1) st = upload(stage_table(p->log_a, prec), prec, &p->tw_a);
            if (st == FFT_OK && p->nd_k >= 2) {
                st = upload(stage_table(p->log_b, prec), prec, &p->tw_b);
                if (st == FFT_OK && p->logf > 0)
                    st = upload_big(p->log_b + p->logf, prec, &p->big_hi, &p->big_lo, &p->big_lbits);
            }
            if (st == FFT_OK && p->nd_k == 3) st = upload(stage_table(p->eff_log[0], prec), prec, &p->tw_c);
            break;
    }
    return st;
}

}  // namespace

extern "C" {

const char* fft_status_string(int status)
{
    switch (status) {
        case FFT_OK: return "FFT_OK";
        case FFT_ERR_INVALID_ARG: return "FFT_ERR_INVALID_ARG: invalid argument";
        case FFT_ERR_NOT_POW2: return "FFT_ERR_NOT_POW2: length is not a power of two";
        case FFT_ERR_UNSUPPORTED_SIZE: return "FFT_ERR_UNSUPPORTED_SIZE: size outside the supported range";
        case FFT_ERR_PRECISION: return "FFT_ERR_PRECISION: operation needs another precision";
        case FFT_ERR_RANK: return "FFT_ERR_RANK: plan rank does not match the call";
        case FFT_ERR_ALIGN: return "FFT_ERR_ALIGN: pointer not aligned to its element size";
        case FFT_ERR_OVERLAP: return "FFT_ERR_OVERLAP: buffers overlap";
        case FFT_ERR_WORKSPACE: return "FFT_ERR_WORKSPACE: workspace missing or overlapping";
        case FFT_ERR_DEVICE: return "FFT_ERR_DEVICE: HIP call failed";
        default: return "unknown status";
    }
}

const char* fft_last_error(void) { return g_last_error.c_str(); }

// Validation and layout of a complex plan, on the host only: every size check
// happens here, before any HIP call.
static int plan_prepare(fft_plan* p, int rank, const int64_t* dims, int prec)
{
    if (rank < 1 || rank > 3) return fail(FFT_ERR_INVALID_ARG, "rank %d not supported (1, 2 or 3)", rank);
    if (!dims) return fail(FFT_ERR_INVALID_ARG, "dims is NULL");
    if (prec != FFT_C32 && prec != FFT_C64) return fail(FFT_ERR_INVALID_ARG, "precision %d unknown", prec);
    bool all_pow2 = true;
    for (int d = 0; d < rank; ++d) {
        if (dims[d] < 1) return fail(FFT_ERR_INVALID_ARG, "dims[%d] = %lld < 1", d, (long long)dims[d]);
        all_pow2 = all_pow2 && is_pow2(dims[d]);
    }
    if (rank > 1 && !all_pow2) {
        // the innermost axis: any length a rank-1 plan takes; the others:
        // 2^a 3^b 5^c 7^d 11^e 13^f, as at most three passes (axis_split)
        int64_t total = 1;
        for (int d = 0; d < rank; ++d) {
            total *= dims[d];
            if (total > max_n(prec))
                return fail(FFT_ERR_UNSUPPORTED_SIZE, "%lld points per transform exceed %lld", (long long)total,
                            (long long)max_n(prec));
        }
        const int64_t w = dims[rank - 1];
        if (!is_pow2(w) && w > kBluesteinMax)
            return fail(FFT_ERR_UNSUPPORTED_SIZE, "dims[%d] = %lld exceeds %lld", rank - 1, (long long)w,
                        (long long)kBluesteinMax);
        for (int d = 0; d < rank - 1; ++d) {
            if (dims[d] == 1) continue;
            MixedSchedule ms;
            int rs[3];
            // 13-smooth: super-stage passes; otherwise the rank-1 plan of the
            // length over the transposed axis
            if (!(mixed_factor(dims[d], &ms) && axis_split(dims[d], rs) > 0) && dims[d] > kBluesteinMax)
                return fail(FFT_ERR_UNSUPPORTED_SIZE, "dims[%d] = %lld exceeds %lld", d, (long long)dims[d],
                            (long long)kBluesteinMax);
        }
    }
    // the innermost axis of length > 1: its rows may take the one-kernel rows
    // of twice the LDS range; the other axes run as columns
    int inner = rank - 1;
    while (inner > 0 && dims[inner] == 1) --inner;
    for (int d = 0; d < rank; ++d) {
        if (!is_pow2(dims[d])) {
            if (rank > 1) continue;
            if (dims[d] > kBluesteinMax)
                return fail(FFT_ERR_UNSUPPORTED_SIZE, "length %lld (not a power of two) exceeds %lld",
                            (long long)dims[d], (long long)kBluesteinMax);
            continue;
        }
        const int64_t lim = rank == 1 || !all_pow2 ? max_n(prec) : d == inner ? big_row_n(prec) : max_lds_n(prec);
        if (dims[d] > lim)
            return fail(FFT_ERR_UNSUPPORTED_SIZE, "dims[%d] = %lld exceeds %lld", d, (long long)dims[d],
                        (long long)lim);
    }
    p->rank = rank;
    p->prec = prec;
    p->elem = elem_bytes(prec);
    p->n = 1;
    for (int d = 0; d < rank; ++d) {
        p->dims[d] = dims[d];
        p->n *= dims[d];
    }
    p->logn = ilog2(p->n);
    return plan_layout(p, rank, dims, prec);
}

int fft_plan_create(fft_plan** out_plan, int rank, const int64_t* dims, int prec)
{
    return plan_create(out_plan, rank, dims, prec, false);
}

static int plan_create(fft_plan** out_plan, int rank, const int64_t* dims, int prec, bool passes_only)
{
    if (!out_plan) return fail(FFT_ERR_INVALID_ARG, "plan pointer is NULL");
    *out_plan = nullptr;
    fft_plan* p = new (std::nothrow) fft_plan;
    if (!p) return fail(FFT_ERR_DEVICE, "out of host memory");
    p->passes_only = passes_only;
    // 1. Layout, on the host only.
    int st = plan_prepare(p, rank, dims, prec);
    if (st != FFT_OK) {
        delete p;
        return st;
    }
    // 2. Device tables.
    hipError_t e = hipGetDevice(&p->device);
    if (e != hipSuccess) {
        delete p;
        return hip_fail(e, "hipGetDevice");
    }
    st = upload_tables(p);
    if (st != FFT_OK) {
        free_plan(p);
        return st;
    }
    *out_plan = p;
    return FFT_OK;
}

int fft_plan_query(int rank, const int64_t* dims, int prec, char* buf, size_t len)
{
    if (!buf || len == 0) return fail(FFT_ERR_INVALID_ARG, "buf is NULL");
    fft_plan p;
    const int st = plan_prepare(&p, rank, dims, prec);
    if (st != FFT_OK) return st;
    return fft_plan_describe(&p, buf, len);
}

int fft_plan_destroy(fft_plan* plan)
{
    free_plan(plan);
    return FFT_OK;
}

int fft_plan_describe(const fft_plan* p, char* buf, size_t len)
{
    if (!p || !buf || len == 0) return fail(FFT_ERR_INVALID_ARG, "plan or buf is NULL");
    const char* prec = p->prec == FFT_C32 ? "c32" : "c64";
    switch (p->path) {
        case PATH_COPY:
            snprintf(buf, len, "rank=%d n=%lld prec=%s path=copy", p->rank, (long long)p->n, prec);
            break;
        case PATH_ROWS:
            snprintf(buf, len, "rank=1 n=%lld prec=%s path=rows stages=%d", (long long)p->n, prec,
                     plan_nstages(p->log_a, plan_lem(p->prec)));
            break;
        case PATH_BLUESTEIN:
            snprintf(buf, len, "rank=1 n=%lld prec=%s path=bluestein m=%lld %s", (long long)p->n, prec,
                     1LL << p->logm, bluestein_fused(p) ? "fused" : "passes");
            break;
        case PATH_MIXED: {
            int off = snprintf(buf, len, "rank=1 n=%lld prec=%s path=mixed radices=", (long long)p->n, prec);
            for (int q = 0; q < p->mixed.nst && off > 0 && (size_t)off < len; ++q)
                off += snprintf(buf + off, len - off, q ? "x%d" : "%d", p->mixed.radix[q]);
            break;
        }
        case PATH_REAL:
            if (p->real_nd) {
                int off = snprintf(buf, len, "real dims=%lldx%lld prec=%s path=real2dmixed rows=real %s",
                                   (long long)p->dims[0], (long long)p->dims[1], prec,
                                   !p->inner || p->inner->n == 1 ? "copy"
                                   : p->inner->real_odd ? "odd" : p->inner->real_fused ? "fused" : "pairs");
                if (p->nx_k && off > 0 && (size_t)off < len) {
                    off += snprintf(buf + off, len - off, " axis1=");
                    if (p->nx_np[0] == 0 && p->nx_plan[0]) {  // transposed: the rank-1 plan's route
                        char ab[160] = "?";
                        fft_plan_describe(p->nx_plan[0], ab, sizeof ab);
                        const char* at = strstr(ab, "path=");
                        if (at) memmove(ab, at + 5, strlen(at + 5) + 1);
                        off += snprintf(buf + off, len - off, "transposed[%s]", ab);
                    }
                    for (int q = 0; q < p->nx_np[0] && off > 0 && (size_t)off < len; ++q)
                        off += snprintf(buf + off, len - off, q ? "x%d" : "%d", p->passes[q].r);
                }
            } else if (p->rank == 2)
                snprintf(buf, len, "real dims=%lldx%lld prec=%s path=real2d col_stage=%d col_len=%lld folded=%d",
                         (long long)p->dims[0], (long long)p->dims[1], prec, 1 << p->logf,
                         p->dims[0] > 1 ? 1LL << p->log_b : 0LL,
                         p->logf > 0 && r2c_fold_supported(p->prec, p->log_a, p->logf) ? 1 : 0);
            else
                snprintf(buf, len, "real n=%lld prec=%s path=real %s", (long long)p->n, prec,
                         p->n == 1 ? "copy" : p->real_odd ? "odd" : p->real_fused ? "fused" : "pairs");
            break;
        case PATH_NDX: {
            // the rows' route, then each axis's radices
            fft_plan rows;
            const int64_t w = p->dims[p->rank - 1];
            char rb[160] = "copy";
            if (w > 1 && plan_prepare(&rows, 1, &w, p->prec) == FFT_OK) {
                fft_plan_describe(&rows, rb, sizeof rb);
                const char* at = strstr(rb, "path=");
                if (at) memmove(rb, at + 5, strlen(at + 5) + 1);
            }
            int off = snprintf(buf, len, "rank=%d dims=%lldx%lldx%lld prec=%s path=ndmixed rows=[%s]", p->rank,
                               (long long)p->dims[0], (long long)(p->rank > 1 ? p->dims[1] : 1),
                               (long long)(p->rank > 2 ? p->dims[2] : 1), prec, rb);
            for (int a = 0; a < p->nx_k && off > 0 && (size_t)off < len; ++a) {
                off += snprintf(buf + off, len - off, " axis%d=", a + 1);
                if (p->nx_np[a] == 0) {  // transposed: the route of the rank-1 plan of its length
                    fft_plan ax;
                    char ab[160] = "?";
                    if (plan_prepare(&ax, 1, &p->nx_len[a], p->prec) == FFT_OK) {
                        fft_plan_describe(&ax, ab, sizeof ab);
                        const char* at = strstr(ab, "path=");
                        if (at) memmove(ab, at + 5, strlen(at + 5) + 1);
                    }
                    off += snprintf(buf + off, len - off, "transposed[%s]", ab);
                }
                for (int q = 0; q < p->nx_np[a] && off > 0 && (size_t)off < len; ++q)
                    off += snprintf(buf + off, len - off, q ? "x%d" : "%d", p->passes[3 * a + q].r);
            }
            break;
        }
        case PATH_MIXPASS: {
            int off = snprintf(buf, len, "rank=1 n=%lld prec=%s path=mixpass radices=", (long long)p->n, prec);
            for (int q = 0; q < p->npass && off > 0 && (size_t)off < len; ++q)
                off += snprintf(buf + off, len - off, q ? "x%d" : "%d", p->passes[q].r);
            break;
        }
        case PATH_MULTIPASS: {
            int off = snprintf(buf, len, "rank=1 n=%lld prec=%s path=multipass radices=", (long long)p->n, prec);
            for (int q = 0; q < p->npass && off > 0 && (size_t)off < len; ++q)
                off += snprintf(buf + off, len - off, q ? "x%lld" : "%lld", 1LL << p->passes[q].logr);
            // the poly-mul split: rows N1 x columns N2
            if (p->log_a > 0 && off > 0 && (size_t)off < len)
                snprintf(buf + off, len - off, " poly=%lldx%lld", 1LL << p->log_a, 1LL << p->log_b);
            break;
        }
        default:
            snprintf(buf, len, "rank=%d dims=%lldx%lldx%lld prec=%s path=nd axes=%d %s=%d col_len=%lld",
                     p->rank, (long long)p->dims[0], (long long)(p->rank > 1 ? p->dims[1] : 1),
                     (long long)(p->rank > 2 ? p->dims[2] : 1), prec, p->nd_k, p->col_split ? "split" : "fold",
                     1 << p->logf, p->nd_k >= 2 ? 1LL << p->log_b : 0LL);
            break;
    }
    return FFT_OK;
}

int fft_workspace_size(const fft_plan* plan, int64_t batch, size_t* bytes)
{
    if (!plan || !bytes) return fail(FFT_ERR_INVALID_ARG, "plan or bytes is NULL");
    if (batch < 0) return fail(FFT_ERR_INVALID_ARG, "batch < 0");
    if (batch > INT64_MAX / (int64_t)(plan->n * plan->elem)) return fail(FFT_ERR_INVALID_ARG, "batch too large");
    *bytes = c2c_workspace(plan, batch);
    return FFT_OK;
}

// Rank-1 execution on validated arguments.  io.in_im / io.out_im non-NULL:
// planar arrays; the multi-pass path then runs its middle passes through the
// workspace (two signal-sized buffers for three passes) instead of `out`.
static int run_1d(const fft_plan* plan, bool inv, const Io& io, int64_t batch, void* workspace, hipStream_t s)
{
    const bool planar = io.in_im != nullptr;
    const double scale = 1.0 / (double)plan->n;
    hipError_t e = hipSuccess;
    switch (plan->path) {
        case PATH_COPY: {
            const size_t bytes = (size_t)batch * plan->elem;
            if (!planar) {
                if (io.in != io.out) e = hipMemcpyAsync(io.out, io.in, bytes, hipMemcpyDeviceToDevice, s);
            } else if (io.in != io.out || io.in_im != io.out_im) {
                e = hipMemcpyAsync(io.out, io.in, bytes / 2, hipMemcpyDeviceToDevice, s);
                if (e == hipSuccess) e = hipMemcpyAsync(io.out_im, io.in_im, bytes / 2, hipMemcpyDeviceToDevice, s);
            }
            break;
        }
        case PATH_ROWS:
            e = launch_rows(plan->prec, plan->log_a, inv, inv, io.in, io.out, batch, plan->tw_a, scale, s, io.in_im,
                            io.out_im);
            break;
        case PATH_MULTIPASS: {
            // Interleaved: in -> ws -> out (two passes) or in -> ws -> out -> out
            // (three, the last in place).  Planar: in -> ws -> out, or
            // in -> ws -> ws2 -> out.
            const size_t sig = (size_t)batch * (size_t)plan->n * plan->elem;
            void* ws2 = (char*)workspace + sig;
            const void* src = io.in;
            for (int q = 0; q < plan->npass && e == hipSuccess; ++q) {
                const PassPlan& pp = plan->passes[q];
                const bool last = q == plan->npass - 1;
                void* dst = q == 0 ? workspace : (last || !planar) ? io.out : ws2;
                const BigTwiddle big{pp.big_hi, pp.big_lo, pp.big_lbits, pp.logns + pp.logr};
                e = launch_stock_pass(plan->prec, pp.logr, pp.kind, src, dst, plan->logn, pp.logns, batch, pp.tw, big,
                                      inv && q == 0, inv && last, scale, s, q == 0 ? io.in_im : nullptr,
                                      last ? io.out_im : nullptr);
                src = dst;
            }
            break;
        }
        case PATH_MIXED:
            e = launch_mixed_rows(plan->prec, (int)plan->n, plan->mixed, inv, io.in, io.out, batch, plan->tw_a,
                                  scale, s, io.in_im, io.out_im);
            break;
        case PATH_MIXPASS: {
            // the buffers of the power-of-two multi-pass path: in -> ws -> out
            // (-> out, the last pass in place), planar in -> ws (-> ws2) -> out
            const size_t sig = (size_t)batch * (size_t)plan->n * plan->elem;
            void* ws2 = (char*)workspace + sig;
            const void* src = io.in;
            for (int q = 0; q < plan->npass && e == hipSuccess; ++q) {
                const PassPlan& pp = plan->passes[q];
                const int lines = mixed_pass_lines(plan->prec, pp.r);
                const bool last = q == plan->npass - 1;
                void* dst = q == 0 ? workspace : (last || !planar) ? io.out : ws2;
                MixedPassArgs a{};
                a.n = (int)plan->n;
                a.r = pp.r;
                a.ns = pp.ns;
                a.stride = (int)(plan->n / pp.r);
                a.tiles = (a.stride + lines - 1) / lines;
                a.tr = mixed_pass_threads(pp.ms, pp.r);
                a.rmagic = (unsigned)(((uint64_t(1) << 32) + pp.r - 1) / pp.r);
                a.conj_in = inv && q == 0;
                a.conj_out = inv && last;
                a.tdiv = 1;
                a.twiddle = q > 0;
                const BigTwiddle big{pp.big_hi, pp.big_lo, pp.big_lbits, 0};
                e = launch_mixed_pass(plan->prec, a, pp.ms, src, dst, batch, pp.tw, big, scale, s,
                                      q == 0 ? io.in_im : nullptr, last ? io.out_im : nullptr);
                src = dst;
            }
            break;
        }
        case PATH_BLUESTEIN: {
            // w = pad(x . c) ; w = F^{-1}(F(w) . B) ; X = c . w  (conjugated for the inverse)
            if (bluestein_fused(plan)) {  // one kernel
                e = launch_bluestein_rows(plan->prec, plan->logm, (int)plan->n, io.in, io.out, batch,
                                          plan->inner->tw_a, plan->chirp, plan->bspec, inv, scale, s, io.in_im,
                                          io.out_im);
                break;
            }
            // M beyond one workgroup: the M-point multi-pass transforms, the
            // chirp products and the product with B riding on their first and
            // last passes; buffers A, B of batch x M in the workspace.
            // forward:  x c -> A (-> B) -> conj(W B) in B
            // inverse:  B -> A (-> B) -> c conj(.) / M -> out
            const fft_plan* mp = plan->inner;
            const int np = mp->npass;
            void* A = workspace;
            void* B = (char*)workspace + ((size_t)batch << plan->logm) * plan->elem;
            const ChirpArgs c{io.in, io.in_im, io.out, io.out_im, plan->chirp, plan->bspec, plan->n, inv, inv, scale};
            const void* src = nullptr;
            for (int q = 0; q < np && e == hipSuccess; ++q) {
                const PassPlan& pp = mp->passes[q];
                const BigTwiddle big{pp.big_hi, pp.big_lo, pp.big_lbits, pp.logns + pp.logr};
                if (q == 0) {
                    e = launch_bluestein_pass(plan->prec, pp.logr, 0, nullptr, A, plan->logm, pp.logns, batch, pp.tw,
                                              big, c, s);
                    src = A;
                } else if (q == np - 1) {
                    e = launch_bluestein_pass(plan->prec, pp.logr, 2, src, B, plan->logm, pp.logns, batch, pp.tw, big,
                                              c, s);
                } else {
                    e = launch_stock_pass(plan->prec, pp.logr, pp.kind, src, B, plan->logm, pp.logns, batch, pp.tw,
                                          big, false, false, 1.0, s);
                    src = B;
                }
            }
            src = B;
            for (int q = 0; q < np && e == hipSuccess; ++q) {
                const PassPlan& pp = mp->passes[q];
                const BigTwiddle big{pp.big_hi, pp.big_lo, pp.big_lbits, pp.logns + pp.logr};
                if (q == np - 1) {
                    e = launch_bluestein_pass(plan->prec, pp.logr, 4, src, nullptr, plan->logm, pp.logns, batch,
                                              pp.tw, big, c, s);
                } else {
                    void* dst = q == 0 ? A : B;
                    e = launch_stock_pass(plan->prec, pp.logr, pp.kind, src, dst, plan->logm, pp.logns, batch, pp.tw,
                                          big, false, false, 1.0, s);
                    src = dst;
                }
            }
            break;
        }
        default:
            return fail(FFT_ERR_RANK, "plan path is not rank 1");
    }
    if (e != hipSuccess) return hip_fail(e, "rank-1 transform launch");
    return FFT_OK;
}

static int sync_if_asked(hipStream_t s, const char* what)
{
    if (getenv("FFTMI_SYNC")) {
        hipError_t e = hipStreamSynchronize(s);
        if (e != hipSuccess) return hip_fail(e, what);
    }
    return FFT_OK;
}

int fft_exec_c2c(const fft_plan* plan, int dir, const void* in, void* out, int64_t batch, void* workspace,
                 void* stream)
{
    bool noop = false;
    const size_t ws = plan && batch > 0 ? c2c_workspace(plan, batch) : 0;
    int st = check_exec(plan, dir, 1, in, out, batch, workspace, ws, &noop);
    if (st != FFT_OK || noop) return st;
    if ((st = check_device(plan)) != FFT_OK) return st;
    hipStream_t s = (hipStream_t)stream;
    const Io io{in, nullptr, out, nullptr};
    st = run_1d(plan, dir == FFT_INVERSE, io, batch, workspace, s);
    if (st != FFT_OK) return st;
    return sync_if_asked(s, "fft_exec_c2c (FFTMI_SYNC)");
}

// Rank-2/3 execution on validated arguments.  Interleaved: the intermediate
// lives in `out` (in the workspace for an in-place folded call).  Planar: the
// first pass reads the caller's planes into the workspace, later passes run
// there, the last writes the caller's planes.
// The passes of axis a of a plan with nx_* axes (signals of length x stride
// points, batch x n / that of them): src -> dst, one pass directly (in place
// when src == dst), two through y, three through y then y2 (planar) or dst
// (the last in place).  src_im / dst_im: planar arrays read by the first
// pass / written by the last.  scale 1/length on the inverse's last pass.
static hipError_t axis_passes(const fft_plan* plan, int a, bool inv, const void* src, const void* src_im, void* dst,
                              void* dst_im, void* y, void* y2, int64_t batch, hipStream_t s)
{
    const int np = plan->nx_np[a];
    const int64_t sig_pts = plan->nx_len[a] * plan->nx_stride[a];
    const int64_t nsig = batch * (plan->n / sig_pts);
    const void* cur = src;
    const void* cur_im = src_im;
    hipError_t e = hipSuccess;
    for (int q = 0; q < np && e == hipSuccess; ++q) {
        const PassPlan& pp = plan->passes[3 * a + q];
        const int lines = mixed_pass_lines(plan->prec, pp.r);
        const bool first = q == 0, last = q == np - 1;
        void* d = last ? dst : q == 0 ? y : (y2 ? y2 : dst);
        void* d_im = last ? dst_im : nullptr;
        MixedPassArgs ar{};
        ar.n = (int)sig_pts;
        ar.r = pp.r;
        ar.ns = pp.ns;
        ar.stride = (int)(sig_pts / pp.r);
        ar.tiles = (ar.stride + lines - 1) / lines;
        ar.tr = mixed_pass_threads(pp.ms, pp.r);
        ar.rmagic = (unsigned)(((uint64_t(1) << 32) + pp.r - 1) / pp.r);
        ar.conj_in = inv && first;
        ar.conj_out = inv && last;
        ar.tdiv = (int)plan->nx_stride[a];
        ar.twiddle = q > 0;
        const BigTwiddle big{pp.big_hi, pp.big_lo, pp.big_lbits, 0};
        e = launch_mixed_pass(plan->prec, ar, pp.ms, cur, d, nsig, pp.tw, big, 1.0 / (double)plan->nx_len[a], s,
                              first ? cur_im : nullptr, d_im);
        cur = d;
        cur_im = d_im;
    }
    return e;
}

// Rank 2 / 3 with a dimension that is not a power of two: the innermost axis
// as rank-1 rows (in -> out), then each other axis in passes over `out` (the
// first axis reads `in` when the rows are one point long).  Planar: the rows
// planar -> planar into out, the axes' first / last passes read / write the
// planes.  Workspace: [Y][Y2][the rows' own].
static int run_ndx(const fft_plan* plan, bool inv, const Io& io, int64_t batch, void* workspace, hipStream_t s)
{
    const bool planar = io.in_im != nullptr;
    const size_t sig = (size_t)batch * (size_t)plan->n * plan->elem;
    const size_t nbuf = ndx_axis_buffers(plan, planar);
    char* y = (char*)workspace;
    char* y2 = planar && nbuf >= 2 ? y + sig : nullptr;
    void* rows_ws = nbuf ? (void*)(y + nbuf * sig) : workspace;
    const int64_t w = plan->dims[plan->rank - 1];
    if (w > 1) {
        const int st = run_1d(plan->inner, inv, io, batch * (plan->n / w), rows_ws, s);
        if (st != FFT_OK) return st;
    }
    const int64_t rows = batch * (plan->n / w);
    char* tbuf = (char*)rows_ws + (w == 1 ? 0 : planar ? planar_ws(plan->inner, rows) : c2c_workspace(plan->inner, rows));
    void* tws = tbuf + sig;
    hipError_t e = hipSuccess;
    for (int a = 0; a < plan->nx_k && e == hipSuccess; ++a) {
        const bool from_in = a == 0 && w == 1;
        const void* src = from_in ? io.in : io.out;
        const void* src_im = from_in ? io.in_im : io.out_im;
        if (plan->nx_np[a] == 0) {
            // [m][L][S] -> [m][S][L], the L-point rows, and back
            const int64_t len = plan->nx_len[a], str = plan->nx_stride[a];
            const int64_t nmat = batch * (plan->n / (len * str));
            e = launch_transpose(plan->prec, src, src_im, tbuf, nullptr, len, str, nmat, s);
            if (e != hipSuccess) break;
            const Io tio{tbuf, nullptr, tbuf, nullptr};
            const int st = run_1d(plan->nx_plan[a], inv, tio, nmat * str, tws, s);
            if (st != FFT_OK) return st;
            e = launch_transpose(plan->prec, tbuf, nullptr, io.out, io.out_im, str, len, nmat, s);
            continue;
        }
        e = axis_passes(plan, a, inv, src, src_im, io.out, io.out_im, y, y2, batch, s);
    }
    if (e != hipSuccess) return hip_fail(e, "rank-2/3 transform launch");
    return FFT_OK;
}

static int run_nd(const fft_plan* plan, bool inv, const Io& io, int64_t batch, void* workspace, hipStream_t s)
{
    if (plan->path == PATH_NDX) return run_ndx(plan, inv, io, batch, workspace, s);
    const bool planar = io.in_im != nullptr;
    const double scale = 1.0 / (double)plan->n;
    const int k = plan->nd_k;
    const BigTwiddle none{nullptr, nullptr, 0, 0};
    hipError_t e = hipSuccess;
    if (k == 0) {
        const size_t bytes = (size_t)batch * plan->elem;
        if (!planar) {
            if (io.in != io.out) e = hipMemcpyAsync(io.out, io.in, bytes, hipMemcpyDeviceToDevice, s);
        } else if (io.in != io.out || io.in_im != io.out_im) {
            e = hipMemcpyAsync(io.out, io.in, bytes / 2, hipMemcpyDeviceToDevice, s);
            if (e == hipSuccess) e = hipMemcpyAsync(io.out_im, io.in_im, bytes / 2, hipMemcpyDeviceToDevice, s);
        }
    } else if (k == 1) {
        e = launch_rows(plan->prec, plan->log_a, inv, inv, io.in, io.out, batch, plan->tw_a, scale, s, io.in_im,
                        io.out_im);
    } else {
        // innermost axis (rows) + next axis (columns of stride W); the first
        // pass conjugates the input, the last conjugates and scales the output.
        const int64_t w = int64_t(1) << plan->log_a;
        const int logh = plan->log_b + plan->logf;
        const int64_t nimg = batch * (plan->n >> (plan->log_a + logh));
        const bool last2 = k == 2;
        // where the column pass writes: the caller's array when it is the last
        void* col_out = planar ? (last2 ? io.out : workspace) : io.out;
        void* col_out_im = planar && last2 ? io.out_im : nullptr;
        if (plan->col_split) {
            // rows (in -> ws), column super-stage (ws -> out, or a second
            // workspace for planar arrays), column pass (-> col_out)
            const size_t sig = (size_t)batch * (size_t)plan->n * plan->elem;
            void* mid = planar ? (char*)workspace + sig : io.out;
            const BigTwiddle hb{plan->big_hi, plan->big_lo, plan->big_lbits, logh};
            e = launch_rows(plan->prec, plan->log_a, inv, false, io.in, workspace, nimg << logh, plan->tw_a, 1.0, s,
                            io.in_im, nullptr);
            if (e == hipSuccess)
                e = launch_colstage(plan->prec, plan->logf, workspace, mid, nimg, w, plan->log_b, s);
            if (e == hipSuccess)
                e = launch_cols2d(plan->prec, plan->log_b, mid, col_out, nimg, w, plan->logf, plan->tw_b, hb,
                                  inv && last2, last2 ? scale : 1.0, s, col_out_im);
        } else if (plan->logf == 0) {
            void* mid = planar ? workspace : io.out;
            e = launch_rows(plan->prec, plan->log_a, inv, false, io.in, mid, nimg << logh, plan->tw_a, 1.0, s,
                            io.in_im, nullptr);
            if (e == hipSuccess)
                e = launch_cols2d(plan->prec, plan->log_b, mid, col_out, nimg, w, 0, plan->tw_b, none, inv && last2,
                                  last2 ? scale : 1.0, s, col_out_im);
        } else {
            void* mid = planar || io.in == io.out ? workspace : io.out;
            const BigTwiddle hb{plan->big_hi, plan->big_lo, plan->big_lbits, logh};
            e = launch_rows2d_fold(plan->prec, plan->log_a, plan->logf, io.in, mid, nimg, plan->log_b, plan->tw_a, inv,
                                   s, io.in_im);
            if (e == hipSuccess)
                e = launch_cols2d(plan->prec, plan->log_b, mid, col_out, nimg, w, plan->logf, plan->tw_b, hb,
                                  inv && last2, last2 ? scale : 1.0, s, col_out_im);
        }
        // outer axis of three: columns of stride H W, in place (or into the planes)
        if (e == hipSuccess && k == 3)
            e = launch_cols2d(plan->prec, plan->eff_log[0], col_out, io.out, batch, w << logh, 0, plan->tw_c, none,
                              inv, scale, s, io.out_im);
    }
    if (e != hipSuccess) return hip_fail(e, "multi-dimensional transform launch");
    return FFT_OK;
}

static int exec_nd(const fft_plan* plan, int rank, const char* what, int dir, const void* in, void* out,
                   int64_t batch, void* workspace, void* stream)
{
    bool noop = false;
    const size_t ws = !plan || batch <= 0 ? 0
                      : plan->path == PATH_ND ? nd_workspace(plan, batch, in == out)
                      : plan->path == PATH_NDX ? c2c_workspace(plan, batch) : 0;
    int st = check_exec(plan, dir, rank, in, out, batch, workspace, ws, &noop);
    if (st != FFT_OK || noop) return st;
    if ((st = check_device(plan)) != FFT_OK) return st;
    hipStream_t s = (hipStream_t)stream;
    st = run_nd(plan, dir == FFT_INVERSE, Io{in, nullptr, out, nullptr}, batch, workspace, s);
    if (st != FFT_OK) return st;
    return sync_if_asked(s, what);
}

int fft_exec_2d(const fft_plan* plan, int dir, const void* in, void* out, int64_t batch, void* workspace,
                void* stream)
{
    return exec_nd(plan, 2, "fft_exec_2d", dir, in, out, batch, workspace, stream);
}

int fft_exec_3d(const fft_plan* plan, int dir, const void* in, void* out, int64_t batch, void* workspace,
                void* stream)
{
    return exec_nd(plan, 3, "fft_exec_3d", dir, in, out, batch, workspace, stream);
}

// Workspace of a planar call: the interleaved intermediates the multi-kernel
// paths keep between their first (planar-reading) and last (planar-writing) pass.
static size_t planar_workspace(const fft_plan* p, int64_t batch)
{
    const size_t sig = (size_t)batch * (size_t)p->n * p->elem;
    switch (p->path) {
        case PATH_MULTIPASS:
        case PATH_MIXPASS: return p->npass >= 3 ? 2 * sig : sig;
        case PATH_BLUESTEIN: return c2c_workspace(p, batch);
        case PATH_ND: return p->nd_k >= 2 ? (p->col_split ? 2 * sig : sig) : 0;
        case PATH_NDX: return ndx_workspace(p, batch, true);
        default: return 0;
    }
}

namespace {
size_t planar_ws(const fft_plan* p, int64_t batch) { return planar_workspace(p, batch); }
}  // namespace

int fft_planar_workspace_size(const fft_plan* plan, int64_t batch, size_t* bytes)
{
    if (!plan || !bytes) return fail(FFT_ERR_INVALID_ARG, "plan or bytes is NULL");
    if (plan->path == PATH_REAL) return fail(FFT_ERR_RANK, "plan is for real rows");
    if (batch < 0) return fail(FFT_ERR_INVALID_ARG, "batch < 0");
    if (batch > INT64_MAX / (int64_t)(2 * plan->n * plan->elem)) return fail(FFT_ERR_INVALID_ARG, "batch too large");
    *bytes = planar_workspace(plan, batch);
    return FFT_OK;
}

int fft_exec_planar(const fft_plan* plan, int dir, const void* in_re, const void* in_im, void* out_re, void* out_im,
                    int64_t batch, void* workspace, void* stream)
{
    if (!plan) return fail(FFT_ERR_INVALID_ARG, "plan is NULL");
    if (plan->path == PATH_REAL) return fail(FFT_ERR_RANK, "plan is for real rows: use fft_exec_r2c / fft_exec_c2r");
    if (dir != FFT_FORWARD && dir != FFT_INVERSE) return fail(FFT_ERR_INVALID_ARG, "dir %d is not FFT_FORWARD/FFT_INVERSE", dir);
    if (batch < 0) return fail(FFT_ERR_INVALID_ARG, "batch %lld < 0", (long long)batch);
    if (batch == 0) return FFT_OK;
    if (!in_re || !in_im || !out_re || !out_im) return fail(FFT_ERR_INVALID_ARG, "a plane pointer is NULL");
    if (batch > INT64_MAX / (int64_t)(2 * plan->n * plan->elem))
        return fail(FFT_ERR_INVALID_ARG, "batch %lld overflows the buffer size", (long long)batch);
    if (((uintptr_t)in_re | (uintptr_t)in_im | (uintptr_t)out_re | (uintptr_t)out_im) % 8)
        return fail(FFT_ERR_ALIGN, "planes must be 8-byte aligned");
    const size_t pb = (size_t)batch * (size_t)plan->n * (plan->elem / 2);  // bytes per plane
    if (ranges_overlap(in_re, pb, in_im, pb) || ranges_overlap(out_re, pb, out_im, pb))
        return fail(FFT_ERR_OVERLAP, "the re and im planes of one array overlap");
    const bool in_place = in_re == out_re && in_im == out_im;
    if (!in_place && (ranges_overlap(in_re, pb, out_re, pb) || ranges_overlap(in_re, pb, out_im, pb) ||
                      ranges_overlap(in_im, pb, out_re, pb) || ranges_overlap(in_im, pb, out_im, pb)))
        return fail(FFT_ERR_OVERLAP, "input and output planes overlap (only in_re == out_re and in_im == out_im "
                                     "is allowed)");
    const size_t ws = planar_workspace(plan, batch);
    if (ws) {
        if (!workspace) return fail(FFT_ERR_WORKSPACE, "workspace of %zu bytes required", ws);
        if ((uintptr_t)workspace % plan->elem) return fail(FFT_ERR_ALIGN, "workspace misaligned");
        const void* planes[4] = {in_re, in_im, out_re, out_im};
        for (const void* q : planes)
            if (ranges_overlap(workspace, ws, q, pb)) return fail(FFT_ERR_WORKSPACE, "workspace overlaps a plane");
    }
    int st = check_device(plan);
    if (st != FFT_OK) return st;
    hipStream_t s = (hipStream_t)stream;
    const Io io{in_re, in_im, out_re, out_im};
    const bool inv = dir == FFT_INVERSE;
    st = plan->rank == 1 ? run_1d(plan, inv, io, batch, workspace, s) : run_nd(plan, inv, io, batch, workspace, s);
    if (st != FFT_OK) return st;
    return sync_if_asked(s, "fft_exec_planar (FFTMI_SYNC)");
}

// Poly-mul plans whose N is not a power of two (and power-of-two rows beyond
// the fused poly-mul row kernels, should the row range outgrow them): the
// plan's own transforms between element-wise pack, product and rounding
// kernels.
static bool poly_any_route(const fft_plan* p)
{
    return p->path == PATH_BLUESTEIN || p->path == PATH_MIXED || p->path == PATH_MIXPASS ||
           (p->path == PATH_ROWS && p->log_a > kPolyRowsMaxLog);
}

// The packed routes' exponent balance at the end of the workspace: per pair
// kPolyExpBlocks partial maxima (int2) and the shift (int, 8 bytes kept).
static size_t poly_shift_bytes(int64_t batch) { return (size_t)batch * (kPolyExpBlocks * 8 + 8); }

int fft_poly_mul_workspace_size(const fft_plan* plan, int64_t batch, size_t* bytes)
{
    if (!plan || !bytes) return fail(FFT_ERR_INVALID_ARG, "plan or bytes is NULL");
    if (batch < 0) return fail(FFT_ERR_INVALID_ARG, "batch < 0");
    if (plan->rank != 1 || plan->path == PATH_REAL) return fail(FFT_ERR_RANK, "poly-mul needs a complex rank-1 plan");
    if (plan->prec != FFT_C64) return fail(FFT_ERR_PRECISION, "poly-mul needs an FFT_C64 plan");
    if (batch > INT64_MAX / (int64_t)(2 * plan->n * plan->elem)) return fail(FFT_ERR_INVALID_ARG, "batch too large");
    if (plan->n > (int64_t(1) << kPolyMaxLog))
        return fail(FFT_ERR_UNSUPPORTED_SIZE, "poly-mul supports N <= 2^%d", kPolyMaxLog);
    if (poly_any_route(plan)) {  // [z: batch x N complex128][the plan's own workspace][shifts]
        *bytes = (size_t)batch * (size_t)plan->n * plan->elem + c2c_workspace(plan, batch) + poly_shift_bytes(batch);
        return FFT_OK;
    }
    // four-step: [batch x N complex128][shifts]
    *bytes = plan->path == PATH_MULTIPASS
                 ? (size_t)batch * (size_t)plan->n * plan->elem + poly_shift_bytes(batch) : 0;
    return FFT_OK;
}

int fft_poly_mul(const fft_plan* plan, const int64_t* a, int64_t la, const int64_t* b, int64_t lb, int64_t* c,
                 int64_t batch, void* workspace, double* d_max_residual, void* stream)
{
    if (!plan) return fail(FFT_ERR_INVALID_ARG, "plan is NULL");
    if (plan->rank != 1 || plan->path == PATH_REAL) return fail(FFT_ERR_RANK, "poly-mul needs a complex rank-1 plan");
    if (plan->prec != FFT_C64) return fail(FFT_ERR_PRECISION, "poly-mul needs an FFT_C64 plan");
    if (batch < 0) return fail(FFT_ERR_INVALID_ARG, "batch < 0");
    if (la < 1 || lb < 1) return fail(FFT_ERR_INVALID_ARG, "la and lb must be >= 1");
    if (plan->n > (int64_t(1) << kPolyMaxLog))
        return fail(FFT_ERR_UNSUPPORTED_SIZE, "poly-mul supports N <= 2^%d", kPolyMaxLog);
    if (la > plan->n || lb > plan->n || la + lb - 1 > plan->n)
        return fail(FFT_ERR_UNSUPPORTED_SIZE, "la + lb - 1 = %lld exceeds the plan's N = %lld",
                    (long long)(la + lb - 1), (long long)plan->n);
    if (batch == 0) return FFT_OK;
    if (!a || !b || !c) return fail(FFT_ERR_INVALID_ARG, "a, b or c is NULL");
    const int64_t lc = la + lb - 1;
    if (batch > INT64_MAX / (int64_t)(2 * plan->n * 16)) return fail(FFT_ERR_INVALID_ARG, "batch too large");
    if (((uintptr_t)a | (uintptr_t)b | (uintptr_t)c) % 8) return fail(FFT_ERR_ALIGN, "a, b, c must be 8-byte aligned");
    if ((uintptr_t)d_max_residual % 8) return fail(FFT_ERR_ALIGN, "d_max_residual must be 8-byte aligned");
    const size_t ba = (size_t)batch * la * 8, bb = (size_t)batch * lb * 8, bc = (size_t)batch * lc * 8;
    if (ranges_overlap(c, bc, a, ba) || ranges_overlap(c, bc, b, bb))
        return fail(FFT_ERR_OVERLAP, "c overlaps a or b");
    if (d_max_residual && (ranges_overlap(d_max_residual, 8, c, bc) || ranges_overlap(d_max_residual, 8, a, ba) ||
                           ranges_overlap(d_max_residual, 8, b, bb)))
        return fail(FFT_ERR_OVERLAP, "d_max_residual overlaps a, b or c");
    size_t ws = 0;
    fft_poly_mul_workspace_size(plan, batch, &ws);
    if (ws) {
        if (!workspace) return fail(FFT_ERR_WORKSPACE, "workspace of %zu bytes required", ws);
        if ((uintptr_t)workspace % 16) return fail(FFT_ERR_ALIGN, "workspace must be 16-byte aligned");
        if (ranges_overlap(workspace, ws, a, ba) || ranges_overlap(workspace, ws, b, bb) ||
            ranges_overlap(workspace, ws, c, bc) ||
            (d_max_residual && ranges_overlap(workspace, ws, d_max_residual, 8)))
            return fail(FFT_ERR_WORKSPACE, "workspace overlaps an operand");
    }
    int st = check_device(plan);
    if (st != FFT_OK) return st;

    hipStream_t s = (hipStream_t)stream;
    hipError_t e = hipSuccess;
    // the exponent balance of the packed routes, at the workspace's end
    void* part = ws ? (char*)workspace + ws - poly_shift_bytes(batch) : nullptr;
    int* shift = ws ? (int*)((char*)part + (size_t)batch * kPolyExpBlocks * 8) : nullptr;
    if (ws) {
        e = launch_poly_shift(a, la, b, lb, batch, part, shift, s);
        if (e != hipSuccess) return hip_fail(e, "fft_poly_mul launch");
    }
    if (poly_any_route(plan)) {
        void* z = workspace;
        void* tws = (char*)workspace + (size_t)batch * (size_t)plan->n * plan->elem;
        const Io zio{z, nullptr, z, nullptr};
        if (d_max_residual) e = launch_zero_resid(d_max_residual, s);
        if (e == hipSuccess) e = launch_polyany_pack(a, la, b, lb, z, plan->n, batch, shift, s);
        if (e != hipSuccess) return hip_fail(e, "fft_poly_mul launch");
        st = run_1d(plan, false, zio, batch, tws, s);
        if (st != FFT_OK) return st;
        e = launch_polyany_product(z, plan->n, batch, s);
        if (e != hipSuccess) return hip_fail(e, "fft_poly_mul launch");
        st = run_1d(plan, true, zio, batch, tws, s);
        if (st != FFT_OK) return st;
        e = launch_polyany_round(z, plan->n, c, lc, batch, shift, d_max_residual, s);
    } else if (d_max_residual && plan->path != PATH_MULTIPASS) {
        // (the four-step route clears the residual in its first kernel)
        e = launch_zero_resid(d_max_residual, s);
    }
    if (e == hipSuccess && !poly_any_route(plan)) {
        if (plan->path == PATH_MULTIPASS) {
            const BigTwiddle big{plan->big_hi, plan->big_lo, plan->big_lbits, plan->logn};
            e = launch_polymul_fourstep(plan->log_a, plan->log_b, a, la, b, lb, c, batch, workspace, plan->tw_a,
                                        plan->tw_b, plan->tw_c, big, shift, d_max_residual, s);
        } else if (plan->path == PATH_ROWS) {
            e = launch_polymul_rows(plan->log_a, a, la, b, lb, c, batch, plan->tw_a, d_max_residual, s);
        } else {
            // N = 1: c_0 = a_0 b_0, done by the N = 2 kernel (la + lb - 1 = 1 <= 2) with no table
            // needed beyond the single radix-2 stage.
            e = launch_polymul_rows(1, a, la, b, lb, c, batch, nullptr, d_max_residual, s);
        }
    }
    if (e != hipSuccess) return hip_fail(e, "fft_poly_mul launch");
    if (getenv("FFTMI_SYNC")) {
        e = hipStreamSynchronize(s);
        if (e != hipSuccess) return hip_fail(e, "fft_poly_mul (FFTMI_SYNC)");
    }
    return FFT_OK;
}

int fft_plan_create_real(fft_plan** out_plan, int64_t n, int prec)
{
    if (!out_plan) return fail(FFT_ERR_INVALID_ARG, "plan pointer is NULL");
    *out_plan = nullptr;
    if (prec != FFT_C32 && prec != FFT_C64) return fail(FFT_ERR_INVALID_ARG, "precision %d unknown", prec);
    if (n < 1) return fail(FFT_ERR_INVALID_ARG, "n = %lld < 1", (long long)n);
    // any even length: the complex plan of N/2 points (any route) and the
    // bin-pair pass; powers of two within one workgroup also fuse the two.
    // Odd lengths: the complex plan of N points itself.
    const bool odd = n > 1 && n % 2;
    const int64_t lim = is_pow2(n) ? 2 * max_n(prec) : odd ? kBluesteinMax : 2 * kBluesteinMax;
    if (n > lim) return fail(FFT_ERR_UNSUPPORTED_SIZE, "n = %lld exceeds %lld", (long long)n, (long long)lim);
    fft_plan* p = new (std::nothrow) fft_plan;
    if (!p) return fail(FFT_ERR_DEVICE, "out of host memory");
    p->rank = 1;
    p->path = PATH_REAL;
    p->prec = prec;
    p->elem = elem_bytes(prec);
    p->dims[0] = p->n = n;
    p->logn = is_pow2(n) ? ilog2(n) : 31;  // 31: w_N lookups of any N take no index mask (k < N)
    p->log_a = is_pow2(n) && p->logn > 0 ? p->logn - 1 : 0;
    p->real_fused = is_pow2(n) && n >= 2 && (n / 2) <= big_row_n(prec);
    p->real_odd = odd;
    hipError_t e = hipGetDevice(&p->device);
    if (e != hipSuccess) {
        delete p;
        return hip_fail(e, "hipGetDevice");
    }
    int st = FFT_OK;
    if (odd) {
        st = fft_plan_create(&p->inner, 1, &n, prec);
    } else if (n >= 2) {
        const int64_t h = n / 2;
        st = fft_plan_create(&p->inner, 1, &h, prec);
        // w_N^{t + i T} = hi[i] lo[t] for the fused kernels (T threads per row)
        const int lem = plan_lem(prec);
        const int want = p->real_fused ? p->log_a - plan_loge(p->log_a, lem) : -1;
        if (st == FFT_OK)
            st = is_pow2(n) ? upload_big(p->logn, prec, &p->big_hi, &p->big_lo, &p->big_lbits, want)
                            : upload_big_any(n, prec, &p->big_hi, &p->big_lo, &p->big_lbits);
    }
    if (st != FFT_OK) {
        free_plan(p);
        return st;
    }
    *out_plan = p;
    return FFT_OK;
}

// Real images outside the power-of-two route: rows by the real-row plan of
// length W (W even or 1), then the H-point column axis (2^a 3^b 5^c 7^d 11^e
// 13^f) as mixed-radix passes over the W/2 + 1 columns of the half spectrum.
static int real_2d_any(fft_plan** out_plan, int64_t h, int64_t w, int prec)
{
    const int64_t wc = w / 2 + 1;
    if (h * wc > max_n(prec))
        return fail(FFT_ERR_UNSUPPORTED_SIZE, "%lld x %lld half-spectrum points exceed %lld", (long long)h,
                    (long long)wc, (long long)max_n(prec));
    // columns of 13-smooth height: super-stage passes over the half
    // spectrum; any other height: transposed, as rows of the rank-1 plan of
    // that length (chirp-z), and transposed back
    MixedSchedule chk;
    int rs[3] = {(int)h, 0, 0};
    const int np = h == 1 || !mixed_factor(h, &chk) ? 0 : axis_split(h, rs);
    if (h > 1 && np == 0 && h > kBluesteinMax)
        return fail(FFT_ERR_UNSUPPORTED_SIZE, "image height %lld exceeds %lld", (long long)h,
                    (long long)kBluesteinMax);
    fft_plan* p = new (std::nothrow) fft_plan;
    if (!p) return fail(FFT_ERR_DEVICE, "out of host memory");
    p->rank = 2;
    p->path = PATH_REAL;
    p->real_nd = true;
    p->prec = prec;
    p->elem = elem_bytes(prec);
    p->dims[0] = h;
    p->dims[1] = w;
    p->n = h * wc;  // points of the half spectrum: the column passes' signal
    if (h > 1) {
        p->nx_k = 1;
        p->nx_len[0] = h;
        p->nx_stride[0] = wc;
        p->nx_np[0] = np;
        int64_t ns = 1;
        for (int q = 0; q < np; ++q) {
            PassPlan& pp = p->passes[q];
            pp.r = rs[q];
            pp.ns = (int)(ns * wc);
            mixed_factor(pp.r, &pp.ms);
            ns *= rs[q];
        }
    }
    hipError_t e = hipGetDevice(&p->device);
    if (e != hipSuccess) {
        delete p;
        return hip_fail(e, "hipGetDevice");
    }
    int st = fft_plan_create_real(&p->inner, w, prec);
    if (st == FFT_OK && h > 1 && np == 0) st = fft_plan_create(&p->nx_plan[0], 1, &p->nx_len[0], prec);
    for (int q = 0; q < p->nx_np[0] && st == FFT_OK; ++q) {
        PassPlan& pp = p->passes[q];
        st = upload(mixed_table(pp.ms), prec, &p->pass_tw[q]);
        pp.tw = p->pass_tw[q];
        if (st == FFT_OK && q > 0)
            st = upload_big_any(pp.ns / wc * pp.r, prec, &pp.big_hi, &pp.big_lo, &pp.big_lbits);
    }
    if (st != FFT_OK) {
        free_plan(p);
        return st;
    }
    *out_plan = p;
    return FFT_OK;
}

int fft_plan_create_real_2d(fft_plan** out_plan, int64_t h, int64_t w, int prec)
{
    if (!out_plan) return fail(FFT_ERR_INVALID_ARG, "plan pointer is NULL");
    *out_plan = nullptr;
    if (prec != FFT_C32 && prec != FFT_C64) return fail(FFT_ERR_INVALID_ARG, "precision %d unknown", prec);
    if (h < 1 || w < 1) return fail(FFT_ERR_INVALID_ARG, "dims %lld x %lld < 1", (long long)h, (long long)w);
    if (!(is_pow2(h) && is_pow2(w) && h <= max_lds_n(prec) && w <= 2 * big_row_n(prec)))
        return real_2d_any(out_plan, h, w, prec);
    fft_plan* p = new (std::nothrow) fft_plan;
    if (!p) return fail(FFT_ERR_DEVICE, "out of host memory");
    p->rank = 2;
    p->path = PATH_REAL;
    p->prec = prec;
    p->elem = elem_bytes(prec);
    p->dims[0] = h;
    p->dims[1] = w;
    p->n = h * w;
    p->logn = ilog2(w);  // the row length; the row tables are for w_W
    p->log_a = p->logn > 0 ? p->logn - 1 : 0;
    p->real_fused = w >= 2;
    const int logh = ilog2(h);
    if (logh > col_pref_log(prec)) p->logf = std::min(4, logh - col_pref_log(prec));
    p->log_b = logh - p->logf;
    hipError_t e = hipGetDevice(&p->device);
    if (e != hipSuccess) {
        delete p;
        return hip_fail(e, "hipGetDevice");
    }
    int st = FFT_OK;
    if (w >= 2) {
        const int64_t half = w / 2;
        st = fft_plan_create(&p->inner, 1, &half, prec);
        const int want = p->log_a - plan_loge(p->log_a, plan_lem(prec));
        if (st == FFT_OK) st = upload_big(p->logn, prec, &p->big_hi, &p->big_lo, &p->big_lbits, want);
    }
    if (st == FFT_OK && h > 1) st = upload(stage_table(p->log_b, prec), prec, &p->tw_b);
    if (st == FFT_OK && p->logf > 0) st = upload_big(logh, prec, &p->col_hi, &p->col_lo, &p->col_lbits);
    if (st != FFT_OK) {
        free_plan(p);
        return st;
    }
    *out_plan = p;
    return FFT_OK;
}

// Checks of fft_exec_r2c / fft_exec_c2r: `in_bytes` / `out_bytes` per row.
static int check_real_exec(const fft_plan* plan, const void* in, size_t in_row, const void* out, size_t out_row,
                           int64_t batch, void* workspace, bool need_ws, bool* noop)
{
    *noop = false;
    if (!plan) return fail(FFT_ERR_INVALID_ARG, "plan is NULL");
    if (plan->path != PATH_REAL) return fail(FFT_ERR_RANK, "plan is not for real rows (fft_plan_create_real)");
    if (batch < 0) return fail(FFT_ERR_INVALID_ARG, "batch %lld < 0", (long long)batch);
    if (batch == 0) {
        *noop = true;
        return FFT_OK;
    }
    if (!in || !out) return fail(FFT_ERR_INVALID_ARG, "in or out is NULL");
    if (batch > INT64_MAX / (int64_t)((plan->n + 2 * plan->dims[0] + 2) * plan->elem))
        return fail(FFT_ERR_INVALID_ARG, "batch %lld overflows the buffer size", (long long)batch);
    if (((uintptr_t)in | (uintptr_t)out) % plan->elem)
        return fail(FFT_ERR_ALIGN, "in/out must be aligned to %zu bytes", plan->elem);
    const size_t bi = (size_t)batch * in_row, bo = (size_t)batch * out_row;
    if (ranges_overlap(in, bi, out, bo)) return fail(FFT_ERR_OVERLAP, "in and out overlap");
    const size_t ws = need_ws ? c2c_workspace(plan, batch) : 0;
    if (ws) {
        if (!workspace) return fail(FFT_ERR_WORKSPACE, "workspace of %zu bytes required", ws);
        if ((uintptr_t)workspace % plan->elem) return fail(FFT_ERR_ALIGN, "workspace misaligned");
        if (ranges_overlap(workspace, ws, in, bi) || ranges_overlap(workspace, ws, out, bo))
            return fail(FFT_ERR_WORKSPACE, "workspace overlaps in or out");
    }
    return check_device(plan);
}

static int real_done(hipError_t e, const char* what, hipStream_t s)
{
    if (e != hipSuccess) return hip_fail(e, what);
    if (getenv("FFTMI_SYNC")) {
        e = hipStreamSynchronize(s);
        if (e != hipSuccess) return hip_fail(e, what);
    }
    return FFT_OK;
}

// Real images outside the power-of-two route.  R2C: the real rows into out,
// then the column passes over out.  C2R: the inverse column passes from in
// into the workspace's Z, then the real rows from Z.  Workspace: [Z][Y][the
// rows' own].
static int exec_real_2d_any(const fft_plan* plan, bool c2r, const void* in, void* out, int64_t batch,
                            void* workspace, hipStream_t s)
{
    const int64_t h = plan->dims[0];
    const size_t half = (size_t)batch * (size_t)plan->n * plan->elem;
    const bool cols = plan->nx_k > 0;
    char* z = (char*)workspace;
    char* y = cols && plan->nx_np[0] != 1 ? z + half : nullptr;
    void* rows_ws = cols ? (void*)(z + half * (y ? 2 : 1)) : workspace;
    const char* what = c2r ? "fft_exec_c2r" : "fft_exec_r2c";
    hipError_t e = hipSuccess;
    if (cols && plan->nx_np[0] == 0) {
        // [b][H][Wc] -> [b][Wc][H] in Y, the H-point rows there, and back
        const int64_t wc = plan->dims[1] / 2 + 1;
        void* tws = (char*)rows_ws + c2c_workspace(plan->inner, batch * h);
        const Io tio{y, nullptr, y, nullptr};
        if (!c2r) {
            int st = fft_exec_r2c(plan->inner, in, out, batch * h, rows_ws, s);
            if (st != FFT_OK) return st;
            e = launch_transpose(plan->prec, out, nullptr, y, nullptr, h, wc, batch, s);
            if (e != hipSuccess) return hip_fail(e, what);
            st = run_1d(plan->nx_plan[0], false, tio, batch * wc, tws, s);
            if (st != FFT_OK) return st;
            return real_done(launch_transpose(plan->prec, y, nullptr, out, nullptr, wc, h, batch, s), what, s);
        }
        e = launch_transpose(plan->prec, in, nullptr, y, nullptr, h, wc, batch, s);
        if (e != hipSuccess) return hip_fail(e, what);
        int st = run_1d(plan->nx_plan[0], true, tio, batch * wc, tws, s);
        if (st != FFT_OK) return st;
        e = launch_transpose(plan->prec, y, nullptr, z, nullptr, wc, h, batch, s);
        if (e != hipSuccess) return hip_fail(e, what);
        return fft_exec_c2r(plan->inner, z, out, batch * h, rows_ws, s);
    }
    if (!c2r) {
        int st = fft_exec_r2c(plan->inner, in, out, batch * h, rows_ws, s);
        if (st != FFT_OK) return st;
        if (cols) e = axis_passes(plan, 0, false, out, nullptr, out, nullptr, y, nullptr, batch, s);
        return real_done(e, what, s);
    }
    if (!cols) return fft_exec_c2r(plan->inner, in, out, batch * h, rows_ws, s);
    e = axis_passes(plan, 0, true, in, nullptr, z, nullptr, y, nullptr, batch, s);
    if (e != hipSuccess) return hip_fail(e, what);
    return fft_exec_c2r(plan->inner, z, out, batch * h, rows_ws, s);
}

// Real images [batch][H][W] <-> [batch][H][W/2 + 1]: the rows (real-row
// kernels), then the columns of the half spectrum (one column per lane).
static int exec_real_2d(const fft_plan* plan, bool c2r, const void* in, void* out, int64_t batch, void* workspace,
                        hipStream_t s)
{
    const int64_t h = plan->dims[0], w = plan->dims[1], wc = w / 2 + 1;
    const int64_t rows = batch * h;
    const BigTwiddle none{nullptr, nullptr, 0, 0};
    const BigTwiddle hb{plan->col_hi, plan->col_lo, plan->col_lbits, plan->log_b + plan->logf};
    hipError_t e = hipSuccess;
    auto row_pass = [&](const void* src, void* dst) {
        return w == 1 ? launch_real_n1(plan->prec, c2r, src, dst, rows, s)
                      : launch_real_rows(plan->prec, plan->log_a, c2r, src, dst, rows, plan->inner->tw_a,
                                         plan->big_hi, plan->big_lo, s);
    };
    if (h == 1) return real_done(row_pass(in, out), c2r ? "fft_exec_c2r" : "fft_exec_r2c", s);
    if (!c2r) {
        // rows -> out (or the workspace ahead of a column stage), columns in place on out
        if (plan->logf == 0) {
            e = row_pass(in, out);
            if (e == hipSuccess)
                e = launch_cols2d(plan->prec, plan->log_b, out, out, batch, wc, 0, plan->tw_b, none, false, 1.0, s,
                                  nullptr, true, false);
        } else {
            if (r2c_fold_supported(plan->prec, plan->log_a, plan->logf)) {
                // the radix-F column stage folded into the row pass
                e = launch_r2c_fold(plan->prec, plan->log_a, plan->logf, in, out, batch, plan->log_b,
                                    plan->inner->tw_a, plan->big_hi, plan->big_lo, s);
            } else {
                e = row_pass(in, workspace);
                if (e == hipSuccess)
                    e = launch_colstage(plan->prec, plan->logf, workspace, out, batch, wc, plan->log_b, s, true,
                                        false);
            }
            if (e == hipSuccess)
                e = launch_cols2d(plan->prec, plan->log_b, out, out, batch, wc, plan->logf, plan->tw_b, hb, false, 1.0,
                                  s, nullptr, true, false);
        }
        return real_done(e, "fft_exec_r2c", s);
    }
    // inverse columns as conj(F(conj X)) / H into the workspace, then the rows
    const double inv_h = 1.0 / (double)h;
    if (plan->logf == 0) {
        e = launch_cols2d(plan->prec, plan->log_b, in, workspace, batch, wc, 0, plan->tw_b, none, true, inv_h, s,
                          nullptr, true, true);
    } else {
        e = launch_colstage(plan->prec, plan->logf, in, workspace, batch, wc, plan->log_b, s, true, true);
        if (e == hipSuccess)
            e = launch_cols2d(plan->prec, plan->log_b, workspace, workspace, batch, wc, plan->logf, plan->tw_b, hb,
                              true, inv_h, s, nullptr, true, false);
    }
    if (e == hipSuccess) e = row_pass(workspace, out);
    return real_done(e, "fft_exec_c2r", s);
}

// Bytes of one transform's real array and of its half spectrum.
static void real_sizes(const fft_plan* p, size_t* real_bytes, size_t* half_bytes)
{
    const size_t rows = p->rank == 2 ? (size_t)p->dims[0] : 1;
    const size_t w = p->rank == 2 ? (size_t)p->dims[1] : (size_t)p->n;
    *real_bytes = rows * w * (p->elem / 2);
    *half_bytes = rows * (w / 2 + 1) * p->elem;
}

int fft_exec_r2c(const fft_plan* plan, const void* in, void* out, int64_t batch, void* workspace, void* stream)
{
    bool noop = false;
    size_t rbytes = 0, hbytes = 0;
    if (plan) real_sizes(plan, &rbytes, &hbytes);
    // Real images: a workspace only where the column stage runs as a pass
    // of its own (the folded row pass writes the caller's output directly).
    const bool need_ws = plan && (plan->rank == 1 || plan->real_nd ||
                                  (plan->logf > 0 && !r2c_fold_supported(plan->prec, plan->log_a, plan->logf)));
    int st = check_real_exec(plan, in, rbytes, out, hbytes, batch, workspace, need_ws, &noop);
    if (st != FFT_OK || noop) return st;
    hipStream_t s = (hipStream_t)stream;
    if (plan->real_nd) return exec_real_2d_any(plan, false, in, out, batch, workspace, s);
    if (plan->rank == 2) return exec_real_2d(plan, false, in, out, batch, workspace, s);
    hipError_t e;
    if (plan->n == 1) {
        e = launch_real_n1(plan->prec, false, in, out, batch, s);
    } else if (plan->real_odd) {
        // widen into the workspace, the N-point transform in place there, bins out
        void* z = workspace;
        void* inner_ws = (char*)workspace + (size_t)batch * (size_t)plan->n * plan->elem;
        e = launch_real_odd(plan->prec, 0, in, z, plan->n, batch, s);
        if (e != hipSuccess) return hip_fail(e, "fft_exec_r2c");
        st = fft_exec_c2c(plan->inner, FFT_FORWARD, z, z, batch, inner_ws, stream);
        if (st != FFT_OK) return st;
        e = launch_real_odd(plan->prec, 1, z, out, plan->n, batch, s);
    } else if (plan->real_fused) {
        e = launch_real_rows(plan->prec, plan->log_a, false, in, out, batch, plan->inner->tw_a, plan->big_hi,
                             plan->big_lo, s);
    } else {
        // Z = F_H(rows read as complex) into the workspace (the out buffer, which
        // holds batch (H + 1) >= batch H values, is the H-point plan's scratch),
        // then the split, two bins per thread.
        void* inner_ws = is_pow2(plan->n) ? out : (char*)workspace + (size_t)batch * (size_t)(plan->n / 2) * plan->elem;
        st = fft_exec_c2c(plan->inner, FFT_FORWARD, in, workspace, batch, inner_ws, stream);
        if (st != FFT_OK) return st;
        const BigTwiddle wn{plan->big_hi, plan->big_lo, plan->big_lbits, plan->logn};
        e = launch_real_pairs(plan->prec, false, workspace, out, plan->n / 2, batch, wn, s);
    }
    return real_done(e, "fft_exec_r2c", s);
}

int fft_exec_c2r(const fft_plan* plan, const void* in, void* out, int64_t batch, void* workspace, void* stream)
{
    bool noop = false;
    size_t rbytes = 0, hbytes = 0;
    if (plan) real_sizes(plan, &rbytes, &hbytes);
    int st = check_real_exec(plan, in, hbytes, out, rbytes, batch, workspace, true, &noop);
    if (st != FFT_OK || noop) return st;
    hipStream_t s = (hipStream_t)stream;
    if (plan->real_nd) return exec_real_2d_any(plan, true, in, out, batch, workspace, s);
    if (plan->rank == 2) return exec_real_2d(plan, true, in, out, batch, workspace, s);
    hipError_t e;
    if (plan->n == 1) {
        e = launch_real_n1(plan->prec, true, in, out, batch, s);
    } else if (plan->real_odd) {
        // the Hermitian extension into the workspace, the inverse in place, real parts out
        void* z = workspace;
        void* inner_ws = (char*)workspace + (size_t)batch * (size_t)plan->n * plan->elem;
        e = launch_real_odd(plan->prec, 2, in, z, plan->n, batch, s);
        if (e != hipSuccess) return hip_fail(e, "fft_exec_c2r");
        st = fft_exec_c2c(plan->inner, FFT_INVERSE, z, z, batch, inner_ws, stream);
        if (st != FFT_OK) return st;
        e = launch_real_odd(plan->prec, 3, z, out, plan->n, batch, s);
    } else if (plan->real_fused) {
        e = launch_real_rows(plan->prec, plan->log_a, true, in, out, batch, plan->inner->tw_a, plan->big_hi,
                             plan->big_lo, s);
    } else {
        // Z from the bin pairs straight into out (N reals = H complex per row),
        // then the inverse H-point transform in place, the workspace its scratch.
        const BigTwiddle wn{plan->big_hi, plan->big_lo, plan->big_lbits, plan->logn};
        e = launch_real_pairs(plan->prec, true, in, out, plan->n / 2, batch, wn, s);
        if (e != hipSuccess) return hip_fail(e, "fft_exec_c2r");
        st = fft_exec_c2c(plan->inner, FFT_INVERSE, out, out, batch, workspace, stream);
        if (st != FFT_OK) return st;
        e = hipSuccess;
    }
    return real_done(e, "fft_exec_c2r", s);
}

}  // extern "C"

// ---------------------------------------------------------------------------
// Scratch for fft_exec_c2c_noalloc: a file-scope device array, one copy per
// GPU (each holds it from the first use until the process ends).  Host code
// never passes `scratch` itself to a kernel: its device address on the current
// device comes from hipGetSymbolAddress, taken once per device and kept.
// ---------------------------------------------------------------------------
namespace {
constexpr int kScratchDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kScratchDevices] = {};
}  // namespace

static __device__ __align__(256) unsigned char scratch[FFT_NOALLOC_SCRATCH_BYTES];

// The device address of `scratch` on device `dev` (current), looked up on the
// first call for that device.
static int scratch_address(int dev, void** ptr)
{
    if (dev < 0 || dev >= kScratchDevices) return fail(FFT_ERR_DEVICE, "device %d beyond the scratch table", dev);
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        void* p = nullptr;
        const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return hip_fail(e, "hipGetSymbolAddress(scratch)");
        if (!p) return fail(FFT_ERR_DEVICE, "hipGetSymbolAddress(scratch) gave NULL");
        g_scratch_ptr[dev] = p;
    }
    *ptr = g_scratch_ptr[dev];
    return FFT_OK;
}

extern "C" {

int fft_exec_c2c_noalloc(const fft_plan* plan, int dir, const void* in, void* out, int64_t batch, void* stream)
{
    // every argument but the workspace, before any HIP call
    bool noop = false;
    int st = check_exec(plan, dir, 1, in, out, batch, nullptr, 0, &noop);
    if (st != FFT_OK || noop) return st;
    const size_t need = c2c_workspace(plan, batch);
    if (need > (size_t)FFT_NOALLOC_SCRATCH_BYTES)
        return fail(FFT_ERR_WORKSPACE, "%zu bytes of workspace needed, more than the %zu bytes of scratch the "
                    "no-allocation entry point holds (use fft_exec_c2c with a workspace)", need,
                    (size_t)FFT_NOALLOC_SCRATCH_BYTES);
    void* ws = nullptr;
    if (need) {
        if ((st = check_device(plan)) != FFT_OK) return st;
        if ((st = scratch_address(plan->device, &ws)) != FFT_OK) return st;
    }
    return fft_exec_c2c(plan, dir, in, out, batch, ws, stream);
}

int fft_stream_copy(const void* src, void* dst, size_t bytes, void* stream)
{
    if (bytes == 0) return FFT_OK;
    if (!src || !dst) return fail(FFT_ERR_INVALID_ARG, "src or dst is NULL");
    if (((uintptr_t)src | (uintptr_t)dst | bytes) & 7)
        return fail(FFT_ERR_ALIGN, "src, dst and bytes must be multiples of 8");
    if (ranges_overlap(src, bytes, dst, bytes)) return fail(FFT_ERR_OVERLAP, "src and dst overlap");
    const hipError_t e = launch_stream_copy(src, dst, (int64_t)(bytes / 8), (hipStream_t)stream);
    if (e != hipSuccess) return hip_fail(e, "fft_stream_copy");
    return FFT_OK;
}

}  // extern "C"
