// bluestein.hip -- the chirp-z (Bluestein) route to a transform of any length
// N, which "FFT on GPU" (section "Algorithm per signal Length") lists for
// lengths that are not powers of two.
//
// With c_j = e^{-i pi j^2 / N} and n k = (n^2 + k^2 - (k - n)^2) / 2,
//     X_k = c_k sum_n (x_n c_n) conj(c_{k-n}),
// a linear convolution, evaluated as a cyclic one of power-of-two length
// M >= 2N - 1 with the library's own power-of-two transforms:
//     w = pad_M(x . c);  W = F_M(w) . B;  y = F_M^{-1}(W);  X_k = c_k y_k,
// where B = F_M(b), b_m = conj(c_m) for m < N, b_{M-m} = conj(c_m) for
// 0 < m < N (computed once, in fp64, when the plan is made).
//
// M within the row kernel's range: the whole route in one kernel (below).
// Larger M: the multi-pass transforms of tiles.hip with the chirp products
// and the product with B carried by their first and last passes
// (chirp_io.hpp).
#include "io.hpp"
#include "launch.hpp"
#include "stockham.hpp"

namespace fftmi {

static inline dim3 ew_grid(int64_t total)
{
    int64_t blocks = (total + 255) / 256;
    if (blocks > (1 << 20)) blocks = 1 << 20;  // grid-stride beyond this
    return dim3((unsigned)(blocks > 0 ? blocks : 1));
}

__global__ void narrow_kernel(const double2* __restrict__ in, float2* __restrict__ out, int64_t total)
{
    for (int64_t e = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; e < total; e += (int64_t)gridDim.x * blockDim.x)
        out[e] = float2{(float)in[e].x, (float)in[e].y};
}

// a w with the rounding pinned: each part is one product rounded, then a fused
// multiply-add.  The chirp and spectrum products sit next to the loads and
// stores, whose form differs between interleaved and planar rows; with the
// fusion left to the compiler the two could round differently.
__device__ __forceinline__ float fma_r(float a, float b, float c) { return __builtin_fmaf(a, b, c); }
__device__ __forceinline__ double fma_r(double a, double b, double c) { return __builtin_fma(a, b, c); }
template <typename V> __device__ __forceinline__ V cmul_pinned(V a, V w)
{
    const auto p = a.y * w.y;
    const auto q = a.y * w.x;
    return V{fma_r(a.x, w.x, -p), fma_r(a.x, w.y, q)};
}

// Rows of one wavefront or less (T <= 64) are packed 256 threads to a
// workgroup and order their exchanges with wavefront-scope fences; longer rows
// take a workgroup each, so that a barrier holds only that row's waves (M =
// 2048, complex64, 1009-point rows: two rows per workgroup 526 us, one 466 us).
template <typename V, int LOGM> constexpr bool bl_in_wave() { return Geom<V, LOGM>::T <= 64; }
template <typename V, int LOGM> constexpr int bl_rows_per_wg() { return bl_in_wave<V, LOGM>() ? 256 / Geom<V, LOGM>::T : 1; }

// The whole chirp-z transform of a row in one kernel, for M = 2^LOGM within
// the row kernel's range: the row is loaded once (times the chirp, zero
// padded to M in registers), transformed, multiplied by B, transformed back
// (conj F conj / M) and stored once (times the chirp) -- the same arithmetic
// as the five-pass route, without its four HBM round trips over M points.
// tw: stage table for M.  INV: the inverse transform (conj in, conj and scale
// out).  The twiddle bases are loaded again for the second transform rather
// than held in registers across the first.
template <typename V, int LOGM, bool PL, bool INV>
__global__ __launch_bounds__((Geom<V, LOGM>::T * bl_rows_per_wg<V, LOGM>()))
void bluestein_rows_kernel(CIn<V, PL> in, COut<V, PL> out, int64_t nrows, int n, const V* __restrict__ tw,
                           const V* __restrict__ chirp, const V* __restrict__ bspec, typename real_of<V>::type scale)
{
    using G = Geom<V, LOGM>;
    static_assert(G::E >= 2, "positions t + i T with i >= E/2 are the upper half");
    using Rl = typename real_of<V>::type;
    constexpr int RPW = bl_rows_per_wg<V, LOGM>();
    __shared__ V lds[G::LDS > 0 ? G::LDS * RPW : 1];

    const int tid = threadIdx.x;
    const int rloc = tid / G::T;
    const int t = tid % G::T;
    const int64_t row = (int64_t)blockIdx.x * RPW + rloc;
    const bool live = row < nrows;
    const LdsLines<V, 1, 4, bl_in_wave<V, LOGM>()> L{lds + rloc * G::LDS, 0};
    constexpr bool BL_COMPACT = G::T * RPW >= 1024;

    V v[G::E];
    const int64_t base = row * n;
    {
        TwBases<V, LOGM> tb;
        tb.load(tw, t);
        // Every load is issued unconditionally, from an address clamped into
        // the row (a dead row reads row 0), and the value is dropped after:
        // loads under a branch each end in a wait for memory, which would
        // serialise the row's loads.  1024-thread rows (registers capped at
        // 128) keep the branches: their clamped form spills.
        const auto src = in.at((live ? row : 0) * n);
#pragma unroll
        for (int i = 0; i < G::E; ++i) {
            const int p = t + i * G::T;
            V x{0, 0};
            // positions from M/2 on are zero padding (n <= M/2): a
            // compile-time zero, so the first stage's x + 0 terms can go
            if constexpr (BL_COMPACT) {
                if (i < G::E / 2 && live && p < n) {
                    x = src.ld32((unsigned)p);
                    if (INV) x = cconj(x);
                    x = cmul_pinned(x, chirp[p]);
                }
            } else if (i < G::E / 2) {
                const int pc = p < n ? p : n - 1;
                V y = src.ld32((unsigned)pc);
                if (INV) y = cconj(y);
                y = cmul_pinned(y, chirp[pc]);
                x = live && p < n ? y : V{0, 0};
            }
            v[i] = x;
        }
        fft_regs<LOGM>(v, t, tb, L);
    }
    // W B, conjugated for the inverse transform
#pragma unroll
    for (int i = 0; i < G::E; ++i) v[i] = cconj(cmul_pinned(v[i], bspec[t + i * G::T]));
    L.sync();  // the forward transform's last exchange is read by now
    {
        // the table pointer through an empty asm statement: these loads are
        // not hoisted above the forward transform and held across it
        const V* tw2 = tw;
        asm volatile("" : "+s"(tw2));
        TwBases<V, LOGM> tb;
        tb.load(tw2, t);
        fft_regs<LOGM>(v, t, tb, L);
    }
    const Rl inv_m = (Rl)1 / (Rl)(1 << LOGM);
    if constexpr (BL_COMPACT) {
        if (!live) return;
#pragma unroll
        for (int i = 0; i < G::E / 2; ++i) {
            const int p = t + i * G::T;
            if (p < n) {
                const V y = cmul_pinned(V{v[i].x * inv_m, -v[i].y * inv_m}, chirp[p]);
                out.st(base + p, INV ? V{y.x * scale, -y.y * scale} : y);
            }
        }
        return;
    }
    // outputs from M/2 on are never stored; the chirp factors and products
    // are formed for every position (clamped), so that only the stores sit
    // under a branch and no load waits inside one
    V y[G::E / 2];
#pragma unroll
    for (int i = 0; i < G::E / 2; ++i) {
        const int p = t + i * G::T;
        y[i] = chirp[p < n ? p : n - 1];
    }
#pragma unroll
    for (int i = 0; i < G::E / 2; ++i) asm volatile("" ::"v"(y[i].x), "v"(y[i].y));  // loaded here, together
#pragma unroll
    for (int i = 0; i < G::E / 2; ++i) {
        y[i] = cmul_pinned(V{v[i].x * inv_m, -v[i].y * inv_m}, y[i]);
        if (INV) y[i] = V{y[i].x * scale, -y[i].y * scale};
    }
#pragma unroll
    for (int i = 0; i < G::E / 2; ++i) {
        const int p = t + i * G::T;
        if (live && p < n) out.st(base + p, y[i]);
    }
}

template <typename V, int LOGM, bool PL, bool INV>
static hipError_t bluestein_rows_t(const Io& io, int64_t nrows, int n, const void* tw, const void* chirp,
                                   const void* bspec, double scale, hipStream_t s)
{
    constexpr int RPW = bl_rows_per_wg<V, LOGM>();
    constexpr int BLOCK = Geom<V, LOGM>::T * RPW;
    const int64_t blocks = (nrows + RPW - 1) / RPW;
    if (blocks > 0x7fffffff) return hipErrorInvalidConfiguration;
    using Rl = typename real_of<V>::type;
    hipLaunchKernelGGL((bluestein_rows_kernel<V, LOGM, PL, INV>), dim3((unsigned)blocks), dim3(BLOCK), 0, s,
                       make_in<V, PL>(io.in, io.in_im), make_out<V, PL>(io.out, io.out_im), nrows, n, (const V*)tw,
                       (const V*)chirp, (const V*)bspec, (Rl)scale);
    return hipGetLastError();
}

template <typename V, int LOGM>
static hipError_t bluestein_rows_pl(const Io& io, int64_t nrows, int n, const void* tw, const void* chirp,
                                    const void* bspec, bool inv, double scale, hipStream_t s)
{
    if (io.in_im)
        return inv ? bluestein_rows_t<V, LOGM, true, true>(io, nrows, n, tw, chirp, bspec, scale, s)
                   : bluestein_rows_t<V, LOGM, true, false>(io, nrows, n, tw, chirp, bspec, scale, s);
    return inv ? bluestein_rows_t<V, LOGM, false, true>(io, nrows, n, tw, chirp, bspec, scale, s)
               : bluestein_rows_t<V, LOGM, false, false>(io, nrows, n, tw, chirp, bspec, scale, s);
}

hipError_t launch_bluestein_rows(int prec, int logm, int n, const void* in, void* out, int64_t nrows, const void* tw,
                                 const void* chirp, const void* bspec, bool inverse, double scale, hipStream_t s,
                                 const void* in_im, void* out_im)
{
    const Io io{in, in_im, out, out_im};
    if ((in_im != nullptr) != (out_im != nullptr)) return hipErrorInvalidValue;
    // the kernel takes every position from M/2 on as zero padding
    if (n < 1 || logm < 1 || logm > 14 || 2 * (int64_t)n - 1 > (int64_t(1) << logm)) return hipErrorInvalidValue;
#define FFTMI_BL(L)                                                                                          \
    case L:                                                                                                  \
        return prec == 0 ? bluestein_rows_pl<float2, L>(io, nrows, n, tw, chirp, bspec, inverse, scale, s)   \
                         : bluestein_rows_pl<double2, L>(io, nrows, n, tw, chirp, bspec, inverse, scale, s);
    if (prec == 1 && logm > 13) return hipErrorInvalidValue;
    switch (logm) {
        FFTMI_BL(2) FFTMI_BL(3) FFTMI_BL(4) FFTMI_BL(5) FFTMI_BL(6) FFTMI_BL(7) FFTMI_BL(8) FFTMI_BL(9)
        FFTMI_BL(10) FFTMI_BL(11) FFTMI_BL(12) FFTMI_BL(13)
        case 14:  // one 1024-thread workgroup a row, 136 KiB of LDS
            if (prec == 0) return bluestein_rows_pl<float2, 14>(io, nrows, n, tw, chirp, bspec, inverse, scale, s);
            return hipErrorInvalidValue;
        default: return hipErrorInvalidValue;
    }
#undef FFTMI_BL
}

hipError_t launch_narrow(const void* in, void* out, int64_t total, hipStream_t s)
{
    hipLaunchKernelGGL(narrow_kernel, ew_grid(total), dim3(256), 0, s, (const double2*)in, (float2*)out, total);
    return hipGetLastError();
}

}  // namespace fftmi
