// polymul.hip -- products of integer polynomials by FFT ("FFT on GPU",
// polynomial-multiplication and whole-process sections): zero-pad a and b to
// N, forward FFT of both, pointwise product, inverse FFT scaled by 1/N, round
// the real part to the nearest integer.  fp64 throughout.
//
// The inverse is evaluated as conj(F(conj(P))) / N with the forward engine,
// and only the real part is kept, which conj does not change.
//
// N <= 4096: one fused kernel per pair (int64 load with implicit zero
// padding, two forward transforms, product, third transform, rint, int64
// store) -- the whole product never leaves the chip.
// N > 4096: the four-step split N = N1 N2 (see tiles.hip) with the pointwise
// product fused between the forward and the inverse row transforms:
//   A : columns (length N2) of both zero-padded operands, times w_N^{n1 k2}
//   B : per row k2 (length N1): F(a-row), F(b-row), product, conj, F, times
//       w_N^{n1 k2}  -- the forward's last pass and the inverse's first pass
//       are one kernel, and the spectra never go back to memory in between
//   A2: columns (length N2) again, Re / N, rint, int64 store.
#include "launch.hpp"
#include "stockham.hpp"
#include "tile_common.hpp"

namespace fftmi {

// Max of non-negative doubles by their bit patterns (which order like the
// values), one atomic per wave.
__device__ __forceinline__ void resid_max(double r, double* d_resid)
{
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) r = fmax(r, __shfl_xor(r, off, 64));
    if ((threadIdx.x & 63) == 0 && d_resid)
        atomicMax((unsigned long long*)d_resid, (unsigned long long)__double_as_longlong(r));
}

__global__ void zero_resid_kernel(double* d) { *d = 0.0; }

template <int LOGN> constexpr int poly_rows_per_wg() { return Geometry<LOGN>::T >= 256 ? 1 : 256 / Geometry<LOGN>::T; }

// ---------------------------------------------------------------------------
// Fused single-kernel product for N = 2^LOGN <= 4096.
// ---------------------------------------------------------------------------
template <int LOGN>
__global__ __launch_bounds__(Geometry<LOGN>::T * poly_rows_per_wg<LOGN>())
void polymul_rows_kernel(const int64_t* __restrict__ a, int64_t la, const int64_t* __restrict__ b, int64_t lb,
                         int64_t* __restrict__ c, int64_t batch, const double2* __restrict__ tw,
                         double* __restrict__ d_resid)
{
    using G = Geometry<LOGN>;
    constexpr int RPW = poly_rows_per_wg<LOGN>();
    __shared__ double2 lds[G::LDS > 0 ? G::LDS * RPW : 1];
    const int tid = threadIdx.x;
    const int rloc = tid / G::T, t = tid % G::T;
    const int64_t pair = (int64_t)blockIdx.x * RPW + rloc;
    const bool live = pair < batch;
    const LdsLines<double2, 1> at{lds + rloc * G::LDS, 0};
    TwBases<double2, LOGN> tb;
    tb.load(tw, t);

    double2 va[G::E], vb[G::E];
#pragma unroll
    for (int i = 0; i < G::E; ++i) {
        const int n = t + i * G::T;
        va[i] = double2{(live && n < la) ? (double)a[pair * la + n] : 0.0, 0.0};
        vb[i] = double2{(live && n < lb) ? (double)b[pair * lb + n] : 0.0, 0.0};
    }
    fft_regs<LOGN>(va, t, tb, at);
    if constexpr (G::S > 1) __syncthreads();
    fft_regs<LOGN>(vb, t, tb, at);
#pragma unroll
    for (int i = 0; i < G::E; ++i) va[i] = cconj(cmul(va[i], vb[i]));
    if constexpr (G::S > 1) __syncthreads();
    fft_regs<LOGN>(va, t, tb, at);

    const int64_t lc = la + lb - 1;
    const double inv_n = 1.0 / (double)G::N;
    double worst = 0.0;
#pragma unroll
    for (int i = 0; i < G::E; ++i) {
        const int n = t + i * G::T;
        if (live && n < lc) {
            const double val = va[i].x * inv_n;
            const double r = rint(val);
            c[pair * lc + n] = (int64_t)r;
            worst = fmax(worst, fabs(val - r));
        }
    }
    resid_max(worst, d_resid);
}

// ---------------------------------------------------------------------------
// Four-step pass A: operand columns.  Tiles run over [operand][pair][n1 tile].
// ---------------------------------------------------------------------------
template <int LOGN2, int C>
__global__ __launch_bounds__(C * Geometry<LOGN2>::T)
void polymul_a_kernel(const int64_t* __restrict__ a, int64_t la, const int64_t* __restrict__ b, int64_t lb,
                      double2* __restrict__ ws, int64_t batch, int logn1, const double2* __restrict__ tw,
                      BigTw<double2> big)
{
    using G = Geometry<LOGN2>;
    __shared__ double2 lds[tile_lds_slots<LOGN2, C>()];
    const int c = threadIdx.x % C, t = threadIdx.x / C;
    const int64_t tile = xcd_tile(blockIdx.x, gridDim.x);
    const int64_t tps = ((int64_t)1 << logn1) / C;
    const int64_t sig = tile / tps;  // operand * batch + pair
    const bool is_b = sig >= batch;
    const int64_t pair = is_b ? sig - batch : sig;
    const int64_t len = is_b ? lb : la;
    const int64_t* src = (is_b ? b : a) + pair * len;
    const int64_t col = (tile % tps) * C + c;  // n1

    double2 v[G::E];
#pragma unroll
    for (int i = 0; i < G::E; ++i) {
        const int64_t n = col + ((int64_t)(t + i * G::T) << logn1);
        v[i] = double2{n < len ? (double)src[n] : 0.0, 0.0};
    }
    TwBases<double2, LOGN2> tb;
    tb.load(tw, t);
    fft_regs<LOGN2>(v, t, tb, LdsLines<double2, C>{lds, c});
    apply_big_twiddle<LOGN2>(v, col, t, big);
    double2* dst = ws + (sig << (logn1 + LOGN2)) + col;
#pragma unroll
    for (int i = 0; i < G::E; ++i) dst[(int64_t)(t + i * G::T) << logn1] = v[i];
}

// ---------------------------------------------------------------------------
// Four-step pass B (fused): rows k2 of both spectra.
// ---------------------------------------------------------------------------
template <int LOGN1>
__global__ __launch_bounds__(Geometry<LOGN1>::T * poly_rows_per_wg<LOGN1>())
void polymul_b_kernel(double2* __restrict__ ws_a, const double2* __restrict__ ws_b, int64_t nrows, int logn2,
                      const double2* __restrict__ tw, BigTw<double2> big)
{
    using G = Geometry<LOGN1>;
    constexpr int RPW = poly_rows_per_wg<LOGN1>();
    __shared__ double2 lds[G::LDS > 0 ? G::LDS * RPW : 1];
    const int tid = threadIdx.x;
    const int rloc = tid / G::T, t = tid % G::T;
    const int64_t row = (int64_t)blockIdx.x * RPW + rloc;  // pair * N2 + k2
    const bool live = row < nrows;
    const int64_t k2 = row & (((int64_t)1 << logn2) - 1);
    const LdsLines<double2, 1> at{lds + rloc * G::LDS, 0};
    TwBases<double2, LOGN1> tb;
    tb.load(tw, t);
    const int64_t base = (row << LOGN1) + t;

    double2 va[G::E], vb[G::E];
#pragma unroll
    for (int i = 0; i < G::E; ++i) {
        va[i] = live ? ws_a[base + i * G::T] : double2{0.0, 0.0};
        vb[i] = live ? ws_b[base + i * G::T] : double2{0.0, 0.0};
    }
    fft_regs<LOGN1>(va, t, tb, at);
    if constexpr (G::S > 1) __syncthreads();
    fft_regs<LOGN1>(vb, t, tb, at);
#pragma unroll
    for (int i = 0; i < G::E; ++i) va[i] = cconj(cmul(va[i], vb[i]));
    if constexpr (G::S > 1) __syncthreads();
    fft_regs<LOGN1>(va, t, tb, at);
    apply_big_twiddle<LOGN1>(va, k2, t, big);
    if (live) {
#pragma unroll
        for (int i = 0; i < G::E; ++i) ws_a[base + i * G::T] = va[i];
    }
}

// ---------------------------------------------------------------------------
// Four-step pass A2: columns of the product's transform, Re / N, rint.
// ---------------------------------------------------------------------------
template <int LOGN2, int C>
__global__ __launch_bounds__(C * Geometry<LOGN2>::T)
void polymul_a2_kernel(const double2* __restrict__ ws_a, int64_t* __restrict__ c_out, int64_t lc, int logn1,
                       const double2* __restrict__ tw, double* __restrict__ d_resid)
{
    using G = Geometry<LOGN2>;
    __shared__ double2 lds[tile_lds_slots<LOGN2, C>()];
    const int c = threadIdx.x % C, t = threadIdx.x / C;
    const int64_t tile = xcd_tile(blockIdx.x, gridDim.x);
    const int64_t tps = ((int64_t)1 << logn1) / C;
    const int64_t pair = tile / tps;
    const int64_t col = (tile % tps) * C + c;  // n1
    const double2* src = ws_a + (pair << (logn1 + LOGN2)) + col;

    double2 v[G::E];
#pragma unroll
    for (int i = 0; i < G::E; ++i) v[i] = src[(int64_t)(t + i * G::T) << logn1];
    TwBases<double2, LOGN2> tb;
    tb.load(tw, t);
    fft_regs<LOGN2>(v, t, tb, LdsLines<double2, C>{lds, c});

    const double inv_n = 1.0 / (double)((int64_t)1 << (logn1 + LOGN2));
    double worst = 0.0;
    int64_t* dst = c_out + pair * lc;
#pragma unroll
    for (int i = 0; i < G::E; ++i) {
        const int64_t n = col + ((int64_t)(t + i * G::T) << logn1);
        if (n < lc) {
            const double val = v[i].x * inv_n;
            const double r = rint(val);
            dst[n] = (int64_t)r;
            worst = fmax(worst, fabs(val - r));
        }
    }
    resid_max(worst, d_resid);
}

// ---------------------------------------------------------------------------
// Launchers
// ---------------------------------------------------------------------------
hipError_t launch_zero_resid(double* d, hipStream_t s)
{
    hipLaunchKernelGGL(zero_resid_kernel, dim3(1), dim3(1), 0, s, d);
    return hipGetLastError();
}

template <int LOGN>
static hipError_t polymul_rows_t(const int64_t* a, int64_t la, const int64_t* b, int64_t lb, int64_t* c,
                                 int64_t batch, const void* tw, double* d_resid, hipStream_t s)
{
    constexpr int RPW = poly_rows_per_wg<LOGN>();
    const int64_t blocks = (batch + RPW - 1) / RPW;
    if (blocks > 0x7fffffff) return hipErrorInvalidConfiguration;
    hipLaunchKernelGGL((polymul_rows_kernel<LOGN>), dim3((unsigned)blocks), dim3(Geometry<LOGN>::T * RPW), 0, s,
                       a, la, b, lb, c, batch, (const double2*)tw, d_resid);
    return hipGetLastError();
}

hipError_t launch_polymul_rows(int logn, const int64_t* a, int64_t la, const int64_t* b, int64_t lb, int64_t* c,
                               int64_t batch, const void* tw, double* d_resid, hipStream_t s)
{
    switch (logn) {
#define PR(L) case L: return polymul_rows_t<L>(a, la, b, lb, c, batch, tw, d_resid, s);
        PR(1) PR(2) PR(3) PR(4) PR(5) PR(6) PR(7) PR(8) PR(9) PR(10) PR(11) PR(12)
#undef PR
        default: return hipErrorInvalidValue;
    }
}

template <int LOGN2>
static hipError_t polymul_a_t(int logn1, const int64_t* a, int64_t la, const int64_t* b, int64_t lb, void* ws,
                              int64_t batch, const void* tw_col, BigTw<double2> big, hipStream_t s)
{
    constexpr int C = TileShape<double2, LOGN2>::C;
    const int64_t n1 = (int64_t)1 << logn1;
    if (n1 % C) return hipErrorInvalidValue;
    const int64_t blocks = 2 * batch * (n1 / C);
    if (blocks > 0x7fffffff) return hipErrorInvalidConfiguration;
    hipLaunchKernelGGL((polymul_a_kernel<LOGN2, C>), dim3((unsigned)blocks), dim3(C * Geometry<LOGN2>::T), 0, s,
                       a, la, b, lb, (double2*)ws, batch, logn1, (const double2*)tw_col, big);
    return hipGetLastError();
}

template <int LOGN1>
static hipError_t polymul_b_t(int logn2, void* ws, int64_t batch, const void* tw_row, BigTw<double2> big,
                              hipStream_t s)
{
    constexpr int RPW = poly_rows_per_wg<LOGN1>();
    const int64_t nrows = batch << logn2;
    const int64_t blocks = (nrows + RPW - 1) / RPW;
    if (blocks > 0x7fffffff) return hipErrorInvalidConfiguration;
    double2* ws_a = (double2*)ws;
    const double2* ws_b = ws_a + (batch << (LOGN1 + logn2));
    hipLaunchKernelGGL((polymul_b_kernel<LOGN1>), dim3((unsigned)blocks), dim3(Geometry<LOGN1>::T * RPW), 0, s,
                       ws_a, ws_b, nrows, logn2, (const double2*)tw_row, big);
    return hipGetLastError();
}

template <int LOGN2>
static hipError_t polymul_a2_t(int logn1, const void* ws, int64_t* c, int64_t lc, int64_t batch,
                               const void* tw_col, double* d_resid, hipStream_t s)
{
    constexpr int C = TileShape<double2, LOGN2>::C;
    const int64_t n1 = (int64_t)1 << logn1;
    if (n1 % C) return hipErrorInvalidValue;
    const int64_t blocks = batch * (n1 / C);
    if (blocks > 0x7fffffff) return hipErrorInvalidConfiguration;
    hipLaunchKernelGGL((polymul_a2_kernel<LOGN2, C>), dim3((unsigned)blocks), dim3(C * Geometry<LOGN2>::T), 0, s,
                       (const double2*)ws, c, lc, logn1, (const double2*)tw_col, d_resid);
    return hipGetLastError();
}

hipError_t launch_polymul_fourstep(int logn1, int logn2, const int64_t* a, int64_t la, const int64_t* b, int64_t lb,
                                   int64_t* c, int64_t batch, void* ws, const void* tw_row, const void* tw_col,
                                   BigTwiddle bigt, double* d_resid, hipStream_t s)
{
    const BigTw<double2> big{(const double2*)bigt.hi, (const double2*)bigt.lo, bigt.lbits, bigt.logn};
    hipError_t e = hipErrorInvalidValue;
    switch (logn2) {
#define PA(L) case L: e = polymul_a_t<L>(logn1, a, la, b, lb, ws, batch, tw_col, big, s); break;
        PA(5) PA(6) PA(7) PA(8) PA(9) PA(10) PA(11) PA(12)
#undef PA
        default: return hipErrorInvalidValue;
    }
    if (e != hipSuccess) return e;
    switch (logn1) {
#define PB(L) case L: e = polymul_b_t<L>(logn2, ws, batch, tw_row, big, s); break;
        PB(5) PB(6) PB(7) PB(8) PB(9) PB(10) PB(11) PB(12)
#undef PB
        default: return hipErrorInvalidValue;
    }
    if (e != hipSuccess) return e;
    const int64_t lc = la + lb - 1;
    switch (logn2) {
#define PA2(L) case L: e = polymul_a2_t<L>(logn1, ws, c, lc, batch, tw_col, d_resid, s); break;
        PA2(5) PA2(6) PA2(7) PA2(8) PA2(9) PA2(10) PA2(11) PA2(12)
#undef PA2
        default: return hipErrorInvalidValue;
    }
    return e;
}

int tile_lines(int prec, int logl)
{
    switch (logl) {
#define TL(L) case L: return prec == 0 ? TileShape<float2, L>::C : TileShape<double2, L>::C;
        TL(1) TL(2) TL(3) TL(4) TL(5) TL(6) TL(7) TL(8) TL(9) TL(10) TL(11) TL(12)
#undef TL
        default: return 0;
    }
}

}  // namespace fftmi
