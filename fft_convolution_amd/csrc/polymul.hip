// polymul.hip -- products of integer polynomials by FFT ("FFT on GPU",
// polynomial-multiplication and whole-process sections): zero-pad a and b to
// N, forward FFT of both, pointwise product, inverse FFT scaled by 1/N, round
// the real part to the nearest integer.  fp64 throughout.
//
// Inverse transforms are evaluated as conj(F(conj(P))) / N with the forward
// engine.
//
// N <= 8192: one fused kernel per pair (int64 load with implicit zero
// padding, z = a + i b transformed once, the product spectrum from the bin
// pairs k, N - k through LDS, the inverse transform, the real part, rint,
// int64 store) -- the whole product never leaves the chip.
// N > 8192: z = a + i b as one complex signal, split N = N1 N2, with the
// pointwise product fused between the forward and the inverse row transforms,
// and the inverse at half length (the real product's even and odd
// coefficients as one complex value, N/2 points):
//   A : columns (length N2) of z, times w_N^{n1 k2}
//   B : rows k2 and N2 - k2 (length N1): F of both, the product spectrum
//       from the pair, the packed spectrum D of the half-length inverse,
//       conj, the N1/2-point F, times w_{N/2}^{k2 m1} -- the forward's last
//       pass and the inverse's first pass are one kernel
//   A2: the N1/2 columns (length N2), c_{2m} and c_{2m+1} from each
//       element, rint, int64 store.
// Pass A has a pipelined form for columns of 512 points or more (one
// workgroup per CU, the next tile's loads in flight during a transform).
#include <atomic>

#include "io.hpp"
#include "launch.hpp"
#include "stockham.hpp"
#include "tile_common.hpp"

namespace fftmi {

// Max of non-negative doubles by their bit patterns (which order like the
// values): reduce over the wave, then over the workgroup through LDS, then one
// vector atomic per workgroup -- skipped when the value already stored is at
// least as large (a stale read can only make it do an unneeded atomic).  All
// threads of the workgroup must call it.
__device__ __forceinline__ void resid_max(double r, double* d_resid)
{
    __shared__ double red[16];
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) r = fmax(r, __shfl_xor(r, off, 64));
    const int wave = threadIdx.x >> 6, nwaves = (blockDim.x + 63) >> 6;
    if ((threadIdx.x & 63) == 0) red[wave] = r;
    __syncthreads();
    if (threadIdx.x == 0 && d_resid) {
        for (int w = 1; w < nwaves; ++w) r = fmax(r, red[w]);
        const unsigned long long bits = (unsigned long long)__double_as_longlong(r);
        if (bits > *(volatile unsigned long long*)d_resid) atomicMax((unsigned long long*)d_resid, bits);
    }
}

__global__ void zero_resid_kernel(double* d) { *d = 0.0; }

// The first kernel of the four-step product clears the residual that its
// last kernel raises (kernels on one stream run one after another): one
// thread of workgroup 0, no launch of its own.
__device__ __forceinline__ void clear_resid(double* d_resid)
{
    if (d_resid && blockIdx.x == 0 && threadIdx.x == 0) *d_resid = 0.0;
}

// The residual of one output value val (= Re(y) / N) rounded to r = rint(val):
// |val - r|, or +infinity where that cannot vouch for the result -- |val| >=
// 2^53, where every double is an integer and a rounding error no longer shows
// as a fraction, or val not finite (NaN fails the comparison too).
__device__ __forceinline__ double out_residual(double val, double r)
{
    return fabs(val) < 0x1p53 ? fabs(val - r) : __builtin_inf();
}

// r as int64 where it is in range; INT64_MIN (a value no exact product of
// this size can take) where it is beyond the int64 range or not finite, so
// that the conversion is always defined.
__device__ __forceinline__ int64_t to_int64(double r)
{
    return fabs(r) < 0x1p63 ? (int64_t)r : INT64_MIN;
}

template <int LOGN> constexpr int poly_rows_per_wg() { return Geom<double2, LOGN>::T >= 256 ? 1 : 256 / Geom<double2, LOGN>::T; }

// ---------------------------------------------------------------------------
// Fused single-kernel product for N = 2^LOGN <= 4096.
// ---------------------------------------------------------------------------
template <int LOGN>
__global__ __launch_bounds__((Geom<double2, LOGN>::T * poly_rows_per_wg<LOGN>()))
void polymul_rows_kernel(const int64_t* __restrict__ a, int64_t la, const int64_t* __restrict__ b, int64_t lb,
                         int64_t* __restrict__ c, int64_t batch, const double2* __restrict__ tw,
                         double* __restrict__ d_resid)
{
    using G = Geom<double2, LOGN>;
    constexpr int RPW = poly_rows_per_wg<LOGN>();
    __shared__ double2 lds[G::LDS > 0 ? G::LDS * RPW : 1];
    const int tid = threadIdx.x;
    const int rloc = tid / G::T, t = tid % G::T;
    const int64_t pair = (int64_t)blockIdx.x * RPW + rloc;
    const bool live = pair < batch;
    const LdsLines<double2, 1> at{lds + rloc * G::LDS, 0};
    // each transform loads the twiddle bases anew, through a pointer passed
    // through an empty asm statement so that the loads are not hoisted and
    // held across the other transforms
    auto transform = [&](double2 (&v)[G::E]) {
        const double2* twp = tw;
        asm volatile("" : "+s"(twp));
        TwBases<double2, LOGN> tb;
        tb.load(twp, t);
        fft_regs<LOGN>(v, t, tb, at);
    };

    // loads from addresses clamped into the rows (a dead row reads pair 0),
    // the values dropped after: a load under a branch would wait alone
    const int64_t* ar = a + (live ? pair : 0) * la;
    const int64_t* br = b + (live ? pair : 0) * lb;
    double2 va[G::E], vb[G::E];
#pragma unroll
    for (int i = 0; i < G::E; ++i) {
        const int n = t + i * G::T;
        const int64_t xa = *at_bytes(ar, 8u * (unsigned)(n < la ? n : la - 1));
        const int64_t xb = *at_bytes(br, 8u * (unsigned)(n < lb ? n : lb - 1));
        va[i] = double2{live && n < la ? (double)xa : 0.0, 0.0};
        vb[i] = double2{live && n < lb ? (double)xb : 0.0, 0.0};
    }
    transform(va);
    if constexpr (G::S > 1) __syncthreads();
    transform(vb);
#pragma unroll
    for (int i = 0; i < G::E; ++i) va[i] = cconj(cmul(va[i], vb[i]));
    if constexpr (G::S > 1) __syncthreads();
    transform(va);

    const int64_t lc = la + lb - 1;
    const double inv_n = 1.0 / (double)G::N;
    double worst = 0.0;
#pragma unroll
    for (int i = 0; i < G::E; ++i) {
        const int n = t + i * G::T;
        if (live && n < lc) {
            const double val = va[i].x * inv_n;
            const double r = rint(val);
            c[pair * lc + n] = to_int64(r);
            worst = fmax(worst, out_residual(val, r));
        }
    }
    resid_max(worst, d_resid);
}

// ---------------------------------------------------------------------------
// Single-kernel product for N = 8192, packed: one forward transform of
// z = a + i 2^s b instead of one each for a and b.  With A, B the spectra of
// the real rows a, 2^s b, Z_k = A_k + i B_k and conj Z_{N-k} = A_k - i B_k, so
//     A_k B_k = (Z_k^2 - conj(Z_{N-k})^2) / (4i),
// formed after one LDS exchange that brings each thread the partner bins of
// its own; then one inverse transform (as conj F conj / N, of which only the
// real part is kept), the exact scaling by 2^-s and the rounding.  One row of
// values per thread instead of two: the row fits the 128 registers of a
// 1024-thread workgroup.
//
// The packed spectra carry the rounding error of |z|: where max|a| and
// max|b| lie far apart, the smaller operand's spectrum is off by the larger
// one's error, and the product's by about max|a|/max|b| times the unpacked
// form's.  The power of two 2^s (s = the difference of their binary
// exponents, per pair) puts both operands in one binade, which leaves about
// twice the unpacked error (fp64 model, 4096 x 4096 coefficients of 2^20 and
// 2^12: unpacked 9.8e-4, packed 2.6e-2, balanced 1.5e-3).  Shorter rows keep
// the unpacked kernel above, whose error is that of the pages' method.
// ---------------------------------------------------------------------------
// The maximum of x over each row of 16 lanes, in every lane of the row.
__device__ __forceinline__ int wave_max16(int x)
{
    x = max(x, __builtin_amdgcn_update_dpp(0, x, 0xB1, 0xF, 0xF, true));   // quad_perm [1,0,3,2]
    x = max(x, __builtin_amdgcn_update_dpp(0, x, 0x4E, 0xF, 0xF, true));   // quad_perm [2,3,0,1]
    x = max(x, __builtin_amdgcn_update_dpp(0, x, 0x124, 0xF, 0xF, true));  // row_ror 4
    x = max(x, __builtin_amdgcn_update_dpp(0, x, 0x128, 0xF, 0xF, true));  // row_ror 8
    return x;
}

// The maximum of x over the wavefront (a uniform value): rows of 16 by DPP,
// then the four rows by lane reads.  (Lane exchanges through LDS addresses
// would share those addresses with the residual's reduction at a kernel's
// end and hold them in registers in between.)
__device__ __forceinline__ int wave_max(int x)
{
    x = wave_max16(x);
    return max(max(__builtin_amdgcn_readlane(x, 0), __builtin_amdgcn_readlane(x, 16)),
               max(__builtin_amdgcn_readlane(x, 32), __builtin_amdgcn_readlane(x, 48)));
}

// The shift s of the packed kernel for row pair rloc of the workgroup (T
// consecutive threads a row; T a multiple of 64 or at most 64): the
// difference of the binary exponents of max|a| and max|b| over the row, 0
// where either row is all zero.  The values are integers, so the exponent
// of frexp is 0 for zero and at least 1 otherwise; the maxima are taken over
// those exponents.
template <int T, int E>
__device__ __forceinline__ int balance_shift(const double2 (&v)[E], int rloc)
{
    double ma = 0.0, mb = 0.0;
#pragma unroll
    for (int i = 0; i < E; ++i) {
        ma = fmax(ma, fabs(v[i].x));
        mb = fmax(mb, fabs(v[i].y));
    }
    int ea = __builtin_amdgcn_frexp_exp(ma), eb = __builtin_amdgcn_frexp_exp(mb);
    if constexpr (T >= 64) {
        ea = wave_max(ea);
        eb = wave_max(eb);
    } else {
#pragma unroll
        for (int off = 1; off < T; off <<= 1) {
            ea = max(ea, __shfl_xor(ea, off, 64));
            eb = max(eb, __shfl_xor(eb, off, 64));
        }
    }
    if constexpr (T > 64) {
        static_assert(T % 64 == 0, "rows of whole wavefronts");
        __shared__ int wmax[2][16];
        if ((threadIdx.x & 63) == 0) {
            wmax[0][threadIdx.x >> 6] = ea;
            wmax[1][threadIdx.x >> 6] = eb;
        }
        __syncthreads();
        const int w0 = rloc * (T / 64);
#pragma unroll
        for (int w = 0; w < T / 64; ++w) {
            ea = max(ea, wmax[0][w0 + w]);
            eb = max(eb, wmax[1][w0 + w]);
        }
    }
    return ea > 0 && eb > 0 ? ea - eb : 0;
}

template <int LOGN>
__global__ __launch_bounds__((Geom<double2, LOGN>::T * poly_rows_per_wg<LOGN>()))
void polypack_rows_kernel(const int64_t* __restrict__ a, int64_t la, const int64_t* __restrict__ b, int64_t lb,
                          int64_t* __restrict__ c, int64_t batch, const double2* __restrict__ tw,
                          double* __restrict__ d_resid)
{
    using G = Geom<double2, LOGN>;
    constexpr int N = G::N, T = G::T, E = G::E;
    constexpr int RPW = poly_rows_per_wg<LOGN>();
    using Lds = LdsLines<double2, 1, 3>;  // one pad slot per 8 (16-byte values)
    constexpr int SL = lds_padded(N, 3);
    __shared__ double2 lds[SL * RPW];
    const int tid = threadIdx.x;
    const int rloc = tid / T, t = tid % T;
    const int64_t pair = (int64_t)blockIdx.x * RPW + rloc;
    const bool live = pair < batch;
    const Lds L{lds + rloc * SL, 0};

    // loads from addresses clamped into the rows (a dead group reads pair 0),
    // the values dropped after: a load under a branch would wait alone
    const int64_t* ar = a + (live ? pair : 0) * la;
    const int64_t* br = b + (live ? pair : 0) * lb;
    double2 v[E];
#pragma unroll
    for (int i = 0; i < E; ++i) {
        const int n = t + i * T;
        const int64_t xa = *at_bytes(ar, 8u * (unsigned)(n < la ? n : la - 1));
        const int64_t xb = *at_bytes(br, 8u * (unsigned)(n < lb ? n : lb - 1));
        v[i] = double2{live && n < la ? (double)xa : 0.0, live && n < lb ? (double)xb : 0.0};
    }
    const int sh = balance_shift<T>(v, rloc);
#pragma unroll
    for (int i = 0; i < E; ++i) v[i].y = __builtin_ldexp(v[i].y, sh);
    {
        // the twiddle bases are loaded again for the inverse transform rather
        // than held in registers across the product.  Each load takes the
        // table pointer through an empty asm statement, so that it is not
        // hoisted above the reduction or the first transform: bases held
        // early spill at 1024 threads.
        const double2* tw1 = tw;
        asm volatile("" : "+s"(tw1));
        TwBases<double2, LOGN> tb;
        tb.load(tw1, t);
        fft_regs<LOGN>(v, t, tb, L);
    }
    __syncthreads();  // the transform's last exchange is read by now
#pragma unroll
    for (int i = 0; i < E; ++i) *L.ptr(t + i * T) = v[i];
    __syncthreads();
#pragma unroll
    for (int i = 0; i < E; ++i) {
        const int k = t + i * T;
        const double2 zk = v[i], zq = *L.ptr((N - k) & (N - 1));
        // s = Z_k^2 - conj(Z_q)^2; C_k = s / (4i) = (s.y / 4, -s.x / 4); the
        // inverse transform takes conj C_k
        const double sx = (zk.x * zk.x - zk.y * zk.y) - (zq.x * zq.x - zq.y * zq.y);
        const double sy = 2.0 * zk.x * zk.y + 2.0 * zq.x * zq.y;
        v[i] = double2{0.25 * sy, 0.25 * sx};
    }
    __syncthreads();  // partners are read before the transform reuses the LDS
    {
        const double2* tw2 = tw;
        asm volatile("" : "+s"(tw2));
        TwBases<double2, LOGN> tb;
        tb.load(tw2, t);
        fft_regs<LOGN>(v, t, tb, L);
    }

    const int64_t lc = la + lb - 1;
    int64_t* cr = c + pair * lc;
    const double inv_n = __builtin_ldexp(1.0 / (double)N, -sh);  // a power of two: exact
    double worst = 0.0;
#pragma unroll
    for (int i = 0; i < E; ++i) {
        const int n = t + i * T;
        if (live && n < lc) {
            const double val = v[i].x * inv_n;
            const double r = rint(val);
            *at_bytes(cr, 8u * n) = to_int64(r);
            worst = fmax(worst, out_residual(val, r));
        }
    }
    resid_max(worst, d_resid);
}

// Tiles of the column passes A and A2: they also move int64 values (8 bytes
// per lane), so 16 lanes per row segment make those 128-byte segments too
// (measured on MI355X, 32 x 2^18 products: 329 -> 322 us); 1024-point columns
// keep 8 (16 would need 2048 threads).
template <int LOGN2> using PolyTile = Tile<double2, LOGN2, (LOGN2 <= 9 ? 16 : 8)>;

// ---------------------------------------------------------------------------
// N > 4096: the two real operands travel as one complex signal z = a + i b
// (both have real coefficients), N = N1 N2 split as n = n1 + N1 n2,
// k = k2 + N2 k1 (the radix-N1 form of the even/odd split of "FFT on GPU",
// section "Fast Fourier Transform").
//
// Pass A: for every column n1, the N2-point transform over n2 of z, times
// w_N^{n1 k2}; written as rows k2 (Y[k2][n1]).
// ---------------------------------------------------------------------------
template <int LOGN2>
__global__ __launch_bounds__((PolyTile<LOGN2>::THREADS))
void polypack_a_kernel(const int64_t* __restrict__ a, int64_t la, const int64_t* __restrict__ b, int64_t lb,
                       double2* __restrict__ ws, int logn1, const double2* __restrict__ tw, BigTw<double2> big,
                       const int* __restrict__ shift, double* __restrict__ d_resid)
{
    using G = Geom<double2, LOGN2>;
    using TL = PolyTile<LOGN2>;
    __shared__ double2 lds[TL::LDS];
    clear_resid(d_resid);
    const int c0 = threadIdx.x % TL::CL, t = threadIdx.x / TL::CL;
    const int64_t tile = xcd_tile(blockIdx.x, gridDim.x);
    const int64_t tps = ((int64_t)1 << logn1) / TL::C;
    const int64_t pair = tile / tps;
    const int64_t col = (tile % tps) * TL::C + c0;  // n1
    const int64_t* pa = a + pair * la;
    const int64_t* pb = b + pair * lb;
    const int sh = shift[pair];  // z = a + i 2^s b

    double2 v[G::E];
#pragma unroll
    for (int i = 0; i < G::E; ++i) {
        const int64_t n = col + ((int64_t)(t + i * G::T) << logn1);
        v[i] = double2{n < la ? (double)pa[n] : 0.0, n < lb ? __builtin_ldexp((double)pb[n], sh) : 0.0};
    }
    TwBases<double2, LOGN2> tb;
    tb.load(tw, t);
    fft_regs<LOGN2>(v, t, tb, LdsLines<double2, TL::CL>{lds, c0});
    apply_big_twiddle<LOGN2>(v, col, t, big);
    double2* dst = ws + (pair << (logn1 + LOGN2)) + col;
#pragma unroll
    for (int i = 0; i < G::E; ++i) dst[(int64_t)(t + i * G::T) << logn1] = v[i];
}

// Pass A when both operands fit in the lower half of every column (la, lb <=
// N/2, so positions n2 >= N2/2 are zero padding, a compile-time fact here).
// Pass A holds one workgroup per CU (its tile's LDS), so a grid of one tile
// per workgroup leaves each CU idle while a tile's loads are in flight.
// Instead a grid of one workgroup per CU walks the tiles of the plain grid's
// order (virtual block j * grid + b, so every workgroup stays on its XCD's
// tile range) and loads tile j + 1's int64 values -- E/2 per operand and lane
// -- while tile j is transformed and stored.
template <int LOGN2>
__global__ __launch_bounds__((PolyTile<LOGN2>::THREADS))
void polypack_a_pipe_kernel(const int64_t* __restrict__ a, int64_t la, const int64_t* __restrict__ b, int64_t lb,
                            double2* __restrict__ ws, int logn1, unsigned ntiles, const double2* __restrict__ tw,
                            BigTw<double2> big, const int* __restrict__ shift, double* __restrict__ d_resid)
{
    clear_resid(d_resid);
    using G = Geom<double2, LOGN2>;
    using TL = PolyTile<LOGN2>;
    constexpr int H = G::E / 2;
    constexpr int LC = __builtin_ctz(TL::C);
    __shared__ double2 lds[TL::LDS];
    const int c0 = threadIdx.x % TL::CL, t = threadIdx.x / TL::CL;
    const LdsLines<double2, TL::CL> L{lds, c0};
    const int lt = logn1 - LC;  // log2 of the tiles per pair
    // Offsets within a pair's signal (< N <= 2^22 elements, so byte offsets
    // fit 32 bits): the lane's first element, and the step between its
    // elements (T rows of N1).
    const unsigned lane = (unsigned)c0 + ((unsigned)t << logn1);
    const unsigned step = (unsigned)G::T << logn1;
    int64_t ra[H], rb[H];
    // Every lane loads (an index past the operand is clamped to its last
    // coefficient and the value dropped in value()), so that the loads are not
    // branched around and the waits for later loads can count them.  With
    // `real` false (the prefetch after a workgroup's last tile) every lane
    // reads coefficient 0: one line, no tile's worth of HBM reads.
    auto load = [&](unsigned vb, bool real) {
        const unsigned tile = (unsigned)xcd_tile(vb, ntiles);
        const unsigned n0 = real ? ((tile & ((1u << lt) - 1)) << LC) + lane : 0u;
        const unsigned st = real ? step : 0u;
        const int64_t* pa = a + (int64_t)(tile >> lt) * la;
        const int64_t* pb = b + (int64_t)(tile >> lt) * lb;
#pragma unroll
        for (int i = 0; i < H; ++i) {
            const unsigned n = n0 + i * st;
            ra[i] = *at_bytes(pa, (unsigned)min((int64_t)n, la - 1) * 8u);
            rb[i] = *at_bytes(pb, (unsigned)min((int64_t)n, lb - 1) * 8u);
        }
    };
    auto value = [&](int i, unsigned n0, int sh) {  // z = a + i 2^s b
        const int64_t n = (int64_t)(n0 + i * step);
        return double2{n < la ? (double)ra[i] : 0.0, n < lb ? __builtin_ldexp((double)rb[i], sh) : 0.0};
    };
    if (blockIdx.x >= ntiles) return;  // the whole workgroup
    // a loop body of one basic block (no early exit), so that the compiler
    // cannot sink the next tile's loads towards their use
    const unsigned iters = (ntiles - blockIdx.x + gridDim.x - 1) / gridDim.x;
    unsigned vb = blockIdx.x;
    load(vb, true);
    for (unsigned k = 0; k < iters; ++k) {
        const unsigned tile = (unsigned)xcd_tile(vb, ntiles);
        const unsigned col = ((tile & ((1u << lt) - 1)) << LC) + c0;  // n1
        double2* dst = ws + ((int64_t)(tile >> lt) << (logn1 + LOGN2));
        const int sh = shift[tile >> lt];
        double2 v[G::E];
#pragma unroll
        for (int i = 0; i < G::E; ++i) v[i] = i < H ? value(i, col - c0 + lane, sh) : double2{0.0, 0.0};
        // The stage twiddle bases are loaded per tile, not held across the
        // loop (the empty asm hides that their offset is loop-invariant), and
        // before the next tile's loads: loads complete in issue order, so a
        // wait for them then leaves the next tile's loads in flight.
        unsigned zero = 0;
        asm volatile("" : "+s"(zero));
        TwBases<double2, LOGN2> tb;
        tb.load(tw + zero, t);
        __builtin_amdgcn_sched_barrier(0);
        vb += gridDim.x;
        const bool more = k + 1 < iters;  // uniform over the workgroup
        load(more ? vb : vb - gridDim.x, more);
        __builtin_amdgcn_sched_barrier(0);
        fft_regs<LOGN2>(v, t, tb, L);
        apply_big_twiddle<LOGN2>(v, (int64_t)col, t, big);
#pragma unroll
        for (int i = 0; i < G::E; ++i) *at_bytes(dst, (col + ((unsigned)t << logn1) + i * step) * 16u) = v[i];
        __syncthreads();  // this tile's last exchange is read before the next one's first write
    }
}

// ---------------------------------------------------------------------------
// Pass B, fused: rows k2 and N2 - k2 together (rows 0 and N2/2 pair with
// themselves).  After the N1-point row transforms a row holds
// Z[k2 + N2 k1]; the partner row holds Z at -k mod N (row N2 - k2, position
// N1 - 1 - k1; row 0: position -k1 mod N1).  With A = (Z_k + conj Z_{-k})/2
// and B = (Z_k - conj Z_{-k})/(2i) the spectra of a and b, the product
// spectrum is C_k = A_k B_k = (Z_k^2 - conj(Z_{-k})^2) / (4i).  The inverse
// starts right here.
//
// The product c is real, so its inverse transform runs at half length.  With
// d_m = c_{2m} + i c_{2m+1} (m < N/2),
//     d = F_{N/2}^{-1}(D) / 2,  D_j = (C_j + C_{j+N/2}) + i (C_j - C_{j+N/2}) w_N^{-j}
// (the even and odd samples of c have the spectra (C_j + C_{j+N/2}) / 2 and
// (C_j - C_{j+N/2}) w_N^{-j} / 2).  j + N/2 is position k1 + N1/2 of the same
// row, held by the same thread, so each row forms conj(D) for k1 < N1/2 and
// runs the inverse's first step on N1/2 points: the transform over k1 (its
// first T/2 threads), times w_{N/2}^{k2 m1} =
// w_N^{2 k2 m1}, written over the first half of the row.  Pass A2 then reads
// N1/2 columns and stores two coefficients per element: half the bytes of
// this pass's writes and of A2's reads.
// ---------------------------------------------------------------------------
template <int LOGN1> constexpr int pack_groups()
{
    return 2 * Geom<double2, LOGN1>::T >= 256 ? 1 : 256 / (2 * Geom<double2, LOGN1>::T);
}

template <int LOGN1>
__global__ __launch_bounds__((2 * Geom<double2, LOGN1>::T * pack_groups<LOGN1>()))
void polypack_b_kernel(double2* __restrict__ ws, int64_t ngroups, int logn2, const double2* __restrict__ tw,
                       const double2* __restrict__ tw_half, BigTw<double2> big)
{
    using G = Geom<double2, LOGN1>;
    constexpr int GR = pack_groups<LOGN1>();
    // one LDS pad slot per 8 complex128 elements (not 16): bank conflicts per
    // wave 352 -> 224, pass 108.7 -> 101.5 us (32 x 2^18 products, same-box A/B)
    constexpr int PS = 3;
    constexpr int SLOTS = lds_padded(G::N, PS);
    __shared__ double2 lds[2 * SLOTS * GR];
    const int tid = threadIdx.x;
    const int gl = tid / (2 * G::T);
    const int rho = (tid / G::T) & 1;
    const int t = tid % G::T;
    const int64_t grp = (int64_t)blockIdx.x * GR + gl;
    const bool live = grp < ngroups;
    const int64_t half = (int64_t)1 << (logn2 - 1);
    const int64_t sig = grp >> (logn2 - 1);
    const int64_t m = grp & (half - 1);
    const int64_t n2 = half * 2;
    const int64_t row = m == 0 ? (rho == 0 ? 0 : half) : (rho == 0 ? m : n2 - m);
    const bool wrap = m == 0 && rho == 0;
    double2* mine = lds + (gl * 2 + rho) * SLOTS;
    double2* partner = m == 0 ? mine : lds + (gl * 2 + (1 - rho)) * SLOTS;
    const LdsLines<double2, 1, PS> L{mine, 0};

    TwBases<double2, LOGN1> tb;
    tb.load(tw, t);
    double2* rp = ws + (sig << (logn2 + LOGN1)) + (row << LOGN1) + t;
    double2 v[G::E];
#pragma unroll
    for (int i = 0; i < G::E; ++i) v[i] = live ? rp[i * G::T] : double2{0.0, 0.0};
    fft_regs<LOGN1>(v, t, tb, L);
    __syncthreads();  // LDS reads of the transforms done
    {
        double2* wp = L.ptr(t);
#pragma unroll
        for (int i = 0; i < G::E; ++i) wp[LdsLines<double2, 1, PS>::off(i * G::T)] = v[i];
    }
    __syncthreads();
    const LdsLines<double2, 1, PS> Lp{partner, 0};
#pragma unroll
    for (int i = 0; i < G::E; ++i) {
        const int k1 = t + i * G::T;
        const int pos = wrap ? ((G::N - k1) & (G::N - 1)) : (G::N - 1 - k1);
        const double2 zq = *Lp.ptr(pos);
        const double2 z = v[i];
        // s = z^2 - conj(zq)^2 ; conj(s / 4i) = (s.y / 4, s.x / 4)
        const double sx = (z.x * z.x - z.y * z.y) - (zq.x * zq.x - zq.y * zq.y);
        const double sy = 2.0 * z.x * z.y + 2.0 * zq.x * zq.y;
        v[i] = double2{0.25 * sy, 0.25 * sx};
    }
    __syncthreads();  // partner reads done before the LDS is reused
    {
        using GH = Geom<double2, LOGN1 - 1>;
        static_assert(GH::E == G::E && 2 * GH::T == G::T, "half rows: the first T/2 threads of the row");
        // conj(D_j) = (v_a + v_b) - i (v_a - v_b) w_N^j, v = conj(C) at k1 and
        // k1 + N1/2 (registers i and i + E/2), j = k2 + N2 k1, staged in LDS
        // at position k1 (slot k1 + k1 / 2^PS, the layout of LdsLines)
        double2 w = big(row + ((int64_t)t << logn2));
        const double2 g = big((int64_t)G::T << logn2);
#pragma unroll
        for (int i = 0; i < G::E / 2; ++i) {
            const double2 va = v[i], vb = v[i + G::E / 2];
            const double2 u = cmul(double2{va.x - vb.x, va.y - vb.y}, w);
            const int k1 = t + i * G::T;
            mine[k1 + (k1 >> PS)] = double2{va.x + vb.x + u.y, va.y + vb.y - u.x};
            if (i + 1 < G::E / 2) w = cmul(w, g);
        }
        __syncthreads();
        if constexpr (GH::T <= 64) {
            // one wavefront: its exchanges need no workgroup barrier, and the
            // row's other threads are done
            if (t < GH::T) {
                double2 y[GH::E];
#pragma unroll
                for (int i = 0; i < GH::E; ++i) {
                    const int k1 = t + i * GH::T;
                    y[i] = mine[k1 + (k1 >> PS)];
                }
                TwBases<double2, LOGN1 - 1> th;
                th.load(tw_half, t);
                fft_regs<LOGN1 - 1>(y, t, th, LdsLines<double2, 1, PS, true>{mine, 0});
                apply_big_twiddle<LOGN1 - 1>(y, 2 * row, t, big);
                if (live) {
                    double2* hp = ws + (sig << (logn2 + LOGN1)) + (row << LOGN1) + t;
#pragma unroll
                    for (int i = 0; i < GH::E; ++i) hp[i * GH::T] = y[i];
                }
            }
        } else {
            // several wavefronts: the exchanges take workgroup barriers, which
            // every thread must meet, so the row's other T/2 threads run the
            // same transform on the second half of the row's LDS (whatever it
            // holds: slots(N1) = 2 slots(N1/2) for PS = 3) and drop the result
            constexpr int HS = lds_padded(GH::N, PS);
            static_assert(2 * HS <= SLOTS, "a second half-row region in the row's LDS");
            const bool kept = t < GH::T;
            const int th_t = kept ? t : t - GH::T;
            double2* reg = kept ? mine : mine + HS;
            double2 y[GH::E];
#pragma unroll
            for (int i = 0; i < GH::E; ++i) {
                const int k1 = th_t + i * GH::T;
                y[i] = reg[k1 + (k1 >> PS)];
            }
            // the transform's first stage writes this region straight from
            // registers: every wavefront's staged reads are done by then
            __syncthreads();
            TwBases<double2, LOGN1 - 1> th;
            th.load(tw_half, th_t);
            fft_regs<LOGN1 - 1>(y, th_t, th, LdsLines<double2, 1, PS>{reg, 0});
            apply_big_twiddle<LOGN1 - 1>(y, 2 * row, th_t, big);
            if (kept && live) {
                double2* hp = ws + (sig << (logn2 + LOGN1)) + (row << LOGN1) + th_t;
#pragma unroll
                for (int i = 0; i < GH::E; ++i) hp[i * GH::T] = y[i];
            }
        }
    }
}

// ---------------------------------------------------------------------------
// Pass A2: columns m1 < N1/2 of pass B's half-length rows (k2 -> m2);
// r = F(conj D) at m = m1 + (N1/2) m2 is N conj(d_m), so c_{2m} = Re(r) / N
// and c_{2m+1} = -Im(r) / N, rint, int64 store.
// ---------------------------------------------------------------------------
template <int LOGN2>
__global__ __launch_bounds__((PolyTile<LOGN2>::THREADS))
void polypack_a2_kernel(const double2* __restrict__ ws, int64_t* __restrict__ c_out, int64_t lc, int logn1,
                         const double2* __restrict__ tw, const int* __restrict__ shift, double* __restrict__ d_resid)
{
    using G = Geom<double2, LOGN2>;
    using TL = PolyTile<LOGN2>;
    __shared__ double2 lds[TL::LDS];
    const int c0 = threadIdx.x % TL::CL, t = threadIdx.x / TL::CL;
    const int64_t tile = xcd_tile(blockIdx.x, gridDim.x);
    const int64_t tps = ((int64_t)1 << (logn1 - 1)) / TL::C;
    const int64_t pair = tile / tps;
    const int64_t col = (tile % tps) * TL::C + c0;  // m1
    const double2* src = ws + (pair << (logn1 + LOGN2)) + col;

    double2 v[G::E];
#pragma unroll
    for (int i = 0; i < G::E; ++i) v[i] = src[(int64_t)(t + i * G::T) << logn1];
    TwBases<double2, LOGN2> tb;
    tb.load(tw, t);
    fft_regs<LOGN2>(v, t, tb, LdsLines<double2, TL::CL>{lds, c0});

    // 1/N and the pair's 2^-s: a power of two, exact
    const double inv_n = __builtin_ldexp(1.0 / (double)((int64_t)1 << (logn1 + LOGN2)), -shift[pair]);
    double worst = 0.0;
    int64_t* dst = c_out + pair * lc;
#pragma unroll
    for (int i = 0; i < G::E; ++i) {
        const int64_t n = 2 * (col + ((int64_t)(t + i * G::T) << (logn1 - 1)));
        const double ve = v[i].x * inv_n, vo = -v[i].y * inv_n;
        const double re = rint(ve), ro = rint(vo);
        if (n < lc) {
            dst[n] = to_int64(re);
            worst = fmax(worst, out_residual(ve, re));
        }
        if (n + 1 < lc) {
            dst[n + 1] = to_int64(ro);
            worst = fmax(worst, out_residual(vo, ro));
        }
    }
    resid_max(worst, d_resid);
}

// ---------------------------------------------------------------------------
// Plans whose length N is not a power of two: the plan's own transforms (mixed
// radix or chirp-z, complex128) run between three element-wise kernels --
//   pack:    z = a + i b, zero padded to N;
//   product: Z -> C, C_k = A_k B_k = (Z_k^2 - conj(Z_{-k})^2) / (4i), in place
//            (one thread per pair k, N - k);
//   round:   c = rint(Re y) of the inverse transform y (scaled 1/N), with the
//            residual.
// ---------------------------------------------------------------------------
static inline dim3 pm_grid(int64_t total)
{
    int64_t blocks = (total + 255) / 256;
    if (blocks > (1 << 20)) blocks = 1 << 20;  // grid-stride beyond this
    return dim3((unsigned)(blocks > 0 ? blocks : 1));
}

// ---------------------------------------------------------------------------
// Exponent balance of the packed routes (the four-step passes, and the plan's
// own transforms for N not a power of two): z = a + i 2^s b, with s per pair
// the difference of the binary exponents of max|a| and max|b|, and the
// outputs scaled by 2^-s (both exact).  The packed spectra carry the
// rounding error of |z|, so without it the smaller operand's spectrum -- and
// the product -- takes the larger one's error (fp64 model, 4096 x 4096
// coefficients of 2^26 and 2^4: error 51 unbalanced, 4.6e-5 balanced, 3.1e-5
// with separate transforms).  Two kernels ahead of the passes: the exponents
// of blocks of 4096 coefficients (at most 64 blocks a pair), then their
// maxima and s.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void polyexp_kernel(const int64_t* __restrict__ a, int64_t la,
                                                      const int64_t* __restrict__ b, int64_t lb,
                                                      int2* __restrict__ part, int nblk)
{
    const int64_t pair = blockIdx.x / nblk;
    const int64_t blk = blockIdx.x % nblk;
    const int64_t ca = (la + nblk - 1) / nblk, cb = (lb + nblk - 1) / nblk;
    const int64_t* pa = a + pair * la;
    const int64_t* pb = b + pair * lb;
    const int64_t a0 = blk * ca, a1 = min(a0 + ca, la), b0 = blk * cb, b1 = min(b0 + cb, lb);
    double ma = 0.0, mb = 0.0;
    // 16 loads of each operand in flight per lane (a block of 4096 takes one
    // round); indices past the block's end are clamped to its last
    // coefficient (a repeat leaves the maximum as it is), so that no load
    // waits alone under a branch
    constexpr int U = 16;
    for (int64_t base = 0; base < max(a1 - a0, b1 - b0); base += 256 * U) {
        int64_t xa[U], xb[U];
#pragma unroll
        for (int j = 0; j < U; ++j) {
            const int64_t o = base + threadIdx.x + j * 256;
            xa[j] = pa[min(a0 + o, a1 - 1)];
            xb[j] = pb[min(b0 + o, b1 - 1)];
        }
#pragma unroll
        for (int j = 0; j < U; ++j) {
            ma = fmax(ma, fabs((double)xa[j]));
            mb = fmax(mb, fabs((double)xb[j]));
        }
    }
    if (a1 <= a0) ma = 0.0;  // an empty block reads the coefficient before it
    if (b1 <= b0) mb = 0.0;
    // integers: the frexp exponent is 0 for zero and at least 1 otherwise
    const int ea = wave_max(__builtin_amdgcn_frexp_exp(ma));
    const int eb = wave_max(__builtin_amdgcn_frexp_exp(mb));
    __shared__ int2 w[4];
    if ((threadIdx.x & 63) == 0) w[threadIdx.x >> 6] = int2{ea, eb};
    __syncthreads();
    if (threadIdx.x == 0)
        part[blockIdx.x] = int2{max(max(w[0].x, w[1].x), max(w[2].x, w[3].x)),
                                max(max(w[0].y, w[1].y), max(w[2].y, w[3].y))};
}

// Pairs of at most 1024 coefficients an operand: one wavefront a pair, 16
// loads in flight per lane, part[pair] its exponents (one block a pair), so
// that large batches of short products do not take a workgroup each.
__global__ __launch_bounds__(256) void polyexp_small_kernel(const int64_t* __restrict__ a, int64_t la,
                                                            const int64_t* __restrict__ b, int64_t lb,
                                                            int2* __restrict__ part, int64_t batch)
{
    const int64_t pair = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
    const int64_t pc = pair < batch ? pair : batch - 1;  // the whole wave stays active
    const int64_t* pa = a + pc * la;
    const int64_t* pb = b + pc * lb;
    const int j = (int)(threadIdx.x & 63);
    constexpr int U = 16;
    int64_t xa[U], xb[U];
#pragma unroll
    for (int i = 0; i < U; ++i) {
        xa[i] = pa[min((int64_t)(j + 64 * i), la - 1)];
        xb[i] = pb[min((int64_t)(j + 64 * i), lb - 1)];
    }
    double ma = 0.0, mb = 0.0;
#pragma unroll
    for (int i = 0; i < U; ++i) {
        ma = fmax(ma, fabs((double)xa[i]));
        mb = fmax(mb, fabs((double)xb[i]));
    }
    const int ea = wave_max(__builtin_amdgcn_frexp_exp(ma));
    const int eb = wave_max(__builtin_amdgcn_frexp_exp(mb));
    if (j == 0 && pair < batch) part[pair] = int2{ea, eb};
}

// One wavefront per pair: lane j takes block j's exponents (nblk <= 64).
__global__ __launch_bounds__(256) void polyshift_kernel(const int2* __restrict__ part, int nblk,
                                                        int* __restrict__ shift, int64_t batch)
{
    const int64_t p = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
    const int j = threadIdx.x & 63;
    const bool in = p < batch && j < nblk;
    const int2 e = part[in ? p * nblk + j : 0];
    const int ea = wave_max(in ? e.x : 0), eb = wave_max(in ? e.y : 0);
    if (j == 0 && p < batch) shift[p] = ea > 0 && eb > 0 ? ea - eb : 0;
}

hipError_t launch_poly_shift(const int64_t* a, int64_t la, const int64_t* b, int64_t lb, int64_t batch,
                             void* part, int* shift, hipStream_t s)
{
    const int64_t longest = la > lb ? la : lb;
    const int nblk = (int)std::min<int64_t>(kPolyExpBlocks, std::max<int64_t>(1, (longest + 4095) / 4096));
    if (batch * nblk > 0x7fffffff) return hipErrorInvalidConfiguration;
    if (la <= 1024 && lb <= 1024)  // (nblk is 1)
        hipLaunchKernelGGL(polyexp_small_kernel, dim3((unsigned)((batch + 3) / 4)), dim3(256), 0, s, a, la, b, lb,
                           (int2*)part, batch);
    else
        hipLaunchKernelGGL(polyexp_kernel, dim3((unsigned)(batch * nblk)), dim3(256), 0, s, a, la, b, lb,
                           (int2*)part, nblk);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    if ((batch + 3) / 4 > 0x7fffffff) return hipErrorInvalidConfiguration;
    hipLaunchKernelGGL(polyshift_kernel, dim3((unsigned)((batch + 3) / 4)), dim3(256), 0, s, (const int2*)part, nblk,
                       shift, batch);
    return hipGetLastError();
}

__global__ void polyany_pack_kernel(const int64_t* __restrict__ a, int64_t la, const int64_t* __restrict__ b,
                                    int64_t lb, double2* __restrict__ z, int64_t n, int64_t total,
                                    const int* __restrict__ shift)
{
    for (int64_t e = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; e < total; e += (int64_t)gridDim.x * blockDim.x) {
        const int64_t p = e / n, k = e - p * n;
        z[e] = double2{k < la ? (double)a[p * la + k] : 0.0,
                       k < lb ? __builtin_ldexp((double)b[p * lb + k], shift[p]) : 0.0};  // a + i 2^s b
    }
}

__global__ void polyany_product_kernel(double2* __restrict__ z, int64_t n, int64_t total)
{
    const int64_t h = n / 2 + 1;  // pairs (k, N - k) per signal, k = 0 .. N/2
    for (int64_t e = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; e < total; e += (int64_t)gridDim.x * blockDim.x) {
        const int64_t p = e / h, k = e - p * h, q = k == 0 ? 0 : n - k;
        double2* row = z + p * n;
        const double2 zk = row[k], zq = row[q];
        // s = Z_k^2 - conj(Z_q)^2, C_k = s / (4i) = (s.y / 4, -s.x / 4); the
        // partner's C_q the same with k and q swapped
        const double skx = (zk.x * zk.x - zk.y * zk.y) - (zq.x * zq.x - zq.y * zq.y);
        const double sky = 2.0 * zk.x * zk.y + 2.0 * zq.x * zq.y;
        row[k] = double2{0.25 * sky, -0.25 * skx};
        if (q != k) row[q] = double2{0.25 * sky, 0.25 * skx};
    }
}

__global__ void polyany_round_kernel(const double2* __restrict__ y, int64_t n, int64_t* __restrict__ c, int64_t lc,
                                     int64_t total, const int* __restrict__ shift, double* __restrict__ d_resid)
{
    double worst = 0.0;
    for (int64_t e = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; e < total; e += (int64_t)gridDim.x * blockDim.x) {
        const int64_t p = e / lc, k = e - p * lc;
        const double val = __builtin_ldexp(y[p * n + k].x, -shift[p]), r = rint(val);
        c[e] = to_int64(r);
        worst = fmax(worst, out_residual(val, r));
    }
    resid_max(worst, d_resid);
}

hipError_t launch_polyany_pack(const int64_t* a, int64_t la, const int64_t* b, int64_t lb, void* z, int64_t n,
                               int64_t batch, const int* shift, hipStream_t s)
{
    const int64_t total = batch * n;
    hipLaunchKernelGGL(polyany_pack_kernel, pm_grid(total), dim3(256), 0, s, a, la, b, lb, (double2*)z, n, total,
                       shift);
    return hipGetLastError();
}

hipError_t launch_polyany_product(void* z, int64_t n, int64_t batch, hipStream_t s)
{
    const int64_t total = batch * (n / 2 + 1);
    hipLaunchKernelGGL(polyany_product_kernel, pm_grid(total), dim3(256), 0, s, (double2*)z, n, total);
    return hipGetLastError();
}

hipError_t launch_polyany_round(const void* y, int64_t n, int64_t* c, int64_t lc, int64_t batch, const int* shift,
                                double* d_resid, hipStream_t s)
{
    const int64_t total = batch * lc;
    hipLaunchKernelGGL(polyany_round_kernel, pm_grid(total), dim3(256), 0, s, (const double2*)y, n, c, lc, total,
                       shift, d_resid);
    return hipGetLastError();
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
    hipLaunchKernelGGL((polymul_rows_kernel<LOGN>), dim3((unsigned)blocks), dim3(Geom<double2, LOGN>::T * RPW), 0, s,
                       a, la, b, lb, c, batch, (const double2*)tw, d_resid);
    return hipGetLastError();
}

template <int LOGN>
static hipError_t polypack_rows_t(const int64_t* a, int64_t la, const int64_t* b, int64_t lb, int64_t* c,
                                  int64_t batch, const void* tw, double* d_resid, hipStream_t s)
{
    constexpr int RPW = poly_rows_per_wg<LOGN>();
    const int64_t blocks = (batch + RPW - 1) / RPW;
    if (blocks > 0x7fffffff) return hipErrorInvalidConfiguration;
    hipLaunchKernelGGL((polypack_rows_kernel<LOGN>), dim3((unsigned)blocks), dim3(Geom<double2, LOGN>::T * RPW), 0,
                       s, a, la, b, lb, c, batch, (const double2*)tw, d_resid);
    return hipGetLastError();
}

hipError_t launch_polymul_rows(int logn, const int64_t* a, int64_t la, const int64_t* b, int64_t lb, int64_t* c,
                               int64_t batch, const void* tw, double* d_resid, hipStream_t s)
{
    switch (logn) {
#define PR(L) case L: return polymul_rows_t<L>(a, la, b, lb, c, batch, tw, d_resid, s);
        PR(1) PR(2) PR(3) PR(4) PR(5) PR(6) PR(7) PR(8) PR(9) PR(10) PR(11) PR(12)
#undef PR
        case 13: return polypack_rows_t<13>(a, la, b, lb, c, batch, tw, d_resid, s);
        default: return hipErrorInvalidValue;
    }
}

// Workgroups of the pipelined pass A: one per CU of the current device (a
// multiple of 8, so that a workgroup keeps its XCD from tile to tile).
static int64_t pipe_grid()
{
    static std::atomic<int> cus_of[64];  // per device, 0 until queried
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
    int cus = cus_of[dev].load(std::memory_order_relaxed);
    if (cus == 0) {
        if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus < 8) cus = 256;
        cus_of[dev].store(cus, std::memory_order_relaxed);
    }
    return (int64_t)(cus & ~7);
}

template <int LOGN2>
static hipError_t polypack_a_t(int logn1, const int64_t* a, int64_t la, const int64_t* b, int64_t lb, void* ws,
                               int64_t batch, const void* tw_col, BigTw<double2> big, const int* shift,
                               double* d_resid, hipStream_t s)
{
    using TL = PolyTile<LOGN2>;
    const int64_t n1 = (int64_t)1 << logn1;
    if (n1 % TL::C || TL::THREADS > 1024) return hipErrorInvalidValue;
    const int64_t blocks = batch * (n1 / TL::C);
    if (blocks > 0x7fffffff) return hipErrorInvalidConfiguration;
    // columns of 512 or more points: the tile's LDS holds a CU to one
    // workgroup, the case the pipelined kernel is for (32 x 2^18 products:
    // pass A 120.1 -> 91.7 us, product 315 -> 288 us)
    if constexpr (TL::LDS * sizeof(double2) > 80 * 1024) {
        const int64_t half = (int64_t)1 << (logn1 + LOGN2 - 1);
        if (la <= half && lb <= half) {
            const int64_t grid = std::min<int64_t>(blocks, pipe_grid());
            hipLaunchKernelGGL((polypack_a_pipe_kernel<LOGN2>), dim3((unsigned)grid), dim3(TL::THREADS), 0, s, a, la,
                               b, lb, (double2*)ws, logn1, (unsigned)blocks, (const double2*)tw_col, big, shift,
                               d_resid);
            return hipGetLastError();
        }
    }
    hipLaunchKernelGGL((polypack_a_kernel<LOGN2>), dim3((unsigned)blocks), dim3(TL::THREADS), 0, s, a, la, b, lb,
                       (double2*)ws, logn1, (const double2*)tw_col, big, shift, d_resid);
    return hipGetLastError();
}

template <int LOGN1>
static hipError_t polypack_b_t(int logn2, void* ws, int64_t batch, const void* tw_row, const void* tw_half,
                               BigTw<double2> big, hipStream_t s)
{
    constexpr int GR = pack_groups<LOGN1>();
    const int64_t ngroups = batch << (logn2 - 1);
    const int64_t blocks = (ngroups + GR - 1) / GR;
    if (blocks > 0x7fffffff) return hipErrorInvalidConfiguration;
    hipLaunchKernelGGL((polypack_b_kernel<LOGN1>), dim3((unsigned)blocks), dim3(2 * Geom<double2, LOGN1>::T * GR),
                       0, s, (double2*)ws, ngroups, logn2, (const double2*)tw_row, (const double2*)tw_half, big);
    return hipGetLastError();
}

template <int LOGN2>
static hipError_t polypack_a2_t(int logn1, const void* ws, int64_t* c, int64_t lc, int64_t batch,
                                 const void* tw_col, const int* shift, double* d_resid, hipStream_t s)
{
    using TL = PolyTile<LOGN2>;
    const int64_t h1 = (int64_t)1 << (logn1 - 1);
    if (h1 % TL::C || TL::THREADS > 1024) return hipErrorInvalidValue;
    const int64_t blocks = batch * (h1 / TL::C);
    if (blocks > 0x7fffffff) return hipErrorInvalidConfiguration;
    hipLaunchKernelGGL((polypack_a2_kernel<LOGN2>), dim3((unsigned)blocks), dim3(TL::THREADS), 0, s,
                       (const double2*)ws, c, lc, logn1, (const double2*)tw_col, shift, d_resid);
    return hipGetLastError();
}

hipError_t launch_polymul_fourstep(int logn1, int logn2, const int64_t* a, int64_t la, const int64_t* b, int64_t lb,
                                   int64_t* c, int64_t batch, void* ws, const void* tw_row, const void* tw_col,
                                   const void* tw_half, BigTwiddle bigt, const int* shift, double* d_resid,
                                   hipStream_t s)
{
    const BigTw<double2> big{(const double2*)bigt.hi, (const double2*)bigt.lo, bigt.lbits, bigt.logn};
    // the half-length inverse: rows of N1/2 points in B, whose N1/2 columns
    // split into whole column tiles in A2
    int tile_cols = 0;
    switch (logn2) {
#define TC(L) case L: tile_cols = PolyTile<L>::C; break;
        TC(5) TC(6) TC(7) TC(8) TC(9) TC(10)
#undef TC
        default: return hipErrorInvalidValue;
    }
    if (tw_half == nullptr || logn1 < 5 || logn1 > 12 || ((1 << (logn1 - 1)) % tile_cols) != 0)
        return hipErrorInvalidValue;
    hipError_t e = hipErrorInvalidValue;
    switch (logn2) {
#define PA(L) case L: e = polypack_a_t<L>(logn1, a, la, b, lb, ws, batch, tw_col, big, shift, d_resid, s); break;
        PA(5) PA(6) PA(7) PA(8) PA(9) PA(10)
#undef PA
        default: return hipErrorInvalidValue;
    }
    if (e != hipSuccess) return e;
    switch (logn1) {
#define PB(L) case L: e = polypack_b_t<L>(logn2, ws, batch, tw_row, tw_half, big, s); break;
        PB(5) PB(6) PB(7) PB(8) PB(9) PB(10) PB(11) PB(12)
#undef PB
        default: return hipErrorInvalidValue;
    }
    if (e != hipSuccess) return e;
    const int64_t lc = la + lb - 1;
    switch (logn2) {
#define PA2(L) case L: e = polypack_a2_t<L>(logn1, ws, c, lc, batch, tw_col, shift, d_resid, s); break;
        PA2(5) PA2(6) PA2(7) PA2(8) PA2(9) PA2(10)
#undef PA2
        default: return hipErrorInvalidValue;
    }
    return e;
}

}  // namespace fftmi
