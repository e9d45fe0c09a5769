// tiles.hip -- tile kernels: one workgroup transforms C adjacent "lines" that
// are not contiguous in memory (the columns of a 2D image, the columns and
// transposed rows of the four-step).  Lanes run over the C lines fastest, so
// every load and store instruction touches C contiguous elements per line;
// the workgroup-to-tile map keeps neighbouring tiles on one XCD so that their
// partial cache lines meet in the same L2.
//
// The 2D column pass follows "Stockham FFT Butterfly Algorithm in Parallel
// GLSL", section "Multi-Dimensional Transforms and Separability" (rows, then
// columns).  The four-step splits an N = N1 N2 transform with the same
// even/odd idea as the radix-2 split of "FFT on GPU" (section "Fast Fourier
// Transform"), with radix N1 instead of 2:
//   n = n1 + N1 n2,  k = k2 + N2 k1,
//   X[k2 + N2 k1] = sum_{n1} w_{N1}^{n1 k1} w_N^{n1 k2} sum_{n2} x[n1 + N1 n2] w_{N2}^{n2 k2}
// pass A: the inner sums (columns, length N2) and the factor w_N^{n1 k2};
// pass B: the outer sums (rows, length N1) with a transposing store.
#include "launch.hpp"
#include "stockham.hpp"
#include "tile_common.hpp"

namespace fftmi {

// ---------------------------------------------------------------------------
// 2D column pass
// ---------------------------------------------------------------------------
template <typename V, int LOGN, int C, bool CONJ_OUT>
__global__ __launch_bounds__(C * Geometry<LOGN>::T)
void cols2d_kernel(const V* in, V* out, int64_t tiles_per_img, int64_t w, const V* __restrict__ tw,
                   typename real_of<V>::type scale)
{
    using G = Geometry<LOGN>;
    __shared__ V lds[tile_lds_slots<LOGN, C>()];
    const int c = threadIdx.x % C, t = threadIdx.x / C;
    const int64_t tile = xcd_tile(blockIdx.x, gridDim.x);
    const int64_t img = tile / tiles_per_img;
    const int64_t col = (tile % tiles_per_img) * C + c;
    const bool live = col < w;
    const int64_t base = img * ((int64_t)G::N * w) + col + (int64_t)t * w;
    const int64_t step = (int64_t)G::T * w;

    V v[G::E];
#pragma unroll
    for (int i = 0; i < G::E; ++i) v[i] = live ? in[base + i * step] : V{0, 0};
    TwBases<V, LOGN> tb;
    tb.load(tw, t);
    fft_regs<LOGN>(v, t, tb, LdsLines<V, C>{lds, c});
    if (live) {
#pragma unroll
        for (int i = 0; i < G::E; ++i) {
            V y = v[i];
            out[base + i * step] = CONJ_OUT ? V{y.x * scale, -y.y * scale} : y;
        }
    }
}

// ---------------------------------------------------------------------------
// Four-step pass A: columns of [N2][N1] (line = n1, position = n2 -> k2),
// then the twiddle w_N^{n1 k2}; written back in the same layout.
// ---------------------------------------------------------------------------
template <typename V, int LOGN, int C, bool CONJ_IN>
__global__ __launch_bounds__(C * Geometry<LOGN>::T)
void fourstep_a_kernel(const V* in, V* ws, int64_t n1, int64_t tiles_per_sig, const V* __restrict__ tw,
                       const V* __restrict__ big_hi, const V* __restrict__ big_lo, int lbits, int logn_total)
{
    using G = Geometry<LOGN>;
    __shared__ V lds[tile_lds_slots<LOGN, C>()];
    const int c = threadIdx.x % C, t = threadIdx.x / C;
    const int64_t tile = xcd_tile(blockIdx.x, gridDim.x);
    const int64_t sig = tile / tiles_per_sig;
    const int64_t col = (tile % tiles_per_sig) * C + c;  // n1 (< n1 always: C divides n1)
    const int64_t base = (sig << logn_total) + col + (int64_t)t * n1;
    const int64_t step = (int64_t)G::T * n1;

    V v[G::E];
#pragma unroll
    for (int i = 0; i < G::E; ++i) {
        V x = in[base + i * step];
        v[i] = CONJ_IN ? cconj(x) : x;
    }
    TwBases<V, LOGN> tb;
    tb.load(tw, t);
    fft_regs<LOGN>(v, t, tb, LdsLines<V, C>{lds, c});
    // element i sits at k2 = t + i T: multiply by w_N^{n1 (t + i T)}
    apply_big_twiddle<LOGN>(v, (int64_t)col, t, BigTw<V>{big_hi, big_lo, lbits, logn_total});
#pragma unroll
    for (int i = 0; i < G::E; ++i) ws[base + i * step] = v[i];
}

// ---------------------------------------------------------------------------
// Four-step pass B: rows of [N2][N1] (line = k2, position = n1 -> k1), stored
// transposed: X[k2 + N2 k1].
// ---------------------------------------------------------------------------
template <typename V, int LOGN, int C, bool CONJ_OUT>
__global__ __launch_bounds__(C * Geometry<LOGN>::T)
void fourstep_b_kernel(const V* ws, V* out, int64_t n2, int64_t tiles_per_sig, const V* __restrict__ tw,
                       typename real_of<V>::type scale, int logn_total)
{
    using G = Geometry<LOGN>;
    __shared__ V lds[tile_lds_slots<LOGN, C>()];
    const int c = threadIdx.x % C, t = threadIdx.x / C;
    const int64_t tile = xcd_tile(blockIdx.x, gridDim.x);
    const int64_t sig = tile / tiles_per_sig;
    const int64_t row = (tile % tiles_per_sig) * C + c;  // k2
    const int64_t sbase = sig << logn_total;
    const int64_t in_base = sbase + (row << LOGN) + t;
    const int64_t out_base = sbase + row + (int64_t)t * n2;
    const int64_t out_step = (int64_t)G::T * n2;

    V v[G::E];
#pragma unroll
    for (int i = 0; i < G::E; ++i) v[i] = ws[in_base + i * G::T];
    TwBases<V, LOGN> tb;
    tb.load(tw, t);
    fft_regs<LOGN>(v, t, tb, LdsLines<V, C>{lds, c});
#pragma unroll
    for (int i = 0; i < G::E; ++i) {
        V y = v[i];
        out[out_base + i * out_step] = CONJ_OUT ? V{y.x * scale, -y.y * scale} : y;
    }
}

// ---------------------------------------------------------------------------
// Launchers
// ---------------------------------------------------------------------------
template <typename V, int LOGN>
static hipError_t cols2d_t(const void* in, void* out, int64_t nimg, int64_t w, const void* tw, bool co,
                           double scale, hipStream_t s)
{
    constexpr int C = TileShape<V, LOGN>::C;
    const int64_t tpi = (w + C - 1) / C;
    const int64_t blocks = tpi * nimg;
    if (blocks > 0x7fffffff) return hipErrorInvalidConfiguration;
    using Rl = typename real_of<V>::type;
    const dim3 grid((unsigned)blocks), block(C * Geometry<LOGN>::T);
    if (co)
        hipLaunchKernelGGL((cols2d_kernel<V, LOGN, C, true>), grid, block, 0, s, (const V*)in, (V*)out, tpi, w,
                           (const V*)tw, (Rl)scale);
    else
        hipLaunchKernelGGL((cols2d_kernel<V, LOGN, C, false>), grid, block, 0, s, (const V*)in, (V*)out, tpi, w,
                           (const V*)tw, (Rl)scale);
    return hipGetLastError();
}

template <typename V, int LOGN>
static hipError_t fourstep_a_t(int64_t n1, const void* in, void* ws, int64_t batch, const void* tw,
                               BigTwiddle big, bool ci, hipStream_t s)
{
    constexpr int C = TileShape<V, LOGN>::C;
    if (n1 % C) return hipErrorInvalidValue;
    const int64_t tps = n1 / C;
    const int64_t blocks = tps * batch;
    if (blocks > 0x7fffffff) return hipErrorInvalidConfiguration;
    const dim3 grid((unsigned)blocks), block(C * Geometry<LOGN>::T);
    if (ci)
        hipLaunchKernelGGL((fourstep_a_kernel<V, LOGN, C, true>), grid, block, 0, s, (const V*)in, (V*)ws, n1, tps,
                           (const V*)tw, (const V*)big.hi, (const V*)big.lo, big.lbits, big.logn);
    else
        hipLaunchKernelGGL((fourstep_a_kernel<V, LOGN, C, false>), grid, block, 0, s, (const V*)in, (V*)ws, n1, tps,
                           (const V*)tw, (const V*)big.hi, (const V*)big.lo, big.lbits, big.logn);
    return hipGetLastError();
}

template <typename V, int LOGN>
static hipError_t fourstep_b_t(int64_t n2, const void* ws, void* out, int64_t batch, const void* tw, bool co,
                               double scale, int logn_total, hipStream_t s)
{
    constexpr int C = TileShape<V, LOGN>::C;
    if (n2 % C) return hipErrorInvalidValue;
    const int64_t tps = n2 / C;
    const int64_t blocks = tps * batch;
    if (blocks > 0x7fffffff) return hipErrorInvalidConfiguration;
    using Rl = typename real_of<V>::type;
    const dim3 grid((unsigned)blocks), block(C * Geometry<LOGN>::T);
    if (co)
        hipLaunchKernelGGL((fourstep_b_kernel<V, LOGN, C, true>), grid, block, 0, s, (const V*)ws, (V*)out, n2, tps,
                           (const V*)tw, (Rl)scale, logn_total);
    else
        hipLaunchKernelGGL((fourstep_b_kernel<V, LOGN, C, false>), grid, block, 0, s, (const V*)ws, (V*)out, n2, tps,
                           (const V*)tw, (Rl)scale, logn_total);
    return hipGetLastError();
}

#define FFTMI_TILE_SWITCH(PREC, LOGN, CALL_F, CALL_D)                                   \
    switch (LOGN) {                                                                       \
        case 1: return PREC == 0 ? CALL_F(1) : CALL_D(1);                                 \
        case 2: return PREC == 0 ? CALL_F(2) : CALL_D(2);                                 \
        case 3: return PREC == 0 ? CALL_F(3) : CALL_D(3);                                 \
        case 4: return PREC == 0 ? CALL_F(4) : CALL_D(4);                                 \
        case 5: return PREC == 0 ? CALL_F(5) : CALL_D(5);                                 \
        case 6: return PREC == 0 ? CALL_F(6) : CALL_D(6);                                 \
        case 7: return PREC == 0 ? CALL_F(7) : CALL_D(7);                                 \
        case 8: return PREC == 0 ? CALL_F(8) : CALL_D(8);                                 \
        case 9: return PREC == 0 ? CALL_F(9) : CALL_D(9);                                 \
        case 10: return PREC == 0 ? CALL_F(10) : CALL_D(10);                              \
        case 11: return PREC == 0 ? CALL_F(11) : CALL_D(11);                              \
        case 12: return PREC == 0 ? CALL_F(12) : CALL_D(12);                              \
        case 13: return PREC == 0 ? CALL_F(13) : hipErrorInvalidValue;                    \
        default: return hipErrorInvalidValue;                                             \
    }

hipError_t launch_cols2d(int prec, int logh, const void* in, void* out, int64_t nimg, int64_t w, const void* tw,
                         bool co, double scale, hipStream_t s)
{
#define CF(L) cols2d_t<float2, L>(in, out, nimg, w, tw, co, scale, s)
#define CD(L) cols2d_t<double2, L>(in, out, nimg, w, tw, co, scale, s)
    FFTMI_TILE_SWITCH(prec, logh, CF, CD)
#undef CF
#undef CD
}

hipError_t launch_fourstep_a(int prec, int logn2, int64_t n1, const void* in, void* ws, int64_t batch,
                             const void* tw, BigTwiddle big, bool ci, hipStream_t s)
{
#define CF(L) fourstep_a_t<float2, L>(n1, in, ws, batch, tw, big, ci, s)
#define CD(L) fourstep_a_t<double2, L>(n1, in, ws, batch, tw, big, ci, s)
    FFTMI_TILE_SWITCH(prec, logn2, CF, CD)
#undef CF
#undef CD
}

hipError_t launch_fourstep_b(int prec, int logn1, int64_t n2, const void* ws, void* out, int64_t batch,
                             const void* tw, bool co, double scale, hipStream_t s)
{
    int logn2 = 0;
    while ((int64_t(1) << logn2) < n2) ++logn2;
    const int logn_total = logn1 + logn2;
#define CF(L) fourstep_b_t<float2, L>(n2, ws, out, batch, tw, co, scale, logn_total, s)
#define CD(L) fourstep_b_t<double2, L>(n2, ws, out, batch, tw, co, scale, logn_total, s)
    FFTMI_TILE_SWITCH(prec, logn1, CF, CD)
#undef CF
#undef CD
}

int tile_lines(int prec, int logl)
{
    switch (logl) {
#define TL(L) case L: return prec == 0 ? TileShape<float2, L>::C : TileShape<double2, L>::C;
        TL(1) TL(2) TL(3) TL(4) TL(5) TL(6) TL(7) TL(8) TL(9) TL(10) TL(11) TL(12)
        case 13: return prec == 0 ? TileShape<float2, 13>::C : 0;
#undef TL
        default: return 0;
    }
}

}  // namespace fftmi
