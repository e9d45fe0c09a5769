// tiles.hip -- passes over lines that are not contiguous in memory: the
// column pass and the folded row pass of the 2D transform, and the
// super-stage passes of the multi-pass Stockham transform for N beyond one
// workgroup's LDS.
//
// Lines run across lanes in 128-byte row segments (Tile in tile_common.hpp);
// in the 2D passes the workgroup-to-tile map gives each XCD a contiguous
// range of tiles.
//
// 2D ("Stockham FFT Butterfly Algorithm in Parallel GLSL", section
// "Multi-Dimensional Transforms and Separability": rows, then columns).  A
// column of H = F Lc points is transformed as two Stockham super-stages: the
// radix-F one (span 1: rows j + r Lc combined into rows j F + r) is folded
// into the row pass, and the radix-Lc one (span F: rows j' + F r, twiddle
// w_H^{r j'}) is the column pass, so that the column tiles stay within LDS at
// 128-byte segments and the whole transform still reads and writes HBM twice.
//
// Large 1D: N = R_1 R_2 ... R_p, one pass per super-stage.  Super-stage q with
// radix R and span Ns (the product of the earlier radices) takes, for every
// butterfly j < N/R, the R inputs x[j + r N/R], multiplies input r by
// w_{Ns R}^{r (j mod Ns)}, does an R-point DFT and writes output r to
// y[(j / Ns) Ns R + (j mod Ns) + r Ns] -- the radix-2 stage of "Stockham FFT
// ... in Parallel GLSL" (section "Execution via GLSL Compute Shaders and
// Textures") with radix R, each R-point DFT itself fused in LDS.  The last
// super-stage writes the positions it reads (in place); the first writes each
// butterfly's R outputs contiguously, so it hands the data from lanes-across-
// lines to lanes-along-a-line inside its LDS exchange (fft_regs_remap).
#include "chirp_io.hpp"
#include "io.hpp"
#include "launch.hpp"
#include "stockham.hpp"
#include "tile_common.hpp"

namespace fftmi {

// ---------------------------------------------------------------------------
// 2D column pass: lines (column, j') of [H][W] images, H = F Lc, line points
// at rows j' + F r (r < Lc); in place allowed.
// ---------------------------------------------------------------------------
// ONE: one column per lane (rows of any length, e.g. the W/2 + 1 columns of
// a real image's half spectrum), 16 lanes per 128-byte segment for complex64.
template <typename V, int LOGL, bool ONE>
using ColTile = Tile<V, LOGL, (ONE && sizeof(V) == 8) ? 16 : 8, ONE ? 1 : 16 / (int)sizeof(V)>;

template <typename V, int LOGL, bool CONJ_OUT, bool POUT, bool ONE = false, bool CONJ_IN = false>
__global__ __launch_bounds__((ColTile<V, LOGL, ONE>::THREADS))
void cols2d_kernel(const V* in, COut<V, POUT> out, int64_t w, int logf, int64_t col_tiles, const V* __restrict__ tw,
                   BigTw<V> htw, typename real_of<V>::type scale)
{
    using G = Geom<V, LOGL>;
    using TL = ColTile<V, LOGL, ONE>;
    __shared__ V lds[TL::LDS];
    const int c0 = threadIdx.x % TL::CL, t = threadIdx.x / TL::CL;
    const int64_t tile = xcd_tile(blockIdx.x, gridDim.x);
    const int64_t per_img = col_tiles << logf;
    const int64_t img = tile / per_img;
    const int64_t rem = tile % per_img;
    const int jp = (int)(rem / col_tiles);
    const int64_t col = (rem % col_tiles) * TL::C + c0 * TL::P;
    const bool live = col < w;
    const int64_t f = (int64_t)1 << logf;
    const int64_t base = img * ((f << LOGL) * w) + (jp + f * t) * w + col;
    const int64_t step = f * G::T * w;

    V v[TL::P][G::E];
#pragma unroll
    for (int i = 0; i < G::E; ++i) {
        V q[TL::P];
        if (live) vload(in + base + i * step, q);
        else
#pragma unroll
            for (int g = 0; g < TL::P; ++g) q[g] = V{0, 0};
#pragma unroll
        for (int g = 0; g < TL::P; ++g) v[g][i] = CONJ_IN ? cconj(q[g]) : q[g];
    }
    TwBases<V, LOGL> tb;
    tb.load(tw, t);
    if (jp > 0) {  // the column super-stage's twiddle w_H^{j' r}
#pragma unroll
        for (int g = 0; g < TL::P; ++g) apply_big_twiddle<LOGL>(v[g], jp, t, htw);
    }
#pragma unroll
    for (int g = 0; g < TL::P; ++g) {
        if (g > 0) __syncthreads();
        fft_regs<LOGL>(v[g], t, tb, LdsLines<V, TL::CL>{lds, c0});
    }
    if (live) {
#pragma unroll
        for (int i = 0; i < G::E; ++i) {
            V q[TL::P];
#pragma unroll
            for (int g = 0; g < TL::P; ++g) {
                const V y = v[g][i];
                q[g] = CONJ_OUT ? V{y.x * scale, -y.y * scale} : y;
            }
            out.stv(base + i * step, q);
        }
    }
}

// ---------------------------------------------------------------------------
// 2D column super-stage of radix F on its own (for rows too wide to fold F of
// them into LDS): rows j + r Lc (r < F) of an image are combined, position by
// position, by an F-point DFT into rows j F + r.  No LDS: each thread takes P
// adjacent columns (one 16-byte vector per row) of one (image, j); lanes run
// along the row, so every row access of a wave is contiguous.  Out of place.
// ---------------------------------------------------------------------------
template <typename V, int LOGF, bool ONE>
__global__ __launch_bounds__(256) void colstage_kernel(const V* __restrict__ in, V* __restrict__ out, int64_t w,
                                                       int log_lc, int64_t total, int conj_in)
{
    constexpr int F = 1 << LOGF;
    constexpr int P = ONE ? 1 : 16 / (int)sizeof(V);
    const int64_t wp = w / P;  // column vectors per row
    const int64_t lc = (int64_t)1 << log_lc;
    for (int64_t g = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; g < total; g += (int64_t)gridDim.x * blockDim.x) {
        const int64_t cv = g % wp, rest = g / wp;
        const int64_t j = rest & (lc - 1), img = rest >> log_lc;
        const int64_t base = (img << (log_lc + LOGF)) * w + cv * P;
        V u[P][F];
#pragma unroll
        for (int r = 0; r < F; ++r) {
            V q[P];
            vload(in + base + (j + ((int64_t)r << log_lc)) * w, q);
#pragma unroll
            for (int e = 0; e < P; ++e) u[e][r] = conj_in ? cconj(q[e]) : q[e];
        }
#pragma unroll
        for (int e = 0; e < P; ++e) Dft<F>::run(u[e]);
#pragma unroll
        for (int r = 0; r < F; ++r) {
            V q[P];
#pragma unroll
            for (int e = 0; e < P; ++e) q[e] = u[e][r];
            vstore(out + base + ((j << LOGF) + r) * w, q);
        }
    }
}

// ---------------------------------------------------------------------------
// 2D row pass with the column super-stage of radix F folded in: a group of F
// threads-rows takes rows j + r Lc (r < F) of one image, transforms each row
// (length W), exchanges through LDS so that every thread holds all F rows at
// E/F positions, does the F-point DFT across the rows and writes row j F + r'.
// Out of place (the rows it writes are read by other groups).
// ---------------------------------------------------------------------------
template <typename V, int LOGW, int LOGF> constexpr int fold_groups()
{
    return (Geom<V, LOGW>::T << LOGF) >= 256 ? 1 : 256 / (Geom<V, LOGW>::T << LOGF);
}

template <typename V, int LOGW, int LOGF, bool CONJ_IN, bool PIN>
__global__ __launch_bounds__(((Geom<V, LOGW>::T << LOGF) * fold_groups<V, LOGW, LOGF>()))
void rows2d_fold_kernel(CIn<V, PIN> in, V* out, int64_t ngroups, int log_lc, const V* __restrict__ tw)
{
    using G = Geom<V, LOGW>;
    constexpr int F = 1 << LOGF;
    constexpr int GR = fold_groups<V, LOGW, LOGF>();
    constexpr int SLOTS = lds_padded(G::N);  // one row, padded (also used when S == 1)
    constexpr int EF = G::E / F;
    static_assert(G::E >= F, "each thread needs at least F positions");
    __shared__ V lds[SLOTS * F * GR];
    const int tid = threadIdx.x;
    const int gl = tid / (F * G::T);
    const int rho = (tid / G::T) % F;
    const int t = tid % G::T;
    const int64_t grp = (int64_t)blockIdx.x * GR + gl;
    const bool live = grp < ngroups;
    const int64_t lc = (int64_t)1 << log_lc;
    const int64_t img = grp >> log_lc, j = grp & (lc - 1);
    const int64_t h = lc << LOGF;
    V* my = lds + (gl * F) * SLOTS;

    TwBases<V, LOGW> tb;
    tb.load(tw, t);
    V v[G::E];
    const int64_t src = ((img * h + j + rho * lc) << LOGW) + t;
#pragma unroll
    for (int i = 0; i < G::E; ++i) {
        const V x = live ? in.ld(src + i * G::T) : V{0, 0};
        v[i] = CONJ_IN ? cconj(x) : x;
    }
    const LdsLines<V, 1> L{my + rho * SLOTS, 0};
    fft_regs<LOGW>(v, t, tb, L);
    __syncthreads();  // every LDS read of the row transforms is done
    {
        V* wp = L.ptr(t);
#pragma unroll
        for (int i = 0; i < G::E; ++i) wp[LdsLines<V, 1>::off(i * G::T)] = v[i];
    }
    __syncthreads();
    V* dst = out + ((img * h + j * F) << LOGW);
#pragma unroll
    for (int k = 0; k < EF; ++k) {
        const int p = t + (rho * EF + k) * G::T;
        V u[F];
#pragma unroll
        for (int r = 0; r < F; ++r) u[r] = *LdsLines<V, 1>{my + r * SLOTS, 0}.ptr(p);
        Dft<F>::run(u);
        if (live) {
#pragma unroll
            for (int r = 0; r < F; ++r) st_stream(dst + ((int64_t)r << LOGW) + p, u[r]);
        }
    }
}

// ---------------------------------------------------------------------------
// Multi-pass Stockham super-stage (large 1D).  KIND 0: first (span 1, stored
// along lines after a remap), 1: middle, 2: last (in place).
// ---------------------------------------------------------------------------
// IN: ldv(index, P values); OUT: st_plain (KIND 0) or stv (KIND 1, 2) -- the
// caller's arrays (io.hpp), or the chirp-z steps of chirp_io.hpp.
template <typename V, int LOGR, int KIND, bool CONJ_IN, bool CONJ_OUT, typename IN, typename OUT>
__global__ __launch_bounds__((Tile<V, LOGR>::THREADS))
void stock_pass_kernel(IN in, OUT out, int logn, int logns, int64_t tiles_per_sig, const V* __restrict__ tw,
                       BigTw<V> big, typename real_of<V>::type scale)
{
    using G = Geom<V, LOGR>;
    using TL = Tile<V, LOGR>;
    __shared__ V lds[TL::LDS];
    const int tid = threadIdx.x;
    const int c0 = tid % TL::CL, t = tid / TL::CL;
    // workgroups in launch order (the XCD-contiguous order of the 2D passes
    // measured slower here: 2^24 points 149 -> 146 us without it)
    const int64_t tile = blockIdx.x;
    const int64_t sig = tile / tiles_per_sig;
    const int64_t j0 = (tile % tiles_per_sig) * TL::C;
    const int64_t j = j0 + c0 * TL::P;
    const int64_t sbase = sig << logn;
    const int64_t stride = (int64_t)1 << (logn - LOGR);  // N / R

    V v[TL::P][G::E];
    {
        const int64_t src = sbase + j + t * stride;
#pragma unroll
        for (int i = 0; i < G::E; ++i) {
            V q[TL::P];
            in.ldv(src + i * G::T * stride, q);
#pragma unroll
            for (int g = 0; g < TL::P; ++g) v[g][i] = CONJ_IN ? cconj(q[g]) : q[g];
        }
    }
    const int64_t ns_mask = ((int64_t)1 << logns) - 1;
    if constexpr (KIND != 0) {
#pragma unroll
        for (int g = 0; g < TL::P; ++g) apply_big_twiddle<LOGR>(v[g], (j + g) & ns_mask, t, big);
    }

    if constexpr (KIND == 0) {
        // Lanes along a line for the store: thread -> (line slot cb, tb_t).
        const int cb = tid / G::T, tb_t = tid % G::T;
        TwBases<V, LOGR> tb;
        tb.load(tw, tb_t);
#pragma unroll
        for (int g = 0; g < TL::P; ++g) {
            if (g > 0) __syncthreads();
            fft_regs_remap<LOGR>(v[g], t, LdsLines<V, TL::CL>{lds, c0}, tb_t, tb, LdsLines<V, TL::CL>{lds, cb});
        }
#pragma unroll
        for (int g = 0; g < TL::P; ++g) {
            const int64_t dst = sbase + ((j0 + cb * TL::P + g) << LOGR) + tb_t;
#pragma unroll
            for (int i = 0; i < G::E; ++i) out.st_plain(dst + i * G::T, v[g][i]);
        }
    } else {
        TwBases<V, LOGR> tb;
        tb.load(tw, t);
#pragma unroll
        for (int g = 0; g < TL::P; ++g) {
            if (g > 0) __syncthreads();
            fft_regs<LOGR>(v[g], t, tb, LdsLines<V, TL::CL>{lds, c0});
        }
        const int64_t ns = (int64_t)1 << logns;
        const int64_t dst = sbase + ((j >> logns) << (logns + LOGR)) + (j & ns_mask) + t * ns;
#pragma unroll
        for (int i = 0; i < G::E; ++i) {
            V q[TL::P];
#pragma unroll
            for (int g = 0; g < TL::P; ++g) {
                const V y = v[g][i];
                q[g] = CONJ_OUT ? V{y.x * scale, -y.y * scale} : y;
            }
            out.stv(dst + i * G::T * ns, q);
        }
    }
}

// ---------------------------------------------------------------------------
// Launchers
// ---------------------------------------------------------------------------
static inline dim3 grid_of(int64_t blocks) { return dim3((unsigned)blocks); }

template <typename V, int LOGL, bool ONE>
static hipError_t cols2d_t(const void* in, void* out, void* out_im, int64_t nimg, int64_t w, int logf,
                           const void* tw, BigTwiddle htw, bool ci, bool co, double scale, hipStream_t s)
{
    using TL = ColTile<V, LOGL, ONE>;
    if constexpr (TL::THREADS > 1024) {
        return hipErrorInvalidValue;
    } else {
        const int64_t col_tiles = (w + TL::C - 1) / TL::C;
        const int64_t blocks = (col_tiles << logf) * nimg;
        if (blocks > 0x7fffffff) return hipErrorInvalidConfiguration;
        if (w % TL::P) return hipErrorInvalidValue;
        using Rl = typename real_of<V>::type;
        const BigTw<V> big{(const V*)htw.hi, (const V*)htw.lo, htw.lbits, htw.logn};
#define FFTMI_C2(CI, CO, PO)                                                                                      \
    hipLaunchKernelGGL((cols2d_kernel<V, LOGL, CO, PO, ONE, CI>), grid_of(blocks), dim3(TL::THREADS), 0, s,         \
                       (const V*)in, make_out<V, PO>(out, out_im), w, logf, col_tiles, (const V*)tw, big, (Rl)scale)
        if constexpr (ONE) {
            // the real-image column passes: forward (no conj), inverse (conj on
            // both sides, or only on the store after a conjugating column stage)
            if (out_im || (ci && !co)) return hipErrorInvalidValue;
            if (ci) FFTMI_C2(true, true, false);
            else if (co) FFTMI_C2(false, true, false);
            else FFTMI_C2(false, false, false);
        } else {
            if (ci) return hipErrorInvalidValue;
            if (out_im) {
                if (co) FFTMI_C2(false, true, true);
                else FFTMI_C2(false, false, true);
            } else {
                if (co) FFTMI_C2(false, true, false);
                else FFTMI_C2(false, false, false);
            }
        }
#undef FFTMI_C2
        return hipGetLastError();
    }
}

template <typename V, int LOGW, int LOGF> constexpr bool fold_ok()
{
    using G = Geom<V, LOGW>;
    constexpr long threads = (long)(G::T << LOGF) * fold_groups<V, LOGW, LOGF>();
    constexpr long lds = (long)lds_padded(G::N) * (1 << LOGF) * fold_groups<V, LOGW, LOGF>() * (long)sizeof(V);
    return G::E >= (1 << LOGF) && threads <= 1024 && lds <= 160 * 1024;
}

template <typename V, int LOGW, int LOGF>
static hipError_t fold_t(const void* in, const void* in_im, void* out, int64_t nimg, int log_lc, const void* tw,
                         bool ci, hipStream_t s)
{
    if constexpr (!fold_ok<V, LOGW, LOGF>()) {
        return hipErrorInvalidValue;
    } else {
        constexpr int GR = fold_groups<V, LOGW, LOGF>();
        const int64_t ngroups = nimg << log_lc;
        const int64_t blocks = (ngroups + GR - 1) / GR;
        if (blocks > 0x7fffffff) return hipErrorInvalidConfiguration;
        const dim3 block((Geom<V, LOGW>::T << LOGF) * GR);
#define FFTMI_FOLD(CI, PI)                                                                           \
    hipLaunchKernelGGL((rows2d_fold_kernel<V, LOGW, LOGF, CI, PI>), grid_of(blocks), block, 0, s,       \
                       make_in<V, PI>(in, in_im), (V*)out, ngroups, log_lc, (const V*)tw)
        if (in_im) {
            if (ci) FFTMI_FOLD(true, true);
            else FFTMI_FOLD(false, true);
        } else {
            if (ci) FFTMI_FOLD(true, false);
            else FFTMI_FOLD(false, false);
        }
#undef FFTMI_FOLD
        return hipGetLastError();
    }
}

template <typename V, int LOGR, int KIND, bool CI, bool CO, typename IN, typename OUT>
static hipError_t stock_launch(IN in, OUT out, int logn, int logns, int64_t batch, const void* tw, BigTwiddle bt,
                               double scale, hipStream_t s)
{
    using TL = Tile<V, LOGR>;
    if (TL::THREADS > 1024) return hipErrorInvalidValue;
    const int64_t butterflies = (int64_t)1 << (logn - LOGR);
    if (butterflies % TL::C) return hipErrorInvalidValue;
    if (KIND == 1 && ((int64_t)1 << logns) % TL::C) return hipErrorInvalidValue;
    const int64_t tps = butterflies / TL::C;
    const int64_t blocks = tps * batch;
    if (blocks > 0x7fffffff) return hipErrorInvalidConfiguration;
    using Rl = typename real_of<V>::type;
    const BigTw<V> big{(const V*)bt.hi, (const V*)bt.lo, bt.lbits, bt.logn};
    hipLaunchKernelGGL((stock_pass_kernel<V, LOGR, KIND, CI, CO, IN, OUT>), grid_of(blocks), dim3(TL::THREADS), 0, s,
                       in, out, logn, logns, tps, (const V*)tw, big, (Rl)scale);
    return hipGetLastError();
}

template <typename V, int LOGR, int KIND>
static hipError_t stock_t(const Io& io, int logn, int logns, int64_t batch, const void* tw, BigTwiddle bt, bool ci,
                          bool co, double scale, hipStream_t s)
{
#define FFTMI_SP(CI, CO, PL)                                                                                 \
    return stock_launch<V, LOGR, KIND, CI, CO>(make_in<V, PL && KIND == 0>(io.in, io.in_im),                \
                                               make_out<V, PL && KIND == 2>(io.out, io.out_im), logn, logns, \
                                               batch, tw, bt, scale, s)
    // Planar: the first pass reads the caller's planes (no conjugated store),
    // the last writes them (no conjugated load).
    const bool pl = io.in_im != nullptr || io.out_im != nullptr;
    if (pl) {
        if constexpr (KIND == 0) {
            if (io.out_im || co) return hipErrorInvalidValue;
            if (ci) FFTMI_SP(true, false, true);
            else FFTMI_SP(false, false, true);
        } else if constexpr (KIND == 2) {
            if (io.in_im || ci) return hipErrorInvalidValue;
            if (co) FFTMI_SP(false, true, true);
            else FFTMI_SP(false, false, true);
        } else {
            return hipErrorInvalidValue;
        }
    } else if (ci && co) FFTMI_SP(true, true, false);
    else if (ci) FFTMI_SP(true, false, false);
    else if (co) FFTMI_SP(false, true, false);
    else FFTMI_SP(false, false, false);
#undef FFTMI_SP
}

// Bluestein's passes (chirp_io.hpp): mode 0 = first forward pass (chirp in),
// 2 = last forward pass (x B, conjugated), 4 = last inverse pass (chirp out).
template <typename V, int LOGR, bool PL>
static hipError_t bluestein_pass_t(int mode, const void* in, void* out, int logm, int logns, int64_t batch,
                                   const void* tw, BigTwiddle bt, const ChirpArgs& c, hipStream_t s)
{
    using Rl = typename real_of<V>::type;
    if (mode == 0) {
        const ChirpIn<V, PL> ci{make_in<V, PL>(c.x, c.x_im), (const V*)c.chirp, c.n, logm, (int)c.conj_in};
        return stock_launch<V, LOGR, 0, false, false>(ci, make_out<V, false>(out, nullptr), logm, logns, batch, tw,
                                                       bt, 1.0, s);
    }
    if constexpr (!PL) {
        if (mode == 2) {
            const MulConjOut<V> mo{(V*)out, (const V*)c.bspec, logm};
            return stock_launch<V, LOGR, 2, false, false>(make_in<V, false>(in, nullptr), mo, logm, logns, batch, tw,
                                                           bt, 1.0, s);
        }
    }
    if (mode == 4) {
        const ChirpOut<V, PL> co{make_out<V, PL>(c.y, c.y_im), (const V*)c.chirp, c.n, logm, (int)c.conj_out,
                                 (Rl)c.scale, (Rl)(1.0 / (double)((int64_t)1 << logm))};
        return stock_launch<V, LOGR, 2, false, false>(make_in<V, false>(in, nullptr), co, logm, logns, batch, tw, bt,
                                                       1.0, s);
    }
    return hipErrorInvalidValue;
}

hipError_t launch_bluestein_pass(int prec, int logr, int mode, const void* in, void* out, int logm, int logns,
                                 int64_t batch, const void* tw, BigTwiddle big, const ChirpArgs& c, hipStream_t s)
{
    // planar only where the pass touches the caller's arrays
    const bool pl = mode == 0 ? c.x_im != nullptr : mode == 4 ? c.y_im != nullptr : false;
#define BP(L) (prec == 0 ? (pl ? bluestein_pass_t<float2, L, true>(mode, in, out, logm, logns, batch, tw, big, c, s)   \
                               : bluestein_pass_t<float2, L, false>(mode, in, out, logm, logns, batch, tw, big, c, s)) \
                         : (pl ? bluestein_pass_t<double2, L, true>(mode, in, out, logm, logns, batch, tw, big, c, s)  \
                               : bluestein_pass_t<double2, L, false>(mode, in, out, logm, logns, batch, tw, big, c, s)))
    switch (logr) {
        case 5: return BP(5);
        case 6: return BP(6);
        case 7: return BP(7);
        case 8: return BP(8);
        case 9: return BP(9);
        default: return hipErrorInvalidValue;
    }
#undef BP
}

#define FFTMI_LOG_SWITCH(PREC, L, CALL_F, CALL_D)                                     \
    switch (L) {                                                                    \
        case 1: return PREC == 0 ? CALL_F(1) : CALL_D(1);                           \
        case 2: return PREC == 0 ? CALL_F(2) : CALL_D(2);                           \
        case 3: return PREC == 0 ? CALL_F(3) : CALL_D(3);                           \
        case 4: return PREC == 0 ? CALL_F(4) : CALL_D(4);                           \
        case 5: return PREC == 0 ? CALL_F(5) : CALL_D(5);                           \
        case 6: return PREC == 0 ? CALL_F(6) : CALL_D(6);                           \
        case 7: return PREC == 0 ? CALL_F(7) : CALL_D(7);                           \
        case 8: return PREC == 0 ? CALL_F(8) : CALL_D(8);                           \
        case 9: return PREC == 0 ? CALL_F(9) : CALL_D(9);                           \
        case 10: return PREC == 0 ? CALL_F(10) : CALL_D(10);                        \
        case 11: return PREC == 0 ? CALL_F(11) : hipErrorInvalidValue;              \
        default: return hipErrorInvalidValue;                                       \
    }

hipError_t launch_cols2d(int prec, int logl, const void* in, void* out, int64_t nimg, int64_t w, int logf,
                         const void* tw, BigTwiddle htw, bool co, double scale, hipStream_t s, void* out_im,
                         bool one_col, bool ci)
{
#define CF(L) (one_col ? cols2d_t<float2, L, true>(in, out, out_im, nimg, w, logf, tw, htw, ci, co, scale, s) \
                       : cols2d_t<float2, L, false>(in, out, out_im, nimg, w, logf, tw, htw, ci, co, scale, s))
#define CD(L) (one_col ? cols2d_t<double2, L, true>(in, out, out_im, nimg, w, logf, tw, htw, ci, co, scale, s) \
                       : cols2d_t<double2, L, false>(in, out, out_im, nimg, w, logf, tw, htw, ci, co, scale, s))
    FFTMI_LOG_SWITCH(prec, logl, CF, CD)
#undef CF
#undef CD
}

template <typename V, int LOGF, bool ONE>
static hipError_t colstage_t(const void* in, void* out, int64_t nimg, int64_t w, int log_lc, bool ci, hipStream_t s)
{
    constexpr int P = ONE ? 1 : 16 / (int)sizeof(V);
    if (w % P) return hipErrorInvalidValue;
    const int64_t total = (nimg << log_lc) * (w / P);
    int64_t blocks = (total + 255) / 256;
    if (blocks > (1 << 20)) blocks = 1 << 20;
    hipLaunchKernelGGL((colstage_kernel<V, LOGF, ONE>), dim3((unsigned)blocks), dim3(256), 0, s, (const V*)in,
                       (V*)out, w, log_lc, total, (int)ci);
    return hipGetLastError();
}

hipError_t launch_colstage(int prec, int logf, const void* in, void* out, int64_t nimg, int64_t w, int log_lc,
                           hipStream_t s, bool one_col, bool ci)
{
#define CS1(F, ONE) (prec == 0 ? colstage_t<float2, F, ONE>(in, out, nimg, w, log_lc, ci, s) \
                               : colstage_t<double2, F, ONE>(in, out, nimg, w, log_lc, ci, s))
#define CS(F) (one_col ? CS1(F, true) : CS1(F, false))
    switch (logf) {
        case 1: return CS(1);
        case 2: return CS(2);
        case 3: return CS(3);
        case 4: return CS(4);
        default: return hipErrorInvalidValue;
    }
#undef CS
#undef CS1
}

hipError_t launch_rows2d_fold(int prec, int logw, int logf, const void* in, void* out, int64_t nimg, int log_lc,
                              const void* tw, bool ci, hipStream_t s, const void* in_im)
{
#define FOLD_F(LW) (logf == 1 ? fold_t<float2, LW, 1>(in, in_im, out, nimg, log_lc, tw, ci, s)   \
                  : logf == 2 ? fold_t<float2, LW, 2>(in, in_im, out, nimg, log_lc, tw, ci, s) \
                  : logf == 3 ? fold_t<float2, LW, 3>(in, in_im, out, nimg, log_lc, tw, ci, s) \
                              : hipErrorInvalidValue)
#define FOLD_D(LW) (logf == 1 ? fold_t<double2, LW, 1>(in, in_im, out, nimg, log_lc, tw, ci, s)   \
                  : logf == 2 ? fold_t<double2, LW, 2>(in, in_im, out, nimg, log_lc, tw, ci, s) \
                  : logf == 3 ? fold_t<double2, LW, 3>(in, in_im, out, nimg, log_lc, tw, ci, s) \
                              : hipErrorInvalidValue)
    switch (logw) {
        case 1: return prec == 0 ? FOLD_F(1) : FOLD_D(1);
        case 2: return prec == 0 ? FOLD_F(2) : FOLD_D(2);
        case 3: return prec == 0 ? FOLD_F(3) : FOLD_D(3);
        case 4: return prec == 0 ? FOLD_F(4) : FOLD_D(4);
        case 5: return prec == 0 ? FOLD_F(5) : FOLD_D(5);
        case 6: return prec == 0 ? FOLD_F(6) : FOLD_D(6);
        case 7: return prec == 0 ? FOLD_F(7) : FOLD_D(7);
        case 8: return prec == 0 ? FOLD_F(8) : FOLD_D(8);
        case 9: return prec == 0 ? FOLD_F(9) : FOLD_D(9);
        case 10: return prec == 0 ? FOLD_F(10) : FOLD_D(10);
        case 11: return prec == 0 ? FOLD_F(11) : FOLD_D(11);
        case 12: return prec == 0 ? FOLD_F(12) : FOLD_D(12);
        case 13: return prec == 0 ? FOLD_F(13) : hipErrorInvalidValue;
        default: return hipErrorInvalidValue;
    }
#undef FOLD_F
#undef FOLD_D
}

hipError_t launch_stock_pass(int prec, int logr, int kind, const void* in, void* out, int logn, int logns,
                             int64_t batch, const void* tw, BigTwiddle big, bool ci, bool co, double scale,
                             hipStream_t s, const void* in_im, void* out_im)
{
    const Io io{in, in_im, out, out_im};
#define SK(L, K, V) stock_t<V, L, K>(io, logn, logns, batch, tw, big, ci, co, scale, s)
#define SF(L) (kind == 0 ? SK(L, 0, float2) : kind == 1 ? SK(L, 1, float2) : SK(L, 2, float2))
#define SD(L) (kind == 0 ? SK(L, 0, double2) : kind == 1 ? SK(L, 1, double2) : SK(L, 2, double2))
    switch (logr) {
        case 5: return prec == 0 ? SF(5) : SD(5);
        case 6: return prec == 0 ? SF(6) : SD(6);
        case 7: return prec == 0 ? SF(7) : SD(7);
        case 8: return prec == 0 ? SF(8) : SD(8);
        case 9: return prec == 0 ? SF(9) : SD(9);
        default: return hipErrorInvalidValue;
    }
#undef SK
#undef SF
#undef SD
}

bool fold_supported(int prec, int logw, int logf)
{
#define FS(LW) (prec == 0 ? (logf == 1 ? fold_ok<float2, LW, 1>() : logf == 2 ? fold_ok<float2, LW, 2>() \
                             : logf == 3 ? fold_ok<float2, LW, 3>() : false)                            \
                          : (logf == 1 ? fold_ok<double2, LW, 1>() : logf == 2 ? fold_ok<double2, LW, 2>() \
                             : logf == 3 ? fold_ok<double2, LW, 3>() : false))
    switch (logw) {
        case 1: return FS(1);
        case 2: return FS(2);
        case 3: return FS(3);
        case 4: return FS(4);
        case 5: return FS(5);
        case 6: return FS(6);
        case 7: return FS(7);
        case 8: return FS(8);
        case 9: return FS(9);
        case 10: return FS(10);
        case 11: return FS(11);
        case 12: return FS(12);
        case 13: return prec == 0 && (logf == 1 ? fold_ok<float2, 13, 1>() : logf == 2 ? fold_ok<float2, 13, 2>()
                                      : logf == 3 ? fold_ok<float2, 13, 3>() : false);
        default: return false;
    }
#undef FS
}

int tile_lines_2d(int prec, int logl)
{
    switch (logl) {
#define TL2(L) case L: return prec == 0 ? Tile<float2, L>::C : Tile<double2, L>::C;
        TL2(1) TL2(2) TL2(3) TL2(4) TL2(5) TL2(6) TL2(7) TL2(8) TL2(9) TL2(10)
        case 11: return prec == 0 ? Tile<float2, 11>::C : 0;
#undef TL2
        default: return 0;
    }
}

// ---------------------------------------------------------------------------
// Transpose of nmat matrices [rows][cols] -> [cols][rows] (complex elements),
// through 32 x 32 tiles in LDS (one pad slot per tile row), for axes whose
// transform runs as rank-1 rows: the axis is brought innermost, transformed,
// and brought back.  Both sides read and write 32 consecutive elements per
// tile row.  Planar input and / or output as for the other first and last
// passes.
// ---------------------------------------------------------------------------
template <typename V, bool PIN, bool POUT>
__global__ __launch_bounds__(256) void transpose_kernel(CIn<V, PIN> in, COut<V, POUT> out, int64_t rows,
                                                        int64_t cols, int64_t nmat)
{
    __shared__ V tile[32][33];
    const int64_t tx = (cols + 31) / 32, ty = (rows + 31) / 32;
    const int64_t per = tx * ty;
    const int lx = threadIdx.x & 31, ly = threadIdx.x >> 5;  // 32 x 8 threads
    for (int64_t b = blockIdx.x; b < per * nmat; b += gridDim.x) {
        const int64_t m = b / per, q = b % per;
        const int64_t r0 = (q / tx) * 32, c0 = (q % tx) * 32;
        const int64_t base = m * rows * cols;
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            const int64_t r = r0 + ly + 8 * k, c = c0 + lx;
            if (r < rows && c < cols) tile[ly + 8 * k][lx] = in.ld_plain(base + r * cols + c);
        }
        __syncthreads();
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            const int64_t c = c0 + ly + 8 * k, r = r0 + lx;  // output row c, column r
            if (r < rows && c < cols) out.st_plain(base + c * rows + r, tile[lx][ly + 8 * k]);
        }
        __syncthreads();  // the tile is read before the next one overwrites it
    }
}

template <typename V, bool PIN, bool POUT>
static hipError_t launch_transpose_t(const void* in, const void* in_im, void* out, void* out_im, int64_t rows,
                                     int64_t cols, int64_t nmat, hipStream_t s)
{
    const int64_t tiles = ((cols + 31) / 32) * ((rows + 31) / 32) * nmat;
    const int64_t blocks = tiles < (1 << 20) ? tiles : (1 << 20);
    if (blocks == 0) return hipSuccess;
    hipLaunchKernelGGL((transpose_kernel<V, PIN, POUT>), dim3((unsigned)blocks), dim3(256), 0, s,
                       make_in<V, PIN>(in, in_im), make_out<V, POUT>(out, out_im), rows, cols, nmat);
    return hipGetLastError();
}

template <typename V>
static hipError_t launch_transpose_v(const void* in, const void* in_im, void* out, void* out_im, int64_t rows,
                                     int64_t cols, int64_t nmat, hipStream_t s)
{
    if (in_im && out_im) return launch_transpose_t<V, true, true>(in, in_im, out, out_im, rows, cols, nmat, s);
    if (in_im) return launch_transpose_t<V, true, false>(in, in_im, out, out_im, rows, cols, nmat, s);
    if (out_im) return launch_transpose_t<V, false, true>(in, in_im, out, out_im, rows, cols, nmat, s);
    return launch_transpose_t<V, false, false>(in, in_im, out, out_im, rows, cols, nmat, s);
}

hipError_t launch_transpose(int prec, const void* in, const void* in_im, void* out, void* out_im, int64_t rows,
                            int64_t cols, int64_t nmat, hipStream_t s)
{
    return prec == 0 ? launch_transpose_v<float2>(in, in_im, out, out_im, rows, cols, nmat, s)
                     : launch_transpose_v<double2>(in, in_im, out, out_im, rows, cols, nmat, s);
}

}  // namespace fftmi
