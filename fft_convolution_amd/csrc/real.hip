// real.hip -- transforms of real rows through the complex transform of half
// their length.
//
// A real row x of N = 2H points, read as H complex values z_n = x_{2n} +
// i x_{2n+1} (the same memory), has the H-point transform Z_k = E_k + i O_k,
// E and O being the transforms of the even and odd samples.  Both of those
// are transforms of real rows, so conj Z_{H-k} = E_k - i O_k and
//     E_k = (Z_k + conj Z_{H-k}) / 2,    O_k = -i (Z_k - conj Z_{H-k}) / 2;
// the radix-2 combine of "FFT on GPU" (section "Fast Fourier Transform") then
// gives X_k = E_k + w_N^k O_k for k = 0 .. H (E_H = E_0, O_H = O_0), the
// N/2 + 1 bins that determine the rest (X_{N-k} = conj X_k).
// The way back undoes the two steps:
//     E_k = (X_k + conj X_{H-k}) / 2,   O_k = w_N^{-k} (X_k - conj X_{H-k}) / 2,
//     Z_k = E_k + i O_k,   z = F_H^{-1} Z,   x_{2n} = Re z_n,  x_{2n+1} = Im z_n,
// with the imaginary parts of X_0 and X_H taken as zero (a real row's are).
//
// H within the one-kernel range: one workgroup per row (group) runs the
// H-point transform in registers and LDS and does the split (or, backwards,
// the merge) through one more LDS exchange, so a row crosses HBM once each
// way.  Longer rows: the H-point multi-pass transform plus one pass that
// handles the bins k and H - k together.  Rows of odd length have no half
// length: they go through the N-point complex transform of the row itself
// (real_odd_kernel, at the end).
#include "io.hpp"
#include "launch.hpp"
#include "stockham.hpp"
#include "tile_common.hpp"

namespace fftmi {

template <typename V> __device__ __forceinline__ V chalf(V a) { return V{a.x * 0.5f, a.y * 0.5f}; }
__device__ __forceinline__ float fmar(float a, float b, float c) { return __builtin_fmaf(a, b, c); }
__device__ __forceinline__ double fmar(double a, double b, double c) { return __builtin_fma(a, b, c); }

// X_k from a = Z_k, b = Z_{H-k} and wh = w_N^k / 2:
//   X_k = (a + conj b) / 2 - i (a - conj b) w_N^k / 2,
// the halves folded into wh and into fused multiply-adds (10 operations).
template <typename V> __device__ __forceinline__ V real_split(V a, V b, V wh)
{
    using Rl = typename real_of<V>::type;
    const Rl px = a.x + b.x, py = a.y - b.y;  // a + conj b
    const Rl qx = a.x - b.x, qy = a.y + b.y;  // a - conj b
    // -i q wh = (qy, -qx)(c, d) = (qy c + qx d, qy d - qx c)
    return V{fmar((Rl)0.5, px, fmar(qy, wh.x, qx * wh.y)), fmar((Rl)0.5, py, fmar(qy, wh.y, -(qx * wh.x)))};
}

// Z_k from a = X_k, b = X_{H-k} and wh = w_N^k / 2:
//   Z_k = (a + conj b) / 2 + i (a - conj b) conj(w_N^k) / 2.
template <typename V> __device__ __forceinline__ V real_merge(V a, V b, V wh)
{
    using Rl = typename real_of<V>::type;
    const Rl px = a.x + b.x, py = a.y - b.y;  // a + conj b
    const Rl qx = a.x - b.x, qy = a.y + b.y;  // a - conj b
    // i q conj(wh) = i (qx c + qy d, qy c - qx d) = (qx d - qy c, qx c + qy d)
    return V{fmar((Rl)0.5, px, fmar(qx, wh.y, -(qy * wh.x))), fmar((Rl)0.5, py, fmar(qx, wh.x, qy * wh.y))};
}

// The partner H - k of a thread's bin k = t + i T in the LDS row (H + 1
// slots, the last one bin H): (T - t) + (E - 1 - i) T, for T a multiple of 16
// one base per thread plus compile-time offsets (the layout pads one slot per
// 16, so a delta that is a multiple of 16 adds a fixed number of slots);
// smaller rows compute each slot.
template <typename V, int T, int E> __device__ __forceinline__ V partner(const LdsLines<V, 1>& L, int t, int i)
{
    if constexpr (T % 16 == 0)
        return L.ptr(T - t)[LdsLines<V, 1>::off((E - 1 - i) * T)];
    else
        return *L.ptr((T - t) + (E - 1 - i) * T);
}

// Slots per row in LDS: the H-point exchange layout plus one for X_H.
template <int LOGH> constexpr int real_slots() { return lds_padded(1 << LOGH) + 1; }

// R2C, one-kernel range.  in: [nrows][2H] real (read as [nrows][H] complex),
// out: [nrows][H + 1].  whi/wlo: w_N^{i T} and w_N^t (N = 2H), so that
// w_N^{t + i T} = whi[i] wlo[t] for the element v[i] of thread t.
template <typename V, int LOGH>
__global__ __launch_bounds__((Geom<V, LOGH>::T * rows_per_wg<V, LOGH>()))
void r2c_rows_kernel(const V* in, V* out, int64_t nrows, const V* __restrict__ tw, const V* __restrict__ whi,
                     const V* __restrict__ wlo)
{
    using G = Geom<V, LOGH>;
    constexpr int H = G::N, T = G::T, E = G::E;
    constexpr int RPW = rows_per_wg<V, LOGH>();
    constexpr int SLOTS = real_slots<LOGH>();
    __shared__ V lds[SLOTS * RPW];

    const int tid = threadIdx.x;
    const int rloc = tid / T;
    const int t = tid % T;
    const int64_t row = (int64_t)blockIdx.x * RPW + rloc;
    const bool live = row < nrows;

    TwBases<V, LOGH> tb;
    tb.load(tw, t);
    V v[E];
    const V* src = in + row * H + t;
#pragma unroll
    for (int i = 0; i < E; ++i) v[i] = live ? ld_stream(src + i * T) : V{0, 0};
    const LdsLines<V, 1> L{lds + rloc * SLOTS, 0};
    if constexpr (LOGH > 0) fft_regs<LOGH>(v, t, tb, L);
    __syncthreads();  // the transform's last exchange is read by now
#pragma unroll
    for (int i = 0; i < E; ++i) *L.ptr(t + i * T) = v[i];
    __syncthreads();
    if (!live) return;
    const V wh0 = chalf(wlo[t]);  // w_N^k / 2 = whi[i] (wlo[t] / 2), exact
    V* dst = out + row * (H + 1);
#pragma unroll
    for (int i = 0; i < E; ++i) {
        const int k = t + i * T;
        // bin 0 pairs with itself (H - 0 wraps to 0)
        const V b = (i == 0 && t == 0) ? v[0] : partner<V, T, E>(L, t, i);
        // rows of H + 1 bins start anywhere in a 128-byte line: nontemporal
        // stores write some lines partially twice (16384 x 8192 real rows:
        // 527 MiB written against 512.5 with plain stores), but plain stores
        // measured slower (186.5 -> 193.6 us, same-box A/B)
        st_stream(at_bytes(dst, (unsigned)k * (unsigned)sizeof(V)), real_split(v[i], b, cmul(whi[i], wh0)));
    }
    if (t == 0) st_stream(dst + H, V{v[0].x - v[0].y, 0});
}

// C2R, one-kernel range.  in: [nrows][H + 1], out: [nrows][2H] real (written
// as [nrows][H] complex).  scale = 1/H (the inverse H-point transform's).
template <typename V, int LOGH>
__global__ __launch_bounds__((Geom<V, LOGH>::T * rows_per_wg<V, LOGH>()))
void c2r_rows_kernel(const V* in, V* out, int64_t nrows, const V* __restrict__ tw, const V* __restrict__ whi,
                     const V* __restrict__ wlo, typename real_of<V>::type scale)
{
    using G = Geom<V, LOGH>;
    constexpr int H = G::N, T = G::T, E = G::E;
    constexpr int RPW = rows_per_wg<V, LOGH>();
    constexpr int SLOTS = real_slots<LOGH>();
    __shared__ V lds[SLOTS * RPW];

    const int tid = threadIdx.x;
    const int rloc = tid / T;
    const int t = tid % T;
    const int64_t row = (int64_t)blockIdx.x * RPW + rloc;
    const bool live = row < nrows;

    TwBases<V, LOGH> tb;
    tb.load(tw, t);
    V v[E];
    const V* src = in + row * (H + 1);
#pragma unroll
    for (int i = 0; i < E; ++i) v[i] = live ? ld_stream(src + t + i * T) : V{0, 0};
    const LdsLines<V, 1> L{lds + rloc * SLOTS, 0};
    if (t == 0) {
        v[0].y = 0;
        const V xh = live ? src[H] : V{0, 0};
        *L.ptr(H) = V{xh.x, 0};
    }
#pragma unroll
    for (int i = 0; i < E; ++i) *L.ptr(t + i * T) = v[i];
    __syncthreads();
    const V wh0 = chalf(wlo[t]);  // w_N^k / 2 = whi[i] (wlo[t] / 2), exact
#pragma unroll
    for (int i = 0; i < E; ++i) {
        // inverse transform as conj(F(conj Z)) / H; the partner of bin 0 is
        // bin H, held in the slot after the row
        v[i] = cconj(real_merge(v[i], partner<V, T, E>(L, t, i), cmul(whi[i], wh0)));
    }
    __syncthreads();  // partners are read before the transform reuses the LDS
    if constexpr (LOGH > 0) fft_regs<LOGH>(v, t, tb, L);
    if (!live) return;
    V* dst = out + row * H + t;
#pragma unroll
    for (int i = 0; i < E; ++i) st_stream(dst + i * T, V{v[i].x * scale, -v[i].y * scale});
}

// Longer rows.  One thread per bin pair (k, H - k), k = 0 .. H/2, of each row.
// R2C: z [batch][H] (the H-point transform) -> out [batch][H + 1].
template <typename V>
__global__ void r2c_pairs_kernel(const V* __restrict__ z, V* __restrict__ out, int64_t h, int64_t batch, BigTw<V> wn)
{
    const int64_t npair = h / 2 + 1;
    for (int64_t row = blockIdx.y; row < batch; row += gridDim.y) {
        const V* zr = z + row * h;
        V* xr = out + row * (h + 1);
        for (int64_t k = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; k < npair;
             k += (int64_t)gridDim.x * blockDim.x) {
            if (k == 0) {
                const V z0 = zr[0];
                xr[0] = V{z0.x + z0.y, 0};
                xr[h] = V{z0.x - z0.y, 0};
                continue;
            }
            const V a = zr[k], b = zr[h - k];
            const V w = chalf(wn(k));
            xr[k] = real_split(a, b, w);
            if (2 * k != h) xr[h - k] = real_split(b, a, V{-w.x, w.y});  // w_N^{H-k} = -conj w_N^k
        }
    }
}

// C2R: x [batch][H + 1] -> z [batch][H], the spectrum of the packed real row.
template <typename V>
__global__ void c2r_pairs_kernel(const V* __restrict__ x, V* __restrict__ z, int64_t h, int64_t batch, BigTw<V> wn)
{
    const int64_t npair = h / 2 + 1;
    for (int64_t row = blockIdx.y; row < batch; row += gridDim.y) {
        const V* xr = x + row * (h + 1);
        V* zr = z + row * h;
        for (int64_t k = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; k < npair;
             k += (int64_t)gridDim.x * blockDim.x) {
            if (k == 0) {
                const auto a = xr[0].x, b = xr[h].x;
                zr[0] = V{(a + b) * 0.5f, (a - b) * 0.5f};
                continue;
            }
            const V a = xr[k], b = xr[h - k];
            const V w = chalf(wn(k));
            zr[k] = real_merge(a, b, w);
            if (2 * k != h) zr[h - k] = real_merge(b, a, V{-w.x, w.y});
        }
    }
}

// N = 1: X_0 = x_0, and back.
template <typename V>
__global__ void real_n1_kernel(const void* in, void* out, int64_t batch, int c2r)
{
    using Rl = typename real_of<V>::type;
    for (int64_t e = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; e < batch; e += (int64_t)gridDim.x * blockDim.x) {
        if (c2r)
            ((Rl*)out)[e] = ((const V*)in)[e].x;
        else
            ((V*)out)[e] = V{((const Rl*)in)[e], 0};
    }
}

template <typename V, int LOGH>
static hipError_t launch_real_rows_t(bool c2r, const void* in, void* out, int64_t nrows, const void* tw,
                                     const void* whi, const void* wlo, hipStream_t s)
{
    constexpr int RPW = rows_per_wg<V, LOGH>();
    constexpr int BLOCK = Geom<V, LOGH>::T * RPW;
    const int64_t blocks = (nrows + RPW - 1) / RPW;
    if (blocks > 0x7fffffff) return hipErrorInvalidConfiguration;
    using Rl = typename real_of<V>::type;
    if (c2r)
        hipLaunchKernelGGL((c2r_rows_kernel<V, LOGH>), dim3((unsigned)blocks), dim3(BLOCK), 0, s, (const V*)in,
                           (V*)out, nrows, (const V*)tw, (const V*)whi, (const V*)wlo, (Rl)(1.0 / (1 << LOGH)));
    else
        hipLaunchKernelGGL((r2c_rows_kernel<V, LOGH>), dim3((unsigned)blocks), dim3(BLOCK), 0, s, (const V*)in,
                           (V*)out, nrows, (const V*)tw, (const V*)whi, (const V*)wlo);
    return hipGetLastError();
}

hipError_t launch_real_rows(int prec, int logh, bool c2r, const void* in, void* out, int64_t nrows, const void* tw,
                            const void* whi, const void* wlo, hipStream_t s)
{
#define FFTMI_REAL_CASE(L) \
    case L: return prec == 0 ? launch_real_rows_t<float2, L>(c2r, in, out, nrows, tw, whi, wlo, s) \
                             : launch_real_rows_t<double2, L>(c2r, in, out, nrows, tw, whi, wlo, s);
    if (prec == 1 && logh > 13) return hipErrorInvalidValue;
    switch (logh) {
        FFTMI_REAL_CASE(0) FFTMI_REAL_CASE(1) FFTMI_REAL_CASE(2) FFTMI_REAL_CASE(3) FFTMI_REAL_CASE(4)
        FFTMI_REAL_CASE(5) FFTMI_REAL_CASE(6) FFTMI_REAL_CASE(7) FFTMI_REAL_CASE(8)
        FFTMI_REAL_CASE(9) FFTMI_REAL_CASE(10) FFTMI_REAL_CASE(11) FFTMI_REAL_CASE(12)
        FFTMI_REAL_CASE(13)
        case 14:  // one 1024-thread workgroup a row, 136 KiB of LDS
            if (prec == 0) return launch_real_rows_t<float2, 14>(c2r, in, out, nrows, tw, whi, wlo, s);
            return hipErrorInvalidValue;
        default: return hipErrorInvalidValue;
    }
#undef FFTMI_REAL_CASE
}

// ---------------------------------------------------------------------------
// R2C rows of [H'][2H] real images with the radix-F column super-stage folded
// in (the real counterpart of rows2d_fold_kernel): a group of F row-groups
// takes real rows j + r Lc (r < F) of one image, makes each row's half
// spectrum (the H-point transform and the even/odd split, as r2c_rows_kernel),
// exchanges through LDS so that every thread holds all F rows at E/F bins,
// does the F-point DFT across the rows and writes half-spectrum rows j F + r'
// ([H'][H + 1]); bin H of the F rows goes to thread 0 of the group.  The
// values the DFT reads are the split's, rounded to V in LDS as they were in
// memory when the column stage ran on its own.  Out of place.
// ---------------------------------------------------------------------------
template <typename V, int LOGH, int LOGF> constexpr int r2c_fold_groups()
{
    return (Geom<V, LOGH>::T << LOGF) >= 256 ? 1 : 256 / (Geom<V, LOGH>::T << LOGF);
}

template <typename V, int LOGH, int LOGF> constexpr bool r2c_fold_ok()
{
    using G = Geom<V, LOGH>;
    constexpr long threads = (long)(G::T << LOGF) * r2c_fold_groups<V, LOGH, LOGF>();
    constexpr long lds = (long)real_slots<LOGH>() * (1 << LOGF) * r2c_fold_groups<V, LOGH, LOGF>() * (long)sizeof(V);
    return LOGH >= 1 && G::E >= (1 << LOGF) && threads <= 1024 && lds <= 160 * 1024;
}

template <typename V, int LOGH, int LOGF>
__global__ __launch_bounds__(((Geom<V, LOGH>::T << LOGF) * r2c_fold_groups<V, LOGH, LOGF>()))
void r2c_fold_kernel(const V* in, V* out, int64_t ngroups, int log_lc, const V* __restrict__ tw,
                     const V* __restrict__ whi, const V* __restrict__ wlo)
{
    using G = Geom<V, LOGH>;
    constexpr int H = G::N, T = G::T, E = G::E, F = 1 << LOGF, EF = E / F;
    constexpr int GR = r2c_fold_groups<V, LOGH, LOGF>();
    constexpr int SLOTS = real_slots<LOGH>();
    __shared__ V lds[SLOTS * F * GR];
    const int tid = threadIdx.x;
    const int gl = tid / (F * T);
    const int rho = (tid / T) % F;
    const int t = tid % T;
    const int64_t grp = (int64_t)blockIdx.x * GR + gl;
    const bool live = grp < ngroups;
    const int64_t lc = (int64_t)1 << log_lc;
    const int64_t img = grp >> log_lc, j = grp & (lc - 1);
    const int64_t hh = lc << LOGF;  // rows per image
    V* my = lds + (gl * F) * SLOTS;
    const LdsLines<V, 1> L{my + rho * SLOTS, 0};

    TwBases<V, LOGH> tb;
    tb.load(tw, t);
    V v[E];
    const V* src = in + (img * hh + j + rho * lc) * H + t;
#pragma unroll
    for (int i = 0; i < E; ++i) v[i] = live ? ld_stream(src + i * T) : V{0, 0};
    fft_regs<LOGH>(v, t, tb, L);
    __syncthreads();  // the transform's last exchange is read by now
#pragma unroll
    for (int i = 0; i < E; ++i) *L.ptr(t + i * T) = v[i];
    __syncthreads();
    const V wh0 = chalf(wlo[t]);  // w_N^k / 2 = whi[i] (wlo[t] / 2), exact
    V y[E];
#pragma unroll
    for (int i = 0; i < E; ++i) {
        const V b = (i == 0 && t == 0) ? v[0] : partner<V, T, E>(L, t, i);
        y[i] = real_split(v[i], b, cmul(whi[i], wh0));
    }
    const V yh{v[0].x - v[0].y, 0};  // bin H, from Z_0 (thread 0)
    __syncthreads();  // every partner read is done
#pragma unroll
    for (int i = 0; i < E; ++i) *L.ptr(t + i * T) = y[i];
    if (t == 0) *L.ptr(H) = yh;
    __syncthreads();
    // Rows of H + 1 bins start anywhere in a 128-byte line, so most store
    // instructions begin and end in a line another one also writes: plain
    // stores let L2 merge those halves, nontemporal ones reached HBM as
    // partial lines (2048^2 x 8 real images: writes 142.6 -> 128.1 MiB, the
    // algorithmic bytes; 116.3 -> 108.9 us for rows and columns, same-box A/B;
    // staging the F rows in LDS and storing 128-byte-aligned windows: 110.4).
    V* dst = out + (img * hh + j * F) * (H + 1);
#pragma unroll
    for (int k = 0; k < EF; ++k) {
        const int p = t + (rho * EF + k) * T;
        V u[F];
#pragma unroll
        for (int r = 0; r < F; ++r) u[r] = *LdsLines<V, 1>{my + r * SLOTS, 0}.ptr(p);
        Dft<F>::run(u);
        if (live) {
#pragma unroll
            for (int r = 0; r < F; ++r) dst[r * (H + 1) + p] = u[r];
        }
    }
    if (rho == 0 && t == 0) {
        V u[F];
#pragma unroll
        for (int r = 0; r < F; ++r) u[r] = *LdsLines<V, 1>{my + r * SLOTS, 0}.ptr(H);
        Dft<F>::run(u);
        if (live) {
#pragma unroll
            for (int r = 0; r < F; ++r) dst[r * (H + 1) + H] = u[r];
        }
    }
}

template <typename V, int LOGH, int LOGF>
static hipError_t r2c_fold_t(const void* in, void* out, int64_t nimg, int log_lc, const void* tw, const void* whi,
                             const void* wlo, hipStream_t s)
{
    if constexpr (!r2c_fold_ok<V, LOGH, LOGF>()) {
        return hipErrorInvalidValue;
    } else {
        constexpr int GR = r2c_fold_groups<V, LOGH, LOGF>();
        const int64_t ngroups = nimg << log_lc;
        const int64_t blocks = (ngroups + GR - 1) / GR;
        if (blocks > 0x7fffffff) return hipErrorInvalidConfiguration;
        hipLaunchKernelGGL((r2c_fold_kernel<V, LOGH, LOGF>), dim3((unsigned)blocks),
                           dim3((Geom<V, LOGH>::T << LOGF) * GR), 0, s, (const V*)in, (V*)out, ngroups, log_lc,
                           (const V*)tw, (const V*)whi, (const V*)wlo);
        return hipGetLastError();
    }
}

template <typename V, int LOGH>
static hipError_t r2c_fold_f(int logf, const void* in, void* out, int64_t nimg, int log_lc, const void* tw,
                             const void* whi, const void* wlo, hipStream_t s)
{
    switch (logf) {
        case 1: return r2c_fold_t<V, LOGH, 1>(in, out, nimg, log_lc, tw, whi, wlo, s);
        case 2: return r2c_fold_t<V, LOGH, 2>(in, out, nimg, log_lc, tw, whi, wlo, s);
        case 3: return r2c_fold_t<V, LOGH, 3>(in, out, nimg, log_lc, tw, whi, wlo, s);
        case 4: return r2c_fold_t<V, LOGH, 4>(in, out, nimg, log_lc, tw, whi, wlo, s);
        default: return hipErrorInvalidValue;
    }
}

bool r2c_fold_supported(int prec, int logh, int logf)
{
#define FFTMI_FOLD_OK(V, L) \
    (logf == 1 ? r2c_fold_ok<V, L, 1>() : logf == 2 ? r2c_fold_ok<V, L, 2>() \
     : logf == 3 ? r2c_fold_ok<V, L, 3>() : logf == 4 ? r2c_fold_ok<V, L, 4>() : false)
#define FFTMI_FOLD_CASE(L) \
    case L: return prec == 0 ? FFTMI_FOLD_OK(float2, L) : FFTMI_FOLD_OK(double2, L);
    switch (logh) {
        FFTMI_FOLD_CASE(1) FFTMI_FOLD_CASE(2) FFTMI_FOLD_CASE(3) FFTMI_FOLD_CASE(4) FFTMI_FOLD_CASE(5)
        FFTMI_FOLD_CASE(6) FFTMI_FOLD_CASE(7) FFTMI_FOLD_CASE(8) FFTMI_FOLD_CASE(9) FFTMI_FOLD_CASE(10)
        FFTMI_FOLD_CASE(11) FFTMI_FOLD_CASE(12)
        default: return false;
    }
#undef FFTMI_FOLD_CASE
#undef FFTMI_FOLD_OK
}

hipError_t launch_r2c_fold(int prec, int logh, int logf, const void* in, void* out, int64_t nimg, int log_lc,
                           const void* tw, const void* whi, const void* wlo, hipStream_t s)
{
    if (!r2c_fold_supported(prec, logh, logf) || nimg < 1 || log_lc < 0) return hipErrorInvalidValue;
#define FFTMI_FOLD_CASE(L)                                                                      \
    case L:                                                                                     \
        return prec == 0 ? r2c_fold_f<float2, L>(logf, in, out, nimg, log_lc, tw, whi, wlo, s) \
                         : r2c_fold_f<double2, L>(logf, in, out, nimg, log_lc, tw, whi, wlo, s);
    switch (logh) {
        FFTMI_FOLD_CASE(1) FFTMI_FOLD_CASE(2) FFTMI_FOLD_CASE(3) FFTMI_FOLD_CASE(4) FFTMI_FOLD_CASE(5)
        FFTMI_FOLD_CASE(6) FFTMI_FOLD_CASE(7) FFTMI_FOLD_CASE(8) FFTMI_FOLD_CASE(9) FFTMI_FOLD_CASE(10)
        FFTMI_FOLD_CASE(11) FFTMI_FOLD_CASE(12)
        default: return hipErrorInvalidValue;
    }
#undef FFTMI_FOLD_CASE
}

template <typename V>
static hipError_t launch_real_pairs_t(bool c2r, const void* in, void* out, int64_t h, int64_t batch, BigTwiddle wn,
                                      hipStream_t s)
{
    const int64_t npair = h / 2 + 1;
    int64_t bx = (npair + 255) / 256;
    if (bx > (1 << 16)) bx = 1 << 16;
    const int64_t by = batch < 65535 ? batch : 65535;
    const BigTw<V> bt{(const V*)wn.hi, (const V*)wn.lo, wn.lbits, wn.logn};
    if (c2r)
        hipLaunchKernelGGL(c2r_pairs_kernel<V>, dim3((unsigned)bx, (unsigned)by), dim3(256), 0, s, (const V*)in,
                           (V*)out, h, batch, bt);
    else
        hipLaunchKernelGGL(r2c_pairs_kernel<V>, dim3((unsigned)bx, (unsigned)by), dim3(256), 0, s, (const V*)in,
                           (V*)out, h, batch, bt);
    return hipGetLastError();
}

hipError_t launch_real_pairs(int prec, bool c2r, const void* in, void* out, int64_t h, int64_t batch,
                             BigTwiddle wn, hipStream_t s)
{
    if (h < 1 || batch < 1) return hipErrorInvalidValue;
    return prec == 0 ? launch_real_pairs_t<float2>(c2r, in, out, h, batch, wn, s)
                     : launch_real_pairs_t<double2>(c2r, in, out, h, batch, wn, s);
}

hipError_t launch_real_n1(int prec, bool c2r, const void* in, void* out, int64_t batch, hipStream_t s)
{
    int64_t blocks = (batch + 255) / 256;
    if (blocks > (1 << 20)) blocks = 1 << 20;
    if (prec == 0)
        hipLaunchKernelGGL(real_n1_kernel<float2>, dim3((unsigned)blocks), dim3(256), 0, s, in, out, batch, (int)c2r);
    else
        hipLaunchKernelGGL(real_n1_kernel<double2>, dim3((unsigned)blocks), dim3(256), 0, s, in, out, batch, (int)c2r);
    return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Real rows of odd length N, around the N-point complex transform of the row
// itself (its route: mixed radix or chirp-z): the bin pairs of the even
// case need N/2 points, which an odd N has not.  Row r of a [rows][len]
// array is handled by blocks (x, r) for r < gridDim.y, (x, r + gridDim.y), ...
//   ODD_WIDEN   z[r][n] = (x[r][n], 0),                    n < N
//   ODD_TAKE    X[r][k] = z[r][k],                          k <= (N - 1) / 2
//   ODD_EXTEND  z[r][k] = X[r][k] (k <= (N - 1) / 2; X_0 with its imaginary
//               part dropped), conj X[r][N - k] beyond
//   ODD_REAL    x[r][n] = Re z[r][n]
// ---------------------------------------------------------------------------
enum { ODD_WIDEN = 0, ODD_TAKE = 1, ODD_EXTEND = 2, ODD_REAL = 3 };

template <typename V, int MODE>
__global__ __launch_bounds__(256) void real_odd_kernel(const void* __restrict__ in, void* __restrict__ out, int64_t n,
                                                       int64_t rows)
{
    using Rl = typename real_of<V>::type;
    const int64_t h1 = (n + 1) / 2;  // bins 0 .. (N - 1) / 2
    const int64_t len = MODE == ODD_TAKE ? h1 : n;  // elements written per row
    const int64_t j = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (j >= len) return;
    for (int64_t r = blockIdx.y; r < rows; r += gridDim.y) {
        if constexpr (MODE == ODD_WIDEN) {
            ((V*)out)[r * n + j] = V{((const Rl*)in)[r * n + j], (Rl)0};
        } else if constexpr (MODE == ODD_TAKE) {
            ((V*)out)[r * h1 + j] = ((const V*)in)[r * n + j];
        } else if constexpr (MODE == ODD_EXTEND) {
            const V* X = (const V*)in + r * h1;
            V z;
            if (j == 0) z = V{X[0].x, (Rl)0};
            else if (j < h1) z = X[j];
            else z = cconj(X[n - j]);
            ((V*)out)[r * n + j] = z;
        } else {
            ((Rl*)out)[r * n + j] = ((const V*)in)[r * n + j].x;
        }
    }
}

template <typename V>
static hipError_t launch_real_odd_t(int mode, const void* in, void* out, int64_t n, int64_t rows, hipStream_t s)
{
    const int64_t len = mode == ODD_TAKE ? (n + 1) / 2 : n;
    const int64_t bx = (len + 255) / 256;
    const int64_t by = rows < 65535 ? rows : 65535;
    if (bx > 0x7fffffff) return hipErrorInvalidConfiguration;
    if (bx == 0 || by == 0) return hipSuccess;
    const dim3 grid((unsigned)bx, (unsigned)by);
    switch (mode) {
        case ODD_WIDEN: hipLaunchKernelGGL((real_odd_kernel<V, ODD_WIDEN>), grid, dim3(256), 0, s, in, out, n, rows); break;
        case ODD_TAKE: hipLaunchKernelGGL((real_odd_kernel<V, ODD_TAKE>), grid, dim3(256), 0, s, in, out, n, rows); break;
        case ODD_EXTEND: hipLaunchKernelGGL((real_odd_kernel<V, ODD_EXTEND>), grid, dim3(256), 0, s, in, out, n, rows); break;
        case ODD_REAL: hipLaunchKernelGGL((real_odd_kernel<V, ODD_REAL>), grid, dim3(256), 0, s, in, out, n, rows); break;
        default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

hipError_t launch_real_odd(int prec, int mode, const void* in, void* out, int64_t n, int64_t rows, hipStream_t s)
{
    return prec == 0 ? launch_real_odd_t<float2>(mode, in, out, n, rows, s)
                     : launch_real_odd_t<double2>(mode, in, out, n, rows, s);
}

}  // namespace fftmi
