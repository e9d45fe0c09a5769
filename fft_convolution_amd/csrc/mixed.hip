// mixed.hip -- rows whose length N = 2^a 3^b 5^c 7^d is not a power of two,
// up to the one-kernel range: the Stockham stages with radices 8, 4, 2, 3, 5
// and 7 ("FFT on GPU", section "Algorithm per signal Length", names mixed
// radix for such lengths, with 12 = 3 x 4 as its example).
//
// The stage is the one of radix_plan.hpp with a radix that varies from stage
// to stage: radix R, span Ns (the product of the earlier radices), for every
// butterfly j < N/R the inputs x[j + r N/R] times w_{Ns R}^{r (j mod Ns)}, an
// R-point DFT, and the outputs at y[(j / Ns) Ns R + (j mod Ns) + r Ns]; after
// the last stage the row is in natural order.
//
// Unlike the power-of-two engine (compile-time geometry), the schedule here is
// a runtime list: a group of TR >= N/8 threads owns a row held in LDS; each
// stage reads its butterflies into registers, and writes them back in place
// after a barrier.  The row crosses HBM once each way.  Twiddles come from a
// table of w_N^m (m < N) in the plan precision; the roots of unity of the odd
// radices are read from the same table (w_R^m = w_N^{m N / R}).
#include "io.hpp"
#include "launch.hpp"
#include "stockham.hpp"

namespace fftmi {

// Odd-radix DFT (R = 3, 5, 7) in registers, natural order in and out, by the
// pairing of x_n with x_{R-n}:
//   y_0 = x_0 + sum_n a_n,   y_k, y_{R-k} = x_0 + sum_n a_n c_{nk} -/+ i sum_n b_n s_{nk},
// a_n = x_n + x_{R-n}, b_n = x_n - x_{R-n}, c_m = cos(2 pi m / R), s_m = sin(2 pi m / R).
template <int R, typename V>
__device__ __forceinline__ void dft_odd(V (&u)[R], const typename real_of<V>::type (&c)[R], const typename real_of<V>::type (&sn)[R])
{
    using Rl = typename real_of<V>::type;
    constexpr int H = (R - 1) / 2;
    V a[H + 1], b[H + 1];
#pragma unroll
    for (int n = 1; n <= H; ++n) {
        a[n] = cadd(u[n], u[R - n]);
        b[n] = csub(u[n], u[R - n]);
    }
    V y[R];
    y[0] = u[0];
#pragma unroll
    for (int n = 1; n <= H; ++n) y[0] = cadd(y[0], a[n]);
#pragma unroll
    for (int k = 1; k <= H; ++k) {
        V A = u[0];
        V B{0, 0};
#pragma unroll
        for (int n = 1; n <= H; ++n) {
            const int m = (n * k) % R;  // c_m = c_{R-m}, s_{R-m} = -s_m
            const Rl cm = c[m];
            const Rl sm = sn[m];
            A = V{A.x + a[n].x * cm, A.y + a[n].y * cm};
            B = V{B.x + b[n].x * sm, B.y + b[n].y * sm};
        }
        // -i B = (B.y, -B.x)
        y[k] = V{A.x + B.y, A.y - B.x};
        y[R - k] = V{A.x - B.y, A.y + B.x};
    }
#pragma unroll
    for (int k = 0; k < R; ++k) u[k] = y[k];
}

// q = j / d and r = j mod d for 0 <= j < 2^15, 1 <= d < 2^15, from a float
// reciprocal (the quotient estimate is off by at most one) and an exact fix.
__device__ __forceinline__ void divmod_small(int j, int d, float inv_d, int& q, int& r)
{
    q = (int)((float)j * inv_d);
    r = j - q * d;
    if (r < 0) {
        --q;
        r += d;
    } else if (r >= d) {
        ++q;
        r -= d;
    }
}

// Butterflies per thread and stage: a row of N points has at least N/8
// threads, so a radix-R stage (N/R butterflies) gives each at most ceil(8/R).
template <int R> constexpr int mixed_bmax() { return (8 + R - 1) / R; }

// One stage of radix R on a row held in LDS (`row`), thread tl of tr.  All
// butterflies are read and computed into registers, then (after a barrier
// across the workgroup) written back in place.
template <int R, typename V>
__device__ __forceinline__ void mixed_stage(V* row, int n, int ns, int tl, int tr, const V* __restrict__ tw)
{
    using Rl = typename real_of<V>::type;
    constexpr int B = mixed_bmax<R>();
    const int stride = n / R;             // input spacing N/R
    const int tstep = n / (ns * R);       // w_{Ns R}^x = w_N^{x tstep}
    const float inv_ns = 1.0f / (float)ns;
    Rl c[R], sn[R];
    if constexpr (R == 3 || R == 5 || R == 7) {
#pragma unroll
        for (int m = 0; m < R; ++m) {
            const V w = tw[m * stride];   // w_R^m = cos - i sin
            c[m] = w.x;
            sn[m] = -w.y;
        }
    }
    V u[B][R];
    int dst[B];
#pragma unroll
    for (int b = 0; b < B; ++b) {
        const int j = tl + b * tr;
        dst[b] = -1;
        if (j < stride) {
            int g, k;
            divmod_small(j, ns, inv_ns, g, k);
#pragma unroll
            for (int r = 0; r < R; ++r) u[b][r] = row[j + r * stride];
            if (ns > 1) {
                // w^r = w_{Ns R}^{r k} as powers of one table value
                const V w = tw[k * tstep];
                V wr = w;
#pragma unroll
                for (int r = 1; r < R; ++r) {
                    u[b][r] = cmul(u[b][r], wr);
                    if (r + 1 < R) wr = cmul(wr, w);
                }
            }
            if constexpr (R == 3 || R == 5 || R == 7)
                dft_odd<R>(u[b], c, sn);
            else
                Dft<R>::run(u[b]);
            dst[b] = g * ns * R + k;
        }
    }
    __syncthreads();  // every read of this stage is done before any write
#pragma unroll
    for (int b = 0; b < B; ++b) {
        if (dst[b] >= 0) {
#pragma unroll
            for (int r = 0; r < R; ++r) row[dst[b] + r * ns] = u[b][r];
        }
    }
    __syncthreads();
}

// rpw rows per workgroup, tr threads per row (blockDim = rpw tr), rows
// contiguous in LDS as in memory (row rl at rl N), so the workgroup's rows are
// loaded and stored as one contiguous, coalesced segment.  CAP: LDS slots.
// Threads per workgroup at most: N/8 for the longest row of each precision.
template <typename V> constexpr int mixed_max_threads() { return sizeof(V) == 8 ? 1024 : 512; }

template <typename V, int CAP, bool PL>
__global__ __launch_bounds__(mixed_max_threads<V>()) void mixed_rows_kernel(CIn<V, PL> in, COut<V, PL> out, int64_t nrows, int n, int tr,
                                                          int rpw, MixedSchedule ms, const V* __restrict__ tw,
                                                          int conj_in, int conj_out, typename real_of<V>::type scale)
{
    __shared__ V lds[CAP];
    const int threads = tr * rpw;
    const int rl = threadIdx.x / tr, tl = threadIdx.x % tr;
    const int64_t row0 = (int64_t)blockIdx.x * rpw;
    const int rows = (int)(nrows - row0 < rpw ? nrows - row0 : rpw);
    const int count = rows * n;
    const int64_t base = row0 * n;
    for (int i = threadIdx.x; i < rpw * n; i += threads) {
        V x = i < count ? in.ld(base + i) : V{0, 0};
        lds[i] = conj_in ? cconj(x) : x;
    }
    __syncthreads();
    V* row = lds + rl * n;
    int ns = 1;
    for (int s = 0; s < ms.nst; ++s) {
        const int R = ms.radix[s];
        switch (R) {
            case 2: mixed_stage<2>(row, n, ns, tl, tr, tw); break;
            case 3: mixed_stage<3>(row, n, ns, tl, tr, tw); break;
            case 4: mixed_stage<4>(row, n, ns, tl, tr, tw); break;
            case 5: mixed_stage<5>(row, n, ns, tl, tr, tw); break;
            case 7: mixed_stage<7>(row, n, ns, tl, tr, tw); break;
            default: mixed_stage<8>(row, n, ns, tl, tr, tw); break;
        }
        ns *= R;
    }
    for (int i = threadIdx.x; i < count; i += threads) {
        const V y = lds[i];
        out.st(base + i, conj_out ? V{y.x * scale, -y.y * scale} : y);
    }
}

// LDS classes (slots): rows of up to 2048 points (several rows per workgroup
// for short ones), and one row of up to 8192 / 4096 points (64 KiB).
template <typename V> constexpr int mixed_cap_small() { return 2048; }
template <typename V> constexpr int mixed_cap_large() { return 8192 * 8 / (int)sizeof(V); }

template <typename V, bool PL>
static hipError_t mixed_t(const Io& io, int64_t nrows, int n, MixedSchedule ms, const void* tw, bool ci, bool co,
                          double scale, hipStream_t s)
{
    // threads per row: the power of two >= N/8 (so no thread has more than
    // ceil(8/R) butterflies in a stage), at most 1024; 256 threads or more
    // per workgroup
    int tr = 1;
    while (tr * 8 < n) tr *= 2;
    if (tr > mixed_max_threads<V>()) return hipErrorInvalidValue;
    const int rpw = tr >= 256 ? 1 : 256 / tr;
    const bool small = rpw * n <= mixed_cap_small<V>();
    if (!small && rpw * n > mixed_cap_large<V>()) return hipErrorInvalidValue;
    const int64_t blocks = (nrows + rpw - 1) / rpw;
    if (blocks > 0x7fffffff) return hipErrorInvalidConfiguration;
    using Rl = typename real_of<V>::type;
    const auto in = make_in<V, PL>(io.in, io.in_im);
    const auto out = make_out<V, PL>(io.out, io.out_im);
    if (small)
        hipLaunchKernelGGL((mixed_rows_kernel<V, mixed_cap_small<V>(), PL>), dim3((unsigned)blocks), dim3(tr * rpw), 0,
                           s, in, out, nrows, n, tr, rpw, ms, (const V*)tw, (int)ci, (int)co, (Rl)scale);
    else
        hipLaunchKernelGGL((mixed_rows_kernel<V, mixed_cap_large<V>(), PL>), dim3((unsigned)blocks), dim3(tr * rpw), 0,
                           s, in, out, nrows, n, tr, rpw, ms, (const V*)tw, (int)ci, (int)co, (Rl)scale);
    return hipGetLastError();
}

hipError_t launch_mixed_rows(int prec, int n, const MixedSchedule& ms, bool ci, bool co, const void* in, void* out,
                             int64_t nrows, const void* tw, double scale, hipStream_t s, const void* in_im,
                             void* out_im)
{
    const Io io{in, in_im, out, out_im};
    const bool pl = in_im != nullptr;
    if (pl != (out_im != nullptr)) return hipErrorInvalidValue;
    if (prec == 0) return pl ? mixed_t<float2, true>(io, nrows, n, ms, tw, ci, co, scale, s)
                             : mixed_t<float2, false>(io, nrows, n, ms, tw, ci, co, scale, s);
    return pl ? mixed_t<double2, true>(io, nrows, n, ms, tw, ci, co, scale, s)
              : mixed_t<double2, false>(io, nrows, n, ms, tw, ci, co, scale, s);
}

int mixed_max_n(int prec) { return prec == 0 ? mixed_cap_large<float2>() : mixed_cap_large<double2>(); }

}  // namespace fftmi
