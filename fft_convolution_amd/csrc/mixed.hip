// mixed.hip -- rows whose length N = 2^a 3^b 5^c 7^d 11^e 13^f is not a power of two,
// up to the one-kernel range: the Stockham stages with radices 8, 4, 2, 9, 3, 5,
// 7, 11 and 13 ("FFT on GPU", section "Algorithm per signal Length", names mixed
// radix for such lengths, with 12 = 3 x 4 as its example).
//
// The stage is the one of radix_plan.hpp with a radix that varies from stage
// to stage: radix R, span Ns (the product of the earlier radices), for every
// butterfly j < N/R the inputs x[j + r N/R] times w_{Ns R}^{r (j mod Ns)}, an
// R-point DFT, and the outputs at y[(j / Ns) Ns R + (j mod Ns) + r Ns]; after
// the last stage the row is in natural order.
//
// Unlike the power-of-two engine (compile-time geometry), the schedule here is
// a runtime list: a group of TR threads owns a row.  The first stage reads its
// butterflies from the input rows and writes the row into LDS; each later
// stage reads its butterflies from LDS into registers and writes them back in
// place after a barrier, except the last, which writes to the output rows.
// The row crosses HBM once each way.  Each stage s >= 1 reads
// its twiddles w_{Ns R}^{r k}, r = 1 .. R-1, as one row of a per-stage table
// (16-byte loads, no products of table values), and splits j into (j / Ns,
// j mod Ns) with a multiply-high by a precomputed reciprocal.
#include "io.hpp"
#include "launch.hpp"
#include "stockham.hpp"

namespace fftmi {

// cos(2 pi m / R) and sin(2 pi m / R), 0 <= m <= (R - 1) / 2, for R = 3, 5, 7,
// 9, 11, 13 (correctly rounded doubles; the float kernels round them once
// more).  m = 0 arises for R = 9, where n k = 9 in the DFT below.
__host__ __device__ constexpr double odd_cos(int r, int m)
{
    if (m == 0) return 1.0;
    switch (r * 16 + m) {
        case 3 * 16 + 1: return -0.5;
        case 5 * 16 + 1: return 0.3090169943749474241023;
        case 5 * 16 + 2: return -0.8090169943749474241023;
        case 7 * 16 + 1: return 0.6234898018587335305251;
        case 7 * 16 + 2: return -0.2225209339563144042890;
        case 7 * 16 + 3: return -0.9009688679024191262361;
        case 9 * 16 + 1: return 0.7660444431189780352024;
        case 9 * 16 + 2: return 0.1736481776669303488517;
        case 9 * 16 + 3: return -0.5;
        case 9 * 16 + 4: return -0.9396926207859083840541;
        case 11 * 16 + 1: return 0.8412535328311811688618;
        case 11 * 16 + 2: return 0.4154150130018864255293;
        case 11 * 16 + 3: return -0.1423148382732851404438;
        case 11 * 16 + 4: return -0.6548607339452850640569;
        case 11 * 16 + 5: return -0.9594929736144973898904;
        case 13 * 16 + 1: return 0.8854560256532098959004;
        case 13 * 16 + 2: return 0.5680647467311558025118;
        case 13 * 16 + 3: return 0.1205366802553230533491;
        case 13 * 16 + 4: return -0.3546048870425356259696;
        case 13 * 16 + 5: return -0.7485107481711010986346;
        case 13 * 16 + 6: return -0.9709418174260520271570;
        default: return 0.0;
    }
}
__host__ __device__ constexpr double odd_sin(int r, int m)
{
    if (m == 0) return 0.0;
    switch (r * 16 + m) {
        case 3 * 16 + 1: return 0.8660254037844386467637;
        case 5 * 16 + 1: return 0.9510565162951535721164;
        case 5 * 16 + 2: return 0.5877852522924731291687;
        case 7 * 16 + 1: return 0.7818314824680298087084;
        case 7 * 16 + 2: return 0.9749279121818236070181;
        case 7 * 16 + 3: return 0.4338837391175581204758;
        case 9 * 16 + 1: return 0.6427876096865393263226;
        case 9 * 16 + 2: return 0.9848077530122080593667;
        case 9 * 16 + 3: return 0.8660254037844386467637;
        case 9 * 16 + 4: return 0.3420201433256687330441;
        case 11 * 16 + 1: return 0.5406408174555975821076;
        case 11 * 16 + 2: return 0.9096319953545183714117;
        case 11 * 16 + 3: return 0.9898214418809327323761;
        case 11 * 16 + 4: return 0.7557495743542582837740;
        case 11 * 16 + 5: return 0.2817325568414296977114;
        case 13 * 16 + 1: return 0.4647231720437685456560;
        case 13 * 16 + 2: return 0.8229838658936563945796;
        case 13 * 16 + 3: return 0.9927088740980539928007;
        case 13 * 16 + 4: return 0.9350162426854148234398;
        case 13 * 16 + 5: return 0.6631226582407952023768;
        case 13 * 16 + 6: return 0.2393156642875577671488;
        default: return 0.0;
    }
}

// Odd-radix DFT (R = 3, 5, 7, 9, 11, 13) in registers, natural order in and out, by the
// pairing of x_n with x_{R-n}:
//   y_0 = x_0 + sum_n a_n,   y_k, y_{R-k} = x_0 + sum_n a_n c_{nk} -/+ i sum_n b_n s_{nk},
// a_n = x_n + x_{R-n}, b_n = x_n - x_{R-n}, c_m = cos(2 pi m / R), s_m = sin(2 pi m / R)
// (c_{R-m} = c_m, s_{R-m} = -s_m).
template <int R, typename V> __device__ __forceinline__ void dft_odd(V (&u)[R])
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
            const int m = (n * k) % R;
            const Rl cm = (Rl)odd_cos(R, m <= H ? m : R - m);
            const Rl sm = m <= H ? (Rl)odd_sin(R, m) : -(Rl)odd_sin(R, R - m);
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

template <int R, typename V> __device__ __forceinline__ void dft_any(V (&u)[R])
{
    if constexpr (R % 2 == 1)
        dft_odd<R>(u);
    else
        Dft<R>::run(u);
}

typedef float mx_f4 __attribute__((ext_vector_type(4)));

// The workgroup's segment [base, base + count) of the input into lds[0, count),
// conjugated for the inverse.  Interleaved complex64 segments that start on
// 16 bytes move two elements per streaming access.
template <bool INV, typename V, bool PL>
__device__ __forceinline__ void seg_load(const CIn<V, PL>& in, int64_t base, int count, V* lds, int threads)
{
    if constexpr (!PL && sizeof(V) == 8) {
        if ((base & 1) == 0) {
            const mx_f4* src = reinterpret_cast<const mx_f4*>(in.p + base);
            const int pairs = count >> 1;
            for (int i = threadIdx.x; i < pairs; i += threads) {
                const mx_f4 q = __builtin_nontemporal_load(at_bytes(src, (unsigned)i * 16u));
                lds[2 * i] = INV ? V{q.x, -q.y} : V{q.x, q.y};
                lds[2 * i + 1] = INV ? V{q.z, -q.w} : V{q.z, q.w};
            }
            if ((count & 1) && threadIdx.x == 0) {
                const V x = in.ld(base + count - 1);
                lds[count - 1] = INV ? cconj(x) : x;
            }
            return;
        }
    }
    for (int i = threadIdx.x; i < count; i += threads) {
        const V x = in.ld(base + i);
        lds[i] = INV ? cconj(x) : x;
    }
}

// lds[0, count) to the output segment [base, base + count); the inverse
// conjugates and scales.
template <bool INV, typename V, bool PL>
__device__ __forceinline__ void seg_store(const COut<V, PL>& out, int64_t base, int count, const V* lds, int threads,
                                          typename real_of<V>::type scale)
{
    if constexpr (!PL && sizeof(V) == 8) {
        if ((base & 1) == 0) {
            mx_f4* dst = reinterpret_cast<mx_f4*>(out.p + base);
            const int pairs = count >> 1;
            for (int i = threadIdx.x; i < pairs; i += threads) {
                const V a = lds[2 * i], b = lds[2 * i + 1];
                const mx_f4 q = INV ? mx_f4{a.x * scale, -a.y * scale, b.x * scale, -b.y * scale}
                                    : mx_f4{a.x, a.y, b.x, b.y};
                __builtin_nontemporal_store(q, at_bytes(dst, (unsigned)i * 16u));
            }
            if ((count & 1) && threadIdx.x == 0) {
                const V y = lds[count - 1];
                out.st(base + count - 1, INV ? V{y.x * scale, -y.y * scale} : y);
            }
            return;
        }
    }
    for (int i = threadIdx.x; i < count; i += threads) {
        const V y = lds[i];
        out.st(base + i, INV ? V{y.x * scale, -y.y * scale} : y);
    }
}

// Butterflies per thread and stage at most (about 8 elements a thread); the
// launcher gives a row enough threads for every stage of its schedule.
__host__ __device__ constexpr int mixed_bmax_of(int r, int bm = 8) { return (bm + r - 1) / r; }
template <int R, int BM = 8> constexpr int mixed_bmax() { return mixed_bmax_of(R, BM); }

// Where a stage reads and writes.  Rows of 64 threads or more (a wave within
// one row): the first stage reads its butterflies straight from the input rows
// (for each r the lanes' inputs j + r N/R are contiguous) and the last writes
// straight to the output rows (its butterflies j < N/R = Ns all have g = 0, so
// the outputs k + r Ns are contiguous too); a row of one stage (N = R) goes
// from input to output.  Shorter rows, where a wave spans several rows, are
// copied into LDS and back as contiguous 16-byte segments instead, and every
// stage works in LDS.
// The rows of one workgroup: input and output from its first element, the
// offset of this thread's row in them, whether that row exists (the last
// workgroup may have fewer), and the inverse's output scale.  load / store:
// the R elements j + r stride of the row (conjugated for the inverse), and
// the R outputs dst + r ns (conjugated and scaled for the inverse).
template <typename V, bool PL, bool INV> struct MixedRows {
    CIn<V, PL> in;
    COut<V, PL> out;
    unsigned rbase;
    bool live;
    typename real_of<V>::type scale;
    template <int R> __device__ __forceinline__ void load(int j, int stride, V (&u)[R]) const
    {
        if (!live) return;
#pragma unroll
        for (int r = 0; r < R; ++r) {
            const V x = in.ld32(rbase + (unsigned)(j + r * stride));
            u[r] = INV ? cconj(x) : x;
        }
    }
    template <int R> __device__ __forceinline__ void store(int dst, int ns, const V (&u)[R]) const
    {
        if (!live) return;
#pragma unroll
        for (int r = 0; r < R; ++r) {
            const V y = u[r];
            out.st32(rbase + (unsigned)(dst + r * ns), INV ? V{y.x * scale, -y.y * scale} : y);
        }
    }
};

// One stage of radix R, thread tl of tr: for every butterfly j < N/R, inputs
// x[j + r N/R], twiddles w_{Ns R}^{r k} from the table row k = j mod Ns (none
// in the first stage, Ns = 1), the R-point DFT, outputs at g Ns R + k + r Ns,
// g = j / Ns.  A stage within LDS reads all its butterflies into registers
// before a barrier across the workgroup and writes them back in place after
// it.  FROM_IN / TO_OUT: the stage reads its inputs through io.load, or
// writes its outputs through io.store, instead of the LDS row.  ES: LDS slots
// between consecutive elements of a row (1 for a row of its own; the tile
// width where rows are interleaved).
template <int R, bool FIRST, bool FROM_IN, bool TO_OUT, int ES = 1, int BM = 8, typename V, typename IO>
__device__ __forceinline__ void mixed_stage(V* row, int tl, int tr, int stride, int ns, unsigned magic,
                                            const V* __restrict__ tw, const IO& io)
{
    constexpr int B = mixed_bmax<R, BM>();
    constexpr int S = mixed_tw_slots(R);
    constexpr int P = 16 / (int)sizeof(V);           // table entries per 16-byte load
    constexpr int NL = ((R - 1 + P - 1) / P) * P;    // entries loaded per row (<= S)
    V u[B][R];
    int dst[B];
#pragma unroll
    for (int b = 0; b < B; ++b) {
        const int j = tl + b * tr;
        dst[b] = -1;
        if (j < stride) {
            if constexpr (FROM_IN) {
                io.template load<R>(j, stride, u[b]);
            } else {
#pragma unroll
                for (int r = 0; r < R; ++r) u[b][r] = row[(j + r * stride) * ES];
            }
            int g = j;
            if constexpr (!FIRST) {
                g = (int)__umulhi((unsigned)j, magic);
                const V* t = at_bytes(tw, (unsigned)((j - g * ns) * S * (int)sizeof(V)));
                V w[NL];
#pragma unroll
                for (int q = 0; q < NL; q += P) {
                    V d[P];
                    vload(t + q, d);
#pragma unroll
                    for (int e = 0; e < P; ++e) w[q + e] = d[e];
                }
#pragma unroll
                for (int r = 1; r < R; ++r) u[b][r] = cmul(u[b][r], w[r - 1]);
            }
            dft_any<R>(u[b]);
            dst[b] = j + g * (ns * (R - 1));  // g Ns R + k
        }
    }
    if constexpr (TO_OUT) {
#pragma unroll
        for (int b = 0; b < B; ++b)
            if (dst[b] >= 0) io.template store<R>(dst[b], ns, u[b]);
    } else {
        if constexpr (!FROM_IN) __syncthreads();  // every read of this stage is done before any write
#pragma unroll
        for (int b = 0; b < B; ++b) {
            if (dst[b] >= 0) {
#pragma unroll
                for (int r = 0; r < R; ++r) row[(dst[b] + r * ns) * ES] = u[b][r];
            }
        }
        __syncthreads();
    }
}

// WIDE: the schedule may hold radices 11 and 13, whose DFTs keep more values
// live; kernels for the other schedules are compiled without them so that
// they keep their lower register count.
template <bool WIDE, bool FIRST, bool FROM_IN, bool TO_OUT, int ES = 1, int BM = 8, typename V, typename IO>
__device__ __forceinline__ void mixed_stage_any(int r, V* row, int tl, int tr, int stride, int ns, unsigned magic,
                                                const V* __restrict__ tw, const IO& io)
{
#define MX_STAGE(R) mixed_stage<R, FIRST, FROM_IN, TO_OUT, ES, BM>(row, tl, tr, stride, ns, magic, tw, io)
    if constexpr (WIDE) {
        if (r == 11) {
            MX_STAGE(11);
            return;
        }
        if (r == 13) {
            MX_STAGE(13);
            return;
        }
    }
    switch (r) {
        case 2: MX_STAGE(2); break;
        case 3: MX_STAGE(3); break;
        case 4: MX_STAGE(4); break;
        case 5: MX_STAGE(5); break;
        case 7: MX_STAGE(7); break;
        case 9: MX_STAGE(9); break;
        default: MX_STAGE(8); break;
    }
#undef MX_STAGE
}

// rpw rows per workgroup, tr threads per row (blockDim = rpw tr), rows
// contiguous in LDS as in memory (row rl at rl N).  LDS: exactly the
// rpw N elements (dynamic, set at launch), so short and odd-sized rows do not
// hold LDS they do not use.  Threads per workgroup at most: N/8 for the
// longest row of each precision.
// INV: conjugate in, conjugate and scale out.
template <typename V> constexpr int mixed_max_threads() { return sizeof(V) == 8 ? 1024 : 512; }

template <typename V, bool PL, bool INV, bool DIRECT, bool WIDE>
__global__ __launch_bounds__(mixed_max_threads<V>()) void mixed_rows_kernel(CIn<V, PL> in, COut<V, PL> out,
                                                                            int64_t nrows, int n, int tr, int rpw,
                                                                            MixedSchedule ms,
                                                                            const V* __restrict__ tw,
                                                                            typename real_of<V>::type scale)
{
    extern __shared__ __align__(16) unsigned char mixed_lds[];
    V* lds = reinterpret_cast<V*>(mixed_lds);
    const int rl = threadIdx.x / tr, tl = threadIdx.x % tr;
    const int64_t row0 = (int64_t)blockIdx.x * rpw;
    const int64_t base = row0 * n;
    const MixedRows<V, PL, INV> io{in.at(base), out.at(base), (unsigned)(rl * n), row0 + rl < nrows, scale};
    V* row = lds + rl * n;
    const int last = ms.nst - 1;
    if constexpr (DIRECT) {
        if (last == 0) {
            mixed_stage_any<WIDE, true, true, true>(ms.radix[0], row, tl, tr, ms.stride[0], 1, 0u, tw, io);
            return;
        }
        mixed_stage_any<WIDE, true, true, false>(ms.radix[0], row, tl, tr, ms.stride[0], 1, 0u, tw, io);
        for (int s = 1; s < last; ++s)
            mixed_stage_any<WIDE, false, false, false>(ms.radix[s], row, tl, tr, ms.stride[s], ms.ns[s], ms.magic[s],
                                                      tw + ms.twoff[s], io);
        mixed_stage_any<WIDE, false, false, true>(ms.radix[last], row, tl, tr, ms.stride[last], ms.ns[last],
                                                 ms.magic[last], tw + ms.twoff[last], io);
    } else {
        // rows past the end of the batch (last workgroup only) are computed
        // on whatever LDS holds and never stored
        const int threads = tr * rpw;
        const int rows = (int)(nrows - row0 < rpw ? nrows - row0 : rpw);
        seg_load<INV>(in, base, rows * n, lds, threads);
        __syncthreads();
        mixed_stage_any<WIDE, true, false, false>(ms.radix[0], row, tl, tr, ms.stride[0], 1, 0u, tw, io);
        for (int s = 1; s <= last; ++s)
            mixed_stage_any<WIDE, false, false, false>(ms.radix[s], row, tl, tr, ms.stride[s], ms.ns[s],
                                                        ms.magic[s], tw + ms.twoff[s], io);
        seg_store<INV>(out, base, rows * n, lds, threads, scale);
    }
}

// Longest row: 64 KiB of LDS (8192 complex64 / 4096 complex128 points).
template <typename V> constexpr int mixed_max_points() { return 65536 / (int)sizeof(V); }

template <typename V, bool PL, bool INV>
static hipError_t mixed_t(const Io& io, int64_t nrows, int n, const MixedSchedule& ms, const void* tw, double scale,
                          hipStream_t s)
{
    // threads per row: the least power of two that covers every stage's N/R
    // butterflies at mixed_bmax(R) each; 256 threads or more per workgroup
    int tr = 1;
    for (int q = 0; q < ms.nst; ++q)
        while ((int64_t)tr * mixed_bmax_of(ms.radix[q]) < n / ms.radix[q]) tr *= 2;
    if (tr > mixed_max_threads<V>()) return hipErrorInvalidValue;
    const int rpw = tr >= 256 ? 1 : 256 / tr;
    const int64_t lds_bytes = (int64_t)rpw * n * (int64_t)sizeof(V);
    if (lds_bytes > 65536) return hipErrorInvalidValue;
    const int64_t blocks = (nrows + rpw - 1) / rpw;
    if (blocks > 0x7fffffff) return hipErrorInvalidConfiguration;
    using Rl = typename real_of<V>::type;
    const auto in = make_in<V, PL>(io.in, io.in_im);
    const auto out = make_out<V, PL>(io.out, io.out_im);
    bool wide = false;
    for (int q = 0; q < ms.nst; ++q) wide = wide || ms.radix[q] > 9;
    const dim3 grid((unsigned)blocks), block(tr * rpw);
#define MX_LAUNCH(D, W)                                                                                        \
    hipLaunchKernelGGL((mixed_rows_kernel<V, PL, INV, D, W>), grid, block, (unsigned)lds_bytes, s, in, out, nrows, n, \
                       tr, rpw, ms, (const V*)tw, (Rl)scale)
    if (tr >= 64) {
        if (wide) MX_LAUNCH(true, true);
        else MX_LAUNCH(true, false);
    } else {
        if (wide) MX_LAUNCH(false, true);
        else MX_LAUNCH(false, false);
    }
#undef MX_LAUNCH
    return hipGetLastError();
}

template <typename V, bool PL>
static hipError_t mixed_dir(const Io& io, int64_t nrows, int n, const MixedSchedule& ms, bool inv, const void* tw,
                            double scale, hipStream_t s)
{
    return inv ? mixed_t<V, PL, true>(io, nrows, n, ms, tw, scale, s)
               : mixed_t<V, PL, false>(io, nrows, n, ms, tw, scale, s);
}

hipError_t launch_mixed_rows(int prec, int n, const MixedSchedule& ms, bool inverse, const void* in, void* out,
                             int64_t nrows, const void* tw, double scale, hipStream_t s, const void* in_im,
                             void* out_im)
{
    const Io io{in, in_im, out, out_im};
    const bool pl = in_im != nullptr;
    if (pl != (out_im != nullptr)) return hipErrorInvalidValue;
    if (prec == 0) return pl ? mixed_dir<float2, true>(io, nrows, n, ms, inverse, tw, scale, s)
                             : mixed_dir<float2, false>(io, nrows, n, ms, inverse, tw, scale, s);
    return pl ? mixed_dir<double2, true>(io, nrows, n, ms, inverse, tw, scale, s)
              : mixed_dir<double2, false>(io, nrows, n, ms, inverse, tw, scale, s);
}

int mixed_max_n(int prec) { return prec == 0 ? mixed_max_points<float2>() : mixed_max_points<double2>(); }

// ---------------------------------------------------------------------------
// Rows beyond one workgroup: N = R_0 R_1 ... as Stockham super-stages, one
// pass each (radix R <= 1024, span Ns = R_0 ... R_{p-1}): for every butterfly
// j < N/R, inputs x[j + q N/R] times w_{Ns R}^{q k} (k = j mod Ns), the
// R-point DFT (the mixed-radix stages above, on a line of the tile), outputs at
// g Ns R + k + q Ns (g = j / Ns).
//
// A workgroup takes LINES consecutive butterflies j (a 128-, 256- or 512-byte
// segment of elements for each q, by radix); element q of line c lives in LDS at q (LINES + 1) + c
// (the extra slot per element row keeps both store orders free of bank
// conflicts).  The first stage of the R-point transform reads its inputs from
// HBM; the first pass (Ns = 1) writes each line's outputs j R + q, so the
// tile's lines together are one contiguous block, stored from LDS; later
// passes write the last stage's outputs straight to HBM (for each q, the
// lines' outputs side by side).
// ---------------------------------------------------------------------------

// w_M^m for any M (m < M < 2^31) from two tables: hi[q] = w_M^{q 2^lbits},
// lo[q] = w_M^q.
template <typename V> struct AnyTw {
    const V* __restrict__ hi;
    const V* __restrict__ lo;
    int lbits;
    __device__ __forceinline__ V operator()(int m) const
    {
        return cmul(hi[m >> lbits], lo[m & ((1 << lbits) - 1)]);
    }
};

// The global side of a pass's line: input element q at ibase + q istride,
// times w^{q k} when twiddled (conjugated first for the inverse's first
// pass); output element q at obase + q ostride (conjugated and scaled for the
// inverse's last pass).  TW: the twiddles are on (a compile-time switch, so
// that each stage's code is built with or without them).  load: the R elements j + r stride of a butterfly,
// the twiddles as w^{k j} times powers of w^{k stride} (R - 1 products,
// exponents below Ns R).
template <typename V, typename IN, typename OUT, bool TW> struct PassIO {
    IN in;
    OUT out;
    int64_t ibase;
    int istride;
    int64_t obase;
    int ostride;
    AnyTw<V> big;
    int k;
    bool conj_in, conj_out, live;
    typename real_of<V>::type scale;
    template <int R> __device__ __forceinline__ void load(int j, int stride, V (&u)[R]) const
    {
        if (!live) return;
        V w{1, 0}, step{1, 0};
        if constexpr (TW) {
            w = big(k * j);
            step = big(k * stride);
        }
#pragma unroll
        for (int r = 0; r < R; ++r) {
            V x = in.ld(ibase + (int64_t)(j + r * stride) * istride);
            if (conj_in) x = cconj(x);
            if constexpr (TW) {
                x = cmul(x, w);
                if (r + 1 < R) w = cmul(w, step);
            }
            u[r] = x;
        }
    }
    template <int R> __device__ __forceinline__ void store(int dst, int ns, const V (&u)[R]) const
    {
        if (!live) return;
#pragma unroll
        for (int r = 0; r < R; ++r) {
            const V y = u[r];
            out.st(obase + (int64_t)(dst + r * ns) * ostride, conj_out ? V{y.x * scale, -y.y * scale} : y);
        }
    }
};

template <typename V> constexpr int mp_lines() { return 128 / (int)sizeof(V); }

// Elements of a line per thread at most: the sub-schedule gives a line R / tr
// <= 14 elements per thread (tr covers every stage at <= ceil(8/r) butterflies
// of radix r); the block store of the first pass moves as many per thread
// (LINES R over a workgroup of LINES tr threads), MP_CHUNK at a time.
constexpr int MP_QMAX = 16;
constexpr int MP_CHUNK = 8;
// Tile widths: 512 bytes of elements per q up to radix MP_R4, 256 bytes up to
// MP_R2, 128 bytes beyond (LDS (lines + 1) r elements: sized at launch up to
// MP_R2, static classes of radix 512 and MP_RMAX beyond).  Threads per line:
// up to 64, with up to twice the butterflies per thread in the widest class,
// which takes no radix-11 or -13 stage (their registers would spill).
constexpr int MP_R4 = 64;
constexpr int MP_R2 = 256;
constexpr int MP_RMAX = 1024;

template <typename V, int LN, bool WIDE, int RCAP, typename IN, typename OUT>
__global__ __launch_bounds__(LN * 64 < 1024 ? LN * 64 : 1024) void mixed_pass_kernel(IN in, OUT out, MixedPassArgs a, MixedSchedule ms,
                                                          const V* __restrict__ tw, AnyTw<V> big,
                                                          typename real_of<V>::type scale)
{
    constexpr int LINES = LN;
    constexpr int P = LINES + 1;
    // RCAP 0: LDS sized at launch to the radix (short lines leave room for
    // many workgroups per CU); otherwise a static class
    __shared__ V lds_static[RCAP > 0 ? P * RCAP : 1];
    extern __shared__ __align__(16) unsigned char mp_lds_dyn[];
    V* const lds = RCAP > 0 ? lds_static : reinterpret_cast<V*>(mp_lds_dyn);
    const int c = threadIdx.x % LINES, tl = threadIdx.x / LINES;
    // Where the element rows of a tile (N/R elements apart) are not a whole
    // number of 128-byte lines apart, a tile's segments straddle lines that
    // the neighbouring tile reads too: each XCD then takes a contiguous range
    // of tiles, so that both go through the same L2.  Otherwise launch order
    // (measured faster there).
    const bool straddle = ((a.stride * (int)sizeof(V)) & 127) != 0;
    const int64_t tile = straddle ? xcd_tile(blockIdx.x, gridDim.x) : (int64_t)blockIdx.x;
    const int64_t sig = tile / a.tiles;
    const int j0 = (int)(tile - sig * a.tiles) * LINES;
    const int j = j0 + c;
    const bool live = j < a.stride;
    const int g = j / a.ns, k = j - g * a.ns;
    const int64_t sbase = sig * (int64_t)a.n;
    // The first stage of the line's transform reads its butterflies straight
    // from the input (element q of line j at j + q N/R, times w^{q k}); for
    // Ns > 1 the last writes straight to the output (element q at
    // g Ns R + k + q Ns); the stages between go through LDS.
    V* row = lds + c;
    const int last = ms.nst - 1;
    constexpr int BM = RCAP > 512 ? 16 : 8;  // butterfly budget per thread and stage (x R elements)
    auto stages = [&](const auto& io) {
        if (a.ns > 1) {
            if (last == 0) {
                mixed_stage_any<WIDE, true, true, true, P, BM>(ms.radix[0], row, tl, a.tr, ms.stride[0], 1, 0u, tw, io);
                return;
            }
            mixed_stage_any<WIDE, true, true, false, P, BM>(ms.radix[0], row, tl, a.tr, ms.stride[0], 1, 0u, tw, io);
            for (int s = 1; s < last; ++s)
                mixed_stage_any<WIDE, false, false, false, P, BM>(ms.radix[s], row, tl, a.tr, ms.stride[s], ms.ns[s],
                                                              ms.magic[s], tw + ms.twoff[s], io);
            mixed_stage_any<WIDE, false, false, true, P, BM>(ms.radix[last], row, tl, a.tr, ms.stride[last],
                                                         ms.ns[last], ms.magic[last], tw + ms.twoff[last], io);
            return;
        }
        mixed_stage_any<WIDE, true, true, false, P, BM>(ms.radix[0], row, tl, a.tr, ms.stride[0], 1, 0u, tw, io);
        for (int s = 1; s <= last; ++s)
            mixed_stage_any<WIDE, false, false, false, P, BM>(ms.radix[s], row, tl, a.tr, ms.stride[s], ms.ns[s],
                                                          ms.magic[s], tw + ms.twoff[s], io);
    };
    const int64_t ibase = sbase + j, obase_l = sbase + (int64_t)g * a.ns * a.r + k;
    if (a.twiddle) {
        const PassIO<V, IN, OUT, true> io{in, out, ibase, a.stride, obase_l, a.ns, big, a.tdiv == 1 ? k : k / a.tdiv,
                                          a.conj_in != 0, a.conj_out != 0, live, scale};
        stages(io);
    } else {
        const PassIO<V, IN, OUT, false> io{in, out, ibase, a.stride, obase_l, a.ns, big, 0,
                                           a.conj_in != 0, a.conj_out != 0, live, scale};
        stages(io);
    }
    if (a.ns > 1) return;
    // Ns = 1: line j's outputs are j R + q, so the tile's lines are one
    // contiguous block: element e = tid + i blockDim of it, in chunks
    const int lines = a.stride - j0 < LINES ? a.stride - j0 : LINES;
    const int count = lines * a.r;
    const int64_t obase = sbase + (int64_t)j0 * a.r;
    for (int e0 = threadIdx.x; e0 < count; e0 += MP_CHUNK * blockDim.x) {
        V y[MP_CHUNK];
#pragma unroll
        for (int i = 0; i < MP_CHUNK; ++i) {
            const int e = e0 + i * blockDim.x;
            if (e < count) {
                const int cl = (int)__umulhi((unsigned)e, a.rmagic);
                y[i] = lds[(e - cl * a.r) * P + cl];
            }
        }
#pragma unroll
        for (int i = 0; i < MP_CHUNK; ++i) {
            const int e = e0 + i * blockDim.x;
            if (e < count) out.st(obase + e, a.conj_out ? V{y[i].x * scale, -y[i].y * scale} : y[i]);
        }
    }
}

// One launch of a pass: the tile width (and LDS sizing) class of its radix.
template <typename V, bool WIDE, typename IN, typename OUT>
static hipError_t mixed_pass_t(IN in, OUT out, int64_t batch, const MixedPassArgs& a, const MixedSchedule& ms,
                               const void* tw, const BigTwiddle& bt, double scale, hipStream_t s)
{
    using Rl = typename real_of<V>::type;
    const int64_t blocks = (int64_t)a.tiles * batch;
    if (blocks > 0x7fffffff) return hipErrorInvalidConfiguration;
    const AnyTw<V> big{(const V*)bt.hi, (const V*)bt.lo, bt.lbits};
    constexpr int L1 = mp_lines<V>(), L2 = 2 * L1, L4 = 4 * L1;
    const dim3 grid((unsigned)blocks);
    if (a.r <= MP_R4)
        hipLaunchKernelGGL((mixed_pass_kernel<V, L4, WIDE, 0, IN, OUT>), grid, dim3(L4 * a.tr),
                           (unsigned)((L4 + 1) * a.r * (int)sizeof(V)), s, in, out, a, ms, (const V*)tw, big,
                           (Rl)scale);
    else if (a.r <= MP_R2)
        hipLaunchKernelGGL((mixed_pass_kernel<V, L2, WIDE, 0, IN, OUT>), grid, dim3(L2 * a.tr),
                           (unsigned)((L2 + 1) * a.r * (int)sizeof(V)), s, in, out, a, ms, (const V*)tw, big,
                           (Rl)scale);
    else if (a.r <= 512)
        hipLaunchKernelGGL((mixed_pass_kernel<V, L1, WIDE, 512, IN, OUT>), grid, dim3(L1 * a.tr), 0, s, in, out, a,
                           ms, (const V*)tw, big, (Rl)scale);
    else if constexpr (!WIDE)
        hipLaunchKernelGGL((mixed_pass_kernel<V, L1, false, MP_RMAX, IN, OUT>), grid, dim3(L1 * a.tr), 0, s, in,
                           out, a, ms, (const V*)tw, big, (Rl)scale);
    else
        return hipErrorInvalidValue;  // radices 11, 13 stay within 512 (the launcher checks)
    return hipGetLastError();
}

template <typename V, typename IN, typename OUT>
static hipError_t mixed_pass_w(IN in, OUT out, int64_t batch, const MixedPassArgs& a, const MixedSchedule& ms,
                               const void* tw, const BigTwiddle& bt, double scale, hipStream_t s)
{
    bool wide = false;
    for (int q = 0; q < ms.nst; ++q) wide = wide || ms.radix[q] > 9;
    return wide ? mixed_pass_t<V, true>(in, out, batch, a, ms, tw, bt, scale, s)
                : mixed_pass_t<V, false>(in, out, batch, a, ms, tw, bt, scale, s);
}

template <typename V>
static hipError_t mixed_pass_v(const Io& io, int64_t batch, const MixedPassArgs& a, const MixedSchedule& ms,
                               const void* tw, const BigTwiddle& bt, double scale, hipStream_t s)
{
    if (io.in_im && io.out_im)
        return mixed_pass_w<V>(make_in<V, true>(io.in, io.in_im), make_out<V, true>(io.out, io.out_im), batch, a, ms,
                               tw, bt, scale, s);
    if (io.in_im) return mixed_pass_w<V>(make_in<V, true>(io.in, io.in_im), make_out<V, false>(io.out, nullptr), batch,
                                         a, ms, tw, bt, scale, s);
    if (io.out_im) return mixed_pass_w<V>(make_in<V, false>(io.in, nullptr), make_out<V, true>(io.out, io.out_im),
                                          batch, a, ms, tw, bt, scale, s);
    return mixed_pass_w<V>(make_in<V, false>(io.in, nullptr), make_out<V, false>(io.out, nullptr), batch, a, ms, tw,
                           bt, scale, s);
}

int mixed_pass_threads(const MixedSchedule& ms, int r)
{
    int tr = 1;
    for (int q = 0; q < ms.nst; ++q)
        while ((int64_t)tr * mixed_bmax_of(ms.radix[q], r > 512 ? 16 : 8) < r / ms.radix[q]) tr *= 2;
    while (tr * MP_QMAX < r) tr *= 2;
    return tr;
}

int mixed_pass_lines(int prec, int r)
{
    const int base = prec == 0 ? mp_lines<float2>() : mp_lines<double2>();
    return r <= MP_R4 ? 4 * base : r <= MP_R2 ? 2 * base : base;
}

hipError_t launch_mixed_pass(int prec, const MixedPassArgs& a, const MixedSchedule& ms, const void* in, void* out,
                             int64_t batch, const void* tw, const BigTwiddle& big, double scale, hipStream_t s,
                             const void* in_im, void* out_im)
{
    bool wide_radix = false;  // an 11- or 13-point stage
    for (int q = 0; q < ms.nst; ++q) wide_radix |= ms.radix[q] == 11 || ms.radix[q] == 13;
    if (a.r > MP_RMAX || (a.r > 512 && wide_radix) || a.r < 2 || a.tr < mixed_pass_threads(ms, a.r) || a.tr > 64 ||
        (a.r + a.tr - 1) / a.tr > MP_QMAX ||
        a.ns < 1 || a.tdiv < 1 || a.ns % a.tdiv || (int64_t)a.stride * a.r != a.n ||
        a.tiles * (int64_t)mixed_pass_lines(prec, a.r) < a.stride || a.tr * mixed_pass_lines(prec, a.r) > 1024 ||
        a.rmagic != (unsigned)(((uint64_t(1) << 32) + a.r - 1) / a.r))
        return hipErrorInvalidValue;
    const Io io{in, in_im, out, out_im};
    return prec == 0 ? mixed_pass_v<float2>(io, batch, a, ms, tw, big, scale, s)
                     : mixed_pass_v<double2>(io, batch, a, ms, tw, big, scale, s);
}

}  // namespace fftmi
