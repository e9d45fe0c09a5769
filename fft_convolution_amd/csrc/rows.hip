// rows.hip -- the LDS-resident row kernel: each workgroup transforms RPW
// contiguous rows of N = 2^LOGN points.  One coalesced global read of every
// row straight into registers, all log2 N butterfly levels fused into the
// radix stages of radix_plan.hpp with LDS exchanges between them, one
// coalesced global write ("Stockham FFT Butterfly Algorithm in Parallel
// GLSL", section "Performance and Pipeline Evaluation": stages batched in
// on-chip memory instead of one global round trip per stage).
#include "io.hpp"
#include "launch.hpp"
#include "stockham.hpp"

namespace fftmi {

// LDS layout of a row: one pad slot per 16 elements, per 32 for 8192-point
// complex64 rows, per 8 for complex128 rows.  Measured on MI355X
// (SQ_LDS_BANK_CONFLICT per wave, same-box A/B): complex64, one per 16 leaves
// 0 conflict cycles for rows of 256 - 2048 points, 64 at 4096 (no padding
// tried -- one per 8, 32, 64, or two levels 16 + 128 / 256 / 512, 32 + 128 /
// 256 / 512 -- went below 64, and none changed the time) and 192 at 8192,
// where one per 32 gives 0 and ran 2-3 % faster (209 against 214.7 us for
// 8192 rows); one per 32 costs 64 at 256 - 2048.  Complex128 (16-byte
// elements), one per 8: 0 / 64 / 96 cycles for rows of 64 / 256 - 512 /
// 1024 - 4096 points, against 96 / 128 / 160 with one per 16 (one per 4:
// 96 - 384, per 32: 192 - 256, per 64: 448 - 512), times equal within noise.
template <typename V, int LOGN> constexpr int row_pad_shift()
{
    return sizeof(V) == 8 ? (LOGN == 13 ? 5 : 4) : 3;
}
// A row's threads share a wavefront (rows of up to 1024 complex64 / 512
// complex128 points): the exchanges need no workgroup barrier (64 rows of
// 1024 points: 4.45 -> 4.22 us per call, same-box A/B).
template <typename V, int LOGN> constexpr bool row_in_wave() { return Geom<V, LOGN>::T <= 64; }
template <typename V, int LOGN> constexpr int row_lds_slots()
{
    return Geom<V, LOGN>::S > 1 ? lds_padded(Geom<V, LOGN>::N, row_pad_shift<V, LOGN>()) : 0;
}
template <typename V, int LOGN>
using RowLds = LdsLines<V, 1, row_pad_shift<V, LOGN>(), row_in_wave<V, LOGN>()>;

// One workgroup per group of RPW rows; the hardware dispatcher starts a new
// workgroup as soon as one retires, so the load, compute and store phases of
// the workgroups resident on a CU overlap.  (Measured on MI355X for 16384 rows
// of 4096 points: this beats a persistent grid with a one-row register
// prefetch, 174 us against 187-201 us per launch.)
template <typename V, int LOGN, bool CONJ_IN, bool CONJ_OUT, bool PIN, bool POUT>
__global__ __launch_bounds__((Geom<V, LOGN>::T * rows_per_wg<V, LOGN>()))
void rows_kernel(CIn<V, PIN> in, COut<V, POUT> out, int64_t nrows, const V* __restrict__ tw,
                 typename real_of<V>::type scale)
{
    using G = Geom<V, LOGN>;
    constexpr int RPW = rows_per_wg<V, LOGN>();
    constexpr int SLOTS = row_lds_slots<V, LOGN>();
    __shared__ V lds[SLOTS > 0 ? SLOTS * RPW : 1];

    const int tid = threadIdx.x;
    const int rloc = tid / G::T;
    const int t = tid % G::T;
    const int64_t row = (int64_t)blockIdx.x * RPW + rloc;
    const bool live = row < nrows;

    TwBases<V, LOGN> tb;
    tb.load(tw, t);

    V v[G::E];
    const int64_t base = row * G::N + t;
#pragma unroll
    for (int i = 0; i < G::E; ++i) {
        const V x = live ? in.ld(base + i * G::T) : V{0, 0};
        v[i] = CONJ_IN ? cconj(x) : x;
    }
    fft_regs<LOGN>(v, t, tb, RowLds<V, LOGN>{lds + rloc * SLOTS, 0});
    if (live) {
#pragma unroll
        for (int i = 0; i < G::E; ++i) {
            const V y = v[i];
            out.st(base + i * G::T, CONJ_OUT ? V{y.x * scale, -y.y * scale} : y);
        }
    }
}

template <typename V, int LOGN, bool CI, bool CO, bool PIN, bool POUT>
static hipError_t launch_rows_t(const Io& io, int64_t nrows, const void* tw, double scale, hipStream_t stream)
{
    constexpr int RPW = rows_per_wg<V, LOGN>();
    constexpr int BLOCK = Geom<V, LOGN>::T * RPW;
    const int64_t blocks = (nrows + RPW - 1) / RPW;
    if (blocks > 0x7fffffff) return hipErrorInvalidConfiguration;
    using Rl = typename real_of<V>::type;
    hipLaunchKernelGGL((rows_kernel<V, LOGN, CI, CO, PIN, POUT>), dim3((unsigned)blocks), dim3(BLOCK), 0, stream,
                       make_in<V, PIN>(io.in, io.in_im), make_out<V, POUT>(io.out, io.out_im), nrows,
                       (const V*)tw, (Rl)scale);
    return hipGetLastError();
}

// Interleaved in and out: every conjugation pattern.  Planar in and out: the
// 1D transform (conj on both sides or neither).  Planar in, interleaved out:
// the first pass of a multi-dimensional transform (no conj on the store).
template <typename V, int LOGN>
static hipError_t launch_rows_dir(bool ci, bool co, const Io& io, int64_t nrows, const void* tw, double scale,
                                  hipStream_t s)
{
    const bool pin = io.in_im != nullptr, pout = io.out_im != nullptr;
    if (!pin && !pout) {
        if (!ci && !co) return launch_rows_t<V, LOGN, false, false, false, false>(io, nrows, tw, scale, s);
        if (ci && co) return launch_rows_t<V, LOGN, true, true, false, false>(io, nrows, tw, scale, s);
        if (ci) return launch_rows_t<V, LOGN, true, false, false, false>(io, nrows, tw, scale, s);
        return launch_rows_t<V, LOGN, false, true, false, false>(io, nrows, tw, scale, s);
    }
    if (pin && pout && ci == co)
        return ci ? launch_rows_t<V, LOGN, true, true, true, true>(io, nrows, tw, scale, s)
                  : launch_rows_t<V, LOGN, false, false, true, true>(io, nrows, tw, scale, s);
    if (pin && !pout && !co)
        return ci ? launch_rows_t<V, LOGN, true, false, true, false>(io, nrows, tw, scale, s)
                  : launch_rows_t<V, LOGN, false, false, true, false>(io, nrows, tw, scale, s);
    return hipErrorInvalidValue;
}

hipError_t launch_rows(int prec, int logn, bool ci, bool co, const void* in, void* out, int64_t nrows,
                       const void* tw, double scale, hipStream_t s, const void* in_im, void* out_im)
{
    const Io io{in, in_im, out, out_im};
#define FFTMI_ROW_CASE(L) \
    case L: return prec == 0 ? launch_rows_dir<float2, L>(ci, co, io, nrows, tw, scale, s) \
                             : launch_rows_dir<double2, L>(ci, co, io, nrows, tw, scale, s);
    if (prec == 1 && logn > 13) return hipErrorInvalidValue;
    switch (logn) {
        FFTMI_ROW_CASE(1) FFTMI_ROW_CASE(2) FFTMI_ROW_CASE(3) FFTMI_ROW_CASE(4)
        FFTMI_ROW_CASE(5) FFTMI_ROW_CASE(6) FFTMI_ROW_CASE(7) FFTMI_ROW_CASE(8)
        FFTMI_ROW_CASE(9) FFTMI_ROW_CASE(10) FFTMI_ROW_CASE(11) FFTMI_ROW_CASE(12)
        case 13:  // complex128: one 1024-thread workgroup per row, 144 KiB of LDS
            return prec == 0 ? launch_rows_dir<float2, 13>(ci, co, io, nrows, tw, scale, s)
                             : launch_rows_dir<double2, 13>(ci, co, io, nrows, tw, scale, s);
        case 14:  // one 1024-thread workgroup per row, 136 KiB of LDS
            if (prec == 0) return launch_rows_dir<float2, 14>(ci, co, io, nrows, tw, scale, s);
            return hipErrorInvalidValue;
        default: return hipErrorInvalidValue;
    }
#undef FFTMI_ROW_CASE
}

}  // namespace fftmi
