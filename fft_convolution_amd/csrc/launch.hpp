// launch.hpp -- host-side entry points of the kernels (internal to the
// library; the public C ABI is include/fftmi.h).
//
// Every launcher enqueues on `stream`, returns the launch's hipError_t and
// never synchronises.  prec: 0 = complex64, 1 = complex128.  The caller (the
// C-ABI layer) has validated every size and pointer already.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fftmi {

// Two-level table for w_N^m with large N: w_N^m = hi[m >> lbits] * lo[m & (2^lbits - 1)],
// hi[q] = w_N^{q 2^lbits}, lo[q] = w_N^q.
struct BigTwiddle {
    const void* hi;
    const void* lo;
    int lbits;
    int logn;
};

// Stages of a mixed-radix row of N points: radix R_s (each 2, 3, 4, 5, 7, 8,
// 9, 11 or 13; product N), span ns_s = R_0 ... R_{s-1}, stride N / R_s, magic_s =
// ceil(2^32 / ns_s) (so j / ns_s = mulhi(j, magic_s) for j ns_s < 2^32), and
// twoff_s: where stage s >= 1 starts in the twiddle table, which holds, for
// every k < ns_s, the row w_{ns_s R_s}^{r k}, r = 1 .. R_s - 1, padded to
// mixed_tw_slots(R_s) entries (stage 0 has none: its twiddles are all 1).
constexpr int kMixedMaxStages = 16;
struct MixedSchedule {
    int nst;
    int radix[kMixedMaxStages];
    int ns[kMixedMaxStages];
    int stride[kMixedMaxStages];
    unsigned magic[kMixedMaxStages];
    int twoff[kMixedMaxStages];
};
constexpr int mixed_tw_slots(int r) { return r & ~1; }

// Mixed-radix rows (mixed.hip): `nrows` contiguous rows of n points,
// n <= mixed_max_n(prec); tw = the schedule's twiddle table.  Inverse:
// conjugate in, conjugate and scale out.  Planar needs both in_im and out_im.
// in -> out, may alias.
hipError_t launch_mixed_rows(int prec, int n, const MixedSchedule& ms, bool inverse, const void* in, void* out,
                             int64_t nrows, const void* tw, double scale, hipStream_t stream,
                             const void* in_im = nullptr, void* out_im = nullptr);
int mixed_max_n(int prec);

// One mixed-radix super-stage pass (mixed.hip) over `batch` signals of n
// points: radix r (<= 1024, above 512 without a radix-11 or -13 stage; its
// stage schedule `ms`, twiddle table `tw` of
// that schedule), span ns, stride n / r, tiles = ceil(stride / lines) per
// signal (lines = mixed_pass_lines(prec, r)), tr threads per line
// (mixed_pass_threads), rmagic = ceil(2^32 / r).
// Twiddles (twiddle != 0): w_M^{q (k / tdiv)} from `big`, k = j mod ns, M =
// r ns / tdiv; tdiv = 1 for a 1D transform, the axis stride for a pass of
// one axis of an image or volume (ns = tdiv ns_axis: the pass runs the
// axis's own super-stage on every column).  conj_in / conj_out + scale: the
// inverse's first / last pass.  Planar: in_im on a first pass, out_im on a
// last pass (both on a pass that is both).  in -> out; in place only for the
// last pass (ns r = n).
struct MixedPassArgs {
    int n, r, ns, stride, tiles, tr;
    unsigned rmagic;
    int conj_in, conj_out;
    int tdiv, twiddle;
};
int mixed_pass_threads(const MixedSchedule& ms, int r);
int mixed_pass_lines(int prec, int r);  // butterflies per tile of a radix-r pass
hipError_t launch_mixed_pass(int prec, const MixedPassArgs& a, const MixedSchedule& ms, const void* in, void* out,
                             int64_t batch, const void* tw, const BigTwiddle& big, double scale, hipStream_t stream,
                             const void* in_im = nullptr, void* out_im = nullptr);

// nmat matrices [rows][cols] -> [cols][rows] (tiles.hip); in_im / out_im
// non-NULL: that side planar.  in and out must not alias.
hipError_t launch_transpose(int prec, const void* in, const void* in_im, void* out, void* out_im, int64_t rows,
                            int64_t cols, int64_t nmat, hipStream_t stream);

// Lines per workgroup of the tile passes (tiles.hip) for lines of 2^logl points.
int tile_lines_2d(int prec, int logl);

// Whether the folded 2D row pass exists for rows of 2^logw points and fold 2^logf.
bool fold_supported(int prec, int logw, int logf);

// The arrays of a launch: `in` / `out` are interleaved complex arrays, or,
// with in_im / out_im non-NULL, the real-part planes of planar arrays whose
// imaginary parts are at in_im / out_im (same indexing, one real per element).
struct Io {
    const void* in;
    const void* in_im;
    void* out;
    void* out_im;
};

// Rows kernel: `nrows` contiguous rows of 2^logn points, in -> out (may alias).
// conj_in conjugates on load; conj_out conjugates and multiplies by `scale` on store.
// Planar in and out need conj_in == conj_out; planar in with interleaved out
// needs conj_out false.
hipError_t launch_rows(int prec, int logn, bool conj_in, bool conj_out, const void* in, void* out,
                       int64_t nrows, const void* tw, double scale, hipStream_t stream,
                       const void* in_im = nullptr, void* out_im = nullptr);

// 2D column pass over `nimg` images [H][w], H = 2^(logf + logl): lines are
// (column, j'), j' < 2^logf, with points at rows j' + 2^logf r; when logf > 0
// point r of line j' is first multiplied by w_H^{r j'} (htw: tables for H).
// in -> out, may alias.  conj_out conjugates and multiplies by `scale`.
// out_im non-NULL: planar output (see Io).  one_col: one column per lane, for
// rows of any length w (the W/2 + 1 columns of a real image's spectrum);
// conj_in (one_col only) conjugates on load.
hipError_t launch_cols2d(int prec, int logl, const void* in, void* out, int64_t nimg, int64_t w, int logf,
                         const void* tw, BigTwiddle htw, bool conj_out, double scale, hipStream_t stream,
                         void* out_im = nullptr, bool one_col = false, bool conj_in = false);

// 2D row pass with the radix-2^logf column super-stage folded in: rows of
// 2^logw points; image rows j + r Lc (r < 2^logf, Lc = 2^log_lc) are
// transformed and combined into rows j 2^logf + r.  in -> out, must not alias.
// in_im non-NULL: planar input (see Io).
hipError_t launch_rows2d_fold(int prec, int logw, int logf, const void* in, void* out, int64_t nimg, int log_lc,
                              const void* tw, bool conj_in, hipStream_t stream, const void* in_im = nullptr);

// 2D column super-stage of radix 2^logf (1..4) as a pass of its own: image
// rows j + r Lc (r < 2^logf, Lc = 2^log_lc) -> rows j 2^logf + r, for
// [nimg][2^logf Lc][w] images (w a multiple of 16 bytes / element).  Must not alias.
// one_col: one element per thread (rows of any length); conj_in conjugates on load.
hipError_t launch_colstage(int prec, int logf, const void* in, void* out, int64_t nimg, int64_t w, int log_lc,
                           hipStream_t stream, bool one_col = false, bool conj_in = false);

// One super-stage pass of a multi-pass Stockham transform of `batch` signals
// of 2^logn points: radix 2^logr, span 2^logns; kind 0 first, 1 middle, 2
// last (in place allowed).  big: tables for w_M, M = 2^(logns + logr).
// Planar (see Io): in_im only for kind 0 (conj_out false), out_im only for
// kind 2 (conj_in false).
hipError_t launch_stock_pass(int prec, int logr, int kind, const void* in, void* out, int logn, int logns,
                             int64_t batch, const void* tw, BigTwiddle big, bool conj_in, bool conj_out,
                             double scale, hipStream_t stream, const void* in_im = nullptr,
                             void* out_im = nullptr);

// Polynomial products, N = 2^logn <= 8192: one fused kernel per row pair
// (z = a + i b packed; raises *d_resid, which the caller clears first).
hipError_t launch_polymul_rows(int logn, const int64_t* a, int64_t la, const int64_t* b, int64_t lb,
                               int64_t* c, int64_t batch, const void* tw, double* d_resid,
                               hipStream_t stream);

// Polynomial products, N = 2^(logn1 + logn2) beyond the LDS range (fp64),
// ws = batch x N complex128:
//  A : z = a + i 2^s b -> column FFTs (length 2^logn2) + w_N^{n1 k2} -> ws
//  B : rows k2, N2 - k2: FFT, product spectrum, the packed spectrum of the
//      real product's even / odd coefficients, N1/2-point FFT, twiddle -> ws
//  A2: the N1/2 column FFTs, two coefficients per element, 2^-s, rint -> c
// shift: s per pair (launch_poly_shift, run first).
// tw_half: the stage table for N1/2 points (the inverse runs at half length).
// d_resid (may be NULL): cleared by A, raised to the largest rounding
// residual by A2 (no separate clearing launch).
hipError_t launch_polymul_fourstep(int logn1, int logn2, const int64_t* a, int64_t la,
                                   const int64_t* b, int64_t lb, int64_t* c, int64_t batch,
                                   void* ws, const void* tw_row, const void* tw_col, const void* tw_half,
                                   BigTwiddle big, const int* shift, double* d_resid, hipStream_t stream);

// Polynomial products by a plan whose N is not a power of two: z = a + i b
// zero padded to N (complex128, batch x N) -> the plan's forward transform ->
// the product spectrum in place -> the plan's inverse -> rint(Re) and the
// residual (raised; the caller clears it first).
hipError_t launch_polyany_pack(const int64_t* a, int64_t la, const int64_t* b, int64_t lb, void* z, int64_t n,
                               int64_t batch, const int* shift, hipStream_t stream);
hipError_t launch_polyany_product(void* z, int64_t n, int64_t batch, hipStream_t stream);
hipError_t launch_polyany_round(const void* y, int64_t n, int64_t* c, int64_t lc, int64_t batch, const int* shift,
                                double* d_resid, hipStream_t stream);

// The exponent balance of the packed routes: shift[p] = s for pair p, the
// difference of the binary exponents of max|a_p| and max|b_p| (0 if either
// is all zero); z = a + i 2^s b and the outputs scaled by 2^-s.  part:
// batch x kPolyExpBlocks int2 scratch.  Two kernels on `stream`.
constexpr int kPolyExpBlocks = 64;
hipError_t launch_poly_shift(const int64_t* a, int64_t la, const int64_t* b, int64_t lb, int64_t batch,
                             void* part, int* shift, hipStream_t stream);

// The whole Bluestein transform of each row in one kernel, M = 2^logm within
// the row kernel's range (logm <= 13 complex64, 12 complex128); tw: stage
// table for M.  Inverse: conjugate in, conjugate and scale out.  Planar needs
// both in_im and out_im.  in -> out, may alias.
hipError_t launch_bluestein_rows(int prec, int logm, int n, const void* in, void* out, int64_t nrows, const void* tw,
                                 const void* chirp, const void* bspec, bool inverse, double scale,
                                 hipStream_t stream, const void* in_im = nullptr, void* out_im = nullptr);
// Bluestein beyond the row kernel's range: the chirp products and the
// product with B carried by the first / last passes of the M-point
// multi-pass transforms (chirp_io.hpp).  x / y: the caller's rows of n points
// (x_im / y_im non-NULL: planar); conj_in / conj_out and scale (1/n) for an
// inverse transform.
struct ChirpArgs {
    const void* x;
    const void* x_im;
    void* y;
    void* y_im;
    const void* chirp;
    const void* bspec;
    int64_t n;
    bool conj_in;
    bool conj_out;
    double scale;
};
// One pass of radix 2^logr of a transform of 2^logm points over [batch][M]:
// mode 0 = first forward pass (reads x times the chirp, zero padded; out:
// interleaved), 2 = last forward pass (stores conj(W B) to out), 4 = last
// inverse pass (stores the chirp times the convolution to y).  Middle passes
// and the inverse's first pass are plain launch_stock_pass calls.
hipError_t launch_bluestein_pass(int prec, int logr, int mode, const void* in, void* out, int logm, int logns,
                                 int64_t batch, const void* tw, BigTwiddle big, const ChirpArgs& c,
                                 hipStream_t stream);
// complex128 -> complex64, `total` elements.
hipError_t launch_narrow(const void* in, void* out, int64_t total, hipStream_t stream);

// Real rows (real.hip), N = 2H points.  One-kernel range (H = 2^logh within
// the rows kernel's): R2C in [nrows][2H] real -> out [nrows][H + 1] complex,
// C2R the reverse (scaled 1/N overall); tw: stage table for H; whi/wlo: w_N
// tables split at T (threads per row).  in and out must not alias.
hipError_t launch_real_rows(int prec, int logh, bool c2r, const void* in, void* out, int64_t nrows, const void* tw,
                            const void* whi, const void* wlo, hipStream_t stream);
// R2C rows of nimg real images [F Lc][2H] (H = 2^logh) with the radix-F
// column super-stage (F = 2^logf) folded in: half-spectrum rows j F + r' of
// out [nimg][F Lc][H + 1] get the F-point DFT over r of the half spectra of
// real rows j + r Lc; tw, whi, wlo as for launch_real_rows.  in and out must
// not alias.  r2c_fold_supported: whether a kernel exists for the sizes
// (launch_r2c_fold returns hipErrorInvalidValue otherwise).
bool r2c_fold_supported(int prec, int logh, int logf);
hipError_t launch_r2c_fold(int prec, int logh, int logf, const void* in, void* out, int64_t nimg, int log_lc,
                           const void* tw, const void* whi, const void* wlo, hipStream_t stream);
// Longer rows, around the H-point complex transform: R2C z [batch][H] -> out
// [batch][H + 1]; C2R x [batch][H + 1] -> z [batch][H].  wn: tables for w_N.
hipError_t launch_real_pairs(int prec, bool c2r, const void* in, void* out, int64_t h, int64_t batch,
                             BigTwiddle wn, hipStream_t stream);
// Real rows of odd length n around the n-point complex transform (real.hip),
// mode: 0 widen (real rows -> complex z), 1 take (z -> bins 0 .. (n-1)/2),
// 2 extend (bins 0 .. (n-1)/2 -> the full Hermitian z), 3 real parts
// (z -> real rows); rows rows each.  in and out must not alias.
hipError_t launch_real_odd(int prec, int mode, const void* in, void* out, int64_t n, int64_t rows,
                           hipStream_t stream);
// N = 1: out = in, real <-> complex.
hipError_t launch_real_n1(int prec, bool c2r, const void* in, void* out, int64_t batch, hipStream_t stream);

// d_resid[0] = 0 (a kernel, not a memset, so the call is safe to capture).
hipError_t launch_zero_resid(double* d_resid, hipStream_t stream);

// Streaming copy of nvec 8-byte elements (copy.hip): src and dst 8-byte
// aligned, not overlapping.  A measurement aid, not part of any transform.
hipError_t launch_stream_copy(const void* src, void* dst, int64_t nvec, hipStream_t stream);

}  // namespace fftmi
