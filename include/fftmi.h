/*
 * fftmi.h -- C ABI of a complex (and real-row) FFT library for one AMD Instinct
 * MI355X (gfx950).
 *
 * The transform computed is the discrete Fourier transform of the page "FFT on
 * GPU" (elwhyjay.github.io/post/fft), section "Discrete Fourier Transform":
 *     forward  X_k = sum_{n<N} x_n e^{-2 pi i k n / N}
 *     inverse  x_n = (1/N) sum_{k<N} X_k e^{+2 pi i k n / N}
 * (the inverse with w -> w^{-1} and the factor 1/N is from the same page, the
 * section on why roots of unity are used as evaluation points).  It is
 * evaluated as log2 N radix-2 butterfly levels (a + w b, a - w b; "The
 * Butterfly: One Thread, One Output") in the out-of-place Stockham autosort
 * form of "Stockham FFT Butterfly Algorithm in Parallel GLSL" (section "The
 * Bit-Reversal Bottleneck and the Stockham Advantage"): no bit-reversal pass,
 * output in natural order.  Rank-1 lengths that are not powers of two run as
 * mixed-radix Stockham stages (radices 2, 3, 4, 5, 7, 8) or by Bluestein's
 * chirp-z convolution on the power-of-two path (fft_plan_create).
 *
 * Conventions shared by every entry point
 *  - Complex data are interleaved (re, im): FFT_C32 = two floats (8 B per
 *    element), FFT_C64 = two doubles (16 B per element); fft_exec_planar takes
 *    split re / im planes instead.
 *  - Every data pointer (in, out, a, b, c, workspace, d_max_residual) is a
 *    DEVICE pointer on the device that was current when the plan was created.
 *    The caller owns all of them; the library never frees or retains them.
 *  - The plan owns only its small twiddle tables (device memory allocated in
 *    fft_plan_create, freed in fft_plan_destroy).  A plan is immutable after
 *    creation: concurrent executions on different streams are safe when each
 *    has its own output and workspace.
 *  - `stream` is a hipStream_t passed as void* (NULL = the null stream).
 *    Execution calls only enqueue work on it and return; they never
 *    synchronise.  A device fault surfaces at the caller's next sync.
 *  - Every call returns an fft_status: 0 on success, a negative code on
 *    failure.  Arguments are validated before any HIP call is made; on a
 *    validation error nothing is enqueued.  Nothing is thrown across the ABI.
 *  - batch == 0 is a no-op that returns FFT_OK (pointers may then be NULL).
 *  - The output is bitwise deterministic for given inputs and plan.
 */
#ifndef FFTMI_H
#define FFTMI_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct fft_plan fft_plan; /* opaque */

/* Precision of a plan: complex64 (fp32 re, im) or complex128 (fp64). */
enum fft_precision { FFT_C32 = 0, FFT_C64 = 1 };

/* Direction: forward uses e^{-i}; inverse uses e^{+i} and scales by 1/N
 * (by 1/(H*W) for a 2D plan), so inverse(forward(x)) = x. */
enum fft_direction { FFT_FORWARD = 0, FFT_INVERSE = 1 };

enum fft_status {
    FFT_OK = 0,
    FFT_ERR_INVALID_ARG = -1,      /* NULL pointer, batch < 0, bad rank/dir/prec value */
    FFT_ERR_NOT_POW2 = -2,         /* a length is not a power of two (no call returns it now) */
    FFT_ERR_UNSUPPORTED_SIZE = -3, /* a dimension outside the supported range, or
                                      la + lb - 1 > N for fft_poly_mul */
    FFT_ERR_PRECISION = -4,        /* operation needs another precision (poly-mul: FFT_C64) */
    FFT_ERR_RANK = -5,             /* plan rank or kind differs from the call (exec_c2c: 1,
                                      exec_2d: 2, exec_3d: 3, exec_r2c/c2r: a real plan) */
    FFT_ERR_ALIGN = -6,            /* a pointer is not aligned to its element size */
    FFT_ERR_OVERLAP = -7,          /* buffers partially overlap (in == out is allowed) */
    FFT_ERR_WORKSPACE = -8,        /* workspace required but NULL, or overlapping data */
    FFT_ERR_DEVICE = -9            /* a HIP call failed; text in fft_last_error() */
};

/* Largest supported transform lengths. */
#define FFT_MAX_LDS_N_C32 8192        /* one-kernel, LDS-resident rows */
#define FFT_MAX_LDS_N_C64 4096
#define FFT_MAX_N_C32 (1LL << 26)     /* multi-pass beyond the LDS-resident range */
#define FFT_MAX_N_C64 (1LL << 24)
#define FFT_MAX_BLUESTEIN_N (1LL << 23) /* rank-1 lengths that are not powers of two */

/*
 * Create a plan.
 *   rank 1: dims = {N};      1 <= N <= FFT_MAX_N_C32 (C32) / FFT_MAX_N_C64 (C64).
 *           N <= FFT_MAX_LDS_N_* runs as one LDS-resident kernel per batch of
 *           rows, and so does N = 2 FFT_MAX_LDS_N_* (16384 C32, 8192 C64: one
 *           1024-thread workgroup a row, 136 / 144 KiB of LDS); larger N runs
 *           as two or three Stockham super-stage passes (radix <= 512 each)
 *           through HBM and needs a workspace of one batch of signals.
 *           N not a power of two (N <= FFT_MAX_BLUESTEIN_N), the two routes
 *           "FFT on GPU" (section "Algorithm per signal Length") names for
 *           such lengths:
 *           - N = 2^a 3^b 5^c 7^d 11^e 13^f up to 8192 (C32) / 4096 (C64):
 *             mixed-radix Stockham stages (radices 8, 4, 2, 9, 3, 5, 7, 11,
 *             13) in one kernel, no workspace;
 *           - such N beyond that: N = R0 R1 (R2), each R <= 512 (<= 1024
 *             where that makes two passes of three, for R without a factor
 *             11 or 13), as two or three super-stage passes whose R-point
 *             transforms run those
 *             mixed-radix stages; a workspace of one batch of signals, like
 *             the power-of-two passes (fft_plan_describe: path=mixpass);
 *           - any other N: chirp-z (Bluestein), X_k = c_k (x.c * conj c)_k
 *             with c_j = e^{-i pi j^2/N}, the convolution done cyclically at
 *             the power-of-two M >= 2N - 1 by the library's own transforms.
 *             Plan creation then also runs one fp64 M-point transform on the
 *             device (the spectrum of the chirp).  M <= 2 FFT_MAX_LDS_N_*
 *             (16384 C32, 8192 C64): one kernel, no workspace; larger M: five
 *             passes and a workspace of batch * M elements plus that of the
 *             M-point plan.
 *   rank 2: dims = {H, W}, row-major with W contiguous ("Stockham FFT ... in
 *           Parallel GLSL", section "Multi-Dimensional Transforms and
 *           Separability": rows, then columns); 1 <= H <= FFT_MAX_LDS_N_*,
 *           1 <= W <= 2 FFT_MAX_LDS_N_* (rows of 16384 C32 / 8192 C64 take
 *           the one-kernel rows of one 1024-thread workgroup each; only the
 *           innermost axis longer than 1 may exceed FFT_MAX_LDS_N_*).
 *           Columns longer than 512 points are split H = F * Lc: the radix-F
 *           column stage is folded into the row pass, or, where F rows of
 *           W points do not fit one workgroup's LDS (e.g. 8192 x 8192
 *           FFT_C32), runs as a pass of its own (fft_plan_describe shows
 *           split=F).
 *   rank 3: dims = {D, H, W}, row-major: the 2D transform of every [H][W]
 *           slice, then the D-point transform along the depth axis of every
 *           (y, x) (the same separability, one axis after another); each
 *           dimension as for rank 2, and the depth D <= 2048 (C32) / 1024 (C64)
 *           unless H = W = 1.
 *   rank 2 / 3 with a dimension that is not a power of two: the innermost
 *           axis W may have any length a rank-1 plan takes (it runs as the
 *           rank-1 plan over every row); every other axis longer than 1 of
 *           2^a 3^b 5^c 7^d 11^e 13^f points runs as one super-stage pass up
 *           to 1024 points (512 with a factor 11 or 13), two or three beyond;
 *           an axis of any other length up to FFT_MAX_BLUESTEIN_N is
 *           transposed to be innermost, transformed as rows by the rank-1
 *           plan of its length (chirp-z), and transposed back
 *           (fft_plan_describe: axisK=transposed[...]); at most FFT_MAX_N_*
 *           points per transform (fft_plan_describe: path=ndmixed).
 *           Workspace: fft_workspace_size, out of place too (a signal-sized
 *           buffer for an axis of two or more passes, plus what the rows
 *           need, plus a signal-sized buffer and the axis plan's workspace
 *           for a transposed axis).
 *   prec:   FFT_C32 or FFT_C64.
 * Builds the twiddle tables in fp64 on the host, rounds them to the plan
 * precision and uploads them (the only synchronous device work of the
 * library).  On success *plan receives the new plan; on failure *plan is set
 * to NULL.  Errors: INVALID_ARG, UNSUPPORTED_SIZE, DEVICE.
 */
int fft_plan_create(fft_plan** plan, int rank, const int64_t* dims, int prec);

/* Free a plan and its device tables.  NULL is accepted (no-op). */
int fft_plan_destroy(fft_plan* plan);

/* Describe a plan: rank, dims, precision and the kernel path chosen, as a
 * NUL-terminated string of at most len bytes.  Host-only. */
int fft_plan_describe(const fft_plan* plan, char* buf, size_t len);

/* The description fft_plan_describe would give for the plan that
 * fft_plan_create(rank, dims, prec) would make, without making it: host-only
 * (no HIP call, no device needed), the same validation and status codes.
 * Errors: INVALID_ARG, UNSUPPORTED_SIZE. */
int fft_plan_query(int rank, const int64_t* dims, int prec, char* buf, size_t len);

/* Bytes of device workspace fft_exec_c2c / fft_exec_2d need for `batch`
 * transforms with this plan (0 when none is needed).  Host-only. */
int fft_workspace_size(const fft_plan* plan, int64_t batch, size_t* bytes);

/*
 * Batched 1D transform with a rank-1 plan: for each row, X_k = sum_n x_n
 * e^{-2 pi i k n / N} (forward) or x_n = (1/N) sum_k X_k e^{+2 pi i k n / N}
 * (inverse) -- "FFT on GPU", sections "Discrete Fourier Transform" and the
 * one on why roots of unity are used (w -> w^{-1}, factor 1/N) -- computed
 * as the Stockham passes of "Stockham FFT Butterfly Algorithm in Parallel
 * GLSL", section "Execution via GLSL Compute Shaders and Textures", fused
 * into on-chip stages as its section "Performance and Pipeline Evaluation"
 * recommends.
 *   in, out:   [batch][N] complex of the plan's precision, rows contiguous.
 *              in == out (in place) is allowed; any other overlap is an error.
 *              in is not modified unless in == out.
 *   workspace: fft_workspace_size(plan, batch) bytes (NULL when that is 0);
 *              must not overlap in or out.
 * Errors: INVALID_ARG, RANK, ALIGN, OVERLAP, WORKSPACE, DEVICE.
 */
int fft_exec_c2c(const fft_plan* plan, int dir, const void* in, void* out, int64_t batch,
                 void* workspace, void* stream);

/*
 * fft_exec_c2c without any allocation, for callers that cannot call
 * hipMalloc (code under HIP graph capture, tight serving loops, harnesses
 * that forbid it).  The same transform, kernels and results as fft_exec_c2c,
 * but plans that need a workspace take it from a scratch array the library
 * holds in device memory: FFT_NOALLOC_SCRATCH_BYTES (128 MiB) per GPU,
 * reserved on each GPU from its first call there until the process ends
 * (enough for one 2^24-point complex64 transform, or batch x N <= 2^24
 * complex64 / 2^23 complex128 elements on the multi-pass path).
 *   in, out, batch, dir, stream: as fft_exec_c2c.
 *   The scratch is shared by every call on a GPU and keeps the last call's
 *   contents; no part of it needs to start at zero (every kernel writes what
 *   it later reads).  Calls on one GPU whose executions overlap (different
 *   streams, or host threads racing) use the same scratch and RACE: order
 *   them on one stream or synchronise between them.
 * Calls no hipMalloc, hipFree or other allocating routine; the first call on
 * a device looks up the scratch's device address (hipGetSymbolAddress).
 * Errors: as fft_exec_c2c, plus WORKSPACE when fft_workspace_size(plan,
 * batch) exceeds FFT_NOALLOC_SCRATCH_BYTES (checked before any HIP call).
 */
#define FFT_NOALLOC_SCRATCH_BYTES (128LL << 20)
int fft_exec_c2c_noalloc(const fft_plan* plan, int dir, const void* in, void* out, int64_t batch, void* stream);

/*
 * Batched 2D transform with a rank-2 plan: row transforms of length W over
 * every row, then column transforms of length H over every column
 * ("Stockham FFT Butterfly Algorithm in Parallel GLSL", section
 * "Multi-Dimensional Transforms and Separability": the 2D transform is the 1D
 * transform along one axis, then along the other); the inverse scales by
 * 1/(H W).
 *   in, out:   [batch][H][W] complex, images contiguous.  in == out allowed.
 *   workspace: fft_workspace_size(plan, batch) bytes for an in-place call
 *              (in == out) on a plan that folds part of the column transform
 *              into the row pass (H > 512; fft_plan_describe shows fold > 1),
 *              and for every call on a split plan (split=F) or a plan with a
 *              dimension that is not a power of two (path=ndmixed) whose
 *              fft_workspace_size is not 0; otherwise it may be NULL.
 * Errors: as fft_exec_c2c.
 */
int fft_exec_2d(const fft_plan* plan, int dir, const void* in, void* out, int64_t batch,
                void* workspace, void* stream);

/*
 * Batched 3D transform with a rank-3 plan: the same separability one axis
 * after another ("Stockham FFT Butterfly Algorithm in Parallel GLSL", section
 * "Multi-Dimensional Transforms and Separability", which names 2D and 3D
 * data); the inverse scales by 1/(D H W).
 *   in, out:   [batch][D][H][W] complex, volumes contiguous.  in == out allowed.
 *   workspace: as fft_exec_2d (power-of-two plans: only in place when the
 *              plan folds).
 * Errors: as fft_exec_c2c.
 */
int fft_exec_3d(const fft_plan* plan, int dir, const void* in, void* out, int64_t batch,
                void* workspace, void* stream);

/*
 * The transform of any complex plan (rank 1, 2 or 3) on split arrays: the real
 * parts in one plane and the imaginary parts in another ("The Butterfly: One
 * Thread, One Output" holds its signal as a [2][N] array, plane 0 the real
 * parts, plane 1 the imaginary parts).  Results equal those of the
 * interleaved calls bit for bit: only the first kernel's loads and the last
 * kernel's stores differ.
 *   in_re, in_im, out_re, out_im: each [batch][dims...] float (FFT_C32) or
 *              double (FFT_C64), the layout of the interleaved call with one
 *              real per element; 8-byte aligned.  A [2][N] array p gives
 *              re = p, im = p + N (batch 1); a [2][batch][N] array gives
 *              im = p + batch N.  The two planes of one array must not overlap.
 *              In place: in_re == out_re and in_im == out_im; any other
 *              overlap of input and output planes is an error.
 *   workspace: fft_planar_workspace_size(plan, batch) bytes (NULL when 0):
 *              none for one-kernel rank-1 plans and rank-2/3 plans with one
 *              axis longer than 1; one batch of signals for two-pass
 *              multi-pass, rank-2/3 and Bluestein plans (these keep their
 *              intermediate there); two for three-pass multi-pass plans.
 * Errors: INVALID_ARG, RANK (real plan), ALIGN, OVERLAP, WORKSPACE, DEVICE.
 */
int fft_exec_planar(const fft_plan* plan, int dir, const void* in_re, const void* in_im, void* out_re,
                    void* out_im, int64_t batch, void* workspace, void* stream);

/* Bytes of device workspace fft_exec_planar needs for `batch` transforms. */
int fft_planar_workspace_size(const fft_plan* plan, int64_t batch, size_t* bytes);

/* Bytes of device workspace fft_poly_mul needs for `batch` pairs. */
int fft_poly_mul_workspace_size(const fft_plan* plan, int64_t batch, size_t* bytes);

/*
 * Products of integer polynomials by FFT ("FFT on GPU", polynomial
 * multiplication and whole-process sections): for each pair p,
 *     c_p[k] = sum_i a_p[i] b_p[k-i],  0 <= k < la + lb - 1,
 * computed as: zero-pad a and b to N, forward FFT of both (fp64), pointwise
 * product, inverse FFT (scaled 1/N), round the real part to the nearest
 * integer (ties to even).
 *   plan:  rank 1, FFT_C64, N >= la + lb - 1, N <= 2^22.  N a power of two:
 *          the fused kernels (one per row pair: a and b transformed apart up
 *          to N = 4096; for N = 8192 z = a + i b transformed once, the
 *          product spectrum from the bin pairs k and N - k, the inverse;
 *          beyond, three four-step passes on z).  Any other N: the plan's
 *          own transforms (mixed radix or chirp-z, "FFT on GPU", section
 *          "Algorithm per signal Length") between element-wise kernels --
 *          z zero padded to N, the forward transform, the product spectrum
 *          (Z_k^2 - conj(Z_{-k})^2) / 4i in place, the inverse, rint.
 *          Wherever a and b are packed into z, b is scaled by 2^s first and
 *          the outputs by 2^-s (exact), s = the difference of the binary
 *          exponents of max|a| and max|b| per pair, so that operands of
 *          unlike magnitudes keep the rounding error of separate transforms.
 *   a:     [batch][la] int64;  b: [batch][lb] int64;  c: [batch][la+lb-1] int64.
 *          c must not overlap a, b or the workspace.
 *   workspace: fft_poly_mul_workspace_size(plan, batch) bytes (none for
 *          N <= 8192 powers of two; else the transforms' space plus 520
 *          bytes per pair for the exponent balance).
 *   d_max_residual: NULL, or a device double that receives
 *          max |Re(y)/N - rint(Re(y)/N)| over all outputs (overwritten, not
 *          accumulated), or +infinity if any output has |Re(y)/N| >= 2^53 or
 *          is not finite: past 2^53 every double is an integer, so a rounding
 *          error no longer shows as a fraction and exactness cannot be
 *          vouched for.  The result is exact when this stays well below 0.5;
 *          callers with large coefficients should check it.  Outputs beyond
 *          the int64 range (or not finite) are stored as INT64_MIN.
 * Errors: INVALID_ARG, RANK, PRECISION, UNSUPPORTED_SIZE, ALIGN, OVERLAP,
 *         WORKSPACE, DEVICE.
 */
int fft_poly_mul(const fft_plan* plan, const int64_t* a, int64_t la, const int64_t* b,
                 int64_t lb, int64_t* c, int64_t batch, void* workspace,
                 double* d_max_residual, void* stream);

/*
 * Plan for transforms of real rows of N points: any N >= 1, up to
 * 2 * FFT_MAX_N_C32 (C32) / 2 * FFT_MAX_N_C64 (C64) for powers of two,
 * 2 * FFT_MAX_BLUESTEIN_N for other even N and FFT_MAX_BLUESTEIN_N for odd N.
 * The operands of polynomial multiplication are real ("FFT on GPU",
 * polynomial-multiplication section); a real row's transform is fixed by
 * its bins X_0 .. X_{floor(N/2)}, since X_{N-k} = conj X_k.  Even N: the row
 * is read as N/2 complex values and goes through the N/2-point complex
 * transform (whichever route that length has), then one split step (and the
 * reverse for C2R).  Odd N: the row goes through the N-point complex
 * transform of the row itself (mixed radix or chirp-z), widened to complex
 * in the workspace (fft_plan_describe: "odd").  prec: FFT_C32 (float rows,
 * complex64 bins) or FFT_C64 (double rows, complex128 bins).  The plan
 * serves only fft_exec_r2c / fft_exec_c2r (other calls give FFT_ERR_RANK);
 * fft_workspace_size and fft_plan_describe accept it.
 * Errors: INVALID_ARG, UNSUPPORTED_SIZE, DEVICE.
 */
int fft_plan_create_real(fft_plan** plan, int64_t n, int prec);

/*
 * Plan for real images [H][W] -- H, W powers of two, 1 <= H <= FFT_MAX_LDS_N_*,
 * 1 <= W <= 4 FFT_MAX_LDS_N_*: the 2D transform's columns 0 .. W/2, the rest
 * following from X[u][v] = conj X[-u][-v].  The rows go through the real-row
 * kernels, then the H-point column transforms run over the W/2 + 1 columns of
 * the half spectrum (one column per lane; for H > 512 a radix-F column stage
 * first, as for complex plans).  The same fft_exec_r2c / fft_exec_c2r calls
 * take it; fft_plan_describe shows path=real2d.
 * Other shapes: any W, any H <= FFT_MAX_BLUESTEIN_N, at most FFT_MAX_N_*
 * points in the half spectrum: the rows by the real-row plan of length W
 * (fft_plan_create_real), then the column axis -- for H = 2^a 3^b 5^c 7^d
 * 11^e 13^f as mixed-radix super-stage passes over the half spectrum; for
 * other H ("FFT on GPU", section "Algorithm per signal Length": the chirp-z
 * route for any length) transposed to [W/2 + 1][H], run as rows by the rank-1
 * plan of length H, and transposed back (fft_plan_describe:
 * "axis1=transposed[...]") -- (path=real2dmixed); a workspace of
 * fft_workspace_size bytes on every call (C2R runs the columns into it and
 * leaves its input as it was).
 * Errors: INVALID_ARG, UNSUPPORTED_SIZE, DEVICE.
 */
int fft_plan_create_real_2d(fft_plan** plan, int64_t h, int64_t w, int prec);

/*
 * Forward transform of real rows: out[b][k] = sum_n in[b][n] e^{-2 pi i k n / N},
 * k = 0 .. floor(N/2).
 *   in:        [batch][N] real (float for C32, double for C64), rows contiguous.
 *   out:       [batch][floor(N/2) + 1] complex, rows contiguous.  in and out
 *              must not overlap (FFT_ERR_OVERLAP); both aligned to the complex
 *              element size (8 bytes C32, 16 bytes C64).
 *   workspace: fft_workspace_size(plan, batch) bytes: none for powers of two
 *              with N/2 <= 2 FFT_MAX_LDS_N_* (one kernel); batch * N/2 complex
 *              values beyond (even N; plus the N/2-point plan's own workspace
 *              where N/2 is not a power of two); batch * N complex values
 *              plus the N-point plan's workspace for odd N.
 *   Images (fft_plan_create_real_2d): in [batch][H][W] real, out
 *              [batch][H][W/2 + 1] complex; the workspace (batch H (W/2 + 1)
 *              complex values, the size fft_workspace_size reports, which
 *              covers fft_exec_c2r too) is needed only for H > 512 on plans
 *              whose radix-F column stage is not folded into the row pass
 *              (fft_plan_describe: folded=0); with folded=1 it may be NULL.
 * Errors: INVALID_ARG, RANK, ALIGN, OVERLAP, WORKSPACE, DEVICE.
 */
int fft_exec_r2c(const fft_plan* plan, const void* in, void* out, int64_t batch, void* workspace, void* stream);

/*
 * Inverse: the real rows whose bins 0 .. floor(N/2) are `in`, scaled by 1/N,
 * so that c2r(r2c(x)) = x.  The imaginary parts of in[b][0] and, for even N,
 * in[b][N/2] are ignored (a real row has real values there); bins above
 * N/2 are taken as conj in[b][N - k].
 *   in:  [batch][floor(N/2) + 1] complex;  out: [batch][N] real.  Not
 *   modified: in.
 *   Images: in [batch][H][W/2 + 1], out [batch][H][W], scaled 1/(H W): the
 *   inverse column transforms, then the rows as above (the imaginary parts of
 *   columns 0 and W/2 of that intermediate are ignored).  The workspace is
 *   needed for every H > 1.
 *   Layout, alignment, overlap and workspace as fft_exec_r2c.
 * Errors: as fft_exec_r2c.
 */
int fft_exec_c2r(const fft_plan* plan, const void* in, void* out, int64_t batch, void* workspace, void* stream);

/*
 * Measurement aid, not part of any transform: copy `bytes` bytes from src to
 * dst (device memory) with a streaming kernel that reads every byte once and
 * writes it once, as the row kernels stream their rows ("Stockham FFT
 * Butterfly Algorithm in Parallel GLSL", section "Performance and Pipeline
 * Evaluation": the transform is bound by memory throughput, so a plain copy
 * of the same bytes is its practical ceiling).  Enqueued on `stream`.
 *   src, dst: 8-byte aligned, not overlapping; bytes a multiple of 8
 *             (0 is a no-op).
 * Errors: INVALID_ARG (NULL), ALIGN, OVERLAP, DEVICE.
 */
int fft_stream_copy(const void* src, void* dst, size_t bytes, void* stream);

/* Static text for a status code ("unknown status" for anything else). */
const char* fft_status_string(int status);

/* Text of the last error on the calling thread (empty if none). */
const char* fft_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* FFTMI_H */
