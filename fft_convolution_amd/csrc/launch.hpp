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

// Workgroups of `kernel` (block threads, static LDS only) the device holds at
// once: blocks per CU at full occupancy times the CU count.  Cached per kernel
// (all devices are assumed alike).  Returns 0 if the query fails.
template <typename K>
int64_t resident_blocks(K kernel, int block)
{
    static const int64_t cached = [&]() -> int64_t {
        int dev = 0, ncu = 0, per = 0;
        if (hipGetDevice(&dev) != hipSuccess) return 0;
        if (hipDeviceGetAttribute(&ncu, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return 0;
        if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per, kernel, block, 0) != hipSuccess) return 0;
        return (int64_t)(per > 0 ? per : 1) * ncu;
    }();
    return cached;
}

// Elements per line that the tile kernels stage in LDS at once, and the
// number of adjacent lines (columns) one workgroup takes.
int tile_lines(int prec, int logl);

// Rows kernel: `nrows` contiguous rows of 2^logn points, in -> out (may alias).
// conj_in conjugates on load; conj_out conjugates and multiplies by `scale` on store.
hipError_t launch_rows(int prec, int logn, bool conj_in, bool conj_out, const void* in, void* out,
                       int64_t nrows, const void* tw, double scale, hipStream_t stream);

// 2D column pass: for each of `nimg` images [2^logh][w], transform every
// column (length 2^logh) in -> out (may alias).
hipError_t launch_cols2d(int prec, int logh, const void* in, void* out, int64_t nimg, int64_t w,
                         const void* tw, bool conj_out, double scale, hipStream_t stream);

// Four-step pass A: for each of `batch` signals of N = n1 * 2^logn2 points
// viewed as [2^logn2][n1], transform every column (length 2^logn2), multiply
// element (k2, col) by w_N^{col k2}, write to ws in the same layout.
hipError_t launch_fourstep_a(int prec, int logn2, int64_t n1, const void* in, void* ws,
                             int64_t batch, const void* tw, BigTwiddle big, bool conj_in,
                             hipStream_t stream);

// Four-step pass B: transform every row k2 (length 2^logn1) of ws [n2][2^logn1]
// and store element k1 of row k2 at out[k2 + n2 k1].
hipError_t launch_fourstep_b(int prec, int logn1, int64_t n2, const void* ws, void* out,
                             int64_t batch, const void* tw, bool conj_out, double scale,
                             hipStream_t stream);

// Polynomial products, N = 2^logn <= LDS range: one fused kernel per row pair.
hipError_t launch_polymul_rows(int logn, const int64_t* a, int64_t la, const int64_t* b, int64_t lb,
                               int64_t* c, int64_t batch, const void* tw, double* d_resid,
                               hipStream_t stream);

// Polynomial products, N = n1 * n2 beyond the LDS range (fp64):
//  A : int64 operands -> column FFTs (length n2) + w_N^{n1 k2}  -> ws_a, ws_b
//  B : per row k2: FFT rows of ws_a and ws_b, product, conjugate, FFT,
//      multiply by w_N^{n1 k2}                                  -> ws_a
//  A2: column FFTs of ws_a, real part / N, rint                 -> c
hipError_t launch_polymul_fourstep(int logn1, int logn2, const int64_t* a, int64_t la,
                                   const int64_t* b, int64_t lb, int64_t* c, int64_t batch,
                                   void* ws, const void* tw_row, const void* tw_col, BigTwiddle big,
                                   double* d_resid, hipStream_t stream);

// d_resid[0] = 0 (a kernel, not a memset, so the call is safe to capture).
hipError_t launch_zero_resid(double* d_resid, hipStream_t stream);

}  // namespace fftmi
