// tile_common.hpp -- pieces shared by the tile kernels (tiles.hip, polymul.hip).
#pragma once

#include "stockham.hpp"

namespace fftmi {

// Tile geometry for passes over lines of L = 2^LOGL points that are not
// contiguous in memory (matrix columns, Stockham butterflies at a stride).
// Each thread owns P adjacent lines, loaded together as one 16-byte vector
// per position; CL threads side by side cover a 128-byte row segment (the
// unit the memory system moves without waste); a workgroup owns C = CL P
// lines and runs the P sets of CL lines through LDS one after another.
// CLMIN: the fewest lanes per row segment (8: 128-byte segments of 16-byte
// vectors; 16 for passes that also move 8-byte values per lane, so that those
// come in 128-byte segments too).
// PV: adjacent lines per thread (16 bytes by default; 1 for arrays whose rows
// are not a multiple of 16 bytes long).
template <typename V, int LOGL, int CLMIN = 8, int PV = 16 / (int)sizeof(V)> struct Tile {
    using G = Geom<V, LOGL>;
    static constexpr int P = PV;                        // complex64: 2, complex128: 1
    static constexpr int CL0 = 256 / G::T;
    static constexpr int CL = CL0 < CLMIN ? CLMIN : (CL0 > 64 ? 64 : CL0);
    static constexpr int C = CL * P;
    static constexpr int THREADS = CL * G::T;
    static constexpr int LDS = G::S > 1 ? lds_padded(CL * G::N) : 1;
};

typedef float vio_f4 __attribute__((ext_vector_type(4)));

// Load / store P adjacent complex values as one 16-byte access.
__device__ __forceinline__ void vload(const float2* p, float2 (&d)[2])
{
    const vio_f4 q = *reinterpret_cast<const vio_f4*>(p);
    d[0] = float2{q.x, q.y};
    d[1] = float2{q.z, q.w};
}
__device__ __forceinline__ void vload(const double2* p, double2 (&d)[1]) { d[0] = *p; }
__device__ __forceinline__ void vload(const float2* p, float2 (&d)[1]) { d[0] = *p; }
__device__ __forceinline__ void vstore(float2* p, const float2 (&s)[2])
{
    const vio_f4 q = {s[0].x, s[0].y, s[1].x, s[1].y};
    *reinterpret_cast<vio_f4*>(p) = q;
}
__device__ __forceinline__ void vstore(double2* p, const double2 (&s)[1]) { *p = s[0]; }
__device__ __forceinline__ void vstore(float2* p, const float2 (&s)[1]) { *p = s[0]; }

// Workgroups are handed to the 8 XCDs round-robin (workgroup b runs on XCD
// b mod 8).  Give each XCD a contiguous range of tiles instead, so that
// neighbouring tiles -- which share cache lines when a tile's row segment is
// shorter than a line -- are read through the same L2.
__device__ __forceinline__ int64_t xcd_tile(unsigned b, unsigned nb)
{
    const unsigned per = nb >> 3;
    if (b < per * 8u) return (int64_t)(b & 7u) * per + (b >> 3);
    return (int64_t)b;
}

// w_N^m for large N from two tables: hi[q] = w_N^{q 2^lbits}, lo[q] = w_N^q.
template <typename V> struct BigTw {
    const V* __restrict__ hi;
    const V* __restrict__ lo;
    int lbits;
    int logn;
    __device__ __forceinline__ V operator()(int64_t m) const
    {
        m &= ((int64_t)1 << logn) - 1;
        return cmul(hi[m >> lbits], lo[m & (((int64_t)1 << lbits) - 1)]);
    }
};

// w_M^m for a power-of-two M held in one table (small M).
template <typename V> struct RootTw {
    const V* __restrict__ tab;
    int logm;
    __device__ __forceinline__ V operator()(int64_t m) const { return tab[m & (((int64_t)1 << logm) - 1)]; }
};

// v[i] holds position p = t + i T of a line; multiply it by w_N^{line p}.
// The factors are w0 = w_N^{line t} times products of g_j = w_N^{line T 2^j}
// over the set bits j of i, every factor read from the exact tables, so each
// twiddle carries a handful of roundings, not a long recurrence.
template <int LOGN, typename V, int E, typename TW>
__device__ __forceinline__ void apply_big_twiddle(V (&v)[E], int64_t line, int t, TW bt)
{
    static_assert(E == kE<V, LOGN>, "register array size");
    using G = Geom<V, LOGN>;
    V p[G::E];
    p[0] = bt(line * t);
#pragma unroll
    for (int j = 0; j < G::LOGE; ++j) {
        const V g = bt((line * G::T) << j);
#pragma unroll
        for (int i = 0; i < (1 << j); ++i) p[i + (1 << j)] = cmul(p[i], g);
    }
#pragma unroll
    for (int i = 0; i < G::E; ++i) v[i] = cmul(v[i], p[i]);
}

}  // namespace fftmi
