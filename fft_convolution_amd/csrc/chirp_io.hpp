// chirp_io.hpp -- load / store policies that carry the element-wise steps of
// Bluestein's chirp-z transform (bluestein.hip) into the first and last
// passes of the multi-pass power-of-two transforms it runs on, so that the
// chirp products and the product with B cost no pass of their own.
//
// The padded signal is [batch][M] (M = 2^logm); element e is (row, p) with
// row = e >> logm, p = e mod M.  The caller's rows hold n <= M/2 points.
#pragma once

#include "io.hpp"

namespace fftmi {

// First pass of the forward transform: element e reads x[row][p] c_p (the
// input conjugated first for an inverse transform), 0 for p >= n.
template <typename V, bool PL> struct ChirpIn {
    CIn<V, PL> x;
    const V* __restrict__ chirp;
    int64_t n;
    int logm;
    int conj;
    __device__ __forceinline__ V at(int64_t e) const
    {
        const int64_t row = e >> logm, p = e & (((int64_t)1 << logm) - 1);
        if (p >= n) return V{0, 0};
        V v = x.ld_plain(row * n + p);
        if (conj) v = cconj(v);
        return cmul(v, chirp[p]);
    }
    template <int P> __device__ __forceinline__ void ldv(int64_t i, V (&d)[P]) const
    {
#pragma unroll
        for (int e = 0; e < P; ++e) d[e] = at(i + e);
    }
};

// Last pass of the forward transform: stores conj(W_e B_{e mod M}), the input
// of the inverse transform taken as conj(F(conj .)).
template <typename V> struct MulConjOut {
    V* p;
    const V* __restrict__ tab;
    int logm;
    template <int P> __device__ __forceinline__ void stv(int64_t i, const V (&s)[P]) const
    {
        const int64_t mask = ((int64_t)1 << logm) - 1;
        V q[P];
#pragma unroll
        for (int e = 0; e < P; ++e) q[e] = cconj(cmul(s[e], tab[(i + e) & mask]));
        vstore(p + i, q);
    }
};

// Last pass of the inverse transform: element e (p < n) is y = conj(s_e) / M,
// the cyclic convolution; out[row][p] = c_p y (conjugated and scaled by
// `scale` for an inverse transform); elements p >= n are dropped.
template <typename V, bool PL> struct ChirpOut {
    using Rl = typename real_of<V>::type;
    COut<V, PL> out;
    const V* __restrict__ chirp;
    int64_t n;
    int logm;
    int conj;
    Rl scale;
    Rl inv_m;
    template <int P> __device__ __forceinline__ void stv(int64_t i, const V (&s)[P]) const
    {
        const int64_t mask = ((int64_t)1 << logm) - 1;
#pragma unroll
        for (int e = 0; e < P; ++e) {
            const int64_t pos = i + e, row = pos >> logm, p = pos & mask;
            if (p < n) {
                const V y = cmul(V{s[e].x * inv_m, -s[e].y * inv_m}, chirp[p]);
                out.st_plain(row * n + p, conj ? V{y.x * scale, -y.y * scale} : y);
            }
        }
    }
};

}  // namespace fftmi
