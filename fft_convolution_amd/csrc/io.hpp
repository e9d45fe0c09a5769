// io.hpp -- how a kernel reads its input and writes its output: complex values
// interleaved (re, im) in one array, or split into two planes of reals, the
// layout of "The Butterfly: One Thread, One Output" (its signal is a [2][N]
// array: plane 0 the real parts, plane 1 the imaginary parts).
//
// Element i of a planar array is (re[i], im[i]); the planes are indexed like
// the interleaved array, so a kernel computes the same index either way and
// only the access changes.  Interleaved accesses are exactly those the kernels
// make without this wrapper (streaming loads / stores of whole elements, or a
// 16-byte vector of P adjacent elements).
#pragma once

#include "stockham.hpp"
#include "tile_common.hpp"

namespace fftmi {

// p advanced by a 32-bit byte offset: lets the compiler address a uniform base
// plus a per-lane 32-bit offset, with no 64-bit arithmetic per access.
template <typename T> __device__ __forceinline__ T* at_bytes(T* p, unsigned off)
{
    return reinterpret_cast<T*>(reinterpret_cast<char*>(p) + off);
}
template <typename T> __device__ __forceinline__ const T* at_bytes(const T* p, unsigned off)
{
    return reinterpret_cast<const T*>(reinterpret_cast<const char*>(p) + off);
}

template <typename Rl> __device__ __forceinline__ Rl ld_nt(const Rl* p) { return __builtin_nontemporal_load(p); }
template <typename Rl> __device__ __forceinline__ void st_nt(Rl* p, Rl x) { __builtin_nontemporal_store(x, p); }

template <typename V, bool PLANAR> struct CIn;
template <typename V, bool PLANAR> struct COut;

template <typename V> struct CIn<V, false> {
    const V* p;
    const V* im_unused;
    __device__ __forceinline__ V ld(int64_t i) const { return ld_stream(p + i); }
    __device__ __forceinline__ V ld_plain(int64_t i) const { return p[i]; }
    template <int P> __device__ __forceinline__ void ldv(int64_t i, V (&d)[P]) const { vload(p + i, d); }
    // the array from element `base` on, then element e < 2^32 / sizeof(V) of it
    __device__ __forceinline__ CIn at(int64_t base) const { return CIn{p + base, nullptr}; }
    __device__ __forceinline__ V ld32(unsigned e) const { return ld_stream(at_bytes(p, e * (unsigned)sizeof(V))); }
};

template <typename V> struct CIn<V, true> {
    using Rl = typename real_of<V>::type;
    const Rl* re;
    const Rl* im;
    __device__ __forceinline__ V ld(int64_t i) const { return V{ld_nt(re + i), ld_nt(im + i)}; }
    __device__ __forceinline__ V ld_plain(int64_t i) const { return V{re[i], im[i]}; }
    // P adjacent elements: P reals from each plane (8 bytes for complex64,
    // whose planes are 8-byte aligned and i even).
    __device__ __forceinline__ void ldv(int64_t i, float2 (&d)[2]) const
    {
        const float2 a = *reinterpret_cast<const float2*>(re + i);
        const float2 b = *reinterpret_cast<const float2*>(im + i);
        d[0] = float2{a.x, b.x};
        d[1] = float2{a.y, b.y};
    }
    __device__ __forceinline__ void ldv(int64_t i, double2 (&d)[1]) const { d[0] = double2{re[i], im[i]}; }
    __device__ __forceinline__ CIn at(int64_t base) const { return CIn{re + base, im + base}; }
    __device__ __forceinline__ V ld32(unsigned e) const
    {
        const unsigned o = e * (unsigned)sizeof(Rl);
        return V{ld_nt(at_bytes(re, o)), ld_nt(at_bytes(im, o))};
    }
};

template <typename V> struct COut<V, false> {
    V* p;
    V* im_unused;
    __device__ __forceinline__ void st(int64_t i, V y) const { st_stream(p + i, y); }
    __device__ __forceinline__ void st_plain(int64_t i, V y) const { p[i] = y; }
    template <int P> __device__ __forceinline__ void stv(int64_t i, const V (&s)[P]) const { vstore(p + i, s); }
    __device__ __forceinline__ COut at(int64_t base) const { return COut{p + base, nullptr}; }
    __device__ __forceinline__ void st32(unsigned e, V y) const { st_stream(at_bytes(p, e * (unsigned)sizeof(V)), y); }
};

template <typename V> struct COut<V, true> {
    using Rl = typename real_of<V>::type;
    Rl* re;
    Rl* im;
    __device__ __forceinline__ void st(int64_t i, V y) const
    {
        st_nt(re + i, y.x);
        st_nt(im + i, y.y);
    }
    __device__ __forceinline__ void st_plain(int64_t i, V y) const
    {
        re[i] = y.x;
        im[i] = y.y;
    }
    __device__ __forceinline__ void stv(int64_t i, const float2 (&s)[2]) const
    {
        *reinterpret_cast<float2*>(re + i) = float2{s[0].x, s[1].x};
        *reinterpret_cast<float2*>(im + i) = float2{s[0].y, s[1].y};
    }
    __device__ __forceinline__ void stv(int64_t i, const double2 (&s)[1]) const
    {
        re[i] = s[0].x;
        im[i] = s[0].y;
    }
    __device__ __forceinline__ COut at(int64_t base) const { return COut{re + base, im + base}; }
    __device__ __forceinline__ void st32(unsigned e, V y) const
    {
        const unsigned o = e * (unsigned)sizeof(Rl);
        st_nt(at_bytes(re, o), y.x);
        st_nt(at_bytes(im, o), y.y);
    }
};

// Host side: build the wrapper from the launcher's pointers (im == NULL for
// an interleaved array).
template <typename V, bool PLANAR> inline CIn<V, PLANAR> make_in(const void* a, const void* im)
{
    if constexpr (PLANAR) {
        using Rl = typename real_of<V>::type;
        return CIn<V, true>{(const Rl*)a, (const Rl*)im};
    } else {
        return CIn<V, false>{(const V*)a, nullptr};
    }
}
template <typename V, bool PLANAR> inline COut<V, PLANAR> make_out(void* a, void* im)
{
    if constexpr (PLANAR) {
        using Rl = typename real_of<V>::type;
        return COut<V, true>{(Rl*)a, (Rl*)im};
    } else {
        return COut<V, false>{(V*)a, nullptr};
    }
}

}  // namespace fftmi
