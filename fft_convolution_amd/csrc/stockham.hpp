// stockham.hpp -- device-side building blocks of the Stockham FFT kernels.
//
//  * complex arithmetic on float2 / double2 (interleaved re, im);
//  * R-point DFTs in registers (R = 2 .. 32) with compile-time constant
//    twiddles: the butterfly a + w b / a - w b of "The Butterfly: One Thread,
//    One Output", fused over log2 R levels;
//  * the workgroup engine `fft_regs`: every thread owns E elements of one
//    transform (positions t + i T); the stages of radix_plan.hpp run in
//    registers, and between stages the outputs go through LDS, written in the
//    Stockham output order and read back in the next stage's input order (the
//    ping-pong of "Stockham FFT ... in Parallel GLSL", section "Execution via
//    GLSL Compute Shaders and Textures", between registers and LDS instead of
//    two textures).  The first stage reads and the last stage writes the
//    positions t + i T, so the kernels' global loads and stores are coalesced.
//
// Every transform here is forward (e^{-i}); the inverse is obtained as
// conj(F(conj(x))) / N by conjugating on load and on store.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "radix_plan.hpp"

namespace fftmi {

template <typename Rl> struct cvec;
template <> struct cvec<float> { using type = float2; };
template <> struct cvec<double> { using type = double2; };

template <typename V> struct real_of;
template <> struct real_of<float2> { using type = float; };
template <> struct real_of<double2> { using type = double; };

template <typename V> __device__ __forceinline__ V cadd(V a, V b) { return V{a.x + b.x, a.y + b.y}; }
template <typename V> __device__ __forceinline__ V csub(V a, V b) { return V{a.x - b.x, a.y - b.y}; }
template <typename V> __device__ __forceinline__ V cmul(V a, V w)
{
    return V{a.x * w.x - a.y * w.y, a.x * w.y + a.y * w.x};
}
template <typename V> __device__ __forceinline__ V cconj(V a) { return V{a.x, -a.y}; }
// a * (-i)
template <typename V> __device__ __forceinline__ V cmul_mi(V a) { return V{a.y, -a.x}; }
// a * (+i)
template <typename V> __device__ __forceinline__ V cmul_pi(V a) { return V{-a.y, a.x}; }

// ---------------------------------------------------------------------------
// Constant twiddles w_R^m = e^{-2 pi i m / R} for R | 32, in 32nds of a turn.
// ---------------------------------------------------------------------------
// cos(2 pi q / 32) for q = 0 .. 8.
constexpr double kCos32[9] = {
    1.0,
    0.98078528040323044912618223613424,
    0.92387953251128675612818318939679,
    0.83146961230254523707878837761791,
    0.70710678118654752440084436210485,
    0.55557023301960222474283081394853,
    0.38268343236508977172845998403040,
    0.19509032201612826784828486847702,
    0.0,
};

constexpr double cos32(int q)
{
    q = ((q % 32) + 32) % 32;
    return q <= 8 ? kCos32[q] : q <= 16 ? -kCos32[16 - q] : q <= 24 ? -kCos32[q - 16] : kCos32[32 - q];
}
constexpr double sin32(int q) { return cos32(q - 8); }

// v *= w_R^m, with the multiples of an eighth turn done by swaps and adds.
template <int M, int R, typename V>
__device__ __forceinline__ V mul_const_tw(V v)
{
    using Rl = typename real_of<V>::type;
    constexpr int q = ((M * (32 / R)) % 32 + 32) % 32;
    constexpr Rl h = (Rl)0.70710678118654752440084436210485;
    if constexpr (q == 0) {
        return v;
    } else if constexpr (q == 8) {
        return cmul_mi(v);
    } else if constexpr (q == 16) {
        return V{-v.x, -v.y};
    } else if constexpr (q == 24) {
        return cmul_pi(v);
    } else if constexpr (q == 4) {  // (1 - i)/sqrt2
        return V{(v.x + v.y) * h, (v.y - v.x) * h};
    } else if constexpr (q == 12) {  // (-1 - i)/sqrt2
        return V{(v.y - v.x) * h, -(v.x + v.y) * h};
    } else if constexpr (q == 20) {  // (-1 + i)/sqrt2
        return V{-(v.x + v.y) * h, (v.x - v.y) * h};
    } else if constexpr (q == 28) {  // (1 + i)/sqrt2
        return V{(v.x - v.y) * h, (v.x + v.y) * h};
    } else {
        constexpr Rl c = (Rl)cos32(q);
        constexpr Rl s = (Rl)(-sin32(q));
        return cmul(v, V{c, s});
    }
}

// ---------------------------------------------------------------------------
// R-point DFT in registers, natural order in and out:  u[k] <- sum_n u[n] w_R^{nk}.
// R = P Q: Q-point DFTs over n2 of u[P n2 + n1], twiddle w_R^{n1 k1}, then
// P-point DFTs over n1, giving X[k1 + Q k2].
// ---------------------------------------------------------------------------
template <int R> struct Dft;

template <> struct Dft<1> {
    template <typename V> __device__ __forceinline__ static void run(V*) {}
};

template <> struct Dft<2> {
    template <typename V> __device__ __forceinline__ static void run(V* u)
    {
        V a = u[0], b = u[1];
        u[0] = cadd(a, b);
        u[1] = csub(a, b);
    }
};

template <> struct Dft<4> {
    template <typename V> __device__ __forceinline__ static void run(V* u)
    {
        V a0 = cadd(u[0], u[2]), a1 = csub(u[0], u[2]);
        V a2 = cadd(u[1], u[3]), a3 = cmul_mi(csub(u[1], u[3]));
        u[0] = cadd(a0, a2);
        u[2] = csub(a0, a2);
        u[1] = cadd(a1, a3);
        u[3] = csub(a1, a3);
    }
};

template <int P, int Q> struct DftSplit {
    template <typename V> __device__ __forceinline__ static void run(V* u)
    {
        constexpr int R = P * Q;
        V y[R];  // y[n1 * Q + k1]
#pragma unroll
        for (int n1 = 0; n1 < P; ++n1) {
            V w[Q];
#pragma unroll
            for (int n2 = 0; n2 < Q; ++n2) w[n2] = u[P * n2 + n1];
            Dft<Q>::run(w);
#pragma unroll
            for (int k1 = 0; k1 < Q; ++k1) y[n1 * Q + k1] = w[k1];
        }
        twiddle_rows<0>(y);
#pragma unroll
        for (int k1 = 0; k1 < Q; ++k1) {
            V z[P];
#pragma unroll
            for (int n1 = 0; n1 < P; ++n1) z[n1] = y[n1 * Q + k1];
            Dft<P>::run(z);
#pragma unroll
            for (int k2 = 0; k2 < P; ++k2) u[k1 + Q * k2] = z[k2];
        }
    }
    // y[n1 * Q + k1] *= w_R^{n1 k1}, unrolled at compile time.
    template <int I, typename V> __device__ __forceinline__ static void twiddle_rows(V* y)
    {
        if constexpr (I < P * Q) {
            constexpr int n1 = I / Q, k1 = I % Q;
            y[I] = mul_const_tw<n1 * k1, P * Q>(y[I]);
            twiddle_rows<I + 1>(y);
        }
    }
};

template <> struct Dft<8> : DftSplit<2, 4> {};
template <> struct Dft<16> : DftSplit<4, 4> {};
template <> struct Dft<32> : DftSplit<4, 8> {};

// ---------------------------------------------------------------------------
// Streaming global access: every element is read once and written once, so
// loads and stores are marked nontemporal (they bypass cache retention).
// ---------------------------------------------------------------------------
typedef float nt_f2 __attribute__((ext_vector_type(2)));
typedef double nt_d2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ float2 ld_stream(const float2* p)
{
    const nt_f2 v = __builtin_nontemporal_load(reinterpret_cast<const nt_f2*>(p));
    return float2{v.x, v.y};
}
__device__ __forceinline__ double2 ld_stream(const double2* p)
{
    const nt_d2 v = __builtin_nontemporal_load(reinterpret_cast<const nt_d2*>(p));
    return double2{v.x, v.y};
}
__device__ __forceinline__ void st_stream(float2* p, float2 x)
{
    const nt_f2 v = {x.x, x.y};
    __builtin_nontemporal_store(v, reinterpret_cast<nt_f2*>(p));
}
__device__ __forceinline__ void st_stream(double2* p, double2 x)
{
    const nt_d2 v = {x.x, x.y};
    __builtin_nontemporal_store(v, reinterpret_cast<nt_d2*>(p));
}

// ---------------------------------------------------------------------------
// The workgroup engine.
// ---------------------------------------------------------------------------
template <typename V> struct lem_of;
template <> struct lem_of<float2> { static constexpr int value = 4; };
template <> struct lem_of<double2> { static constexpr int value = 3; };

template <int LOGN, int LEM> struct Geometry {
    static constexpr int N = 1 << LOGN;
    static constexpr int LOGE = plan_loge(LOGN, LEM);
    static constexpr int E = 1 << LOGE;         // elements per thread
    static constexpr int T = N / E;             // threads per transform
    static constexpr int S = plan_nstages(LOGN, LEM);
    static constexpr int LDS = S > 1 ? lds_padded(N) : 0;  // LDS slots per transform
};

// The geometry of a transform of 2^LOGN points of element type V.
template <typename V, int LOGN> using Geom = Geometry<LOGN, lem_of<V>::value>;
// Elements per thread, for array parameters.
template <typename V, int LOGN> constexpr int kE = Geom<V, LOGN>::E;

// Rows per workgroup of the row kernels: at least 256 threads per workgroup.
template <typename V, int LOGN> constexpr int rows_per_wg() { return Geom<V, LOGN>::T >= 256 ? 1 : 256 / Geom<V, LOGN>::T; }

template <typename V, int LOGN, int STAGE> struct StageInfo {
    using G = Geom<V, LOGN>;
    static constexpr int LEM = lem_of<V>::value;
    static constexpr int LR = plan_stage_logr(LOGN, LEM, STAGE), R = 1 << LR;
    static constexpr int LNS = plan_stage_lns(LOGN, LEM, STAGE), NS = 1 << LNS;
    static constexpr int B = G::E / R;           // butterflies per thread
    static constexpr bool TW = NS > 1;           // stage 0 needs no twiddles
    static constexpr int NB = TW ? B * LR : 1;   // twiddle bases per thread
    static constexpr bool LAST = STAGE == G::S - 1;
};

// The twiddle bases a thread needs for every stage, loaded once (they depend
// only on the thread's position t) and kept in registers.
template <typename V, int LOGN, int STAGE = 0, bool END = (STAGE >= Geom<V, LOGN>::S)>
struct TwBases {
    using I = StageInfo<V, LOGN, STAGE>;
    V w[I::NB];
    TwBases<V, LOGN, STAGE + 1> next;
    __device__ __forceinline__ void load(const V* __restrict__ tw, int t)
    {
        if constexpr (I::TW) {
            const V* __restrict__ tws = tw + plan_tw_offset(LOGN, I::LEM, STAGE);
#pragma unroll
            for (int b = 0; b < I::B; ++b) {
                const int k = (t + b * Geom<V, LOGN>::T) & (I::NS - 1);
#pragma unroll
                for (int l = 0; l < I::LR; ++l) w[b * I::LR + l] = tws[l * I::NS + k];
            }
        }
        next.load(tw, t);
    }
    template <int Q> __device__ __forceinline__ const V* get() const
    {
        if constexpr (Q == STAGE) return w;
        else return next.template get<Q>();
    }
};
template <typename V, int LOGN, int STAGE> struct TwBases<V, LOGN, STAGE, true> {
    __device__ __forceinline__ void load(const V*, int) {}
};

// LDS layout of C interleaved transforms (line c of C): element `pos` of line
// c sits at f = pos C + c, slot f + floor(f / 2^PS) (one pad slot per 16 by
// default).  C = 1 is one transform.
//
// sync() orders the exchange: every thread's LDS writes of one stage before
// any read of the next, and every read before the next stage's writes.  With
// WAVE the threads sharing this region all sit in one wavefront (a row of at
// most 64 threads, rows never straddling waves), whose LDS instructions
// execute in issue order: a wavefront-scope fence keeps the compiler from
// moving LDS accesses across it and no workgroup barrier is needed.
template <typename V, int C, int PS = 4, bool WAVE = false> struct LdsLines {
    V* base;
    int c;
    __device__ __forceinline__ V* ptr(int pos) const
    {
        const int f = pos * C + c;
        return base + f + (f >> PS);
    }
    static constexpr int off(int dpos) { return lds_off(dpos * C, PS); }
    static constexpr int LINES = C;
    // LDS slots of C interleaved transforms of n points
    static constexpr int slots(int n) { return lds_padded(n * C, PS); }
    __device__ __forceinline__ static void sync()
    {
        if constexpr (WAVE) {
            __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
            __builtin_amdgcn_wave_barrier();
            __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
        } else {
            __syncthreads();
        }
    }
};

// u[r] *= w^r for r = 1 .. R-1, w^r built from the bases w^{2^l} (wb[l]).
template <int LR, typename V>
__device__ __forceinline__ void apply_stage_twiddles(V* u, const V* wb)
{
    constexpr int R = 1 << LR;
    V p[R];
    p[1] = wb[0];
#pragma unroll
    for (int l = 1; l < LR; ++l) {
        p[1 << l] = wb[l];
#pragma unroll
        for (int i = 1; i < (1 << l); ++i) p[(1 << l) + i] = cmul(p[i], wb[l]);
    }
#pragma unroll
    for (int r = 1; r < R; ++r) u[r] = cmul(u[r], p[r]);
}

// One Stockham stage on the registers of thread t.  Not the last stage:
// outputs go to LDS in the stage's output order.  Last stage: outputs stay in
// v (position t + i T in v[i]).
template <int LOGN, int STAGE, typename V, int E, typename TB, typename L>
__device__ __forceinline__ void fft_stage(V (&v)[E], int t, const TB& tb, const L& lds)
{
    static_assert(E == kE<V, LOGN>, "register array size");
    using G = Geom<V, LOGN>;
    using I = StageInfo<V, LOGN, STAGE>;
#pragma unroll
    for (int b = 0; b < I::B; ++b) {
        V u[I::R];
#pragma unroll
        for (int r = 0; r < I::R; ++r) u[r] = v[b + r * I::B];
        if constexpr (I::TW) apply_stage_twiddles<I::LR>(u, tb.template get<STAGE>() + b * I::LR);
        Dft<I::R>::run(u);
        if constexpr (I::LAST) {
#pragma unroll
            for (int r = 0; r < I::R; ++r) v[b + r * I::B] = u[r];
        } else {
            const int j = t + b * G::T;
            const int base = ((j >> I::LNS) << (I::LNS + I::LR)) + (j & (I::NS - 1));
            V* wp = lds.ptr(base);
#pragma unroll
            for (int r = 0; r < I::R; ++r) wp[L::off(r * I::NS)] = u[r];
        }
    }
}

template <int LOGN, int STAGE, typename V, int E, typename TB, typename L>
__device__ __forceinline__ void fft_stages_from(V (&v)[E], int t, const TB& tb, const L& lds)
{
    static_assert(E == kE<V, LOGN>, "register array size");
    using G = Geom<V, LOGN>;
    if constexpr (STAGE < G::S) {
        if constexpr (STAGE > 0) {
            L::sync();  // the previous stage's LDS writes are visible
            const V* rp = lds.ptr(t);
#pragma unroll
            for (int i = 0; i < G::E; ++i) v[i] = rp[L::off(i * G::T)];
            if constexpr (STAGE < G::S - 1) L::sync();  // all reads done before rewriting
        }
        fft_stage<LOGN, STAGE>(v, t, tb, lds);
        fft_stages_from<LOGN, STAGE + 1>(v, t, tb, lds);
    }
}

// Race and index check, compiled in with -DFFTMI_LDS_POISON (the same
// kernels, not a second path): before the first stage every slot of the LDS
// region the transform's threads share is set to NaN, so that a read of a
// slot the previous stage did not write -- a wrong index, or a missing
// barrier -- turns the output into NaN instead of a stale value.
template <int LOGN, typename V, typename L>
__device__ __forceinline__ void lds_poison(const L& lds, int t)
{
#ifdef FFTMI_LDS_POISON
    using G = Geom<V, LOGN>;
    using Rl = typename real_of<V>::type;
    if constexpr (G::S > 1) {
        constexpr int threads = G::T * L::LINES;
        const Rl nan = __builtin_nan("");
        for (int k = t * L::LINES + lds.c; k < L::slots(G::N); k += threads) lds.base[k] = V{nan, nan};
        L::sync();
    }
#else
    (void)lds;
    (void)t;
#endif
}

// Forward transform of N = 2^LOGN points held as v[i] = x[t + i T]; on return
// v[i] = X[t + i T].  Every thread of the workgroup must call it (barriers).
// If the caller reuses the LDS afterwards it must put a barrier first.
template <int LOGN, typename V, int E, typename TB, typename L>
__device__ __forceinline__ void fft_regs(V (&v)[E], int t, const TB& tb, const L& lds)
{
    static_assert(E == kE<V, LOGN>, "register array size");
    lds_poison<LOGN, V>(lds, t);
    fft_stages_from<LOGN, 0>(v, t, tb, lds);
}

// The same transform with the thread <-> (line, t) map changed at the first
// exchange: stage 0 runs on the registers of thread (line la.c, ta); the LDS
// exchange hands the data over, and the later stages run on thread (line
// lb.c, tb_t), which ends with v[i] = X[tb_t + i T] of line lb.c.  Every
// (line, t) pair must be held by exactly one thread under each map.  The
// twiddle bases `tb` must have been loaded for tb_t (stage 0 needs none).
// This lets a kernel load with lanes running across lines and store with
// lanes running along a line (or the reverse) at no extra LDS traffic.
template <int LOGN, typename V, int E, typename TB, typename LA, typename LB>
__device__ __forceinline__ void fft_regs_remap(V (&v)[E], int ta, const LA& la, int tb_t, const TB& tb,
                                               const LB& lb)
{
    static_assert(E == kE<V, LOGN>, "register array size");
    static_assert(Geom<V, LOGN>::S > 1, "a remap needs at least one exchange");
    lds_poison<LOGN, V>(la, ta);
    fft_stage<LOGN, 0>(v, ta, tb, la);
    fft_stages_from<LOGN, 1>(v, tb_t, tb, lb);
}

}  // namespace fftmi
