// radix_plan.hpp -- compile-time radix schedule shared by the host (twiddle
// tables) and the device (kernels).
//
// A transform of N = 2^LOGN points runs as a sequence of Stockham stages.
// The stage with radix R = 2^LR and input span Ns (the product of the radices
// before it) takes, for each butterfly j in [0, N/R):
//     inputs  x[j + r N/R],                      r = 0 .. R-1
//     twiddle w_{Ns R}^{r k}, k = j mod Ns,      (w_M = e^{-2 pi i / M})
//     an R-point DFT,
//     outputs y[(j / Ns) Ns R + k + r Ns].
// With R = 2 this is the stage of "Stockham FFT Butterfly Algorithm in
// Parallel GLSL" (section "Execution via GLSL Compute Shaders and Textures")
// written from the input side; larger R fuses log2 R of those radix-2 levels.
// After the last stage the output is in natural order (no bit reversal).
//
// Each thread owns E = 2^LOGE elements of a row (positions t + i T, T = N/E);
// a stage of radix R gives every thread E/R butterflies.
#pragma once

namespace fftmi {

// `lem` is log2 of the elements a thread holds for long rows: 4 (16) for
// complex64, 3 (8) for complex128, whose registers are twice as wide.
//
// log2 of elements per thread: rows up to 2^lem points live in one thread;
// with lem = 4, 8192 points use 32 per thread (three stages 32 x 16 x 16).
constexpr int plan_loge(int logn, int lem)
{
    return logn <= lem ? logn : (lem == 4 && logn == 13 ? 5 : lem);
}

constexpr int plan_nstages(int logn, int lem)
{
    return logn <= lem ? 1 : (lem == 4 && logn == 13 ? 3 : (logn + lem - 1) / lem);
}

// log2 of the radix of stage s.  Radix 2^lem first (the first stage needs no
// twiddles), the remainder last; 8192 = 32 x 16 x 16 with lem = 4.
constexpr int plan_stage_logr(int logn, int lem, int s)
{
    return logn <= lem ? logn
         : (lem == 4 && logn == 13) ? (s == 0 ? 5 : 4)
         : (s < logn / lem ? lem : logn % lem);
}

// log2 of Ns, the span of the sub-transforms a stage combines.
constexpr int plan_stage_lns(int logn, int lem, int s)
{
    int acc = 0;
    for (int q = 0; q < s; ++q) acc += plan_stage_logr(logn, lem, q);
    return acc;
}

// Twiddle table of stage s >= 1: the bases w_{Ns R}^{k 2^l} for l < log2 R and
// k < Ns, laid out [l][k] so that consecutive butterflies read consecutive
// entries.  A thread multiplies its R inputs by w^r = w_{Ns R}^{r k}, built as
// products of the bases over the set bits of r (at most log2 R factors, each
// read from the exactly rounded table).  Stage 0 has Ns = 1 and no table.
constexpr long plan_tw_offset(int logn, int lem, int s)
{
    long off = 0;
    for (int q = 1; q < s; ++q)
        off += (long)plan_stage_logr(logn, lem, q) << plan_stage_lns(logn, lem, q);
    return off;
}

constexpr long plan_tw_entries(int logn, int lem) { return plan_tw_offset(logn, lem, plan_nstages(logn, lem)); }

// lem for a plan precision (0 = complex64, 1 = complex128).
constexpr int plan_lem(int prec) { return prec == 0 ? 4 : 3; }

// LDS slots for `n` elements with one pad slot after every 16, which spreads
// the power-of-two strides of the stage writes over all banks.  The slot of
// element f is f + floor(f / 16); for every access the engine makes (a base
// f0 plus a delta that is a multiple of a power of two g with f0 mod 16 < g,
// or of 16) the slot of f0 + d is slot(f0) + lds_off(d), a compile-time
// constant, so the per-element LDS addresses cost no instructions.
//
// The row kernels may take one pad slot per 32 instead (ps = 5): the same
// argument holds with 32 in place of 16 for the accesses they make.
constexpr int lds_padded(int n, int ps = 4) { return n + (n >> ps); }
constexpr int lds_off(int d, int ps = 4) { return d + (d >> ps); }

}  // namespace fftmi
