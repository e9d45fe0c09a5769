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

// log2 of elements per thread: rows up to 16 points live in one thread;
// 8192 points use 32 per thread (three stages 32 x 16 x 16); the rest 16.
constexpr int plan_loge(int logn) { return logn <= 4 ? logn : (logn == 13 ? 5 : 4); }

constexpr int plan_nstages(int logn)
{
    return logn <= 4 ? 1 : (logn == 13 ? 3 : (logn + 3) / 4);
}

// log2 of the radix of stage s.  Radix 16 first (the first stage needs no
// twiddles), the remainder last; 8192 = 32 x 16 x 16.
constexpr int plan_stage_logr(int logn, int s)
{
    return logn <= 4 ? logn
         : logn == 13 ? (s == 0 ? 5 : 4)
         : (s < logn / 4 ? 4 : logn % 4);
}

// log2 of Ns, the span of the sub-transforms a stage combines.
constexpr int plan_stage_lns(int logn, int s)
{
    int acc = 0;
    for (int q = 0; q < s; ++q) acc += plan_stage_logr(logn, q);
    return acc;
}

// Offset (in complex entries) of stage s's table: stage s >= 1 holds
// (R - 1) Ns entries laid out [r - 1][k], so consecutive butterflies read
// consecutive entries.  Stage 0 has Ns = 1 and no table.
constexpr long plan_tw_offset(int logn, int s)
{
    long off = 0;
    for (int q = 1; q < s; ++q)
        off += (long)((1 << plan_stage_logr(logn, q)) - 1) << plan_stage_lns(logn, q);
    return off;
}

constexpr long plan_tw_entries(int logn) { return plan_tw_offset(logn, plan_nstages(logn)); }

// LDS slots for `n` elements with one pad slot after every 16, which spreads
// the power-of-two strides of the stage writes over all banks.
constexpr int lds_padded(int n) { return n + (n >> 4); }

}  // namespace fftmi
