"""Seeded random cases across the routes (GPU): lengths, shapes and batches
drawn from a fixed seed rather than picked by hand, so that combinations no
listed case names are exercised too -- powers of two, 13-smooth lengths,
primes and arbitrary lengths for 1D transforms in both precisions (forward
and inverse), real rows of even and odd length (R2C and the C2R round trip),
and 2D images whose axes mix those kinds.  Each case prints its draw before
running, so a failure names it.

Oracle: the radix-2 FFT for powers of two, the direct DFT up to 8192 points,
sampled bins of the direct DFT (computed one by one) for longer rows; 2D
against the separable direct DFT.  Bar: per-transform relative RMS <=
1e-6 log2 N (complex64) / 1e-14 log2 N (complex128)."""
import numpy as np
import pytest
import torch

import fft_convolution_amd as fm
import oracle
from fft_convolution_amd import workloads as wl

from conftest import fft_tol, rel_rms_rows

pytestmark = pytest.mark.gpu

SMOOTH = (2, 3, 5, 7, 11, 13)


def _draw_length(rng, top):
    kind = int(rng.integers(0, 4))
    if kind == 0:  # a power of two
        return 1 << int(rng.integers(1, int(np.log2(top)) + 1)), "pow2"
    if kind == 1:  # 13-smooth, built from random prime factors
        n = 1
        while True:
            p = int(rng.choice(SMOOTH))
            if n * p > top:
                break
            n *= p
            if rng.random() < 0.15:
                break
        return max(n, 2), "smooth"
    n = int(rng.integers(2, top))
    if kind == 2:  # the next prime
        while any(n % q == 0 for q in range(2, int(n ** 0.5) + 1)):
            n += 1
        return n, "prime"
    return n, "any"


def _cases_1d(seed, count, top):
    rng = np.random.default_rng(seed)
    out = []
    for _ in range(count):
        n, kind = _draw_length(rng, top)
        batch = int(rng.integers(1, 4))
        out.append((n, kind, batch))
    return out


def _check_rows(y, x, n, inverse, tol, rng):
    if n & (n - 1) == 0:
        ref = oracle.fft(x, inverse=inverse)
        err = rel_rms_rows(y, ref)
    elif n <= 8192:
        err = rel_rms_rows(y, oracle.dft(x, inverse=inverse))
    else:
        ks = np.unique(np.concatenate([[0, 1, n // 2, n - 1], rng.integers(0, n, 44)]))
        ref = oracle.dft_sample(x, ks, inverse=inverse)
        err = np.sqrt(np.mean(np.abs(y[:, ks] - ref) ** 2, axis=1)) / np.sqrt(np.mean(np.abs(ref) ** 2, axis=1))
    assert err.max() <= tol, err.max()


@pytest.mark.parametrize("prec", [torch.complex64, torch.complex128])
@pytest.mark.parametrize("idx", range(24))
def test_random_c2c(dev, prec, idx):
    c128 = prec == torch.complex128
    n, kind, batch = _cases_1d(77 if c128 else 76, 24, 1 << 20)[idx]
    print("case c2c n=%d (%s) batch=%d %s" % (n, kind, batch, prec), flush=True)
    npdt = np.complex128 if c128 else np.complex64
    x_np = wl.batched_uniform(n, batch, seed=n % 1013, dtype=npdt)
    plan = fm.Plan(n, prec)
    x = torch.from_numpy(x_np).to(dev)
    oracle.set_threads(8)
    rng = np.random.default_rng(n)
    tol = fft_tol(n, c128)
    for inverse in (False, True):
        y = (plan.ifft(x) if inverse else plan.fft(x)).cpu().numpy()
        _check_rows(y, x_np, n, inverse, tol, rng)


@pytest.mark.parametrize("idx", range(16))
def test_random_real(dev, idx):
    rng = np.random.default_rng(78)
    draws = [(int(rng.integers(2, 1 << 17)), int(rng.integers(1, 4)), bool(rng.integers(0, 2))) for _ in range(16)]
    n, batch, c128 = draws[idx]
    if idx % 4 == 0:
        n = 1 << int(np.log2(n))  # some powers of two too
    dtype = torch.float64 if c128 else torch.float32
    print("case real n=%d batch=%d %s" % (n, batch, dtype), flush=True)
    x_np = wl.real_normal(n, batch, seed=n % 1013, dtype=np.float64 if c128 else np.float32)
    plan = fm.RealPlan(n, dtype)
    x = torch.from_numpy(x_np).to(dev)
    X = plan.rfft(x)
    tol = fft_tol(n, c128)
    oracle.set_threads(8)
    Xn = X.cpu().numpy()
    if n <= 8192 or n & (n - 1) == 0:
        assert rel_rms_rows(Xn, oracle.rfft(x_np)).max() <= tol
    else:
        ks = np.unique(np.concatenate([[0, 1, n // 2], np.random.default_rng(n).integers(0, n // 2 + 1, 40)]))
        ref = oracle.dft_sample(x_np.astype(np.float64), ks)
        err = np.sqrt(np.mean(np.abs(Xn[:, ks] - ref) ** 2, axis=1)) / np.sqrt(np.mean(np.abs(ref) ** 2, axis=1))
        assert err.max() <= tol, err.max()
    back = plan.irfft(X).cpu().numpy()
    assert rel_rms_rows(back, x_np).max() <= tol


@pytest.mark.parametrize("idx", range(12))
def test_random_2d(dev, idx):
    rng = np.random.default_rng(79)
    draws = []
    for _ in range(12):
        h, _ = _draw_length(rng, 600)
        w, _ = _draw_length(rng, 600)
        draws.append((h, w, int(rng.integers(1, 3)), bool(rng.integers(0, 2))))
    h, w, batch, c128 = draws[idx]
    prec = torch.complex128 if c128 else torch.complex64
    print("case 2d %dx%d batch=%d %s" % (h, w, batch, prec), flush=True)
    npdt = np.complex128 if c128 else np.complex64
    x_np = wl.batched_uniform(h * w, batch, seed=(h * w) % 1013, dtype=npdt).reshape(batch, h, w)
    plan = fm.Plan((h, w), prec)
    x = torch.from_numpy(x_np).to(dev)
    oracle.set_threads(8)
    tol = fft_tol(h * w, c128)
    for inverse in (False, True):
        y = (plan.ifft2(x) if inverse else plan.fft2(x)).cpu().numpy()
        ref = oracle.dftn(x_np, 2, inverse=inverse)
        err = rel_rms_rows(y.reshape(batch, -1), ref.reshape(batch, -1)).max()
        assert err <= tol, err
