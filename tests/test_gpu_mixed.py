"""Lengths N = 2^a 3^b 5^c 7^d that are not powers of two, within one
workgroup's LDS (8192 points complex64, 4096 complex128): the mixed-radix
Stockham kernel, against the fp64 oracle's direct DFT (GPU).

Bar: per-row relative RMS <= 1e-6 log2 N (complex64) / 1e-14 log2 N
(complex128), the bound of the power-of-two transforms."""
import numpy as np
import pytest
import torch

import fft_convolution_amd as fm
import oracle
from fft_convolution_amd import workloads as wl

from conftest import fft_tol, rel_rms_rows

pytestmark = pytest.mark.gpu

F32 = [3, 5, 6, 7, 11, 12, 13, 15, 30, 49, 60, 100, 105, 143, 210, 343, 360, 1000, 1001, 1331, 2187, 2197, 2401,
       3125, 6000, 6144, 7168, 8000, 8008]
F64 = [3, 11, 12, 13, 100, 105, 1000, 1001, 2187, 2401, 3000, 3072, 4000, 4095]


def _radices(desc):
    return [int(r) for r in desc.split("radices=")[1].split()[0].split("x")]


def _check(n, batch, dtype, seed):
    print("case n=%d batch=%d %s" % (n, batch, dtype), flush=True)
    npdt = np.complex64 if dtype == torch.complex64 else np.complex128
    x_np = wl.batched_uniform(n, batch, seed=seed, dtype=npdt)
    plan = fm.Plan(n, dtype)
    desc = plan.describe()
    assert "path=mixed" in desc
    assert int(np.prod(_radices(desc))) == n
    x = torch.from_numpy(x_np).cuda()
    tol = fft_tol(n, dtype == torch.complex128)
    y = plan.fft(x).cpu().numpy()
    assert rel_rms_rows(y, oracle.dft(x_np)).max() <= tol
    z = plan.ifft(x).cpu().numpy()
    assert rel_rms_rows(z, oracle.dft(x_np, inverse=True)).max() <= tol
    back = plan.ifft(plan.fft(x)).cpu().numpy()
    assert rel_rms_rows(back, x_np).max() <= tol


@pytest.mark.parametrize("n", F32)
def test_mixed_f32(dev, n):
    _check(n, 67 if n <= 360 else 3, torch.complex64, n)


@pytest.mark.parametrize("n", F64)
def test_mixed_f64(dev, n):
    _check(n, 33 if n <= 360 else 2, torch.complex128, n + 1)


def test_mixed_closed_forms_and_in_place(dev):
    """A single tone e^{2 pi i f t / N} gives N at bin f; an impulse at m gives
    w^{mk}; in place equals out of place."""
    n = 1260  # 4 * 3^2 * 5 * 7
    t = np.arange(n)
    plan = fm.Plan(n, torch.complex128)
    for f in (0, 1, 419, n - 1):
        # the phase from (f t) mod N, reduced in integers (exact input tone)
        tone = np.exp(2j * np.pi * ((f * t) % n) / n)
        y = plan.fft(torch.from_numpy(tone[None, :]).cuda()).cpu().numpy()[0]
        want = np.zeros(n, dtype=complex)
        want[f] = n
        assert np.abs(y - want).max() < 1e-10
    m = 5
    imp = np.zeros((1, n), dtype=np.complex128)
    imp[0, m] = 1
    y = plan.fft(torch.from_numpy(imp).cuda()).cpu().numpy()[0]
    assert np.abs(y - np.exp(-2j * np.pi * ((m * t) % n) / n)).max() < 1e-13
    x = torch.from_numpy(wl.batched_normal(n, 9, seed=3, dtype=np.complex128)).cuda()
    ref = plan.fft(x)
    xx = x.clone()
    plan.fft(xx, out=xx)
    torch.cuda.synchronize()
    assert torch.equal(xx, ref)


def test_mixed_range_limits(dev):
    # beyond one workgroup's LDS: super-stage passes; a prime factor above
    # 13: Bluestein
    assert "mixpass" in fm.Plan(3 * 4096, torch.complex64).describe()
    assert "mixpass" in fm.Plan(3 * 2048, torch.complex128).describe()
    assert "bluestein" in fm.Plan(17 * 64, torch.complex64).describe()
    assert "mixed" in fm.Plan(11 * 13 * 32, torch.complex64).describe()
    assert "mixed" in fm.Plan(3 * 2048, torch.complex64).describe()
    # a large batch of short rows (many rows per workgroup, ragged last group)
    n, batch = 12, 100003
    x_np = wl.batched_uniform(n, batch, seed=8)
    y = fm.Plan(n).fft(torch.from_numpy(x_np).cuda()).cpu().numpy()
    assert rel_rms_rows(y, oracle.dft(x_np)).max() <= fft_tol(n)


def _smooth13(limit):
    out = []
    for n in range(3, limit + 1):
        m = n
        for p in (2, 3, 5, 7, 11, 13):
            while m % p == 0:
                m //= p
        if m == 1 and n & (n - 1):
            out.append(n)
    return out


@pytest.mark.parametrize("dtype,limit", [(torch.complex64, 8192), (torch.complex128, 4096)])
def test_mixed_every_smooth_length(dev, dtype, limit):
    """Every length 2^a 3^b 5^c 7^d 11^e 13^f (not a power of two) in the
    mixed-radix range: two rows, forward and inverse, against the direct DFT
    (all bins up to 2048 points, 48 bins spread over the spectrum beyond)."""
    npdt = np.complex64 if dtype == torch.complex64 else np.complex128
    oracle.set_threads(8)
    bad = []
    for n in _smooth13(limit):
        plan = fm.Plan(n, dtype)
        assert "path=mixed" in plan.describe(), n
        x_np = wl.batched_uniform(n, 2, seed=7000 + n, dtype=npdt)
        x = torch.from_numpy(x_np).cuda()
        ks = None if n <= 2048 else np.unique(np.linspace(0, n - 1, 48).astype(np.int64))
        tol = fft_tol(n, dtype == torch.complex128)
        for inverse in (False, True):
            y = (plan.ifft(x) if inverse else plan.fft(x)).cpu().numpy()
            if ks is None:
                ref = oracle.dft(x_np, inverse=inverse)
            else:
                y, ref = y[:, ks], oracle.dft_sample(x_np, ks, inverse=inverse)
            err = rel_rms_rows(y, ref).max()
            if not err <= tol:
                bad.append((n, inverse, float(err)))
    assert not bad, bad


# Beyond one kernel: 2-3 mixed-radix super-stage passes, radices from 50 to
# 1024 in both precisions (each tile width and LDS class of the pass kernel:
# radix <= 64, <= 256, <= 512, and the wide class up to 1024 where it saves a
# pass: 10^6 = 1000 1000, 3 2^18 = 1024 768; 1001000 = 7 11 13 ... keeps its
# radices within 512 and takes three).
MIXPASS = [(9000, torch.complex64, 3), (10000, torch.complex64, 2), (12288, torch.complex64, 2),
           (30030, torch.complex64, 2), (60060, torch.complex64, 1), (3 * 65536, torch.complex64, 1),
           (10 ** 6, torch.complex64, 1), (3 << 20, torch.complex64, 1), (6000, torch.complex128, 3),
           (4608, torch.complex128, 3), (5000, torch.complex128, 2), (10000, torch.complex128, 2),
           (30030, torch.complex128, 1), (3 * 65536, torch.complex128, 1), (5 ** 9, torch.complex128, 1),
           (8 * 10 ** 6, torch.complex64, 1), (3 << 18, torch.complex64, 1), (3 << 18, torch.complex128, 1),
           (10 ** 6, torch.complex128, 1), (1001000, torch.complex64, 1)]


@pytest.mark.parametrize("n,dtype,batch", MIXPASS)
def test_mixpass(dev, n, dtype, batch):
    """Forward and inverse against the direct DFT (every bin up to 20000
    points, 64 bins beyond, relative to the spectrum's RMS), the round trip,
    and in place equal to out of place."""
    print("case n=%d %s batch=%d" % (n, dtype, batch), flush=True)
    npdt = np.complex64 if dtype == torch.complex64 else np.complex128
    plan = fm.Plan(n, dtype)
    assert "path=mixpass" in plan.describe()
    x_np = wl.batched_normal(n, batch, seed=n % 1009, dtype=npdt)
    x = torch.from_numpy(x_np).to(dev)
    tol = fft_tol(n, dtype == torch.complex128)
    oracle.set_threads(8)
    ks = None if n <= 20000 else np.unique(np.concatenate(
        [[0, 1, n // 2, n - 1], np.random.default_rng(n).integers(0, n, 60)]))
    for inverse in (False, True):
        y = (plan.ifft(x) if inverse else plan.fft(x)).cpu().numpy()
        if ks is None:
            err = rel_rms_rows(y, oracle.dft(x_np, inverse=inverse)).max()
        else:
            ref = oracle.dft_sample(x_np, ks, inverse=inverse)
            err = (np.sqrt(np.mean(np.abs(y[:, ks] - ref) ** 2, axis=1)) /
                   np.sqrt(np.mean(np.abs(ref) ** 2, axis=1))).max()
        assert err <= tol, (inverse, err)
    back = plan.ifft(plan.fft(x)).cpu().numpy()
    assert rel_rms_rows(back, x_np).max() <= tol
    z = x.clone()
    plan.fft(z, out=z)
    ref = plan.fft(x)
    torch.cuda.synchronize()
    assert torch.equal(z, ref)


def test_mixpass_needs_workspace_and_sizes_poly_mul(dev):
    n, batch = 10000, 2
    plan = fm.Plan(n, torch.complex64)
    assert fm.fft_workspace_size(plan.handle, batch) == batch * n * 8
    x = torch.zeros(batch, n, dtype=torch.complex64, device=dev)
    with pytest.raises(fm.FFTError) as e:
        fm.fft_exec_c2c(plan.handle, fm.FFT_FORWARD, x, torch.empty_like(x), batch, None)
    assert e.value.status == fm.FFT_ERR_WORKSPACE
    p64 = fm.Plan(n, torch.complex128)  # poly-mul: z (N complex128) and the plan's own workspace
    # z, the plan's own workspace, 520 bytes per pair for the exponent balance
    assert fm.fft_poly_mul_workspace_size(p64.handle, 1) == n * 16 + fm.fft_workspace_size(p64.handle, 1) + 520
