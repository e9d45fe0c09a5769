"""The largest transforms each path accepts, against the fp64 oracle (GPU):
complex 2^26 points (complex64) / 2^24 (complex128), every output; Bluestein
at 2^23 - 1 points (M = 2^24), sampled bins by the direct DFT; real rows of
2^27 / 2^25 points, every bin; plus round trips.  Sizes one past each limit
are rejected before any device work."""
import numpy as np
import pytest
import torch

import fft_convolution_amd as fm
import oracle
from fft_convolution_amd import workloads as wl

from conftest import fft_tol, rel_rms_rows

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("logn,dtype", [(26, torch.complex64), (24, torch.complex128)])
def test_max_power_of_two(dev, logn, dtype):
    n = 1 << logn
    print("case n=2^%d %s" % (logn, dtype), flush=True)
    npdt = np.complex64 if dtype == torch.complex64 else np.complex128
    x_np = wl.batched_uniform(n, 1, seed=logn, dtype=npdt)
    plan = fm.Plan(n, dtype)
    x = torch.from_numpy(x_np).to(dev)
    X = plan.fft(x)
    tol = fft_tol(n, dtype == torch.complex128)
    assert rel_rms_rows(X.cpu().numpy(), oracle.fft(x_np)).max() <= tol
    assert rel_rms_rows(plan.ifft(X).cpu().numpy(), x_np).max() <= tol
    with pytest.raises(fm.FFTError) as e:
        fm.Plan(2 * n, dtype)
    assert e.value.status == fm.FFT_ERR_UNSUPPORTED_SIZE


@pytest.mark.parametrize("dtype", [torch.complex64, torch.complex128])
def test_max_bluestein(dev, dtype):
    n = (1 << 23) - 1  # 47 * 178481
    print("case n=%d %s" % (n, dtype), flush=True)
    npdt = np.complex64 if dtype == torch.complex64 else np.complex128
    x_np = wl.batched_normal(n, 1, seed=23, dtype=npdt)
    plan = fm.Plan(n, dtype)
    assert "bluestein m=16777216" in plan.describe()
    x = torch.from_numpy(x_np).to(dev)
    X = plan.fft(x)
    Xn = X.cpu().numpy()
    ks = np.unique(np.concatenate([[0, 1, n // 2, n - 1], np.random.default_rng(5).integers(0, n, 20)]))
    ref = oracle.dft_sample(x_np, ks)
    # relative RMS over the sampled bins, against the reference's own RMS there
    err = np.sqrt(np.mean(np.abs(Xn[:, ks] - ref) ** 2)) / np.sqrt(np.mean(np.abs(ref) ** 2))
    assert err <= fft_tol(n, dtype == torch.complex128)
    assert rel_rms_rows(plan.ifft(X).cpu().numpy(), x_np).max() <= fft_tol(n, dtype == torch.complex128)
    with pytest.raises(fm.FFTError) as e:
        fm.Plan((1 << 23) + 1, dtype)
    assert e.value.status == fm.FFT_ERR_UNSUPPORTED_SIZE


@pytest.mark.parametrize("logn,dtype", [(27, torch.float32), (25, torch.float64)])
def test_max_real(dev, logn, dtype):
    n = 1 << logn
    print("case real n=2^%d %s" % (logn, dtype), flush=True)
    npdt = np.float32 if dtype == torch.float32 else np.float64
    x_np = wl.real_normal(n, 1, seed=logn, dtype=npdt)
    plan = fm.RealPlan(n, dtype)
    assert "pairs" in plan.describe()
    x = torch.from_numpy(x_np).to(dev)
    X = plan.rfft(x)
    tol = fft_tol(n, dtype == torch.float64)
    assert rel_rms_rows(X.cpu().numpy(), oracle.rfft(x_np)).max() <= tol
    assert rel_rms_rows(plan.irfft(X).cpu().numpy(), x_np).max() <= tol
    with pytest.raises(fm.FFTError) as e:
        fm.RealPlan(2 * n, dtype)
    assert e.value.status == fm.FFT_ERR_UNSUPPORTED_SIZE
