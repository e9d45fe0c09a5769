"""Parity of the 1D HIP path with the fp64 oracle (GPU).

Bar: per-transform relative RMS error <= 1e-6 log2 N for complex64
(1e-14 log2 N for complex128) against the oracle on identical inputs."""
import math

import numpy as np
import pytest
import torch

import fft_convolution_amd as fm
import oracle
from fft_convolution_amd import workloads as wl

from conftest import fft_tol, rel_rms_rows

pytestmark = pytest.mark.gpu


def _run(plan, x_np, dev, inverse=False):
    x = torch.from_numpy(x_np).to(dev)
    y = plan.ifft(x) if inverse else plan.fft(x)
    torch.cuda.synchronize()
    return y.cpu().numpy()


def _case(n, batch, dtype, seed):
    print("case n=%d batch=%d dtype=%s seed=%d" % (n, batch, dtype.__name__, seed), flush=True)
    return wl.batched_uniform(n, batch, seed, dtype=dtype)


@pytest.mark.parametrize("logn", list(range(0, 15)))  # to 16384: one 1024-thread workgroup a row
@pytest.mark.parametrize("batch", [1, 3, 67])
def test_c2c_c64_sweep(dev, logn, batch):
    n = 1 << logn
    x = _case(n, batch, np.complex64, 100 + logn)
    plan = fm.Plan(n, torch.complex64)
    for inverse in (False, True):
        y = _run(plan, x, dev, inverse)
        ref = oracle.fft(x, inverse=inverse)
        err = rel_rms_rows(y, ref)
        assert err.max() <= fft_tol(n), (inverse, err.max())


@pytest.mark.parametrize("logn", list(range(0, 14)))  # to 8192: one 1024-thread workgroup a row
@pytest.mark.parametrize("batch", [1, 5])
def test_c2c_c128_sweep(dev, logn, batch):
    n = 1 << logn
    x = _case(n, batch, np.complex128, 200 + logn)
    plan = fm.Plan(n, torch.complex128)
    for inverse in (False, True):
        y = _run(plan, x, dev, inverse)
        ref = oracle.fft(x, inverse=inverse)
        assert rel_rms_rows(y, ref).max() <= fft_tol(n, True)


# every multi-pass size below the largest (2^26, test_gpu_max_sizes): each
# has its own split into super-stages (2 passes up to 2^18, 3 beyond); the
# 2^14-point passes run under the chirp-z route (test_gpu_bluestein)
@pytest.mark.parametrize("logn,batch", [(15, 3), (16, 1), (17, 2), (18, 2), (19, 1), (20, 1), (21, 1),
                                        (22, 1), (23, 1), (25, 1)])
def test_c2c_c64_multipass(dev, logn, batch):
    n = 1 << logn
    x = _case(n, batch, np.complex64, 300 + logn)
    plan = fm.Plan(n, torch.complex64)
    assert "multipass" in plan.describe()
    for inverse in (False, True):
        y = _run(plan, x, dev, inverse)
        ref = oracle.fft(x, inverse=inverse)
        assert rel_rms_rows(y, ref).max() <= fft_tol(n)


@pytest.mark.parametrize("logn,batch", [(14, 1), (15, 2), (16, 3), (17, 1), (18, 1), (19, 1), (20, 1),
                                        (21, 1), (22, 1), (23, 1)])
def test_c2c_c128_multipass(dev, logn, batch):
    n = 1 << logn
    x = _case(n, batch, np.complex128, 400 + logn)
    plan = fm.Plan(n, torch.complex128)
    assert "multipass" in plan.describe()
    for inverse in (False, True):
        y = _run(plan, x, dev, inverse)
        ref = oracle.fft(x, inverse=inverse)
        assert rel_rms_rows(y, ref).max() <= fft_tol(n, True)


def test_workload_n1024_b64_forward_and_round_trip(dev):
    # 1024 points x 64 rows, uniform [-1, 1), seed 1: forward against the
    # oracle, then the inverse of the GPU's own output back to the input.
    x_np = wl.workload_input("c2c_n1024_b64")
    plan = fm.Plan(1024, torch.complex64)
    x = torch.from_numpy(x_np).to(dev)
    X = plan.fft(x)
    back = plan.ifft(X)
    torch.cuda.synchronize()
    assert rel_rms_rows(X.cpu().numpy(), oracle.fft(x_np)).max() <= fft_tol(1024)
    assert rel_rms_rows(back.cpu().numpy(), x_np).max() <= fft_tol(1024)


def test_workload_n4096_b16384_every_row(dev):
    # The full 16384 x 4096 batch in the launch the benchmark times; every row
    # against the oracle (in chunks of 2048 rows to bound host memory), and
    # every row must also satisfy Parseval.
    x_np = wl.workload_input("c2c_n4096_b16384")
    plan = fm.Plan(4096, torch.complex64)
    x = torch.from_numpy(x_np).to(dev)
    y = torch.empty_like(x)
    fm.fft_exec_c2c(plan.handle, fm.FFT_FORWARD, x, y, 16384, None)
    torch.cuda.synchronize()
    y_np = y.cpu().numpy()
    worst = 0.0
    for r0 in range(0, 16384, 2048):
        err = rel_rms_rows(y_np[r0:r0 + 2048], oracle.fft(x_np[r0:r0 + 2048]))
        assert err.shape == (2048,)
        worst = max(worst, float(err.max()))
    assert worst <= fft_tol(4096), worst
    ex = (x.abs() ** 2).sum(dim=1).double()
    ey = (y.abs() ** 2).sum(dim=1).double() / 4096
    assert float(((ey - ex).abs() / ex).max()) < 1e-5


def test_workload_n2p24_b1(dev):
    n = 1 << 24
    x_np = wl.workload_input("c2c_n16777216_b1")
    plan = fm.Plan(n, torch.complex64)
    y = _run(plan, x_np, dev)
    assert rel_rms_rows(y, oracle.fft(x_np)).max() <= fft_tol(n)


@pytest.mark.parametrize("n", [4096, 1 << 16])
def test_in_place_equals_out_of_place_and_deterministic(dev, n):
    x_np = wl.batched_normal(n, 4, seed=7)
    plan = fm.Plan(n, torch.complex64)
    x = torch.from_numpy(x_np).to(dev)
    y1 = plan.fft(x)
    y2 = plan.fft(x)
    z = x.clone()
    plan.fft(z, out=z)
    torch.cuda.synchronize()
    assert torch.equal(y1, y2)
    assert torch.equal(y1, z)
    assert torch.equal(x, torch.from_numpy(x_np).to(dev))  # input untouched out of place


def test_closed_form_tone_and_delta(dev):
    n = 4096
    k = np.arange(n)
    x = np.zeros((3, n), np.complex64)
    x[0, 0] = 1
    x[1] = np.exp(2j * np.pi * ((37 * k) % n) / n)
    x[2, 5] = 1
    plan = fm.Plan(n, torch.complex64)
    y = _run(plan, x, dev)
    assert np.allclose(y[0], 1, atol=1e-6)
    ref = np.zeros(n, complex)
    ref[37] = n
    assert np.max(np.abs(y[1] - ref)) < 1e-6 * n
    assert np.allclose(y[2], np.exp(-2j * np.pi * ((5 * k) % n) / n), atol=1e-6)
