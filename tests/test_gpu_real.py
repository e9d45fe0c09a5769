"""Transforms of real rows (R2C / C2R) against the fp64 oracle's rfft / irfft
(GPU).  N/2 within the one-kernel range runs the fused kernels; longer rows run
the N/2-point multi-pass transform plus the bin-pair pass.

Bar: per-row relative RMS <= 1e-6 log2 N (float32 rows) / 1e-14 log2 N
(float64 rows), the bound of the complex transform of the same length."""
import numpy as np
import pytest
import torch

import fft_convolution_amd as fm
import oracle
from fft_convolution_amd import workloads as wl

from conftest import fft_tol, rel_rms_rows

pytestmark = pytest.mark.gpu

F32_FUSED = [0, 1, 2, 3, 4, 5, 6, 7, 8, 9, 10, 11, 12, 13, 14, 15]
F64_FUSED = [0, 1, 2, 3, 4, 5, 8, 11, 12, 13, 14]


def _run(logn, batch, dtype, seed):
    n = 1 << logn
    print("case n=%d batch=%d %s" % (n, batch, np.dtype(dtype).name), flush=True)
    tdt = torch.float32 if dtype == np.float32 else torch.float64
    plan = fm.RealPlan(n, tdt)
    x_np = wl.real_normal(n, batch, seed=seed, dtype=dtype)
    x = torch.from_numpy(x_np).cuda()
    X = plan.rfft(x).cpu().numpy()
    tol = fft_tol(n, dtype == np.float64)
    ref = oracle.rfft(x_np)
    assert X.shape == (batch, n // 2 + 1)
    assert rel_rms_rows(X, ref).max() <= tol, rel_rms_rows(X, ref).max()
    # the inverse of an arbitrary half spectrum (DC / Nyquist imaginary parts ignored)
    cdt = np.complex64 if dtype == np.float32 else np.complex128
    S_np = wl.real_spectrum(n, batch, seed=seed + 1, dtype=cdt)
    y = plan.irfft(torch.from_numpy(S_np).cuda()).cpu().numpy()
    yref = oracle.irfft(S_np, n)
    assert y.shape == (batch, n)
    assert rel_rms_rows(y, yref).max() <= tol, rel_rms_rows(y, yref).max()
    # round trip
    back = plan.irfft(plan.rfft(x)).cpu().numpy()
    assert rel_rms_rows(back, x_np).max() <= tol
    return plan


@pytest.mark.parametrize("logn", F32_FUSED)
def test_real_fused_f32(dev, logn):
    plan = _run(logn, 3 if logn > 10 else 67, np.float32, 100 + logn)
    assert ("fused" in plan.describe()) == (logn >= 1)


@pytest.mark.parametrize("logn", F64_FUSED)
def test_real_fused_f64(dev, logn):
    plan = _run(logn, 3 if logn > 10 else 33, np.float64, 200 + logn)
    assert ("fused" in plan.describe()) == (logn >= 1)


@pytest.mark.parametrize("logn,batch", [(16, 3), (17, 2), (18, 2), (21, 1), (24, 1)])
def test_real_pairs_f32(dev, logn, batch):
    plan = _run(logn, batch, np.float32, 300 + logn)
    assert "pairs" in plan.describe()


@pytest.mark.parametrize("logn,batch", [(15, 3), (16, 2), (17, 1), (20, 1)])
def test_real_pairs_f64(dev, logn, batch):
    plan = _run(logn, batch, np.float64, 400 + logn)
    assert "pairs" in plan.describe()


@pytest.mark.parametrize("n", [64, 1 << 13, 1 << 16])
def test_real_closed_forms(dev, n):
    """cos(2 pi f t / N) -> N/2 at bin f; sin -> -i N/2; an impulse back from w^{3k}."""
    t = np.arange(n)
    plan = fm.RealPlan(n, torch.float64)
    for f in (0, 1, n // 4 + 3, n // 2):
        X = plan.rfft(torch.from_numpy(np.cos(2 * np.pi * f * t / n)[None, :]).cuda()).cpu().numpy()[0]
        want = np.zeros(n // 2 + 1, dtype=complex)
        want[f] = n if f in (0, n // 2) else n / 2
        assert np.abs(X - want).max() < 1e-9 * n
    k = np.arange(n // 2 + 1)
    imp = plan.irfft(torch.from_numpy(np.exp(-2j * np.pi * 3 * k / n)[None, :]).cuda()).cpu().numpy()[0]
    want = np.zeros(n)
    want[3] = 1.0
    assert np.abs(imp - want).max() < 1e-13


def test_real_every_row_at_full_size(dev):
    """The real-row workload (16384 rows of 8192 points) in the launch the
    benchmark times: every row against the oracle (in chunks of 2048 rows to
    bound host memory), then every row back through C2R."""
    spec = wl.WORKLOADS["r2c_n8192_b16384"]
    n, batch = spec["n"], spec["batch"]
    x_np = wl.real_normal(n, batch, seed=spec["seed"])
    x = torch.from_numpy(x_np).cuda()
    plan = fm.RealPlan(n, torch.float32)
    Xt = plan.rfft(x)
    X = Xt.cpu().numpy()
    back = plan.irfft(Xt).cpu().numpy()
    for r0 in range(0, batch, 2048):
        sl = slice(r0, r0 + 2048)
        assert rel_rms_rows(X[sl], oracle.rfft(x_np[sl])).max() <= fft_tol(n)
        assert rel_rms_rows(back[sl], x_np[sl]).max() <= fft_tol(n)


def test_real_errors_and_kinds(dev):
    n = 1 << 16
    rp = fm.RealPlan(n, torch.float32)
    x = torch.zeros(2, n, device=dev)
    X = torch.zeros(2, n // 2 + 1, dtype=torch.complex64, device=dev)
    ws = torch.empty(fm.fft_workspace_size(rp.handle, 2), dtype=torch.uint8, device=dev)
    assert ws.numel() == 2 * (n // 2) * 8
    with pytest.raises(fm.FFTError) as e:
        fm.fft_exec_r2c(rp.handle, x, X, 2, None)
    assert e.value.status == fm.FFT_ERR_WORKSPACE
    # out overlapping in
    with pytest.raises(fm.FFTError) as e:
        fm.fft_exec_r2c(rp.handle, x, x.data_ptr() + 8, 1, ws)
    assert e.value.status == fm.FFT_ERR_OVERLAP
    with pytest.raises(fm.FFTError) as e:
        fm.fft_exec_r2c(rp.handle, x.data_ptr() + 4, X, 1, ws)
    assert e.value.status == fm.FFT_ERR_ALIGN
    # plan kinds
    cp = fm.Plan(n, torch.complex64)
    with pytest.raises(fm.FFTError) as e:
        fm.fft_exec_r2c(cp.handle, x, X, 1, ws)
    assert e.value.status == fm.FFT_ERR_RANK
    with pytest.raises(fm.FFTError) as e:
        fm.fft_exec_c2c(rp.handle, fm.FFT_FORWARD, X, X, 1, ws)
    assert e.value.status == fm.FFT_ERR_RANK
    rp64 = fm.RealPlan(1024, torch.float64)
    a = torch.ones(1, 8, dtype=torch.int64, device=dev)
    c = torch.empty(1, 15, dtype=torch.int64, device=dev)
    with pytest.raises(fm.FFTError) as e:
        fm.fft_poly_mul(rp64.handle, a, 8, a, 8, c, 1)
    assert e.value.status == fm.FFT_ERR_RANK
    # batch 0 is a no-op; fused plans need no workspace
    fm.fft_exec_r2c(rp.handle, x, X, 0, None)
    assert fm.fft_workspace_size(fm.RealPlan(1 << 15, torch.float32).handle, 5) == 0
    assert fm.fft_workspace_size(fm.RealPlan(1 << 14, torch.float64).handle, 5) == 0
    assert fm.fft_workspace_size(fm.RealPlan(1 << 16, torch.float32).handle, 5) == 5 * (1 << 15) * 8
    assert fm.fft_workspace_size(fm.RealPlan(1 << 15, torch.float64).handle, 5) == 5 * (1 << 14) * 16
    # input untouched by both directions
    xr = torch.randn(3, 4096, device=dev)
    x0 = xr.clone()
    Y = fm.RealPlan(4096).rfft(xr)
    Y0 = Y.clone()
    fm.RealPlan(4096).irfft(Y)
    torch.cuda.synchronize()
    assert torch.equal(xr, x0) and torch.equal(Y, Y0)


# Even lengths that are not powers of two: the N/2-point complex plan by its
# route (mixed radix, 11 x 13, Bluestein fused and in passes, mixed-radix
# passes) plus the bin-pair pass.
@pytest.mark.parametrize("n,dtype,batch", [
    (6, np.float32, 5), (10, np.float32, 3), (12, np.float64, 4), (100, np.float32, 3), (1000, np.float32, 2),
    (2002, np.float32, 2), (2 * 1009, np.float32, 2), (20000, np.float32, 2), (2 * 10007, np.float32, 1),
    (1000, np.float64, 2), (2 * 1009, np.float64, 2), (20000, np.float64, 1)])
def test_real_even_lengths(dev, n, dtype, batch):
    print("case n=%d %s batch=%d" % (n, np.dtype(dtype).name, batch), flush=True)
    tdt = torch.float32 if dtype == np.float32 else torch.float64
    cdt = np.complex64 if dtype == np.float32 else np.complex128
    plan = fm.RealPlan(n, tdt)
    assert "pairs" in plan.describe()
    h = n // 2
    route = fm.fft_plan_query(1, [h], 0 if dtype == np.float32 else 1)
    size = n
    if "bluestein" in route:  # the tolerance of the convolution length
        m = 1
        while m < 2 * h - 1:
            m *= 2
        size = 2 * m
    tol = fft_tol(size, dtype == np.float64)
    oracle.set_threads(8)
    x_np = wl.real_normal(n, batch, seed=n % 997, dtype=dtype)
    x = torch.from_numpy(x_np).cuda()
    X = plan.rfft(x).cpu().numpy()
    assert X.shape == (batch, h + 1)
    assert rel_rms_rows(X, oracle.rfft(x_np)).max() <= tol
    S_np = wl.real_spectrum(n, batch, seed=n % 991, dtype=cdt)
    y = plan.irfft(torch.from_numpy(S_np).cuda()).cpu().numpy()
    assert rel_rms_rows(y, oracle.irfft(S_np, n)).max() <= tol
    back = plan.irfft(plan.rfft(x)).cpu().numpy()
    assert rel_rms_rows(back, x_np).max() <= tol


def _run_any(n, batch, dtype, seed):
    """Real rows of any length n against the oracle: forward, the inverse of
    an arbitrary half spectrum, and the round trip."""
    print("case real n=%d batch=%d %s" % (n, batch, np.dtype(dtype).name), flush=True)
    tdt = torch.float32 if dtype == np.float32 else torch.float64
    plan = fm.RealPlan(n, tdt)
    x_np = wl.real_normal(n, batch, seed=seed, dtype=dtype)
    x = torch.from_numpy(x_np).cuda()
    X = plan.rfft(x).cpu().numpy()
    tol = fft_tol(n, dtype == np.float64)
    assert X.shape == (batch, n // 2 + 1)
    cdt = np.complex64 if dtype == np.float32 else np.complex128
    S_np = wl.real_spectrum(n, batch, seed=seed + 1, dtype=cdt)
    S = torch.from_numpy(S_np).cuda()
    y = plan.irfft(S).cpu().numpy()
    if n <= 20000 or n & (n - 1) == 0:  # every output
        assert rel_rms_rows(X, oracle.rfft(x_np)).max() <= tol, rel_rms_rows(X, oracle.rfft(x_np)).max()
        yref = oracle.irfft(S_np, n)
        assert rel_rms_rows(y, yref).max() <= tol, rel_rms_rows(y, yref).max()
    else:  # the direct DFT is O(N^2): 64 outputs, each from the definition
        oracle.set_threads(8)
        rng = np.random.default_rng(n)
        ks = np.unique(np.concatenate([[0, 1, n // 2], rng.integers(0, n // 2 + 1, 61)]))
        ref = oracle.dft_sample(x_np.astype(np.float64), ks)
        err = np.sqrt(np.mean(np.abs(X[:, ks] - ref) ** 2, axis=1)) / np.sqrt(np.mean(np.abs(ref) ** 2, axis=1))
        assert err.max() <= tol, err.max()
        js = np.unique(np.concatenate([[0, n - 1], rng.integers(0, n, 62)]))
        yref = oracle.irfft_sample(S_np, n, js)
        err = np.sqrt(np.mean((y[:, js] - yref) ** 2, axis=1)) / np.sqrt(np.mean(yref ** 2, axis=1))
        assert err.max() <= tol, err.max()
    assert torch.equal(S.cpu(), torch.from_numpy(S_np))  # the C2R input is left as it was
    back = plan.irfft(plan.rfft(x)).cpu().numpy()
    assert rel_rms_rows(back, x_np).max() <= tol
    return plan


# odd lengths through each route of the N-point complex plan: mixed radix in
# one kernel (15, 105, 1001 = 7 11 13, 2187 = 3^7), mixed-radix passes
# (19683 = 3^9, 78125 = 5^7), chirp-z in one kernel (17, 97, 1009, 4097) and
# in passes (100003)
ODD = [(3, 5), (15, 7), (105, 3), (1001, 2), (2187, 2), (19683, 2), (78125, 1), (17, 9), (97, 4), (1009, 3),
       (4097, 2), (100003, 1)]


@pytest.mark.parametrize("n,batch", ODD)
def test_real_odd_lengths_f32(dev, n, batch):
    plan = _run_any(n, batch, np.float32, 300 + n % 97)
    assert "odd" in plan.describe()


@pytest.mark.parametrize("n,batch", [(3, 4), (45, 3), (1001, 2), (97, 3), (19683, 1)])
def test_real_odd_lengths_f64(dev, n, batch):
    _run_any(n, batch, np.float64, 400 + n % 89)


def test_real_odd_closed_form(dev):
    """A cosine of frequency 4 in a 15-point row: 15/2 at bin 4 and nothing
    else; and back."""
    n = 15
    t = np.arange(n)
    x = np.cos(2 * np.pi * ((4 * t) % n) / n)[None, :]
    plan = fm.RealPlan(n, torch.float64)
    X = plan.rfft(torch.from_numpy(x).cuda())
    want = np.zeros(n // 2 + 1, complex)
    want[4] = n / 2
    assert np.abs(X.cpu().numpy()[0] - want).max() < 1e-12
    assert np.abs(plan.irfft(X).cpu().numpy() - x).max() < 1e-13
