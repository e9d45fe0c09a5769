"""Exec calls inside a captured HIP graph, and on concurrent streams (GPU).

The exec entry points only enqueue kernels (and a device-to-device copy for
N = 1), so a caller can capture them: every replay must equal the eager
result, with the caller's own eager work and synchronisations between
replays.  Plans on two streams at the default priority run concurrently and
each must equal its eager result."""
import numpy as np
import pytest
import torch

import fft_convolution_amd as fm
from fft_convolution_amd import workloads as wl

pytestmark = pytest.mark.gpu


def _ws(nbytes, dev):
    return torch.empty(nbytes, dtype=torch.uint8, device=dev) if nbytes else None


def test_graph_replays_equal_eager(dev):
    cases = []
    # one-kernel rows, multi-pass, 2D fold, Bluestein, mixed radix (11 x 13 too), N = 1 copy
    for dims, dtype in (((4096,), torch.complex64), ((1 << 20,), torch.complex64), ((2048, 256), torch.complex64),
                        ((1009,), torch.complex64), ((1001,), torch.complex64), ((10 ** 6,), torch.complex64), ((1000, 60), torch.complex64), ((360,), torch.complex128), ((1,), torch.complex64)):
        n = int(np.prod(dims))
        batch = max(1, (1 << 20) // n)
        npdt = np.complex64 if dtype == torch.complex64 else np.complex128
        x = torch.from_numpy(wl.batched_uniform(n, batch, seed=n % 89, dtype=npdt).reshape((batch,) + dims)).to(dev)
        plan = fm.Plan(dims, dtype)
        y = torch.empty_like(x)
        ws = _ws(fm.fft_workspace_size(plan.handle, batch), dev)
        fn = {1: fm.fft_exec_c2c, 2: fm.fft_exec_2d, 3: fm.fft_exec_3d}[len(dims)]
        cases.append((plan, fn, x, y, ws, batch))
    # poly-mul (four-step) and R2C
    a_np, b_np = wl.random_polys(5000, 3, seed=5)
    a, b = torch.from_numpy(a_np).to(dev), torch.from_numpy(b_np).to(dev)
    pp = fm.Plan(16384, torch.complex128)
    c = torch.empty(3, 9999, dtype=torch.int64, device=dev)
    pws = _ws(fm.fft_poly_mul_workspace_size(pp.handle, 3), dev)
    resid = torch.empty(1, dtype=torch.float64, device=dev)
    rp = fm.RealPlan(8192)
    xr = torch.randn(64, 8192, device=dev)
    yr = torch.empty(64, 4097, dtype=torch.complex64, device=dev)

    s = torch.cuda.Stream()

    def work(stream):
        for plan, fn, x, y, ws, batch in cases:
            fn(plan.handle, fm.FFT_FORWARD, x, y, batch, ws, stream)
        fm.fft_poly_mul(pp.handle, a, 5000, b, 5000, c, 3, pws, resid, stream)
        fm.fft_exec_r2c(rp.handle, xr, yr, 64, None, stream)

    # eager reference
    with torch.cuda.stream(s):
        work(s.cuda_stream)
    torch.cuda.synchronize()
    ref = [case[3].clone() for case in cases]
    ref_c, ref_r = c.clone(), yr.clone()

    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        work(s.cuda_stream)
    torch.cuda.synchronize()
    for rep in range(4):
        for (_, _, _, y, _, _) in cases:
            y.zero_()
        c.zero_()
        yr.zero_()
        torch.cuda.synchronize()
        junk = torch.randn(1 << 20, device=dev).sum()   # eager work between replays
        g.replay()
        torch.cuda.synchronize()
        assert float(junk) == float(junk)
        for r, (plan, _, _, y, _, _) in zip(ref, cases):
            assert torch.equal(y, r), (rep, plan.describe())
        assert torch.equal(c, ref_c) and torch.equal(yr, ref_r), rep


def test_two_streams_concurrently(dev):
    n1, b1 = 4096, 2048
    n2 = 1 << 20
    x1 = torch.randn(b1, n1, dtype=torch.complex64, device=dev)
    x2 = torch.randn(1, n2, dtype=torch.complex64, device=dev)
    p1, p2 = fm.Plan(n1), fm.Plan(n2)
    ws2 = _ws(fm.fft_workspace_size(p2.handle, 1), dev)
    r1, r2 = p1.fft(x1), torch.empty_like(x2)
    fm.fft_exec_c2c(p2.handle, 0, x2, r2, 1, ws2)
    torch.cuda.synchronize()
    sa, sb = torch.cuda.Stream(), torch.cuda.Stream()
    y1, y2 = torch.empty_like(x1), torch.empty_like(x2)
    ws2b = _ws(fm.fft_workspace_size(p2.handle, 1), dev)
    for _ in range(5):
        fm.fft_exec_c2c(p1.handle, 0, x1, y1, b1, None, sa.cuda_stream)
        fm.fft_exec_c2c(p2.handle, 0, x2, y2, 1, ws2b, sb.cuda_stream)
    torch.cuda.synchronize()
    assert torch.equal(y1, r1) and torch.equal(y2, r2)
