"""Every benchmark workload, at full size and in the very launch the benchmark
times (``bench.setup_workload``: same plan, buffers, workspace and stream),
against the fp64 oracle (GPU): every transform of the batch for the
power-of-two workloads; 64 sampled rows where the oracle's route is the O(N^2)
direct DFT (with 64 bins of each row for rows of 10^6 points); sampled
coefficients of the first and last pair against the schoolbook sum for the
polynomial products (every coefficient of every pair is compared bit for bit
with the oracle in test_gpu_polymul).

Two buffer sets are run, as the benchmark rotates them; the second holds a copy
of the same input and must give bit-identical output.  Bars: per-transform
relative RMS <= 1e-6 log2(size) for the float32 transforms, exact int64
coefficients (against the schoolbook sum) for the polynomial products."""
import numpy as np
import pytest
import torch

import bench
import fft_convolution_amd as fm
import oracle
from fft_convolution_amd import workloads as wl

from conftest import fft_tol, rel_rms_rows

pytestmark = pytest.mark.gpu


def _out(name, bufs, k):
    if name.startswith("c2cpl"):  # split planes: the complex result
        return torch.complex(bufs[k][2], bufs[k][3])
    return bufs[k][2] if name.startswith("polymul") else bufs[k][1]


@pytest.mark.parametrize("name", list(wl.WORKLOADS))
def test_bench_workload(dev, name):
    print("workload %s" % name, flush=True)
    step, info = bench.setup_workload(name, dev, fm, torch, sets=2)
    step(0)
    step(1)
    torch.cuda.synchronize()
    bufs = info["keep"][1]
    y0, y1 = _out(name, bufs, 0), _out(name, bufs, 1)
    assert torch.equal(y0, y1)
    spec = wl.WORKLOADS[name]
    oracle.set_threads(8)

    if name.startswith("polymul"):
        a, b = wl.workload_input(name)
        length = spec["length"]
        rng = np.random.default_rng(12345)
        ks = np.unique(np.concatenate([[0, 1, length - 1, length, 2 * length - 2],
                                       rng.integers(0, 2 * length - 1, 60)]))
        for p in (0, spec["batch"] - 1):
            want = oracle.schoolbook_sample(a[p:p + 1], b[p:p + 1], ks)[0]
            got = y0[p].cpu().numpy()[ks]
            assert np.array_equal(got, want), p
        return

    x = wl.workload_input(name)
    batch = spec["batch"]
    n = spec.get("n", 0)
    if name.startswith("c2c_n") and n & (n - 1):
        # lengths that are not powers of two: the oracle's route is the O(N^2)
        # direct DFT, so rows are sampled (64 of them), and for rows of 10^6
        # points 64 bins of each picked row, computed one by one
        picks = np.unique(np.concatenate([[0, batch - 1], np.random.default_rng(7).integers(0, batch, 62)]))
        got = y0[torch.from_numpy(picks).to(dev)].cpu().numpy()
        xs = x[picks]
        if n > 20000:
            ks = np.unique(np.concatenate([[0, 1, n // 2, n - 1], np.random.default_rng(n).integers(0, n, 60)]))
            ref = oracle.dft_sample(xs, ks)
            err = (np.sqrt(np.mean(np.abs(got[:, ks] - ref) ** 2, axis=1)) /
                   np.sqrt(np.mean(np.abs(ref) ** 2, axis=1)))
        else:
            err = rel_rms_rows(got, oracle.dft(xs))
        assert err.max() <= fft_tol(n), (name, err.max())
        return
    # power-of-two workloads: every transform of the batch, in chunks
    if name.startswith("c2c3d"):
        fn, size = oracle.fft3, spec["d"] * spec["h"] * spec["w"]
    elif name.startswith("c2c2d"):
        fn, size = oracle.fft2, spec["h"] * spec["w"]
    elif name.startswith("r2c2d"):
        fn, size = oracle.rfft2, spec["h"] * spec["w"]
    elif name.startswith("r2c"):
        fn, size = oracle.rfft, n
    else:
        fn, size = oracle.fft, n
    y_np = y0.cpu().numpy()
    chunk = max(1, (1 << 24) // size)
    worst = 0.0
    for r0 in range(0, batch, chunk):
        ref = fn(x[r0:r0 + chunk])
        got = y_np[r0:r0 + chunk]
        err = rel_rms_rows(got.reshape(got.shape[0], -1), ref.reshape(ref.shape[0], -1))
        worst = max(worst, float(err.max()))
    assert worst <= fft_tol(size), (name, worst)
