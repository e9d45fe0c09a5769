"""Every benchmark workload, at full size and in the very launch the benchmark
times (``bench.setup_workload``: same plan, buffers, workspace and stream),
against the fp64 oracle on sampled outputs (GPU).

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
    picks = sorted({0, batch // 2, batch - 1})
    got = y0[picks].cpu().numpy()
    xs = x[picks]
    if name.startswith("c2c3d"):
        ref, size = oracle.fft3(xs), spec["d"] * spec["h"] * spec["w"]
    elif name.startswith("c2c2d"):
        ref, size = oracle.fft2(xs), spec["h"] * spec["w"]
    elif name.startswith("r2c2d"):
        ref, size = oracle.rfft2(xs), spec["h"] * spec["w"]
    elif name.startswith("r2c"):
        ref, size = oracle.rfft(xs), spec["n"]
    else:
        n = spec["n"]
        if n > 20000 and n & (n - 1):
            # 64 bins of each picked row, relative to the row spectrum's RMS
            ks = np.unique(np.concatenate([[0, 1, n // 2, n - 1], np.random.default_rng(n).integers(0, n, 60)]))
            ref = oracle.dft_sample(xs, ks)
            err = (np.sqrt(np.mean(np.abs(got[:, ks] - ref) ** 2, axis=1)) /
                   np.sqrt(np.mean(np.abs(got) ** 2, axis=1)))
            assert err.max() <= fft_tol(n), (name, err)
            return
        ref, size = (oracle.fft(xs) if n & (n - 1) == 0 else oracle.dft(xs)), n
    err = rel_rms_rows(got.reshape(len(picks), -1), ref.reshape(len(picks), -1))
    assert err.max() <= fft_tol(size), (name, err)
