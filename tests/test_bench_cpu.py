"""The benchmark's CPU baseline leg (the oracle on a bounded sample of a
workload) for each oracle route of the 1D workloads: the radix-2 FFT for
power-of-two rows, the direct DFT for other rows, and a bounded set of direct
DFT bins for rows too long for an O(N^2) pass.  CPU only, small budgets."""
import math

import numpy as np
import pytest

import bench
from fft_convolution_amd import workloads as wl


@pytest.mark.parametrize("n,batch,fn", [(1024, 64, "fft"), (1000, 64, "dft"), (10 ** 6, 2, "dft_bins")])
def test_cpu_baseline_routes(n, batch, fn):
    x = wl.batched_normal(n, batch, seed=5)
    info = dict(n=n, batch=batch, sample_rows=lambda rows: x[:rows], oracle_fn=fn,
                oracle_unit=5.0 * n * math.log2(n))
    out = bench.cpu_baseline("c2c_n%d_b%d" % (n, batch), info, 0.2)
    assert out["kind"] == "oracle" and out["unit"] == "GFLOP/s" and out["cores"] >= 1
    assert np.isfinite(out["value"]) and out["value"] > 0
    assert ("bins" in out["sample"]) == (fn == "dft_bins")
