"""The kernels built with -DFFTMI_LDS_POISON (libfftmi_poison.so): every LDS
region is set to NaN before a transform's first stage, so a read of a slot
the previous stage did not write -- a wrong exchange index, or a missing
barrier -- shows up as NaN in the output (GPU).

Each case runs through the normal library and through the poisoned one in the
same process; the outputs must be bit-identical (the fill changes nothing a
correct kernel reads) and free of NaN, and the 1D rows also match the oracle.
Covered: the row kernels (every power of two, both precisions, wave-scope and
workgroup exchanges), the multi-pass super-stages, the 2D fold and column
passes and the split column stage, 3D, poly-mul in one kernel and in the
four-step passes (512-point columns: the pipelined pass A), real rows (fused and paired) and real images, chirp-z rows
in one kernel and in passes."""
import os

import numpy as np
import pytest
import torch

import fft_convolution_amd as fm
import oracle
from fft_convolution_amd import build as fbuild
from fft_convolution_amd import workloads as wl

from conftest import fft_tol, rel_rms_rows

pytestmark = pytest.mark.gpu


def _cases():
    c = []
    for logn in range(1, 15):  # up to 16384 points: one 1024-thread workgroup a row
        c.append(("c2c", (1 << logn,), torch.complex64, 5))
    for logn in range(1, 14):
        c.append(("c2c", (1 << logn,), torch.complex128, 3))
    c += [("c2c", (1 << 16,), torch.complex64, 2), ("c2c", (1 << 20,), torch.complex64, 1),
          ("c2c", (1 << 16,), torch.complex128, 1), ("c2c", (1009,), torch.complex64, 3),
          ("c2c", (100003,), torch.complex64, 1), ("c2c", (5003,), torch.complex64, 1),
          ("c2c", (4093,), torch.complex128, 1), ("c2c", (64, 128), torch.complex64, 2),
          ("c2c", (2048, 64), torch.complex64, 1), ("c2c", (8192, 2), torch.complex64, 2),
          ("c2c", (1024, 1024), torch.complex64, 1), ("c2c", (1024, 64), torch.complex128, 1),
          ("c2c", (16, 32, 64), torch.complex64, 1),
          ("poly", (1000,), torch.complex128, 2), ("poly", (3000,), torch.complex128, 2),
          ("poly", (40000,), torch.complex128, 2), ("poly", (1 << 19,), torch.complex128, 1),
          ("real", (1024,), torch.float32, 4), ("real", (1 << 15,), torch.float32, 2),
          ("real", (1 << 16,), torch.float32, 1), ("real", (1 << 14,), torch.float64, 2),
          ("real", (1024, 512), torch.float32, 1), ("real", (64, 64), torch.float64, 2)]
    return c


def _run(kind, dims, dtype, batch, seed):
    """Forward and inverse outputs of one case through whichever library the
    binding has loaded."""
    dev = torch.device("cuda:0")
    n = int(np.prod(dims))
    if kind == "poly":
        a, b = wl.random_polys(dims[0], batch, seed=seed)
        m = 1
        while m < 2 * dims[0] - 1:
            m *= 2
        plan = fm.Plan(m, torch.complex128)
        c = plan.poly_mul(torch.from_numpy(a).to(dev), torch.from_numpy(b).to(dev))
        torch.cuda.synchronize()
        out = [c.cpu()]
    elif kind == "real":
        npdt = np.float32 if dtype == torch.float32 else np.float64
        x = torch.from_numpy(wl.real_normal(n, batch, seed=seed, dtype=npdt).reshape((batch,) + dims)).to(dev)
        plan = fm.RealPlan(dims if len(dims) > 1 else dims[0], dtype)
        X = plan.rfft(x)
        out = [X.cpu(), plan.irfft(X).cpu()]
    else:
        npdt = np.complex64 if dtype == torch.complex64 else np.complex128
        x = torch.from_numpy(wl.batched_uniform(n, batch, seed=seed, dtype=npdt).reshape((batch,) + dims)).to(dev)
        plan = fm.Plan(dims if len(dims) > 1 else dims[0], dtype)
        fwd, inv = {1: (plan.fft, plan.ifft), 2: (plan.fft2, plan.ifft2), 3: (plan.fft3, plan.ifft3)}[len(dims)]
        out = [fwd(x).cpu(), inv(x).cpu()]
    torch.cuda.synchronize()
    del plan
    return out


def test_poisoned_lds_changes_nothing(dev, monkeypatch):
    if not os.path.exists(fbuild.POISON_LIB):
        pytest.fail("libfftmi_poison.so is not built (fft_convolution_amd.build.build())")
    cases = _cases()
    ref = [_run(*c, seed=50 + i) for i, c in enumerate(cases)]
    # the same calls through the poisoned build
    monkeypatch.setattr(fm, "_lib", None)
    monkeypatch.setattr(fm, "lib_path", fbuild.POISON_LIB)
    for i, c in enumerate(cases):
        print("case poison %s" % (c,), flush=True)
        got = _run(*c, seed=50 + i)
        for g, r in zip(got, ref[i]):
            if g.is_floating_point() or g.is_complex():
                assert not torch.isnan(torch.view_as_real(g) if g.is_complex() else g).any(), c
            assert torch.equal(g, r), c
        if c[0] == "c2c" and len(c[1]) == 1 and c[1][0] & (c[1][0] - 1) == 0:
            n = c[1][0]
            npdt = np.complex64 if c[2] == torch.complex64 else np.complex128
            x = wl.batched_uniform(n, c[3], seed=50 + i, dtype=npdt)
            assert rel_rms_rows(got[0].numpy(), oracle.fft(x)).max() <= fft_tol(n, c[2] == torch.complex128)
    import gc
    gc.collect()
