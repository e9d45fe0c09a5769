"""Parity of the 2D HIP path (row kernel + tiled column pass) with the fp64
oracle (GPU).  Bar: per-image relative RMS <= 1e-6 log2(H W) for complex64,
1e-14 log2(H W) for complex128."""
import numpy as np
import pytest
import torch

import fft_convolution_amd as fm
import oracle
from fft_convolution_amd import workloads as wl

from conftest import fft_tol, rel_rms_rows

pytestmark = pytest.mark.gpu


def _flat(a):
    return a.reshape(a.shape[0], -1)


@pytest.mark.parametrize("h,w,batch", [
    (1, 1, 2), (1, 64, 3), (64, 1, 3), (2, 2, 1), (2, 4096, 1), (4096, 2, 1), (16, 16, 5),
    (32, 64, 3), (64, 32, 2), (8, 8192, 1), (8192, 8, 1), (128, 256, 2), (512, 512, 1),
    (1024, 64, 1), (2048, 2048, 1),
    (8192, 4, 1), (4096, 8192, 1),   # 2048-point column passes (the cap)
    # rows of 16384 (one 1024-thread workgroup a row), short to the cap
    (1, 16384, 2), (2, 16384, 2), (64, 16384, 1), (1024, 16384, 1), (8192, 16384, 1),
])
def test_fft2_c64(dev, h, w, batch):
    print("case h=%d w=%d batch=%d" % (h, w, batch), flush=True)
    x_np = wl.batched_uniform(h * w, batch, seed=h * 31 + w).reshape(batch, h, w)
    plan = fm.Plan((h, w), torch.complex64)
    x = torch.from_numpy(x_np).to(dev)
    for inverse in (False, True):
        y = plan.ifft2(x) if inverse else plan.fft2(x)
        torch.cuda.synchronize()
        ref = oracle.fft2(x_np, inverse=inverse)
        err = rel_rms_rows(_flat(y.cpu().numpy()), _flat(ref))
        assert err.max() <= fft_tol(h * w), (inverse, err.max())


@pytest.mark.parametrize("h,w,batch", [(1, 8, 2), (8, 1, 2), (16, 32, 3), (256, 128, 2), (4096, 16, 1),
                                       (16, 4096, 1), (1024, 1024, 1),
                                       (2048, 2, 2), (4096, 4, 1), (4096, 2048, 1),  # 1024-point columns
                                       (2, 8192, 2), (512, 8192, 1), (4096, 8192, 1)])  # rows of 8192
def test_fft2_c128(dev, h, w, batch):
    x_np = wl.batched_uniform(h * w, batch, seed=h * 17 + w, dtype=np.complex128).reshape(batch, h, w)
    plan = fm.Plan((h, w), torch.complex128)
    x = torch.from_numpy(x_np).to(dev)
    for inverse in (False, True):
        y = plan.ifft2(x) if inverse else plan.fft2(x)
        torch.cuda.synchronize()
        ref = oracle.fft2(x_np, inverse=inverse)
        assert rel_rms_rows(_flat(y.cpu().numpy()), _flat(ref)).max() <= fft_tol(h * w, True)


def test_workload_2048x2048_b8(dev):
    # The full 8-image plane-wave workload in the launch the benchmark times.
    # Every image against the oracle; on every image the 16 largest bins are
    # also exactly the planted frequencies, with value ~H W e^{i phi}.
    h = w = 2048
    x_np, (fy, fx, phi) = wl.plane_waves_2d(h, w, 8, seed=4, with_params=True)
    plan = fm.Plan((h, w), torch.complex64)
    x = torch.from_numpy(x_np).to(dev)
    y = torch.empty_like(x)
    fm.fft_exec_2d(plan.handle, fm.FFT_FORWARD, x, y, 8, None)
    torch.cuda.synchronize()
    for b in range(8):
        ref = oracle.fft2(x_np[b])
        err = rel_rms_rows(y[b].cpu().numpy().reshape(1, -1), ref.reshape(1, -1))
        assert err.max() <= fft_tol(h * w)
    mag = y.abs().reshape(8, -1)
    top = torch.topk(mag, 16, dim=1).indices.cpu().numpy()
    for b in range(8):
        assert set(top[b].tolist()) == set((fy[b] * w + fx[b]).tolist())
        vals = y[b].cpu().numpy()[fy[b], fx[b]]
        assert np.max(np.abs(vals - h * w * np.exp(1j * phi[b]))) < 1e-3 * h * w


def test_fft2_round_trip_and_in_place(dev):
    h, w = 256, 512
    x_np = wl.batched_normal(h * w, 3, seed=9).reshape(3, h, w)
    plan = fm.Plan((h, w), torch.complex64)
    x = torch.from_numpy(x_np).to(dev)
    X = plan.fft2(x)
    z = x.clone()
    plan.fft2(z, out=z)
    back = plan.ifft2(X)
    torch.cuda.synchronize()
    assert torch.equal(X, z)
    assert rel_rms_rows(_flat(back.cpu().numpy()), _flat(x_np)).max() <= fft_tol(h * w)


def test_fft2_folded_in_place_needs_workspace(dev):
    # 2048 rows fold a radix-4 column super-stage into the row pass; in place
    # that pass cannot write its output over rows other groups still read, so
    # an in-place call takes a workspace (and is rejected without one).
    h, w = 2048, 64
    plan = fm.Plan((h, w), torch.complex64)
    assert "fold=4" in plan.describe()
    x_np = wl.batched_normal(h * w, 2, seed=11).reshape(2, h, w)
    x = torch.from_numpy(x_np).to(dev)
    ws_bytes = fm.fft_workspace_size(plan.handle, 2)
    assert ws_bytes == 2 * h * w * 8
    z = x.clone()
    with pytest.raises(fm.FFTError) as e:
        fm.fft_exec_2d(plan.handle, fm.FFT_FORWARD, z, z, 2, None)
    assert e.value.status == fm.FFT_ERR_WORKSPACE
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device=dev)
    fm.fft_exec_2d(plan.handle, fm.FFT_FORWARD, z, z, 2, ws)
    y = plan.fft2(x)
    torch.cuda.synchronize()
    assert torch.equal(y, z)
    assert rel_rms_rows(_flat(y.cpu().numpy()), _flat(oracle.fft2(x_np))).max() <= fft_tol(h * w)


@pytest.mark.parametrize("h,w,dtype,batch", [(8192, 2, torch.complex64, 3), (4096, 2, torch.complex128, 3),
                                             (4096, 4096, torch.complex128, 1), (8192, 8192, torch.complex64, 1)])
def test_fft2_split_column_stage(dev, h, w, dtype, batch):
    """Rows too narrow (fewer points per thread than F) or too wide (F rows
    over the LDS) to fold the column stage: rows, a separate radix-F column
    stage, then the column pass -- against the oracle, both directions, in
    place; these plans need a workspace on every call."""
    print("case %dx%d %s batch=%d" % (h, w, dtype, batch), flush=True)
    npdt = np.complex64 if dtype == torch.complex64 else np.complex128
    x_np = wl.batched_uniform(h * w, batch, seed=h + w, dtype=npdt).reshape(batch, h, w)
    plan = fm.Plan((h, w), dtype)
    assert "split=" in plan.describe()
    x = torch.from_numpy(x_np).to(dev)
    tol = fft_tol(h * w, dtype == torch.complex128)
    X = plan.fft2(x)
    assert rel_rms_rows(_flat(X.cpu().numpy()), _flat(oracle.fft2(x_np))).max() <= tol
    back = plan.ifft2(X).cpu().numpy()
    assert rel_rms_rows(_flat(back), _flat(x_np)).max() <= tol
    z = x.clone()
    plan.fft2(z, out=z)
    torch.cuda.synchronize()
    assert torch.equal(z, X)
    # a workspace is required even out of place
    out = torch.empty_like(x)
    with pytest.raises(fm.FFTError) as e:
        fm.fft_exec_2d(plan.handle, fm.FFT_FORWARD, x, out, batch, None)
    assert e.value.status == fm.FFT_ERR_WORKSPACE
