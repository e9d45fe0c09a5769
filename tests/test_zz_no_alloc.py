"""fft_exec_c2c_noalloc, the entry point that allocates nothing: through the C
ABI, its output must equal fft_exec_c2c's (same kernels, workspace from the
library's scratch instead of the caller's) bit for bit, and match the fp64
oracle at the usual bound, on two calls in a row -- the second with a smaller
input, so that stale scratch contents from the first call would show -- and
sizes beyond the scratch are rejected before any device work (GPU)."""
import ctypes

import numpy as np
import pytest
import torch

import fft_convolution_amd as fm
import oracle
from fft_convolution_amd import workloads as wl

from conftest import fft_tol, rel_rms_rows

pytestmark = pytest.mark.gpu


def _both(plan, x, inverse=False):
    """(noalloc output, fft_exec_c2c output) for the same input and direction."""
    batch = x.shape[0]
    d = fm.FFT_INVERSE if inverse else fm.FFT_FORWARD
    stream = torch.cuda.current_stream().cuda_stream
    y_na = torch.empty_like(x)
    st = fm.lib().fft_exec_c2c_noalloc(plan.handle, d, x.data_ptr(), y_na.data_ptr(), batch, stream)
    assert st == fm.FFT_OK, fm.fft_last_error()
    nbytes = fm.fft_workspace_size(plan.handle, batch)
    ws = torch.empty(nbytes, dtype=torch.uint8, device=x.device) if nbytes else None
    y_ref = torch.empty_like(x)
    fm.fft_exec_c2c(plan.handle, d, x, y_ref, batch, ws, stream)
    torch.cuda.synchronize()
    return y_na, y_ref


@pytest.mark.parametrize("n,dtype,batches", [
    (1 << 20, torch.complex64, (16, 3)),      # multi-pass, 128 MiB then 24 MiB of scratch
    (1 << 24, torch.complex64, (1, 1)),       # the 2^24-point workload: exactly the scratch size
    (1 << 16, torch.complex128, (32, 5)),     # multi-pass complex128
    (100003, torch.complex64, (3, 1)),        # Bluestein, M = 2^18 (multi-pass inner transforms)
    (4096, torch.complex64, (64, 7)),         # one kernel, no workspace at all
])
def test_noalloc_matches_c2c_twice(dev, n, dtype, batches):
    npdt = np.complex64 if dtype == torch.complex64 else np.complex128
    plan = fm.Plan(n, dtype)
    for call, batch in enumerate(batches):
        print("case noalloc n=%d %s batch=%d call=%d" % (n, dtype, batch, call), flush=True)
        x_np = wl.batched_uniform(n, batch, seed=1000 + call, dtype=npdt)
        x = torch.from_numpy(x_np).to(dev)
        for inverse in (False, True):
            y_na, y_ref = _both(plan, x, inverse)
            assert torch.equal(y_na, y_ref), (call, inverse)
        if n * batch <= (1 << 21) and n & (n - 1) == 0:
            ref = oracle.fft(x_np)
            y_na, _ = _both(plan, x)
            assert rel_rms_rows(y_na.cpu().numpy(), ref).max() <= fft_tol(n, dtype == torch.complex128)


def test_noalloc_rejects_beyond_scratch(dev):
    plan = fm.Plan(1 << 20, torch.complex64)
    need = fm.fft_workspace_size(plan.handle, 17)
    assert need > fm.FFT_NOALLOC_SCRATCH_BYTES
    # rejected from the sizes alone, before any device work
    st = fm.lib().fft_exec_c2c_noalloc(plan.handle, fm.FFT_FORWARD, 1 << 20, 1 << 40, 17, None)
    assert st == fm.FFT_ERR_WORKSPACE
    assert "scratch" in fm.fft_last_error()
    st = fm.lib().fft_exec_c2c_noalloc(plan.handle, 7, 1 << 20, 1 << 40, 1, None)
    assert st == fm.FFT_ERR_INVALID_ARG
    p2 = fm.Plan((64, 64), torch.complex64)
    st = fm.lib().fft_exec_c2c_noalloc(p2.handle, fm.FFT_FORWARD, 1 << 20, 1 << 40, 1, None)
    assert st == fm.FFT_ERR_RANK
    assert fm.lib().fft_exec_c2c_noalloc(plan.handle, fm.FFT_FORWARD, None, None, 0, None) == fm.FFT_OK
