"""Exec-time validation of the C ABI with real plans (GPU): every status code
documented in include/fftmi.h for fft_exec_c2c / fft_exec_2d, checked before
anything is enqueued."""
import pytest
import torch

import fft_convolution_amd as fm

pytestmark = pytest.mark.gpu


def _status(fn, *args):
    try:
        fn(*args)
    except fm.FFTError as e:
        return e.status
    return fm.FFT_OK


def test_exec_validation(dev):
    p1 = fm.Plan(1024, torch.complex64)
    p2 = fm.Plan((32, 32), torch.complex64)
    pbig = fm.Plan(1 << 16, torch.complex64)
    x = torch.zeros(4, 1024, dtype=torch.complex64, device=dev)
    y = torch.zeros_like(x)
    h = p1.handle
    assert _status(fm.fft_exec_c2c, h, 2, x, y, 4) == fm.FFT_ERR_INVALID_ARG
    assert _status(fm.fft_exec_c2c, h, 0, x, y, -1) == fm.FFT_ERR_INVALID_ARG
    assert _status(fm.fft_exec_c2c, h, 0, None, y, 4) == fm.FFT_ERR_INVALID_ARG
    assert _status(fm.fft_exec_c2c, h, 0, x, y, 0) == fm.FFT_OK
    assert _status(fm.fft_exec_c2c, h, 0, None, None, 0) == fm.FFT_OK
    assert _status(fm.fft_exec_2d, h, 0, x, y, 4) == fm.FFT_ERR_RANK
    assert _status(fm.fft_exec_c2c, p2.handle, 0, x, y, 1) == fm.FFT_ERR_RANK
    assert _status(fm.fft_exec_c2c, h, 0, x.data_ptr() + 4, y, 1) == fm.FFT_ERR_ALIGN
    flat = torch.zeros(5 * 1024, dtype=torch.complex64, device=dev)
    assert _status(fm.fft_exec_c2c, h, 0, flat, flat.data_ptr() + 8 * 1024, 4) == fm.FFT_ERR_OVERLAP
    xb = torch.zeros(2, 1 << 16, dtype=torch.complex64, device=dev)
    yb = torch.zeros_like(xb)
    assert fm.fft_workspace_size(pbig.handle, 2) == 2 * (1 << 16) * 8
    assert fm.fft_workspace_size(h, 2) == 0
    assert _status(fm.fft_exec_c2c, pbig.handle, 0, xb, yb, 2, None) == fm.FFT_ERR_WORKSPACE
    assert _status(fm.fft_exec_c2c, pbig.handle, 0, xb, yb, 2, yb) == fm.FFT_ERR_WORKSPACE
    ws = torch.empty(2 * (1 << 16) * 8, dtype=torch.uint8, device=dev)
    assert _status(fm.fft_exec_c2c, pbig.handle, 0, xb, yb, 2, ws) == fm.FFT_OK
    torch.cuda.synchronize()
    assert "path=rows" in p1.describe() and "path=multipass" in pbig.describe()
    assert "path=nd" in p2.describe()
    p3 = fm.Plan((4, 8, 16), torch.complex64)
    assert _status(fm.fft_exec_3d, p2.handle, 0, x, y, 1) == fm.FFT_ERR_RANK
    assert _status(fm.fft_exec_2d, p3.handle, 0, x, y, 1) == fm.FFT_ERR_RANK
    assert _status(fm.fft_exec_3d, p3.handle, 0, x, y, 2) == fm.FFT_OK


@pytest.mark.parametrize("nbytes", [8, 4096, 32768, 32768 + 8, 5 * 32768 + 1000, 1 << 26])
def test_stream_copy_copies_every_byte(dev, nbytes):
    """fft_stream_copy (the benchmark's ceiling) copies exactly `nbytes`:
    full 32 KiB blocks, a partial last block, and leaves the bytes after the
    range untouched."""
    g = torch.Generator(device="cpu").manual_seed(nbytes % 1000)
    src = torch.randint(0, 256, (nbytes + 64,), dtype=torch.uint8, generator=g).to(dev)
    dst = torch.zeros(nbytes + 64, dtype=torch.uint8, device=dev)
    fm.fft_stream_copy(src, dst, nbytes)
    torch.cuda.synchronize()
    assert torch.equal(dst[:nbytes], src[:nbytes])
    assert int(dst[nbytes:].count_nonzero()) == 0
