"""Planar (split re / im) arrays through fft_exec_planar (GPU).

Only the first kernel's loads and the last kernel's stores differ from the
interleaved calls, so every result must equal the interleaved call's bit for
bit, on every path (one-kernel rows, two- and three-pass multi-pass,
Bluestein, mixed radix, 2D with and without the folded column stage, 3D, axes of length
1); a few cases are also checked against the fp64 oracle directly, and the
[2][N] layout of "The Butterfly: One Thread, One Output" is passed as one
buffer."""
import numpy as np
import pytest
import torch

import fft_convolution_amd as fm
import oracle
from fft_convolution_amd import workloads as wl

from conftest import fft_tol, rel_rms_rows

pytestmark = pytest.mark.gpu

CASES = [
    # dims, dtype, batch
    ((1,), torch.complex64, 5),
    ((8,), torch.complex64, 33),
    ((1024,), torch.complex64, 7),
    ((8192,), torch.complex64, 2),
    ((4096,), torch.complex128, 3),
    ((1 << 16,), torch.complex64, 2),      # two passes
    ((1 << 20,), torch.complex64, 1),      # three passes
    ((1 << 13,), torch.complex128, 2),     # two passes, fp64
    ((1 << 19,), torch.complex128, 1),     # three passes, fp64
    ((1009,), torch.complex64, 3),         # Bluestein
    ((1001,), torch.complex64, 3),         # mixed radix with 11 and 13
    ((10000,), torch.complex64, 2),        # mixed-radix passes (two)
    ((10 ** 6,), torch.complex64, 1),      # mixed-radix passes (three)
    ((6000,), torch.complex128, 2),
    ((100, 7), torch.complex64, 2),        # non-power-of-two images: rows, one column pass
    ((1000, 60), torch.complex64, 1),      # two column passes
    ((12, 30, 50), torch.complex128, 1),
    ((4097,), torch.complex128, 2),
    ((60,), torch.complex64, 7),           # mixed radix
    ((2401,), torch.complex128, 2),
    ((64, 128), torch.complex64, 3),
    ((2048, 256), torch.complex64, 1),     # folded column stage
    ((1024, 64), torch.complex128, 2),     # folded, fp64
    ((8192, 2), torch.complex64, 3),       # column stage as a pass of its own
    ((4096, 2), torch.complex128, 2),
    ((4, 8192, 2), torch.complex64, 1),
    ((1, 1024), torch.complex64, 3),       # one axis longer than 1
    ((1, 1), torch.complex128, 4),
    ((16, 32, 64), torch.complex64, 2),    # 3D
    ((8, 2048, 16), torch.complex64, 1),   # 3D, folded
    ((4, 1, 128), torch.complex128, 2),
    ((17, 8), torch.complex64, 2),         # a transposed axis (chirp-z columns)
    ((29, 31, 1), torch.complex128, 1),    # two transposed axes, no rows
]


def _exec_interleaved(plan, x, inverse):
    d = fm.FFT_INVERSE if inverse else fm.FFT_FORWARD
    out = torch.empty_like(x)
    n = x.shape[-plan.rank:].numel()
    batch = x.numel() // n
    nb = fm.fft_workspace_size(plan.handle, batch)
    ws = torch.empty(nb, dtype=torch.uint8, device=x.device) if nb else None
    fn = {1: fm.fft_exec_c2c, 2: fm.fft_exec_2d, 3: fm.fft_exec_3d}[plan.rank]
    fn(plan.handle, d, x, out, batch, ws)
    return out


@pytest.mark.parametrize("dims,dtype,batch", CASES, ids=lambda v: str(v))
def test_planar_equals_interleaved(dev, dims, dtype, batch):
    print("case dims=%s %s batch=%d" % (dims, dtype, batch), flush=True)
    n = int(np.prod(dims))
    npdt = np.complex64 if dtype == torch.complex64 else np.complex128
    x_np = wl.batched_uniform(n, batch, seed=n % 97 + batch, dtype=npdt).reshape((batch,) + dims)
    x = torch.from_numpy(x_np).to(dev)
    plan = fm.Plan(dims, dtype)
    re, im = x.real.contiguous(), x.imag.contiguous()
    for inverse in (False, True):
        ref = _exec_interleaved(plan, x, inverse)
        pr, pi = plan.planar(re, im, inverse=inverse)
        torch.cuda.synchronize()
        assert torch.equal(pr, ref.real.contiguous()) and torch.equal(pi, ref.imag.contiguous()), inverse
    # in place
    r2, i2 = re.clone(), im.clone()
    plan.planar(r2, i2, out=(r2, i2))
    ref = _exec_interleaved(plan, x, False)
    torch.cuda.synchronize()
    assert torch.equal(r2, ref.real.contiguous()) and torch.equal(i2, ref.imag.contiguous())


@pytest.mark.parametrize("dims,dtype", [((4096,), torch.complex64), ((1 << 18,), torch.complex128),
                                        ((999,), torch.complex64), ((1001,), torch.complex64),
                                        ((128, 256), torch.complex64), ((16, 16384), torch.complex64),
                                        ((8, 8192), torch.complex128)])
def test_planar_against_oracle(dev, dims, dtype):
    n = int(np.prod(dims))
    npdt = np.complex64 if dtype == torch.complex64 else np.complex128
    x_np = wl.batched_normal(n, 2, seed=11, dtype=npdt).reshape((2,) + dims)
    plan = fm.Plan(dims, dtype)
    re = torch.from_numpy(np.ascontiguousarray(x_np.real)).to(dev)
    im = torch.from_numpy(np.ascontiguousarray(x_np.imag)).to(dev)
    yr, yi = plan.planar(re, im)
    y = (yr.cpu().numpy() + 1j * yi.cpu().numpy()).reshape(2, n)
    ref = (oracle.fft2(x_np) if len(dims) == 2 else
           (oracle.fft(x_np) if (n & (n - 1)) == 0 else oracle.dft(x_np))).reshape(2, n)
    assert rel_rms_rows(y, ref).max() <= fft_tol(n, dtype == torch.complex128)


def test_planar_two_by_n_buffer(dev):
    """One [2][N] buffer (plane 0 re, plane 1 im), and [2][batch][N]."""
    n, batch = 2048, 3
    plan = fm.Plan(n, torch.complex64)
    x_np = wl.batched_uniform(n, batch, seed=5)
    buf = torch.from_numpy(np.stack([x_np.real, x_np.imag])).to(dev)       # [2][batch][N]
    out = torch.empty_like(buf)
    fm.fft_exec_planar(plan.handle, fm.FFT_FORWARD, buf[0], buf[1], out[0], out[1], batch)
    y = out[0].cpu().numpy() + 1j * out[1].cpu().numpy()
    assert rel_rms_rows(y, oracle.fft(x_np)).max() <= fft_tol(n)
    one = buf[:, 0].contiguous()                                           # [2][N], batch 1
    o1 = torch.empty_like(one)
    fm.fft_exec_planar(plan.handle, fm.FFT_FORWARD, one.data_ptr(), one.data_ptr() + 4 * n,
                       o1.data_ptr(), o1.data_ptr() + 4 * n, 1)
    torch.cuda.synchronize()
    assert torch.equal(o1, out[:, 0])


def test_planar_errors(dev):
    plan = fm.Plan(1 << 20, torch.complex64)
    n = 1 << 20
    re = torch.zeros(n, device=dev)
    im = torch.zeros(n, device=dev)
    assert fm.fft_planar_workspace_size(plan.handle, 1) == 2 * n * 8      # three passes
    assert fm.fft_planar_workspace_size(fm.Plan(4096).handle, 9) == 0
    assert fm.fft_planar_workspace_size(fm.Plan(1 << 16).handle, 1) == (1 << 16) * 8
    ws = torch.empty(2 * n * 8, dtype=torch.uint8, device=dev)
    with pytest.raises(fm.FFTError) as e:
        fm.fft_exec_planar(plan.handle, 0, re, im, re, im, 1, None)
    assert e.value.status == fm.FFT_ERR_WORKSPACE
    with pytest.raises(fm.FFTError) as e:    # out_re on in_im
        fm.fft_exec_planar(plan.handle, 0, re, im, im, re, 1, ws)
    assert e.value.status == fm.FFT_ERR_OVERLAP
    with pytest.raises(fm.FFTError) as e:    # re and im planes overlap
        fm.fft_exec_planar(plan.handle, 0, re, re.data_ptr() + 8, re, re.data_ptr() + 8, 1, ws)
    assert e.value.status == fm.FFT_ERR_OVERLAP
    with pytest.raises(fm.FFTError) as e:
        fm.fft_exec_planar(plan.handle, 0, re.data_ptr() + 4, im, re.data_ptr() + 4, im, 1, ws)
    assert e.value.status == fm.FFT_ERR_ALIGN
    with pytest.raises(fm.FFTError) as e:
        fm.fft_exec_planar(fm.RealPlan(64).handle, 0, re, im, re, im, 1, ws)
    assert e.value.status == fm.FFT_ERR_RANK
    fm.fft_exec_planar(plan.handle, 0, re, im, re, im, 0, None)          # batch 0: no-op
