"""2D / 3D transforms with a dimension that is not a power of two (GPU): the
innermost axis by its rank-1 route (mixed radix, super-stage passes,
Bluestein, or power of two), every other axis as mixed-radix super-stage
passes over the flattened image, against the fp64 oracle's separable direct
DFT (``oracle.dftn``).

Axes other than the innermost whose length has a prime factor above 13 are
transposed to be innermost, run as rows by the rank-1 plan of their length
(chirp-z) and transposed back.

Bar: per-image relative RMS <= 1e-6 log2(size) (complex64), 1e-14 log2(size)
(complex128)."""
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


def _tol(dims, c128):
    return fft_tol(int(np.prod(dims)), c128)


CASES = [
    ((12, 20), torch.complex64, 3),
    ((100, 7), torch.complex64, 2),      # 7-point rows, one 100-point column pass
    ((7, 100), torch.complex64, 2),
    ((1000, 1), torch.complex64, 2),     # a column of 1000: one pass, no rows
    ((3000, 1), torch.complex64, 1),     # a column of 3000: two passes, no rows
    ((1, 1000), torch.complex64, 2),     # rows only
    ((64, 97), torch.complex64, 2),      # Bluestein rows
    ((1000, 600), torch.complex64, 1),   # 1000-point columns: one pass of radix 1000
    ((2000, 60), torch.complex64, 1),    # 2000-point columns: two passes
    ((1024, 100), torch.complex64, 1),   # power-of-two columns: one pass of radix 1024
    ((1001, 12), torch.complex64, 1),    # 7 11 13: two passes (radices 11, 13 stay within 512)
    ((845, 6), torch.complex128, 1),     # 5 13 13: two passes
    ((720, 1280), torch.complex64, 1),
    ((12, 30, 50), torch.complex64, 2),
    ((3, 5, 7), torch.complex64, 3),
    ((10, 100, 10), torch.complex64, 1),
    ((100, 7), torch.complex128, 2),
    ((1000, 60), torch.complex128, 1),
    ((729, 40), torch.complex128, 1),    # radix 729 = 9^3, the widest pass class in complex128
    ((12, 30, 50), torch.complex128, 1),
    # axes other than the innermost with a prime factor above 13: transposed
    ((17, 8), torch.complex64, 3),
    ((97, 64), torch.complex64, 2),
    ((1009, 12), torch.complex64, 1),
    ((4099, 3), torch.complex64, 1),     # chirp-z at M = 16384: the multi-pass route
    ((34, 97), torch.complex64, 2),      # both axes by chirp-z
    ((19, 5, 8), torch.complex64, 2),
    ((6, 23, 7), torch.complex64, 2),
    ((29, 31, 1), torch.complex64, 2),   # two transposed axes, no rows
    ((17, 16), torch.complex128, 2),
    ((6, 23, 7), torch.complex128, 1),
]


@pytest.mark.parametrize("dims,dtype,batch", CASES)
def test_ndmixed(dev, dims, dtype, batch):
    print("case dims=%s %s batch=%d" % (dims, dtype, batch), flush=True)
    c128 = dtype == torch.complex128
    npdt = np.complex128 if c128 else np.complex64
    n = int(np.prod(dims))
    x_np = wl.batched_uniform(n, batch, seed=n % 991, dtype=npdt).reshape((batch,) + dims)
    plan = fm.Plan(dims, dtype)
    assert "path=ndmixed" in plan.describe()
    x = torch.from_numpy(x_np).to(dev)
    k = len(dims)
    tol = _tol(dims, c128)
    oracle.set_threads(8)
    fwd, inv = (plan.fft2, plan.ifft2) if k == 2 else (plan.fft3, plan.ifft3)
    for inverse in (False, True):
        y = (inv(x) if inverse else fwd(x)).cpu().numpy()
        ref = oracle.dftn(x_np, k, inverse=inverse)
        err = rel_rms_rows(_flat(y), _flat(ref)).max()
        assert err <= tol, (inverse, err)
    back = inv(fwd(x)).cpu().numpy()
    assert rel_rms_rows(_flat(back), _flat(x_np)).max() <= tol
    z = x.clone()
    fwd(z, out=z)
    ref = fwd(x)
    torch.cuda.synchronize()
    assert torch.equal(z, ref)


def test_ndmixed_three_pass_axis(dev):
    """A column axis of 1161216 = 2^11 3^4 7 points (three passes: beyond
    1024^2) over two-point rows, on sampled bins: with W = 2 the image
    transform at (k1, k2) is the column transform of x[:, 0] + (-1)^k2 x[:, 1]."""
    h, w = 1161216, 2
    plan = fm.Plan((h, w), torch.complex64)
    d = plan.describe()
    assert "axis1=" in d and d.split("axis1=")[1].count("x") == 2, d
    x_np = wl.batched_normal(h * w, 1, seed=17).reshape(1, h, w)
    y = plan.fft2(torch.from_numpy(x_np).to(dev)).cpu().numpy()[0]
    ks = np.unique(np.concatenate([[0, 1, h // 2, h - 1], np.random.default_rng(3).integers(0, h, 60)]))
    oracle.set_threads(8)
    for k2, sign in ((0, 1.0), (1, -1.0)):
        col = (x_np[0, :, 0].astype(np.complex128) + sign * x_np[0, :, 1])[None, :]
        ref = oracle.dft_sample(col, ks)[0]
        err = np.sqrt(np.mean(np.abs(y[ks, k2] - ref) ** 2)) / np.sqrt(np.mean(np.abs(ref) ** 2))
        assert err <= fft_tol(h * w), (k2, err)


def test_ndmixed_workspace_rules(dev):
    # two-pass columns (beyond 1024 points) need a signal-sized buffer, out
    # of place too
    plan = fm.Plan((2000, 600), torch.complex64)
    need = fm.fft_workspace_size(plan.handle, 1)
    assert need >= 2000 * 600 * 8
    x = torch.zeros(1, 2000, 600, dtype=torch.complex64, device=dev)
    with pytest.raises(fm.FFTError) as e:
        fm.fft_exec_2d(plan.handle, fm.FFT_FORWARD, x, torch.empty_like(x), 1, None)
    assert e.value.status == fm.FFT_ERR_WORKSPACE
    # one-pass columns (up to 1024 points) over mixed-radix rows: none
    assert fm.fft_workspace_size(fm.Plan((100, 7), torch.complex64).handle, 5) == 0
    assert fm.fft_workspace_size(fm.Plan((1000, 600), torch.complex64).handle, 2) == 0
