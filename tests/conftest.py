import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line(
        "markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")


import math

import numpy as np
import pytest


def rel_rms_rows(y, ref):
    """Per-transform relative RMS error ||y - ref||_2 / ||ref||_2 over the last
    `axes` dims, as a flat array (one value per transform)."""
    y = np.asarray(y, dtype=np.complex128)
    ref = np.asarray(ref, dtype=np.complex128)
    num = np.sqrt(np.sum(np.abs(y - ref) ** 2, axis=-1))
    den = np.sqrt(np.sum(np.abs(ref) ** 2, axis=-1))
    return num / np.maximum(den, 1e-300)


def fft_tol(n, complex128=False):
    """Per-transform relative RMS bound: 1e-6 log2 N for complex64; for
    complex128 the same form scaled to the fp64 unit roundoff (1e-14 log2 N)."""
    return (1e-14 if complex128 else 1e-6) * max(1.0, math.log2(n))


@pytest.fixture(scope="session")
def dev():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import fft_convolution_amd as fm
    fm.lib()  # fail loudly if the HIP library is missing
    return torch.device("cuda:0")
