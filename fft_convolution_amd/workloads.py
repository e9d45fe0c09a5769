"""Seeded synthetic inputs for the FFT library's workloads.

This module holds input generation only -- none of the transform's arithmetic
-- so that the tests can hand the very same arrays to the HIP library and to
the fp64 CPU oracle.  All draws use numpy's PCG64 (``numpy.random.default_rng``).

Workloads (every complex array is interleaved (re, im), complex64 unless
stated):

* ``batched_uniform`` -- rows of N points, re and im i.i.d. uniform [-1, 1).
  N = 1024 x 64 rows (seed 1) is the small forward + inverse round-trip case;
  N = 2^24 x 1 row (seed 3) is the single large transform.
* ``batched_normal`` -- rows of N points, re and im i.i.d. standard normal.
  N = 4096 x 16384 rows (seed 2) is the batched throughput case (512 MiB in).
* ``plane_waves_2d`` -- [batch][H][W] images, each the sum of 16 complex 2D
  plane waves e^{i(2 pi (fy y / H + fx x / W) + phi)} with distinct random
  integer frequencies, unit amplitude and random phase, plus i.i.d. normal
  noise of std 0.01 on re and im.  2048 x 2048 x 8 images (seed 4).
* ``random_polys`` -- pairs of integer polynomials with coefficients i.i.d.
  uniform in [0, 1000).  32 pairs of 2^18 coefficients (seed 5).
* a 256^3 volume, re and im uniform [-1, 1) (seed 6), for the 3D transform.
* ``real_normal`` -- real rows of N points, i.i.d. standard normal: the real
  operands of the R2C / C2R transforms.  N = 8192 x 16384 rows (seed 7).
* rows of 1000 and 1009 points x 65536, ``batched_normal`` (seeds 8, 9): the
  mixed-radix and Bluestein paths.
* real 2048 x 2048 images x 8, ``real_normal`` (seed 10): the 2D R2C path.
* rows of 10^6 points x 64, ``batched_normal`` (seed 11): the mixed-radix
  super-stage passes.
"""
from __future__ import annotations

import numpy as np

# The five workloads: name -> (kind, shape, seed).
WORKLOADS = {
    "c2c_n1024_b64": dict(kind="uniform", n=1024, batch=64, seed=1),
    "c2c_n4096_b16384": dict(kind="normal", n=4096, batch=16384, seed=2),
    "c2c_n16777216_b1": dict(kind="uniform", n=1 << 24, batch=1, seed=3),
    "c2c2d_2048x2048_b8": dict(kind="plane_waves", h=2048, w=2048, batch=8, seed=4),
    "polymul_l262144_b32": dict(kind="polys", length=1 << 18, batch=32, seed=5),
    # 3D separable transform (beyond the five workloads above): one 256^3 volume.
    "c2c3d_256x256x256_b1": dict(kind="uniform3d", d=256, h=256, w=256, batch=1, seed=6),
    # real rows, the R2C transform (512 MiB of float32 in)
    "r2c_n8192_b16384": dict(kind="real_normal", n=8192, batch=16384, seed=7),
    # lengths that are not powers of two (~500 MiB in): 1000 = 8 * 5^3 (mixed
    # radix), 1009 prime (Bluestein, M = 2048)
    "c2c_n1000_b65536": dict(kind="normal", n=1000, batch=65536, seed=8),
    "c2c_n1009_b65536": dict(kind="normal", n=1009, batch=65536, seed=9),
    # real 2048 x 2048 images, the 2D R2C transform
    "r2c2d_2048x2048_b8": dict(kind="real_images", h=2048, w=2048, batch=8, seed=10),
    # 10^6 = 1000 x 1000: two mixed-radix super-stage passes (~500 MiB in)
    "c2c_n1000000_b64": dict(kind="normal", n=10 ** 6, batch=64, seed=11),
    # the 4096 x 16384 transform on split re / im planes (the [2][N] signal
    # layout): 256 MiB per plane each way
    "c2cpl_n4096_b16384": dict(kind="normal", n=4096, batch=16384, seed=12),
}


def _complex_from_planes(re: np.ndarray, im: np.ndarray, dtype) -> np.ndarray:
    out = np.empty(re.shape, dtype=dtype)
    out.real = re
    out.imag = im
    return out


def batched_uniform(n: int, batch: int, seed: int, dtype=np.complex64,
                    rows: slice | None = None) -> np.ndarray:
    """[batch, n] complex, re then im drawn i.i.d. uniform [-1, 1).

    The re plane is drawn for the whole batch, then the im plane.  ``rows``
    returns only a slice of the rows (the full draw is still made, so the
    values are those of the full array)."""
    rng = np.random.default_rng(seed)
    real_dt = np.float32 if np.dtype(dtype) == np.complex64 else np.float64
    re = rng.random((batch, n), dtype=real_dt) * 2 - 1
    im = rng.random((batch, n), dtype=real_dt) * 2 - 1
    if rows is not None:
        re, im = re[rows], im[rows]
    return _complex_from_planes(re, im, dtype)


def batched_normal(n: int, batch: int, seed: int, dtype=np.complex64,
                   rows: slice | None = None) -> np.ndarray:
    """[batch, n] complex, re then im drawn i.i.d. standard normal."""
    rng = np.random.default_rng(seed)
    real_dt = np.float32 if np.dtype(dtype) == np.complex64 else np.float64
    re = rng.standard_normal((batch, n), dtype=real_dt)
    im = rng.standard_normal((batch, n), dtype=real_dt)
    if rows is not None:
        re, im = re[rows], im[rows]
    return _complex_from_planes(re, im, dtype)


def real_normal(n: int, batch: int, seed: int, dtype=np.float32) -> np.ndarray:
    """[batch, n] real, i.i.d. standard normal."""
    rng = np.random.default_rng(seed)
    return rng.standard_normal((batch, n), dtype=np.dtype(dtype).type)


def real_spectrum(n: int, batch: int, seed: int, dtype=np.complex64) -> np.ndarray:
    """[batch, n // 2 + 1] complex, re then im i.i.d. standard normal: a half
    spectrum for the C2R transform (its DC and Nyquist imaginary parts need
    not be zero)."""
    rng = np.random.default_rng(seed)
    real_dt = np.float32 if np.dtype(dtype) == np.complex64 else np.float64
    re = rng.standard_normal((batch, n // 2 + 1), dtype=real_dt)
    im = rng.standard_normal((batch, n // 2 + 1), dtype=real_dt)
    return _complex_from_planes(re, im, dtype)


def plane_wave_params(h: int, w: int, batch: int, seed: int, waves: int = 16):
    """Per image: `waves` distinct integer frequency pairs (fy, fx) uniform over
    [0, H) x [0, W), and phases uniform [0, 2 pi).  Returns (fy, fx, phi) arrays
    of shape [batch, waves]."""
    rng = np.random.default_rng(seed)
    fy = np.empty((batch, waves), dtype=np.int64)
    fx = np.empty((batch, waves), dtype=np.int64)
    for b in range(batch):
        flat = rng.choice(h * w, size=waves, replace=False)
        fy[b] = flat // w
        fx[b] = flat % w
    phi = rng.random((batch, waves)) * (2 * np.pi)
    return fy, fx, phi, rng


def plane_waves_2d(h: int, w: int, batch: int, seed: int, noise_std: float = 0.01,
                   waves: int = 16, dtype=np.complex64, with_params: bool = False):
    """[batch, h, w] images: sum of `waves` unit complex plane waves plus noise.

    The phase of each wave at (y, x) is built in fp64 from the exact integer
    residues (fy*y mod H) and (fx*x mod W), then the image is rounded to
    `dtype`.  Noise: re then im, i.i.d. normal with std `noise_std`, drawn
    after the wave parameters from the same generator."""
    fy, fx, phi, rng = plane_wave_params(h, w, batch, seed, waves)
    y = np.arange(h, dtype=np.int64)[:, None]
    x = np.arange(w, dtype=np.int64)[None, :]
    out = np.empty((batch, h, w), dtype=dtype)
    for b in range(batch):
        acc = np.zeros((h, w), dtype=np.complex128)
        for m in range(waves):
            ph = 2 * np.pi * (((fy[b, m] * y) % h) / h + ((fx[b, m] * x) % w) / w) + phi[b, m]
            acc += np.exp(1j * ph)
        if noise_std:
            acc.real += rng.standard_normal((h, w)) * noise_std
            acc.imag += rng.standard_normal((h, w)) * noise_std
        out[b] = acc
    if with_params:
        return out, (fy, fx, phi)
    return out


def random_polys(length: int, batch: int, seed: int, lo: int = 0, hi: int = 1000):
    """Two [batch, length] int64 arrays (a then b), i.i.d. uniform in [lo, hi)."""
    rng = np.random.default_rng(seed)
    a = rng.integers(lo, hi, size=(batch, length), dtype=np.int64)
    b = rng.integers(lo, hi, size=(batch, length), dtype=np.int64)
    return a, b


def workload_input(name: str, **overrides):
    """The seeded input of one of the named workloads (see ``WORKLOADS``)."""
    spec = dict(WORKLOADS[name])
    spec.update(overrides)
    kind = spec.pop("kind")
    if kind == "uniform":
        return batched_uniform(spec["n"], spec["batch"], spec["seed"])
    if kind == "normal":
        return batched_normal(spec["n"], spec["batch"], spec["seed"])
    if kind == "plane_waves":
        return plane_waves_2d(spec["h"], spec["w"], spec["batch"], spec["seed"])
    if kind == "polys":
        return random_polys(spec["length"], spec["batch"], spec["seed"])
    if kind == "real_normal":
        return real_normal(spec["n"], spec["batch"], spec["seed"])
    if kind == "real_images":
        return real_normal(spec["h"] * spec["w"], spec["batch"], spec["seed"]).reshape(
            spec["batch"], spec["h"], spec["w"])
    if kind == "uniform3d":
        d, h, w = spec["d"], spec["h"], spec["w"]
        return batched_uniform(d * h * w, spec["batch"], spec["seed"]).reshape(spec["batch"], d, h, w)
    raise KeyError(kind)
