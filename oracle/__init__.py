"""fp64 CPU oracle for the FFT library -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package.  The product path (the HIP library and
its binding) never imports, links or runs anything from here, and this package
imports nothing from the product: the two share no code, headers, tables or
constant generators.

What it computes, and the passage each part follows:

* ``dft`` -- the direct O(N^2) definition X_k = sum_n x_n e^{-2 pi i k n / N}
  ("FFT on GPU", section "Discrete Fourier Transform"), in C (``oracle.c``), for
  any N; ``dft_sample`` -- the same definition for selected outputs only.
* ``fft`` / ``ifft`` -- recursive radix-2 decimation in time, X_k = E_k + w^k O_k,
  X_{k+N/2} = E_k - w^k O_k ("FFT on GPU", section "Fast Fourier Transform"); the
  inverse swaps w for w^{-1} and scales by 1/N (same page, the section on why
  roots of unity are used as evaluation points).
* ``fft2`` / ``ifft2`` -- rows then columns ("Stockham FFT Butterfly Algorithm in
  Parallel GLSL", section "Multi-Dimensional Transforms and Separability");
  ``fft3`` / ``ifft3`` -- the same, one axis after another, for 3D data.
  ``dftn`` -- that separable evaluation with ``dft`` along each of the last
  k axes, for any lengths (shapes that are not powers of two).
* ``rfft`` / ``irfft`` -- transforms of real rows: the first N/2 + 1 outputs of
  ``fft`` of the row widened to complex (the other half follows from
  X_{N-k} = conj X_k, since the inputs are real), and back: the real part of
  ``ifft`` of the Hermitian extension of N/2 + 1 values, the imaginary parts
  of X_0 and X_{N/2} taken as zero.  The operands of polynomial multiplication
  are real ("FFT on GPU", polynomial-multiplication section).
  ``rfft2`` / ``irfft2`` -- the same for real [H][W] images: columns 0 .. W/2
  of ``fft2``; back, the inverse column transforms (complex), then ``irfft``
  of every row.
* ``polymul_fft`` -- forward both zero-padded operands, pointwise product,
  inverse, rint ("FFT on GPU", polynomial-multiplication and whole-process
  sections); ``schoolbook`` / ``schoolbook_sample`` -- the exact convolution
  c_k = sum_i a_i b_{k-i} from the same section.
* Pure-Python helpers for tiny inputs: ``dft_py`` (the definition, with cmath),
  ``bitrev_order`` (the bit-reversed order from the "reverse bit order" section
  of "FFT on GPU"), ``butterfly_pass_half`` (the one-output-per-thread pass of
  "The Butterfly: One Thread, One Output") and ``stockham_pass`` (the stage
  indices and twiddle of "Stockham FFT ... in Parallel GLSL", section
  "Execution via GLSL Compute Shaders and Textures").

Every function here is pinned by ``tests/test_oracle.py`` to closed forms,
invariants, the pages' printed example, brute force on tiny inputs and an
independent library FFT (numpy's pocketfft).
"""
from __future__ import annotations

import cmath
import ctypes
import math
import os
import subprocess
import threading

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB_PATH = os.path.join(_HERE, "liboracle.so")
_lock = threading.Lock()
_lib = None

__all__ = [
    "build", "load", "set_threads", "get_threads",
    "dft", "dft_sample", "fft", "ifft", "fft2", "ifft2", "fft3", "ifft3",
    "polymul_fft", "schoolbook", "schoolbook_sample",
    "dft_py", "bitrev_order", "butterfly_pass_half", "stockham_pass",
    "poly_eval_mod", "MOD_P",
]


def build(force: bool = True) -> str:
    """Compile ``oracle.c`` into ``liboracle.so`` with gcc (-O2 -fopenmp)."""
    if not force and os.path.exists(_LIB_PATH) and \
            os.path.getmtime(_LIB_PATH) >= os.path.getmtime(_SRC):
        return _LIB_PATH
    tmp = _LIB_PATH + ".tmp%d" % os.getpid()
    cmd = ["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-std=c11",
           "-o", tmp, _SRC, "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def load():
    """Load (building first if needed) the C part of the oracle."""
    global _lib
    with _lock:
        if _lib is not None:
            return _lib
        if not os.path.exists(_LIB_PATH) or \
                os.path.getmtime(_LIB_PATH) < os.path.getmtime(_SRC):
            build()
        lib = ctypes.CDLL(_LIB_PATH)
        i64, dbl_p, i64_p, c_int = ctypes.c_int64, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int
        lib.oracle_dft_direct.argtypes = [dbl_p, dbl_p, i64, i64, c_int]
        lib.oracle_fft.argtypes = [dbl_p, dbl_p, i64, i64, c_int]
        lib.oracle_dft_sample.argtypes = [dbl_p, i64, i64, i64_p, i64, dbl_p, c_int]
        lib.oracle_fft2.argtypes = [dbl_p, dbl_p, i64, i64, i64, c_int]
        lib.oracle_fft3.argtypes = [dbl_p, dbl_p, i64, i64, i64, i64, c_int]
        lib.oracle_schoolbook.argtypes = [i64_p, i64, i64_p, i64, i64_p, i64]
        lib.oracle_schoolbook_sample.argtypes = [i64_p, i64, i64_p, i64, i64, i64_p, i64, i64_p]
        lib.oracle_schoolbook_coeff.argtypes = [i64_p, i64, i64_p, i64, i64]
        lib.oracle_schoolbook_coeff.restype = i64
        lib.oracle_polymul_fft.argtypes = [i64_p, i64, i64_p, i64, i64_p, i64, i64,
                                           ctypes.POINTER(ctypes.c_double)]
        lib.oracle_set_threads.argtypes = [c_int]
        lib.oracle_get_threads.restype = c_int
        for name in ("oracle_dft_direct", "oracle_dft_sample", "oracle_fft", "oracle_fft2", "oracle_fft3",
                     "oracle_schoolbook", "oracle_schoolbook_sample",
                     "oracle_polymul_fft", "oracle_set_threads"):
            if name != "oracle_set_threads":
                getattr(lib, name).restype = c_int
        _lib = lib
        return lib


def set_threads(n: int) -> None:
    load().oracle_set_threads(int(n))


def get_threads() -> int:
    return int(load().oracle_get_threads())


def _as_c128(x) -> np.ndarray:
    """Widen to complex128 exactly (fp32 -> fp64 is exact) and make contiguous."""
    return np.ascontiguousarray(np.asarray(x), dtype=np.complex128)


def _ptr(a: np.ndarray) -> int:
    return a.ctypes.data


def _check(rc: int, what: str) -> None:
    if rc != 0:
        raise ValueError("oracle %s rejected its arguments (rc=%d)" % (what, rc))


def dft(x, inverse: bool = False) -> np.ndarray:
    """Direct O(N^2) DFT along the last axis, any N >= 1, fp64."""
    x = _as_c128(x)
    n = x.shape[-1]
    out = np.empty_like(x)
    batch = x.size // n if n else 0
    _check(load().oracle_dft_direct(_ptr(x), _ptr(out), n, batch, int(inverse)), "dft")
    return out


def dft_sample(x, ks, inverse: bool = False) -> np.ndarray:
    """Selected outputs X_k, k in ks, of the direct DFT of each row (any N),
    each computed from the definition in O(N): returns [batch, len(ks)]."""
    x = _as_c128(x)
    if x.ndim == 1:
        x = x[None]
    n = x.shape[-1]
    ks = np.ascontiguousarray(np.asarray(ks), dtype=np.int64)
    out = np.empty((x.size // n, ks.size), dtype=np.complex128)
    _check(load().oracle_dft_sample(_ptr(x), n, x.size // n, _ptr(ks), ks.size, _ptr(out), int(inverse)),
           "dft_sample")
    return out


def fft(x, inverse: bool = False) -> np.ndarray:
    """Recursive radix-2 FFT along the last axis (power-of-two length), fp64."""
    x = _as_c128(x)
    n = x.shape[-1]
    out = np.empty_like(x)
    batch = x.size // n if n else 0
    _check(load().oracle_fft(_ptr(x), _ptr(out), n, batch, int(inverse)), "fft")
    return out


def ifft(X) -> np.ndarray:
    """Inverse of :func:`fft`: conjugate twiddles and 1/N."""
    return fft(X, inverse=True)


def rfft(x) -> np.ndarray:
    """X_0 .. X_{N/2} of the transform of each real row: [..., N] real ->
    [..., N // 2 + 1] complex128 (``fft`` for a power-of-two N, else ``dft``)."""
    x = np.asarray(x)
    if np.iscomplexobj(x):
        raise TypeError("rfft takes real rows")
    n = x.shape[-1]
    full = fft(x.astype(np.float64)) if n & (n - 1) == 0 else dft(x.astype(np.float64))
    return full[..., : n // 2 + 1]


def irfft(X, n: int) -> np.ndarray:
    """The real rows of length n whose transform has X_0 .. X_{floor(n/2)}
    equal to the rows of X ([..., n // 2 + 1]): every bin k > n/2 is set to
    conj X_{n-k}, the imaginary part of X_0 is dropped, and for even n that
    of X_{n/2} too (a real row has real values there; an odd n has no such
    middle bin), then the real part of :func:`ifft`."""
    full = _hermitian_full(X, n)
    return (ifft(full) if n & (n - 1) == 0 else dft(full, inverse=True)).real


def _hermitian_full(X, n: int) -> np.ndarray:
    """The n bins of a real row's transform from its X_0 .. X_{floor(n/2)}
    (the reading of :func:`irfft`)."""
    X = _as_c128(X)
    h = n // 2
    if X.shape[-1] != h + 1:
        raise ValueError("irfft of length %d takes %d values per row" % (n, h + 1))
    full = np.empty(X.shape[:-1] + (n,), dtype=np.complex128)
    full[..., : h + 1] = X[..., : h + 1] if n > 1 else X[..., :1]
    full[..., 0] = full[..., 0].real
    if n > 1 and n % 2 == 0:
        full[..., h] = full[..., h].real
        full[..., h + 1:] = np.conj(X[..., 1:h][..., ::-1])
    elif n > 1:
        full[..., h + 1:] = np.conj(X[..., 1:h + 1][..., ::-1])
    return full


def irfft_sample(X, n: int, ks) -> np.ndarray:
    """Selected samples x_j, j in ks, of :func:`irfft` (X, n), each computed
    from the inverse DFT's definition in O(n) (:func:`dft_sample`)."""
    full = _hermitian_full(X, n)
    return dft_sample(full.reshape(-1, n), ks, inverse=True).real


def rfft2(x) -> np.ndarray:
    """Columns 0 .. W/2 of the 2D transform of real [..., H, W] images:
    [..., H, W // 2 + 1] complex128 (``fft2`` for power-of-two shapes, else
    ``dftn``)."""
    x = np.asarray(x)
    if np.iscomplexobj(x):
        raise TypeError("rfft2 takes real images")
    h, w = x.shape[-2], x.shape[-1]
    pow2 = h & (h - 1) == 0 and w & (w - 1) == 0
    full = fft2(x.astype(np.float64)) if pow2 else dftn(x.astype(np.float64), 2)
    return full[..., : w // 2 + 1]


def irfft2(X, shape) -> np.ndarray:
    """Real [..., H, W] images from columns 0 .. W/2 of their 2D transform:
    the inverse transform along the columns (complex, 1/H), then
    :func:`irfft` of every row (1/W; the imaginary parts of columns 0 and W/2
    of that intermediate are dropped, as a real row's are real there)."""
    h, w = shape
    X = _as_c128(X)
    if X.shape[-2:] != (h, w // 2 + 1):
        raise ValueError("irfft2 of %dx%d takes %dx%d values" % (h, w, h, w // 2 + 1))
    col_t = np.ascontiguousarray(np.swapaxes(X, -1, -2))
    cols = np.swapaxes(ifft(col_t) if h & (h - 1) == 0 else dft(col_t, inverse=True), -1, -2)
    return irfft(np.ascontiguousarray(cols), w)


def fft2(x, inverse: bool = False) -> np.ndarray:
    """Separable 2D transform over the last two axes ([..., H, W], row-major)."""
    x = _as_c128(x)
    h, w = x.shape[-2], x.shape[-1]
    out = np.empty_like(x)
    batch = x.size // (h * w) if h * w else 0
    _check(load().oracle_fft2(_ptr(x), _ptr(out), h, w, batch, int(inverse)), "fft2")
    return out


def ifft2(X) -> np.ndarray:
    return fft2(X, inverse=True)


def fft3(x, inverse: bool = False) -> np.ndarray:
    """Separable 3D transform over the last three axes ([..., D, H, W])."""
    x = _as_c128(x)
    d, h, w = x.shape[-3], x.shape[-2], x.shape[-1]
    out = np.empty_like(x)
    batch = x.size // (d * h * w) if d * h * w else 0
    _check(load().oracle_fft3(_ptr(x), _ptr(out), d, h, w, batch, int(inverse)), "fft3")
    return out


def ifft3(X) -> np.ndarray:
    return fft3(X, inverse=True)


def dftn(x, k: int, inverse: bool = False) -> np.ndarray:
    """The k-dimensional transform over the last k axes, any lengths: ``dft``
    along the last axis, then along each axis before it (the sums over the
    k indices evaluated one index at a time)."""
    y = _as_c128(x)
    for ax in range(1, k + 1):
        moved = np.ascontiguousarray(np.moveaxis(y, -ax, -1))
        y = np.ascontiguousarray(np.moveaxis(dft(moved, inverse=inverse), -1, -ax))
    return y


def _as_i64(a) -> np.ndarray:
    return np.ascontiguousarray(np.asarray(a), dtype=np.int64)


def polymul_fft(a, b, n: int | None = None):
    """FFT route to the product of each pair of rows of a [batch, la] and
    b [batch, lb]: returns (c [batch, la+lb-1] int64, max |Re - rint(Re)|)."""
    a = _as_i64(a)
    b = _as_i64(b)
    if a.ndim == 1:
        a = a[None]
    if b.ndim == 1:
        b = b[None]
    batch, la = a.shape
    lb = b.shape[1]
    if n is None:
        n = 1
        while n < la + lb - 1:
            n *= 2
    c = np.empty((batch, la + lb - 1), dtype=np.int64)
    resid = ctypes.c_double(0.0)
    _check(load().oracle_polymul_fft(_ptr(a), la, _ptr(b), lb, _ptr(c), n, batch,
                                     ctypes.byref(resid)), "polymul_fft")
    return c, float(resid.value)


def schoolbook(a, b) -> np.ndarray:
    """Exact product c_k = sum_i a_i b_{k-i} of each pair of rows, int64."""
    a = _as_i64(a)
    b = _as_i64(b)
    if a.ndim == 1:
        a = a[None]
    if b.ndim == 1:
        b = b[None]
    batch, la = a.shape
    lb = b.shape[1]
    c = np.empty((batch, la + lb - 1), dtype=np.int64)
    _check(load().oracle_schoolbook(_ptr(a), la, _ptr(b), lb, _ptr(c), batch), "schoolbook")
    return c


def schoolbook_sample(a, b, ks) -> np.ndarray:
    """Exact coefficients c_k, k in ks, of each pair: returns [batch, len(ks)]."""
    a = _as_i64(a)
    b = _as_i64(b)
    if a.ndim == 1:
        a = a[None]
    if b.ndim == 1:
        b = b[None]
    ks = _as_i64(ks)
    batch, la = a.shape
    lb = b.shape[1]
    out = np.empty((batch, ks.size), dtype=np.int64)
    _check(load().oracle_schoolbook_sample(_ptr(a), la, _ptr(b), lb, batch, _ptr(ks),
                                           ks.size, _ptr(out)), "schoolbook_sample")
    return out


# --------------------------------------------------------------------------
# Pure-Python helpers for tiny inputs.
# --------------------------------------------------------------------------

def dft_py(x, inverse: bool = False) -> list:
    """The DFT definition with Python complex numbers, for tiny N.  The angle is
    2 pi ((k n) mod N) / N, formed from an exact integer."""
    x = [complex(v) for v in x]
    n = len(x)
    sgn = 1.0 if inverse else -1.0
    out = []
    for k in range(n):
        s = 0j
        for t in range(n):
            s += x[t] * cmath.exp(sgn * 2j * math.pi * ((k * t) % n) / n)
        out.append(s / n if inverse else s)
    return out


def bitrev_order(n: int) -> list:
    """Indices in bit-reversed order: the order the recursive even/odd split
    leaves the input in ("FFT on GPU", section "reverse bit order")."""
    bits = n.bit_length() - 1
    if 1 << bits != n:
        raise ValueError("n must be a power of two")
    out = []
    for i in range(n):
        r, t = 0, i
        for _ in range(bits):
            r = (r << 1) | (t & 1)
            t >>= 1
        out.append(r)
    return out


def butterfly_pass_half(x, half: int, twiddle_sign: float = -1.0) -> list:
    """One radix-2 pass in the one-output-per-thread form of "The Butterfly: One
    Thread, One Output": output i is the lower (j = 0) or upper (j = 1) member
    of the pair (base, base + half), base = i - j*half, with twiddle
    w = e^{-i pi r / half}, r = i mod half; lower gets a + w b, upper a - w b.

    ``twiddle_sign`` exists so a test can plant the page's own cautionary
    mistake (a flipped twiddle sign) and watch the pins catch it."""
    x = [complex(v) for v in x]
    n = len(x)
    out = []
    for i in range(n):
        j = (i // half) % 2
        base = i - j * half
        r = i % half
        w = cmath.exp(twiddle_sign * 1j * math.pi * r / half)
        a, b = x[base], x[base + half]
        out.append(a + w * b if j == 0 else a - w * b)
    return out


def stockham_pass(x, s: int) -> list:
    """Stage s of the radix-2 Stockham form ("Stockham FFT ... in Parallel GLSL",
    section "Execution via GLSL Compute Shaders and Textures"): output x_idx
    reads in[j] and in[k] with j = floor(x_idx / 2^{s+1}) 2^s + (x_idx mod 2^s),
    k = j + N/2, and twiddle W_N^r with r = (x_idx mod 2^{s+1}) N / 2^{s+1}.
    The page prints no combine rule; the reading used is out = in[j] + W_N^r in[k]
    (the sign of the pair's lower/upper member is carried by r >= N/2)."""
    x = [complex(v) for v in x]
    n = len(x)
    out = []
    for xi in range(n):
        j = (xi // (2 << s)) * (1 << s) + (xi % (1 << s))
        k = j + n // 2
        r = (xi % (2 << s)) * (n // (2 << s))
        w = cmath.exp(-2j * math.pi * r / n)
        out.append(x[j] + w * x[k])
    return out


MOD_P = (1 << 61) - 1


def poly_eval_mod(coeffs, z: int, p: int = MOD_P) -> int:
    """Horner evaluation of sum_k coeffs[k] z^k mod p with Python integers."""
    acc = 0
    for c in reversed([int(v) for v in coeffs]):
        acc = (acc * z + c) % p
    return acc
