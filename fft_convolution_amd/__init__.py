"""Python binding of ``libfftmi.so``, the MI355X (gfx950) Stockham FFT library.

The functions below carry the names of the C ABI in ``include/fftmi.h`` and do
argument marshalling only: device pointers come from PyTorch tensors (or plain
integers), streams from ``torch.cuda.current_stream()``, and every step of a
transform runs in the library's HIP kernels.  A nonzero status raises
:class:`FFTError`.  There is no fallback: if the library is not built, or a
call fails, the error propagates.

Thin conveniences built on those calls:

* :class:`Plan` -- owns a plan handle; ``fft``/``ifft`` (rank 1, any length up
  to the limits: power-of-two, mixed-radix 2/3/5/7/11/13 or Bluestein), ``fft2``/``ifft2``
  (rank 2), ``fft3``/``ifft3`` (rank 3), ``planar`` (split re / im tensors, any
  rank) and ``poly_mul`` (rank 1, complex128) on contiguous device tensors.
* :class:`RealPlan` -- ``rfft``/``irfft`` of real rows.
* :func:`poly_mul` -- one-shot integer polynomial products.
"""
from __future__ import annotations

import ctypes
import os
import threading

__all__ = [
    "FFTError", "FFT_C32", "FFT_C64", "FFT_FORWARD", "FFT_INVERSE",
    "FFT_OK", "FFT_ERR_INVALID_ARG", "FFT_ERR_NOT_POW2", "FFT_ERR_UNSUPPORTED_SIZE",
    "FFT_ERR_PRECISION", "FFT_ERR_RANK", "FFT_ERR_ALIGN", "FFT_ERR_OVERLAP",
    "FFT_ERR_WORKSPACE", "FFT_ERR_DEVICE",
    "FFT_MAX_LDS_N_C32", "FFT_MAX_LDS_N_C64", "FFT_MAX_N_C32", "FFT_MAX_N_C64", "FFT_MAX_BLUESTEIN_N",
    "lib", "lib_path", "EXPORTS",
    "fft_plan_create", "fft_plan_destroy", "fft_plan_describe", "fft_plan_query", "fft_workspace_size",
    "fft_exec_c2c", "fft_exec_c2c_noalloc", "fft_exec_2d", "fft_exec_3d", "fft_poly_mul_workspace_size",
    "fft_poly_mul", "fft_plan_create_real", "fft_plan_create_real_2d", "fft_exec_r2c", "fft_exec_c2r",
    "fft_exec_planar", "fft_planar_workspace_size", "fft_stream_copy", "fft_status_string", "fft_last_error",
    "FFT_NOALLOC_SCRATCH_BYTES", "Plan", "RealPlan", "poly_mul",
]

FFT_C32, FFT_C64 = 0, 1
FFT_FORWARD, FFT_INVERSE = 0, 1
FFT_OK = 0
FFT_ERR_INVALID_ARG = -1
FFT_ERR_NOT_POW2 = -2
FFT_ERR_UNSUPPORTED_SIZE = -3
FFT_ERR_PRECISION = -4
FFT_ERR_RANK = -5
FFT_ERR_ALIGN = -6
FFT_ERR_OVERLAP = -7
FFT_ERR_WORKSPACE = -8
FFT_ERR_DEVICE = -9
FFT_MAX_LDS_N_C32 = 8192
FFT_MAX_LDS_N_C64 = 4096
FFT_MAX_N_C32 = 1 << 26
FFT_MAX_N_C64 = 1 << 24
FFT_MAX_BLUESTEIN_N = 1 << 23
FFT_NOALLOC_SCRATCH_BYTES = 128 << 20

_HERE = os.path.dirname(os.path.abspath(__file__))
lib_path = os.path.join(_HERE, "libfftmi.so")

# Every symbol include/fftmi.h declares.
EXPORTS = (
    "fft_plan_create", "fft_plan_destroy", "fft_plan_describe", "fft_plan_query", "fft_workspace_size",
    "fft_exec_c2c", "fft_exec_c2c_noalloc", "fft_exec_2d", "fft_exec_3d", "fft_poly_mul_workspace_size",
    "fft_poly_mul", "fft_plan_create_real", "fft_plan_create_real_2d", "fft_exec_r2c", "fft_exec_c2r",
    "fft_exec_planar", "fft_planar_workspace_size", "fft_stream_copy", "fft_status_string", "fft_last_error",
)

# Reentrant: a finalizer that the garbage collector runs while lib() is
# loading the library (its allocations can trigger a collection) may call
# back into the binding on the same thread.
_lock = threading.RLock()
_lib = None


class FFTError(RuntimeError):
    """A nonzero status from the library."""

    def __init__(self, status: int, where: str, detail: str = ""):
        self.status = status
        msg = "%s failed: %s" % (where, fft_status_string(status))
        if detail:
            msg += " (%s)" % detail
        super().__init__(msg)


def lib():
    """The loaded library.  Raises if it has not been built."""
    global _lib
    with _lock:
        if _lib is not None:
            return _lib
        if not os.path.exists(lib_path):
            raise ImportError(
                "libfftmi.so is not built (expected at %s); run "
                "`python -m fft_convolution_amd.build`" % lib_path)
        L = ctypes.CDLL(lib_path)
        vp, i64, c_int, sz = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int, ctypes.c_size_t
        L.fft_plan_create.argtypes = [ctypes.POINTER(vp), c_int, ctypes.POINTER(i64), c_int]
        L.fft_plan_destroy.argtypes = [vp]
        L.fft_plan_describe.argtypes = [vp, ctypes.c_char_p, sz]
        L.fft_plan_query.argtypes = [c_int, ctypes.POINTER(i64), c_int, ctypes.c_char_p, sz]
        L.fft_workspace_size.argtypes = [vp, i64, ctypes.POINTER(sz)]
        L.fft_exec_c2c.argtypes = [vp, c_int, vp, vp, i64, vp, vp]
        L.fft_exec_c2c_noalloc.argtypes = [vp, c_int, vp, vp, i64, vp]
        L.fft_exec_2d.argtypes = [vp, c_int, vp, vp, i64, vp, vp]
        L.fft_exec_3d.argtypes = [vp, c_int, vp, vp, i64, vp, vp]
        L.fft_poly_mul_workspace_size.argtypes = [vp, i64, ctypes.POINTER(sz)]
        L.fft_poly_mul.argtypes = [vp, vp, i64, vp, i64, vp, i64, vp, vp, vp]
        L.fft_plan_create_real.argtypes = [ctypes.POINTER(vp), i64, c_int]
        L.fft_plan_create_real_2d.argtypes = [ctypes.POINTER(vp), i64, i64, c_int]
        L.fft_exec_r2c.argtypes = [vp, vp, vp, i64, vp, vp]
        L.fft_exec_c2r.argtypes = [vp, vp, vp, i64, vp, vp]
        L.fft_exec_planar.argtypes = [vp, c_int, vp, vp, vp, vp, i64, vp, vp]
        L.fft_planar_workspace_size.argtypes = [vp, i64, ctypes.POINTER(sz)]
        L.fft_stream_copy.argtypes = [vp, vp, sz, vp]
        L.fft_status_string.argtypes = [c_int]
        L.fft_status_string.restype = ctypes.c_char_p
        L.fft_last_error.argtypes = []
        L.fft_last_error.restype = ctypes.c_char_p
        for name in EXPORTS:
            if name in ("fft_status_string", "fft_last_error"):
                continue
            getattr(L, name).restype = c_int
        _lib = L
        return L


def _ptr(x) -> int | None:
    """Device address of a tensor, or an integer address, or None for NULL."""
    if x is None:
        return None
    if isinstance(x, int):
        return x or None
    if hasattr(x, "data_ptr"):
        return x.data_ptr() or None
    raise TypeError("expected a tensor, an integer address or None, got %r" % type(x))


def _stream(stream) -> int | None:
    if stream is None:
        import torch
        return torch.cuda.current_stream().cuda_stream or None
    if isinstance(stream, int):
        return stream or None
    return stream.cuda_stream or None


def _check(status: int, where: str) -> None:
    if status != FFT_OK:
        raise FFTError(status, where, fft_last_error())


def fft_status_string(status: int) -> str:
    return lib().fft_status_string(int(status)).decode()


def fft_last_error() -> str:
    return lib().fft_last_error().decode()


def fft_plan_create(rank: int, dims, prec: int = FFT_C32) -> int:
    """Create a plan (rank 1: dims = [N]; rank 2: [H, W]; rank 3: [D, H, W]); returns its handle."""
    dims = [int(d) for d in dims]
    arr = (ctypes.c_int64 * max(len(dims), 1))(*dims)
    h = ctypes.c_void_p()
    _check(lib().fft_plan_create(ctypes.byref(h), int(rank), arr if dims else None, int(prec)),
           "fft_plan_create")
    return h.value


def fft_plan_destroy(plan) -> None:
    _check(lib().fft_plan_destroy(plan), "fft_plan_destroy")


def fft_plan_describe(plan) -> str:
    buf = ctypes.create_string_buffer(256)
    _check(lib().fft_plan_describe(plan, buf, 256), "fft_plan_describe")
    return buf.value.decode()


def fft_plan_query(rank: int, dims, prec: int = FFT_C32) -> str:
    """Description of the plan fft_plan_create would make (host only, no device)."""
    dims = [int(d) for d in dims]
    arr = (ctypes.c_int64 * max(len(dims), 1))(*dims)
    buf = ctypes.create_string_buffer(256)
    _check(lib().fft_plan_query(int(rank), arr if dims else None, int(prec), buf, 256), "fft_plan_query")
    return buf.value.decode()


def fft_workspace_size(plan, batch: int) -> int:
    out = ctypes.c_size_t()
    _check(lib().fft_workspace_size(plan, int(batch), ctypes.byref(out)), "fft_workspace_size")
    return out.value


def fft_exec_c2c(plan, dir: int, in_, out, batch: int, workspace=None, stream=None) -> None:
    _check(lib().fft_exec_c2c(plan, int(dir), _ptr(in_), _ptr(out), int(batch), _ptr(workspace),
                              _stream(stream)), "fft_exec_c2c")


def fft_exec_c2c_noalloc(plan, dir: int, in_, out, batch: int, stream=None) -> None:
    _check(lib().fft_exec_c2c_noalloc(plan, int(dir), _ptr(in_), _ptr(out), int(batch), _stream(stream)),
           "fft_exec_c2c_noalloc")


def fft_exec_2d(plan, dir: int, in_, out, batch: int, workspace=None, stream=None) -> None:
    _check(lib().fft_exec_2d(plan, int(dir), _ptr(in_), _ptr(out), int(batch), _ptr(workspace),
                             _stream(stream)), "fft_exec_2d")


def fft_exec_3d(plan, dir: int, in_, out, batch: int, workspace=None, stream=None) -> None:
    _check(lib().fft_exec_3d(plan, int(dir), _ptr(in_), _ptr(out), int(batch), _ptr(workspace),
                             _stream(stream)), "fft_exec_3d")


def fft_poly_mul_workspace_size(plan, batch: int) -> int:
    out = ctypes.c_size_t()
    _check(lib().fft_poly_mul_workspace_size(plan, int(batch), ctypes.byref(out)),
           "fft_poly_mul_workspace_size")
    return out.value


def fft_poly_mul(plan, a, la: int, b, lb: int, c, batch: int, workspace=None,
                 d_max_residual=None, stream=None) -> None:
    _check(lib().fft_poly_mul(plan, _ptr(a), int(la), _ptr(b), int(lb), _ptr(c), int(batch),
                              _ptr(workspace), _ptr(d_max_residual), _stream(stream)),
           "fft_poly_mul")


def fft_plan_create_real(n: int, prec: int = FFT_C32) -> int:
    """Create a plan for transforms of real rows of n points; returns its handle."""
    h = ctypes.c_void_p()
    _check(lib().fft_plan_create_real(ctypes.byref(h), int(n), int(prec)), "fft_plan_create_real")
    return h.value


def fft_plan_create_real_2d(h: int, w: int, prec: int = FFT_C32) -> int:
    """Create a plan for real [h][w] images; returns its handle."""
    hd = ctypes.c_void_p()
    _check(lib().fft_plan_create_real_2d(ctypes.byref(hd), int(h), int(w), int(prec)), "fft_plan_create_real_2d")
    return hd.value


def fft_exec_r2c(plan, in_, out, batch: int, workspace=None, stream=None) -> None:
    _check(lib().fft_exec_r2c(plan, _ptr(in_), _ptr(out), int(batch), _ptr(workspace), _stream(stream)),
           "fft_exec_r2c")


def fft_exec_c2r(plan, in_, out, batch: int, workspace=None, stream=None) -> None:
    _check(lib().fft_exec_c2r(plan, _ptr(in_), _ptr(out), int(batch), _ptr(workspace), _stream(stream)),
           "fft_exec_c2r")


def fft_exec_planar(plan, dir: int, in_re, in_im, out_re, out_im, batch: int, workspace=None,
                    stream=None) -> None:
    _check(lib().fft_exec_planar(plan, int(dir), _ptr(in_re), _ptr(in_im), _ptr(out_re), _ptr(out_im),
                                 int(batch), _ptr(workspace), _stream(stream)), "fft_exec_planar")


def fft_planar_workspace_size(plan, batch: int) -> int:
    out = ctypes.c_size_t()
    _check(lib().fft_planar_workspace_size(plan, int(batch), ctypes.byref(out)), "fft_planar_workspace_size")
    return out.value


def fft_stream_copy(src, dst, nbytes: int, stream=None) -> None:
    _check(lib().fft_stream_copy(_ptr(src), _ptr(dst), int(nbytes), _stream(stream)), "fft_stream_copy")


# --------------------------------------------------------------------------
# Conveniences over torch tensors (allocation and shape checks only)
# --------------------------------------------------------------------------

def _release(obj) -> None:
    """Free a plan object's handle through the library that created it (a
    finalizer: no lock, no library loading, and the right library even after
    the binding has been pointed at another build)."""
    h = getattr(obj, "handle", None)
    L = getattr(obj, "_lib", None)
    if h and L is not None:
        try:
            L.fft_plan_destroy(h)
        except Exception:
            pass
    obj.handle = None


class Plan:
    """A plan handle.  ``Plan(n)``, ``Plan((h, w))`` or ``Plan((d, h, w))``; dtype torch.complex64/128."""

    def __init__(self, dims, dtype=None):
        import torch
        if dtype is None:
            dtype = torch.complex64
        if dtype not in (torch.complex64, torch.complex128):
            raise TypeError("dtype must be torch.complex64 or torch.complex128")
        self.dtype = dtype
        self.prec = FFT_C32 if dtype == torch.complex64 else FFT_C64
        self.dims = (int(dims),) if isinstance(dims, int) else tuple(int(d) for d in dims)
        self.rank = len(self.dims)
        self.handle = fft_plan_create(self.rank, self.dims, self.prec)
        self._lib = lib()  # the library that made the handle, which frees it

    # the finalizer is bound at class creation: at interpreter exit the
    # module's globals may already be gone when a plan is collected
    def __del__(self, _free=_release):
        _free(self)

    def describe(self) -> str:
        return fft_plan_describe(self.handle)

    def _check_tensor(self, x):
        import torch
        if not isinstance(x, torch.Tensor) or not x.is_cuda:
            raise TypeError("expected a device tensor")
        if x.dtype != self.dtype:
            raise TypeError("expected %s, got %s" % (self.dtype, x.dtype))
        if not x.is_contiguous():
            raise ValueError("tensor must be contiguous")
        if tuple(x.shape[-self.rank:]) != self.dims:
            raise ValueError("trailing dims %s do not match the plan %s" % (tuple(x.shape), self.dims))
        n = 1
        for d in self.dims:
            n *= d
        return x.numel() // n

    def _exec(self, x, out, direction, fn):
        import torch
        batch = self._check_tensor(x)
        if out is None:
            out = torch.empty_like(x)
        else:
            self._check_tensor(out)
        ws_bytes = fft_workspace_size(self.handle, batch)
        # A power-of-two rank-2/3 plan uses its workspace only for an in-place
        # call, unless its column stage runs as a pass of its own ("split").
        desc = self.describe()
        if self.rank >= 2 and out.data_ptr() != x.data_ptr() and "path=nd " in desc and "split=" not in desc:
            ws_bytes = 0
        ws = torch.empty(ws_bytes, dtype=torch.uint8, device=x.device) if ws_bytes else None
        fn(self.handle, direction, x, out, batch, ws)
        return out

    def fft(self, x, out=None):
        if self.rank != 1:
            raise ValueError("fft needs a rank-1 plan")
        return self._exec(x, out, FFT_FORWARD, fft_exec_c2c)

    def ifft(self, x, out=None):
        if self.rank != 1:
            raise ValueError("ifft needs a rank-1 plan")
        return self._exec(x, out, FFT_INVERSE, fft_exec_c2c)

    def fft2(self, x, out=None):
        if self.rank != 2:
            raise ValueError("fft2 needs a rank-2 plan")
        return self._exec(x, out, FFT_FORWARD, fft_exec_2d)

    def ifft2(self, x, out=None):
        if self.rank != 2:
            raise ValueError("ifft2 needs a rank-2 plan")
        return self._exec(x, out, FFT_INVERSE, fft_exec_2d)

    def fft3(self, x, out=None):
        if self.rank != 3:
            raise ValueError("fft3 needs a rank-3 plan")
        return self._exec(x, out, FFT_FORWARD, fft_exec_3d)

    def ifft3(self, x, out=None):
        if self.rank != 3:
            raise ValueError("ifft3 needs a rank-3 plan")
        return self._exec(x, out, FFT_INVERSE, fft_exec_3d)

    def planar(self, re, im, inverse=False, out=None):
        """The transform of re + i im, real and imaginary parts in separate
        float32/float64 tensors of shape [..., *dims]; returns (out_re, out_im)."""
        import torch
        rdt = torch.float32 if self.dtype == torch.complex64 else torch.float64
        for t in (re, im):
            if not isinstance(t, torch.Tensor) or not t.is_cuda or t.dtype != rdt or not t.is_contiguous():
                raise TypeError("re and im must be contiguous %s device tensors" % rdt)
        if re.shape != im.shape or tuple(re.shape[-self.rank:]) != self.dims:
            raise ValueError("re/im shapes %s %s do not match the plan %s" % (tuple(re.shape), tuple(im.shape),
                                                                              self.dims))
        n = 1
        for d in self.dims:
            n *= d
        batch = re.numel() // n
        if out is None:
            out = (torch.empty_like(re), torch.empty_like(im))
        nb = fft_planar_workspace_size(self.handle, batch)
        ws = torch.empty(nb, dtype=torch.uint8, device=re.device) if nb else None
        fft_exec_planar(self.handle, FFT_INVERSE if inverse else FFT_FORWARD, re, im, out[0], out[1], batch, ws)
        return out

    def poly_mul(self, a, b, out=None, residual=False):
        """Products of the rows of int64 device tensors a [batch, la], b [batch, lb]."""
        import torch
        if self.rank != 1:
            raise ValueError("poly_mul needs a rank-1 plan")
        for t in (a, b):
            if not isinstance(t, torch.Tensor) or not t.is_cuda or t.dtype != torch.int64 \
                    or not t.is_contiguous():
                raise TypeError("a and b must be contiguous int64 device tensors")
        a2 = a.reshape(-1, a.shape[-1])
        b2 = b.reshape(-1, b.shape[-1])
        if a2.shape[0] != b2.shape[0]:
            raise ValueError("a and b must have the same batch")
        batch, la, lb = a2.shape[0], a2.shape[1], b2.shape[1]
        if out is None:
            out = torch.empty((batch, la + lb - 1), dtype=torch.int64, device=a.device)
        ws_bytes = fft_poly_mul_workspace_size(self.handle, batch)
        ws = torch.empty(ws_bytes, dtype=torch.uint8, device=a.device) if ws_bytes else None
        resid = torch.empty(1, dtype=torch.float64, device=a.device) if residual else None
        fft_poly_mul(self.handle, a2, la, b2, lb, out, batch, ws, resid)
        return (out, resid) if residual else out


class RealPlan:
    """A plan for real rows of n points (``RealPlan(n)``) or real [h][w]
    images (``RealPlan((h, w))``): ``rfft`` [..., n] / [..., h, w] float32/64
    -> [..., n // 2 + 1] / [..., h, w // 2 + 1] complex64/128, ``irfft`` the
    reverse."""

    def __init__(self, dims, dtype=None):
        import torch
        if dtype is None:
            dtype = torch.float32
        if dtype not in (torch.float32, torch.float64):
            raise TypeError("dtype must be torch.float32 or torch.float64")
        self.dtype = dtype
        self.cdtype = torch.complex64 if dtype == torch.float32 else torch.complex128
        self.prec = FFT_C32 if dtype == torch.float32 else FFT_C64
        self.dims = (int(dims),) if isinstance(dims, int) else tuple(int(d) for d in dims)
        self.n = self.dims[-1]
        self.rows = self.dims[0] if len(self.dims) == 2 else 1
        if len(self.dims) == 1:
            self.handle = fft_plan_create_real(self.n, self.prec)
        elif len(self.dims) == 2:
            self.handle = fft_plan_create_real_2d(self.dims[0], self.dims[1], self.prec)
        else:
            raise ValueError("real plans have one or two dims")
        self._lib = lib()  # the library that made the handle, which frees it

    # the finalizer is bound at class creation: at interpreter exit the
    # module's globals may already be gone when a plan is collected
    def __del__(self, _free=_release):
        _free(self)

    def describe(self) -> str:
        return fft_plan_describe(self.handle)

    def _check(self, x, dtype, last):
        """Validates a tensor ending in [rows][last] (rows = h for images);
        returns the number of transforms."""
        import torch
        if not isinstance(x, torch.Tensor) or not x.is_cuda:
            raise TypeError("expected a device tensor")
        if x.dtype != dtype:
            raise TypeError("expected %s, got %s" % (dtype, x.dtype))
        if not x.is_contiguous():
            raise ValueError("tensor must be contiguous")
        if x.shape[-1] != last or (len(self.dims) == 2 and (x.dim() < 2 or x.shape[-2] != self.rows)):
            raise ValueError("trailing dims %s do not fit the plan %s" % (tuple(x.shape), self.dims))
        return x.numel() // (last * self.rows)

    def _ws(self, batch, device):
        import torch
        nb = fft_workspace_size(self.handle, batch)
        return torch.empty(nb, dtype=torch.uint8, device=device) if nb else None

    def rfft(self, x, out=None):
        import torch
        batch = self._check(x, self.dtype, self.n)
        if out is None:
            out = torch.empty(x.shape[:-1] + (self.n // 2 + 1,), dtype=self.cdtype, device=x.device)
        elif self._check(out, self.cdtype, self.n // 2 + 1) != batch:
            raise ValueError("out has another batch")
        fft_exec_r2c(self.handle, x, out, batch, self._ws(batch, x.device))
        return out

    def irfft(self, X, out=None):
        import torch
        batch = self._check(X, self.cdtype, self.n // 2 + 1)
        if out is None:
            out = torch.empty(X.shape[:-1] + (self.n,), dtype=self.dtype, device=X.device)
        elif self._check(out, self.dtype, self.n) != batch:
            raise ValueError("out has another batch")
        fft_exec_c2r(self.handle, X, out, batch, self._ws(batch, X.device))
        return out


def poly_mul(a, b, residual=False):
    """Integer polynomial products with the smallest power-of-two N >= la + lb - 1."""
    import torch
    la, lb = a.shape[-1], b.shape[-1]
    n = 1
    while n < la + lb - 1:
        n *= 2
    return Plan(n, torch.complex128).poly_mul(a, b, residual=residual)
