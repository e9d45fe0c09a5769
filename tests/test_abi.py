"""The C ABI on the CPU: the library loads, exports every symbol the header
declares, and rejects bad arguments with the documented status codes before
any HIP call.  Valid arguments on a host without a GPU give FFT_ERR_DEVICE."""
import ctypes
import os
import re

import pytest

import fft_convolution_amd as fm

HEADER = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "include", "fftmi.h")


def _have_gpu():
    try:
        import torch
        return torch.cuda.is_available()
    except Exception:
        return False


def test_header_declarations_match_exports():
    text = open(HEADER).read()
    declared = set(re.findall(r"^\s*(?:int|const char\*)\s+(fft_\w+)\s*\(", text, flags=re.M))
    assert declared == set(fm.EXPORTS)
    L = fm.lib()
    for name in declared:
        assert hasattr(L, name), name


def test_header_constants_match_binding():
    text = open(HEADER).read()
    for name in ("FFT_OK", "FFT_ERR_INVALID_ARG", "FFT_ERR_NOT_POW2", "FFT_ERR_UNSUPPORTED_SIZE",
                 "FFT_ERR_PRECISION", "FFT_ERR_RANK", "FFT_ERR_ALIGN", "FFT_ERR_OVERLAP",
                 "FFT_ERR_WORKSPACE", "FFT_ERR_DEVICE", "FFT_C32", "FFT_C64", "FFT_FORWARD",
                 "FFT_INVERSE"):
        m = re.search(r"\b%s\s*=\s*(-?\d+)" % name, text)
        assert m and int(m.group(1)) == getattr(fm, name), name
    for name in ("FFT_MAX_LDS_N_C32", "FFT_MAX_LDS_N_C64"):
        m = re.search(r"#define %s (\d+)" % name, text)
        assert int(m.group(1)) == getattr(fm, name)
    for name in ("FFT_MAX_N_C32", "FFT_MAX_N_C64", "FFT_MAX_BLUESTEIN_N"):
        m = re.search(r"#define %s \(1LL << (\d+)\)" % name, text)
        assert (1 << int(m.group(1))) == getattr(fm, name)


def test_status_strings_cover_every_code():
    codes = [fm.FFT_OK, fm.FFT_ERR_INVALID_ARG, fm.FFT_ERR_NOT_POW2, fm.FFT_ERR_UNSUPPORTED_SIZE,
             fm.FFT_ERR_PRECISION, fm.FFT_ERR_RANK, fm.FFT_ERR_ALIGN, fm.FFT_ERR_OVERLAP,
             fm.FFT_ERR_WORKSPACE, fm.FFT_ERR_DEVICE]
    texts = [fm.fft_status_string(c) for c in codes]
    assert len(set(texts)) == len(codes)
    assert all(t != "unknown status" for t in texts)
    assert fm.fft_status_string(-1000) == "unknown status"
    assert fm.fft_status_string(0) == "FFT_OK"


def _create_status(rank, dims, prec):
    L = fm.lib()
    h = ctypes.c_void_p(12345)
    arr = (ctypes.c_int64 * max(len(dims), 1))(*dims) if dims is not None else None
    st = L.fft_plan_create(ctypes.byref(h), rank, arr, prec)
    return st, h.value


@pytest.mark.parametrize("rank,dims,prec,status", [
    (0, [8], 0, fm.FFT_ERR_INVALID_ARG),
    (4, [8, 8, 8, 8], 0, fm.FFT_ERR_INVALID_ARG),
    (1, None, 0, fm.FFT_ERR_INVALID_ARG),
    (1, [8], 2, fm.FFT_ERR_INVALID_ARG),
    (1, [0], 0, fm.FFT_ERR_INVALID_ARG),
    (1, [-4], 0, fm.FFT_ERR_INVALID_ARG),
    (1, [(1 << 23) + 1], 0, fm.FFT_ERR_UNSUPPORTED_SIZE),   # beyond the Bluestein range
    (1, [3 << 22], 1, fm.FFT_ERR_UNSUPPORTED_SIZE),
    # not powers of two: every axis at most 2^23 points unless 13-smooth, and
    # the transform at most 2^26 / 2^24 points
    (2, [(1 << 23) + 1, 2], 0, fm.FFT_ERR_UNSUPPORTED_SIZE),
    (3, [2, (1 << 23) + 1, 1], 1, fm.FFT_ERR_UNSUPPORTED_SIZE),
    (2, [10000, 10000], 0, fm.FFT_ERR_UNSUPPORTED_SIZE),
    (2, [1200, 16000], 1, fm.FFT_ERR_UNSUPPORTED_SIZE),
    (2, [2, (1 << 23) + 1], 0, fm.FFT_ERR_UNSUPPORTED_SIZE),
    (1, [1 << 27], 0, fm.FFT_ERR_UNSUPPORTED_SIZE),
    (1, [1 << 25], 1, fm.FFT_ERR_UNSUPPORTED_SIZE),
    (2, [16384, 8], 0, fm.FFT_ERR_UNSUPPORTED_SIZE),
    (2, [8, 16384], 1, fm.FFT_ERR_UNSUPPORTED_SIZE),  # rows beyond 8192 (complex128)
    (3, [0, 8, 8], 0, fm.FFT_ERR_INVALID_ARG),
    (3, [4096, 8, 8], 0, fm.FFT_ERR_UNSUPPORTED_SIZE),  # depth beyond the column-pass range
    (3, [2048, 8, 8], 1, fm.FFT_ERR_UNSUPPORTED_SIZE),
    (3, [8, 8, 32768], 0, fm.FFT_ERR_UNSUPPORTED_SIZE),  # rows beyond 16384 (complex64)
    (3, [8, 16384, 8], 0, fm.FFT_ERR_UNSUPPORTED_SIZE),
])
def test_plan_create_rejects(rank, dims, prec, status):
    st, h = _create_status(rank, dims, prec)
    assert st == status
    assert h is None  # *plan is set to NULL on failure
    assert fm.fft_last_error() != ""


def test_plan_create_null_out_pointer():
    arr = (ctypes.c_int64 * 1)(8)
    assert fm.lib().fft_plan_create(None, 1, arr, 0) == fm.FFT_ERR_INVALID_ARG


@pytest.mark.skipif(_have_gpu(), reason="host without a GPU only")
def test_valid_plan_without_gpu_is_a_device_error():
    for rank, dims, prec in ((1, [1024], 0), (1, [1 << 24], 0), (2, [64, 32], 1), (1, [1], 0),
                             (3, [16, 8, 32], 0), (3, [4096, 1, 1], 0), (2, [8192, 8], 0),
                             (1, [1000], 0), (1, [12], 1), (1, [1 << 23], 0),
                             (2, [8192, 8192], 0), (2, [4096, 4096], 1), (2, [8192, 2], 0),
                             (3, [2048, 8192, 8192], 0), (2, [97, 8], 0), (2, [51, 12], 1),
                             (3, [8, 19, 6], 0)):
        st, h = _create_status(rank, dims, prec)
        assert st == fm.FFT_ERR_DEVICE and h is None
        assert "hipGetDevice" in fm.fft_last_error()


@pytest.mark.parametrize("n,prec,status", [
    (0, 0, fm.FFT_ERR_INVALID_ARG),
    (-8, 0, fm.FFT_ERR_INVALID_ARG),
    (8, 2, fm.FFT_ERR_INVALID_ARG),
    ((1 << 23) + 1, 0, fm.FFT_ERR_UNSUPPORTED_SIZE),  # odd: the N-point complex plan's limit
    (2 * ((1 << 23) + 1), 0, fm.FFT_ERR_UNSUPPORTED_SIZE),
    (1 << 28, 0, fm.FFT_ERR_UNSUPPORTED_SIZE),
    (1 << 26, 1, fm.FFT_ERR_UNSUPPORTED_SIZE),
])
def test_real_plan_create_rejects(n, prec, status):
    h = ctypes.c_void_p(12345)
    assert fm.lib().fft_plan_create_real(ctypes.byref(h), n, prec) == status
    assert h.value is None
    assert fm.lib().fft_plan_create_real(None, 8, 0) == fm.FFT_ERR_INVALID_ARG


@pytest.mark.skipif(_have_gpu(), reason="host without a GPU only")
def test_valid_real_plan_without_gpu_is_a_device_error():
    for n, prec in ((1, 0), (2, 1), (16384, 0), (1 << 27, 0), (1 << 25, 1), (7, 0), (1001, 1), ((1 << 23) - 1, 0)):
        h = ctypes.c_void_p(12345)
        assert fm.lib().fft_plan_create_real(ctypes.byref(h), n, prec) == fm.FFT_ERR_DEVICE
        assert h.value is None


def test_exec_and_queries_with_null_plan():
    L = fm.lib()
    assert L.fft_exec_c2c(None, 0, None, None, 1, None, None) == fm.FFT_ERR_INVALID_ARG
    assert L.fft_exec_2d(None, 0, None, None, 1, None, None) == fm.FFT_ERR_INVALID_ARG
    assert L.fft_exec_3d(None, 0, None, None, 1, None, None) == fm.FFT_ERR_INVALID_ARG
    assert L.fft_exec_r2c(None, None, None, 1, None, None) == fm.FFT_ERR_INVALID_ARG
    assert L.fft_exec_planar(None, 0, None, None, None, None, 1, None, None) == fm.FFT_ERR_INVALID_ARG
    assert L.fft_exec_c2r(None, None, None, 1, None, None) == fm.FFT_ERR_INVALID_ARG
    assert L.fft_poly_mul(None, None, 1, None, 1, None, 1, None, None, None) == fm.FFT_ERR_INVALID_ARG
    sz = ctypes.c_size_t()
    assert L.fft_workspace_size(None, 1, ctypes.byref(sz)) == fm.FFT_ERR_INVALID_ARG
    assert L.fft_poly_mul_workspace_size(None, 1, ctypes.byref(sz)) == fm.FFT_ERR_INVALID_ARG
    assert L.fft_planar_workspace_size(None, 1, ctypes.byref(sz)) == fm.FFT_ERR_INVALID_ARG
    assert L.fft_plan_describe(None, ctypes.create_string_buffer(8), 8) == fm.FFT_ERR_INVALID_ARG
    assert L.fft_plan_destroy(None) == fm.FFT_OK


def test_binding_raises_fft_error():
    with pytest.raises(fm.FFTError) as ei:
        fm.fft_plan_create(2, [(1 << 23) + 1, 2], fm.FFT_C32)
    assert ei.value.status == fm.FFT_ERR_UNSUPPORTED_SIZE
    assert "exceeds" in str(ei.value)


def test_missing_library_fails_loudly(monkeypatch, tmp_path):
    """No fallback: without the built library every entry point raises."""
    monkeypatch.setattr(fm, "_lib", None)
    monkeypatch.setattr(fm, "lib_path", str(tmp_path / "libfftmi.so"))
    with pytest.raises(ImportError):
        fm.lib()
    with pytest.raises(ImportError):
        fm.fft_plan_query(1, [1024], fm.FFT_C32)
    with pytest.raises(ImportError):
        fm.fft_status_string(0)


@pytest.mark.parametrize("h,w,prec,status", [
    (0, 8, 0, fm.FFT_ERR_INVALID_ARG),
    (8, 0, 0, fm.FFT_ERR_INVALID_ARG),
    (8, 8, 3, fm.FFT_ERR_INVALID_ARG),
    (8388617, 1, 0, fm.FFT_ERR_UNSUPPORTED_SIZE),  # prime height beyond the chirp-z range
    (65536, 2048, 0, fm.FFT_ERR_UNSUPPORTED_SIZE),  # half spectrum beyond 2^26 points
    (16384, 2048, 1, fm.FFT_ERR_UNSUPPORTED_SIZE),  # beyond 2^24 points
])
def test_real_2d_plan_create_rejects(h, w, prec, status):
    hd = ctypes.c_void_p(12345)
    assert fm.lib().fft_plan_create_real_2d(ctypes.byref(hd), h, w, prec) == status
    assert hd.value is None


@pytest.mark.skipif(_have_gpu(), reason="host without a GPU only")
def test_valid_real_2d_plan_without_gpu_is_a_device_error():
    for h, w, prec in ((1, 1, 0), (8192, 16384, 0), (4096, 8192, 1), (64, 2, 0), (8, 7, 0), (6, 15, 1),
                       (97, 8, 0), (51, 16, 1)):
        hd = ctypes.c_void_p(12345)
        assert fm.lib().fft_plan_create_real_2d(ctypes.byref(hd), h, w, prec) == fm.FFT_ERR_DEVICE
        assert hd.value is None


def test_stream_copy_rejects_before_any_hip_call():
    L = fm.lib()
    assert L.fft_stream_copy(None, None, 0, None) == fm.FFT_OK  # nothing to copy
    assert L.fft_stream_copy(None, 4096, 64, None) == fm.FFT_ERR_INVALID_ARG
    assert L.fft_stream_copy(4096, None, 64, None) == fm.FFT_ERR_INVALID_ARG
    assert L.fft_stream_copy(4096 + 4, 1 << 20, 64, None) == fm.FFT_ERR_ALIGN
    assert L.fft_stream_copy(4096, 1 << 20, 60, None) == fm.FFT_ERR_ALIGN
    assert L.fft_stream_copy(4096, 4096 + 32, 64, None) == fm.FFT_ERR_OVERLAP
