"""The planner on the CPU (fft_plan_query: the plan fft_plan_create would
make, without a device): which path each size takes and the sizes the
kernels are given, checked against the rules the kernels rely on."""
import math

import pytest

import fft_convolution_amd as fm

LDS_MAX = {0: 8192, 1: 4096}
MIXED_MAX = {0: 8192, 1: 4096}


def _q(rank, dims, prec):
    return fm.fft_plan_query(rank, dims, prec)


def _field(desc, key):
    for tok in desc.split():
        if tok.startswith(key + "="):
            return tok.split("=", 1)[1]
    return None


def _smooth(n):
    for p in (2, 3, 5, 7, 11, 13):
        while n % p == 0:
            n //= p
    return n == 1


@pytest.mark.parametrize("prec", [0, 1])
def test_power_of_two_paths(prec):
    top = 26 if prec == 0 else 24
    for logn in range(0, top + 1):
        n = 1 << logn
        d = _q(1, [n], prec)
        if n == 1:
            assert "path=copy" in d
        elif n <= 2 * LDS_MAX[prec]:
            # rows of twice the LDS range (16384 complex64, 8192 complex128):
            # one 1024-thread workgroup a row
            assert "path=rows" in d, d
        else:
            assert "path=multipass" in d
            r = [int(x) for x in _field(d, "radices").split("x")]
            # super-stages of at most 512 points, as few as possible, as even as possible, larger first
            assert math.prod(r) == n and max(r) <= 512
            assert len(r) == math.ceil(logn / 9)
            assert r == sorted(r, reverse=True) and r[0] <= 2 * r[-1]


@pytest.mark.parametrize("prec", [0, 1])
def test_every_length_up_to_20000(prec):
    for n in range(2, 20001):
        d = _q(1, [n], prec)
        if n & (n - 1) == 0:
            continue
        if _smooth(n) and n <= MIXED_MAX[prec]:
            assert "path=mixed" in d, (n, d)
            r = [int(x) for x in _field(d, "radices").split("x")]
            assert math.prod(r) == n and set(r) <= {2, 3, 4, 5, 7, 8, 9, 11, 13}, (n, d)
            assert len(r) <= 16
        elif _smooth(n):
            # beyond one kernel: two super-stage passes of radix <= 512 (three
            # only past 512^2), as even as possible, larger first
            assert "path=mixpass" in d, (n, d)
            r = [int(x) for x in _field(d, "radices").split("x")]
            assert math.prod(r) == n and max(r) <= 512 and len(r) == 2, (n, d)
            assert r == sorted(r, reverse=True), (n, d)
            best = max(min(a, n // a) for a in range(2, 513) if n % a == 0 and n // a <= 512)
            assert r[1] == best, (n, d)
        else:
            assert "path=bluestein" in d, (n, d)
            m = int(_field(d, "m"))
            assert m & (m - 1) == 0 and m >= 2 * n - 1 and m < 4 * n - 2, (n, d)
            # one kernel for M up to twice the LDS range (a 1024-thread workgroup a row)
            assert d.endswith("fused") == (m <= 2 * LDS_MAX[prec]), (n, d)


@pytest.mark.parametrize("prec", [0, 1])
def test_every_2d_shape_has_a_layout(prec):
    top = 13 if prec == 0 else 12
    cap = 2048 if prec == 0 else 1024
    for lh in range(0, top + 1):
        for lw in range(0, top + 1):
            h, w = 1 << lh, 1 << lw
            d = _q(2, [h, w], prec)
            assert "path=nd" in d, (h, w, d)
            axes = int(_field(d, "axes"))
            assert axes == (h > 1) + (w > 1)
            if axes < 2:
                continue
            f = int(_field(d, "fold") or _field(d, "split"))
            lc = int(_field(d, "col_len"))
            # the column transform of H points is split H = F * Lc
            assert f * lc == h and lc <= cap and f <= 16, (h, w, d)
            if h <= 512:
                assert f == 1 and "fold=" in d, (h, w, d)
            if "split=" in d:
                # only where F rows cannot be folded into the row pass
                assert w == 2 or w * (1 if prec == 0 else 2) >= 8192 or lc > 512, (h, w, d)


def test_3d_layouts():
    assert "axes=3" in _q(3, [256, 256, 256], 0)
    assert "axes=2" in _q(3, [1, 64, 128], 0)
    assert "axes=1" in _q(3, [1, 1, 4096], 1)
    assert "split=" in _q(3, [4, 8192, 2], 0)
    with pytest.raises(fm.FFTError) as e:
        _q(3, [4096, 8, 8], 0)
    assert e.value.status == fm.FFT_ERR_UNSUPPORTED_SIZE


@pytest.mark.parametrize("rank,dims,prec,status", [
    (0, [8], 0, fm.FFT_ERR_INVALID_ARG),
    (1, [0], 0, fm.FFT_ERR_INVALID_ARG),
    (1, [8], 5, fm.FFT_ERR_INVALID_ARG),
    (2, [(1 << 23) + 1, 2], 0, fm.FFT_ERR_UNSUPPORTED_SIZE),
    (1, [(1 << 23) + 1], 1, fm.FFT_ERR_UNSUPPORTED_SIZE),
    (1, [1 << 27], 0, fm.FFT_ERR_UNSUPPORTED_SIZE),
    (2, [8, 16384], 1, fm.FFT_ERR_UNSUPPORTED_SIZE),   # rows beyond 8192 (complex128)
    (2, [8, 32768], 0, fm.FFT_ERR_UNSUPPORTED_SIZE),   # rows beyond 16384 (complex64)
    (2, [16384, 8], 0, fm.FFT_ERR_UNSUPPORTED_SIZE),   # an outer axis beyond 8192
    (3, [4, 16384, 4], 0, fm.FFT_ERR_UNSUPPORTED_SIZE),
])
def test_query_rejects_as_create_does(rank, dims, prec, status):
    with pytest.raises(fm.FFTError) as e:
        _q(rank, dims, prec)
    assert e.value.status == status


def test_mixpass_splits():
    """Large 13-smooth lengths: the fewest passes, the most even split
    (largest smallest radix), larger radices first; radices up to 512, or up
    to 1024 where two passes then do instead of three (radices above 512 take
    no factor 11 or 13)."""
    cases = {10 ** 6: [1000, 1000], 3 << 18: [1024, 768], 1001000: [110, 100, 91], 3 << 20: [192, 128, 128],
             5 ** 9: [125, 125, 125], 12288: [128, 96], 30030: [182, 165], 3 * 65536: [512, 384],
             7 << 20: [448, 128, 128]}
    for n, want in cases.items():
        for prec in (0, 1):
            d = _q(1, [n], prec)
            assert "path=mixpass" in d and _field(d, "radices") == "x".join(map(str, want)), (n, d)
    # between the one-kernel limits of the two precisions: complex128 only
    assert "path=mixpass" in _q(1, [6000], 1) and "path=mixed" in _q(1, [6000], 0)
    # a prime factor above 13, or beyond 2^23: Bluestein or rejected
    assert "path=bluestein" in _q(1, [1000003], 0)


def test_ndmixed_layouts():
    """Rank 2 / 3 with a dimension that is not a power of two: the innermost
    axis by its rank-1 route, every other axis longer than 1 as passes (one
    up to 1024 points when the length has no factor 11 or 13, else up to
    512)."""
    d = _q(2, [1000, 1000], 0)
    assert "path=ndmixed" in d and "rows=[mixed radices=8x5x5x5]" in d and d.endswith("axis1=1000")
    assert _q(2, [1024, 1000], 0).endswith("axis1=1024")
    assert _q(2, [2000, 8], 0).endswith("axis1=50x40")
    assert _q(2, [1001, 8], 1).endswith("axis1=77x13")
    assert _q(2, [845, 6], 0).endswith("axis1=65x13")
    d = _q(2, [64, 97], 1)
    assert "rows=[bluestein" in d and d.endswith("axis1=64")
    d = _q(3, [12, 30, 50], 0)
    assert d.endswith("axis1=30 axis2=12")
    d = _q(2, [1000, 1], 0)
    assert "rows=[copy]" in d and d.endswith("axis1=1000")
    assert "axis" not in _q(2, [1, 1000], 0)
    # the power-of-two shapes keep their own path
    assert "path=nd " in _q(2, [64, 32], 0)


def test_transposed_axes_planned():
    """Axes other than the innermost whose length has a prime factor above 13
    are planned as the rank-1 route of their length over the transposed axis;
    13-smooth axes keep their passes."""
    d = _q(2, [17, 8], 0)
    assert "axis1=transposed[bluestein" in d, d
    d = _q(3, [19, 5, 8], 0)
    assert "axis1=5 " in d and "axis2=transposed[bluestein" in d, d
    d = _q(2, [4099, 3], 1)
    assert "axis1=transposed[bluestein m=16384" in d, d
    assert "transposed" not in _q(2, [1001, 12], 0)


def test_poly_mul_split_described():
    """complex128 plans in passes carry the poly-mul split N1 x N2 (columns of
    at most 512 points, 1024 beyond 2^21; rows of at most 4096); 8192 points
    run as one kernel and carry none."""
    assert "poly=" not in _q(1, [1 << 13], 1)
    for logn, n1, n2 in [(14, 128, 128), (17, 256, 512), (19, 1024, 512), (20, 2048, 512), (21, 4096, 512),
                         (22, 4096, 1024)]:
        d = _q(1, [1 << logn], 1)
        assert _field(d, "poly") == "%dx%d" % (n1, n2), d
    assert "poly=" not in _q(1, [1 << 20], 0)   # complex64 plans have no poly-mul split
