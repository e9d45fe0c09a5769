"""Polynomial products on the GPU: bit-exact int64 against the fp64 oracle's
FFT route, against the exact schoolbook convolution (full on small cases,
sampled at full size) and against evaluation mod p = 2^61 - 1 at random
points (Schwartz-Zippel), which covers every coefficient."""
import math

import numpy as np
import pytest
import torch

import fft_convolution_amd as fm
import oracle
from fft_convolution_amd import workloads as wl

pytestmark = pytest.mark.gpu


def _ws(plan, batch, dev):
    nbytes = fm.fft_poly_mul_workspace_size(plan.handle, batch)
    return torch.empty(nbytes, dtype=torch.uint8, device=dev) if nbytes else None


def _gpu_mul(a_np, b_np, n, dev):
    a = torch.from_numpy(np.ascontiguousarray(a_np)).to(dev)
    b = torch.from_numpy(np.ascontiguousarray(b_np)).to(dev)
    plan = fm.Plan(n, torch.complex128)
    c, r = plan.poly_mul(a, b, residual=True)
    torch.cuda.synchronize()
    return c.cpu().numpy(), float(r.item())


@pytest.mark.parametrize("la,lb,batch", [
    (1, 1, 3), (1, 5, 2), (2, 3, 4), (7, 9, 3), (16, 17, 2), (64, 64, 5), (100, 29, 3),
    (1000, 24, 2), (2048, 2049, 2), (2048, 2048, 1),
])
def test_small_exact(dev, la, lb, batch):
    print("case la=%d lb=%d batch=%d" % (la, lb, batch), flush=True)
    rng = np.random.default_rng(la * 1000 + lb)
    a = rng.integers(-1000, 1000, size=(batch, la))
    b = rng.integers(-1000, 1000, size=(batch, lb))
    n = 1 << max(0, math.ceil(math.log2(la + lb - 1)))
    c, resid = _gpu_mul(a, b, n, dev)
    assert np.array_equal(c, oracle.schoolbook(a, b))
    assert resid < 0.1


@pytest.mark.parametrize("la,lb,n,batch", [
    (3000, 1097, 4096, 2),     # LDS-resident, largest fp64 row
    (4096, 4097, 8192, 2),     # 8192 points: the packed one-kernel product (1024 threads)
    (1, 8192, 8192, 3),        # b filling the row, a one coefficient
    (5000, 700, 8192, 5),      # ragged, a longer than N/2
    (8192, 8193, 16384, 2),    # smallest four-step
    (5000, 3000, 16384, 3),    # four-step, ragged lengths
    (1 << 15, 1 << 15, 1 << 16, 2),
    (10, 20, 1 << 16, 1),      # mostly zero padding
    # 512-point columns, operands in the lower half: the pipelined pass A
    (40000, 50001, 1 << 17, 3),    # 48 tiles: one per workgroup, grid not a multiple of 8
    (1 << 19, 3, 1 << 20, 1),      # mostly zero padding in b
    # rows of 2048 / 4096: half-length inverse rows spanning several wavefronts
    (1 << 19, 1 << 19, 1 << 20, 2),
    (1 << 20, (1 << 20) - 7, 1 << 21, 1),
    (1 << 21, 1 << 21, 1 << 22, 1),  # 1024-point columns, two tiles per workgroup
    (70000, 10, 1 << 17, 2),       # a longer than N/2: the plain pass A
    (600000, 100, 1 << 20, 1),     # the same with rows of 2048
    (5, 3000000, 1 << 22, 1),      # b longer than N/2, rows of 4096
])
def test_larger_against_oracle(dev, la, lb, n, batch):
    print("case la=%d lb=%d n=%d batch=%d" % (la, lb, n, batch), flush=True)
    a, b = wl.random_polys(max(la, lb), batch, seed=la + lb)
    a, b = a[:, :la], b[:, :lb]
    c, resid = _gpu_mul(a, b, n, dev)
    ref, _ = oracle.polymul_fft(a, b, n=n)
    assert np.array_equal(c, ref)
    ks = np.unique(np.concatenate([[0, 1, la + lb - 2], np.random.default_rng(0).integers(0, la + lb - 1, 50)]))
    assert np.array_equal(c[:, ks], oracle.schoolbook_sample(a, b, ks))
    assert resid < 0.1


@pytest.mark.parametrize("logn", list(range(13, 23)))
def test_random_split_sizes(dev, logn):
    """Every four-step size (N = 2^13 .. 2^22: rows of 64 .. 4096, columns
    of 128 .. 1024), with operand lengths and batch drawn from a seed: ragged
    lengths, either operand longer than N/2 or both within it, a batch not
    a multiple of anything.  Bit-exact against the oracle's fp64 FFT route."""
    n = 1 << logn
    rng = np.random.default_rng(1000 + logn)
    batch = int(rng.integers(1, 4))
    la = int(rng.integers(1, n))
    lb = int(rng.integers(max(1, n // 2 - la), n - la + 2))
    if la + lb - 1 > n:
        lb = n - la + 1
    print("case logn=%d la=%d lb=%d batch=%d" % (logn, la, lb, batch), flush=True)
    a, b = wl.random_polys(max(la, lb), batch, seed=logn)
    a, b = a[:, :la], b[:, :lb]
    c, resid = _gpu_mul(a, b, n, dev)
    ref, _ = oracle.polymul_fft(a, b, n=n)
    assert np.array_equal(c, ref)
    assert resid < 0.1


@pytest.mark.parametrize("n", [8192, 16384, 1 << 17, 12288, 10006])
def test_unbalanced_operands(dev, n):
    """Coefficients of 2^26 against 2^4: the packed routes (z = a + i b) give
    the smaller operand the larger one's rounding error unless b is scaled
    to a's binade first (fp64 model at N = 8192: error 51 unscaled, 5e-5
    scaled).  Every packed route: one kernel (8192), four-step passes (16384,
    2^17 with the pipelined pass A), mixed radix (12288) and chirp-z (10006)
    transforms between element-wise kernels.  Exact against the oracle's
    separate transforms, and both ways round (a small, b large)."""
    print("case unbalanced n=%d" % n, flush=True)
    rng = np.random.default_rng(n)
    la = lb = n // 2
    big = rng.integers(-(1 << 26), 1 << 26, size=(2, la))
    small = rng.integers(-(1 << 4), 1 << 4, size=(2, lb))
    oracle.set_threads(8)
    for a, b in ((big, small), (small, big)):
        c, resid = _gpu_mul(a, b, n, dev)
        ref, _ = oracle.polymul_fft(a, b)  # (the oracle's own power-of-two length)
        assert np.array_equal(c, ref)
        ks = np.unique(np.concatenate([[0, la + lb - 2], rng.integers(0, la + lb - 1, 30)]))
        assert np.array_equal(c[:, ks], oracle.schoolbook_sample(a, b, ks))
        assert resid < 0.1, resid


def test_closed_forms(dev):
    L = 4096
    k = np.arange(2 * L - 1)
    tri = np.minimum(k + 1, 2 * L - 1 - k)
    c, _ = _gpu_mul(np.full((1, L), 999), np.full((1, L), 999), 2 * L, dev)
    assert np.array_equal(c[0], 999 * 999 * tri)
    p, q = 30, 25
    c, _ = _gpu_mul(np.array([[math.comb(p, i) for i in range(p + 1)]]),
                    np.array([[math.comb(q, i) for i in range(q + 1)]]), 64, dev)
    assert c[0].tolist() == [math.comb(p + q, i) for i in range(p + q + 1)]


def test_workload_32_pairs_of_2p18(dev):
    # The full workload in the launch the benchmark times: bit-exact against
    # the oracle's fp64 FFT route on all 32 x (2^19 - 1) coefficients, sampled
    # schoolbook, the sum invariants and mod-p evaluation on every pair.
    L = 1 << 18
    a, b = wl.workload_input("polymul_l262144_b32")
    c, resid = _gpu_mul(a, b, 1 << 19, dev)
    assert c.shape == (32, 2 * L - 1)
    ref, ref_resid = oracle.polymul_fft(a, b, n=1 << 19)
    assert np.array_equal(c, ref)
    assert resid < 0.1
    rng = np.random.default_rng(5)
    ks = np.unique(np.concatenate([[0, 1, L - 1, L, 2 * L - 3, 2 * L - 2], rng.integers(0, 2 * L - 1, 250)]))
    assert np.array_equal(c[:, ks], oracle.schoolbook_sample(a, b, ks))
    for p in range(32):
        assert int(c[p].sum()) == int(a[p].sum()) * int(b[p].sum())
        z = int(rng.integers(2, oracle.MOD_P - 1))
        assert oracle.poly_eval_mod(c[p], z) == \
            oracle.poly_eval_mod(a[p], z) * oracle.poly_eval_mod(b[p], z) % oracle.MOD_P


def test_validation_on_device(dev):
    plan32 = fm.Plan(64, torch.complex64)
    plan = fm.Plan(64, torch.complex128)
    a = torch.ones(2, 40, dtype=torch.int64, device=dev)
    b = torch.ones(2, 30, dtype=torch.int64, device=dev)
    c = torch.empty(2, 69, dtype=torch.int64, device=dev)
    with pytest.raises(fm.FFTError) as e:
        fm.fft_poly_mul(plan32.handle, a, 40, b, 30, c, 2)
    assert e.value.status == fm.FFT_ERR_PRECISION
    with pytest.raises(fm.FFTError) as e:
        fm.fft_poly_mul(plan.handle, a, 40, b, 30, c, 2)   # 69 > 64
    assert e.value.status == fm.FFT_ERR_UNSUPPORTED_SIZE
    with pytest.raises(fm.FFTError) as e:
        fm.fft_poly_mul(plan.handle, a, 0, b, 30, c, 2)
    assert e.value.status == fm.FFT_ERR_INVALID_ARG
    with pytest.raises(fm.FFTError) as e:
        fm.fft_poly_mul(plan.handle, a, 20, b, 30, a, 2)   # c overlaps a
    assert e.value.status == fm.FFT_ERR_OVERLAP
    fm.fft_poly_mul(plan.handle, a, 20, b, 30, c, 0)        # batch 0: no-op


@pytest.mark.parametrize("n", [64, 8192, 16384])
def test_residual_flags_results_past_2p53(dev, n):
    """Products of at least 2^53 cannot be vouched for by the rounding
    residual (every double there is an integer): the residual must then read
    +inf, and values beyond int64 come back as INT64_MIN.  The one-kernel
    routes (N = 64, and N = 8192 packed) and the split route (N = 16384)."""
    print("case residual flag n=%d" % n, flush=True)
    plan = fm.Plan(n, torch.complex128)
    resid = torch.full((1,), -1.0, dtype=torch.float64, device=dev)
    # exact: small coefficients, residual finite and small
    a = torch.tensor([[3, 1, 4, 1, 5]], dtype=torch.int64, device=dev)
    b = torch.tensor([[2, 7, 1]], dtype=torch.int64, device=dev)
    c = torch.empty(1, 7, dtype=torch.int64, device=dev)
    fm.fft_poly_mul(plan.handle, a, 5, b, 3, c, 1, _ws(plan, 1, dev), resid)
    torch.cuda.synchronize()
    assert c.cpu().numpy().tolist() == oracle.schoolbook(a.cpu().numpy(), b.cpu().numpy()).tolist()
    assert 0.0 <= float(resid) < 0.1
    # (2^27 + 2^27 z)^2 = 2^54 + 2^55 z + 2^54 z^2: every coefficient >= 2^53
    big = torch.full((1, 2), 1 << 27, dtype=torch.int64, device=dev)
    c2 = torch.empty(1, 3, dtype=torch.int64, device=dev)
    fm.fft_poly_mul(plan.handle, big, 2, big, 2, c2, 1, _ws(plan, 1, dev), resid)
    torch.cuda.synchronize()
    assert math.isinf(float(resid)) and float(resid) > 0
    # (2^40)^2 = 2^80, beyond int64: stored as INT64_MIN, residual +inf
    huge = torch.full((1, 1), 1 << 40, dtype=torch.int64, device=dev)
    c3 = torch.empty(1, 1, dtype=torch.int64, device=dev)
    fm.fft_poly_mul(plan.handle, huge, 1, huge, 1, c3, 1, _ws(plan, 1, dev), resid)
    torch.cuda.synchronize()
    assert int(c3[0, 0]) == -(1 << 63)
    assert math.isinf(float(resid))

# Plans whose N is not a power of two: the plan's own transforms (mixed radix
# in one kernel or in passes, chirp-z fused or in passes) between the
# element-wise pack, product and rounding kernels.  Bit-exact against the
# oracle's FFT route (at the next power of two) and the schoolbook product.
@pytest.mark.parametrize("la,lb,n,batch", [
    (1, 1, 3, 2),               # smallest odd N: bins 1 and 2 pair
    (7, 6, 12, 2),              # even N: bin N/2 pairs with itself
    (500, 501, 1000, 3),        # mixed radix, one kernel
    (600, 409, 1009, 2),        # prime: chirp-z, one kernel (M = 2048)
    (6000, 6289, 12288, 2),     # mixed-radix passes (beyond 4096 complex128 points)
    (3000, 2004, 5003, 1),      # prime: chirp-z passes (M = 16384)
    (1, 200003, 200003, 1),     # a = constant, b fills N
    (100000, 100001, 200003, 1),  # prime N of 2 x 10^5: chirp-z passes, M = 2^19
])
def test_any_length_plan(dev, la, lb, n, batch):
    print("case la=%d lb=%d n=%d batch=%d" % (la, lb, n, batch), flush=True)
    rng = np.random.default_rng(la + 7 * lb + n)
    a = rng.integers(-1000, 1000, size=(batch, la))
    b = rng.integers(-1000, 1000, size=(batch, lb))
    plan = fm.Plan(n, torch.complex128)
    assert any(k in plan.describe() for k in ("path=mixed", "path=mixpass", "path=bluestein")), plan.describe()
    ws = fm.fft_poly_mul_workspace_size(plan.handle, batch)
    assert ws >= batch * n * 16
    c, resid = _gpu_mul(a, b, n, dev)
    oracle.set_threads(8)
    ref, _ = oracle.polymul_fft(a, b)
    assert np.array_equal(c, ref)
    if la * lb <= 4 * 10 ** 7:
        assert np.array_equal(c, oracle.schoolbook(a, b))
    else:
        ks = np.unique(np.concatenate([[0, 1, la + lb - 2], rng.integers(0, la + lb - 1, 30)]))
        assert np.array_equal(c[:, ks], oracle.schoolbook_sample(a, b, ks))
    assert 0.0 <= resid < 0.1

