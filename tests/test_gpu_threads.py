"""Several host threads using the library at once (GPU): each creates its own
plans of every route (power-of-two rows, mixed radix, chirp-z in one kernel
and in passes, 2D with a transposed axis, real rows, poly-mul), runs them on a
stream of its own and destroys them, over several rounds.  The binding's
calls release the interpreter lock, so plan creation, execution and
destruction really overlap in the C library.  Every result must equal, bit for
bit, the same call made by one thread beforehand (the kernels are
deterministic), and no call may fail."""
import threading

import numpy as np
import pytest
import torch

import fft_convolution_amd as fm

pytestmark = pytest.mark.gpu

CASES = [
    ("c2c", 4096, 64), ("c2c", 1000, 96), ("c2c", 1009, 80), ("c2c", 4099, 8), ("c2c", 12288, 4),
    ("2d", (97, 48), 3), ("r2c", 1000, 40), ("poly", 1 << 13, 6),
]


def _inputs(dev):
    g = torch.Generator(device="cpu").manual_seed(31)
    out = []
    for kind, n, batch in CASES:
        if kind == "c2c":
            out.append(torch.randn(batch, n, dtype=torch.complex64, generator=g).to(dev))
        elif kind == "2d":
            out.append(torch.randn(batch, *n, dtype=torch.complex64, generator=g).to(dev))
        elif kind == "r2c":
            out.append(torch.randn(batch, n, dtype=torch.float32, generator=g).to(dev))
        else:
            a = torch.randint(-1000, 1000, (batch, n // 2), generator=g).to(dev)
            b = torch.randint(-1000, 1000, (batch, n // 2), generator=g).to(dev)
            out.append((a, b))
    return out


def _run(case, x):
    kind, n, _ = case
    if kind == "c2c":
        p = fm.Plan(n)
        return p.ifft(p.fft(x))
    if kind == "2d":
        return fm.Plan(n).fft2(x)
    if kind == "r2c":
        p = fm.RealPlan(n)
        return p.irfft(p.rfft(x))
    a, b = x
    return fm.Plan(n, torch.complex128).poly_mul(a, b)


def test_threads_share_the_library(dev):
    xs = _inputs(dev)
    want = [_run(c, x).cpu() for c, x in zip(CASES, xs)]
    errors, mismatches = [], []

    def worker(k):
        try:
            s = torch.cuda.Stream()
            with torch.cuda.stream(s):
                for rnd in range(3):
                    order = list(range(len(CASES)))
                    np.random.default_rng(100 * k + rnd).shuffle(order)
                    for i in order:
                        y = _run(CASES[i], xs[i])
                        s.synchronize()
                        if not torch.equal(y.cpu(), want[i]):
                            mismatches.append((k, rnd, CASES[i]))
        except Exception as e:  # reported below; a thread's exception is not raised here
            errors.append((k, repr(e)))

    threads = [threading.Thread(target=worker, args=(k,)) for k in range(4)]
    for t in threads:
        t.start()
    for t in threads:
        t.join(timeout=300)
    assert not any(t.is_alive() for t in threads), "a worker did not finish"
    assert not errors, errors
    assert not mismatches, mismatches
