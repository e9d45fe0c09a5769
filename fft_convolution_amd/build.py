"""Build the HIP library ``libfftmi.so`` in-tree for gfx950.

Each source under ``csrc/`` is compiled with hipcc in parallel, then linked
into ``fft_convolution_amd/libfftmi.so``.  Run ``python -m
fft_convolution_amd.build``.

Also built: ``libfftmi_poison.so``, the same library with the sources whose
kernels exchange through LDS compiled with ``-DFFTMI_LDS_POISON`` (every LDS
region set to NaN before a transform's first stage; a race or index check
for the GPU tests, never loaded by the product).
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(PKG, "libfftmi.so")
POISON_LIB = os.path.join(PKG, "libfftmi_poison.so")
BUILD_DIR = os.path.join(PKG, "_build")
# the sources whose kernels run the LDS exchange engine (stockham.hpp)
POISON_SOURCES = ["rows.hip", "tiles.hip", "polymul.hip", "bluestein.hip", "real.hip"]

SOURCES = ["api.cpp", "rows.hip", "tiles.hip", "polymul.hip", "bluestein.hip", "real.hip", "mixed.hip", "copy.hip"]
ARCH = "gfx950"
FLAGS = [
    "--offload-arch=" + ARCH, "-O3", "-std=c++17", "-fPIC",
    # no packed-FP32 instructions anywhere in the device code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I" + INCLUDE, "-I" + CSRC,
]
# Per-file additions.  The chirp-z kernel's forward transform reads a row
# whose upper half is zero (M >= 2N - 1): without signed zeros the compiler
# may drop the x + 0 terms of its first stage and the unused half of the
# inverse's last (17 % fewer instructions in the kernel's code, 1-2 % less
# time: 1009-point rows 534 -> 529 us); results differ at most in the sign
# of a zero.
FILE_FLAGS = {"bluestein.hip": ["-fno-signed-zeros"]}


def _hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found; the HIP library cannot be built")


def _compile(src: str, poison: bool = False) -> str:
    obj = os.path.join(BUILD_DIR, os.path.splitext(src)[0] + ("_poison.o" if poison else ".o"))
    cmd = [_hipcc()] + FLAGS + FILE_FLAGS.get(src, []) + (["-DFFTMI_LDS_POISON"] if poison else []) + \
        ["-c", os.path.join(CSRC, src), "-o", obj]
    if src.endswith(".cpp"):
        cmd.insert(1, "-x")
        cmd.insert(2, "hip")
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError("hipcc failed on %s:\n%s" % (src, res.stderr))
    return obj


def _link(objs, lib: str) -> None:
    tmp = lib + ".tmp%d" % os.getpid()
    cmd = [_hipcc(), "--offload-arch=" + ARCH, "-shared", "-fPIC", "-o", tmp] + objs
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError("link failed:\n%s" % res.stderr)
    os.replace(tmp, lib)


def build(verbose: bool = True) -> str:
    """Compile every source and link libfftmi.so (and libfftmi_poison.so);
    returns the path of libfftmi.so."""
    os.makedirs(BUILD_DIR, exist_ok=True)
    jobs = [(src, False) for src in SOURCES] + [(src, True) for src in POISON_SOURCES]
    # the longest compiles first
    jobs.sort(key=lambda j: -os.path.getsize(os.path.join(CSRC, j[0])))
    workers = max(1, min(8, os.cpu_count() or 1))
    with cf.ThreadPoolExecutor(workers) as ex:
        built = dict(zip(jobs, ex.map(lambda j: _compile(*j), jobs)))
    objs = [built[(src, False)] for src in SOURCES]
    _link(objs, LIB)
    _link([built[(src, True)] if src in POISON_SOURCES else built[(src, False)] for src in SOURCES], POISON_LIB)
    if verbose:
        print("built", LIB, "and", POISON_LIB)
    return LIB


if __name__ == "__main__":
    build()
    sys.exit(0)
