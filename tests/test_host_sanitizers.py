"""The host code under AddressSanitizer and UndefinedBehaviorSanitizer (CPU).

Two drivers in tests/sanitize/ are built with -fsanitize=address,undefined
(host code only: the .hip files are compiled with --cuda-host-only) and run:

* host_driver.cpp -- the library's planner, twiddle / schedule generators and
  argument validation (api.cpp included whole, the kernels' host launchers
  linked from host-only objects, with no-op code-object registration from
  no_device_code.c; no GPU is touched, no kernel launched);
* oracle_driver.c -- the C oracle's routines on many small shapes, checked
  against one another.

Each must exit 0 with no sanitizer report.  The binaries are cached under
tests/sanitize/_build and rebuilt when a source is newer."""
import os
import shutil
import subprocess

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
SAN = os.path.join(HERE, "sanitize")
BUILD = os.path.join(SAN, "_build")
CSRC = os.path.join(ROOT, "fft_convolution_amd", "csrc")
HIP_SOURCES = ["rows.hip", "tiles.hip", "polymul.hip", "bluestein.hip", "real.hip", "mixed.hip", "copy.hip"]
SAN_ENV = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:abort_on_error=0:halt_on_error=1",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")


def _newer(target, sources):
    return not os.path.exists(target) or any(os.path.getmtime(s) > os.path.getmtime(target) for s in sources)


def _run(cmd, **kw):
    res = subprocess.run(cmd, capture_output=True, text=True, **kw)
    assert res.returncode == 0, "%s\n%s\n%s" % (" ".join(cmd), res.stdout[-3000:], res.stderr[-5000:])
    return res


def _hipcc():
    for cand in (os.environ.get("HIPCC"), shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    pytest.skip("hipcc not found")


# Host-only compilation: each -fsanitize= goes to the host pass alone.
HOST_SAN = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
            "-Xarch_host", "-fno-sanitize-recover=all", "-Xarch_host", "-fno-omit-frame-pointer"]


def test_oracle_under_sanitizers():
    cc = shutil.which("gcc") or pytest.skip("gcc not found")
    os.makedirs(BUILD, exist_ok=True)
    exe = os.path.join(BUILD, "oracle_driver")
    srcs = [os.path.join(SAN, "oracle_driver.c"), os.path.join(ROOT, "oracle", "oracle.c")]
    if _newer(exe, srcs):
        _run([cc, "-O1", "-g", "-fopenmp", "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
              "-fno-omit-frame-pointer", "-I" + os.path.join(ROOT, "oracle"), srcs[0], "-lm", "-o", exe])
    res = _run([exe], env=SAN_ENV, timeout=600)
    assert "0 failed" in res.stdout
    assert "runtime error" not in res.stderr and "AddressSanitizer" not in res.stderr


def test_host_library_under_sanitizers():
    hipcc = _hipcc()
    clang = "/opt/rocm/lib/llvm/bin/clang++"
    if not os.path.exists(clang):
        pytest.skip("ROCm clang++ not found")
    os.makedirs(BUILD, exist_ok=True)
    flags = ["--offload-arch=gfx950", "--cuda-host-only", "-O1", "-g", "-std=c++17", "-fPIC",
             "-I" + os.path.join(ROOT, "include"), "-I" + CSRC] + HOST_SAN
    headers = [os.path.join(CSRC, f) for f in os.listdir(CSRC) if f.endswith(".hpp")]
    headers.append(os.path.join(ROOT, "include", "fftmi.h"))
    objs = []
    jobs = []
    for src in HIP_SOURCES + ["host_driver.cpp"]:
        path = os.path.join(SAN if src == "host_driver.cpp" else CSRC, src)
        deps = [path] + headers + ([os.path.join(CSRC, "api.cpp")] if src == "host_driver.cpp" else [])
        obj = os.path.join(BUILD, os.path.splitext(src)[0] + ".o")
        objs.append(obj)
        if _newer(obj, deps):
            jobs.append(subprocess.Popen([hipcc] + flags + ["-x", "hip", "-c", path, "-o", obj],
                                         stdout=subprocess.PIPE, stderr=subprocess.PIPE, text=True))
    for j in jobs:
        out, err = j.communicate()
        assert j.returncode == 0, err[-5000:]
    # Host-only objects still name their (absent) code objects: give those
    # symbols storage, and link no-op registration hooks in place of the
    # HIP runtime's (tests/sanitize/no_device_code.c).
    names = set()
    for obj in objs:
        res = _run(["nm", "-u", obj])
        names.update(w for w in res.stdout.split() if w.startswith(("__hip_fatbin_", "__hip_gpubin_handle_")))
    gen = os.path.join(BUILD, "code_object_symbols.c")
    with open(gen, "w") as f:
        for n in sorted(names):
            f.write(("char %s[64];\n" if n.startswith("__hip_fatbin_") else "void* %s;\n") % n)
    exe = os.path.join(BUILD, "host_driver")
    _run([clang, "-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-o", exe] + objs +
         ["-x", "c", gen, os.path.join(SAN, "no_device_code.c"), "-x", "none",
          "-L/opt/rocm/lib", "-Wl,-rpath,/opt/rocm/lib", "-lamdhip64", "-lm"])
    res = _run([exe], env=SAN_ENV, timeout=600)
    assert "0 failed" in res.stdout
    assert "runtime error" not in res.stderr and "AddressSanitizer" not in res.stderr
