"""The Python binding stays usable when the garbage collector runs a plan's
finalizer while lib() is loading a library (CPU).

lib() holds its lock while it loads a build, and the allocations of the load
can trigger a collection; a plan object caught in a reference cycle (say, one
a pytest.raises traceback still holds) is then finalized on the same thread
and frees its handle.  With a non-reentrant lock that call blocked forever.
The scenario is forced here in a child process: the library path is an
object whose __fspath__ runs a collection (lib() reads the path under its
lock), and an object in a cycle calls into the binding when finalized."""
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

CHILD = r"""
import gc, os, sys
sys.path.insert(0, %r)
import fft_convolution_amd as fm

class CollectingPath(os.PathLike):
    def __init__(self, p):
        self.p = p
    def __fspath__(self):
        gc.collect()          # under lib()'s lock
        return self.p

class Finalized:
    def __del__(self):
        try:
            fm.fft_plan_destroy(None)   # calls lib() from the finalizer
        except Exception:
            pass
        print("finalizer ran", flush=True)

built = fm.lib_path
gc.disable()
f = Finalized()
f.cycle = f
del f
fm._lib = None
fm.lib_path = CollectingPath(built)
fm.lib()
print("loaded", flush=True)
""" % ROOT


def test_finalizer_during_library_load_does_not_deadlock():
    r = subprocess.run([sys.executable, "-c", CHILD], capture_output=True, text=True, timeout=60)
    assert r.returncode == 0, r.stderr
    assert "finalizer ran" in r.stdout and "loaded" in r.stdout, r.stdout + r.stderr
