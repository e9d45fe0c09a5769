"""Plans still referenced from the main module when the interpreter exits
are collected during teardown, when the binding module's globals may
already be cleared (to None): the finalizer must not look them up then.
Runs in a child process; no GPU needed (the plan objects carry no handle).
With torch imported first, the teardown order clears the binding's globals
before the main module's, which is what this reproduces."""
import os
import subprocess
import sys

CHILD = r"""
import torch
import fft_convolution_amd as fm
p = fm.Plan.__new__(fm.Plan)
p.handle = None
p._lib = None
q = fm.RealPlan.__new__(fm.RealPlan)
q.handle = None
q._lib = None
"""
ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_plan_finalized_cleanly_at_exit():
    r = subprocess.run([sys.executable, "-c", CHILD], capture_output=True, text=True, timeout=300, cwd=ROOT)
    assert r.returncode == 0, r.stderr
    assert "Exception ignored" not in r.stderr, r.stderr
