"""GPU: the race-hunting build (JFA_DEBUG_SYNC: an extra workgroup barrier before
every LDS stage refill and epilogue) gives bit-for-bit the outputs of the normal
build on forward, backward (causal, GQA, d = 64 / 96 / 128 / 256, broadcast-Q) and
decode problems.  Every output is written by one workgroup in a fixed order, so any
difference would mean that a stage of the normal build is refilled while a reader
is unfinished (the hazard of the B300 page's bug-hunting section).  Each build runs
in a process of its own (tests/debug_sync_run.py)."""
import os
import subprocess
import sys

import numpy as np
import pytest

pytestmark = pytest.mark.gpu

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
PKG = os.path.join(ROOT, "bwd_varlen_flashattention_amd")


def _run(lib, out):
    env = dict(os.environ, JFA_LIBRARY=lib)
    print(f"running {os.path.basename(lib)}", flush=True)
    r = subprocess.run([sys.executable, "-u", os.path.join(HERE, "debug_sync_run.py"), out], env=env,
                       capture_output=True, text=True, timeout=240)
    print(r.stdout[-2000:], r.stderr[-2000:], flush=True)
    assert r.returncode == 0, f"{os.path.basename(lib)} run failed (rc {r.returncode})"
    return np.load(out)


def test_debug_sync_build_matches_normal_build(tmp_path):
    normal = os.path.join(PKG, "libjfa.so")
    debug = os.path.join(PKG, "libjfa_debug_sync.so")
    for lib in (normal, debug):
        assert os.path.exists(lib), f"{lib} is not built (run __graft_entry__.build())"
    a = _run(normal, str(tmp_path / "normal.npz"))
    b = _run(debug, str(tmp_path / "debug.npz"))
    assert sorted(a.files) == sorted(b.files) and len(a.files) > 20
    for name in a.files:
        np.testing.assert_array_equal(a[name], b[name], err_msg=name)
