"""Build libjfa.so (gfx950) in-tree with hipcc.

Every HIP source under csrc/ is compiled for gfx950 and linked into
``bwd_varlen_flashattention_amd/libjfa.so``.  Packed-FP32 VALU instructions are
disabled for all device code.  Run ``python -m bwd_varlen_flashattention_amd.build``.
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import shutil
import subprocess
import sys
import tempfile

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libjfa.so")
# Race-hunting variant: the same sources with JFA_DEBUG_SYNC (extra workgroup
# barriers before every LDS stage refill and epilogue); selected at run time with
# the JFA_LIBRARY environment variable.
DEBUG_SYNC_LIB = os.path.join(PKG, "libjfa_debug_sync.so")
SOURCES = ["api.cpp", "sched.hip", "fwd.hip", "fwd_ilp.hip", "bwd.hip", "bwd_wide.hip", "decode.hip", "check.hip"]
ARCH = "gfx950"
# Per-source code-generation options.  The backward's key-stationary kernel runs
# one wave per SIMD, so its LDS reads must be issued well ahead of the MFMAs that
# consume them; LLVM's iterative ILP scheduler does that (about 20% faster there).
# The forward's kernels are split over two units built from the same source:
# the latency-first scheduler for d <= 96 and the non-causal d = 128 kernels
# (3-7% faster there), the iterative ILP scheduler for the causal d = 128 and
# all d >= 192 kernels (3-13% faster there).  The backward's d >= 192 kernels
# are a unit of their own whose MFMA builtins take the VGPR form (their dK/dV
# accumulators are kept in AGPRs by hand-written MFMAs instead).
EXTRA_FLAGS = {"bwd.hip": ["-mllvm", "-amdgpu-sched-strategy=iterative-ilp"],
               "bwd_wide.hip": ["-mllvm", "-amdgpu-sched-strategy=iterative-ilp", "-mllvm", "-amdgpu-mfma-vgpr-form"],
               "fwd.hip": ["-mllvm", "-amdgpu-sched-strategy=max-ilp"],
               "fwd_ilp.hip": ["-mllvm", "-amdgpu-sched-strategy=iterative-ilp"]}


def _hipcc() -> str:
    for c in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if c and os.path.exists(c):
            return c
    raise RuntimeError("hipcc not found: the ROCm toolchain is required to build libjfa.so")


def common_flags() -> list[str]:
    return [
        f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-munsafe-fp-atomics",
        "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
        "-I", os.path.join(ROOT, "include"), "-I", CSRC,
        "-Wno-unused-result",
    ]


def _compile(src: str, build_dir: str = BUILD, defines: tuple = ()) -> str:
    obj = os.path.join(build_dir, os.path.splitext(src)[0] + ".o")
    cmd = [_hipcc(), *common_flags(), *EXTRA_FLAGS.get(src, []), *[f"-D{d}" for d in defines],
           "-x", "hip", "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"compile failed: {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    return obj


def device_asm(src: str, defines: tuple = ()) -> str:
    """gfx950 assembly of one source, compiled with the options the build uses."""
    with tempfile.TemporaryDirectory() as d:
        out = os.path.join(d, "unit.s")
        cmd = [_hipcc(), *common_flags(), *EXTRA_FLAGS.get(src, []), *[f"-D{x}" for x in defines],
               "-x", "hip", "-S", "--cuda-device-only", os.path.join(CSRC, src), "-o", out]
        r = subprocess.run(cmd, capture_output=True, text=True)
        if r.returncode != 0:
            raise RuntimeError(f"compile failed: {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
        with open(out) as f:
            return f.read()


def build(verbose: bool = False, debug_sync: bool = False) -> str:
    lib = DEBUG_SYNC_LIB if debug_sync else LIB
    build_dir = os.path.join(BUILD, "debug_sync") if debug_sync else BUILD
    defines = ("JFA_DEBUG_SYNC",) if debug_sync else ()
    os.makedirs(build_dir, exist_ok=True)
    with cf.ThreadPoolExecutor(max_workers=min(len(SOURCES), os.cpu_count() or 4)) as ex:
        objs = list(ex.map(lambda src: _compile(src, build_dir, defines), SOURCES))
    tmp = lib + ".tmp"
    cmd = [_hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed: {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, lib)
    if verbose:
        print(f"built {lib}")
    return lib


if __name__ == "__main__":
    build(verbose=True)
    build(verbose=True, debug_sync=True)
    sys.exit(0)
