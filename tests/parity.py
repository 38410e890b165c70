"""Helpers shared by the GPU parity tests: device upload and the tolerance checks.

Tolerances (bf16 inputs, fp32 accumulation):
  O     max |O_gpu - O_ref| <= 1e-2 + half a bf16 ulp of O_ref.  The output is
        stored in bf16, whose rounding alone exceeds 1e-2 once |O| >= 4; the
        added half-ulp is that unavoidable rounding, nothing more.
  LSE   max-abs <= 1e-3, and -inf exactly where the reference is -inf.
  dQ, dK, dV   relative L2 error (whole tensor) <= 1e-2.  Where the reference
        is exactly zero (e.g. dQ of a one-key sequence, whose dS vanishes
        analytically) a relative error is undefined; there max |x| <= 1e-3.
"""
from __future__ import annotations

import math

import numpy as np

O_ATOL = 1e-2
LSE_ATOL = 1e-3
GRAD_REL_L2 = 1e-2
ZERO_ATOL = 1e-3


def dev(x, torch, dtype=None):
    """float32 array of bf16 values (or int32) -> contiguous CUDA tensor."""
    t = torch.from_numpy(np.ascontiguousarray(x))
    if dtype is None:
        dtype = torch.bfloat16 if x.dtype == np.float32 else torch.int32
    return t.to(device="cuda", dtype=dtype).contiguous()


def host(t):
    return t.float().cpu().numpy().astype(np.float64)


def half_ulp_bf16(x):
    a = np.abs(x)
    e = np.floor(np.log2(np.where(a > 0, a, 1.0)))
    return np.where(a > 0, np.exp2(e - 8), 0.0)


def check_o(got, ref, what="O"):
    got, ref = np.asarray(got, np.float64), np.asarray(ref, np.float64)
    assert got.shape == ref.shape, (what, got.shape, ref.shape)
    assert np.isfinite(got).all(), f"{what}: non-finite values"
    err = np.abs(got - ref) - half_ulp_bf16(ref)
    worst = float(err.max(initial=0.0))
    assert worst <= O_ATOL, f"{what}: max abs error beyond bf16 rounding {worst:.3e} > {O_ATOL}"
    return float(np.abs(got - ref).max(initial=0.0))


def check_lse(got, ref, what="LSE"):
    got, ref = np.asarray(got, np.float64), np.asarray(ref, np.float64)
    assert got.shape == ref.shape
    ninf = np.isneginf(ref)
    assert np.array_equal(np.isneginf(got), ninf), f"{what}: -inf pattern differs"
    assert np.isfinite(got[~ninf]).all(), f"{what}: non-finite values"
    worst = float(np.abs(got[~ninf] - ref[~ninf]).max(initial=0.0))
    assert worst <= LSE_ATOL, f"{what}: max abs error {worst:.3e} > {LSE_ATOL}"
    return worst


def rel_l2(got, ref):
    got, ref = np.asarray(got, np.float64), np.asarray(ref, np.float64)
    den = np.linalg.norm(ref)
    num = np.linalg.norm(got - ref)
    return num / den if den > 0 else num


def check_grad(got, ref, what):
    got = np.asarray(got, np.float64)
    assert got.shape == np.shape(ref), (what, got.shape, np.shape(ref))
    assert np.isfinite(got).all(), f"{what}: non-finite values"
    if np.linalg.norm(ref) == 0:
        worst = float(np.abs(got).max(initial=0.0))
        assert worst <= ZERO_ATOL, f"{what}: reference is zero, max |got| {worst:.3e} > {ZERO_ATOL}"
        return worst
    e = rel_l2(got, ref)
    assert e <= GRAD_REL_L2, f"{what}: rel L2 error {e:.3e} > {GRAD_REL_L2}"
    return e
