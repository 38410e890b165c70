"""Helpers shared by the GPU parity tests: device upload and the tolerance checks.

Tolerances (bf16 inputs, fp32 accumulation):
  O     |O_gpu - O_ref| <= max(1e-2, half a bf16 ulp of O_ref) per element.  The
        output is stored in bf16, whose rounding alone (half an ulp) exceeds
        1e-2 once |O_ref| >= 4; only there does the bound exceed 1e-2.
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
    err = np.abs(got - ref)
    bound = np.maximum(O_ATOL, half_ulp_bf16(ref))
    bad = err > bound
    if bad.any():
        i = np.unravel_index(int(np.argmax(err - bound)), err.shape)
        raise AssertionError(f"{what}: |error| {err[i]:.3e} > bound {bound[i]:.3e} at {i} "
                             f"(ref {ref[i]:.5g}, got {got[i]:.5g}); {int(bad.sum())} elements out of bound")
    return float(err.max(initial=0.0))


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


# ----------------------------------------------------------------------------- oracle runs
# The oracle evaluates sequences one at a time; these helpers run independent
# sequences (or broadcast items) on a thread pool with single-threaded BLAS, and
# assemble the packed outputs.  Nothing here changes what the oracle computes.

def oracle_workers() -> int:
    import os
    return max(1, min(16, len(os.sched_getaffinity(0))))


def _pool_map(fn, items):
    from concurrent.futures import ThreadPoolExecutor
    from threadpoolctl import threadpool_limits
    with threadpool_limits(limits=1):
        with ThreadPoolExecutor(oracle_workers()) as ex:
            return list(ex.map(fn, items))


def oracle_self_full(oracle, inp, scale=None):
    """Oracle O, LSE, dQ, dK, dV of a jagged self-attention input, whole tensors (float64)."""
    f64 = lambda x: x.astype(np.float64)
    hq, hkv, d = inp.q.shape[1], inp.k.shape[1], inp.q.shape[2]

    def one(b):
        qs, qe, ks, ke = inp.cu_q[b], inp.cu_q[b + 1], inp.cu_k[b], inp.cu_k[b + 1]
        cq, ck = np.array([0, qe - qs]), np.array([0, ke - ks])
        q, k, v = f64(inp.q[qs:qe]), f64(inp.k[ks:ke]), f64(inp.v[ks:ke])
        o, lse = oracle.attention_forward(q, k, v, cq, ck, inp.causal, scale)
        dq, dk, dv = oracle.attention_backward(q, k, v, f64(inp.do[qs:qe]), cq, ck, inp.causal, scale)
        return o, lse, dq, dk, dv

    res = _pool_map(one, range(len(inp.cu_q) - 1))
    tq, tk = inp.q.shape[0], inp.k.shape[0]
    o, dq = np.zeros((tq, hq, d)), np.zeros((tq, hq, d))
    lse = np.full((hq, tq), -np.inf)
    dk, dv = np.zeros((tk, hkv, d)), np.zeros((tk, hkv, d))
    for b, (ob, lb, dqb, dkb, dvb) in enumerate(res):
        qs, qe, ks, ke = inp.cu_q[b], inp.cu_q[b + 1], inp.cu_k[b], inp.cu_k[b + 1]
        o[qs:qe], lse[:, qs:qe], dq[qs:qe] = ob, lb, dqb
        dk[ks:ke], dv[ks:ke] = dkb, dvb
    return o, lse, dq, dk, dv


def oracle_bcast_full(oracle, inp):
    """Oracle outputs of a broadcast-Q input, whole tensors; dQ is the sum of the
    items' dQ taken in item order."""
    f64 = lambda x: x.astype(np.float64)
    q = f64(inp.q)

    def one(b):
        ks, ke = inp.cu_k[b], inp.cu_k[b + 1]
        k, v, ck = f64(inp.k[ks:ke]), f64(inp.v[ks:ke]), np.array([0, ke - ks])
        o, lse = oracle.broadcast_q_forward(q, k, v, ck)
        dq, dk, dv = oracle.broadcast_q_backward(q, k, v, f64(inp.do[b:b + 1]), ck)
        return o[0], lse[0], dq, dk, dv

    nb = len(inp.cu_k) - 1
    res = _pool_map(one, range(nb))
    tk = inp.k.shape[0]
    o = np.stack([r[0] for r in res]) if nb else np.zeros((0,) + inp.q.shape)
    lse = np.stack([r[1] for r in res]) if nb else np.zeros((0, inp.q.shape[1], inp.q.shape[0]))
    dq = np.zeros(inp.q.shape)
    dk, dv = np.zeros((tk,) + inp.k.shape[1:]), np.zeros((tk,) + inp.k.shape[1:])
    for b, r in enumerate(res):
        ks, ke = inp.cu_k[b], inp.cu_k[b + 1]
        dq += r[2]
        dk[ks:ke], dv[ks:ke] = r[3], r[4]
    return o, lse, dq, dk, dv
