"""fp64 CPU oracle for exact attention over jagged packed sequences.

TEST INFRASTRUCTURE ONLY.  This module is the reference the GPU path is held to.
Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import it; the product (the HIP library and its Python
binding) never calls it and shares no code with it.

What it computes is the plain definition of attention, written out per sequence
and per head in float64 with the full score matrix S materialised -- the naive
form described before tiling in the recap section of "Cutting edge isn't
plug-and-play: customising FlashAttention-4 on B300" (twelvelabs), and which
tiling reproduces exactly up to rounding (same page, same section).  No blocking, online softmax or fusion happens here.

Definitions followed (notation of the pages):
  forward   S = Q K^T * scale, scale = 1/sqrt(d) unless given (the pages write
            S = Q K^T and omit the scale; the 1/sqrt(d) factor is the standard
            attention scale and the reading adopted);
            softmax in two passes: row max m, then LSE = m + ln sum_j exp(S - m);
            P = exp(S - LSE); O = P V.
  backward  P is recomputed from S and the LSE saved by the forward (B300
            page, Phase 2 chunked-backward section and its pseudocode);
            dP = dO V^T (that pseudocode omits the transpose on V; the product
            only has shape [Bq, Bk] as dO V^T);
            delta = rowsum(P * dP), which equals rowsum(dO * O);
            dS = P * (dP - delta); dQ = scale dS K; dK = scale dS^T Q; dV = P^T dO.
  jagged    sequences are packed contiguously, boundaries in an offsets array
            ("Optimizing Jagged Flash Attention with TLX", the paragraph on GEM's
            jagged user sequences); each sequence attends only to itself.
  broadcast one dense Q is shared by every item; dQ is the sum over all items
            (same page and paragraph, the broadcast-Q production case).
  decode    one query per sequence against that sequence's whole KV
            ("Optimizing FlashAttention-4 for Efficient Inference", PR 1940,
            PR 1999/2104 and PR 2186 sections; paging and KV splitting change
            the memory layout and the order of reduction, not the result);
            a few new tokens per sequence (same page, "one or a few tokens at a
            time") are the last q_len rows of that sequence, so the optional
            causal mask is the bottom-right one below.

Readings where the pages are silent:
  * causal masking is bottom-right aligned: key j is visible to query i iff
    j <= i + (Lk - Lq); identical to top-left when Lq == Lk;
  * GQA: query head h uses kv head h // (Hq / Hkv);
  * a query row that sees no key gets O = 0 and LSE = -inf and contributes no
    gradient;
  * LSE uses the natural logarithm and is laid out [Hq, Tq] (broadcast-Q
    [B, Hq, Nq], decode [B, Hq]).
"""
from __future__ import annotations

import math

import numpy as np

__all__ = [
    "default_scale", "sequence_forward", "sequence_backward",
    "attention_forward", "attention_backward",
    "broadcast_q_forward", "broadcast_q_backward", "decode_forward", "decode_forward_multi",
]


def default_scale(head_dim: int, softmax_scale=None) -> float:
    """1/sqrt(d) unless an explicit positive scale is given."""
    if softmax_scale is None or softmax_scale <= 0:
        return 1.0 / math.sqrt(head_dim)
    return float(softmax_scale)


def _visible(lq: int, lk: int, causal: bool) -> np.ndarray:
    """Boolean [Lq, Lk] mask of the keys each query may attend to."""
    if not causal:
        return np.ones((lq, lk), dtype=bool)
    i = np.arange(lq)[:, None]
    j = np.arange(lk)[None, :]
    return j <= i + (lk - lq)


def sequence_forward(q, k, v, scale: float, causal: bool = False):
    """One sequence, one head.  q [Lq, d], k/v [Lk, d] (float64).

    Returns (O [Lq, d], LSE [Lq], P [Lq, Lk]).
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    lq, lk = q.shape[0], k.shape[0]
    vis = _visible(lq, lk, causal)
    has_key = vis.any(axis=1)

    s = scale * (q @ k.T)                                  # S = Q K^T * scale
    s = np.where(vis, s, -np.inf)
    lse = np.full(lq, -np.inf)
    p = np.zeros((lq, lk))
    if has_key.any():
        sr = s[has_key]
        m = sr.max(axis=1)                                   # pass 1: row max
        l = np.exp(sr - m[:, None]).sum(axis=1)              # pass 2: row sum
        lse[has_key] = m + np.log(l)                         # natural-log LSE
        p[has_key] = np.exp(sr - lse[has_key][:, None])      # P = exp(S - LSE); masked -> 0
    o = p @ v                                                # O = P V (rows with no key stay 0)
    return o, lse, p


def sequence_backward(q, k, v, do, scale: float, causal: bool = False):
    """One sequence, one head: analytic gradients of O = softmax(scale Q K^T) V.

    Returns (dQ, dK, dV, delta).  P is rebuilt from LSE by ``sequence_forward``.
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    do = np.asarray(do, dtype=np.float64)
    o, _lse, p = sequence_forward(q, k, v, scale, causal)
    dp = do @ v.T                                            # dP = dO V^T
    delta = (p * dp).sum(axis=1)                             # rowsum(P * dP)
    delta_o = (do * o).sum(axis=1)                           # the same number, as rowsum(dO * O)
    tol = 1e-9 * (1.0 + np.abs(delta_o).max(initial=0.0))
    if not np.allclose(delta, delta_o, rtol=1e-9, atol=tol):
        raise AssertionError("delta = rowsum(P*dP) disagrees with rowsum(dO*O)")
    ds = p * (dp - delta[:, None])                           # dS = P * (dP - delta)
    dq = scale * (ds @ k)
    dk = scale * (ds.T @ q)
    dv = p.T @ do
    return dq, dk, dv, delta


def _check_offsets(cu, total):
    cu = np.asarray(cu, dtype=np.int64)
    assert cu.ndim == 1 and cu[0] == 0 and cu[-1] == total and np.all(np.diff(cu) >= 0), "bad offsets"
    return cu


def attention_forward(q, k, v, cu_seqlens_q, cu_seqlens_k, causal: bool = False, softmax_scale=None):
    """Jagged packed attention forward.

    q [Tq, Hq, d], k/v [Tk, Hkv, d], offsets int [B+1].
    Returns O float64 [Tq, Hq, d] and LSE float64 [Hq, Tq].
    """
    tq, hq, d = q.shape
    tk, hkv, _ = k.shape
    assert hq % hkv == 0
    r = hq // hkv
    cq = _check_offsets(cu_seqlens_q, tq)
    ck = _check_offsets(cu_seqlens_k, tk)
    assert len(cq) == len(ck)
    scale = default_scale(d, softmax_scale)
    o = np.zeros((tq, hq, d))
    lse = np.full((hq, tq), -np.inf)
    for b in range(len(cq) - 1):
        qs, qe, ks, ke = cq[b], cq[b + 1], ck[b], ck[b + 1]
        for h in range(hq):
            g = h // r
            ob, lb, _ = sequence_forward(q[qs:qe, h], k[ks:ke, g], v[ks:ke, g], scale, causal)
            o[qs:qe, h] = ob
            lse[h, qs:qe] = lb
    return o, lse


def attention_backward(q, k, v, do, cu_seqlens_q, cu_seqlens_k, causal: bool = False, softmax_scale=None):
    """Jagged packed attention backward.  Returns dQ [Tq,Hq,d], dK, dV [Tk,Hkv,d] (float64).

    GQA: dK/dV of a kv head sum the contributions of all r query heads in its group.
    """
    tq, hq, d = q.shape
    tk, hkv, _ = k.shape
    r = hq // hkv
    cq = _check_offsets(cu_seqlens_q, tq)
    ck = _check_offsets(cu_seqlens_k, tk)
    scale = default_scale(d, softmax_scale)
    dq = np.zeros((tq, hq, d))
    dk = np.zeros((tk, hkv, d))
    dv = np.zeros((tk, hkv, d))
    for b in range(len(cq) - 1):
        qs, qe, ks, ke = cq[b], cq[b + 1], ck[b], ck[b + 1]
        for h in range(hq):
            g = h // r
            gq, gk, gv, _ = sequence_backward(q[qs:qe, h], k[ks:ke, g], v[ks:ke, g], do[qs:qe, h], scale, causal)
            dq[qs:qe, h] = gq
            dk[ks:ke, g] += gk
            dv[ks:ke, g] += gv
    return dq, dk, dv


def broadcast_q_forward(q, k, v, cu_seqlens_k, softmax_scale=None):
    """Broadcast-Q: item b attends with the shared Q [Nq, Hq, d] to its own jagged K/V.

    Returns O [B, Nq, Hq, d] and LSE [B, Hq, Nq] (float64).  No causal mask is defined here.
    """
    nq, hq, d = q.shape
    tk, hkv, _ = k.shape
    r = hq // hkv
    ck = _check_offsets(cu_seqlens_k, tk)
    nb = len(ck) - 1
    scale = default_scale(d, softmax_scale)
    o = np.zeros((nb, nq, hq, d))
    lse = np.full((nb, hq, nq), -np.inf)
    for b in range(nb):
        ks, ke = ck[b], ck[b + 1]
        for h in range(hq):
            g = h // r
            ob, lb, _ = sequence_forward(q[:, h], k[ks:ke, g], v[ks:ke, g], scale, False)
            o[b, :, h] = ob
            lse[b, h] = lb
    return o, lse


def broadcast_q_backward(q, k, v, do, cu_seqlens_k, softmax_scale=None):
    """Broadcast-Q backward.  do [B, Nq, Hq, d].  dQ [Nq, Hq, d] is summed over items in index order."""
    nq, hq, d = q.shape
    tk, hkv, _ = k.shape
    r = hq // hkv
    ck = _check_offsets(cu_seqlens_k, tk)
    nb = len(ck) - 1
    scale = default_scale(d, softmax_scale)
    dq = np.zeros((nq, hq, d))
    dk = np.zeros((tk, hkv, d))
    dv = np.zeros((tk, hkv, d))
    for b in range(nb):
        ks, ke = ck[b], ck[b + 1]
        for h in range(hq):
            g = h // r
            gq, gk, gv, _ = sequence_backward(q[:, h], k[ks:ke, g], v[ks:ke, g], do[b, :, h], scale, False)
            dq[:, h] += gq
            dk[ks:ke, g] += gk
            dv[ks:ke, g] += gv
    return dq, dk, dv


def decode_forward(q, k, v, cu_seqlens_k, softmax_scale=None):
    """Single-token decode: q [B, Hq, d] against the contiguous (pre-paging) K/V [Tk, Hkv, d].

    This is the jagged forward with one query per sequence and no mask.
    Returns O [B, Hq, d] and LSE [B, Hq] (float64).
    """
    nb, hq, d = q.shape
    cq = np.arange(nb + 1, dtype=np.int64)
    o, lse = attention_forward(q, k, v, cq, cu_seqlens_k, False, softmax_scale)
    return o, np.ascontiguousarray(lse.T)


def decode_forward_multi(q, k, v, cu_seqlens_k, causal: bool = False, softmax_scale=None):
    """Decode of q_len new tokens per sequence: q [B, q_len, Hq, d] against the
    contiguous (pre-paging) K/V [Tk, Hkv, d].

    The jagged forward with q_len queries per sequence; with causal the queries
    are the last q_len positions of the sequence (bottom-right alignment).
    Returns O [B, q_len, Hq, d] and LSE [B, q_len, Hq] (float64).
    """
    nb, lq, hq, d = q.shape
    cq = np.arange(nb + 1, dtype=np.int64) * lq
    o, lse = attention_forward(q.reshape(nb * lq, hq, d), k, v, cq, cu_seqlens_k, causal, softmax_scale)
    return o.reshape(nb, lq, hq, d), np.ascontiguousarray(lse.T).reshape(nb, lq, hq)
