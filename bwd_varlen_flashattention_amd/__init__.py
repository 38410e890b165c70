"""Python binding of libjfa.so: exact jagged FlashAttention fwd/bwd and split-KV
paged decode on MI355X (gfx950).

The functions keep the C ABI's names and only marshal arguments: they check
dtypes and shapes, allocate outputs and the workspace with torch on the current
device, and call the library on torch's current stream.  Every step of the
computation runs in the library's HIP kernels; there is no CPU or PyTorch
fallback.
"""
from __future__ import annotations

import ctypes
import math
from typing import Optional

from . import _lib
from ._lib import AttnParams, DecodeParams, JfaError, load  # noqa: F401

__all__ = ["jfa_fwd", "jfa_bwd", "jfa_decode_paged", "jfa_decode_num_splits", "timing", "JfaError", "load"]


def _torch():
    import torch
    return torch


def _ptr(t) -> Optional[int]:
    return None if t is None or t.numel() == 0 else t.data_ptr()


def _stream():
    torch = _torch()
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def _check_bf16(name, t, ndim):
    torch = _torch()
    if t.dtype != torch.bfloat16 or t.dim() != ndim or not t.is_cuda or not t.is_contiguous():
        raise ValueError(f"{name}: expected a contiguous bfloat16 CUDA tensor with {ndim} dims, got "
                         f"{t.dtype} {tuple(t.shape)} cuda={t.is_cuda} contiguous={t.is_contiguous()}")


def _check_i32(name, t):
    torch = _torch()
    if t.dtype != torch.int32 or not t.is_cuda or not t.is_contiguous():
        raise ValueError(f"{name}: expected a contiguous int32 CUDA tensor")


def _attn_params(q, k, cu_q, cu_k, max_q, max_k, causal, scale, broadcast_q, batch, fp8=False,
                 q_scale=None, k_scale=None, v_scale=None):
    nb = batch if batch is not None else (cu_k.numel() - 1)
    sc = lambda x: float(x) if x is not None else 1.0
    return AttnParams(
        batch=nb, num_heads_q=q.shape[1], num_heads_kv=k.shape[1], head_dim=q.shape[2],
        total_q=q.shape[0], total_k=k.shape[0], max_seqlen_q=int(max_q), max_seqlen_k=int(max_k),
        causal=int(bool(causal)), broadcast_q=int(bool(broadcast_q)),
        softmax_scale=float(scale) if scale is not None else 0.0,
        qkv_dtype=1 if fp8 else 0, q_scale=sc(q_scale), k_scale=sc(k_scale), v_scale=sc(v_scale))


def _is_fp8(t) -> bool:
    torch = _torch()
    return t.dtype in (getattr(torch, "float8_e4m3fn", None), torch.uint8)


def _check_fp8(name, t, ndim):
    if not _is_fp8(t) or t.dim() != ndim or not t.is_cuda or not t.is_contiguous():
        raise ValueError(f"{name}: expected a contiguous float8_e4m3fn (or uint8 e4m3 bytes) CUDA tensor "
                         f"with {ndim} dims, got {t.dtype} {tuple(t.shape)}")


def jfa_fwd(q, k, v, cu_seqlens_q, cu_seqlens_k, max_seqlen_q: int, max_seqlen_k: int,
            causal: bool = False, softmax_scale: Optional[float] = None, broadcast_q: bool = False,
            out=None, lse=None, workspace=None, q_scale: Optional[float] = None,
            k_scale: Optional[float] = None, v_scale: Optional[float] = None):
    """Jagged forward.  Self-attention: q [Tq,Hq,d], k/v [Tk,Hkv,d] -> o [Tq,Hq,d], lse [Hq,Tq].
    Broadcast-Q: q [Nq,Hq,d] shared by B items -> o [B,Nq,Hq,d], lse [B,Hq,Nq].
    q, k, v are all bfloat16, or all e4m3 (float8_e4m3fn or raw uint8 bytes) with
    per-tensor scales q_scale, k_scale, v_scale (default 1); o is bfloat16 either way."""
    torch = _torch()
    lib = load()
    fp8 = _is_fp8(q)
    chk = _check_fp8 if fp8 else _check_bf16
    chk("q", q, 3); chk("k", k, 3); chk("v", v, 3)
    _check_i32("cu_seqlens_k", cu_seqlens_k)
    if not broadcast_q:
        _check_i32("cu_seqlens_q", cu_seqlens_q)
    nb = cu_seqlens_k.numel() - 1
    p = _attn_params(q, k, cu_seqlens_q, cu_seqlens_k, max_seqlen_q, max_seqlen_k, causal, softmax_scale,
                     broadcast_q, nb, fp8, q_scale, k_scale, v_scale)
    if broadcast_q:
        o_shape, lse_shape = (nb, q.shape[0], q.shape[1], q.shape[2]), (nb, q.shape[1], q.shape[0])
    else:
        o_shape, lse_shape = tuple(q.shape), (q.shape[1], q.shape[0])
    o = out if out is not None else torch.empty(o_shape, dtype=torch.bfloat16, device=q.device)
    l = lse if lse is not None else torch.empty(lse_shape, dtype=torch.float32, device=q.device)
    need = lib.jfa_fwd_workspace_size(ctypes.byref(p))
    ws = workspace if workspace is not None else torch.empty(max(need, 1), dtype=torch.uint8, device=q.device)
    st = lib.jfa_fwd(ctypes.byref(p), _ptr(q), _ptr(k), _ptr(v),
                     None if broadcast_q else _ptr(cu_seqlens_q), _ptr(cu_seqlens_k),
                     _ptr(o), _ptr(l), ws.data_ptr(), ws.numel(), _stream())
    _lib.check(st, "jfa_fwd")
    return o, l


def jfa_bwd(q, k, v, o, lse, dout, cu_seqlens_q, cu_seqlens_k, max_seqlen_q: int, max_seqlen_k: int,
            causal: bool = False, softmax_scale: Optional[float] = None, broadcast_q: bool = False,
            dq=None, dk=None, dv=None, workspace=None):
    """Jagged backward: returns (dq, dk, dv) in the layouts of q, k, v."""
    torch = _torch()
    lib = load()
    for n, t in (("q", q), ("k", k), ("v", v)):
        _check_bf16(n, t, 3)
    _check_bf16("o", o, 4 if broadcast_q else 3)
    _check_bf16("dout", dout, 4 if broadcast_q else 3)
    if lse.dtype != torch.float32 or not lse.is_contiguous():
        raise ValueError("lse: expected contiguous float32")
    nb = cu_seqlens_k.numel() - 1
    p = _attn_params(q, k, cu_seqlens_q, cu_seqlens_k, max_seqlen_q, max_seqlen_k, causal, softmax_scale,
                     broadcast_q, nb)
    dq = dq if dq is not None else torch.empty_like(q)
    dk = dk if dk is not None else torch.empty_like(k)
    dv = dv if dv is not None else torch.empty_like(v)
    need = lib.jfa_bwd_workspace_size(ctypes.byref(p))
    ws = workspace if workspace is not None else torch.empty(max(need, 1), dtype=torch.uint8, device=q.device)
    st = lib.jfa_bwd(ctypes.byref(p), _ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), _ptr(dout),
                     None if broadcast_q else _ptr(cu_seqlens_q), _ptr(cu_seqlens_k),
                     _ptr(dq), _ptr(dk), _ptr(dv), ws.data_ptr(), ws.numel(), _stream())
    _lib.check(st, "jfa_bwd")
    return dq, dk, dv


def _kv_fp8(k_cache) -> bool:
    torch = _torch()
    return k_cache.dtype in (getattr(torch, "float8_e4m3fn", None), torch.uint8)


def _decode_params(q, k_cache, page_table, num_splits, scale, causal=False, k_scale=None, v_scale=None,
                   q_scale=None):
    """q is [B, Hq, d] (one token per sequence) or [B, q_len, Hq, d]; an fp8 cache
    or query (float8_e4m3fn, or its raw bytes as uint8) selects the e4m3 path."""
    q_len = 1 if q.dim() == 3 else q.shape[1]
    fp8 = _kv_fp8(k_cache)
    q8 = _is_fp8(q)
    return DecodeParams(
        batch=q.shape[0], num_heads_q=q.shape[-2], num_heads_kv=k_cache.shape[2], head_dim=q.shape[-1],
        page_size=k_cache.shape[1], num_pages=k_cache.shape[0], max_pages_per_seq=page_table.shape[1],
        num_splits=int(num_splits), softmax_scale=float(scale) if scale is not None else 0.0,
        q_len=int(q_len), causal=int(bool(causal)), kv_dtype=1 if fp8 else 0,
        k_scale=float(k_scale) if k_scale is not None else 0.0, v_scale=float(v_scale) if v_scale is not None else 0.0,
        q_dtype=1 if q8 else 0, q_scale=float(q_scale) if q_scale is not None else 0.0)


def _check_cache(name, t):
    torch = _torch()
    if _kv_fp8(t):
        if t.dim() != 4 or not t.is_cuda or not t.is_contiguous():
            raise ValueError(f"{name}: expected a contiguous 4-d CUDA fp8 (e4m3) tensor, got {tuple(t.shape)}")
    else:
        _check_bf16(name, t, 4)


def jfa_decode_num_splits(q, k_cache, page_table, num_splits: int = 0) -> int:
    p = _decode_params(q, k_cache, page_table, num_splits, None)
    return int(load().jfa_decode_num_splits(ctypes.byref(p)))


def jfa_decode_paged(q, k_cache, v_cache, page_table, seqlens_k, num_splits: int = 0,
                     softmax_scale: Optional[float] = None, out=None, lse=None, workspace=None,
                     causal: bool = False, k_scale: Optional[float] = None, v_scale: Optional[float] = None,
                     q_scale: Optional[float] = None):
    """Paged decode of q_len new tokens per sequence against a paged KV cache.

    q [B, Hq, d] (one token) or [B, q_len, Hq, d] (q_len <= 16); caches
    [num_pages, page_size, Hkv, d] -> o (bfloat16, shaped like q), lse [B, Hq] or [B, q_len, Hq].
    causal: the q_len tokens are the last ones of each sequence (bottom-right mask).
    FP8 caches (torch.float8_e4m3fn or raw uint8 bytes): K = k_scale * cache value,
    V = v_scale * cache value.  An FP8 q: Q = q_scale * q value.
    """
    torch = _torch()
    lib = load()
    if q.dim() not in (3, 4):
        raise ValueError("q must be [B, Hq, d] or [B, q_len, Hq, d]")
    (_check_fp8 if _is_fp8(q) else _check_bf16)("q", q, q.dim())
    _check_cache("k_cache", k_cache); _check_cache("v_cache", v_cache)
    if _kv_fp8(k_cache) != _kv_fp8(v_cache):
        raise ValueError("k_cache and v_cache must have the same element type")
    _check_i32("page_table", page_table); _check_i32("seqlens_k", seqlens_k)
    p = _decode_params(q, k_cache, page_table, num_splits, softmax_scale, causal, k_scale, v_scale, q_scale)
    o = out if out is not None else torch.empty(q.shape, dtype=torch.bfloat16, device=q.device)
    l = lse if lse is not None else torch.empty(q.shape[:-1], dtype=torch.float32, device=q.device)
    need = lib.jfa_decode_workspace_size(ctypes.byref(p))
    ws = workspace if workspace is not None else torch.empty(max(need, 1), dtype=torch.uint8, device=q.device)
    st = lib.jfa_decode_paged(ctypes.byref(p), _ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(page_table),
                              _ptr(seqlens_k), _ptr(o), _ptr(l), ws.data_ptr(), ws.numel(), _stream())
    _lib.check(st, "jfa_decode_paged")
    return o, l


class timing:
    """Kernel timing through the library's own HIP events (see jfa_timing_enable)."""

    @staticmethod
    def enable(on: bool = True) -> None:
        _lib.check(load().jfa_timing_enable(int(on)), "jfa_timing_enable")

    SLOTS = ("fwd", "bwd_dq", "bwd_dkdv", "decode")

    @staticmethod
    def collect():
        """Returns {'fwd': (total_ms, launches), 'bwd_dq': ..., 'bwd_dkdv': ..., 'decode': ...}
        and clears the record."""
        n = len(timing.SLOTS)
        ms = (ctypes.c_double * n)()
        cnt = (ctypes.c_int64 * n)()
        _lib.check(load().jfa_timing_collect(ms, cnt), "jfa_timing_collect")
        return {name: (ms[i], cnt[i]) for i, name in enumerate(timing.SLOTS)}


def default_scale(head_dim: int, softmax_scale: Optional[float] = None) -> float:
    return softmax_scale if softmax_scale and softmax_scale > 0 else 1.0 / math.sqrt(head_dim)
