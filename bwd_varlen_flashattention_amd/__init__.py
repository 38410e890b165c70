"""Python binding of libjfa.so: exact jagged FlashAttention fwd/bwd and split-KV
paged decode on MI355X (gfx950).

The functions keep the C ABI's names and only marshal arguments: they check
every tensor's dtype, shape, layout and device, allocate missing outputs and
the workspace with torch on the inputs' device, and call the library on
torch's current stream.  Every step of the computation runs in the library's
HIP kernels; there is no CPU or PyTorch fallback.
"""
from __future__ import annotations

import ctypes
from typing import Optional

from . import _lib
from ._lib import AttnParams, DecodeParams, JfaError, KernelEventsStruct, load  # noqa: F401

__all__ = ["jfa_fwd", "jfa_bwd", "jfa_decode_paged", "jfa_decode_num_splits", "jfa_fwd_workspace_size",
           "jfa_bwd_workspace_size", "jfa_decode_workspace_size", "jfa_decode_paged_noalloc", "KernelEvents",
           "JfaError", "load", "jfa_check_offsets", "jfa_check_paged_cache"]


def _torch():
    import torch
    return torch


def _ptr(t) -> Optional[int]:
    return None if t is None or t.numel() == 0 else t.data_ptr()


def _stream():
    torch = _torch()
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


class KernelEvents:
    """Caller-owned timing events of one call (the C ABI's jfa_kernel_events_t).

    Pass as ``events=`` to jfa_fwd / jfa_bwd / jfa_decode_paged; after the
    stream has reached the call, ``elapsed_ms(slot)`` is the time of that
    kernel: "fwd", "bwd_dq", "bwd_dkdv" or "decode"."""

    SLOTS = ("fwd", "bwd_dq", "bwd_dkdv", "decode")

    def __init__(self):
        torch = _torch()
        self._ev = {}
        fields = {}
        for s in self.SLOTS:
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record()   # torch creates the underlying hipEvent_t on its first record
            b.record()
            self._ev[s] = (a, b)
            fields[f"{s}_start"], fields[f"{s}_stop"] = a.cuda_event, b.cuda_event
        self.struct = KernelEventsStruct(**fields)

    def pointer(self):
        return ctypes.pointer(self.struct)

    def elapsed_ms(self, slot: str) -> float:
        a, b = self._ev[slot]
        return a.elapsed_time(b)


# ----------------------------------------------------------------------------- validation
# Dtype, shape and layout of every tensor are checked before any device, so that
# the checks are testable without a GPU; every failure raises ValueError before
# the library is called.

def _is_fp8(t) -> bool:
    torch = _torch()
    return t.dtype in (getattr(torch, "float8_e4m3fn", None), torch.uint8)


def _check(name, t, dtypes, shape):
    """t must be a contiguous tensor of one of `dtypes` with exactly `shape`
    (None entries match any size)."""
    if t is None:
        raise ValueError(f"{name}: missing tensor")
    if t.dtype not in dtypes:
        raise ValueError(f"{name}: dtype {t.dtype}, expected one of {tuple(str(d) for d in dtypes)}")
    if t.dim() != len(shape) or any(s is not None and int(a) != int(s) for a, s in zip(t.shape, shape)):
        want = tuple("*" if s is None else int(s) for s in shape)
        raise ValueError(f"{name}: shape {tuple(t.shape)}, expected {want}")
    if not t.is_contiguous():
        raise ValueError(f"{name}: must be contiguous")


def _check_devices(**tensors):
    """Every tensor given (None skipped) lives on one CUDA device."""
    dev = None
    for name, t in tensors.items():
        if t is None:
            continue
        if not t.is_cuda:
            raise ValueError(f"{name}: must be a CUDA tensor")
        if dev is None:
            dev = t.device
        elif t.device != dev:
            raise ValueError(f"{name}: on {t.device}, the other tensors are on {dev}")


def _check_workspace(ws, need):
    torch = _torch()
    _check("workspace", ws, (torch.uint8,), (None,))
    if ws.numel() < need:
        raise ValueError(f"workspace: {ws.numel()} bytes, the call needs {need}")


def _bf16(torch):
    return (torch.bfloat16,)


def _e4m3_types(torch):
    return tuple(t for t in (getattr(torch, "float8_e4m3fn", None), torch.uint8) if t is not None)


def _qkv_shapes(q, k, v, broadcast_q, fp8):
    """Checks q/k/v shapes against each other; returns (Hq, Hkv, d)."""
    torch = _torch()
    dts = _e4m3_types(torch) if fp8 else _bf16(torch)
    if q.dim() != 3:
        raise ValueError(f"q: shape {tuple(q.shape)}, expected [{'Nq' if broadcast_q else 'total_q'}, Hq, d]")
    hq, d = q.shape[1], q.shape[2]
    if k.dim() != 3:
        raise ValueError(f"k: shape {tuple(k.shape)}, expected [total_k, Hkv, {d}]")
    hkv = k.shape[1]
    _check("q", q, dts, (None, hq, d))
    _check("k", k, dts, (None, hkv, d))
    _check("v", v, dts, tuple(k.shape))
    if hkv < 1 or hq % hkv != 0:
        raise ValueError(f"q heads {hq} must be a multiple of k/v heads {hkv}")
    return hq, hkv, d


def _offsets(cu_seqlens_q, cu_seqlens_k, broadcast_q):
    """Checks the offsets tensors; returns the batch B."""
    torch = _torch()
    if cu_seqlens_k is None or cu_seqlens_k.dim() != 1 or cu_seqlens_k.numel() < 2:
        raise ValueError("cu_seqlens_k: expected an int32 tensor of B + 1 >= 2 offsets")
    nb = cu_seqlens_k.numel() - 1
    _check("cu_seqlens_k", cu_seqlens_k, (torch.int32,), (nb + 1,))
    if not broadcast_q:
        _check("cu_seqlens_q", cu_seqlens_q, (torch.int32,), (nb + 1,))
    return nb


def _attn_params(q, k, nb, max_q, max_k, causal, scale, broadcast_q, fp8=False,
                 q_scale=None, k_scale=None, v_scale=None, events=None, query_tile=0):
    sc = lambda x: float(x) if x is not None else 1.0
    if query_tile not in (0, 128, 256):
        raise ValueError(f"query_tile: {query_tile!r}, expected 0 (chosen from the lengths), 128 or 256")
    return AttnParams(
        batch=nb, num_heads_q=q.shape[1], num_heads_kv=k.shape[1], head_dim=q.shape[2],
        total_q=q.shape[0], total_k=k.shape[0], max_seqlen_q=int(max_q), max_seqlen_k=int(max_k),
        causal=int(bool(causal)), broadcast_q=int(bool(broadcast_q)),
        softmax_scale=float(scale) if scale is not None else 0.0,
        qkv_dtype=1 if fp8 else 0, q_scale=sc(q_scale), k_scale=sc(k_scale), v_scale=sc(v_scale),
        query_tile=int(query_tile), events=events.pointer() if events is not None else None)


def _out_shapes(q, nb, broadcast_q):
    """(o shape, lse shape) of the forward for this q."""
    nq, hq, d = q.shape
    if broadcast_q:
        return (nb, nq, hq, d), (nb, hq, nq)
    return (nq, hq, d), (hq, nq)


# ----------------------------------------------------------------------------- entry points

def jfa_fwd_workspace_size(q, k, cu_seqlens_k, max_seqlen_q: int, max_seqlen_k: int, causal: bool = False,
                           broadcast_q: bool = False, query_tile: int = 0) -> int:
    """Workspace bytes jfa_fwd needs for these shapes (q may be bf16 or e4m3)."""
    p = _attn_params(q, k, cu_seqlens_k.numel() - 1, max_seqlen_q, max_seqlen_k, causal, None, broadcast_q,
                     _is_fp8(q), query_tile=query_tile)
    return int(load().jfa_fwd_workspace_size(ctypes.byref(p)))


def jfa_bwd_workspace_size(q, k, cu_seqlens_k, max_seqlen_q: int, max_seqlen_k: int, causal: bool = False,
                           broadcast_q: bool = False, query_tile: int = 0) -> int:
    """Workspace bytes jfa_bwd needs for these shapes."""
    p = _attn_params(q, k, cu_seqlens_k.numel() - 1, max_seqlen_q, max_seqlen_k, causal, None, broadcast_q,
                     query_tile=query_tile)
    return int(load().jfa_bwd_workspace_size(ctypes.byref(p)))


def jfa_fwd(q, k, v, cu_seqlens_q, cu_seqlens_k, max_seqlen_q: int, max_seqlen_k: int,
            causal: bool = False, softmax_scale: Optional[float] = None, broadcast_q: bool = False,
            out=None, lse=None, workspace=None, q_scale: Optional[float] = None,
            k_scale: Optional[float] = None, v_scale: Optional[float] = None,
            events: Optional[KernelEvents] = None, query_tile: int = 0):
    """Jagged forward.  Self-attention: q [Tq,Hq,d], k/v [Tk,Hkv,d] -> o [Tq,Hq,d], lse [Hq,Tq].
    Broadcast-Q: q [Nq,Hq,d] shared by B items -> o [B,Nq,Hq,d], lse [B,Hq,Nq].
    q, k, v are all bfloat16, or all e4m3 (float8_e4m3fn or raw uint8 bytes) with
    per-tensor scales q_scale, k_scale, v_scale (default 1); o is bfloat16 either way.
    query_tile: rows per work item (0: chosen from the lengths; 128 / 256 where the
    kernel has both) -- a speed choice with the same result."""
    torch = _torch()
    fp8 = _is_fp8(q)
    _qkv_shapes(q, k, v, broadcast_q, fp8)
    nb = _offsets(cu_seqlens_q, cu_seqlens_k, broadcast_q)
    o_shape, lse_shape = _out_shapes(q, nb, broadcast_q)
    if out is not None:
        _check("out", out, _bf16(torch), o_shape)
    if lse is not None:
        _check("lse", lse, (torch.float32,), lse_shape)
    if workspace is not None:
        _check_workspace(workspace, 0)
    _check_devices(q=q, k=k, v=v, cu_seqlens_q=None if broadcast_q else cu_seqlens_q, cu_seqlens_k=cu_seqlens_k,
                   out=out, lse=lse, workspace=workspace)
    lib = load()
    p = _attn_params(q, k, nb, max_seqlen_q, max_seqlen_k, causal, softmax_scale, broadcast_q, fp8,
                     q_scale, k_scale, v_scale, events, query_tile)
    need = lib.jfa_fwd_workspace_size(ctypes.byref(p))
    if workspace is not None:
        _check_workspace(workspace, need)
    o = out if out is not None else torch.empty(o_shape, dtype=torch.bfloat16, device=q.device)
    l = lse if lse is not None else torch.empty(lse_shape, dtype=torch.float32, device=q.device)
    ws = workspace if workspace is not None else torch.empty(max(need, 1), dtype=torch.uint8, device=q.device)
    st = lib.jfa_fwd(ctypes.byref(p), _ptr(q), _ptr(k), _ptr(v),
                     None if broadcast_q else _ptr(cu_seqlens_q), _ptr(cu_seqlens_k),
                     _ptr(o), _ptr(l), ws.data_ptr(), ws.numel(), _stream())
    _lib.check(st, "jfa_fwd")
    return o, l


def jfa_bwd(q, k, v, o, lse, dout, cu_seqlens_q, cu_seqlens_k, max_seqlen_q: int, max_seqlen_k: int,
            causal: bool = False, softmax_scale: Optional[float] = None, broadcast_q: bool = False,
            dq=None, dk=None, dv=None, workspace=None, events: Optional[KernelEvents] = None,
            query_tile: int = 0):
    """Jagged backward: returns (dq, dk, dv) in the layouts of q, k, v (query_tile as in jfa_fwd)."""
    torch = _torch()
    _qkv_shapes(q, k, v, broadcast_q, False)
    dev = q.device
    nb = _offsets(cu_seqlens_q, cu_seqlens_k, broadcast_q)
    o_shape, lse_shape = _out_shapes(q, nb, broadcast_q)
    _check("o", o, _bf16(torch), o_shape)
    _check("dout", dout, _bf16(torch), o_shape)
    _check("lse", lse, (torch.float32,), lse_shape)
    for name, t, like in (("dq", dq, q), ("dk", dk, k), ("dv", dv, v)):
        if t is not None:
            _check(name, t, _bf16(torch), tuple(like.shape))
    if workspace is not None:
        _check_workspace(workspace, 0)
    _check_devices(q=q, k=k, v=v, o=o, lse=lse, dout=dout, cu_seqlens_q=None if broadcast_q else cu_seqlens_q,
                   cu_seqlens_k=cu_seqlens_k, dq=dq, dk=dk, dv=dv, workspace=workspace)
    lib = load()
    p = _attn_params(q, k, nb, max_seqlen_q, max_seqlen_k, causal, softmax_scale, broadcast_q, events=events,
                     query_tile=query_tile)
    need = lib.jfa_bwd_workspace_size(ctypes.byref(p))
    if workspace is not None:
        _check_workspace(workspace, need)
    dq = dq if dq is not None else torch.empty_like(q)
    dk = dk if dk is not None else torch.empty_like(k)
    dv = dv if dv is not None else torch.empty_like(v)
    ws = workspace if workspace is not None else torch.empty(max(need, 1), dtype=torch.uint8, device=dev)
    st = lib.jfa_bwd(ctypes.byref(p), _ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), _ptr(dout),
                     None if broadcast_q else _ptr(cu_seqlens_q), _ptr(cu_seqlens_k),
                     _ptr(dq), _ptr(dk), _ptr(dv), ws.data_ptr(), ws.numel(), _stream())
    _lib.check(st, "jfa_bwd")
    return dq, dk, dv


def _decode_shapes(q, k_cache, v_cache, page_table, seqlens_k):
    """Checks the decode tensors against each other; returns q_len."""
    torch = _torch()
    if q.dim() not in (3, 4):
        raise ValueError(f"q: shape {tuple(q.shape)}, expected [B, Hq, d] or [B, q_len, Hq, d]")
    b, hq, d = q.shape[0], q.shape[-2], q.shape[-1]
    q_len = 1 if q.dim() == 3 else q.shape[1]
    _check("q", q, _e4m3_types(torch) if _is_fp8(q) else _bf16(torch), tuple(q.shape))
    if k_cache.dim() != 4:
        raise ValueError(f"k_cache: shape {tuple(k_cache.shape)}, expected [num_pages, page_size, Hkv, {d}]")
    fp8 = _is_fp8(k_cache)
    kdt = _e4m3_types(torch) if fp8 else _bf16(torch)
    _check("k_cache", k_cache, kdt, (None, None, None, d))
    _check("v_cache", v_cache, kdt, tuple(k_cache.shape))
    if _is_fp8(v_cache) != fp8:
        raise ValueError("k_cache and v_cache must have the same element type")
    if page_table is None or page_table.dim() != 2:
        raise ValueError("page_table: expected an int32 tensor [B, max_pages_per_seq]")
    _check("page_table", page_table, (torch.int32,), (b, None))
    _check("seqlens_k", seqlens_k, (torch.int32,), (b,))
    hkv = k_cache.shape[2]
    if hkv < 1 or hq % hkv != 0:
        raise ValueError(f"q heads {hq} must be a multiple of the cache's KV heads {hkv}")
    return q_len


def _decode_params(q, k_cache, page_table, num_splits, scale, causal=False, k_scale=None, v_scale=None,
                   q_scale=None, events=None, single_launch=False):
    """q is [B, Hq, d] (one token per sequence) or [B, q_len, Hq, d]; an fp8 cache
    or query (float8_e4m3fn, or its raw bytes as uint8) selects the e4m3 path."""
    q_len = 1 if q.dim() == 3 else q.shape[1]
    fp8 = _is_fp8(k_cache)
    q8 = _is_fp8(q)
    return DecodeParams(
        batch=q.shape[0], num_heads_q=q.shape[-2], num_heads_kv=k_cache.shape[2], head_dim=q.shape[-1],
        page_size=k_cache.shape[1], num_pages=k_cache.shape[0], max_pages_per_seq=page_table.shape[1],
        num_splits=int(num_splits), softmax_scale=float(scale) if scale is not None else 0.0,
        q_len=int(q_len), causal=int(bool(causal)), kv_dtype=1 if fp8 else 0,
        k_scale=float(k_scale) if k_scale is not None else 0.0, v_scale=float(v_scale) if v_scale is not None else 0.0,
        q_dtype=1 if q8 else 0, q_scale=float(q_scale) if q_scale is not None else 0.0,
        single_launch=int(bool(single_launch)), events=events.pointer() if events is not None else None)


def jfa_decode_workspace_size(q, k_cache, page_table, num_splits: int = 0) -> int:
    """Workspace bytes jfa_decode_paged needs for these shapes and split count."""
    p = _decode_params(q, k_cache, page_table, num_splits, None)
    return int(load().jfa_decode_workspace_size(ctypes.byref(p)))


def jfa_check_offsets(offsets, total: int) -> int:
    """Device-side check of packed offsets [B + 1] (int32, on the GPU): the OR of the
    violated JFA_CHECK_* bits (start at 0, non-decreasing, end at `total`), 0 if valid.
    Waits for the check kernel."""
    torch = _torch()
    _check("offsets", offsets, (torch.int32,), (None,))
    _check_devices(offsets=offsets)
    if offsets.numel() < 1:
        raise ValueError("offsets: needs at least one entry")
    res = torch.empty(1, dtype=torch.int32, device=offsets.device)
    st = load().jfa_check_offsets(_ptr(offsets), offsets.numel() - 1, int(total), res.data_ptr(), _stream())
    _lib.check(st, "jfa_check_offsets")
    return int(res.item())


def jfa_check_paged_cache(q, k_cache, page_table, seqlens_k) -> int:
    """Device-side check of a paged cache's lengths and page table against the cache
    shape (as jfa_decode_paged would see them): the OR of the violated JFA_CHECK_* bits,
    0 if valid.  Waits for the check kernel."""
    torch = _torch()
    _decode_shapes(q, k_cache, k_cache, page_table, seqlens_k)
    _check_devices(q=q, k_cache=k_cache, page_table=page_table, seqlens_k=seqlens_k)
    p = _decode_params(q, k_cache, page_table, 0, None)
    res = torch.empty(1, dtype=torch.int32, device=q.device)
    st = load().jfa_check_paged_cache(ctypes.byref(p), _ptr(page_table), _ptr(seqlens_k), res.data_ptr(), _stream())
    _lib.check(st, "jfa_check_paged_cache")
    return int(res.item())


def jfa_decode_num_splits(q, k_cache, page_table, num_splits: int = 0) -> int:
    p = _decode_params(q, k_cache, page_table, num_splits, None)
    return int(load().jfa_decode_num_splits(ctypes.byref(p)))


def jfa_decode_paged(q, k_cache, v_cache, page_table, seqlens_k, num_splits: int = 0,
                     softmax_scale: Optional[float] = None, out=None, lse=None, workspace=None,
                     causal: bool = False, k_scale: Optional[float] = None, v_scale: Optional[float] = None,
                     q_scale: Optional[float] = None, events: Optional[KernelEvents] = None,
                     single_launch: bool = False):
    """Paged decode of q_len new tokens per sequence against a paged KV cache.

    q [B, Hq, d] (one token) or [B, q_len, Hq, d] (q_len <= 16); caches
    [num_pages, page_size, Hkv, d] -> o (bfloat16, shaped like q), lse [B, Hq] or [B, q_len, Hq].
    causal: the q_len tokens are the last ones of each sequence (bottom-right mask).
    FP8 caches (torch.float8_e4m3fn or raw uint8 bytes): K = k_scale * cache value,
    V = v_scale * cache value.  An FP8 q: Q = q_scale * q value.
    single_launch: the split partials are merged by the last split of each unit inside
    the decode launch instead of a second launch; a caller's workspace must then have
    been zero-filled once when it was allocated (its arrival counters, see jfa.h).
    """
    torch = _torch()
    _decode_shapes(q, k_cache, v_cache, page_table, seqlens_k)
    if out is not None:
        _check("out", out, _bf16(torch), tuple(q.shape))
    if lse is not None:
        _check("lse", lse, (torch.float32,), tuple(q.shape[:-1]))
    if workspace is not None:
        _check_workspace(workspace, 0)
    _check_devices(q=q, k_cache=k_cache, v_cache=v_cache, page_table=page_table, seqlens_k=seqlens_k, out=out,
                   lse=lse, workspace=workspace)
    lib = load()
    p = _decode_params(q, k_cache, page_table, num_splits, softmax_scale, causal, k_scale, v_scale, q_scale,
                       events, single_launch)
    need = lib.jfa_decode_workspace_size(ctypes.byref(p))
    if workspace is not None:
        _check_workspace(workspace, need)
    o = out if out is not None else torch.empty(q.shape, dtype=torch.bfloat16, device=q.device)
    l = lse if lse is not None else torch.empty(q.shape[:-1], dtype=torch.float32, device=q.device)
    # a fresh workspace starts with its arrival counters zero (see jfa.h); a
    # caller's workspace must have been zero-filled once when it was allocated
    ws = workspace if workspace is not None else torch.zeros(max(need, 1), dtype=torch.uint8, device=q.device)
    st = lib.jfa_decode_paged(ctypes.byref(p), _ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(page_table),
                              _ptr(seqlens_k), _ptr(o), _ptr(l), ws.data_ptr(), ws.numel(), _stream())
    _lib.check(st, "jfa_decode_paged")
    return o, l


def jfa_decode_paged_noalloc(q, k_cache, v_cache, page_table, seqlens_k, num_splits: int = 0,
                             softmax_scale: Optional[float] = None, out=None, lse=None, causal: bool = False,
                             k_scale: Optional[float] = None, v_scale: Optional[float] = None,
                             q_scale: Optional[float] = None, events: Optional[KernelEvents] = None,
                             single_launch: bool = False):
    """jfa_decode_paged with its split partials in the library's static device array
    instead of a workspace (the library allocates nothing; pass out and lse to
    allocate nothing here either).  Calls overlapping on one GPU race."""
    torch = _torch()
    _decode_shapes(q, k_cache, v_cache, page_table, seqlens_k)
    if out is not None:
        _check("out", out, _bf16(torch), tuple(q.shape))
    if lse is not None:
        _check("lse", lse, (torch.float32,), tuple(q.shape[:-1]))
    _check_devices(q=q, k_cache=k_cache, v_cache=v_cache, page_table=page_table, seqlens_k=seqlens_k, out=out,
                   lse=lse)
    lib = load()
    p = _decode_params(q, k_cache, page_table, num_splits, softmax_scale, causal, k_scale, v_scale, q_scale,
                       events, single_launch)
    o = out if out is not None else torch.empty(q.shape, dtype=torch.bfloat16, device=q.device)
    l = lse if lse is not None else torch.empty(q.shape[:-1], dtype=torch.float32, device=q.device)
    st = lib.jfa_decode_paged_noalloc(ctypes.byref(p), _ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(page_table),
                                      _ptr(seqlens_k), _ptr(o), _ptr(l), _stream())
    _lib.check(st, "jfa_decode_paged_noalloc")
    return o, l
