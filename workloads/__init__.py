"""Seeded synthetic inputs for jagged (packed variable-length) attention.

This module only draws random numbers and lays them out; it holds none of the
attention arithmetic.  Both the fp64 CPU checker under ``oracle/`` and the GPU
path are fed from here, so they see bit-identical bf16 values.

Recipe (one for every workload):
  1. ``rng = numpy.random.default_rng(seed)``
  2. draw the sequence lengths (jagged workloads) or KV lengths (decode)
  3. decode only: draw the physical page permutation
  4. draw Q, K, V, dO in that order: each tensor takes one 64-bit integer from
     ``rng`` to seed 16 PCG64 child streams that fill 16 equal contiguous
     chunks with ``standard_normal(float32)``; values are then rounded to bf16
     with round-to-nearest-even.

Workloads follow the pages' statement of the problem: packed ``[total_tokens,
heads, head_dim]`` tensors plus an int32 offsets array (Meta's Jagged Flash
Attention page, the paragraph on GEM's jagged user sequences and broadcast-Q),
and a paged KV cache with a page table of arbitrary page size (the Modal
FlashAttention-4 inference page, the PR 1999/2104 and PR 1940 sections).
The length recipe ``L = min(U{1 .. floor(max_len*(1-s)*2)}, max_len)`` is the
plain reading of "sparsity s" (the expected unclipped mean length is
``max_len*(1-s)``); the jagged page sweeps sparsity 0.1/0.5/0.9 without giving
its distribution.
"""
from __future__ import annotations

import math
import os
from dataclasses import dataclass, field
from typing import Optional

import numpy as np

__all__ = [
    "bf16_round", "bf16_bits", "bits_to_f32", "sparsity_lengths", "offsets",
    "JaggedInputs", "BroadcastInputs", "DecodeInputs",
    "jagged", "broadcast", "decode", "tiny", "gem", "broadcast_q", "dense_causal",
    "decode_paged", "repage", "TINY_LENGTHS",
]

TINY_LENGTHS = (37, 64, 1, 90)


# --------------------------------------------------------------------------- bf16
def bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 to bfloat16 (round to nearest, ties to even); return the uint16 bit patterns."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    lsb = (u >> np.uint32(16)) & np.uint32(1)
    r = (u + np.uint32(0x7FFF) + lsb) >> np.uint32(16)
    return r.astype(np.uint16)


def bits_to_f32(b: np.ndarray) -> np.ndarray:
    """Widen bf16 bit patterns (uint16) to float32 exactly."""
    return (np.ascontiguousarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def bf16_round(x: np.ndarray) -> np.ndarray:
    """float32 array holding the bf16-rounded values of ``x``."""
    return bits_to_f32(bf16_bits(x))


_CHUNKS = 16
_POOL = None


def _pool():
    global _POOL
    if _POOL is None:
        from concurrent.futures import ThreadPoolExecutor
        _POOL = ThreadPoolExecutor(max_workers=min(_CHUNKS, os.cpu_count() or 1))
    return _POOL


def _normal_bf16(rng: np.random.Generator, shape) -> np.ndarray:
    """N(0,1) float32 rounded to bf16.

    The tensor takes one 64-bit draw from ``rng`` as the entropy of its own
    SeedSequence, spawns 16 child PCG64 streams and fills 16 equal contiguous
    chunks from them (in parallel threads; the values do not depend on the
    thread count).
    """
    n = int(np.prod(shape))
    out = np.empty(n, dtype=np.float32)
    kids = np.random.SeedSequence(int(rng.integers(0, 2**63))).spawn(_CHUNKS)
    step = -(-n // _CHUNKS) if n else 0

    def fill(i):
        lo, hi = i * step, min(n, (i + 1) * step)
        if lo < hi:
            g = np.random.Generator(np.random.PCG64(kids[i]))
            seg = out[lo:hi]
            g.standard_normal(out=seg, dtype=np.float32)
            seg[:] = bf16_round(seg)

    list(_pool().map(fill, range(_CHUNKS)))
    return out.reshape(shape)


# ------------------------------------------------------------------------ lengths
def sparsity_lengths(rng: np.random.Generator, batch: int, max_len: int, sparsity: float) -> np.ndarray:
    """L_b = min(U{1..floor(max_len*(1-s)*2)}, max_len), inclusive bounds."""
    hi = max(1, int(math.floor(max_len * (1.0 - sparsity) * 2.0)))
    lengths = rng.integers(1, hi + 1, size=batch)
    return np.minimum(lengths, max_len).astype(np.int32)


def offsets(lengths) -> np.ndarray:
    """int32 offsets [B+1]: offsets[0] = 0, offsets[b+1] = offsets[b] + L_b."""
    lengths = np.asarray(lengths, dtype=np.int64)
    out = np.zeros(len(lengths) + 1, dtype=np.int64)
    np.cumsum(lengths, out=out[1:])
    assert out[-1] < 2**31, "offsets overflow int32"
    return out.astype(np.int32)


# ---------------------------------------------------------------------- containers
@dataclass
class JaggedInputs:
    """Packed self-attention inputs. Arrays are float32 holding exact bf16 values."""
    q: np.ndarray          # [Tq, Hq, d]
    k: np.ndarray          # [Tk, Hkv, d]
    v: np.ndarray          # [Tk, Hkv, d]
    do: np.ndarray         # [Tq, Hq, d]
    cu_q: np.ndarray       # int32 [B+1]
    cu_k: np.ndarray       # int32 [B+1]
    causal: bool = False
    name: str = ""
    meta: dict = field(default_factory=dict)

    @property
    def batch(self): return len(self.cu_q) - 1
    @property
    def heads_q(self): return self.q.shape[1]
    @property
    def heads_kv(self): return self.k.shape[1]
    @property
    def head_dim(self): return self.q.shape[2]
    @property
    def max_len_q(self): return int(np.diff(self.cu_q).max(initial=0))
    @property
    def max_len_k(self): return int(np.diff(self.cu_k).max(initial=0))


@dataclass
class BroadcastInputs:
    """One dense Q shared by all items; jagged K/V; per-item dO."""
    q: np.ndarray          # [Nq, Hq, d]
    k: np.ndarray          # [Tk, Hkv, d]
    v: np.ndarray          # [Tk, Hkv, d]
    do: np.ndarray         # [B, Nq, Hq, d]
    cu_k: np.ndarray       # int32 [B+1]
    name: str = ""
    meta: dict = field(default_factory=dict)

    @property
    def batch(self): return len(self.cu_k) - 1
    @property
    def heads_q(self): return self.q.shape[1]
    @property
    def heads_kv(self): return self.k.shape[1]
    @property
    def head_dim(self): return self.q.shape[2]
    @property
    def max_len_k(self): return int(np.diff(self.cu_k).max(initial=0))


@dataclass
class DecodeInputs:
    """Decode of one (q [B, Hq, d]) or a few (q [B, q_len, Hq, d]) new tokens per
    sequence against a paged KV cache.

    ``k``/``v`` are the contiguous (pre-paging) packed caches; ``k_cache``/``v_cache``
    hold the very same rows scattered into pages through ``page_table``.
    """
    q: np.ndarray            # [B, Hq, d] or [B, q_len, Hq, d]
    k: np.ndarray            # [Tk, Hkv, d] contiguous
    v: np.ndarray            # [Tk, Hkv, d]
    cu_k: np.ndarray         # int32 [B+1]
    seqlens_k: np.ndarray    # int32 [B]
    page_size: int
    page_table: np.ndarray   # int32 [B, max_pages_per_seq]
    k_cache: np.ndarray      # [num_pages, page_size, Hkv, d]
    v_cache: np.ndarray
    name: str = ""
    meta: dict = field(default_factory=dict)

    @property
    def batch(self): return self.q.shape[0]
    @property
    def num_pages(self): return self.k_cache.shape[0]


# ----------------------------------------------------------------------- builders
def jagged(seed: int, lengths_q, lengths_k=None, heads_q: int = 2, heads_kv: Optional[int] = None,
           head_dim: int = 64, causal: bool = False, name: str = "") -> JaggedInputs:
    """Packed self/cross attention over explicit lengths (drawn by the caller or fixed)."""
    rng = np.random.default_rng(seed)
    return _jagged_from_rng(rng, lengths_q, lengths_k, heads_q, heads_kv, head_dim, causal, name)


def _jagged_from_rng(rng, lengths_q, lengths_k, heads_q, heads_kv, head_dim, causal, name, meta=None):
    heads_kv = heads_q if heads_kv is None else heads_kv
    lengths_k = lengths_q if lengths_k is None else lengths_k
    cu_q, cu_k = offsets(lengths_q), offsets(lengths_k)
    tq, tk = int(cu_q[-1]), int(cu_k[-1])
    q = _normal_bf16(rng, (tq, heads_q, head_dim))
    k = _normal_bf16(rng, (tk, heads_kv, head_dim))
    v = _normal_bf16(rng, (tk, heads_kv, head_dim))
    do = _normal_bf16(rng, (tq, heads_q, head_dim))
    return JaggedInputs(q, k, v, do, cu_q, cu_k, causal, name, dict(meta or {}))


def tiny(seed: int = 0) -> JaggedInputs:
    """4 sequences [37, 64, 1, 90] packed as [192, 2, 64]; non-causal."""
    rng = np.random.default_rng(seed)
    return _jagged_from_rng(rng, TINY_LENGTHS, None, 2, 2, 64, False, "tiny")


def gem(seed: int = 0, sparsity: float = 0.5, batch: int = 256, max_len: int = 1024,
        heads: int = 8, head_dim: int = 128) -> JaggedInputs:
    """GEM-style jagged self-attention: lengths from the sparsity recipe; non-causal."""
    rng = np.random.default_rng(seed)
    lengths = sparsity_lengths(rng, batch, max_len, sparsity)
    meta = {"sparsity": sparsity, "realised_sparsity": 1.0 - float(lengths.mean()) / max_len,
            "max_len": max_len}
    return _jagged_from_rng(rng, lengths, None, heads, heads, head_dim, False, f"gem_s{sparsity}", meta)


def dense_causal(seed: int = 0, batch: int = 4, seqlen: int = 8192, heads: int = 32,
                 head_dim: int = 128) -> JaggedInputs:
    """Dense LLM-style causal self-attention: every sequence full length."""
    rng = np.random.default_rng(seed)
    lengths = np.full(batch, seqlen, dtype=np.int32)
    return _jagged_from_rng(rng, lengths, None, heads, heads, head_dim, True, f"dense_causal_d{head_dim}")


def broadcast(seed: int, nq: int, lengths_k, heads_q: int = 4, heads_kv: Optional[int] = None,
              head_dim: int = 128, name: str = "") -> BroadcastInputs:
    rng = np.random.default_rng(seed)
    return _broadcast_from_rng(rng, nq, lengths_k, heads_q, heads_kv, head_dim, name)


def _broadcast_from_rng(rng, nq, lengths_k, heads_q, heads_kv, head_dim, name, meta=None):
    heads_kv = heads_q if heads_kv is None else heads_kv
    cu_k = offsets(lengths_k)
    tk = int(cu_k[-1])
    b = len(lengths_k)
    q = _normal_bf16(rng, (nq, heads_q, head_dim))
    k = _normal_bf16(rng, (tk, heads_kv, head_dim))
    v = _normal_bf16(rng, (tk, heads_kv, head_dim))
    do = _normal_bf16(rng, (b, nq, heads_q, head_dim))
    return BroadcastInputs(q, k, v, do, cu_k, name, dict(meta or {}))


def broadcast_q(seed: int = 0, sparsity: float = 0.5, batch: int = 512, max_len: int = 2048,
                nq: int = 256, heads: int = 4, head_dim: int = 128) -> BroadcastInputs:
    """Broadcast-Q cross-attention: Q [256, 4, 128] shared by 512 jagged items."""
    rng = np.random.default_rng(seed)
    lengths = sparsity_lengths(rng, batch, max_len, sparsity)
    meta = {"sparsity": sparsity, "realised_sparsity": 1.0 - float(lengths.mean()) / max_len,
            "max_len": max_len}
    return _broadcast_from_rng(rng, nq, lengths, heads, heads, head_dim, f"bcast_s{sparsity}", meta)


def decode(seed: int, seqlens, heads_q: int = 32, heads_kv: int = 8, head_dim: int = 128,
           page_size: int = 16, max_pages_per_seq: Optional[int] = None, tail_fill: float = float("nan"),
           name: str = "", _rng=None, q_len: int = 1, kv_fp8: bool = False, k_scale: float = 1.0,
           v_scale: float = 1.0) -> DecodeInputs:
    """Paged decode inputs over explicit KV lengths.

    kv_fp8: the caches hold OCP e4m3 bytes (uint8) of K / k_scale and V / v_scale,
    rounded to nearest by torch's float8_e4m3fn; ``k``/``v`` then hold the exact
    dequantised values (byte value times scale) and unused slots the NaN byte 0x7F.

    q is [B, Hq, d] for q_len = 1, else [B, q_len, Hq, d] (the new tokens are the
    last q_len of each sequence's KV length).

    num_pages = sum_b ceil(L_b / page_size).  Physical page ids are a seeded
    permutation of [0, num_pages) handed out in (sequence, logical page) order.
    Unused cache slots past L_b hold ``tail_fill`` (NaN by default, so that any
    read past the end of a sequence poisons the result).  Unused page-table
    entries hold 0 (a valid page id).
    """
    rng = np.random.default_rng(seed) if _rng is None else _rng
    seqlens = np.asarray(seqlens, dtype=np.int32)
    b = len(seqlens)
    pages_per = -(-seqlens.astype(np.int64) // page_size)
    num_pages = int(pages_per.sum())
    if max_pages_per_seq is None:
        max_pages_per_seq = int(pages_per.max(initial=1))
    assert pages_per.max(initial=0) <= max_pages_per_seq
    perm = rng.permutation(num_pages).astype(np.int32)
    cu_k = offsets(seqlens)
    tk = int(cu_k[-1])
    q = _normal_bf16(rng, (b, heads_q, head_dim) if q_len == 1 else (b, q_len, heads_q, head_dim))
    k = _normal_bf16(rng, (tk, heads_kv, head_dim))
    v = _normal_bf16(rng, (tk, heads_kv, head_dim))

    meta = {"num_pages": num_pages}
    if kv_fp8:
        kb, k = _e4m3(k, k_scale)
        vb, v = _e4m3(v, v_scale)
        page_table, k_cache, v_cache = _page(kb, vb, seqlens, cu_k, page_size, max_pages_per_seq, perm,
                                             0x7F, np.uint8)
        meta.update(k_scale=float(k_scale), v_scale=float(v_scale))
    else:
        page_table, k_cache, v_cache = _page(k, v, seqlens, cu_k, page_size, max_pages_per_seq, perm, tail_fill)
    return DecodeInputs(q, k, v, cu_k, seqlens, page_size, page_table, k_cache, v_cache, name, meta)


def _e4m3(x, scale: float):
    """Round x / scale to OCP e4m3 (torch float8_e4m3fn, nearest even); returns the
    bytes and the exact dequantised values byte_value * scale (float32)."""
    import torch
    t = torch.from_numpy(np.ascontiguousarray(x / scale, dtype=np.float32)).to(torch.float8_e4m3fn)
    return t.view(torch.uint8).numpy().copy(), (t.float() * scale).numpy()


def e4m3(x, scale: float):
    """OCP e4m3 bytes of x / scale (nearest even) and their exact dequantised values."""
    return _e4m3(x, scale)


def fp8_qkv(inp, q_scale=None, k_scale=None, v_scale=None):
    """e4m3 copies of q, k, v with per-tensor scales (default: amax / 448, the
    largest finite e4m3 value).  Returns (same inputs with q, k, v replaced by the
    exact dequantised values, {"q": bytes, "k": bytes, "v": bytes, "q_scale": ...})."""
    from dataclasses import replace
    out, enc = {}, {}
    for name, x, sc in (("q", inp.q, q_scale), ("k", inp.k, k_scale), ("v", inp.v, v_scale)):
        amax = float(np.abs(x).max(initial=0.0))
        if sc is None:
            sc = amax / 448.0 if amax > 0 else 1.0
        if amax / sc > 448.0 * (1 + 1e-6):   # the default scale lands on 448 up to rounding
            raise ValueError(f"{name}: |x| / scale reaches {amax / sc:.1f}, beyond e4m3's largest finite 448")
        enc[name], out[name] = _e4m3(x, float(sc))
        enc[name + "_scale"] = float(sc)
    return replace(inp, q=out["q"], k=out["k"], v=out["v"]), enc


def _page(k, v, seqlens, cu_k, page_size, max_pages_per_seq, perm, tail_fill, dtype=np.float32):
    """Scatter contiguous K/V rows into pages; physical ids come from `perm` in (sequence, page) order."""
    b = len(seqlens)
    tk, heads_kv, head_dim = k.shape
    pages_per = -(-seqlens.astype(np.int64) // page_size)
    num_pages = int(pages_per.sum())
    page_table = np.zeros((b, max_pages_per_seq), dtype=np.int32)
    first_page = np.zeros(b + 1, dtype=np.int64)
    np.cumsum(pages_per, out=first_page[1:])
    for i in range(b):
        page_table[i, :pages_per[i]] = perm[first_page[i]:first_page[i + 1]]
    # every token goes to (physical page, slot)
    seq_of_token = np.repeat(np.arange(b), seqlens)
    pos = np.arange(tk, dtype=np.int64) - cu_k[seq_of_token].astype(np.int64)
    phys = page_table[seq_of_token, pos // page_size].astype(np.int64)
    slot = phys * page_size + pos % page_size
    k_cache = np.full((num_pages * page_size, heads_kv, head_dim), tail_fill, dtype=dtype)
    v_cache = np.full((num_pages * page_size, heads_kv, head_dim), tail_fill, dtype=dtype)
    k_cache[slot] = k
    v_cache[slot] = v
    return (page_table, k_cache.reshape(num_pages, page_size, heads_kv, head_dim),
            v_cache.reshape(num_pages, page_size, heads_kv, head_dim))


def repage(inp: DecodeInputs, page_size: int, seed: int, tail_fill: float = float("nan")) -> DecodeInputs:
    """The same q and contiguous K/V laid out in pages of another size under a fresh permutation."""
    rng = np.random.default_rng(seed)
    pages_per = -(-inp.seqlens_k.astype(np.int64) // page_size)
    perm = rng.permutation(int(pages_per.sum())).astype(np.int32)
    max_pages = int(pages_per.max(initial=1))
    pt, kc, vc = _page(inp.k, inp.v, inp.seqlens_k, inp.cu_k, page_size, max_pages, perm, tail_fill)
    return DecodeInputs(inp.q, inp.k, inp.v, inp.cu_k, inp.seqlens_k, page_size, pt, kc, vc,
                        inp.name + f"_repaged{page_size}", {"num_pages": kc.shape[0]})


def decode_paged(seed: int = 0, page_size: int = 16, batch: int = 32, heads_q: int = 32, heads_kv: int = 8,
                 head_dim: int = 128, min_len: int = 4096, max_len: int = 16384,
                 tail_fill: float = float("nan")) -> DecodeInputs:
    """Split-KV paged decode workload: KV lengths U{4096..16384}, GQA 4:1, d=128."""
    rng = np.random.default_rng(seed)
    seqlens = rng.integers(min_len, max_len + 1, size=batch).astype(np.int32)
    max_pages = -(-max_len // page_size)
    return decode(seed, seqlens, heads_q, heads_kv, head_dim, page_size, max_pages, tail_fill,
                  f"decode_ps{page_size}", _rng=rng)
