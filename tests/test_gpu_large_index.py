"""Tensors past 2^31 elements: the kernels' element offsets must not wrap in 32 bits.

Each case puts a sequence, an item or a set of KV pages on both sides of the
element offset 2^31 of its largest tensors.  The outputs start as NaN and must all
come back finite, and the oracle checks the sequences, items and pages before, across
and after that offset.  The inputs are too large to generate on the host in a test's
time, so they come from torch's seeded CUDA generator (standard normal, rounded to
bf16); the oracle reads host copies of the same slices.  About 40 GB of device memory
per case.
"""
import numpy as np
import pytest

import oracle
import workloads
from parity import check_grad, check_lse, check_o, dev, host

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

INT32_ELEMS = 1 << 31


def _say(*a):
    print(*a, flush=True)


@pytest.fixture(scope="module")
def jfa():
    import bwd_varlen_flashattention_amd as m
    m.load()
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    return m


def _normal(shape, gen):
    return torch.randn(shape, generator=gen, device="cuda", dtype=torch.bfloat16)


def _all_finite(**tensors):
    for name, t in tensors.items():
        assert bool(torch.isfinite(t).all()), f"{name}: some element is not finite (unwritten or wrong)"


@pytest.fixture(autouse=True)
def _free_memory():
    yield
    torch.cuda.empty_cache()


def test_self_attention_beyond_int32_offsets(jfa):
    """1051 causal sequences of 1000 tokens, 16 heads, d = 128: Q, K, V, O, dO, dQ, dK, dV
    hold 2.15e9 elements each; sequence 1048 straddles element 2^31."""
    L, n, H, D = 1000, 1051, 16, 128
    T = L * n
    assert T * H * D > INT32_ELEMS
    gen = torch.Generator(device="cuda")
    gen.manual_seed(2024)
    q, k, v, do = (_normal((T, H, D), gen) for _ in range(4))
    cu = torch.arange(0, T + 1, L, dtype=torch.int32, device="cuda")
    o = torch.full_like(q, float("nan"))
    lse = torch.full((H, T), float("nan"), device="cuda")
    _say(f"large self-attention: T={T} H={H} d={D} causal fwd")
    jfa.jfa_fwd(q, k, v, cu, cu, L, L, True, out=o, lse=lse)
    dq, dk, dv = (torch.full_like(x, float("nan")) for x in (q, k, v))
    _say("large self-attention: bwd")
    jfa.jfa_bwd(q, k, v, o, lse, do, cu, cu, L, L, True, dq=dq, dk=dk, dv=dv)
    torch.cuda.synchronize()
    _all_finite(O=o, LSE=lse, dQ=dq, dK=dk, dV=dv)

    straddle = INT32_ELEMS // (H * D) // L
    assert straddle * L * H * D < INT32_ELEMS < (straddle + 1) * L * H * D
    cq = np.array([0, L])
    for b in (0, straddle - 1, straddle, n - 1):
        s, e = b * L, (b + 1) * L
        _say(f"  oracle: sequence {b} (elements {s * H * D} .. {e * H * D})")
        qs, ks, vs, dos = (host(x[s:e]) for x in (q, k, v, do))
        ro, rl = oracle.attention_forward(qs, ks, vs, cq, cq, True)
        rdq, rdk, rdv = oracle.attention_backward(qs, ks, vs, dos, cq, cq, True)
        check_o(host(o[s:e]), ro)
        check_lse(host(lse[:, s:e]), rl)
        check_grad(host(dq[s:e]), rdq, "dQ")
        check_grad(host(dk[s:e]), rdk, "dK")
        check_grad(host(dv[s:e]), rdv, "dV")


def test_broadcast_q_beyond_int32_offsets(jfa):
    """1052 items share Nq = 1000 queries (16 heads, d = 128), so O and dO [B, Nq, Hq, d]
    hold 2.15e9 elements; item 1048 straddles element 2^31.  dQ is the sum over all items."""
    nq, H, D, B = 1000, 16, 128, 1052
    assert B * nq * H * D > INT32_ELEMS
    lens = np.random.default_rng(77).integers(1, 49, size=B)
    cu_k = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    tk = int(cu_k[-1])
    gen = torch.Generator(device="cuda")
    gen.manual_seed(4048)
    q = _normal((nq, H, D), gen)
    k, v = _normal((tk, H, D), gen), _normal((tk, H, D), gen)
    do = _normal((B, nq, H, D), gen)
    ck = dev(cu_k, torch)
    o = torch.full((B, nq, H, D), float("nan"), device="cuda", dtype=torch.bfloat16)
    lse = torch.full((B, H, nq), float("nan"), device="cuda")
    _say(f"large broadcast-Q: B={B} Nq={nq} H={H} d={D} Tk={tk} fwd")
    jfa.jfa_fwd(q, k, v, None, ck, nq, int(lens.max()), False, broadcast_q=True, out=o, lse=lse)
    dq, dk, dv = (torch.full_like(x, float("nan")) for x in (q, k, v))
    _say("large broadcast-Q: bwd")
    jfa.jfa_bwd(q, k, v, o, lse, do, None, ck, nq, int(lens.max()), False, broadcast_q=True,
                dq=dq, dk=dk, dv=dv)
    torch.cuda.synchronize()
    _all_finite(O=o, LSE=lse, dQ=dq, dK=dk, dV=dv)

    straddle = INT32_ELEMS // (nq * H * D)
    assert straddle * nq * H * D < INT32_ELEMS < (straddle + 1) * nq * H * D
    sampled = {0, straddle - 1, straddle, B - 1}
    qh, kh, vh = host(q), host(k), host(v)
    rdq = np.zeros(qh.shape)
    _say(f"  oracle: {B} items (dQ sums all; O, LSE, dK, dV compared on items {sorted(sampled)})")
    for b in range(B):
        ks, ke = int(cu_k[b]), int(cu_k[b + 1])
        c1 = np.array([0, ke - ks])
        dqb, dkb, dvb = oracle.broadcast_q_backward(qh, kh[ks:ke], vh[ks:ke], host(do[b:b + 1]), c1)
        rdq += dqb
        if b in sampled:
            ro, rl = oracle.broadcast_q_forward(qh, kh[ks:ke], vh[ks:ke], c1)
            check_o(host(o[b:b + 1]), ro)
            check_lse(host(lse[b:b + 1]), rl)
            check_grad(host(dk[ks:ke]), dkb, "dK")
            check_grad(host(dv[ks:ke]), dvb, "dV")
    check_grad(host(dq), rdq, "dQ")


def test_decode_pages_beyond_int32_offsets(jfa):
    """Paged decode whose pages lie on both sides of element 2^31 of a 4.3 GB cache; every
    other page is NaN, so a page address that wrapped would poison the result."""
    inp = workloads.decode(13, np.array([1000, 37, 2049, 16, 512, 1]), heads_q=32, heads_kv=8, head_dim=128,
                           page_size=16)
    per_page = inp.page_size * 8 * 128
    base = INT32_ELEMS // per_page - inp.num_pages // 2
    n_pages = base + inp.num_pages + 8
    assert n_pages * per_page > INT32_ELEMS and base * per_page < INT32_ELEMS
    kc = torch.full((n_pages, inp.page_size, 8, 128), float("nan"), device="cuda", dtype=torch.bfloat16)
    vc = torch.full_like(kc, float("nan"))
    kc[base:base + inp.num_pages] = dev(inp.k_cache, torch)
    vc[base:base + inp.num_pages] = dev(inp.v_cache, torch)
    pt = dev((inp.page_table.astype(np.int64) + base).astype(np.int32), torch)
    q, sl = dev(inp.q, torch), dev(inp.seqlens_k, torch)
    f = lambda x: x.astype(np.float64)
    ro, rl = oracle.decode_forward(f(inp.q), f(inp.k), f(inp.v), inp.cu_k)
    for single_launch in (False, True):
        _say(f"large decode: pages {base}..{base + inp.num_pages} of {n_pages}, single_launch={single_launch}")
        o, lse = jfa.jfa_decode_paged(q, kc, vc, pt, sl, 0, single_launch=single_launch)
        torch.cuda.synchronize()
        check_o(host(o), ro)
        check_lse(host(lse), rl)
