"""GPU parity: e4m3 (FP8) forward through the C ABI against the fp64 oracle on the
dequantised inputs ("Optimizing FlashAttention-4 for Efficient Inference", PR 2109).

Q K^T runs on the e4m3 matrix cores with exact products and fp32 accumulation, and V
is widened exactly to bf16, so the result is the bf16 path's attention on the scaled
e4m3 values: the bf16 tolerances apply unchanged."""
import sys

import numpy as np
import pytest

import oracle
import workloads
from parity import check_lse, check_o, dev, host

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


def _say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module")
def jfa():
    import bwd_varlen_flashattention_amd as m
    m.load()
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    return m


def _u8(x):
    return torch.from_numpy(x).to("cuda").view(torch.float8_e4m3fn)


def _run(jfa, inp, enc, broadcast=False):
    q, k, v = _u8(enc["q"]), _u8(enc["k"]), _u8(enc["v"])
    ck = dev(inp.cu_k, torch)
    sc = dict(q_scale=enc["q_scale"], k_scale=enc["k_scale"], v_scale=enc["v_scale"])
    if broadcast:
        o, lse = jfa.jfa_fwd(q, k, v, None, ck, q.shape[0], inp.max_len_k, False, None, broadcast_q=True, **sc)
    else:
        o, lse = jfa.jfa_fwd(q, k, v, dev(inp.cu_q, torch), ck, inp.max_len_q, inp.max_len_k, inp.causal, None, **sc)
    torch.cuda.synchronize()
    return host(o), host(lse)


def _oracle(inp, seqs=None):
    f = lambda x: x.astype(np.float64)
    if seqs is None:
        return oracle.attention_forward(f(inp.q), f(inp.k), f(inp.v), inp.cu_q, inp.cu_k, inp.causal)
    out = {}
    for b in seqs:
        qs, qe, ks, ke = inp.cu_q[b], inp.cu_q[b + 1], inp.cu_k[b], inp.cu_k[b + 1]
        out[b] = oracle.attention_forward(f(inp.q[qs:qe]), f(inp.k[ks:ke]), f(inp.v[ks:ke]),
                                          np.array([0, qe - qs]), np.array([0, ke - ks]), inp.causal)
    return out


RAGGED = [1, 31, 32, 33, 63, 64, 65, 127, 128, 129, 200, 0, 257, 5]


@pytest.mark.parametrize("d", [64, 128, 192, 256])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("hq,hkv", [(2, 2), (4, 2)])
def test_fp8_ragged(jfa, d, causal, hq, hkv):
    inp, enc = workloads.fp8_qkv(workloads.jagged(200 + d, RAGGED, None, hq, hkv, d, causal))
    _say(f"fp8 ragged d={d} causal={causal} hq={hq} hkv={hkv}")
    o, lse = _run(jfa, inp, enc)
    ro, rl = _oracle(inp)
    check_o(o, ro)
    check_lse(lse, rl)


@pytest.mark.parametrize("scales", [(0.5, 0.25, 2.0), (0.05, 0.04, 0.03)])
def test_fp8_explicit_scales(jfa, scales):
    """Scales fold into the scores (Q and K) and the output (V)."""
    inp, enc = workloads.fp8_qkv(workloads.jagged(7, [300, 1, 77], [100, 50, 260], 4, 4, 128, True), *scales)
    o, lse = _run(jfa, inp, enc)
    ro, rl = _oracle(inp)
    check_o(o, ro)
    check_lse(lse, rl)


def test_fp8_broadcast_q(jfa):
    base = workloads.broadcast(8, 130, [70, 0, 200, 129, 1], 4, 2, 128)
    inp, enc = workloads.fp8_qkv(base)
    o, lse = _run(jfa, inp, enc, broadcast=True)
    f = lambda x: x.astype(np.float64)
    ro, rl = oracle.broadcast_q_forward(f(inp.q), f(inp.k), f(inp.v), inp.cu_k)
    check_o(o, ro)
    check_lse(lse, rl)


def test_fp8_gem_full_size_sampled(jfa):
    """GEM s = 0.5 (256 sequences, 8 heads, d = 128) in e4m3; oracle on sampled sequences."""
    inp, enc = workloads.fp8_qkv(workloads.gem(0, 0.5))
    o, lse = _run(jfa, inp, enc)
    lens = np.diff(inp.cu_q)
    order = np.argsort(lens)
    seqs = sorted(set(order[:2].tolist() + order[-2:].tolist() + [0, 100, 255]))
    for b, (ro, rl) in _oracle(inp, seqs).items():
        qs, qe = inp.cu_q[b], inp.cu_q[b + 1]
        check_o(o[qs:qe], ro, f"O[seq {b}]")
        check_lse(lse[:, qs:qe], rl, f"LSE[seq {b}]")


def test_fp8_matches_bf16_path_on_the_same_values(jfa):
    """The e4m3 forward equals the bf16 forward run on the dequantised values up to
    summation order (both round P to bf16 and accumulate in fp32).  Power-of-two
    scales keep the dequantised values exact in bf16."""
    inp, enc = workloads.fp8_qkv(workloads.jagged(9, [513, 64, 1000], None, 4, 2, 128, False), 0.015625, 0.015625, 0.03125)
    o8, l8 = _run(jfa, inp, enc)
    q, k, v = (dev(x, torch) for x in (inp.q, inp.k, inp.v))
    cq, ck = dev(inp.cu_q, torch), dev(inp.cu_k, torch)
    o, l = jfa.jfa_fwd(q, k, v, cq, ck, inp.max_len_q, inp.max_len_k, False)
    torch.cuda.synchronize()
    assert np.abs(host(l) - l8).max() <= 1e-4
    assert np.abs(host(o) - o8).max() <= 2e-2
