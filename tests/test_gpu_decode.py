"""GPU parity: split-KV paged decode through the C ABI against the fp64 oracle."""
import sys

import numpy as np
import pytest

import oracle
import workloads
from parity import check_lse, check_o, dev, half_ulp_bf16, host

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


class _Dev:
    def __init__(self, inp):
        self.q = dev(inp.q, torch)
        self.kc = dev(inp.k_cache, torch)
        self.vc = dev(inp.v_cache, torch)
        self.pt = dev(inp.page_table, torch)
        self.sl = dev(inp.seqlens_k, torch)


def _run(jfa, d, splits, scale=None):
    o, lse = jfa.jfa_decode_paged(d.q, d.kc, d.vc, d.pt, d.sl, splits, scale)
    torch.cuda.synchronize()
    return host(o), host(lse)


def _ref(inp, scale=None):
    f = lambda x: x.astype(np.float64)
    return oracle.decode_forward(f(inp.q), f(inp.k), f(inp.v), inp.cu_k, scale)


@pytest.mark.parametrize("page_size", [1, 3, 16, 64, 128])
@pytest.mark.parametrize("hq,hkv", [(8, 2), (6, 6), (16, 1)])
def test_decode_small(jfa, page_size, hq, hkv):
    lens = [1, 63, 64, 65, 300, 0, 1000, 17]
    inp = workloads.decode(20 + page_size, lens, hq, hkv, 128, page_size)
    _say(f"decode small ps={page_size} hq={hq} hkv={hkv}")
    d = _Dev(inp)
    ro, rl = _ref(inp)
    for splits in (1, 2, 5, 16):
        o, lse = _run(jfa, d, splits)
        check_o(o, ro, f"O splits={splits}")
        check_lse(lse, rl, f"LSE splits={splits}")


@pytest.mark.parametrize("scale", [4.0, 1e-3])
def test_decode_extreme_scales(jfa, scale):
    """Nearly one-hot (scale 4) and nearly flat (1e-3) rows, across split counts."""
    inp = workloads.decode(61, [1, 900, 64, 2500, 17], 8, 2, 128, 16)
    _say(f"decode extreme scale {scale}")
    d = _Dev(inp)
    ro, rl = _ref(inp, scale)
    for splits in (1, 3, 0):
        o, lse = _run(jfa, d, splits, scale)
        check_o(o, ro, f"O splits={splits}")
        check_lse(lse, rl, f"LSE splits={splits}")


@pytest.mark.parametrize("dim", [64, 96, 192, 256])
def test_decode_head_dims(jfa, dim):
    inp = workloads.decode(31, [5, 200, 129], 8, 2, dim, 16)
    d = _Dev(inp)
    ro, rl = _ref(inp)
    for splits in (1, 3):
        o, lse = _run(jfa, d, splits)
        check_o(o, ro)
        check_lse(lse, rl)


@pytest.mark.parametrize("page_size", [16, 1, 128])
def test_decode_config_full(jfa, page_size):
    """The decode config at full size (B=32, Hq=32/Hkv=8, d=128, L ~ U{4096..16384}), all splits."""
    inp = workloads.decode_paged(0, page_size)
    _say(f"decode config ps={page_size} pages={inp.num_pages}")
    d = _Dev(inp)
    ro, rl = _ref(inp)
    outs = []
    for splits in (1, 2, 4, 8, 16, 0):
        o, lse = _run(jfa, d, splits)
        check_o(o, ro, f"O splits={splits}")
        check_lse(lse, rl, f"LSE splits={splits}")
        outs.append(o)
    # independent of the split count up to fp32 rounding
    for o in outs[1:]:
        assert np.abs(o - outs[0]).max() <= 2e-2


def test_decode_page_permutation_invariance(jfa):
    """Same contiguous KV under two different page permutations and page sizes gives the same result."""
    lens = [700, 33, 4096]
    a = workloads.decode(41, lens, 8, 2, 128, 16)
    b = workloads.repage(a, 7, seed=5)
    assert not np.array_equal(a.page_table[:, :5], b.page_table[:, :5])
    oa, la = _run(jfa, _Dev(a), 4)
    ob, lb = _run(jfa, _Dev(b), 4)
    assert np.abs(oa - ob).max() <= 2e-2
    assert np.abs(la - lb).max() <= 1e-3


def test_decode_equals_forward_with_one_query(jfa):
    """GPU decode equals the GPU jagged forward with Lq = 1 and the contiguous KV."""
    import bwd_varlen_flashattention_amd as m
    inp = workloads.decode(43, [50, 129, 1], 8, 2, 128, 16)
    o, lse = _run(jfa, _Dev(inp), 2)
    q = dev(inp.q, torch)
    k, v = dev(inp.k, torch), dev(inp.v, torch)
    cq = torch.arange(4, dtype=torch.int32, device="cuda")
    ck = dev(inp.cu_k, torch)
    of, lf = m.jfa_fwd(q, k, v, cq, ck, 1, 129)
    torch.cuda.synchronize()
    assert np.abs(o - host(of)).max() <= 2e-2
    assert np.abs(lse - host(lf).T).max() <= 1e-3


# ------------------------------------------------------------ a few new tokens per sequence
def _ref_multi(inp, causal, scale=None):
    f = lambda x: x.astype(np.float64)
    return oracle.decode_forward_multi(f(inp.q), f(inp.k), f(inp.v), inp.cu_k, causal, scale)


@pytest.mark.parametrize("q_len", [2, 3, 4, 8, 16])
@pytest.mark.parametrize("hq,hkv", [(8, 2), (6, 6), (16, 1)])
@pytest.mark.parametrize("causal", [False, True])
def test_decode_multi_token(jfa, q_len, hq, hkv, causal):
    """Speculative-decode / chunked-prefill shapes: q_len tokens per sequence, GQA
    ratios 4, 1 and 16 (up to 256 query columns per KV head), lengths shorter than
    q_len included (causal tokens that see no key get O = 0, LSE = -inf)."""
    lens = [1, 63, 64, 65, 300, 0, 700, 17, 5]
    inp = workloads.decode(40 + q_len, lens, hq, hkv, 128, 16, q_len=q_len)
    _say(f"decode multi q_len={q_len} hq={hq} hkv={hkv} causal={causal}")
    d = _Dev(inp)
    ro, rl = _ref_multi(inp, causal)
    for splits in (1, 3, 0):
        o, lse = jfa.jfa_decode_paged(d.q, d.kc, d.vc, d.pt, d.sl, splits, causal=causal)
        torch.cuda.synchronize()
        check_o(host(o), ro, f"O splits={splits}")
        check_lse(host(lse), rl, f"LSE splits={splits}")


@pytest.mark.parametrize("page_size", [1, 128])
@pytest.mark.parametrize("dim", [64, 96, 256])
def test_decode_multi_token_pages_dims(jfa, page_size, dim):
    inp = workloads.decode(55, [3, 200, 129, 64], 8, 2, dim, page_size, q_len=5)
    d = _Dev(inp)
    ro, rl = _ref_multi(inp, True)
    for splits in (1, 2):
        o, lse = jfa.jfa_decode_paged(d.q, d.kc, d.vc, d.pt, d.sl, splits, causal=True)
        torch.cuda.synchronize()
        check_o(host(o), ro)
        check_lse(host(lse), rl)


def test_decode_multi_token_config_sampled(jfa):
    """Speculative decode at the decode config's size: B=32, 4 new tokens, Hq 32 / Hkv 8,
    d=128, KV lengths U{4096..16384}, page 16, causal; sampled sequences vs the oracle."""
    rng = np.random.default_rng(0)
    lens = rng.integers(4096, 16385, size=32)
    inp = workloads.decode(0, lens, 32, 8, 128, 16, max_pages_per_seq=1024, tail_fill=0.0, q_len=4)
    d = _Dev(inp)
    o, lse = jfa.jfa_decode_paged(d.q, d.kc, d.vc, d.pt, d.sl, 0, causal=True)
    torch.cuda.synchronize()
    o, lse = host(o), host(lse)
    f = lambda x: x.astype(np.float64)
    for b in (0, 13, 31):
        ks, ke = inp.cu_k[b], inp.cu_k[b + 1]
        ro, rl = oracle.decode_forward_multi(f(inp.q[b:b + 1]), f(inp.k[ks:ke]), f(inp.v[ks:ke]),
                                             np.array([0, ke - ks]), True)
        check_o(o[b:b + 1], ro, f"O[seq {b}]")
        check_lse(lse[b:b + 1], rl, f"LSE[seq {b}]")


# ------------------------------------------------------------ fp8 (e4m3) KV cache
class _DevFp8(_Dev):
    def __init__(self, inp):
        self.q = dev(inp.q, torch)
        self.kc = torch.from_numpy(inp.k_cache).to("cuda").view(torch.float8_e4m3fn)
        self.vc = torch.from_numpy(inp.v_cache).to("cuda").view(torch.float8_e4m3fn)
        self.pt = dev(inp.page_table, torch)
        self.sl = dev(inp.seqlens_k, torch)


@pytest.mark.parametrize("q_len,causal", [(1, False), (4, True), (9, False)])
@pytest.mark.parametrize("page_size", [1, 16, 128])
@pytest.mark.parametrize("dim", [64, 96, 128, 192, 256])
def test_decode_fp8_kv(jfa, q_len, causal, page_size, dim):
    """FP8 caches: the result equals attention on the dequantised K/V (scales 0.5 and
    2.0 exercise both scale paths); unused slots hold NaN bytes."""
    lens = [1, 63, 64, 65, 300, 0, 700, 17]
    inp = workloads.decode(60 + dim, lens, 8, 2, dim, page_size, q_len=q_len, kv_fp8=True,
                           k_scale=0.5, v_scale=2.0)
    d = _DevFp8(inp)
    f = lambda x: x.astype(np.float64)
    if q_len == 1:
        ro, rl = oracle.decode_forward(f(inp.q), f(inp.k), f(inp.v), inp.cu_k)
    else:
        ro, rl = oracle.decode_forward_multi(f(inp.q), f(inp.k), f(inp.v), inp.cu_k, causal)
    for splits in (1, 3, 0):
        o, lse = jfa.jfa_decode_paged(d.q, d.kc, d.vc, d.pt, d.sl, splits, causal=causal, k_scale=0.5, v_scale=2.0)
        torch.cuda.synchronize()
        check_o(host(o), ro, f"O splits={splits}")
        check_lse(host(lse), rl, f"LSE splits={splits}")


def test_decode_fp8_config_sampled(jfa):
    """FP8 cache at the decode config's size (B=32, Hq 32 / Hkv 8, d=128, U{4096..16384}, page 16)."""
    rng = np.random.default_rng(0)
    lens = rng.integers(4096, 16385, size=32)
    inp = workloads.decode(0, lens, 32, 8, 128, 16, max_pages_per_seq=1024, kv_fp8=True, k_scale=0.25, v_scale=0.25)
    d = _DevFp8(inp)
    o, lse = jfa.jfa_decode_paged(d.q, d.kc, d.vc, d.pt, d.sl, 0, k_scale=0.25, v_scale=0.25)
    torch.cuda.synchronize()
    o, lse = host(o), host(lse)
    f = lambda x: x.astype(np.float64)
    for b in (0, 13, 31):
        ks, ke = inp.cu_k[b], inp.cu_k[b + 1]
        ro, rl = oracle.decode_forward(f(inp.q[b:b + 1]), f(inp.k[ks:ke]), f(inp.v[ks:ke]), np.array([0, ke - ks]))
        check_o(o[b:b + 1], ro, f"O[seq {b}]")
        check_lse(lse[b:b + 1], rl, f"LSE[seq {b}]")


@pytest.mark.parametrize("kv_fp8", [False, True])
@pytest.mark.parametrize("q_len,causal", [(1, False), (4, True)])
@pytest.mark.parametrize("dim", [64, 128, 256])
def test_decode_fp8_query(jfa, kv_fp8, q_len, causal, dim):
    """An e4m3 query (with bf16 or e4m3 caches): the result is attention of the
    dequantised query; the query scale folds into the scores."""
    lens = [1, 63, 300, 0, 129]
    inp = workloads.decode(70 + dim, lens, 8, 2, dim, 16, q_len=q_len, kv_fp8=kv_fp8, k_scale=0.5, v_scale=2.0)
    q8, qd = workloads.e4m3(inp.q, 0.03125)
    d = _DevFp8(inp) if kv_fp8 else _Dev(inp)
    qdev = torch.from_numpy(q8).to("cuda").view(torch.float8_e4m3fn)
    f = lambda x: x.astype(np.float64)
    if q_len == 1:
        ro, rl = oracle.decode_forward(f(qd), f(inp.k), f(inp.v), inp.cu_k)
    else:
        ro, rl = oracle.decode_forward_multi(f(qd), f(inp.k), f(inp.v), inp.cu_k, causal)
    sc = dict(k_scale=0.5, v_scale=2.0) if kv_fp8 else {}
    for splits in (1, 3):
        o, lse = jfa.jfa_decode_paged(qdev, d.kc, d.vc, d.pt, d.sl, splits, causal=causal, q_scale=0.03125, **sc)
        torch.cuda.synchronize()
        check_o(host(o), ro, f"O splits={splits}")
        check_lse(host(lse), rl, f"LSE splits={splits}")


def test_decode_one_very_long_sequence(jfa):
    """One sequence of 262144 cached tokens (16384 pages of 16), Hq 32 / Hkv 8, d = 128,
    automatic and explicit splits."""
    inp = workloads.decode(90, [262144], 32, 8, 128, 16)
    d = _Dev(inp)
    ro, rl = _ref(inp)
    for splits in (0, 7, 128):
        o, lse = _run(jfa, d, splits)
        check_o(o, ro, f"O splits={splits}")
        check_lse(lse, rl, f"LSE splits={splits}")


def test_decode_large_batch(jfa):
    """4096 short sequences (0-100 tokens): past the batch size up to which the
    units are dispatched longest first, so the given order is kept."""
    rng = np.random.default_rng(91)
    lens = rng.integers(0, 101, 4096).tolist()
    inp = workloads.decode(92, lens, 8, 2, 64, 16)
    d = _Dev(inp)
    ro, rl = _ref(inp)
    for splits in (0, 1, 3):
        o, lse = _run(jfa, d, splits)
        check_o(o, ro, f"O splits={splits}")
        check_lse(lse, rl, f"LSE splits={splits}")


@pytest.mark.parametrize("dim", [64, 128, 256])
def test_decode_v_beyond_fp16_range(jfa, dim):
    """V entries of magnitude 2^16 .. 2^27 (beyond fp16) in some units: in fp16 those V values
    become infinite, so the units are computed again with P V in bf16; |error| <= 1e-2 +
    half a bf16 ulp of O + 2^-7 (P |V|) (the output's bf16 rounding, plus bf16 P (2^-8 per
    term) and the normalisation by the unrounded sum (2^-8), relative to P |V|)."""
    import dataclasses
    base = workloads.decode(97, [5, 300, 1000, 64, 1], 8, 2, dim, 16)
    rng = np.random.default_rng(9)
    v = base.v.copy()
    big = [65536.0, -98304.0, 1048576.0, -16777216.0, 2.0 ** 27]
    for i in range(12):
        v[rng.integers(0, v.shape[0]), rng.integers(0, v.shape[1]), rng.integers(0, v.shape[2])] = big[i % 5]
    inp = workloads.repage(dataclasses.replace(base, v=v), 16, 3)
    d = _Dev(inp)
    f = lambda x: x.astype(np.float64)
    ro, rl = oracle.decode_forward(f(inp.q), f(inp.k), f(inp.v), inp.cu_k)
    mag, _ = oracle.decode_forward(f(inp.q), f(inp.k), np.abs(f(inp.v)), inp.cu_k)
    for splits in (1, 3):
        o, lse = _run(jfa, d, splits)
        err, bound = np.abs(o - ro), 1e-2 + half_ulp_bf16(ro) + 2.0 ** -7 * mag
        assert np.isfinite(o).all() and (err <= bound).all(), f"splits={splits}: excess {(err - bound).max():.3e}"
        check_lse(lse, rl)


def test_decode_single_launch_workspace_reuse(jfa):
    """single_launch: the last split of each (sequence, KV head) to finish merges the
    partials inside the decode launch, found through arrival counters at the workspace
    start that must be zero when a call begins.  One workspace, zeroed once, serves
    calls of different shapes, split counts and both modes back to back; after every
    call its counter region is zero again, and each single-launch result equals the
    two-launch one bit for bit (same sums in the same order) and matches the oracle."""
    import bwd_varlen_flashattention_amd._lib as L
    probs = [(workloads.decode(93, [700, 5, 0, 2000, 64], 32, 8, 128, 16), 7, 1),
             (workloads.decode(94, [3000, 1], 8, 2, 64, 3), 16, 1),
             (workloads.decode(95, [33, 900, 4000], 16, 4, 128, 16, q_len=3), 5, 3),
             (workloads.decode(96, [1500] * 40, 32, 8, 256, 128), 3, 1),
             (workloads.decode(97, [100, 20000], 32, 8, 128, 1), 128, 1)]
    need = 0
    for inp, splits, _ in probs:
        d = _Dev(inp)
        need = max(need, jfa.jfa_decode_workspace_size(d.q, d.kc, d.pt, splits))
    ws = torch.zeros(need, dtype=torch.uint8, device="cuda")
    f = lambda x: x.astype(np.float64)
    for rep in range(2):
        for i, (inp, splits, q_len) in enumerate(probs):
            _say(f"workspace reuse: problem {i} splits={splits} rep={rep}")
            d = _Dev(inp)
            o1, l1 = jfa.jfa_decode_paged(d.q, d.kc, d.vc, d.pt, d.sl, splits, workspace=ws, single_launch=True)
            torch.cuda.synchronize()
            assert int(ws[:L.DECODE_COUNTER_BYTES].count_nonzero()) == 0, f"problem {i}: counters left non-zero"
            o2, l2 = jfa.jfa_decode_paged(d.q, d.kc, d.vc, d.pt, d.sl, splits, workspace=ws)
            torch.cuda.synchronize()
            assert int(ws[:L.DECODE_COUNTER_BYTES].count_nonzero()) == 0, f"problem {i}: two-launch call wrote counters"
            np.testing.assert_array_equal(host(o1), host(o2))
            np.testing.assert_array_equal(host(l1), host(l2))
            if q_len == 1:
                ro, rl = oracle.decode_forward(f(inp.q), f(inp.k), f(inp.v), inp.cu_k)
            else:
                ro, rl = oracle.decode_forward_multi(f(inp.q), f(inp.k), f(inp.v), inp.cu_k, False)
            check_o(host(o1), ro, f"O problem {i}")
            check_lse(host(l1), rl, f"LSE problem {i}")


def test_decode_more_units_than_counters(jfa):
    """8200 sequences x 8 KV heads (one query head each): 65600 units, more than the
    65536 arrival counters, so a single-launch call merges in a second launch after all.
    Against the oracle, and bit for bit against the single-launch merge of the first
    8000 sequences (the same tensors, sliced)."""
    rng = np.random.default_rng(98)
    lens = rng.integers(0, 41, 8200).tolist()
    inp = workloads.decode(99, lens, 8, 8, 64, 16)
    d = _Dev(inp)
    ro, rl = _ref(inp)
    o, lse = jfa.jfa_decode_paged(d.q, d.kc, d.vc, d.pt, d.sl, 2, single_launch=True)
    torch.cuda.synchronize()
    o, lse = host(o), host(lse)
    check_o(o, ro, "O (two launches)")
    check_lse(lse, rl, "LSE (two launches)")
    o2, l2 = jfa.jfa_decode_paged(d.q[:8000].contiguous(), d.kc, d.vc, d.pt[:8000].contiguous(),
                                  d.sl[:8000].contiguous(), 2, single_launch=True)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(host(o2), o[:8000])
    np.testing.assert_array_equal(host(l2), lse[:8000])
