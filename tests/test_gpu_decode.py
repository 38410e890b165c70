"""GPU parity: split-KV paged decode through the C ABI against the fp64 oracle."""
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


@pytest.mark.parametrize("dim", [64, 96])
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
