"""jfa_decode_paged_noalloc (split partials in the library's static device array, no
workspace) through the C ABI, against jfa_decode_paged with a caller workspace: two
calls in a row, the second with a smaller problem, outputs compared bit for bit (the
same kernels run on the same inputs) and against the fp64 oracle."""
import numpy as np
import pytest

import oracle
import workloads
from parity import check_lse, check_o, dev, host

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


@pytest.fixture(scope="module")
def jfa():
    import bwd_varlen_flashattention_amd as m
    m.load()
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    return m


def _run_both(jfa, inp, splits, causal=False, single_launch=False):
    q, kc, vc = dev(inp.q, torch), dev(inp.k_cache, torch), dev(inp.v_cache, torch)
    pt, sl = dev(inp.page_table, torch), dev(inp.seqlens_k, torch)
    o_ref, l_ref = jfa.jfa_decode_paged(q, kc, vc, pt, sl, splits, causal=causal)
    o = torch.full_like(o_ref, float("nan"))
    lse = torch.full_like(l_ref, float("nan"))
    jfa.jfa_decode_paged_noalloc(q, kc, vc, pt, sl, splits, out=o, lse=lse, causal=causal,
                                 single_launch=single_launch)
    torch.cuda.synchronize()
    return host(o), host(lse), host(o_ref), host(l_ref)


def test_noalloc_decode_matches_workspace_entry_point(jfa):
    rng = np.random.default_rng(7)
    big = workloads.decode(101, rng.integers(1000, 9000, 32).tolist(), 32, 8, 128, 16)     # 8 splits: 4.2 MB partials
    small = workloads.decode(102, [5, 300, 64, 1], 8, 2, 128, 16, q_len=3)                 # then a smaller one
    # the static array's arrival counters (single-launch mode) start zero and every call
    # leaves them zero, also between calls of the other mode
    for inp, splits, causal, one in ((big, 0, False, False), (small, 5, True, False), (big, 0, False, True),
                                     (small, 5, True, True), (big, 7, False, False), (small, 3, True, True)):
        o, lse, o_ref, l_ref = _run_both(jfa, inp, splits, causal, one)
        np.testing.assert_array_equal(o, o_ref)
        np.testing.assert_array_equal(lse, l_ref)
        f = lambda x: x.astype(np.float64)
        if inp.q.ndim == 3:
            ro, rl = oracle.decode_forward(f(inp.q), f(inp.k), f(inp.v), inp.cu_k)
        else:
            ro, rl = oracle.decode_forward_multi(f(inp.q), f(inp.k), f(inp.v), inp.cu_k, causal)
        check_o(o, ro)
        check_lse(lse, rl)
