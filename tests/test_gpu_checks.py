"""GPU: the device-side input checks (jfa_check_offsets, jfa_check_paged_cache) report
exactly the violated conditions, and 0 for valid inputs.  Only the check kernels read
the corrupted arrays: no attention kernel is launched on them."""
import numpy as np
import pytest

import workloads
from parity import dev

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


@pytest.fixture(scope="module")
def jfa():
    import bwd_varlen_flashattention_amd as m
    m.load()
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    return m


def _off(a):
    return torch.tensor(np.asarray(a, dtype=np.int32), device="cuda")


def test_check_offsets(jfa):
    from bwd_varlen_flashattention_amd import _lib as L
    inp = workloads.gem(0, 0.5)
    cu = inp.cu_q.astype(np.int32)
    total = int(cu[-1])
    assert jfa.jfa_check_offsets(_off(cu), total) == 0
    assert jfa.jfa_check_offsets(_off([0]), 0) == 0                       # no sequences
    assert jfa.jfa_check_offsets(_off([0, 0, 0, 5, 5]), 5) == 0           # empty sequences are legal
    bad = cu.copy(); bad[0] = 3
    assert jfa.jfa_check_offsets(_off(bad), total) == L.CHECK_OFFSETS_START | L.CHECK_OFFSETS_ORDER * int((np.diff(bad) < 0).any())
    bad = cu.copy(); bad[100] = bad[99] - 1
    assert jfa.jfa_check_offsets(_off(bad), total) == L.CHECK_OFFSETS_ORDER
    assert jfa.jfa_check_offsets(_off(cu), total + 1) == L.CHECK_OFFSETS_END
    bad = cu.copy(); bad[0] = -1; bad[-1] = total + 7; bad[200], bad[201] = bad[201], bad[200] - 1
    assert jfa.jfa_check_offsets(_off(bad), total) == (L.CHECK_OFFSETS_START | L.CHECK_OFFSETS_ORDER
                                                       | L.CHECK_OFFSETS_END)
    # past one workgroup's stride: 5000 sequences, a decrease near the end
    many = np.concatenate([[0], np.cumsum(np.arange(5000) % 7)]).astype(np.int32)
    assert jfa.jfa_check_offsets(_off(many), int(many[-1])) == 0
    many[4990] = many[4989] - 1
    assert jfa.jfa_check_offsets(_off(many), int(many[-1])) == L.CHECK_OFFSETS_ORDER


def test_check_paged_cache(jfa):
    from bwd_varlen_flashattention_amd import _lib as L
    inp = workloads.decode(3, [40, 300, 0, 7, 4096], 8, 2, 128, 16)
    q, kc, pt, sl = dev(inp.q, torch), dev(inp.k_cache, torch), dev(inp.page_table, torch), dev(inp.seqlens_k, torch)
    assert jfa.jfa_check_paged_cache(q, kc, pt, sl) == 0
    npages = kc.shape[0]
    cap = pt.shape[1] * kc.shape[1]
    bad = pt.clone(); bad[1, 18] = npages                               # last page of sequence 1 (300 tokens)
    assert jfa.jfa_check_paged_cache(q, kc, bad, sl) == L.CHECK_PAGE_RANGE
    bad = pt.clone(); bad[4, 0] = -2
    assert jfa.jfa_check_paged_cache(q, kc, bad, sl) == L.CHECK_PAGE_RANGE
    bad = pt.clone(); bad[0, 3] = npages + 5                            # past sequence 0's pages: unused
    assert jfa.jfa_check_paged_cache(q, kc, bad, sl) == 0
    bl = sl.clone(); bl[2] = -1
    assert jfa.jfa_check_paged_cache(q, kc, pt, bl) == L.CHECK_SEQLEN_RANGE
    bl = sl.clone(); bl[3] = cap + 1
    assert jfa.jfa_check_paged_cache(q, kc, pt, bl) == L.CHECK_SEQLEN_RANGE
    bl = sl.clone(); bl[3] = cap                                        # capacity itself is legal
    assert jfa.jfa_check_paged_cache(q, kc, pt, bl) == L.CHECK_PAGE_RANGE * int((pt[3] < 0).any() or (pt[3] >= npages).any())
    bad = pt.clone(); bad[1, 0] = npages
    bl = sl.clone(); bl[0] = -5
    assert jfa.jfa_check_paged_cache(q, kc, bad, bl) == L.CHECK_PAGE_RANGE | L.CHECK_SEQLEN_RANGE


def test_check_paged_cache_decode_workload(jfa):
    for ps in (1, 16, 128):
        inp = workloads.decode_paged(0, ps)
        q, kc, pt, sl = (dev(x, torch) for x in (inp.q, inp.k_cache, inp.page_table, inp.seqlens_k))
        assert jfa.jfa_check_paged_cache(q, kc, pt, sl) == 0
