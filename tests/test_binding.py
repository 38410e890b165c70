"""The Python binding validates every tensor before the library is called (no GPU needed).

Each call below passes host tensors with one thing wrong and expects ValueError
naming it; the library loader is replaced by one that fails the test, so a
check that let the call through would be caught even without a GPU.
"""
import pytest

torch = pytest.importorskip("torch")

import bwd_varlen_flashattention_amd as jfa


@pytest.fixture(autouse=True)
def no_library(monkeypatch):
    def fail():
        raise AssertionError("the library was reached before the arguments were rejected")
    monkeypatch.setattr(jfa, "load", fail)


def bf(*shape):
    return torch.zeros(shape, dtype=torch.bfloat16)


def i32(*vals):
    return torch.tensor(vals, dtype=torch.int32)


def fwd_args(**kw):
    a = dict(q=bf(10, 4, 64), k=bf(12, 2, 64), v=bf(12, 2, 64), cu_seqlens_q=i32(0, 4, 10),
             cu_seqlens_k=i32(0, 5, 12), max_seqlen_q=6, max_seqlen_k=7)
    a.update(kw)
    return a


def bwd_args(**kw):
    a = fwd_args()
    a.update(o=bf(10, 4, 64), lse=torch.zeros(4, 10), dout=bf(10, 4, 64))
    a.update(kw)
    return a


FWD_BAD = [
    (dict(q=torch.zeros(10, 4, 64)), "q: dtype"),
    (dict(q=bf(10, 4)), "q: shape"),
    (dict(k=bf(12, 2, 32)), "k: shape"),
    (dict(v=bf(11, 2, 64)), "v: shape"),
    (dict(k=bf(12, 3, 64), v=bf(12, 3, 64)), "multiple"),
    (dict(cu_seqlens_q=i32(0, 10)), "cu_seqlens_q: shape"),
    (dict(cu_seqlens_k=torch.tensor([0, 5, 12])), "cu_seqlens_k: dtype"),
    (dict(out=bf(10, 4, 32)), "out: shape"),
    (dict(lse=torch.zeros(10, 4)), "lse: shape"),
    (dict(q=bf(10, 64, 4).transpose(1, 2)), "q: must be contiguous"),
    ({}, "must be a CUDA tensor"),
]


@pytest.mark.parametrize("kw,msg", FWD_BAD)
def test_fwd_rejects(kw, msg):
    with pytest.raises(ValueError, match=msg):
        jfa.jfa_fwd(**fwd_args(**kw))


def test_fwd_broadcast_shapes():
    with pytest.raises(ValueError, match="out: shape"):
        jfa.jfa_fwd(**fwd_args(cu_seqlens_q=None, broadcast_q=True, out=bf(10, 4, 64)))
    with pytest.raises(ValueError, match="lse: shape"):
        jfa.jfa_fwd(**fwd_args(cu_seqlens_q=None, broadcast_q=True, out=bf(2, 10, 4, 64), lse=torch.zeros(4, 10)))


BWD_BAD = [
    (dict(o=bf(9, 4, 64)), "o: shape"),
    (dict(dout=bf(10, 4, 32)), "dout: shape"),
    (dict(lse=torch.zeros(4, 10, dtype=torch.float64)), "lse: dtype"),
    (dict(lse=torch.zeros(10, 4)), "lse: shape"),
    (dict(cu_seqlens_q=None), "cu_seqlens_q: missing"),
    (dict(dq=bf(10, 4, 32)), "dq: shape"),
    (dict(dk=bf(12, 4, 64)), "dk: shape"),
    (dict(dv=torch.zeros(12, 2, 64)), "dv: dtype"),
    ({}, "must be a CUDA tensor"),
]


@pytest.mark.parametrize("kw,msg", BWD_BAD)
def test_bwd_rejects(kw, msg):
    with pytest.raises(ValueError, match=msg):
        jfa.jfa_bwd(**bwd_args(**kw))


def dec_args(**kw):
    a = dict(q=bf(3, 8, 128), k_cache=bf(20, 16, 2, 128), v_cache=bf(20, 16, 2, 128),
             page_table=torch.zeros(3, 7, dtype=torch.int32), seqlens_k=i32(5, 100, 1))
    a.update(kw)
    return a


DEC_BAD = [
    (dict(q=bf(3, 128)), "q: shape"),
    (dict(k_cache=bf(20, 16, 2, 64)), "k_cache: shape"),
    (dict(v_cache=bf(20, 8, 2, 128)), "v_cache: shape"),
    (dict(v_cache=torch.zeros(20, 16, 2, 128, dtype=torch.uint8)), "v_cache: dtype"),
    (dict(page_table=torch.zeros(2, 7, dtype=torch.int32)), "page_table: shape"),
    (dict(seqlens_k=i32(5, 100)), "seqlens_k: shape"),
    (dict(k_cache=bf(20, 16, 3, 128), v_cache=bf(20, 16, 3, 128)), "multiple"),
    (dict(out=bf(3, 8, 64)), "out: shape"),
    (dict(lse=torch.zeros(3, 8, 1)), "lse: shape"),
    ({}, "must be a CUDA tensor"),
]


@pytest.mark.parametrize("kw,msg", DEC_BAD)
def test_decode_rejects(kw, msg):
    with pytest.raises(ValueError, match=msg):
        jfa.jfa_decode_paged(**dec_args(**kw))
