"""C ABI checks that need no GPU: the library loads, exports every declared symbol,
and rejects bad arguments with the documented status before touching the device."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "jfa.h")


def _lib():
    from bwd_varlen_flashattention_amd import _lib as L
    if not os.path.exists(L.LIB_PATH):
        pytest.fail("libjfa.so is not built (run __graft_entry__.build())")
    return L, L.load()


def _declared():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"\b(jfa_[a-z_0-9]+)\s*\(", text)) - {"jfa_status_t"})


def test_header_declares_and_library_exports():
    L, lib = _lib()
    names = _declared()
    assert "jfa_fwd" in names and "jfa_bwd" in names and "jfa_decode_paged" in names
    for n in names:
        assert hasattr(lib, n), f"missing export {n}"
    assert set(names) == set(L.EXPORTS)
    assert lib.jfa_abi_version() == L.ABI_VERSION == 6


def test_header_compiles_as_c(tmp_path):
    src = tmp_path / "t.c"
    src.write_text('#include "jfa.h"\nint main(void){ jfa_attn_params_t p; (void)p; return JFA_OK; }\n')
    r = os.system(f"gcc -std=c99 -Wall -Werror -I {os.path.dirname(HEADER)} -c {src} -o {tmp_path / 't.o'}")
    assert r == 0


def _params(L, **kw):
    base = dict(batch=2, num_heads_q=4, num_heads_kv=2, head_dim=128, total_q=10, total_k=10,
                max_seqlen_q=5, max_seqlen_k=5, causal=0, broadcast_q=0, softmax_scale=0.0)
    base.update(kw)
    return L.AttnParams(**base)


BAD = [
    (dict(head_dim=80), 2), (dict(head_dim=320), 2), (dict(head_dim=160), 2), (dict(num_heads_q=3), 1), (dict(batch=0), 1),
    (dict(total_q=-1), 1), (dict(causal=2), 1), (dict(broadcast_q=1, causal=1), 2),
    (dict(softmax_scale=float("nan")), 1),
    (dict(qkv_dtype=2), 1), (dict(qkv_dtype=1, q_scale=0.0, k_scale=1.0, v_scale=1.0), 1),
    (dict(qkv_dtype=1, q_scale=1.0, k_scale=float("inf"), v_scale=1.0), 1),
    (dict(qkv_dtype=1, q_scale=1.0, k_scale=1.0, v_scale=float("nan")), 1),
    (dict(qkv_dtype=1, q_scale=1.0, k_scale=1.0, v_scale=1.0, head_dim=96), 2),
    (dict(query_tile=64), 1), (dict(query_tile=-1), 1), (dict(query_tile=512), 1),
]


@pytest.mark.parametrize("kw,status", BAD)
def test_invalid_attention_arguments(kw, status):
    L, lib = _lib()
    p = _params(L, **kw)
    dummy = ctypes.c_void_p(16)
    assert lib.jfa_fwd_workspace_size(ctypes.byref(p)) == 0
    st = lib.jfa_fwd(ctypes.byref(p), dummy, dummy, dummy, dummy, dummy, dummy, dummy, dummy, 1 << 20, None)
    assert st == status, L.status_string(st)
    st = lib.jfa_bwd(ctypes.byref(p), dummy, dummy, dummy, dummy, dummy, dummy, dummy, dummy,
                     dummy, dummy, dummy, dummy, 1 << 20, None)
    assert st == status


def test_null_pointers_and_small_workspace():
    L, lib = _lib()
    p = _params(L)
    d = ctypes.c_void_p(256)
    need = lib.jfa_fwd_workspace_size(ctypes.byref(p))
    assert need > 0
    assert lib.jfa_fwd(None, d, d, d, d, d, d, d, d, need, None) == L.JFA_ERR_INVALID_ARGUMENT
    assert lib.jfa_fwd(ctypes.byref(p), None, d, d, d, d, d, d, d, need, None) == L.JFA_ERR_INVALID_ARGUMENT
    assert lib.jfa_fwd(ctypes.byref(p), d, d, d, d, d, d, d, d, need - 1, None) == L.JFA_ERR_WORKSPACE_TOO_SMALL
    nb = lib.jfa_bwd_workspace_size(ctypes.byref(p))
    assert nb >= 4 * 10 * 4           # at least delta (fp32 per query row and head)
    pb = _params(L, broadcast_q=1)
    assert lib.jfa_bwd_workspace_size(ctypes.byref(pb)) >= 10 * 4 * 128 * 4   # + at least one fp32 dQ partial
    assert lib.jfa_bwd(ctypes.byref(p), d, d, d, d, d, d, d, d, d, d, d, d, nb - 1, None) == L.JFA_ERR_WORKSPACE_TOO_SMALL
    assert lib.jfa_bwd(ctypes.byref(p), d, d, d, None, d, d, d, d, d, d, d, d, nb, None) == L.JFA_ERR_INVALID_ARGUMENT


def test_misaligned_workspace_is_rejected():
    L, lib = _lib()
    p = _params(L)
    d, mis = ctypes.c_void_p(256), ctypes.c_void_p(256 + 16)
    nf, nb = lib.jfa_fwd_workspace_size(ctypes.byref(p)), lib.jfa_bwd_workspace_size(ctypes.byref(p))
    assert lib.jfa_fwd(ctypes.byref(p), d, d, d, d, d, d, d, mis, nf, None) == L.JFA_ERR_INVALID_ARGUMENT
    assert lib.jfa_bwd(ctypes.byref(p), d, d, d, d, d, d, d, d, d, d, d, mis, nb, None) == L.JFA_ERR_INVALID_ARGUMENT
    pd = L.DecodeParams(batch=2, num_heads_q=32, num_heads_kv=8, head_dim=128, page_size=16, num_pages=10,
                        max_pages_per_seq=5, num_splits=4, softmax_scale=0.0, q_len=1, causal=0)
    nd = lib.jfa_decode_workspace_size(ctypes.byref(pd))
    assert lib.jfa_decode_paged(ctypes.byref(pd), d, d, d, d, d, d, d, mis, nd, None) == L.JFA_ERR_INVALID_ARGUMENT


def test_query_tile_sizes_the_work_lists():
    """query_tile picks the forward / dQ item size where the kernel has two (bf16, d = 64 / 128):
    128-row items need longer work lists than 256-row ones; elsewhere it changes nothing."""
    L, lib = _lib()
    size = lambda f, **kw: f(ctypes.byref(_params(L, batch=4, total_q=4000, total_k=4000, **kw)))
    for f in (lib.jfa_fwd_workspace_size, lib.jfa_bwd_workspace_size):
        wide, narrow = size(f, query_tile=256), size(f, query_tile=128)
        assert narrow > wide > 0
        # mean 1000 query rows per sequence: the automatic choice is the 256-row item
        assert size(f, query_tile=0) == wide
    # mean 100 rows: the automatic choice is the 128-row item
    p = lambda qt: _params(L, batch=40, total_q=4000, total_k=4000, query_tile=qt)
    assert lib.jfa_fwd_workspace_size(ctypes.byref(p(0))) == lib.jfa_fwd_workspace_size(ctypes.byref(p(128)))
    # d = 96 has one shape
    assert size(lib.jfa_fwd_workspace_size, head_dim=96, query_tile=128) == \
        size(lib.jfa_fwd_workspace_size, head_dim=96, query_tile=256)


def test_empty_problem_is_a_no_op():
    L, lib = _lib()
    p = _params(L, total_q=0, total_k=0)
    assert lib.jfa_fwd(ctypes.byref(p), None, None, None, None, None, None, None, None, 0, None) == L.JFA_OK


DEC_BAD = [
    (dict(page_size=0), 1), (dict(num_splits=129), 1), (dict(num_splits=-1), 1), (dict(head_dim=48), 2),
    (dict(num_heads_q=514, num_heads_kv=2), 2), (dict(num_heads_q=34, num_heads_kv=2, q_len=16), 2),
    (dict(num_heads_q=30), 1), (dict(num_pages=0), 1),
    (dict(q_len=0), 1), (dict(q_len=17), 1), (dict(causal=2), 1),
    (dict(q_dtype=2), 1), (dict(q_dtype=1, q_scale=float("nan")), 1), (dict(kv_dtype=3), 1),
    (dict(single_launch=2), 1), (dict(single_launch=-1), 1),
]


@pytest.mark.parametrize("kw,status", DEC_BAD)
def test_invalid_decode_arguments(kw, status):
    L, lib = _lib()
    base = dict(batch=2, num_heads_q=32, num_heads_kv=8, head_dim=128, page_size=16, num_pages=10,
                max_pages_per_seq=5, num_splits=4, softmax_scale=0.0, q_len=1, causal=0)
    base.update(kw)
    p = L.DecodeParams(**base)
    d = ctypes.c_void_p(16)
    assert lib.jfa_decode_paged(ctypes.byref(p), d, d, d, d, d, d, d, d, 1 << 20, None) == status


def test_decode_workspace_query():
    L, lib = _lib()
    p = L.DecodeParams(batch=32, num_heads_q=32, num_heads_kv=8, head_dim=128, page_size=16, num_pages=100,
                       max_pages_per_seq=1024, num_splits=4, softmax_scale=0.0, q_len=1, causal=0)
    assert lib.jfa_decode_workspace_size(ctypes.byref(p)) >= 4 * 32 * 32 * 129 * 4
    p.q_len = 4
    assert lib.jfa_decode_workspace_size(ctypes.byref(p)) >= 4 * 32 * 4 * 32 * 129 * 4   # partials per token
    p.q_len = 1
    # the arrival counters, then the fp32 partials O_s and LSE_s (each 256-byte aligned)
    assert lib.jfa_decode_workspace_size(ctypes.byref(p)) == L.DECODE_COUNTER_BYTES + 4 * 32 * 32 * 128 * 4 + 4 * 32 * 32 * 4
    assert "#define JFA_DECODE_COUNTER_BYTES ((size_t)256 << 10)" in open(HEADER).read()
    p.num_splits = 1
    assert lib.jfa_decode_workspace_size(ctypes.byref(p)) == 0
    d = ctypes.c_void_p(256)
    p.num_splits = 4
    assert lib.jfa_decode_paged(ctypes.byref(p), d, d, d, d, d, d, d, d, 16, None) == L.JFA_ERR_WORKSPACE_TOO_SMALL


def test_status_strings():
    L, lib = _lib()
    assert L.status_string(0) == "JFA_OK"
    assert L.status_string(2) == "JFA_ERR_UNSUPPORTED"


@pytest.mark.parametrize("d", [192, 256])
def test_large_head_dims_are_accepted(d):
    """d = 192 and 256 are supported: workspace queries succeed, and at d = 256 the
    dK/dV work list holds one item per 128-column head-dim slice (more workspace)."""
    L, lib = _lib()
    p = _params(L, head_dim=d, total_q=5000, total_k=5000, max_seqlen_q=2500, max_seqlen_k=2500)
    assert lib.jfa_fwd_workspace_size(ctypes.byref(p)) > 0
    wd = lib.jfa_bwd_workspace_size(ctypes.byref(p))
    p128 = _params(L, total_q=5000, total_k=5000, max_seqlen_q=2500, max_seqlen_k=2500)
    w128 = lib.jfa_bwd_workspace_size(ctypes.byref(p128))
    assert wd >= w128
    if d == 256:
        items = (5000 // 128 + 1 + 2) * 2 * 16      # (key tiles + batch) x Hkv x 16-byte items
        assert wd - w128 >= items - 256             # one more item per slice, up to a 256-byte pad
    pd = L.DecodeParams(batch=2, num_heads_q=8, num_heads_kv=2, head_dim=d, page_size=16, num_pages=10,
                        max_pages_per_seq=5, num_splits=2, softmax_scale=0.0, q_len=1, causal=0)
    assert lib.jfa_decode_workspace_size(ctypes.byref(pd)) >= 2 * 2 * 8 * (d + 1) * 4


def test_fp8_forward_only():
    """e4m3 Q/K/V is an inference input: the forward accepts it (d a multiple of 64),
    the backward reports JFA_ERR_UNSUPPORTED and needs no workspace."""
    L, lib = _lib()
    p = _params(L, qkv_dtype=1, q_scale=0.5, k_scale=0.25, v_scale=2.0)
    assert lib.jfa_fwd_workspace_size(ctypes.byref(p)) > 0
    assert lib.jfa_bwd_workspace_size(ctypes.byref(p)) == 0
    d = ctypes.c_void_p(256)
    st = lib.jfa_bwd(ctypes.byref(p), d, d, d, d, d, d, d, d, d, d, d, d, 1 << 20, None)
    assert st == L.JFA_ERR_UNSUPPORTED


def test_empty_broadcast_query_workspace_query():
    """Broadcast-Q with Nq = 0 (and keys present): the workspace queries answer without
    dividing by the zero query-tile count, and the call's host checks pass."""
    L, lib = _lib()
    p = _params(L, broadcast_q=1, total_q=0, total_k=10)
    assert lib.jfa_fwd_workspace_size(ctypes.byref(p)) > 0
    assert lib.jfa_bwd_workspace_size(ctypes.byref(p)) > 0
    # nothing to write in the forward: returns before any launch
    assert lib.jfa_fwd(ctypes.byref(p), None, None, None, None, ctypes.c_void_p(256), None, None,
                       ctypes.c_void_p(256), 1 << 20, None) == L.JFA_OK


def test_struct_layouts_match_the_header(tmp_path):
    """The ctypes structs have the sizes and field offsets the C compiler gives the header's."""
    L, _ = _lib()
    structs = {"jfa_attn_params_t": L.AttnParams, "jfa_decode_params_t": L.DecodeParams,
               "jfa_kernel_events_t": L.KernelEventsStruct}
    lines = ['#include <stdio.h>', '#include <stddef.h>', '#include "jfa.h"', "int main(void) {"]
    for cname, cls in structs.items():
        lines.append(f'  printf("{cname} size %zu\\n", sizeof({cname}));')
        for f, _t in cls._fields_:
            lines.append(f'  printf("{cname} {f} %zu\\n", offsetof({cname}, {f}));')
    lines += ["  return 0;", "}"]
    src = tmp_path / "layout.c"
    src.write_text("\n".join(lines) + "\n")
    exe = tmp_path / "layout"
    assert os.system(f"gcc -std=c99 -I {os.path.dirname(HEADER)} {src} -o {exe}") == 0
    out = os.popen(str(exe)).read().split("\n")
    got = {tuple(l.split()[:2]): int(l.split()[2]) for l in out if l.strip()}
    for cname, cls in structs.items():
        assert got[(cname, "size")] == ctypes.sizeof(cls), cname
        for f, _t in cls._fields_:
            assert got[(cname, f)] == getattr(cls, f).offset, (cname, f)


def test_noalloc_decode_rejects_problems_beyond_its_scratch():
    """jfa_decode_paged_noalloc: partials larger than its static array are refused before
    any launch; invalid params keep their usual status."""
    L, lib = _lib()
    d = ctypes.c_void_p(256)
    p = L.DecodeParams(batch=256, num_heads_q=64, num_heads_kv=8, head_dim=128, page_size=16, num_pages=10,
                       max_pages_per_seq=1024, num_splits=16, softmax_scale=0.0, q_len=1, causal=0)
    assert lib.jfa_decode_workspace_size(ctypes.byref(p)) > L.DECODE_SCRATCH_BYTES
    assert lib.jfa_decode_paged_noalloc(ctypes.byref(p), d, d, d, d, d, d, d, None) == L.JFA_ERR_WORKSPACE_TOO_SMALL
    p.page_size = 0
    assert lib.jfa_decode_paged_noalloc(ctypes.byref(p), d, d, d, d, d, d, d, None) == L.JFA_ERR_INVALID_ARGUMENT
    text = open(HEADER).read()
    assert "#define JFA_DECODE_SCRATCH_BYTES ((size_t)8 << 20)" in text and L.DECODE_SCRATCH_BYTES == 8 << 20


def test_input_checks_reject_host_errors_before_launch():
    """jfa_check_offsets / jfa_check_paged_cache: null pointers and bad sizes are
    refused on the host; the JFA_CHECK_* bits match the binding's constants."""
    L, lib = _lib()
    d = ctypes.c_void_p(256)
    assert lib.jfa_check_offsets(None, 4, 10, d, None) == L.JFA_ERR_INVALID_ARGUMENT
    assert lib.jfa_check_offsets(d, 4, 10, None, None) == L.JFA_ERR_INVALID_ARGUMENT
    assert lib.jfa_check_offsets(d, -1, 10, d, None) == L.JFA_ERR_INVALID_ARGUMENT
    assert lib.jfa_check_offsets(d, 4, -10, d, None) == L.JFA_ERR_INVALID_ARGUMENT
    p = L.DecodeParams(batch=2, num_heads_q=32, num_heads_kv=8, head_dim=128, page_size=16, num_pages=10,
                       max_pages_per_seq=5, num_splits=0, softmax_scale=0.0, q_len=1, causal=0)
    assert lib.jfa_check_paged_cache(None, d, d, d, None) == L.JFA_ERR_INVALID_ARGUMENT
    assert lib.jfa_check_paged_cache(ctypes.byref(p), None, d, d, None) == L.JFA_ERR_INVALID_ARGUMENT
    assert lib.jfa_check_paged_cache(ctypes.byref(p), d, d, None, None) == L.JFA_ERR_INVALID_ARGUMENT
    p.page_size = 0
    assert lib.jfa_check_paged_cache(ctypes.byref(p), d, d, d, None) == L.JFA_ERR_INVALID_ARGUMENT
    text = open(HEADER).read()
    for name in ("OFFSETS_START", "OFFSETS_ORDER", "OFFSETS_END", "SEQLEN_RANGE", "PAGE_RANGE"):
        m = re.search(rf"#define JFA_CHECK_{name} (\d+)", text)
        assert m and int(m.group(1)) == getattr(L, f"CHECK_{name}"), name
