"""GPU parity: jagged forward and backward through the C ABI against the fp64 oracle."""
import dataclasses
import math
import sys

import numpy as np
import pytest

import oracle
import workloads
from parity import check_grad, check_lse, check_o, dev, host, oracle_bcast_full, oracle_self_full

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


def _run_self(jfa, inp, scale=None, query_tile=0):
    q, k, v, do = (dev(x, torch) for x in (inp.q, inp.k, inp.v, inp.do))
    cq, ck = dev(inp.cu_q, torch), dev(inp.cu_k, torch)
    mq, mk = inp.max_len_q, inp.max_len_k
    o, lse = jfa.jfa_fwd(q, k, v, cq, ck, mq, mk, inp.causal, scale, query_tile=query_tile)
    dq, dk, dv = jfa.jfa_bwd(q, k, v, o, lse, do, cq, ck, mq, mk, inp.causal, scale, query_tile=query_tile)
    torch.cuda.synchronize()
    return host(o), host(lse), host(dq), host(dk), host(dv)


def _oracle_self(inp, scale=None, seqs=None):
    """Oracle outputs; with `seqs`, only for those sequences (a sample the oracle computes one by one)."""
    q, k, v, do = inp.q, inp.k, inp.v, inp.do
    if seqs is None:
        f = lambda x: x.astype(np.float64)
        o, lse = oracle.attention_forward(f(q), f(k), f(v), inp.cu_q, inp.cu_k, inp.causal, scale)
        dq, dk, dv = oracle.attention_backward(f(q), f(k), f(v), f(do), inp.cu_q, inp.cu_k, inp.causal, scale)
        return o, lse, dq, dk, dv
    out = {}
    for b in seqs:
        qs, qe, ks, ke = inp.cu_q[b], inp.cu_q[b + 1], inp.cu_k[b], inp.cu_k[b + 1]
        cq, ck = np.array([0, qe - qs]), np.array([0, ke - ks])
        args = [x.astype(np.float64) for x in (q[qs:qe], k[ks:ke], v[ks:ke])]
        o, lse = oracle.attention_forward(*args, cq, ck, inp.causal, scale)
        dq, dk, dv = oracle.attention_backward(*args, do[qs:qe].astype(np.float64), cq, ck, inp.causal, scale)
        out[b] = (o, lse, dq, dk, dv)
    return out


def _compare_full(got, ref):
    o, lse, dq, dk, dv = got
    ro, rl, rdq, rdk, rdv = ref
    eo = check_o(o, ro)
    el = check_lse(lse, rl)
    e = [check_grad(dq, rdq, "dQ"), check_grad(dk, rdk, "dK"), check_grad(dv, rdv, "dV")]
    _say(f"  O max-abs {eo:.2e}  LSE {el:.2e}  dQ/dK/dV rel-L2 {e[0]:.2e} {e[1]:.2e} {e[2]:.2e}")


def _compare_sampled(inp, got, ref):
    o, lse, dq, dk, dv = got
    for b, (ro, rl, rdq, rdk, rdv) in ref.items():
        qs, qe, ks, ke = inp.cu_q[b], inp.cu_q[b + 1], inp.cu_k[b], inp.cu_k[b + 1]
        check_o(o[qs:qe], ro, f"O[seq {b}]")
        check_lse(lse[:, qs:qe], rl, f"LSE[seq {b}]")
        check_grad(dq[qs:qe], rdq, f"dQ[seq {b}]")
        check_grad(dk[ks:ke], rdk, f"dK[seq {b}]")
        check_grad(dv[ks:ke], rdv, f"dV[seq {b}]")


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_tiny(jfa, seed):
    inp = workloads.tiny(seed)
    _say(f"tiny seed={seed} lengths={list(np.diff(inp.cu_q))}")
    _compare_full(_run_self(jfa, inp), _oracle_self(inp))


RAGGED = [1, 31, 32, 33, 63, 64, 65, 127, 128, 129, 200, 0, 257, 5]


@pytest.mark.parametrize("d", [64, 96, 128, 192, 256])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("hq,hkv", [(2, 2), (4, 2), (3, 1)])
def test_ragged(jfa, d, causal, hq, hkv):
    inp = workloads.jagged(100 + d, RAGGED, None, hq, hkv, d, causal)
    _say(f"ragged d={d} causal={causal} hq={hq} hkv={hkv}")
    _compare_full(_run_self(jfa, inp), _oracle_self(inp))


@pytest.mark.parametrize("d", [64, 128, 192, 256])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("hq,hkv", [(16, 2), (16, 1)])
def test_wide_gqa_groups(jfa, d, causal, hq, hkv):
    """GQA ratios 8 and 16: every dK/dV item sums its gradients over that many query heads
    (at d >= 192 in the AGPR accumulators of the hand-written MFMAs, across that many
    steps), and the forward / dQ items of one KV head run together."""
    inp = workloads.jagged(300 + d + hq // hkv, [1, 77, 300, 129, 0, 513], None, hq, hkv, d, causal)
    _say(f"wide GQA d={d} causal={causal} hq={hq} hkv={hkv}")
    _compare_full(_run_self(jfa, inp), _oracle_self(inp))


# Lengths around the 256-row query tiles of the 8-wave forward / dQ workgroups (d = 64, 128):
# every count of waves past the sequence end (0..7) occurs in some tile.
WIDE_TILE = [255, 256, 257, 288, 289, 320, 352, 384, 416, 448, 480, 511, 512, 513, 40]


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
def test_wide_query_tiles(jfa, d, causal):
    inp = workloads.jagged(300 + d, WIDE_TILE, None, 4, 2, d, causal)
    _say(f"wide tiles d={d} causal={causal}")
    _compare_full(_run_self(jfa, inp), _oracle_self(inp))


@pytest.mark.parametrize("qt", [128, 256])
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
def test_both_query_tiles(jfa, qt, d, causal):
    """Both item shapes of the forward / dQ (128 and 256 query rows; the automatic
    choice takes 128 for short sequences) on lengths around either tile size."""
    inp = workloads.jagged(500 + d + qt, RAGGED + WIDE_TILE, None, 4, 2, d, causal)
    _say(f"query tile {qt} d={d} causal={causal}")
    _compare_full(_run_self(jfa, inp, query_tile=qt), _oracle_self(inp))


def test_cross_lengths_bottom_right_causal(jfa):
    """Lq != Lk per sequence, causal aligned bottom-right (rows with no key get O=0, LSE=-inf)."""
    lq = [5, 130, 64, 1, 77, 300]
    lk = [9, 64, 200, 0, 77, 129]
    for causal in (False, True):
        inp = workloads.jagged(7, lq, lk, 4, 2, 128, causal)
        _say(f"cross lengths causal={causal}")
        _compare_full(_run_self(jfa, inp), _oracle_self(inp))


@pytest.mark.parametrize("causal", [False, True])
def test_many_sequences(jfa, causal):
    """More (sequence, KV head) groups than the scheduler keeps on chip (its per-group
    arrays then live in the workspace), many of them empty or one token long."""
    rng = np.random.default_rng(31)
    lengths = rng.integers(0, 40, 1600).tolist()
    inp = workloads.jagged(11, lengths, None, 8, 4, 64, causal)
    _say(f"many sequences: batch {len(lengths)}, groups {len(lengths) * 4}, causal={causal}")
    _compare_full(_run_self(jfa, inp), _oracle_self(inp))


def test_explicit_scale(jfa):
    inp = workloads.jagged(8, [70, 129], None, 2, 2, 64, False)
    _compare_full(_run_self(jfa, inp, 0.3), _oracle_self(inp, 0.3))


@pytest.mark.parametrize("scale", [4.0, 1e-3])
@pytest.mark.parametrize("causal", [False, True])
def test_extreme_scales(jfa, scale, causal):
    """Scale 4 at d = 128: scores spread over hundreds of log2 units, so rows are nearly one-hot
    and the forward's running max moves many times; scale 1e-3: nearly flat rows."""
    inp = workloads.jagged(60, [700, 33, 257, 1], None, 4, 2, 128, causal)
    _say(f"extreme scale {scale} causal={causal}")
    _compare_full(_run_self(jfa, inp, scale), _oracle_self(inp, scale))


def test_outputs_overwritten(jfa):
    """Outputs pre-filled with NaN must be fully overwritten (catches unwritten rows)."""
    inp = workloads.jagged(9, [3, 130, 64, 0, 1], None, 4, 2, 64, True)
    q, k, v, do = (dev(x, torch) for x in (inp.q, inp.k, inp.v, inp.do))
    cq, ck = dev(inp.cu_q, torch), dev(inp.cu_k, torch)
    o = torch.full_like(q, float("nan"))
    lse = torch.full((4, q.shape[0]), float("nan"), device="cuda")
    jfa.jfa_fwd(q, k, v, cq, ck, 130, 130, True, out=o, lse=lse)
    dq, dk, dv = (torch.full_like(x, float("nan")) for x in (q, k, v))
    jfa.jfa_bwd(q, k, v, o, lse, do, cq, ck, 130, 130, True, dq=dq, dk=dk, dv=dv)
    torch.cuda.synchronize()
    _compare_full((host(o), host(lse), host(dq), host(dk), host(dv)), _oracle_self(inp))


# ----------------------------------------------------------------------------- guarded outputs
# Every output (and the workspace) lives in the middle of a larger buffer whose
# guard bands before and after must come back untouched: NaN for the outputs,
# a byte pattern for the workspace.  The outputs themselves start as NaN, so a
# row the kernels never write fails the comparison.
GUARD_ELEMS = 1 << 16
GUARD_BYTES = 1 << 16
WS_PATTERN = 0xA5


class Guarded:
    def __init__(self, shape, dtype, fill=float("nan")):
        n = int(np.prod(shape))
        g = GUARD_BYTES if dtype == torch.uint8 else GUARD_ELEMS
        self.full = torch.full((n + 2 * g,), fill, dtype=dtype, device="cuda")
        self.lo, self.hi = g, g + n
        self.fill = fill
        self.t = self.full[self.lo:self.hi].view(shape)

    def intact(self):
        outside = torch.cat([self.full[:self.lo], self.full[self.hi:]])
        if self.full.dtype == torch.uint8:
            return bool((outside == self.fill).all())
        return bool(torch.isnan(outside.float()).all())


def _run_guarded(jfa, inp, bcast=False):
    """Forward + backward into guarded NaN-filled outputs and guarded workspaces."""
    q, k, v, do = (dev(x, torch) for x in (inp.q, inp.k, inp.v, inp.do))
    ck = dev(inp.cu_k, torch)
    cq = None if bcast else dev(inp.cu_q, torch)
    causal = False if bcast else inp.causal
    mq = inp.q.shape[0] if bcast else inp.max_len_q
    nb = len(inp.cu_k) - 1
    o_shape = (nb,) + tuple(q.shape) if bcast else tuple(q.shape)
    lse_shape = (nb, q.shape[1], q.shape[0]) if bcast else (q.shape[1], q.shape[0])
    o, lse = Guarded(o_shape, torch.bfloat16), Guarded(lse_shape, torch.float32)
    wsf = Guarded((jfa.jfa_fwd_workspace_size(q, k, ck, mq, inp.max_len_k, causal, bcast),), torch.uint8, WS_PATTERN)
    wsb = Guarded((jfa.jfa_bwd_workspace_size(q, k, ck, mq, inp.max_len_k, causal, bcast),), torch.uint8, WS_PATTERN)
    jfa.jfa_fwd(q, k, v, cq, ck, mq, inp.max_len_k, causal, broadcast_q=bcast, out=o.t, lse=lse.t, workspace=wsf.t)
    dq, dk, dv = Guarded(tuple(q.shape), torch.bfloat16), Guarded(tuple(k.shape), torch.bfloat16), \
        Guarded(tuple(v.shape), torch.bfloat16)
    jfa.jfa_bwd(q, k, v, o.t, lse.t, do, cq, ck, mq, inp.max_len_k, causal, broadcast_q=bcast,
                dq=dq.t, dk=dk.t, dv=dv.t, workspace=wsb.t)
    torch.cuda.synchronize()
    for name, g in (("O", o), ("LSE", lse), ("dQ", dq), ("dK", dk), ("dV", dv), ("fwd workspace", wsf),
                    ("bwd workspace", wsb)):
        assert g.intact(), f"{name}: guard band overwritten"
    return host(o.t), host(lse.t), host(dq.t), host(dk.t), host(dv.t)


@pytest.mark.parametrize("s", [0.9, 0.5, 0.1])
def test_gem_full_size(jfa, s):
    """GEM config at full size (256 sequences, 8 heads, d = 128): O, LSE, dQ, dK and dV
    of every sequence against the oracle, outputs guarded and NaN-prefilled."""
    inp = workloads.gem(0, s)
    _say(f"gem s={s} T={inp.q.shape[0]}")
    got = _run_guarded(jfa, inp)
    _compare_full(got, oracle_self_full(oracle, inp))


@pytest.mark.parametrize("d", [128, 96])
def test_dense_causal_full_size_sampled(jfa, d):
    """4 x 8192 causal, 32 heads, at full size; the oracle on one head of every
    sequence (and two more of sequence 0), whole rows and keys of each."""
    inp = workloads.dense_causal(0, head_dim=d)
    _say(f"dense causal d={d}")
    got = _run_self(jfa, inp)
    L = 8192
    picks = [(0, 0), (0, 17), (0, 31), (1, 9), (2, 22), (3, 5)]

    def one(bh):
        b, h = bh
        sl = slice(b * L, (b + 1) * L)
        args = [x[sl, h:h + 1].astype(np.float64) for x in (inp.q, inp.k, inp.v)]
        cu = np.array([0, L])
        ro, rl = oracle.attention_forward(*args, cu, cu, True)
        rdq, rdk, rdv = oracle.attention_backward(*args, inp.do[sl, h:h + 1].astype(np.float64), cu, cu, True)
        return ro, rl, rdq, rdk, rdv

    from parity import _pool_map
    for (b, h), (ro, rl, rdq, rdk, rdv) in zip(picks, _pool_map(one, picks)):
        sl = slice(b * L, (b + 1) * L)
        check_o(got[0][sl, h:h + 1], ro, f"O[seq {b} h{h}]")
        check_lse(got[1][h:h + 1, sl], rl, f"LSE[seq {b} h{h}]")
        check_grad(got[2][sl, h:h + 1], rdq, f"dQ[seq {b} h{h}]")
        check_grad(got[3][sl, h:h + 1], rdk, f"dK[seq {b} h{h}]")
        check_grad(got[4][sl, h:h + 1], rdv, f"dV[seq {b} h{h}]")
        _say(f"  seq {b} head {h} ok")


def _run_bcast(jfa, inp, query_tile=0):
    q, k, v, do = (dev(x, torch) for x in (inp.q, inp.k, inp.v, inp.do))
    ck = dev(inp.cu_k, torch)
    nq = inp.q.shape[0]
    o, lse = jfa.jfa_fwd(q, k, v, None, ck, nq, inp.max_len_k, False, None, broadcast_q=True, query_tile=query_tile)
    dq, dk, dv = jfa.jfa_bwd(q, k, v, o, lse, do, None, ck, nq, inp.max_len_k, False, None, broadcast_q=True,
                             query_tile=query_tile)
    torch.cuda.synchronize()
    return host(o), host(lse), host(dq), host(dk), host(dv)


def _oracle_bcast(inp):
    f = lambda x: x.astype(np.float64)
    o, lse = oracle.broadcast_q_forward(f(inp.q), f(inp.k), f(inp.v), inp.cu_k)
    dq, dk, dv = oracle.broadcast_q_backward(f(inp.q), f(inp.k), f(inp.v), f(inp.do), inp.cu_k)
    return o, lse, dq, dk, dv


@pytest.mark.parametrize("nq,lengths,hq,hkv", [
    (37, [5, 0, 64, 129, 1], 2, 2),
    (256, [300, 17, 0, 128, 64, 1000, 3], 4, 4),
    (130, [70, 70, 200], 4, 2),
    (300, [33, 0, 257, 512], 2, 1),   # a second 256-row query tile with 44 rows
])
def test_broadcast_q(jfa, nq, lengths, hq, hkv):
    inp = workloads.broadcast(3, nq, lengths, hq, hkv, 128)
    _say(f"broadcast nq={nq} lengths={lengths}")
    _compare_full(_run_bcast(jfa, inp), _oracle_bcast(inp))


@pytest.mark.parametrize("qt", [128, 256])
@pytest.mark.parametrize("d", [64, 128])
def test_broadcast_q_both_query_tiles(jfa, qt, d):
    """Broadcast-Q with either item shape: Nq = 300 is two 256-row tiles or three 128-row ones."""
    inp = workloads.broadcast(9 + d, 300, [33, 0, 257, 512, 129, 1], 4, 2, d)
    _say(f"broadcast query tile {qt} d={d}")
    _compare_full(_run_bcast(jfa, inp, query_tile=qt), _oracle_bcast(inp))


@pytest.mark.parametrize("d", [64, 96, 128])
def test_broadcast_q_chunks_split_items(jfa, d):
    """Broadcast-Q dQ cuts its item chunks at equal cost, at key-tile granularity, so a
    long item's tiles are shared by two chunks: 40 items of 0-900 keys (ragged tails,
    empty items), Nq = 100, at each dQ tile shape (d = 96: one 64-key stage)."""
    rng = np.random.default_rng(40 + d)
    lengths = rng.integers(0, 901, 40).tolist()
    lengths[3] = 0
    lengths[17] = 900
    inp = workloads.broadcast(50 + d, 100, lengths, 4, 2, d)
    _say(f"broadcast split chunks d={d}")
    _compare_full(_run_bcast(jfa, inp), _oracle_bcast(inp))


@pytest.mark.parametrize("s", [0.9, 0.5, 0.1])
def test_broadcast_q_config(jfa, s):
    """Broadcast-Q config (Nq = 256, 512 items, 4 heads, d = 128) at full size, whole
    tensors, outputs guarded and NaN-prefilled."""
    inp = workloads.broadcast_q(0, s)
    _say(f"broadcast config s={s} Tk={inp.k.shape[0]}")
    _compare_full(_run_guarded(jfa, inp, bcast=True), oracle_bcast_full(oracle, inp))


def test_broadcast_q_without_queries(jfa):
    """Nq = 0: no key is seen by a query, so dK = dV = 0 (outputs start as NaN)."""
    inp = workloads.broadcast(8, 1, [5, 0, 130], 4, 2, 128)
    k, v = dev(inp.k, torch), dev(inp.v, torch)
    q = torch.empty((0, 4, 128), dtype=torch.bfloat16, device="cuda")
    ck = dev(inp.cu_k, torch)
    o = torch.empty((3, 0, 4, 128), dtype=torch.bfloat16, device="cuda")
    lse = torch.empty((3, 4, 0), dtype=torch.float32, device="cuda")
    dk, dv = torch.full_like(k, float("nan")), torch.full_like(v, float("nan"))
    jfa.jfa_bwd(q, k, v, o, lse, o, None, ck, 0, 130, False, broadcast_q=True, dk=dk, dv=dv)
    torch.cuda.synchronize()
    assert (dk == 0).all() and (dv == 0).all()


def test_broadcast_dq_is_sum_of_items(jfa):
    """dQ of a broadcast batch equals the sum of the single-item runs (GPU against GPU)."""
    inp = workloads.broadcast(4, 64, [40, 130, 7], 2, 2, 64)
    full = _run_bcast(jfa, inp)
    acc = np.zeros_like(full[2])
    for b in range(3):
        ks, ke = inp.cu_k[b], inp.cu_k[b + 1]
        one = workloads.BroadcastInputs(inp.q, inp.k[ks:ke], inp.v[ks:ke], inp.do[b:b + 1],
                                        np.array([0, ke - ks], np.int32))
        acc += _run_bcast(jfa, one)[2]
    assert np.abs(full[2] - acc).max() <= 2e-2 * max(1.0, np.abs(acc).max())


def test_repeatability(jfa):
    """Ten runs give bitwise-identical O, LSE, dQ, dK and dV: no atomics anywhere,
    and the work-list order does not change any reduction order."""
    inp = workloads.jagged(12, [300, 129, 64], None, 4, 4, 128, False)
    ref = _oracle_self(inp)
    first = None
    for _ in range(10):
        got = _run_self(jfa, inp)
        check_grad(got[2], ref[2], "dQ")
        if first is None:
            first = got
        else:
            for x, y in zip(got, first):
                np.testing.assert_array_equal(x, y)


def test_broadcast_repeatability(jfa):
    """Broadcast-Q: dQ (summed over the items through per-chunk partials added in a
    fixed order) and every other output are bitwise identical across runs."""
    inp = workloads.broadcast(5, 256, [300, 17, 0, 128, 64, 1000, 3, 500, 200, 90], 4, 4, 128)
    first = _run_bcast(jfa, inp)
    for _ in range(5):
        got = _run_bcast(jfa, inp)
        for x, y in zip(got, first):
            np.testing.assert_array_equal(x, y)

@pytest.mark.parametrize("d", [192, 256])
def test_broadcast_q_large_head_dims(jfa, d):
    """Broadcast-Q at d = 192 / 256 (d = 256: dK/dV split into two head-dim slices)."""
    inp = workloads.broadcast(6, 130, [70, 0, 200, 129, 1], 4, 2, d)
    _say(f"broadcast d={d}")
    _compare_full(_run_bcast(jfa, inp), _oracle_bcast(inp))


@pytest.mark.parametrize("d", [192, 256])
def test_large_head_dim_long_causal_sampled(jfa, d):
    """Long causal sequences (2048 and 2500 + ragged) at d = 192 / 256, 4 heads over 2 KV
    heads; oracle on the two long sequences, every head."""
    inp = workloads.jagged(70 + d, [2048, 1, 2500, 77], None, 4, 2, d, True)
    _say(f"long causal d={d}")
    got = _run_self(jfa, inp)
    _compare_sampled(inp, got, _oracle_self(inp, seqs=[0, 2]))


@pytest.mark.parametrize("d", [192, 256])
def test_large_head_dim_repeatability(jfa, d):
    """d = 192 / 256 (at 256 the sliced dK/dV): every output is bitwise identical across runs."""
    inp = workloads.jagged(13, [300, 129, 64], None, 4, 2, d, True)
    first = _run_self(jfa, inp)
    for _ in range(4):
        got = _run_self(jfa, inp)
        for x, y in zip(got, first):
            np.testing.assert_array_equal(x, y)


@pytest.mark.parametrize("causal", [False, True])
def test_twenty_thousand_short_sequences(jfa, causal):
    """80 000 (sequence, KV head) groups of 0-12 tokens: the work lists far exceed
    the scheduler's on-chip arrays; oracle on a sample of sequences."""
    rng = np.random.default_rng(41)
    lengths = rng.integers(0, 13, 20000).tolist()
    inp = workloads.jagged(12, lengths, None, 4, 4, 64, causal)
    _say(f"20000 short sequences, causal={causal}, tokens {sum(lengths)}")
    got = _run_self(jfa, inp)
    seqs = sorted(set(rng.integers(0, 20000, 40).tolist() + [0, 19999]))
    _compare_sampled(inp, got, _oracle_self(inp, seqs=seqs))


def test_one_long_causal_sequence(jfa):
    """One 32768-token causal sequence (2 query heads on 1 KV head, d = 64).  Rows of a
    causal sequence depend only on their own keys, so O, LSE and dQ of sampled row
    blocks come from the oracle on (those rows, keys up to the block's end); dK and dV
    are checked through the softmax-Jacobian invariants (sum dK = 0, sum dV = sum dO)."""
    L = 32768
    inp = workloads.jagged(13, [L], None, 2, 1, 64, True)
    got = _run_self(jfa, inp)
    o, lse, dq, dk, dv = got
    f = lambda x: x.astype(np.float64)
    for i0 in (0, 16000, L - 64):
        i1 = i0 + 64
        cq, ck = np.array([0, 64]), np.array([0, i1])
        ro, rl = oracle.attention_forward(f(inp.q[i0:i1]), f(inp.k[:i1]), f(inp.v[:i1]), cq, ck, True)
        rdq, _, _ = oracle.attention_backward(f(inp.q[i0:i1]), f(inp.k[:i1]), f(inp.v[:i1]), f(inp.do[i0:i1]),
                                              cq, ck, True)
        check_o(o[i0:i1], ro, f"O rows {i0}..")
        check_lse(lse[:, i0:i1], rl, f"LSE rows {i0}..")
        check_grad(dq[i0:i1], rdq, f"dQ rows {i0}..")
        _say(f"  rows {i0}..{i1} ok")
    # dK sums to zero over the keys; dV sums to the group's dO summed over the queries
    dk_sum = dk.sum(axis=0)
    dv_sum, do_sum = dv.sum(axis=0), inp.do.astype(np.float64).sum(axis=(0, 1))[None, :]
    scale = np.abs(dk).sum(axis=0).max()
    assert np.abs(dk_sum).max() <= 2e-3 * scale, (np.abs(dk_sum).max(), scale)
    assert np.abs(dv_sum - do_sum).max() <= 2e-3 * np.abs(dv).sum(axis=0).max()


# bf16 values beyond the fp16 range (|v| >= 65520), placed in a few V rows
LARGE_V = [65536.0, -98304.0, 1048576.0, -16777216.0, 2.0 ** 27]


def _plant_large_v(v, rng, n):
    """Put LARGE_V values at n random (row, head, column) positions of v (float32 array, bf16 values)."""
    v = v.copy()
    for i in range(n):
        r, h, c = rng.integers(0, v.shape[0]), rng.integers(0, v.shape[1]), rng.integers(0, v.shape[2])
        v[r, h, c] = LARGE_V[i % len(LARGE_V)]
    return v


def _check_large(got, ref, mag, what):
    """|error| <= 1e-2 + half a bf16 ulp of O + 2^-7 (P |V|): the output's own bf16
    rounding, plus the rounding of P (bf16, 8 significant bits, in the recomputation such
    inputs take: 2^-8 per term) and the normalisation by the unrounded sum (another
    2^-8), relative to the magnitudes summed, P |V|, not to O."""
    from parity import half_ulp_bf16
    err = np.abs(got - ref)
    bound = 1e-2 + half_ulp_bf16(ref) + 2.0 ** -7 * mag
    assert np.isfinite(got).all(), f"{what}: non-finite values"
    assert (err <= bound).all(), f"{what}: max excess {(err - bound).max():.3e}"


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("d", [64, 128, 256])
def test_forward_v_beyond_fp16_range(jfa, causal, d):
    """V entries of magnitude 2^16 .. 2^27 (beyond fp16) in several items: in fp16 those V
    values become infinite, so the items are computed again with P V in bf16."""
    inp = workloads.jagged(77 + d, [5, 130, 64, 200, 1], None, 4, 2, d, causal)
    rng = np.random.default_rng(5)
    inp = dataclasses.replace(inp, v=_plant_large_v(inp.v, rng, 12))
    q, k, v = (dev(x, torch) for x in (inp.q, inp.k, inp.v))
    cq, ck = dev(inp.cu_q, torch), dev(inp.cu_k, torch)
    o, lse = jfa.jfa_fwd(q, k, v, cq, ck, inp.max_len_q, inp.max_len_k, causal)
    torch.cuda.synchronize()
    f = lambda x: x.astype(np.float64)
    ro, rl = oracle.attention_forward(f(inp.q), f(inp.k), f(inp.v), inp.cu_q, inp.cu_k, causal)
    mag, _ = oracle.attention_forward(f(inp.q), f(inp.k), np.abs(f(inp.v)), inp.cu_q, inp.cu_k, causal)
    _check_large(host(o), ro, mag, "O")
    check_lse(host(lse), rl)
