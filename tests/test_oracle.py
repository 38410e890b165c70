"""Pins for the fp64 oracle: each check comes from something other than the oracle itself.

* hand-derived closed-form examples (tests/golden/hand_examples.json);
* closed forms: a single key gives O = V and LSE = S; identical keys give O = mean(V);
* brute force: scalar Python loops with math.fsum on tiny inputs;
* an independent library routine: torch's CPU float64 scaled_dot_product_attention and
  its autograd gradients, per sequence;
* central finite differences of f = sum(O * dO) for every input, including GQA,
  causal and broadcast-Q;
* invariants of the softmax Jacobian: sum_j dK_j = 0 and sum_j dV_j = sum_i dO_i;
* symmetries: adding a constant vector to every key, permuting keys with values.
"""
import json
import math
import os

import numpy as np
import pytest

import oracle
import workloads

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "hand_examples.json")


def _ev(x):
    return np.array([[_ev1(e) for e in row] for row in x]) if isinstance(x[0], list) else np.array([_ev1(e) for e in x])


def _ev1(s):
    if s == "-inf":
        return -math.inf
    return float(eval(s, {"__builtins__": {}}, {"log": math.log}))


def _cases():
    with open(GOLDEN) as f:
        return json.load(f)["cases"]


@pytest.mark.parametrize("case", _cases(), ids=lambda c: c["name"])
def test_golden_hand_examples(case):
    q, k, v, do = (_ev(case[n])[:, None, :] for n in ("q", "k", "v", "do"))
    cq = np.array([0, q.shape[0]])
    ck = np.array([0, k.shape[0]])
    scale = case["scale"]
    o, lse = oracle.attention_forward(q, k, v, cq, ck, case["causal"], scale)
    np.testing.assert_allclose(o[:, 0], _ev(case["o"]), atol=1e-14)
    exp_lse = _ev(case["lse"])
    assert np.array_equal(np.isinf(lse[0]), np.isinf(exp_lse))
    fin = np.isfinite(exp_lse)
    np.testing.assert_allclose(lse[0][fin], exp_lse[fin], atol=1e-14)
    dq, dk, dv = oracle.attention_backward(q, k, v, do, cq, ck, case["causal"], scale)
    np.testing.assert_allclose(dq[:, 0], _ev(case["dq"]), atol=1e-14)
    np.testing.assert_allclose(dk[:, 0], _ev(case["dk"]), atol=1e-14)
    np.testing.assert_allclose(dv[:, 0], _ev(case["dv"]), atol=1e-14)


def _rand(rng, *shape):
    return rng.standard_normal(shape)


def test_single_key_gives_value_row():
    rng = np.random.default_rng(1)
    q, k, v = _rand(rng, 5, 2, 16), _rand(rng, 1, 2, 16), _rand(rng, 1, 2, 16)
    o, lse = oracle.attention_forward(q, k, v, [0, 5], [0, 1])
    for h in range(2):
        np.testing.assert_array_equal(o[:, h], np.broadcast_to(v[0, h], (5, 16)))
        np.testing.assert_allclose(lse[h], (q[:, h] @ k[0, h]) / 4.0, rtol=0, atol=1e-14)


def test_identical_keys_give_mean_value():
    rng = np.random.default_rng(2)
    L = 7
    q = _rand(rng, 3, 1, 8)
    k = np.repeat(_rand(rng, 1, 1, 8), L, axis=0)
    v = _rand(rng, L, 1, 8)
    o, lse = oracle.attention_forward(q, k, v, [0, 3], [0, L])
    np.testing.assert_allclose(o[:, 0], np.broadcast_to(v[:, 0].mean(0), (3, 8)), atol=1e-14)
    s = q[:, 0] @ k[0, 0] / math.sqrt(8)
    np.testing.assert_allclose(lse[0], s + math.log(L), atol=1e-13)


def test_rows_of_p_sum_to_one():
    # with one-hot values, row i of O is row i of P
    rng = np.random.default_rng(3)
    L, d = 12, 16
    q, k = _rand(rng, 9, 1, d), _rand(rng, L, 1, d)
    v = np.eye(L, d)[:, None, :]
    for causal in (False, True):
        o, _ = oracle.attention_forward(q, k, v, [0, 9], [0, L], causal)
        p = o[:, 0, :L]
        assert (p >= 0).all()
        np.testing.assert_allclose(p.sum(1), 1.0, atol=1e-12)
        if causal:   # bottom-right: query i sees keys j <= i + (L - 9)
            for i in range(9):
                assert np.all(p[i, i + L - 9 + 1:] == 0)


def _brute_force(q, k, v, scale, causal):
    """Scalar loops over the definition, sums with math.fsum."""
    lq, lk = len(q), len(k)
    o, lse = [], []
    for i in range(lq):
        keys = [j for j in range(lk) if (not causal) or j <= i + (lk - lq)]
        if not keys:
            o.append([0.0] * len(v[0]) if lk else [0.0] * len(q[0]))
            lse.append(-math.inf)
            continue
        s = {j: scale * math.fsum(q[i][t] * k[j][t] for t in range(len(q[i]))) for j in keys}
        mx = max(s.values())
        lsum = math.fsum(math.exp(s[j] - mx) for j in keys)
        l_i = mx + math.log(lsum)
        lse.append(l_i)
        o.append([math.fsum(math.exp(s[j] - l_i) * v[j][t] for j in keys) for t in range(len(v[0]))])
    return np.array(o), np.array(lse)


@pytest.mark.parametrize("lq,lk,causal", [(4, 6, False), (5, 5, True), (6, 3, True), (3, 7, True), (2, 1, False)])
def test_brute_force_forward(lq, lk, causal):
    rng = np.random.default_rng(4 + lq * 10 + lk)
    d = 5
    q, k, v = _rand(rng, lq, 1, d) * 2, _rand(rng, lk, 1, d) * 2, _rand(rng, lk, 1, d)
    o, lse = oracle.attention_forward(q, k, v, [0, lq], [0, lk], causal, 0.7)
    bo, bl = _brute_force(q[:, 0].tolist(), k[:, 0].tolist(), v[:, 0].tolist(), 0.7, causal)
    np.testing.assert_allclose(o[:, 0], bo, atol=1e-13)
    np.testing.assert_array_equal(np.isinf(lse[0]), np.isinf(bl))
    np.testing.assert_allclose(lse[0][np.isfinite(bl)], bl[np.isfinite(bl)], atol=1e-13)


# ----------------------------------------------------------------- torch SDPA (independent routine)
torch = pytest.importorskip("torch")


def _sdpa_per_sequence(q, k, v, do, cq, ck, causal, r):
    """torch CPU float64 SDPA + autograd, one sequence at a time, heads repeated for GQA."""
    import torch.nn.functional as F
    tq, hq, d = q.shape
    outs, dqs = np.zeros_like(q), np.zeros_like(q)
    dks, dvs = np.zeros_like(k), np.zeros_like(v)
    for b in range(len(cq) - 1):
        qs, qe, ks, ke = cq[b], cq[b + 1], ck[b], ck[b + 1]
        if qe == qs or ke == ks:
            continue
        tq_ = torch.tensor(q[qs:qe].transpose(1, 0, 2), dtype=torch.float64, requires_grad=True)
        tk_ = torch.tensor(k[ks:ke].transpose(1, 0, 2), dtype=torch.float64, requires_grad=True)
        tv_ = torch.tensor(v[ks:ke].transpose(1, 0, 2), dtype=torch.float64, requires_grad=True)
        kr = tk_.repeat_interleave(r, dim=0)
        vr = tv_.repeat_interleave(r, dim=0)
        o = F.scaled_dot_product_attention(tq_[None], kr[None], vr[None], is_causal=causal)[0]
        g = torch.tensor(do[qs:qe].transpose(1, 0, 2), dtype=torch.float64)
        o.backward(g)
        outs[qs:qe] = o.detach().numpy().transpose(1, 0, 2)
        dqs[qs:qe] = tq_.grad.numpy().transpose(1, 0, 2)
        dks[ks:ke] = tk_.grad.numpy().transpose(1, 0, 2)
        dvs[ks:ke] = tv_.grad.numpy().transpose(1, 0, 2)
    return outs, dqs, dks, dvs


@pytest.mark.parametrize("causal,hq,hkv", [(False, 2, 2), (True, 2, 2), (False, 4, 2), (True, 6, 2)])
def test_matches_torch_sdpa_fp64(causal, hq, hkv):
    lengths = [7, 1, 19, 33, 0, 12]
    inp = workloads.jagged(11, lengths, None, hq, hkv, 16, causal)
    q, k, v, do = (x.astype(np.float64) for x in (inp.q, inp.k, inp.v, inp.do))
    o, lse = oracle.attention_forward(q, k, v, inp.cu_q, inp.cu_k, causal)
    dq, dk, dv = oracle.attention_backward(q, k, v, do, inp.cu_q, inp.cu_k, causal)
    ro, rdq, rdk, rdv = _sdpa_per_sequence(q, k, v, do, inp.cu_q, inp.cu_k, causal, hq // hkv)
    for a, b in ((o, ro), (dq, rdq), (dk, rdk), (dv, rdv)):
        np.testing.assert_allclose(a, b, atol=1e-12, rtol=1e-10)


def test_decode_matches_torch_sdpa():
    inp = workloads.decode(5, [9, 1, 40, 17], heads_q=8, heads_kv=2, head_dim=16, page_size=4)
    q, k, v = (x.astype(np.float64) for x in (inp.q, inp.k, inp.v))
    o, lse = oracle.decode_forward(q, k, v, inp.cu_k)
    cq = np.arange(len(inp.seqlens_k) + 1)
    ro, _, _, _ = _sdpa_per_sequence(q, k, v, np.zeros_like(q), cq, inp.cu_k, False, 4)
    np.testing.assert_allclose(o, ro, atol=1e-12)
    assert lse.shape == (4, 8)


# ----------------------------------------------------------------- finite differences
def _fd_check(f, params, grads, eps=1e-6, rtol=1e-6):
    for name, x in params.items():
        g = grads[name]
        num = np.zeros_like(x)
        it = np.nditer(x, flags=["multi_index"])
        for _ in it:
            idx = it.multi_index
            old = x[idx]
            x[idx] = old + eps
            fp = f()
            x[idx] = old - eps
            fm = f()
            x[idx] = old
            num[idx] = (fp - fm) / (2 * eps)
        err = np.linalg.norm(num - g) / max(np.linalg.norm(num), 1e-30)
        assert err <= rtol, f"{name}: rel err {err:.2e}"


@pytest.mark.parametrize("causal,hq,hkv,lq,lk", [
    (False, 2, 2, [3, 5], [4, 2]),
    (True, 2, 1, [4, 6], [4, 6]),        # GQA r=2, causal
    (True, 2, 2, [5, 2], [3, 4]),        # causal with Lq != Lk (bottom-right)
    (False, 4, 2, [1, 6], [6, 1]),
])
def test_finite_differences_jagged(causal, hq, hkv, lq, lk):
    rng = np.random.default_rng(21)
    d = 6
    cq, ck = workloads.offsets(lq), workloads.offsets(lk)
    q, k, v = _rand(rng, cq[-1], hq, d), _rand(rng, ck[-1], hkv, d), _rand(rng, ck[-1], hkv, d)
    do = _rand(rng, cq[-1], hq, d)
    f = lambda: float((oracle.attention_forward(q, k, v, cq, ck, causal, 0.6)[0] * do).sum())
    dq, dk, dv = oracle.attention_backward(q, k, v, do, cq, ck, causal, 0.6)
    _fd_check(f, {"q": q, "k": k, "v": v}, {"q": dq, "k": dk, "v": dv})


def test_finite_differences_broadcast_q():
    rng = np.random.default_rng(22)
    nq, hq, hkv, d = 4, 2, 1, 5
    ck = workloads.offsets([3, 1, 5])
    q, k, v = _rand(rng, nq, hq, d), _rand(rng, ck[-1], hkv, d), _rand(rng, ck[-1], hkv, d)
    do = _rand(rng, 3, nq, hq, d)
    f = lambda: float((oracle.broadcast_q_forward(q, k, v, ck)[0] * do).sum())
    dq, dk, dv = oracle.broadcast_q_backward(q, k, v, do, ck)
    _fd_check(f, {"q": q, "k": k, "v": v}, {"q": dq, "k": dk, "v": dv})


# ----------------------------------------------------------------- head-dim-sliced backward
def _sliced_backward(q, k, v, o, lse, do, causal, hc, bq=16, bk=8):
    """The chunked backward of "Cutting edge isn't plug-and-play: customising FlashAttention-4
    on B300" (Phase 2 pseudocode and buffer list), for one sequence and head: per
    (Q tile, KV tile) and output slice c of width hc, S and dP are summed over every
    slice of the head dimension, P is rebuilt from the saved LSE, and only dQ[:, c],
    dK[:, c], dV[:, c] are written."""
    lq, d = q.shape
    lk = k.shape[0]
    scale = 1.0 / math.sqrt(d)
    delta = (do * o).sum(1)
    dq, dk, dv = np.zeros_like(q), np.zeros_like(k), np.zeros_like(v)
    for c0 in range(0, d, hc):
        c = slice(c0, c0 + hc)
        for i0 in range(0, lq, bq):
            i = slice(i0, min(i0 + bq, lq))
            for j0 in range(0, lk, bk):
                j = slice(j0, min(j0 + bk, lk))
                s_t = np.zeros((i.stop - i.start, j.stop - j.start))
                dp_t = np.zeros_like(s_t)
                for h0 in range(0, d, hc):
                    h = slice(h0, h0 + hc)
                    s_t += q[i, h] @ k[j, h].T
                    dp_t += do[i, h] @ v[j, h].T
                p_t = np.exp(s_t * scale - lse[i, None])
                if causal:
                    rows = np.arange(i.start, i.stop)[:, None] + (lk - lq)
                    p_t = np.where(np.arange(j.start, j.stop)[None, :] <= rows, p_t, 0.0)
                ds_t = p_t * (dp_t - delta[i, None])
                dq[i, c] += scale * ds_t @ k[j, c]
                dk[j, c] += scale * ds_t.T @ q[i, c]
                dv[j, c] += p_t.T @ do[i, c]
    return dq, dk, dv


@pytest.mark.parametrize("hc", [128, 64])
@pytest.mark.parametrize("causal", [False, True])
def test_head_dim_sliced_backward_equals_oracle(hc, causal):
    """At d = 256 the slice-by-slice backward (S and dP summed over all slices, each
    slice writing its own dQ/dK/dV columns) equals the oracle's unsliced gradients."""
    rng = np.random.default_rng(40)
    lq, lk, d = 37, 29, 256
    q, k, v, do = (rng.standard_normal((n, 1, d)) for n in (lq, lk, lk, lq))
    cq, ck = np.array([0, lq]), np.array([0, lk])
    o, lse = oracle.attention_forward(q, k, v, cq, ck, causal)
    dq, dk, dv = oracle.attention_backward(q, k, v, do, cq, ck, causal)
    got = _sliced_backward(q[:, 0], k[:, 0], v[:, 0], o[:, 0], lse[0], do[:, 0], causal, hc)
    for g, r in zip(got, (dq[:, 0], dk[:, 0], dv[:, 0])):
        np.testing.assert_allclose(g, r, rtol=1e-10, atol=1e-12)


# ----------------------------------------------------------------- invariants and symmetries
@pytest.mark.parametrize("causal", [False, True])
def test_softmax_jacobian_invariants(causal):
    inp = workloads.jagged(31, [9, 20, 1, 14], None, 4, 2, 16, causal)
    q, k, v, do = (x.astype(np.float64) for x in (inp.q, inp.k, inp.v, inp.do))
    dq, dk, dv = oracle.attention_backward(q, k, v, do, inp.cu_q, inp.cu_k, causal)
    for b in range(inp.batch):
        qs, qe, ks, ke = inp.cu_q[b], inp.cu_q[b + 1], inp.cu_k[b], inp.cu_k[b + 1]
        np.testing.assert_allclose(dk[ks:ke].sum(0), 0.0, atol=1e-11)
        do_sum = do[qs:qe].reshape(qe - qs, 2, 2, 16).sum(axis=(0, 2))   # summed over the group
        np.testing.assert_allclose(dv[ks:ke].sum(0), do_sum, atol=1e-11)


def test_key_shift_and_permutation():
    rng = np.random.default_rng(41)
    q, k, v = _rand(rng, 6, 1, 8), _rand(rng, 10, 1, 8), _rand(rng, 10, 1, 8)
    c = _rand(rng, 8)
    o, lse = oracle.attention_forward(q, k, v, [0, 6], [0, 10])
    o2, lse2 = oracle.attention_forward(q, k + c, v, [0, 6], [0, 10])
    np.testing.assert_allclose(o2, o, atol=1e-13)
    np.testing.assert_allclose(lse2[0], lse[0] + (q[:, 0] @ c) / math.sqrt(8), atol=1e-12)
    perm = rng.permutation(10)
    o3, lse3 = oracle.attention_forward(q, k[perm], v[perm], [0, 6], [0, 10])
    np.testing.assert_allclose(o3, o, atol=1e-13)
    np.testing.assert_allclose(lse3, lse, atol=1e-13)


def test_gqa_equals_mha_with_repeated_kv():
    inp = workloads.jagged(51, [5, 11], None, 6, 2, 8, True)
    q, k, v, do = (x.astype(np.float64) for x in (inp.q, inp.k, inp.v, inp.do))
    o, lse = oracle.attention_forward(q, k, v, inp.cu_q, inp.cu_k, True)
    dq, dk, dv = oracle.attention_backward(q, k, v, do, inp.cu_q, inp.cu_k, True)
    kr, vr = np.repeat(k, 3, axis=1), np.repeat(v, 3, axis=1)
    o2, lse2 = oracle.attention_forward(q, kr, vr, inp.cu_q, inp.cu_k, True)
    dq2, dk2, dv2 = oracle.attention_backward(q, kr, vr, do, inp.cu_q, inp.cu_k, True)
    np.testing.assert_allclose(o, o2, atol=1e-14)
    np.testing.assert_allclose(lse, lse2, atol=1e-14)
    np.testing.assert_allclose(dq, dq2, atol=1e-14)
    np.testing.assert_allclose(dk, dk2.reshape(-1, 2, 3, 8).sum(2), atol=1e-13)
    np.testing.assert_allclose(dv, dv2.reshape(-1, 2, 3, 8).sum(2), atol=1e-13)


def test_jagged_equals_per_sequence_dense():
    inp = workloads.jagged(61, [3, 8, 5], None, 2, 2, 8, False)
    q, k, v = (x.astype(np.float64) for x in (inp.q, inp.k, inp.v))
    o, lse = oracle.attention_forward(q, k, v, inp.cu_q, inp.cu_k)
    for b in range(3):
        s, e = inp.cu_q[b], inp.cu_q[b + 1]
        ob, lb = oracle.attention_forward(q[s:e], k[s:e], v[s:e], [0, e - s], [0, e - s])
        np.testing.assert_array_equal(o[s:e], ob)
        np.testing.assert_array_equal(lse[:, s:e], lb)


def test_broadcast_q_is_sum_over_items():
    inp = workloads.broadcast(71, 5, [4, 0, 7], 2, 1, 8)
    q, k, v, do = (x.astype(np.float64) for x in (inp.q, inp.k, inp.v, inp.do))
    o, lse = oracle.broadcast_q_forward(q, k, v, inp.cu_k)
    dq, dk, dv = oracle.broadcast_q_backward(q, k, v, do, inp.cu_k)
    assert o.shape == (3, 5, 2, 8) and lse.shape == (3, 2, 5)
    # the empty item has no keys: O = 0, LSE = -inf
    assert np.all(o[1] == 0) and np.all(np.isneginf(lse[1]))
    acc = np.zeros_like(dq)
    for b in range(3):
        ks, ke = inp.cu_k[b], inp.cu_k[b + 1]
        gq, _, _ = oracle.attention_backward(q, k[ks:ke], v[ks:ke], do[b], [0, 5], [0, ke - ks])
        acc += gq
    np.testing.assert_allclose(dq, acc, atol=1e-13)


def test_empty_sequences_and_rows():
    inp = workloads.jagged(81, [0, 4, 0], [3, 0, 0], 2, 2, 8, False)
    q, k, v, do = (x.astype(np.float64) for x in (inp.q, inp.k, inp.v, inp.do))
    o, lse = oracle.attention_forward(q, k, v, inp.cu_q, inp.cu_k)
    assert np.all(o == 0) and np.all(np.isneginf(lse))      # sequence 1 has 4 queries and no keys
    dq, dk, dv = oracle.attention_backward(q, k, v, do, inp.cu_q, inp.cu_k)
    assert np.all(dq == 0) and np.all(dk == 0) and np.all(dv == 0)


def test_decode_is_forward_with_one_query():
    inp = workloads.decode(91, [5, 12, 1], heads_q=4, heads_kv=2, head_dim=8, page_size=3)
    q, k, v = (x.astype(np.float64) for x in (inp.q, inp.k, inp.v))
    o, lse = oracle.decode_forward(q, k, v, inp.cu_k)
    for b in range(3):
        ks, ke = inp.cu_k[b], inp.cu_k[b + 1]
        for h in range(4):
            ob, lb, _ = oracle.sequence_forward(q[b, h][None], k[ks:ke, h // 2], v[ks:ke, h // 2], 1 / math.sqrt(8))
            np.testing.assert_allclose(o[b, h], ob[0], atol=1e-14)
            np.testing.assert_allclose(lse[b, h], lb[0], atol=1e-14)


@pytest.mark.parametrize("causal", [False, True])
def test_decode_multi_token_is_prefix_attention(causal):
    """q_len new tokens per sequence: with the bottom-right mask token t attends to
    exactly the key prefix [0, L - q_len + t] (checked with an unmasked call on the
    truncated keys), without it to all L keys; a token with an empty prefix gets
    O = 0 and LSE = -inf."""
    lq = 3
    inp = workloads.decode(92, [6, 2, 9, 3], heads_q=4, heads_kv=2, head_dim=8, page_size=4, q_len=lq)
    q, k, v = (x.astype(np.float64) for x in (inp.q, inp.k, inp.v))
    o, lse = oracle.decode_forward_multi(q, k, v, inp.cu_k, causal)
    assert o.shape == q.shape and lse.shape == q.shape[:3]
    for b in range(4):
        ks, ke = inp.cu_k[b], inp.cu_k[b + 1]
        L = ke - ks
        for t in range(lq):
            n = max(0, min(L, L - lq + t + 1)) if causal else L
            for h in range(4):
                if n == 0:
                    assert np.all(o[b, t, h] == 0) and np.isneginf(lse[b, t, h])
                    continue
                ob, lb, _ = oracle.sequence_forward(q[b, t, h][None], k[ks:ks + n, h // 2], v[ks:ks + n, h // 2],
                                                    1 / math.sqrt(8))
                np.testing.assert_allclose(o[b, t, h], ob[0], atol=1e-14)
                np.testing.assert_allclose(lse[b, t, h], lb[0], atol=1e-14)


# ----------------------------------------------------------------- planted mistakes are caught
def test_pins_catch_planted_mistakes(monkeypatch):
    """A wrong sign, a missing scale or a transposed operand in the oracle fails a pin."""
    import oracle.attention as oa
    case = _cases()[0]
    orig = oa.sequence_backward

    def wrong_sign(q, k, v, do, scale, causal=False):
        dq, dk, dv, delta = orig(q, k, v, do, scale, causal)
        return -dq, dk, dv, delta

    monkeypatch.setattr(oa, "sequence_backward", wrong_sign)
    with pytest.raises(AssertionError):
        test_golden_hand_examples(case)
    monkeypatch.setattr(oa, "sequence_backward", orig)

    orig_fwd = oa.sequence_forward

    def no_scale(q, k, v, scale, causal=False):
        return orig_fwd(q, k, v, 1.0, causal)

    monkeypatch.setattr(oa, "sequence_forward", no_scale)
    with pytest.raises(AssertionError):
        test_golden_hand_examples(_cases()[1])
