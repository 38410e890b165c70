"""CPU checks of the parity-test helpers: the tolerance check and the threaded,
per-sequence oracle runs that assemble whole tensors (they must equal the oracle's
own whole-batch calls)."""
import numpy as np
import pytest

import oracle
import workloads
from parity import check_o, half_ulp_bf16, oracle_bcast_full, oracle_self_full


def test_o_bound_is_the_larger_of_1e2_and_half_an_ulp():
    assert half_ulp_bf16(np.array([1.0]))[0] == 2.0 ** -8
    check_o(np.array([1.0 + 0.0099]), np.array([1.0]))
    check_o(np.array([3.0 - 0.0099]), np.array([3.0]))
    with pytest.raises(AssertionError):
        check_o(np.array([2.0 + 0.0101]), np.array([2.0]))     # half an ulp there is 0.0078
    check_o(np.array([5.0 + 0.0155]), np.array([5.0]))         # half an ulp at 5 is 0.0156
    with pytest.raises(AssertionError):
        check_o(np.array([5.0 + 0.0157]), np.array([5.0]))
    with pytest.raises(AssertionError):
        check_o(np.array([np.nan]), np.array([0.0]))


@pytest.mark.parametrize("causal", [False, True])
def test_self_full_equals_whole_batch_oracle(causal):
    inp = workloads.jagged(5, [7, 0, 33, 64, 1], [9, 4, 33, 50, 0], 4, 2, 32, causal)
    f = lambda x: x.astype(np.float64)
    o, lse = oracle.attention_forward(f(inp.q), f(inp.k), f(inp.v), inp.cu_q, inp.cu_k, causal)
    g = oracle.attention_backward(f(inp.q), f(inp.k), f(inp.v), f(inp.do), inp.cu_q, inp.cu_k, causal)
    got = oracle_self_full(oracle, inp)
    for x, y in zip(got, (o, lse) + tuple(g)):
        np.testing.assert_allclose(x, y, rtol=1e-12, atol=1e-12)


def test_bcast_full_equals_whole_batch_oracle():
    inp = workloads.broadcast(6, 19, [5, 0, 40, 17], 4, 2, 32)
    f = lambda x: x.astype(np.float64)
    o, lse = oracle.broadcast_q_forward(f(inp.q), f(inp.k), f(inp.v), inp.cu_k)
    g = oracle.broadcast_q_backward(f(inp.q), f(inp.k), f(inp.v), f(inp.do), inp.cu_k)
    got = oracle_bcast_full(oracle, inp)
    for x, y in zip(got, (o, lse) + tuple(g)):
        np.testing.assert_allclose(x, y, rtol=1e-12, atol=1e-12)
