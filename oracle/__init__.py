"""fp64 CPU oracle (test infrastructure only; see ``oracle.attention``).

Parity pins: every function here is pinned by CPU tests in ``tests/test_oracle.py``
(hand-derived golden values, closed forms, brute force, torch's CPU fp64 SDPA with
autograd, central finite differences, and invariants of the softmax Jacobian).
"""
from .attention import (  # noqa: F401
    default_scale, sequence_forward, sequence_backward,
    attention_forward, attention_backward,
    broadcast_q_forward, broadcast_q_backward, decode_forward, decode_forward_multi,
)
