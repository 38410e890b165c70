"""Run a fixed set of forward / backward / decode problems with the library that
JFA_LIBRARY names (or the default one) and save every output to an .npz file
(argv[1]).  Used by test_gpu_debug_sync.py to compare the JFA_DEBUG_SYNC build
with the normal build in separate processes."""
import os
import sys

import numpy as np
import torch

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
sys.path.insert(0, os.path.dirname(os.path.abspath(__file__)))

import bwd_varlen_flashattention_amd as jfa  # noqa: E402
import workloads  # noqa: E402
from parity import dev, host  # noqa: E402


def main(out_path):
    jfa.load()
    print("library:", jfa._lib.LIB_PATH, flush=True)
    res = {}
    cases = [("ragged_d128_causal_gqa", workloads.jagged(61, [5, 300, 0, 1000, 77, 513], None, 8, 2, 128, True)),
             ("ragged_d96", workloads.jagged(62, [64, 129, 700, 1], None, 4, 4, 96, False)),
             ("ragged_d256_causal", workloads.jagged(63, [400, 37, 650], None, 4, 2, 256, True)),
             ("ragged_d64_short", workloads.jagged(64, list(range(1, 90, 7)), None, 4, 1, 64, False))]
    for name, inp in cases:
        print("case", name, flush=True)
        q, k, v, do = (dev(x, torch) for x in (inp.q, inp.k, inp.v, inp.do))
        cq, ck = dev(inp.cu_q, torch), dev(inp.cu_k, torch)
        o, lse = jfa.jfa_fwd(q, k, v, cq, ck, inp.max_len_q, inp.max_len_k, inp.causal)
        dq, dk, dv = jfa.jfa_bwd(q, k, v, o, lse, do, cq, ck, inp.max_len_q, inp.max_len_k, inp.causal)
        torch.cuda.synchronize()
        for tag, t in (("o", o), ("lse", lse), ("dq", dq), ("dk", dk), ("dv", dv)):
            res[f"{name}_{tag}"] = host(t)
    print("case broadcast", flush=True)
    inp = workloads.broadcast(65, 300, [33, 0, 900, 512, 129, 1, 2000], 4, 2, 128)
    q, k, v, do = (dev(x, torch) for x in (inp.q, inp.k, inp.v, inp.do))
    ck = dev(inp.cu_k, torch)
    o, lse = jfa.jfa_fwd(q, k, v, None, ck, 300, inp.max_len_k, False, None, broadcast_q=True)
    dq, dk, dv = jfa.jfa_bwd(q, k, v, o, lse, do, None, ck, 300, inp.max_len_k, False, None, broadcast_q=True)
    torch.cuda.synchronize()
    for tag, t in (("o", o), ("lse", lse), ("dq", dq), ("dk", dk), ("dv", dv)):
        res[f"bcast_{tag}"] = host(t)
    print("case decode", flush=True)
    inp = workloads.decode(66, [40, 3000, 7, 900], 32, 8, 128, 16)
    args = [dev(x, torch) for x in (inp.q, inp.k_cache, inp.v_cache, inp.page_table, inp.seqlens_k)]
    for splits in (1, 5):
        o, lse = jfa.jfa_decode_paged(*args, splits)
        torch.cuda.synchronize()
        res[f"decode_s{splits}_o"], res[f"decode_s{splits}_lse"] = host(o), host(lse)
    np.savez(out_path, **res)
    print("saved", len(res), "arrays", flush=True)


if __name__ == "__main__":
    main(sys.argv[1])
