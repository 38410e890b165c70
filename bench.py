#!/usr/bin/env python3
"""Throughput of the jagged attention hot path on one MI355X.

One step = one pass of the whole path over resident synthetic inputs:
  * jagged forward + backward on the GEM workload (256 sequences, max_len 1024,
    sparsity 0.5, 8 heads, d = 128, bf16, non-causal): work-list build,
    forward, backward preprocess, backward, dQ convert;
  * split-KV paged decode on the decode workload (B = 32, Hq 32 / Hkv 8,
    d = 128, KV lengths U{4096..16384}, page size 16, automatic splits) with
    its LSE-weighted combine.
`value` is the useful (unpadded) fwd+bwd TFLOP/s: 4*d*Hq*pairs + 10*d*Hq*pairs
over the fwd+bwd time, pairs = sum_b Lq_b*Lk_b.  The decode rate is reported
beside it in TB/s of algorithmic HBM bytes.

Prints ONE JSON line.  --sweep prints one extra line per workload instead.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

MFMA_BF16_PEAK_TFLOPS = 2516.6     # 256 CU x 4096 flop/clk x 2.4 GHz, dense
HBM_PEAK_GBS = 8000.0
METRIC = "jagged attn fwd+bwd useful TFLOP/s (% bf16 MFMA peak); decode HBM TB/s"


def pairs_of(cu_q, cu_k, causal, nq=None):
    lk = np.diff(cu_k).astype(np.int64)
    if nq is not None:
        return int(nq * lk.sum())
    lq = np.diff(cu_q).astype(np.int64)
    if not causal:
        return int((lq * lk).sum())
    # key j visible to query i iff j <= i + (Lk - Lq)
    tot = 0
    for a, b in zip(lq, lk):
        i = np.arange(a)
        tot += int(np.clip(i + (b - a) + 1, 0, b).sum())
    return tot


def decode_bytes(inp):
    """Algorithmic bytes: K+V once, q and o, lse, page-table entries, lengths."""
    hkv, d = inp.k.shape[1], inp.k.shape[2]
    elem = 1 if inp.k_cache.dtype == np.uint8 else 2          # fp8 (e4m3) or bf16 cache
    kv = int(inp.seqlens_k.astype(np.int64).sum()) * hkv * d * elem * 2
    b = inp.q.shape[0]
    rows = int(np.prod(inp.q.shape[:-1]))          # B * q_len * Hq
    pages = int(sum(-(-int(L) // inp.page_size) for L in inp.seqlens_k))
    return kv + rows * d * 2 * 2 + rows * 4 + pages * 4 + b * 4


def dev(x, torch):
    """float32 array of bf16 values -> bf16 CUDA tensor; int32 stays int32."""
    t = torch.from_numpy(np.ascontiguousarray(x))
    dt = torch.bfloat16 if x.dtype == np.float32 else torch.int32
    return t.to(device="cuda", dtype=dt).contiguous()


class JaggedCase:
    def __init__(self, torch, jfa, inp=None, bcast=None):
        self.torch, self.jfa = torch, jfa
        self.bcast = bcast is not None
        x = bcast if self.bcast else inp
        self.inp = x
        self.q, self.k, self.v, self.do = (dev(a, torch) for a in (x.q, x.k, x.v, x.do))
        self.ck = dev(x.cu_k, torch)
        self.cq = None if self.bcast else dev(x.cu_q, torch)
        self.causal = False if self.bcast else x.causal
        self.mq = x.q.shape[0] if self.bcast else x.max_len_q
        self.mk = x.max_len_k
        d, hq = x.q.shape[2], x.q.shape[1]
        self.pairs = pairs_of(None if self.bcast else x.cu_q, x.cu_k, self.causal, x.q.shape[0] if self.bcast else None)
        self.fwd_flops = 4.0 * d * hq * self.pairs
        self.bwd_flops = 10.0 * d * hq * self.pairs
        self.o, self.lse = jfa.jfa_fwd(self.q, self.k, self.v, self.cq, self.ck, self.mq, self.mk, self.causal,
                                       broadcast_q=self.bcast)
        self.dq, self.dk, self.dv = (torch.empty_like(t) for t in (self.q, self.k, self.v))
        from bwd_varlen_flashattention_amd import _lib
        import ctypes
        p = jfa._attn_params(self.q, self.k, self.cq, self.ck, self.mq, self.mk, self.causal, None, self.bcast,
                             self.ck.numel() - 1)
        lib = _lib.load()
        self.ws_f = torch.empty(max(1, lib.jfa_fwd_workspace_size(ctypes.byref(p))), dtype=torch.uint8, device="cuda")
        self.ws_b = torch.empty(max(1, lib.jfa_bwd_workspace_size(ctypes.byref(p))), dtype=torch.uint8, device="cuda")

    def step(self):
        j = self.jfa
        j.jfa_fwd(self.q, self.k, self.v, self.cq, self.ck, self.mq, self.mk, self.causal, broadcast_q=self.bcast,
                  out=self.o, lse=self.lse, workspace=self.ws_f)
        j.jfa_bwd(self.q, self.k, self.v, self.o, self.lse, self.do, self.cq, self.ck, self.mq, self.mk, self.causal,
                  broadcast_q=self.bcast, dq=self.dq, dk=self.dk, dv=self.dv, workspace=self.ws_b)


class DecodeCase:
    def __init__(self, torch, jfa, inp, splits=0, causal=False):
        self.torch, self.jfa, self.inp = torch, jfa, inp
        self.causal = causal
        self.q = dev(inp.q, torch)
        if inp.k_cache.dtype == np.uint8:       # e4m3 bytes
            self.kc = torch.from_numpy(inp.k_cache).to("cuda").view(torch.float8_e4m3fn)
            self.vc = torch.from_numpy(inp.v_cache).to("cuda").view(torch.float8_e4m3fn)
        else:
            self.kc, self.vc = dev(inp.k_cache, torch), dev(inp.v_cache, torch)
        self.pt, self.sl = dev(inp.page_table, torch), dev(inp.seqlens_k, torch)
        self.splits = splits
        self.nsplits = jfa.jfa_decode_num_splits(self.q, self.kc, self.pt, splits)
        self.bytes = decode_bytes(inp)
        self.o, self.lse = jfa.jfa_decode_paged(self.q, self.kc, self.vc, self.pt, self.sl, splits, causal=causal)
        import ctypes
        from bwd_varlen_flashattention_amd import _lib
        p = jfa._decode_params(self.q, self.kc, self.pt, splits, None, causal)
        n = _lib.load().jfa_decode_workspace_size(ctypes.byref(p))
        self.ws = torch.empty(max(1, n), dtype=torch.uint8, device="cuda")

    def step(self):
        self.jfa.jfa_decode_paged(self.q, self.kc, self.vc, self.pt, self.sl, self.splits, out=self.o, lse=self.lse,
                                  workspace=self.ws, causal=self.causal)


TRAFFIC_PROFILE = os.path.join(ROOT, "profiles", "hbm_traffic_gem_s0.5_bench_step.txt")
KERNEL_SLOTS = (("bwd_dkdv_kernel", "bwd_dkdv"), ("bwd_dq_kernel", "bwd_dq"), ("fwd_kernel", "fwd"),
                ("decode_kernel", "decode"))


def source_digest() -> str:
    """Digest of the kernel sources and build options: stored counter data is only
    reported while it still describes the kernels that run."""
    import hashlib
    pkg = os.path.join(ROOT, "bwd_varlen_flashattention_amd")
    files = [os.path.join(pkg, "csrc", f) for f in sorted(os.listdir(os.path.join(pkg, "csrc")))]
    h = hashlib.sha256()
    for f in files + [os.path.join(pkg, "build.py")]:
        h.update(os.path.basename(f).encode())
        with open(f, "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def stored_traffic(sparsity: float):
    """HBM bytes per launch of each main kernel from the committed counter summary, or None."""
    if abs(sparsity - 0.5) > 1e-9 or not os.path.exists(TRAFFIC_PROFILE):
        return None
    for line in open(TRAFFIC_PROFILE):
        if line.startswith('{"source_digest"'):
            rec = json.loads(line)
            return rec["bytes_per_launch"] if rec["source_digest"] == source_digest() else None
    return None


def pmc_summary(fetch_db: str, write_db: str, copy_mib: int, out: str):
    """Turn two rocprofv3 --pmc databases of this benchmark (FETCH_SIZE, then WRITE_SIZE)
    into per-launch byte counts, scaled by what the same counters read for the plain
    device copy of copy_mib MiB that the benchmark runs after timing."""
    import collections
    import sqlite3

    def per_dispatch(db, counter):
        val, name = collections.defaultdict(float), {}
        con = sqlite3.connect(db)
        q = "select kernel_name, counter_name, value, dispatch_id from counters_collection"
        for kname, cname, v, disp in con.execute(q):
            if cname == counter:
                val[disp] += v           # sum the per-XCD / per-channel instances of one dispatch
                name[disp] = kname
        return val, name

    known = copy_mib * float(1 << 20)
    res = {}
    for counter, db in (("FETCH_SIZE", fetch_db), ("WRITE_SIZE", write_db)):
        val, name = per_dispatch(db, counter)
        copies = [d for d in val if "copy" in name[d].lower()]
        if not copies:
            raise SystemExit(f"no copy kernel among the dispatches of {db}")
        cal = max(copies, key=lambda d: val[d])
        factor = known / (val[cal] * 1024.0)
        kib = collections.defaultdict(list)
        for d, v in val.items():
            for key, slot in KERNEL_SLOTS:
                if key in name[d]:
                    kib[slot].append(v)
        res[counter] = (factor, val[cal], {k: sum(v) / len(v) for k, v in kib.items()})
    ff, fcal, fk = res["FETCH_SIZE"]
    wf, wcal, wk = res["WRITE_SIZE"]
    bytes_per = {s: fk.get(s, 0.0) * 1024.0 * ff + wk.get(s, 0.0) * 1024.0 * wf for _, s in KERNEL_SLOTS if s in fk}
    lines = [
        "# HBM traffic per launch: bench step (GEM jagged fwd+bwd, sparsity 0.5, + paged decode, page 16)",
        "",
        "Commands (repository root on the MI355X box = $REPO; one counter per run):",
        "",
        "```",
        "cd /tmp && export TMPDIR=/tmp && rocprofv3 --pmc FETCH_SIZE -d $REPO/gpurun_out/pmc_fetch -o fetch "
        "-- python3 $REPO/bench.py --steps 2 --warmup 1 --cpu-seqs 0",
        "cd /tmp && export TMPDIR=/tmp && rocprofv3 --pmc WRITE_SIZE -d $REPO/gpurun_out/pmc_write -o write "
        "-- python3 $REPO/bench.py --steps 2 --warmup 1 --cpu-seqs 0",
        "python3 bench.py --pmc-summary gpurun_out/pmc_fetch/fetch_results.db gpurun_out/pmc_write/write_results.db",
        "```",
        "",
        f"Calibration: the benchmark's plain device copy of {copy_mib} MiB reads {fcal:.0f} KiB (FETCH_SIZE) and "
        f"writes {wcal:.0f} KiB (WRITE_SIZE); scale factors {ff:.4f} (fetch) and {wf:.4f} (write) map the "
        "counters to bytes.  FETCH_SIZE counts L2 misses served by the memory side, so reads that hit the "
        "last-level MALL count too.",
        "",
        "| kernel | FETCH_SIZE (KiB/launch) | WRITE_SIZE (KiB/launch) | scaled bytes/launch |",
        "|---|---|---|---|",
    ]
    for _, s in KERNEL_SLOTS:
        if s in bytes_per:
            lines.append(f"| {s} | {fk[s]:.0f} | {wk.get(s, 0.0):.0f} | {bytes_per[s]:.4g} |")
    lines += ["", "Machine-readable line (the digest covers the kernel sources and build options):", ""]
    lines.append(json.dumps({"source_digest": source_digest(), "workload": "gem_s0.5",
                             "fetch_factor": ff, "write_factor": wf, "bytes_per_launch": bytes_per}))
    with open(out, "w") as f:
        f.write("\n".join(lines) + "\n")
    print("\n".join(lines))


def cpu_baseline(inp, n_seq: int):
    """Time the fp64 oracle on the first n_seq sequences of the same workload (fwd + bwd)."""
    import oracle
    from threadpoolctl import threadpool_info
    cu = inp.cu_q
    te = int(cu[n_seq])
    sub = [x[:te].astype(np.float64) for x in (inp.q, inp.k, inp.v, inp.do)]
    cs = cu[:n_seq + 1]
    t0 = time.perf_counter()
    oracle.attention_forward(sub[0], sub[1], sub[2], cs, cs, False)
    oracle.attention_backward(*sub, cs, cs, False)
    dt = time.perf_counter() - t0
    pairs = pairs_of(cs, cs, False)
    flops = 14.0 * inp.q.shape[2] * inp.q.shape[1] * pairs
    threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    return {"value": flops / dt / 1e12, "unit": "TFLOP/s", "cores": int(threads), "kind": "oracle",
            "sample": f"fp64 numpy oracle, fwd+bwd of the first {n_seq} of 256 sequences "
                      f"({te} tokens, {pairs * inp.q.shape[1]} query-key pairs) of the same workload; "
                      f"{dt:.1f} s wall"}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--sparsity", type=float, default=0.5)
    ap.add_argument("--page-size", type=int, default=16)
    ap.add_argument("--cpu-seqs", type=int, default=256, help="sequences in the oracle timing sample (0 = skip)")
    ap.add_argument("--sweep", action="store_true", help="one JSON line per workload (GEM s, broadcast-Q, dense, decode)")
    ap.add_argument("--copy-calibration-mib", type=int, default=1024,
                    help="run one device copy of this size after timing (reference for HBM byte counters)")
    ap.add_argument("--pmc-summary", nargs=2, metavar=("FETCH_DB", "WRITE_DB"),
                    help="summarise two rocprofv3 --pmc runs of this benchmark into the traffic profile and exit")
    args = ap.parse_args()
    if args.pmc_summary:
        return pmc_summary(*args.pmc_summary, args.copy_calibration_mib, TRAFFIC_PROFILE)

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(json.dumps({"error": "this benchmark runs on one GPU only; --gpus must be 1"}))
        sys.exit(2)

    import torch
    import bwd_varlen_flashattention_amd as jfa
    import workloads
    assert torch.cuda.is_available(), "bench.py needs a GPU"
    jfa.load()

    def log(*a):
        print(*a, file=sys.stderr, flush=True)

    if args.sweep:
        return sweep(torch, jfa, workloads, args, log)

    t0 = time.time()
    gem_inp = workloads.gem(0, args.sparsity)
    dec_inp = workloads.decode_paged(0, args.page_size, tail_fill=0.0)
    log(f"inputs generated in {time.time() - t0:.1f}s")
    jc = JaggedCase(torch, jfa, gem_inp)
    dc = DecodeCase(torch, jfa, dec_inp)
    del dec_inp

    for _ in range(args.warmup):
        jc.step()
        dc.step()
    torch.cuda.synchronize()

    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(args.steps)]
    jfa.timing.enable(True)
    torch.cuda.synchronize()
    t_start = time.perf_counter()
    for i in range(args.steps):
        ev[i][0].record()
        jc.step()
        ev[i][1].record()
        dc.step()
        ev[i][2].record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t_start
    jfa.timing.enable(False)
    kt = jfa.timing.collect()
    fb_ms = sum(e[0].elapsed_time(e[1]) for e in ev)
    dec_ms = sum(e[1].elapsed_time(e[2]) for e in ev)
    step_ms = wall * 1e3 / args.steps

    tflops = (jc.fwd_flops + jc.bwd_flops) * args.steps / (fb_ms * 1e-3) / 1e12
    dec_tbs = dc.bytes * args.steps / (dec_ms * 1e-3) / 1e12
    avg = {k: (ms / n if n else 0.0) for k, (ms, n) in kt.items()}
    # Algorithmic flops per launch of each main kernel (per query-key pair, times Hq):
    #   fwd       4d  (S = Q K^T, O = P V)
    #   bwd_dkdv  8d  (S recomputed, dP, dV, dK: the backward's contractions except dQ)
    #   bwd_dq    2d  (dQ = dS K; its own S/dP recomputation is not counted)
    d, hq = 128, 8
    alg = {"fwd": 4.0 * d * hq * jc.pairs, "bwd_dkdv": 8.0 * d * hq * jc.pairs, "bwd_dq": 2.0 * d * hq * jc.pairs}
    dominant = max(alg, key=lambda k: avg[k])
    ach = alg[dominant] / (avg[dominant] * 1e-3) / 1e12
    names = {"fwd": "fwd_kernel (jagged forward)", "bwd_dkdv": "bwd_dkdv_kernel (key-stationary dK/dV)",
             "bwd_dq": "bwd_dq_kernel (query-stationary dQ)"}

    # plain device copy of known size: reference for FETCH_SIZE / WRITE_SIZE scaling
    if args.copy_calibration_mib > 0:
        n = args.copy_calibration_mib * (1 << 20) // 4
        src = torch.empty(n, dtype=torch.float32, device="cuda").fill_(1.0)
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    stored = stored_traffic(args.sparsity)
    traffic = round(stored[dominant]) if stored and dominant in stored else None

    cpu = None
    if args.cpu_seqs > 0:
        cpu = cpu_baseline(gem_inp, min(args.cpu_seqs, gem_inp.batch))

    meta = gem_inp.meta
    out = {
        "metric": METRIC,
        "value": round(tflops, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(step_ms, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "pct_mfma_peak": round(100 * tflops / MFMA_BF16_PEAK_TFLOPS, 2),
        "config": {
            "workload": f"GEM jagged self-attention fwd+bwd (sparsity {args.sparsity}) + paged split-KV decode",
            "jagged": {"batch": 256, "max_len": 1024, "sparsity": args.sparsity,
                       "realised_sparsity": round(meta["realised_sparsity"], 4), "heads": 8, "head_dim": 128,
                       "total_tokens": int(gem_inp.q.shape[0]), "causal": False,
                       "fwd_gflop": round(jc.fwd_flops / 1e9, 2), "bwd_gflop": round(jc.bwd_flops / 1e9, 2)},
            "decode": {"batch": 32, "heads_q": 32, "heads_kv": 8, "head_dim": 128, "page_size": args.page_size,
                       "splits": dc.nsplits, "kv_len": "U{4096..16384}", "gbytes": round(dc.bytes / 1e9, 4)},
        },
        "fwd_bwd_ms": round(fb_ms / args.steps, 4),
        "decode": {"value": round(dec_tbs, 3), "unit": "TB/s", "pct_hbm_peak": round(100 * dec_tbs * 1e3 / HBM_PEAK_GBS, 2),
                   "ms": round(dec_ms / args.steps, 4)},
        "kernels_ms": {k: round(v, 4) for k, v in avg.items()},
        "roofline": {"kernel": names[dominant], "bound": "mfma",
                     "achieved": round(ach, 2), "peak": MFMA_BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(ach / MFMA_BF16_PEAK_TFLOPS, 4), "traffic": traffic,
                     "algorithmic_flop_per_launch": alg[dominant]},
        "cpu_baseline": cpu,
    }
    print(json.dumps(out), flush=True)


def sweep(torch, jfa, workloads, args, log):
    """Per-workload numbers (fwd, bwd and decode separately), one JSON line each."""
    def timeit(fn, n=10, w=3):
        for _ in range(w):
            fn()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(n):
            fn()
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / n

    cases = [("gem_s0.1", lambda: workloads.gem(0, 0.1)), ("gem_s0.5", lambda: workloads.gem(0, 0.5)),
             ("gem_s0.9", lambda: workloads.gem(0, 0.9)),
             ("bcast_s0.1", lambda: workloads.broadcast_q(0, 0.1)), ("bcast_s0.5", lambda: workloads.broadcast_q(0, 0.5)),
             ("bcast_s0.9", lambda: workloads.broadcast_q(0, 0.9)),
             ("dense_causal_d128", lambda: workloads.dense_causal(0, head_dim=128)),
             ("dense_causal_d96", lambda: workloads.dense_causal(0, head_dim=96)),
             ("gem_s0.5_d256", lambda: workloads.gem(0, 0.5, head_dim=256)),
             ("dense_causal_d256_h16", lambda: workloads.dense_causal(0, heads=16, head_dim=256))]
    for name, make in cases:
        inp = make()
        jc = JaggedCase(torch, jfa, bcast=inp) if name.startswith("bcast") else JaggedCase(torch, jfa, inp)
        del inp
        f_ms = timeit(lambda: jfa.jfa_fwd(jc.q, jc.k, jc.v, jc.cq, jc.ck, jc.mq, jc.mk, jc.causal, broadcast_q=jc.bcast,
                                          out=jc.o, lse=jc.lse, workspace=jc.ws_f))
        b_ms = timeit(lambda: jfa.jfa_bwd(jc.q, jc.k, jc.v, jc.o, jc.lse, jc.do, jc.cq, jc.ck, jc.mq, jc.mk, jc.causal,
                                          broadcast_q=jc.bcast, dq=jc.dq, dk=jc.dk, dv=jc.dv, workspace=jc.ws_b))
        line = {"workload": name, "fwd_ms": round(f_ms, 4), "bwd_ms": round(b_ms, 4),
                "fwd_tflops": round(jc.fwd_flops / f_ms / 1e9, 1), "bwd_tflops": round(jc.bwd_flops / b_ms / 1e9, 1),
                "fwd_pct_peak": round(100 * jc.fwd_flops / f_ms / 1e9 / MFMA_BF16_PEAK_TFLOPS, 2),
                "bwd_pct_peak": round(100 * jc.bwd_flops / b_ms / 1e9 / MFMA_BF16_PEAK_TFLOPS, 2)}
        print(json.dumps(line), flush=True)
        del jc
        torch.cuda.empty_cache()
    # e4m3 forward (Q K^T on the fp8 matrix cores) against the bf16 forward of the same workload
    for name, make in (("gem_s0.5", lambda: workloads.gem(0, 0.5)),
                       ("dense_causal_d128", lambda: workloads.dense_causal(0, head_dim=128))):
        base = make()
        inp, enc = workloads.fp8_qkv(base)
        del base
        jc = JaggedCase(torch, jfa, inp)
        q8, k8, v8 = (torch.from_numpy(enc[n]).to("cuda").view(torch.float8_e4m3fn) for n in ("q", "k", "v"))
        sc = dict(q_scale=enc["q_scale"], k_scale=enc["k_scale"], v_scale=enc["v_scale"])
        del inp, enc
        # the forward's workspace (its work list) does not depend on the element type
        f8_ms = timeit(lambda: jfa.jfa_fwd(q8, k8, v8, jc.cq, jc.ck, jc.mq, jc.mk, jc.causal, out=jc.o, lse=jc.lse,
                                           workspace=jc.ws_f, **sc))
        bf_ms = timeit(lambda: jfa.jfa_fwd(jc.q, jc.k, jc.v, jc.cq, jc.ck, jc.mq, jc.mk, jc.causal,
                                           out=jc.o, lse=jc.lse, workspace=jc.ws_f))
        print(json.dumps({"workload": name + "_fp8_fwd", "fwd_ms": round(f8_ms, 4), "bf16_fwd_ms": round(bf_ms, 4),
                          "fwd_tflops": round(jc.fwd_flops / f8_ms / 1e9, 1), "speedup": round(bf_ms / f8_ms, 3)}),
              flush=True)
        del jc, q8, k8, v8
        torch.cuda.empty_cache()
    for ps in (16, 1, 128):
        inp = workloads.decode_paged(0, ps, tail_fill=0.0)
        for splits in (1, 2, 4, 8, 16, 0):
            dc = DecodeCase(torch, jfa, inp, splits)
            ms = timeit(dc.step)
            print(json.dumps({"workload": f"decode_ps{ps}", "splits": dc.nsplits, "ms": round(ms, 4),
                              "tb_s": round(dc.bytes / ms / 1e9, 3)}), flush=True)
            del dc
        del inp
        torch.cuda.empty_cache()
    # a few new tokens per sequence (speculative decode): 4 tokens, causal, page 16
    rng = np.random.default_rng(0)
    lens = rng.integers(4096, 16385, size=32)
    inp = workloads.decode(0, lens, 32, 8, 128, 16, max_pages_per_seq=1024, tail_fill=0.0, q_len=4)
    for splits in (4, 8, 0):
        dc = DecodeCase(torch, jfa, inp, splits, causal=True)
        ms = timeit(dc.step)
        print(json.dumps({"workload": "decode_ps16_q4_causal", "splits": dc.nsplits, "ms": round(ms, 4),
                          "tb_s": round(dc.bytes / ms / 1e9, 3)}), flush=True)
        del dc
    del inp
    # head dim 256, single token, page 16 (same lengths and heads as the decode config)
    inp = workloads.decode(0, lens, 32, 8, 256, 16, max_pages_per_seq=1024, tail_fill=0.0)
    for splits in (4, 8, 0):
        dc = DecodeCase(torch, jfa, inp, splits)
        ms = timeit(dc.step)
        print(json.dumps({"workload": "decode_ps16_d256", "splits": dc.nsplits, "ms": round(ms, 4),
                          "tb_s": round(dc.bytes / ms / 1e9, 3)}), flush=True)
        del dc
    del inp
    # fp8 (e4m3) KV cache, single token, page 16 (same lengths as the decode config)
    inp = workloads.decode(0, lens, 32, 8, 128, 16, max_pages_per_seq=1024, kv_fp8=True)
    for splits in (4, 8, 0):
        dc = DecodeCase(torch, jfa, inp, splits)
        ms = timeit(dc.step)
        print(json.dumps({"workload": "decode_ps16_fp8kv", "splits": dc.nsplits, "ms": round(ms, 4),
                          "tb_s": round(dc.bytes / ms / 1e9, 3)}), flush=True)
        del dc
    del inp
    torch.cuda.empty_cache()


if __name__ == "__main__":
    main()
