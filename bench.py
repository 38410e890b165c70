#!/usr/bin/env python3
"""Throughput of the jagged attention hot path on one MI355X.

One step = one pass of the whole path over resident synthetic inputs:
  * jagged forward + backward on the dense causal workload (4 sequences of
    8192 tokens, 32 heads, d = 128, bf16, causal): work-list build, forward,
    backward (dQ with delta, dK/dV);
  * split-KV paged decode on the decode workload (B = 32, Hq 32 / Hkv 8,
    d = 128, KV lengths U{4096..16384}, page size 16, automatic splits) with
    its LSE-weighted combine.
`value` is the useful (unpadded) fwd+bwd TFLOP/s of the dense causal part:
4*d*Hq*pairs + 10*d*Hq*pairs over its fwd+bwd time, pairs = visible
query-key pairs.  The decode rate is reported beside it in TB/s of
algorithmic HBM bytes, and the GEM (sparsity 0.5) and broadcast-Q (sparsity
0.5) jagged workloads as extra keys, timed after the steps.

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
    """One jagged workload resident on the GPU, with outputs and workspaces allocated once."""

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
        self.d, self.hq = x.q.shape[2], x.q.shape[1]
        self.pairs = pairs_of(None if self.bcast else x.cu_q, x.cu_k, self.causal, x.q.shape[0] if self.bcast else None)
        self.fwd_flops = 4.0 * self.d * self.hq * self.pairs
        self.bwd_flops = 10.0 * self.d * self.hq * self.pairs
        # Algorithmic HBM bytes (each tensor read or written once): forward reads Q, K, V
        # and writes O, LSE; backward reads Q, K, V, O, dO, LSE, delta and writes dQ, dK, dV.
        # Broadcast-Q: Q and dQ are [Nq, Hq, d], O, dO, LSE and delta per item.
        hkv, tk = x.k.shape[1], x.k.shape[0]
        nq = x.q.shape[0]
        rows_o = (len(x.cu_k) - 1) * nq if self.bcast else nq     # rows of O / dO / LSE
        q_el, o_el, k_el = nq * self.hq * self.d, rows_o * self.hq * self.d, tk * hkv * self.d
        self.fwd_bytes = 2.0 * (q_el + 2 * k_el + o_el) + 4.0 * rows_o * self.hq
        self.bwd_bytes = 2.0 * (2 * q_el + 4 * k_el + 2 * o_el) + 8.0 * rows_o * self.hq
        # Algorithmic flops per launch of each main kernel (per visible query-key pair, times Hq):
        #   fwd       4d  (S = Q K^T, O = P V)
        #   bwd_dkdv  8d  (S recomputed, dP, dV, dK: the backward's contractions except dQ)
        #   bwd_dq    2d  (dQ = dS K; its own S/dP recomputation is not counted)
        u = self.d * self.hq * self.pairs
        self.kernel_flops = {"fwd": 4.0 * u, "bwd_dkdv": 8.0 * u, "bwd_dq": 2.0 * u}
        sizes = (self.q, self.k, self.ck, self.mq, self.mk, self.causal, self.bcast)
        self.ws_f = torch.empty(max(1, jfa.jfa_fwd_workspace_size(*sizes)), dtype=torch.uint8, device="cuda")
        self.ws_b = torch.empty(max(1, jfa.jfa_bwd_workspace_size(*sizes)), dtype=torch.uint8, device="cuda")
        self.o, self.lse = jfa.jfa_fwd(self.q, self.k, self.v, self.cq, self.ck, self.mq, self.mk, self.causal,
                                       broadcast_q=self.bcast, workspace=self.ws_f)
        self.dq, self.dk, self.dv = (torch.empty_like(t) for t in (self.q, self.k, self.v))

    def fwd(self, events=None):
        self.jfa.jfa_fwd(self.q, self.k, self.v, self.cq, self.ck, self.mq, self.mk, self.causal,
                         broadcast_q=self.bcast, out=self.o, lse=self.lse, workspace=self.ws_f, events=events)

    def bwd(self, events=None):
        self.jfa.jfa_bwd(self.q, self.k, self.v, self.o, self.lse, self.do, self.cq, self.ck, self.mq, self.mk,
                         self.causal, broadcast_q=self.bcast, dq=self.dq, dk=self.dk, dv=self.dv,
                         workspace=self.ws_b, events=events)

    def step(self, events=None):
        self.fwd(events)
        self.bwd(events)


class DecodeCase:
    def __init__(self, torch, jfa, inp, splits=0, causal=False, single_launch=False):
        self.torch, self.jfa, self.inp = torch, jfa, inp
        self.causal = causal
        self.single_launch = single_launch
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
        n = jfa.jfa_decode_workspace_size(self.q, self.kc, self.pt, splits)
        self.ws = torch.zeros(max(1, n), dtype=torch.uint8, device="cuda")   # arrival counters start at zero
        self.o, self.lse = jfa.jfa_decode_paged(self.q, self.kc, self.vc, self.pt, self.sl, splits, causal=causal,
                                                workspace=self.ws, single_launch=single_launch)

    def step(self, events=None):
        self.jfa.jfa_decode_paged(self.q, self.kc, self.vc, self.pt, self.sl, self.splits, out=self.o, lse=self.lse,
                                  workspace=self.ws, causal=self.causal, events=events,
                                  single_launch=self.single_launch)


# ----------------------------------------------------------------------------- stored counter data
KERNEL_SLOTS = ("fwd", "bwd_dq", "bwd_dkdv", "decode")
# kernel name prefixes of the slots
SLOT_KERNEL = {"fwd": "fwd_kernel", "bwd_dq": "bwd_dq_kernel", "bwd_dkdv": "bwd_dkdv_kernel", "decode": "decode_kernel"}
# template arguments that tell the bench step's workloads apart (head dim, causal, broadcast[, fp8])
# (fwd_kernel<d, causal, broadcast, fp8, narrow>, bwd_dq_kernel<d, causal, broadcast, narrow>,
#  bwd_dkdv_kernel<d, causal, broadcast>; the bench workloads take the 256-row shapes)
WORKLOAD_KERNELS = {
    "dense_causal_d128": {"fwd": "fwd_kernel<128, true, false, false, false>",
                          "bwd_dq": "bwd_dq_kernel<128, true, false, false>",
                          "bwd_dkdv": "bwd_dkdv_kernel<128, true, false>"},
    "gem_s0.5": {"fwd": "fwd_kernel<128, false, false, false, false>", "bwd_dq": "bwd_dq_kernel<128, false, false, false>",
                 "bwd_dkdv": "bwd_dkdv_kernel<128, false, false>"},
    "bcast_s0.5": {"fwd": "fwd_kernel<128, false, true, false, false>", "bwd_dq": "bwd_dq_kernel<128, false, true, false>",
                   "bwd_dkdv": "bwd_dkdv_kernel<128, false, true>"},
    "decode_ps16": {"decode": "decode_kernel<128, 1, false>"},
}
TRAFFIC_PROFILE = os.path.join(ROOT, "profiles", "hbm_traffic_bench_step.txt")
COUNTER_PROFILE = os.path.join(ROOT, "profiles", "mfma_lds_counters_bench_step.md")
STALL_PROFILE = os.path.join(ROOT, "profiles", "wave_state_counters_bench_step.md")
BENCH_CMD = "python3 $REPO/bench.py --steps 2 --warmup 1 --cpu-sample 0 --single-launch-steps 0"


def _run_of(db: str):
    """(directory, -o name) of a rocprofv3 output database path such as <dir>/<name>_results.db,
    for quoting the command that wrote it."""
    d = os.path.dirname(db) or "."
    name = os.path.basename(db)
    return d, name[: -len("_results.db")] if name.endswith("_results.db") else name


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


def stored_traffic(workload: str):
    """HBM bytes per launch of each main kernel of `workload` from the committed
    counter summary, or None when the summary describes other kernel sources."""
    if not os.path.exists(TRAFFIC_PROFILE):
        return None
    for line in open(TRAFFIC_PROFILE):
        if line.startswith('{"source_digest"'):
            rec = json.loads(line)
            if rec["source_digest"] != source_digest():
                return None
            return rec["bytes_per_launch"].get(workload)
    return None


def _per_dispatch(db, counters):
    """{dispatch: {counter: value}} (instances of one dispatch summed), {dispatch: kernel name},
    {dispatch: duration ns}."""
    import collections
    import sqlite3
    val = collections.defaultdict(lambda: collections.defaultdict(float))
    name, dur = {}, {}
    con = sqlite3.connect(db)
    q = "select kernel_name, counter_name, value, dispatch_id, duration from counters_collection"
    for kname, cname, v, disp, d in con.execute(q):
        if cname in counters:
            val[disp][cname] += v
            name[disp] = kname
            dur[disp] = d
    return val, name, dur


def _workload_dispatches(name):
    """{(workload, slot): [dispatch ids]} for the bench step's main kernels."""
    out = {}
    for disp, kname in name.items():
        for wl, slots in WORKLOAD_KERNELS.items():
            for slot, key in slots.items():
                if key + "(" in kname.replace("jfa::", ""):
                    out.setdefault((wl, slot), []).append(disp)
    return out


def _reference_dispatches(name):
    """{("library_gemm_bf16_8192", "gemm"): [dispatch ids]}: the library GEMM of --gemm-probe,
    summarised beside the attention kernels as a reference for clock and MFMA busy."""
    ds = [d for d, k in name.items() if k.startswith("Cijk_")]
    return {("library_gemm_bf16_8192", "gemm"): ds} if ds else {}


def pmc_summary(fetch_db: str, write_db: str, copy_mib: int, out: str):
    """Turn two rocprofv3 --pmc databases of this benchmark (FETCH_SIZE, then WRITE_SIZE)
    into per-launch byte counts, scaled by what the same counters read for the plain
    device copy of copy_mib MiB that the benchmark runs after timing."""
    known = copy_mib * float(1 << 20)
    res = {}
    for counter, db in (("FETCH_SIZE", fetch_db), ("WRITE_SIZE", write_db)):
        val, name, _ = _per_dispatch(db, {counter})
        copies = [d for d in val if "copy" in name[d].lower()]
        if not copies:
            raise SystemExit(f"no copy kernel among the dispatches of {db}")
        cal = max(copies, key=lambda d: val[d][counter])
        factor = known / (val[cal][counter] * 1024.0)
        per = {k: sum(val[d][counter] for d in ds) / len(ds) for k, ds in _workload_dispatches(name).items()}
        res[counter] = (factor, val[cal][counter], per)
    ff, fcal, fk = res["FETCH_SIZE"]
    wf, wcal, wk = res["WRITE_SIZE"]
    keys = sorted(set(fk) | set(wk))
    bytes_per = {}
    for wl, slot in keys:
        bytes_per.setdefault(wl, {})[slot] = fk.get((wl, slot), 0.0) * 1024.0 * ff + wk.get((wl, slot), 0.0) * 1024.0 * wf
    lines = [
        "# HBM traffic per launch: bench step kernels (dense causal d = 128, GEM s = 0.5, broadcast-Q s = 0.5, "
        "paged decode page 16)",
        "",
        "Commands (repository root on the MI355X box = $REPO; one counter per run):",
        "",
        "```",
        f"cd /tmp && export TMPDIR=/tmp && timeout -s KILL 300 rocprofv3 --pmc FETCH_SIZE -d $REPO/{_run_of(fetch_db)[0]} "
        f"-o {_run_of(fetch_db)[1]} -- {BENCH_CMD}",
        f"cd /tmp && export TMPDIR=/tmp && timeout -s KILL 300 rocprofv3 --pmc WRITE_SIZE -d $REPO/{_run_of(write_db)[0]} "
        f"-o {_run_of(write_db)[1]} -- {BENCH_CMD}",
        f"python3 bench.py --pmc-summary {fetch_db} {write_db}",
        "```",
        "",
        f"Calibration: the benchmark's plain device copy of {copy_mib} MiB reads {fcal:.0f} KiB (FETCH_SIZE) and "
        f"writes {wcal:.0f} KiB (WRITE_SIZE); scale factors {ff:.4f} (fetch) and {wf:.4f} (write) map the "
        "counters to bytes.  FETCH_SIZE counts L2 misses served by the memory side, so reads that hit the "
        "last-level MALL count too.",
        "",
        "| workload | kernel | FETCH_SIZE (KiB/launch) | WRITE_SIZE (KiB/launch) | scaled bytes/launch |",
        "|---|---|---|---|---|",
    ]
    for wl, slot in keys:
        lines.append(f"| {wl} | {slot} | {fk.get((wl, slot), 0.0):.0f} | {wk.get((wl, slot), 0.0):.0f} | "
                     f"{bytes_per[wl][slot]:.4g} |")
    lines += ["", "Machine-readable line (the digest covers the kernel sources and build options):", ""]
    lines.append(json.dumps({"source_digest": source_digest(), "fetch_factor": ff, "write_factor": wf,
                             "bytes_per_launch": bytes_per}))
    with open(out, "w") as f:
        f.write("\n".join(lines) + "\n")
    print("\n".join(lines))


COUNTERS = ("SQ_VALU_MFMA_BUSY_CYCLES", "SQ_INSTS_VALU_MFMA_MOPS_BF16", "SQ_INSTS_VALU_MFMA_MOPS_F16", "SQ_INSTS_MFMA",
            "SQ_INSTS_LDS", "SQ_INSTS_VALU_TRANS_F32", "SQ_LDS_BANK_CONFLICT", "SQ_BUSY_CU_CYCLES", "GRBM_GUI_ACTIVE")
XCDS, CUS, SIMDS_PER_CU = 8, 256, 4


def counter_summary(db: str, out: str):
    """Summarise one rocprofv3 --pmc run (the COUNTERS above) of this benchmark: per main
    kernel of each workload, the counters per launch and what follows from them."""
    import workloads
    val, name, dur = _per_dispatch(db, set(COUNTERS))
    groups = {**_workload_dispatches(name), **_reference_dispatches(name)}
    # algorithmic flops per launch, from the same seeded workloads the benchmark runs
    alg = {}
    for wl, make in (("dense_causal_d128", lambda: workloads.dense_causal(0, head_dim=128)),
                     ("gem_s0.5", lambda: workloads.gem(0, 0.5)), ("bcast_s0.5", lambda: workloads.broadcast_q(0, 0.5))):
        x = make()
        bc = wl.startswith("bcast")
        pairs = pairs_of(None if bc else x.cu_q, x.cu_k, False if bc else x.causal, x.q.shape[0] if bc else None)
        u = x.q.shape[2] * x.q.shape[1] * pairs
        alg[wl] = {"fwd": 4.0 * u, "bwd_dkdv": 8.0 * u, "bwd_dq": 2.0 * u}
        del x
    alg["library_gemm_bf16_8192"] = {"gemm": 2.0 * 8192 ** 3}
    peak = MFMA_BF16_PEAK_TFLOPS * 1e12
    lines = [
        "# MFMA, LDS and transcendental counters: bench step kernels",
        "",
        "Command (repository root on the MI355X box = $REPO):",
        "",
        "```",
        "cd /tmp && export TMPDIR=/tmp && timeout -s KILL 300 rocprofv3 --pmc " + " ".join(COUNTERS)
        + f" --kernel-trace -d $REPO/{_run_of(db)[0]} -o {_run_of(db)[1]} -- {BENCH_CMD}",
        f"python3 bench.py --counter-summary {db}",
        "```",
        "",
        "Per launch (mean over the run's launches of each kernel).  Derived columns:",
        "",
        "* `MFMA TFLOP/s` = 512 x (SQ_INSTS_VALU_MFMA_MOPS_BF16 + SQ_INSTS_VALU_MFMA_MOPS_F16) / launch duration "
        "(executed 16-bit MFMA work: S and the backward on bf16, P V on fp16; the duration is the dispatch's own, "
        "taken with the counters on);",
        "* `MFMA util` = that rate / 2516.6 TFLOP/s (dense bf16/fp16 peak at 2.4 GHz);",
        "* `clock` = GRBM_GUI_ACTIVE / 8 XCDs / duration (GHz): the engine clock the kernel actually ran at;",
        "* `MFMA busy` = SQ_VALU_MFMA_BUSY_CYCLES / (GRBM_GUI_ACTIVE / 8 x 256 CUs x 4 SIMDs): the fraction of "
        "SIMD cycles the matrix core was busy, at the actual clock (the counter sums over SIMDs);",
        "* `exec/alg` = executed MFMA flops / the kernel's algorithmic flops (fwd 4d, dK/dV 8d, dQ 2d per pair "
        "and head: the dQ kernel recomputes S and dP, 6d executed);",
        "* `LDS/MFMA` = SQ_INSTS_LDS / SQ_INSTS_MFMA; `exp/MFMA` = SQ_INSTS_VALU_TRANS_F32 / SQ_INSTS_MFMA;",
        "* `bank confl/LDS` = SQ_LDS_BANK_CONFLICT / SQ_INSTS_LDS (conflict cycles per LDS instruction).",
        "",
        "`library_gemm_bf16_8192` is the reference GEMM the benchmark times after its steps (torch.matmul, "
        "bf16, 8192 x 8192 x 8192, contiguous operands): the clock and MFMA busy a tuned library kernel "
        "sustains on this GPU.",
        "",
        "| workload | kernel | ms | MFMA TFLOP/s | MFMA util | clock | MFMA busy | exec/alg | SQ_INSTS_MFMA | LDS/MFMA | "
        "exp/MFMA | bank confl/LDS |",
        "|---|---|---|---|---|---|---|---|---|---|---|---|",
    ]
    rec = {}
    for (wl, slot), ds in sorted(groups.items()):
        m = {c: sum(val[d][c] for d in ds) / len(ds) for c in COUNTERS}
        ms = sum(dur[d] for d in ds) / len(ds) * 1e-6
        flops = 512.0 * (m["SQ_INSTS_VALU_MFMA_MOPS_BF16"] + m["SQ_INSTS_VALU_MFMA_MOPS_F16"])
        rate = flops / (ms * 1e-3) if ms > 0 else 0.0
        cyc = m["GRBM_GUI_ACTIVE"] / XCDS
        clock = cyc / (ms * 1e-3) / 1e9 if ms > 0 else 0.0
        busy = m["SQ_VALU_MFMA_BUSY_CYCLES"] / max(1.0, cyc * CUS * SIMDS_PER_CU)
        a = alg.get(wl, {}).get(slot)
        mf = max(1.0, m["SQ_INSTS_MFMA"])
        row = {"ms": ms, "mfma_tflops": rate / 1e12, "mfma_util": rate / peak, "clock_ghz": clock, "mfma_busy": busy,
               "exec_over_alg": flops / a if a else None, "lds_per_mfma": m["SQ_INSTS_LDS"] / mf,
               "exp_per_mfma": m["SQ_INSTS_VALU_TRANS_F32"] / mf,
               "bank_conflict_per_lds": m["SQ_LDS_BANK_CONFLICT"] / max(1.0, m["SQ_INSTS_LDS"]),
               "counters": m}
        rec.setdefault(wl, {})[slot] = row
        ea = f"{row['exec_over_alg']:.2f}" if a else "-"
        lines.append(f"| {wl} | {slot} | {ms:.3f} | {rate / 1e12:.1f} | {rate / peak:.3f} | {clock:.2f} | {busy:.3f} | {ea} | "
                     f"{m['SQ_INSTS_MFMA']:.4g} | {row['lds_per_mfma']:.2f} | {row['exp_per_mfma']:.2f} | "
                     f"{row['bank_conflict_per_lds']:.3f} |")
    lines += ["", "Raw counters per launch:", "", "| workload | kernel | " + " | ".join(COUNTERS) + " |",
              "|---|---|" + "---|" * len(COUNTERS)]
    for wl in sorted(rec):
        for slot, row in sorted(rec[wl].items()):
            lines.append(f"| {wl} | {slot} | " + " | ".join(f"{row['counters'][c]:.4g}" for c in COUNTERS) + " |")
    lines += ["", "Machine-readable line (the digest covers the kernel sources and build options):", ""]
    lines.append(json.dumps({"source_digest": source_digest(),
                             "per_launch": {wl: {s: {k: v for k, v in r.items() if k != "counters"}
                                                 for s, r in d.items()} for wl, d in rec.items()}}))
    with open(out, "w") as f:
        f.write("\n".join(lines) + "\n")
    print("\n".join(lines))


STALL_COUNTERS = ("SQ_WAVE_CYCLES", "SQ_ACTIVE_INST_ANY", "SQ_ACTIVE_INST_VALU", "SQ_ACTIVE_INST_LDS",
                  "SQ_ACTIVE_INST_VMEM", "SQ_WAIT_ANY", "SQ_WAIT_INST_ANY", "SQ_WAIT_INST_LDS", "GRBM_GUI_ACTIVE")


def stall_summary(db: str, out: str):
    """Summarise one rocprofv3 --pmc run of the wave-state counters (STALL_COUNTERS) of this
    benchmark: per main kernel, where its waves spend their resident cycles."""
    val, name, dur = _per_dispatch(db, set(STALL_COUNTERS))
    groups = {**_workload_dispatches(name), **_reference_dispatches(name)}
    lines = [
        "# Wave-state counters: where the bench step kernels' waves spend their cycles",
        "",
        "Command (repository root on the MI355X box = $REPO):",
        "",
        "```",
        "cd /tmp && export TMPDIR=/tmp && timeout -s KILL 300 rocprofv3 --pmc " + " ".join(STALL_COUNTERS)
        + f" --kernel-trace -d $REPO/{_run_of(db)[0]} -o {_run_of(db)[1]} -- {BENCH_CMD}",
        f"python3 bench.py --stall-summary {db}",
        "```",
        "",
        "The SQ counters are wave-cycles summed over all resident waves (quad-cycle units), so every column but the "
        "first two is a fraction of SQ_WAVE_CYCLES, the cycles the waves were resident:",
        "",
        "* `waves/SIMD` = 4 x SQ_WAVE_CYCLES / (GRBM_GUI_ACTIVE / 8 XCDs x 1024 SIMDs): mean resident waves per SIMD;",
        "* `issuing` = SQ_ACTIVE_INST_ANY (cycles a wave was executing some instruction); `valu`, `lds`, `vmem` = "
        "SQ_ACTIVE_INST_VALU (MFMA included), _LDS, _VMEM;",
        "* `wait dep` = SQ_WAIT_ANY (waiting at s_waitcnt or a barrier for memory, LDS or other waves); "
        "`wait issue` = SQ_WAIT_INST_ANY (ready but not issued: its unit busy, or a dependency on an unfinished "
        "instruction such as an MFMA in flight); `wait LDS issue` = SQ_WAIT_INST_LDS.",
        "",
        "The categories overlap (an issuing wave can also be waiting on another counter) and the hardware "
        "documents them as nondeterministic: read them as proportions, not as a partition.",
        "",
        "| workload | kernel | ms | waves/SIMD | issuing | valu | lds | vmem | wait dep | wait issue | wait LDS issue |",
        "|---|---|---|---|---|---|---|---|---|---|---|",
    ]
    rec = {}
    for (wl, slot), ds in sorted(groups.items()):
        m = {c: sum(val[d][c] for d in ds) / len(ds) for c in STALL_COUNTERS}
        ms = sum(dur[d] for d in ds) / len(ds) * 1e-6
        wc = max(1.0, m["SQ_WAVE_CYCLES"])
        cyc = m["GRBM_GUI_ACTIVE"] / XCDS
        row = {"ms": ms, "waves_per_simd": 4.0 * wc / max(1.0, cyc * CUS * SIMDS_PER_CU),
               "issuing": m["SQ_ACTIVE_INST_ANY"] / wc, "valu": m["SQ_ACTIVE_INST_VALU"] / wc,
               "lds": m["SQ_ACTIVE_INST_LDS"] / wc, "vmem": m["SQ_ACTIVE_INST_VMEM"] / wc,
               "wait_dep": m["SQ_WAIT_ANY"] / wc, "wait_issue": m["SQ_WAIT_INST_ANY"] / wc,
               "wait_lds_issue": m["SQ_WAIT_INST_LDS"] / wc, "counters": m}
        rec.setdefault(wl, {})[slot] = row
        lines.append(f"| {wl} | {slot} | {ms:.3f} | {row['waves_per_simd']:.2f} | " + " | ".join(
            f"{row[k]:.3f}" for k in ("issuing", "valu", "lds", "vmem", "wait_dep", "wait_issue", "wait_lds_issue"))
            + " |")
    lines += ["", "Raw counters per launch:", "", "| workload | kernel | " + " | ".join(STALL_COUNTERS) + " |",
              "|---|---|" + "---|" * len(STALL_COUNTERS)]
    for wl in sorted(rec):
        for slot, row in sorted(rec[wl].items()):
            lines.append(f"| {wl} | {slot} | " + " | ".join(f"{row['counters'][c]:.4g}" for c in STALL_COUNTERS) + " |")
    lines += ["", "Machine-readable line (the digest covers the kernel sources and build options):", ""]
    lines.append(json.dumps({"source_digest": source_digest(),
                             "per_launch": {wl: {s: {k: v for k, v in r.items() if k != "counters"}
                                                 for s, r in d.items()} for wl, d in rec.items()}}))
    with open(out, "w") as f:
        f.write("\n".join(lines) + "\n")
    print("\n".join(lines))


def trace_summary(db: str, timed: str, out: str):
    """Summarise a rocprofv3 --kernel-trace --stats run of this benchmark: per kernel the
    calls and durations, plus the mean of the timed launches of the bench step's main
    kernels (the last `steps` launches), next to what bench.py measured itself in that run
    (`timed`: its JSON output line)."""
    import sqlite3
    con = sqlite3.connect(db)
    rows = list(con.execute("select name, total_calls, total_duration, average, percentage from top_kernels"))
    bench = json.loads(open(timed).read().strip().splitlines()[-1])
    steps = bench["steps"]
    per = {}
    for name, dur in con.execute("select name, duration from kernels order by start"):
        per.setdefault(name, []).append(dur)
    lines = [
        "# Kernel trace: bench step (dense causal d = 128 fwd+bwd + paged decode page 16; then GEM s = 0.5 and "
        "broadcast-Q s = 0.5 extras)",
        "",
        "Command (repository root on the MI355X box; $REPO = that root):",
        "",
        "```",
        "cd /tmp && export TMPDIR=/tmp && timeout -s KILL 300 rocprofv3 --kernel-trace --stats -d "
        f"$REPO/{_run_of(db)[0]} -o {_run_of(db)[1]} -- python3 $REPO/bench.py --steps 10 --warmup 3 --cpu-sample 0 "
        f"--single-launch-steps 0 > $REPO/{timed}",
        f"python3 bench.py --trace-summary {db} {timed}",
        "```",
        "",
        "Per-kernel summary (top_kernels view of the rocpd database; all launches, warmup included):",
        "",
        "| kernel | calls | total (us) | average (us) | % of GPU time |",
        "|---|---|---|---|---|",
    ]
    for name, calls, tot, avg, pct in rows:
        short = name if len(name) <= 120 else name[:117] + "..."   # library kernels' template names run to pages
        lines.append(f"| `{short}` | {calls} | {tot:.1f} | {avg:.1f} | {pct:.2f} |")
    lines += ["", f"Timed launches of the step's main kernels (the first {steps} launches after the "
              f"warmup of each; bench.py's own HIP-event means from the same run beside them):", "",
              "| workload | kernel | trace mean (ms) | bench.py events (ms) |", "|---|---|---|---|"]
    warm = bench.get("warmup", 0)
    measured = {"dense_causal_d128": bench.get("kernels_ms", {}),
                "gem_s0.5": bench.get("gem_s0.5", {}).get("kernels_ms", {}),
                "bcast_s0.5": bench.get("bcast_s0.5", {}).get("kernels_ms", {})}
    for wl, slots in WORKLOAD_KERNELS.items():
        for slot, key in slots.items():
            durs = [d for n, ds in per.items() if key + "(" in n.replace("jfa::", "") for d in ds]
            if not durs:
                continue
            if wl in ("dense_causal_d128", "decode_ps16"):
                setup = 1 if slot in ("fwd", "decode") else 0   # the case's setup call launches these once
                t = durs[setup + warm:setup + warm + steps]
                ref = measured["dense_causal_d128"].get(slot)
            else:
                t = durs[-bench.get("extra_steps", 10):]
                ref = measured[wl].get(slot)
            lines.append(f"| {wl} | {slot} | {sum(t) / len(t) * 1e-6:.4f} | {ref if ref is not None else '-'} |")
    with open(out, "w") as f:
        f.write("\n".join(lines) + "\n")
    print("\n".join(lines))


def cpu_model() -> str:
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    import platform
    return platform.processor() or "unknown"


def cpu_baseline(inp, heads):
    """Time the fp64 oracle, as it stands, on a bounded sample of the headline workload:
    forward + backward of sequence 0 for the given heads (all its rows and keys)."""
    import oracle
    from threadpoolctl import threadpool_info
    L = int(inp.cu_q[1])
    cu = np.array([0, L])
    t0 = time.perf_counter()
    for h in heads:
        args = [x[:L, h:h + 1].astype(np.float64) for x in (inp.q, inp.k, inp.v, inp.do)]
        oracle.attention_forward(*args[:3], cu, cu, inp.causal)
        oracle.attention_backward(*args, cu, cu, inp.causal)
    dt = time.perf_counter() - t0
    pairs = pairs_of(cu, cu, inp.causal) * len(heads)
    flops = 14.0 * inp.q.shape[2] * pairs
    blas = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    affinity = len(os.sched_getaffinity(0))
    return {"value": flops / dt / 1e12, "unit": "TFLOP/s", "cores": int(min(blas, affinity)), "kind": "oracle",
            "affinity_cores": affinity, "blas_threads": int(blas), "cpu_model": cpu_model(),
            "sample": f"fp64 numpy oracle (BLAS matmuls on {blas} threads, the rest on one), fwd+bwd of sequence 0 "
                      f"(8192 causal rows) for {len(heads)} of 32 heads of the same dense causal workload, "
                      f"{pairs} visible query-key pairs; {dt:.1f} s wall"}


def _time_case(torch, jfa, case, steps, warmup):
    """fwd and bwd of one jagged case, `steps` times after `warmup`: mean ms of each call
    and of each main kernel (the library's caller-owned events on the launch stream)."""
    for _ in range(warmup):
        case.step()
    evs = [jfa.KernelEvents() for _ in range(steps)]
    marks = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(steps)]
    torch.cuda.synchronize()
    for i in range(steps):
        marks[i][0].record()
        case.fwd(evs[i])
        marks[i][1].record()
        case.bwd(evs[i])
        marks[i][2].record()
    torch.cuda.synchronize()
    f_ms = sum(m[0].elapsed_time(m[1]) for m in marks) / steps
    b_ms = sum(m[1].elapsed_time(m[2]) for m in marks) / steps
    kern = {s: sum(e.elapsed_ms(s) for e in evs) / steps for s in ("fwd", "bwd_dq", "bwd_dkdv")}
    return f_ms, b_ms, kern


def _pct(flops, ms):
    return round(100.0 * flops / (ms * 1e-3) / 1e12 / MFMA_BF16_PEAK_TFLOPS, 2)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--page-size", type=int, default=16)
    ap.add_argument("--extra-steps", type=int, default=10, help="timed calls of each extra workload (GEM, broadcast-Q)")
    ap.add_argument("--single-launch-steps", type=int, default=20,
                    help="timed calls of the decode in single-launch mode, after the steps (0 = skip)")
    ap.add_argument("--cpu-sample", type=int, default=16, help="heads of sequence 0 in the oracle timing sample (0 = skip)")
    ap.add_argument("--sweep", action="store_true", help="one JSON line per workload (GEM s, broadcast-Q, dense, decode)")
    ap.add_argument("--copy-calibration-mib", type=int, default=1024,
                    help="run one device copy of this size after timing (reference for HBM byte counters)")
    ap.add_argument("--gemm-probe", type=int, default=1,
                    help="time a library bf16 GEMM (8192^3) after the steps: the sustained MFMA rate (0 = skip)")
    ap.add_argument("--pmc-summary", nargs=2, metavar=("FETCH_DB", "WRITE_DB"),
                    help="summarise two rocprofv3 --pmc runs of this benchmark into the traffic profile and exit")
    ap.add_argument("--counter-summary", metavar="DB",
                    help="summarise a rocprofv3 --pmc run of the MFMA/LDS counters into the counter profile and exit")
    ap.add_argument("--stall-summary", metavar="DB",
                    help="summarise a rocprofv3 --pmc run of the wave-state counters into the stall profile and exit")
    ap.add_argument("--trace-summary", nargs=2, metavar=("DB", "BENCH_JSON"),
                    help="summarise a rocprofv3 --kernel-trace run of this benchmark and exit")
    args = ap.parse_args()
    if args.pmc_summary:
        return pmc_summary(*args.pmc_summary, args.copy_calibration_mib, TRAFFIC_PROFILE)
    if args.counter_summary:
        return counter_summary(args.counter_summary, COUNTER_PROFILE)
    if args.stall_summary:
        return stall_summary(args.stall_summary, STALL_PROFILE)
    if args.trace_summary:
        return trace_summary(*args.trace_summary,
                             os.path.join(ROOT, "profiles", "kernel_trace_bench_step_dense_causal_d128.md"))

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(json.dumps({"error": "this benchmark runs on one GPU only: --gpus must be 1 (there is no "
                                   "multi-GPU path; each GPU's share is the single-GPU workload)"}))
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
    dense_inp = workloads.dense_causal(0, head_dim=128)
    dec_inp = workloads.decode_paged(0, args.page_size, tail_fill=0.0)
    log(f"inputs generated in {time.time() - t0:.1f}s")
    jc = JaggedCase(torch, jfa, dense_inp)
    dc = DecodeCase(torch, jfa, dec_inp)

    for _ in range(args.warmup):
        jc.step()
        dc.step()
    torch.cuda.synchronize()

    evs = [jfa.KernelEvents() for _ in range(args.steps)]
    marks = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(args.steps)]
    torch.cuda.synchronize()
    t_start = time.perf_counter()
    for i in range(args.steps):
        marks[i][0].record()
        jc.fwd(evs[i])
        marks[i][1].record()
        jc.bwd(evs[i])
        marks[i][2].record()
        dc.step(evs[i])
        marks[i][3].record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t_start
    K = args.steps
    f_ms = sum(m[0].elapsed_time(m[1]) for m in marks) / K
    b_ms = sum(m[1].elapsed_time(m[2]) for m in marks) / K
    dec_ms = sum(m[2].elapsed_time(m[3]) for m in marks) / K
    kern = {s: sum(e.elapsed_ms(s) for e in evs) / K for s in ("fwd", "bwd_dq", "bwd_dkdv", "decode")}
    step_ms = wall * 1e3 / K

    tflops = (jc.fwd_flops + jc.bwd_flops) / ((f_ms + b_ms) * 1e-3) / 1e12
    dec_tbs = dc.bytes / (dec_ms * 1e-3) / 1e12
    dominant = max(jc.kernel_flops, key=lambda k: kern[k])
    ach = jc.kernel_flops[dominant] / (kern[dominant] * 1e-3) / 1e12
    names = {"fwd": "fwd_kernel (jagged forward)", "bwd_dkdv": "bwd_dkdv_kernel (key-stationary dK/dV)",
             "bwd_dq": "bwd_dq_kernel (query-stationary dQ)"}

    # extra workloads, timed after the steps (not part of `value`)
    extras = {}
    for name, make, bc in (("gem_s0.5", lambda: workloads.gem(0, 0.5), False),
                           ("bcast_s0.5", lambda: workloads.broadcast_q(0, 0.5), True)):
        x = make()
        case = JaggedCase(torch, jfa, bcast=x) if bc else JaggedCase(torch, jfa, x)
        del x
        ef, eb, ek = _time_case(torch, jfa, case, args.extra_steps, 3)
        extras[name] = {"fwd_ms": round(ef, 4), "bwd_ms": round(eb, 4),
                        "tflops": round((case.fwd_flops + case.bwd_flops) / ((ef + eb) * 1e-3) / 1e12, 2),
                        "fwd_pct_peak": _pct(case.fwd_flops, ef), "bwd_pct_peak": _pct(case.bwd_flops, eb),
                        "fwd_gflop": round(case.fwd_flops / 1e9, 2), "bwd_gflop": round(case.bwd_flops / 1e9, 2),
                        "kernels_ms": {k: round(v, 4) for k, v in ek.items()}}
        del case
        torch.cuda.empty_cache()

    # the same decode, back to back in both modes: split merge in a second launch
    # (the default, as in the steps) and inside the decode launch (single_launch)
    if args.single_launch_steps > 0:
        dc1 = DecodeCase(torch, jfa, dc.inp, single_launch=True)
        for mode, case in (("decode_two_launches", dc), ("decode_single_launch", dc1)):
            for _ in range(3):
                case.step()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            for _ in range(args.single_launch_steps):
                case.step()
            e1.record()
            torch.cuda.synchronize()
            ms1 = e0.elapsed_time(e1) / args.single_launch_steps
            extras[mode] = {"value": round(dc.bytes / (ms1 * 1e-3) / 1e12, 3), "unit": "TB/s", "ms": round(ms1, 4)}
        del dc1

    # plain device copy of known size: reference for FETCH_SIZE / WRITE_SIZE scaling,
    # and a measured HBM ceiling reported beside the published peak (never instead of it)
    copy_tbs = None
    if args.copy_calibration_mib > 0:
        n = args.copy_calibration_mib * (1 << 20) // 4
        src = torch.empty(n, dtype=torch.float32, device="cuda").fill_(1.0)
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(5):
            dst.copy_(src)
        e1.record()
        torch.cuda.synchronize()
        copy_tbs = round(2 * 4 * n * 5 / (e0.elapsed_time(e1) * 1e-3) / 1e12, 3)   # read + write bytes
        del src, dst

    # a library bf16 GEMM (8192^3, contiguous operands): the dense MFMA rate this GPU
    # sustains under its power limit, reported beside the published peak (never instead of it)
    gemm_tflops = None
    if args.gemm_probe:
        ga = torch.randn(8192, 8192, device="cuda").to(torch.bfloat16)
        gb = torch.randn(8192, 8192, device="cuda").to(torch.bfloat16)
        gc = torch.empty(8192, 8192, device="cuda", dtype=torch.bfloat16)
        for _ in range(5):
            torch.matmul(ga, gb, out=gc)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(10):
            torch.matmul(ga, gb, out=gc)
        e1.record()
        torch.cuda.synchronize()
        gemm_tflops = round(2 * 8192 ** 3 * 10 / (e0.elapsed_time(e1) * 1e-3) / 1e12, 1)
        del ga, gb, gc

    stored = stored_traffic("dense_causal_d128")
    traffic = round(stored[dominant]) if stored and dominant in stored else None

    cpu = None
    if args.cpu_sample > 0:
        cpu = cpu_baseline(dense_inp, list(range(min(args.cpu_sample, 32))))

    out = {
        "metric": METRIC,
        "value": round(tflops, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup,
        "ms_per_step": round(step_ms, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "pct_mfma_peak": round(100 * tflops / MFMA_BF16_PEAK_TFLOPS, 2),
        "config": {
            "workload": "dense causal jagged self-attention fwd+bwd, 4 x 8192 tokens, 32 heads, d = 128 "
                        "+ paged split-KV decode",
            "jagged": {"batch": 4, "seq_len": 8192, "heads": 32, "head_dim": 128, "total_tokens": 32768,
                       "causal": True, "fwd_gflop": round(jc.fwd_flops / 1e9, 2),
                       "bwd_gflop": round(jc.bwd_flops / 1e9, 2)},
            "decode": {"batch": 32, "heads_q": 32, "heads_kv": 8, "head_dim": 128, "page_size": args.page_size,
                       "splits": dc.nsplits, "kv_len": "U{4096..16384}", "gbytes": round(dc.bytes / 1e9, 4)},
        },
        "fwd_ms": round(f_ms, 4),
        "bwd_ms": round(b_ms, 4),
        "fwd_pct_peak": _pct(jc.fwd_flops, f_ms),
        "bwd_pct_peak": _pct(jc.bwd_flops, b_ms),
        "decode": {"value": round(dec_tbs, 3), "unit": "TB/s", "pct_hbm_peak": round(100 * dec_tbs * 1e3 / HBM_PEAK_GBS, 2),
                   "ms": round(dec_ms, 4)},
        "measured_hbm_copy_tbs": copy_tbs,
        "measured_bf16_gemm_tflops": gemm_tflops,
        "kernels_ms": {k: round(v, 4) for k, v in kern.items()},
        "extra_steps": args.extra_steps,
        **extras,
        "roofline": {"kernel": names[dominant], "bound": "mfma",
                     "achieved": round(ach, 2), "peak": MFMA_BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(ach / MFMA_BF16_PEAK_TFLOPS, 4), "traffic": traffic,
                     "algorithmic_flop_per_launch": jc.kernel_flops[dominant]},
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

    scrub = None

    def per_call(fn, n=20, w=5, cold=False):
        """Each call timed on its own (HIP events on the launch stream): (median, min) ms.
        cold: a 512 MB buffer is written before every call (outside the events), so the
        call finds none of its inputs in the 256 MB MALL."""
        nonlocal scrub
        if cold and scrub is None:
            scrub = torch.empty(512 << 20, dtype=torch.uint8, device="cuda")
        for _ in range(w):
            fn()
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(n)]
        for e0, e1 in ev:
            if cold:
                scrub.fill_(1)
            e0.record()
            fn()
            e1.record()
        torch.cuda.synchronize()
        t = sorted(e0.elapsed_time(e1) for e0, e1 in ev)
        return t[len(t) // 2], t[0]

    def roof(flops, nbytes, ms):
        """Roofline time of the work (MFMA or HBM bound) and the fraction of it reached."""
        t = max(flops / (MFMA_BF16_PEAK_TFLOPS * 1e9), nbytes / (HBM_PEAK_GBS * 1e6))
        return {"roofline_ms": round(t, 4), "bound": "hbm" if nbytes / HBM_PEAK_GBS * 1e3 > flops / MFMA_BF16_PEAK_TFLOPS
                else "mfma", "frac_of_roofline": round(t / ms, 3)}

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
        fwd_call = lambda: jfa.jfa_fwd(jc.q, jc.k, jc.v, jc.cq, jc.ck, jc.mq, jc.mk, jc.causal, broadcast_q=jc.bcast,
                                       out=jc.o, lse=jc.lse, workspace=jc.ws_f)
        bwd_call = lambda: jfa.jfa_bwd(jc.q, jc.k, jc.v, jc.o, jc.lse, jc.do, jc.cq, jc.ck, jc.mq, jc.mk, jc.causal,
                                       broadcast_q=jc.bcast, dq=jc.dq, dk=jc.dk, dv=jc.dv, workspace=jc.ws_b)
        # back to back (mean) first, which also warms the GPU up after the inputs were
        # written; then each call timed on its own: median (the reported time) and
        # min; the working sets near or within the MALL also cold
        f_b2b, b_b2b = timeit(fwd_call, w=5), timeit(bwd_call, w=5)
        f_ms, fmin = per_call(fwd_call)
        b_ms, bmin = per_call(bwd_call)
        line = {"workload": name, "fwd_ms": round(f_ms, 4), "bwd_ms": round(b_ms, 4),
                "fwd_tflops": round(jc.fwd_flops / f_ms / 1e9, 1), "bwd_tflops": round(jc.bwd_flops / b_ms / 1e9, 1),
                "fwd_pct_peak": round(100 * jc.fwd_flops / f_ms / 1e9 / MFMA_BF16_PEAK_TFLOPS, 2),
                "bwd_pct_peak": round(100 * jc.bwd_flops / b_ms / 1e9 / MFMA_BF16_PEAK_TFLOPS, 2),
                "fwd_ms_min": round(fmin, 4), "bwd_ms_min": round(bmin, 4),
                "fwd_ms_back_to_back": round(f_b2b, 4), "bwd_ms_back_to_back": round(b_b2b, 4),
                "fwd_gb": round(jc.fwd_bytes / 1e9, 3), "bwd_gb": round(jc.bwd_bytes / 1e9, 3),
                "fwd_roofline": roof(jc.fwd_flops, jc.fwd_bytes, f_ms),
                "bwd_roofline": roof(jc.bwd_flops, jc.bwd_bytes, b_ms)}
        if jc.fwd_bytes < 0.4e9:   # GEM and broadcast-Q at sparsity 0.9: near or within the 256 MB MALL
            fc, _ = per_call(fwd_call, cold=True)
            bc, _ = per_call(bwd_call, cold=True)
            line.update({"fwd_ms_cold": round(fc, 4), "bwd_ms_cold": round(bc, 4),
                         "fwd_roofline_cold": roof(jc.fwd_flops, jc.fwd_bytes, fc),
                         "bwd_roofline_cold": roof(jc.bwd_flops, jc.bwd_bytes, bc)})
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
        ws8 = torch.empty(max(1, jfa.jfa_fwd_workspace_size(q8, k8, jc.ck, jc.mq, jc.mk, jc.causal)),
                          dtype=torch.uint8, device="cuda")
        f8_ms = timeit(lambda: jfa.jfa_fwd(q8, k8, v8, jc.cq, jc.ck, jc.mq, jc.mk, jc.causal, out=jc.o, lse=jc.lse,
                                           workspace=ws8, **sc))
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
