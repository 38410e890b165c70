"""Host logic of bench.py (CPU): the one-GPU contract and the counter summaries.

The summaries read rocprofv3's SQLite output; here they read small databases of the
same schema written by the test, so the arithmetic (calibration scaling, per-launch
means, wave-state fractions) and the source-digest rule are checked without a GPU.
"""
import json
import os
import sqlite3
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402

FWD = "void jfa::" + bench.WORKLOAD_KERNELS["dense_causal_d128"]["fwd"] + "(jfa::FwdArgs)"
DKDV = "void jfa::" + bench.WORKLOAD_KERNELS["dense_causal_d128"]["bwd_dkdv"] + "(jfa::BwdArgs)"
COPY = "__amd_rocclr_copyBuffer"


def _counter_db(path, rows):
    """rows: (dispatch id, kernel name, duration ns, {counter: value}); each value is split
    over two instances, as rocprofv3 reports one row per counter instance."""
    con = sqlite3.connect(path)
    con.execute("create table counters_collection (kernel_name text, counter_name text, value real, "
                "dispatch_id integer, duration integer)")
    for disp, name, dur, counters in rows:
        for c, v in counters.items():
            for part in (0.25 * v, 0.75 * v):
                con.execute("insert into counters_collection values (?, ?, ?, ?, ?)", (name, c, part, disp, dur))
    con.commit()
    con.close()


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120, cwd=ROOT)
    assert r.returncode == 2
    line = json.loads(r.stdout.strip().splitlines()[-1])
    assert "one GPU" in line["error"]


def test_traffic_summary_scales_by_the_copy_calibration(tmp_path, monkeypatch):
    # the copy of 1 MiB: FETCH_SIZE reads half of it, WRITE_SIZE all of it (KiB)
    fetch_db, write_db = str(tmp_path / "fetch_results.db"), str(tmp_path / "write_results.db")
    _counter_db(fetch_db, [(1, FWD, 1000, {"FETCH_SIZE": 300.0}), (2, FWD, 1000, {"FETCH_SIZE": 500.0}),
                           (3, DKDV, 2000, {"FETCH_SIZE": 64.0}), (4, COPY, 10, {"FETCH_SIZE": 512.0})])
    _counter_db(write_db, [(1, FWD, 1000, {"WRITE_SIZE": 10.0}), (2, FWD, 1000, {"WRITE_SIZE": 30.0}),
                           (3, DKDV, 2000, {"WRITE_SIZE": 8.0}), (4, COPY, 10, {"WRITE_SIZE": 1024.0})])
    out = tmp_path / "traffic.txt"
    monkeypatch.setattr(bench, "source_digest", lambda: "digest-a")
    bench.pmc_summary(fetch_db, write_db, 1, str(out))
    rec = json.loads(out.read_text().strip().splitlines()[-1])
    assert rec["fetch_factor"] == pytest.approx(2.0) and rec["write_factor"] == pytest.approx(1.0)
    per = rec["bytes_per_launch"]["dense_causal_d128"]
    assert per["fwd"] == pytest.approx((400.0 * 2.0 + 20.0) * 1024.0)   # mean of the two launches
    assert per["bwd_dkdv"] == pytest.approx((64.0 * 2.0 + 8.0) * 1024.0)
    # the command quotes the databases it was given
    assert f"--pmc-summary {fetch_db} {write_db}" in out.read_text()

    # stored figures are reported only while the kernel sources still match
    monkeypatch.setattr(bench, "TRAFFIC_PROFILE", str(out))
    assert bench.stored_traffic("dense_causal_d128")["fwd"] == pytest.approx(per["fwd"])
    monkeypatch.setattr(bench, "source_digest", lambda: "digest-b")
    assert bench.stored_traffic("dense_causal_d128") is None


def test_wave_state_fractions(tmp_path, monkeypatch):
    db = str(tmp_path / "stall_results.db")
    cycles = 1_000_000.0    # GRBM_GUI_ACTIVE summed over 8 XCDs: 125000 cycles each
    wave_quads = 125000.0 * 256 * 4 / 4 * 2   # two resident waves per SIMD, in quad-cycles
    counters = {"SQ_WAVE_CYCLES": wave_quads, "SQ_ACTIVE_INST_ANY": 0.5 * wave_quads,
                "SQ_ACTIVE_INST_VALU": 0.25 * wave_quads, "SQ_ACTIVE_INST_LDS": 0.1 * wave_quads,
                "SQ_ACTIVE_INST_VMEM": 0.01 * wave_quads, "SQ_WAIT_ANY": 0.2 * wave_quads,
                "SQ_WAIT_INST_ANY": 0.3 * wave_quads, "SQ_WAIT_INST_LDS": 0.05 * wave_quads,
                "GRBM_GUI_ACTIVE": cycles}
    _counter_db(db, [(1, FWD, 50_000, counters)])
    out = tmp_path / "stall.md"
    monkeypatch.setattr(bench, "source_digest", lambda: "digest-a")
    bench.stall_summary(db, str(out))
    row = json.loads(out.read_text().strip().splitlines()[-1])["per_launch"]["dense_causal_d128"]["fwd"]
    assert row["waves_per_simd"] == pytest.approx(2.0)
    assert row["issuing"] == pytest.approx(0.5) and row["wait_issue"] == pytest.approx(0.3)
    assert row["wait_dep"] == pytest.approx(0.2) and row["lds"] == pytest.approx(0.1)


def test_mfma_summary_derived_columns(tmp_path, monkeypatch):
    """The library GEMM row: executed flops from the MOPS counter, clock from GRBM_GUI_ACTIVE
    over the 8 XCDs, MFMA busy over all 1024 SIMDs at that clock."""
    import types
    import numpy as np
    import workloads
    tiny = types.SimpleNamespace(cu_q=np.array([0, 4]), cu_k=np.array([0, 4]), causal=False,
                                 q=np.zeros((4, 1, 8)))
    for f in ("dense_causal", "gem", "broadcast_q"):
        monkeypatch.setattr(workloads, f, lambda *a, **k: tiny)
    db = str(tmp_path / "mfma_results.db")
    ms, ghz, busy = 1.0, 1.7, 0.7
    cyc = ghz * 1e9 * ms * 1e-3
    flops = 2.0 * 8192 ** 3
    counters = {c: 0.0 for c in bench.COUNTERS}
    counters.update({"SQ_INSTS_VALU_MFMA_MOPS_BF16": flops / 512.0, "GRBM_GUI_ACTIVE": 8 * cyc,
                     "SQ_VALU_MFMA_BUSY_CYCLES": busy * cyc * 1024, "SQ_INSTS_MFMA": flops / 32768.0,
                     "SQ_INSTS_LDS": 0.5 * flops / 32768.0})
    _counter_db(db, [(1, "Cijk_Ailk_Bljk_BBS_BH_test", int(ms * 1e6), counters)])
    out = tmp_path / "mfma.md"
    monkeypatch.setattr(bench, "source_digest", lambda: "digest-a")
    bench.counter_summary(db, str(out))
    row = json.loads(out.read_text().strip().splitlines()[-1])["per_launch"]["library_gemm_bf16_8192"]["gemm"]
    assert row["mfma_tflops"] == pytest.approx(flops / (ms * 1e-3) / 1e12)
    assert row["mfma_util"] == pytest.approx(row["mfma_tflops"] / bench.MFMA_BF16_PEAK_TFLOPS)
    assert row["clock_ghz"] == pytest.approx(ghz) and row["mfma_busy"] == pytest.approx(busy)
    assert row["exec_over_alg"] == pytest.approx(1.0) and row["lds_per_mfma"] == pytest.approx(0.5)
