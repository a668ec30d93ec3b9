"""Host-side logic of bench.py: the one-GPU guard, the algorithmic work counts that every
roofline fraction divides by, and the GEMM group statistics of the maxvio sweep."""
import os
import subprocess
import sys

import numpy as np

import bench
import workload as W

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr and r.stdout == ""


def _train_work(slot_rows=0):
    cfg = W.CONFIGS["train"]
    R, E, B, S, K = cfg.R, cfg.E, cfg.B, cfg.S, cfg.K
    Mr = R * S * K
    st = np.zeros(16, dtype=np.int64)
    cu = np.zeros((R, E + B + 1), dtype=np.int64)
    topk = np.zeros((R, S, K), dtype=np.int32)
    if slot_rows:
        st[2] = 1                              # one slot replica: rank 0, slot 0, of expert 5
        cu[0, E + 1:] = slot_rows
        topk.reshape(-1)[:slot_rows] = 5
    return cfg, bench.algorithmic_work(cfg, st, cu, np.arange(Mr), topk)


def test_algorithmic_work_matches_the_closed_forms():
    # R8 E256 S4096 K8 H7168 I2048: every token read once and written K times (dispatch), the
    # K expert rows read and one row written per token (combine); GEMMs count real rows only
    cfg, w = _train_work()
    assert round(w["dispatch"][1] / 1e9, 3) == 4.229
    assert round(w["combine"][1] / 1e9, 3) == 4.230
    assert round(w["dispatch_bwd"][1] / 1e9, 3) == 4.230   # + the float32 scale per pair
    mhi = cfg.R * cfg.S * cfg.K * cfg.H * cfg.I
    fwd = w["gemm_gate_up"][1] + w["gemm_down"][1]
    bwd = sum(w[k][1] for k in ("gemm_dact", "gemm_dx", "gemm_dw2", "gemm_dw13"))
    assert fwd == 6 * mhi and bwd == 12 * mhi
    assert round(fwd / 1e12, 2) == 23.09 and round(bwd / 1e12, 2) == 46.18
    assert w["reduce_grad"][1] == 0.0 and w["prefetch"][1] == 0.0


def test_one_slot_replica_costs_one_weight_copy_and_one_reduction():
    cfg, w = _train_work(slot_rows=7)
    nw = 3 * cfg.H * cfg.I
    assert w["prefetch"][1] == 2 * nw * 2             # bf16 weights read and written once
    assert w["reduce_grad"][1] == (8 + 8 * 1) * nw    # fp32 home grad read + written, replica read + cleared
    assert round(w["reduce_grad"][1] / 1e6) == 705


def test_group_stats():
    cu = np.array([[0, 0, 300, 300, 556, 556], [0, 100, 100, 100, 100, 100]])
    g = bench.group_stats(cu)
    # groups of 300, 256 and 100 rows -> 2 + 1 + 1 tiles of 256 rows, 656 real rows of 1024
    assert g == {"groups": 3, "row_tiles": 4, "padding_frac": round(1 - 656 / 1024, 4)}
    assert bench.group_stats(np.zeros((2, 4), dtype=np.int64))["groups"] == 0


def test_traffic_digest_ignores_comments_only():
    """Stored counter traffic stays valid across comment edits and is voided by a code change."""
    a = "int a = 1;  // one\nint b = 2;\n"
    b = "// header\nint a = 1;\n/* two\n   lines */\nint b = 2;   \n"
    assert bench._code_only(a) == bench._code_only(b)
    assert bench._code_only(a) != bench._code_only("int a = 3;\nint b = 2;\n")


def _write_pmc(d, counters, kernel, dispatches, start=1000):
    """A rocprofv3 -f csv counter_collection + kernel_trace pair: two instances per counter (the
    reducer sums them per dispatch), durations of 1 ms per dispatch."""
    import csv
    os.makedirs(d, exist_ok=True)
    with open(os.path.join(d, "p_counter_collection.csv"), "w", newline="") as f:
        w = csv.writer(f)
        w.writerow(["Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value"])
        for i in range(dispatches):
            for c, v in counters.items():
                w.writerow([i, kernel, c, v / 2])
                w.writerow([i, kernel, c, v / 2])
    with open(os.path.join(d, "p_kernel_trace.csv"), "w", newline="") as f:
        w = csv.writer(f)
        w.writerow(["Dispatch_Id", "Kernel_Name", "Start_Timestamp", "End_Timestamp"])
        for i in range(dispatches):
            w.writerow([i, kernel, start, start + 1_000_000])


def test_l2_reducer_on_synthetic_counters(tmp_path):
    """--l2-from: hit rate = hits / (hits + misses), reads in 128-byte requests, latency =
    outstanding-request cycles / requests, per GEMM call matched by its kernel name."""
    kernel = "void " + bench.KERNEL_NAMES["gemm_dw13"] + "(moonep::GemmArgs)"
    d1, d2 = str(tmp_path / "p1"), str(tmp_path / "p2")
    _write_pmc(d1, {"TCC_HIT_sum": 600.0, "TCC_MISS_sum": 400.0, "TCC_EA0_RDREQ_sum": 1e6,
                    "TCC_EA0_RDREQ_LEVEL_sum": 7e8}, kernel, 2)
    _write_pmc(d2, {"TCC_TAG_STALL_sum": 5.0, "TCC_EA0_WRREQ_sum": 2e6, "TCC_EA0_WRREQ_LEVEL_sum": 5e8,
                    "TCC_EA0_RDREQ_32B_sum": 0.0}, kernel, 2)
    rows = bench.l2_rows(d1, d2)
    assert len(rows) == 1
    r = rows[0]
    assert r["call"] == "gemm_dw13" and abs(r["ms"] - 1.0) < 1e-9
    assert abs(r["hit"] - 0.6) < 1e-12
    assert abs(r["read_GB"] - 1e6 * 128 / 1e9) < 1e-12
    assert abs(r["read_latency"] - 700.0) < 1e-9 and abs(r["write_latency"] - 250.0) < 1e-9
    assert r["tag_stall"] == 5.0
