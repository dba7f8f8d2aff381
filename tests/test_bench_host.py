"""bench.py's host logic on the CPU: the one-GPU refusal, the algorithmic
flop count, and the rocprofv3 summaries the committed profiles come from
(kernel-trace statistics, counter tables, HBM bytes scaled by the
calibration copy, MFMA occupancy and clock), each on small synthetic CSV
files whose answers are worked out by hand here."""
import csv
import os
import subprocess
import sys

import pytest

import bench
from inputs.configs import WORKLOADS

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _write_csv(path, rows):
    os.makedirs(os.path.dirname(path), exist_ok=True)
    with open(path, "w", newline="") as f:
        wr = csv.DictWriter(f, fieldnames=list(rows[0]))
        wr.writeheader()
        wr.writerows(rows)


def _counter_rows(kernel, dispatch0, values):
    """One row per (dispatch, counter): values is a list of {counter: value}."""
    rows = []
    for i, vals in enumerate(values):
        for name, val in vals.items():
            rows.append({"Dispatch_Id": dispatch0 + i, "Kernel_Name": kernel, "Counter_Name": name,
                         "Counter_Value": val})
    return rows


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, "bench.py", "--gpus", "2"], cwd=ROOT, capture_output=True, text=True,
                       timeout=300)
    assert r.returncode == 2, r
    assert "one GPU" in r.stderr and r.stdout == ""


def test_algorithmic_flops_counts_visible_pairs():
    # 4*d flops per visible (query, key) pair: S^2 pairs, or S(S+1)/2 causal
    assert bench.algorithmic_flops(1, 4, 1, 1, False) == 4 * 16
    assert bench.algorithmic_flops(1, 4, 1, 1, True) == 4 * 10
    assert bench.algorithmic_flops(2, 3, 5, 7, True) == 4 * 2 * 5 * 7 * 6
    w = WORKLOADS["encoder_s32k"]
    assert bench.algorithmic_flops(w.B, w.S, 8, w.d, w.causal) == 4 * 8 * 128 * 32768 ** 2


def test_trace_summary_statistics(tmp_path):
    # kernel A: 2 warm-up launches then durations 1, 3, 2 ms; kernel B ignored by the pattern
    rows, t = [], 0
    for dur_ms in (9.0, 9.0, 1.0, 3.0, 2.0):
        rows.append({"Kernel_Name": "attn_fwd_bf16<128>", "Start_Timestamp": t,
                     "End_Timestamp": t + int(dur_ms * 1e6)})
        t += 10 ** 8
    rows.append({"Kernel_Name": "other", "Start_Timestamp": 0, "End_Timestamp": 5})
    _write_csv(str(tmp_path / "run" / "kt_kernel_trace.csv"), rows)
    out = bench.summarize_trace(str(tmp_path), "attn_fwd", 2, flops=2.0e12)
    line = [ln for ln in out.splitlines() if ln.startswith("| attn_fwd_bf16<128>")]
    assert line == ["| attn_fwd_bf16<128> | 5 | 3 | 2.0000 | 2.0000 | 1.0000 | 3.0000 |"], out
    assert "other" not in out
    # 2e12 flop in 2 ms on the mean: 1000 TFLOP/s
    assert "1000.0 TFLOP/s on the mean" in out
    # --count takes the launches after the skipped ones
    out2 = bench.summarize_trace(str(tmp_path), "attn_fwd", 2, count=2)
    assert "| attn_fwd_bf16<128> | 5 | 2 | 2.0000 | 3.0000 | 1.0000 | 3.0000 |" in out2


def test_traffic_scaled_by_the_calibration_copy(tmp_path):
    w = WORKLOADS["encoder_s32k"]
    kern = "attn_fwd_bf16<128, false, 8, 128, 1>"
    copy = "__amd_rocclr_copyBuffer"
    # the 1 GiB copy reads 2^20 KiB but its counter shows half: factor 2;
    # writes show a quarter: factor 4
    fetch = (_counter_rows(kern, 1, [{"FETCH_SIZE": 1.0e6}, {"FETCH_SIZE": 100.0}, {"FETCH_SIZE": 200.0}])
             + _counter_rows(copy, 10, [{"FETCH_SIZE": 2.0 ** 19}]))
    write = (_counter_rows(kern, 1, [{"WRITE_SIZE": 1.0e6}, {"WRITE_SIZE": 30.0}, {"WRITE_SIZE": 50.0}])
             + _counter_rows(copy, 10, [{"WRITE_SIZE": 2.0 ** 18}]))
    _write_csv(str(tmp_path / "f" / "a_counter_collection.csv"), fetch)
    _write_csv(str(tmp_path / "w" / "b_counter_collection.csv"), write)
    out = bench.traffic_summary(str(tmp_path / "f"), str(tmp_path / "w"), "attn_fwd", 1, w, "sqa")
    # after the skipped first dispatch: reads 150 KiB x 2, writes 40 KiB x 4
    want = 150 * 1024 * 2 + 40 * 1024 * 4
    got = float([ln for ln in out.splitlines() if ln.startswith("hbm_bytes_per_launch:")][0].split()[1])
    assert got == pytest.approx(want, rel=1e-4)
    assert f"kernel_source_sha256_16: {bench.kernel_source_hash()}" in out
    assert "calibration factor 2.000" in out and "calibration factor 4.000" in out


def test_counter_table_means_after_warmups(tmp_path):
    rows = _counter_rows("k", 5, [{"C": 100.0, "D": 1.0}, {"C": 1.0, "D": 2.0}, {"C": 3.0, "D": 4.0}])
    _write_csv(str(tmp_path / "c" / "x_counter_collection.csv"), rows)
    per, cal = bench.summarize_counters([str(tmp_path / "c")], "k", 1)
    assert per == {"C": [1.0, 3.0], "D": [2.0, 4.0]} and cal == {}
    md = bench.counters_markdown(per, cal)
    assert "| C | 2 | 2.00000e+00 |" in md and "| D | 2 | 3.00000e+00 |" in md


def test_mfma_summary_share_and_clock(tmp_path):
    w = WORKLOADS["encoder_s32k"]
    flops = bench.algorithmic_flops(w.B, w.S, 8, w.d, w.causal)
    launch_ms = 4.0
    # 8 XCDs active for 2e6 cycles each over 4 ms: 0.5 GHz; 1024 SIMDs busy
    # 1.5e6 cycles each: 75 % of the active cycles
    vals = {"SQ_VALU_MFMA_BUSY_CYCLES": 1024 * 1.5e6, "SQ_BUSY_CYCLES": 1.0, "GRBM_GUI_ACTIVE": 8 * 2.0e6,
            "GRBM_COUNT": 1.0, "SQ_INSTS_VALU_MFMA_MOPS_BF16": flops / 512}
    _write_csv(str(tmp_path / "m" / "x_counter_collection.csv"), _counter_rows("attn_fwd_bf16", 1, [vals]))
    out = bench.mfma_summary(str(tmp_path / "m"), "attn_fwd", 0, w, "sqa", launch_ms)
    assert "MFMA busy share of active cycles: 75.0 %" in out
    assert "0.500 GHz" in out
    assert f"algorithmic {flops:.4e} (1.000x)" in out


def test_traffic_from_profile_follows_the_kernel_source(tmp_path, monkeypatch):
    prof = tmp_path / "profiles"
    prof.mkdir()
    path = prof / "attn_fwd_bf16_encoder_s32k_sqa_counters.md"
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    assert bench.traffic_from_profile("encoder_s32k", "sqa") is None        # no summary
    # the hash is taken over the kernel sources under ROOT: give the temporary
    # root a copy of them
    for rel in bench.KERNEL_SOURCES:
        dst = tmp_path / rel
        dst.parent.mkdir(parents=True, exist_ok=True)
        dst.write_bytes(open(os.path.join(ROOT, rel), "rb").read())
    h = bench.kernel_source_hash()
    path.write_text(f"kernel_source_sha256_16: {h}\nhbm_bytes_per_launch: 1.2500e+08\n")
    assert bench.traffic_from_profile("encoder_s32k", "sqa") == 1.25e8
    path.write_text("kernel_source_sha256_16: 0000000000000000\nhbm_bytes_per_launch: 1.2500e+08\n")
    assert bench.traffic_from_profile("encoder_s32k", "sqa") is None        # taken on another source
