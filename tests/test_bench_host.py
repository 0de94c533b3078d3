"""Host-side pieces of bench.py (no GPU): the one-GPU guard, the algorithmic
byte formula, and the counter summary that feeds the roofline's traffic."""
import csv
import json
import os
import subprocess
import sys

import pytest

import bench
from combine_ep_layout_07_amd.workloads import WORKLOADS

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout == ""


# Expected totals at each workload's expected row counts (N deduplicated
# entries, V valid lanes), worked out per stage by hand from the byte model:
# layout S*T*K*12 (+4 per lane for expand), scatter reads x and the ids,
# slots, weights and writes N staging rows with their records, the epilogue
# reads the N staging rows and writes the receive rows, combine reads the ids,
# weights and slots, the expert rows and writes the output.
@pytest.mark.parametrize("cfg,n,v,total,tol", [
    (1, 441, 512, 1.1e6, 0.05),
    (2, 26719, 32768, 1.657e9, 0.002),
    (3, 26719, 32768, 1.072e9, 0.002),
    (4, 35600, 65536, 1.31e9, 0.01),
    (5, 213755, 262144, 14.63e9, 0.002),
])
def test_algorithmic_bytes_match_the_worked_totals(cfg, n, v, total, tol):
    b = bench.alg_bytes(WORKLOADS[cfg], n, v)
    assert b["total"] == b["layout"] + b["scatter"] + b["epilogue"] + b["combine"]
    assert abs(b["total"] - total) / total < tol


def test_algorithmic_bytes_per_stage_dsv3_share():
    b = bench.alg_bytes(WORKLOADS[2], 26719, 32768)
    row = 7168 * 2
    assert b["layout"] == 4096 * 8 * 12
    assert b["scatter"] == 4096 * row + 4096 * 8 * 16 + 26719 * (row + 4 * 17)
    assert b["epilogue"] == 26719 * (row + 4 * 17) + 26719 * (row + 4 + 64)
    assert b["combine"] == 4096 * 8 * 16 + 26719 * row + 4096 * row
    d = bench.alg_bytes(WORKLOADS[2], 26719, 32768, direct=True)
    assert d["scatter"] == b["scatter"]
    assert d["epilogue"] == 26719 * 4 * 17 + 26719 * (4 + 64)


def test_source_digest_ignores_comments_only(tmp_path):
    a, b, c = tmp_path / "a.hip", tmp_path / "b.hip", tmp_path / "c.hip"
    a.write_text("// header\nint f(int x) { return x + 1; }  /* tail */\n")
    b.write_text("/* another\n header */\nint f(int x) {\n  return x + 1;  // same code\n}\n")
    c.write_text("int f(int x) { return x + 2; }\n")
    assert bench.source_digest([str(a)]) == bench.source_digest([str(b)])
    assert bench.source_digest([str(a)]) != bench.source_digest([str(c)])


def _counter_csv(path, counter, rows):
    with open(path, "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=["Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value"])
        w.writeheader()
        for i, (name, value) in enumerate(rows):
            w.writerow({"Dispatch_Id": i + 1, "Kernel_Name": name, "Counter_Name": counter, "Counter_Value": value})


def test_counter_summary_round_trip(tmp_path, monkeypatch):
    """Per-kernel traffic from two counter CSVs, scaled by the calibration copy,
    read back for the roofline, and invalidated by a code change to the
    kernel's sources (not by a comment)."""
    csrc = tmp_path / "csrc"
    csrc.mkdir()
    for f in ("ep_layout.hip", "ep_dispatch.hip", "ep_combine.hip", "ep_device.h", "ep_kernels.h", "ep_rows.h"):
        (csrc / f).write_text("int k;\n")
    monkeypatch.setattr(bench, "CSRC", str(csrc))
    monkeypatch.setattr(bench, "PROFILES", str(tmp_path))
    cal_kib = bench.COPY_CAL_BYTES / 1024
    epi = "void ep::(anonymous namespace)::k_epilogue_pf<14>(ep::DispatchArgs, int)"
    comb = "void ep::(anonymous namespace)::k_combine<2>(ep::CombineArgs)"
    fetch, write, js = tmp_path / "f.csv", tmp_path / "w.csv", tmp_path / "b.json"
    # FETCH_SIZE reads half the copy's bytes (scale 2), WRITE_SIZE all of them (scale 1); the run's
    # last five copies are the calibration, an earlier (larger) copy is the benchmark's own.
    cal = [("__amd_rocclr_copyBuffer", None)] * bench.COPY_CAL_REPS
    _counter_csv(fetch, "FETCH_SIZE", [("__amd_rocclr_copyBuffer", 3 * cal_kib), (epi, 1000.0), (epi, 1002.0),
                                       (comb, 500.0)] + [(n, cal_kib / 2) for n, _ in cal])
    _counter_csv(write, "WRITE_SIZE", [("__amd_rocclr_copyBuffer", 6 * cal_kib), (epi, 3000.0), (comb, 100.0)]
                 + [(n, cal_kib) for n, _ in cal])
    js.write_text("[bench] progress\n" + json.dumps({
        "config": {"workload": "dsv3_share: test"},
        "alg_bytes_per_step": {"layout": 1, "scatter": 2, "epilogue": 5000 * 1024, "combine": 1100 * 1024}}) + "\n")
    out = tmp_path / "dsv3_share_traffic.md"
    bench.summarize_counters(str(fetch), str(write), str(js), str(out), command="rocprofv3 --pmc ...")
    want = (1001.0 * 2 + 3000.0) * 1024
    assert bench.read_traffic("dsv3_share", "epilogue") == pytest.approx(want)
    assert bench.read_traffic("dsv3_share", "combine") == pytest.approx((500.0 * 2 + 100.0) * 1024)
    assert "| 1.0004 |" in out.read_text()  # epilogue traffic / algorithmic bytes
    (csrc / "ep_dispatch.hip").write_text("int k;  // a comment keeps the counters valid\n")
    assert bench.read_traffic("dsv3_share", "epilogue") == pytest.approx(want)
    (csrc / "ep_dispatch.hip").write_text("int k2;\n")
    assert bench.read_traffic("dsv3_share", "epilogue") is None
    assert bench.read_traffic("dsv3_share", "combine") is not None  # combine's sources did not change
    assert bench.read_traffic("other_workload", "epilogue") is None


def test_algorithmic_bytes_padding_and_bias_terms():
    w = WORKLOADS[2].with_(expand=True, alignment=128)
    base = bench.alg_bytes(w, 26719, 32768)
    padded = bench.alg_bytes(w, 26719, 32768, pad_rows=1000)
    assert padded["epilogue"] - base["epilogue"] == 1000 * (7168 * 2 + 8)
    assert padded["combine"] == base["combine"]          # padding rows are never combined
    b2 = bench.alg_bytes(WORKLOADS[2], 26719, 32768, n_bias=2)
    b0 = bench.alg_bytes(WORKLOADS[2], 26719, 32768)
    assert b2["combine"] - b0["combine"] == 2 * 4096 * 7168 * 2


def test_kernel_runs_split_back_to_back_from_in_step(tmp_path):
    p = tmp_path / "kt_kernel_trace.csv"
    epi, sc, cb = ("void ep::k_epilogue_pf<14>(ep::DispatchArgs, int)", "void ep::k_scatter<14>(ep::DispatchArgs)",
                   "void ep::k_combine<2>(ep::CombineArgs)")
    # two steps (scatter, epilogue 120 us, combine), then three epilogues back to
    # back of 130 us each with 2 us between them; rows deliberately out of order
    seq = [(sc, 0, 70), (epi, 71, 191), (cb, 192, 270), (sc, 300, 370), (epi, 371, 491), (cb, 492, 570),
           (epi, 600, 730), (epi, 732, 862), (epi, 864, 994)]
    with open(p, "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=["Kernel_Name", "Start_Timestamp", "End_Timestamp"])
        w.writeheader()
        for name, a, b in reversed(seq):
            w.writerow({"Kernel_Name": name, "Start_Timestamp": a * 1000, "End_Timestamp": b * 1000})
    g = bench.kernel_runs(str(p), lambda n: "k_epilogue_pf" in n)
    assert g["in_step"] == {"n": 2, "avg_us": 120.0}
    assert g["back_to_back"]["n"] == 3
    assert g["back_to_back"]["avg_us"] == pytest.approx(130.0)
    assert g["back_to_back"]["span_us_per_launch"] == pytest.approx(394 / 3)


def test_trace_summary_end_to_end(tmp_path):
    stats, trace, js, md = (tmp_path / "kt_kernel_stats.csv", tmp_path / "kt_kernel_trace.csv", tmp_path / "b.json",
                            tmp_path / "out.md")
    epi = "void ep::(anonymous namespace)::k_epilogue_pf<14>(ep::DispatchArgs, int)"
    with open(stats, "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=["Name", "Calls", "AverageNs", "MinNs", "MaxNs", "Percentage"])
        w.writeheader()
        w.writerow({"Name": epi, "Calls": 3, "AverageNs": 128000, "MinNs": 120000, "MaxNs": 134000, "Percentage": 52})
        w.writerow({"Name": "void at::native::fill", "Calls": 1, "AverageNs": 5, "MinNs": 5, "MaxNs": 5,
                    "Percentage": 1})
    with open(trace, "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=["Kernel_Name", "Start_Timestamp", "End_Timestamp"])
        w.writeheader()
        for name, a, b in [("void ep::k_scatter<14>(ep::DispatchArgs)", 0, 70), (epi, 70, 190),
                           ("void ep::k_combine<2>(ep::CombineArgs)", 190, 268), (epi, 300, 434), (epi, 434, 568)]:
            w.writerow({"Kernel_Name": name, "Start_Timestamp": a * 1000, "End_Timestamp": b * 1000})
    js.write_text("[bench] progress\n" + json.dumps({
        "config": {"workload": "dsv3_share: test"}, "value": 5900.0, "ms_per_step": 0.282,
        "stage_us": {"epilogue": 130.0, "epilogue_back_to_back": 134.5},
        "roofline": {"kernel": "k_epilogue_pf (epilogue)", "stage": "epilogue", "achieved": 5731.0, "frac": 0.716,
                     "alg_bytes_per_launch": 770844464, "timing": "events"}}) + "\n")
    bench.summarize_trace(str(stats), str(js), str(md), command="rocprofv3 --kernel-trace --stats ...")
    text = md.read_text()
    assert "| `void ep::k_epilogue_pf<14>(ep::DispatchArgs, int)` | 3 | 128.00 |" in text
    assert "at::native" not in text                                   # library kernels only
    assert "| back to back (roofline loop) | 2 | 134.00 | 134.00 | 134.5 |" in text
    assert "| inside steps | 1 | 120.00 |" in text
    assert "5752.6 GB/s = 71.9% of 8 TB/s" in text                     # 770844464 B / 134 us (back to back)


def test_cpu_baseline_legs_on_the_tiny_workload(monkeypatch):
    """Both CPU legs run the unthreaded oracle; the all-cores leg uses the
    threads the host grants and checks every thread's result against the
    one-thread pass."""
    from combine_ep_layout_07_amd.workloads import generate, seed_for
    monkeypatch.setenv("OMP_NUM_THREADS", "3")
    w = WORKLOADS[1]
    inputs = generate(w, seed_for(1))
    import oracle
    lay = oracle.layout(w.S, w.T, w.K, w.E, w.R, w.Nmax, inputs["topk_idx"])
    n = int(lay["recv_base"][-1])
    r = bench.cpu_baseline(w, inputs, n, int(((inputs["topk_idx"] >= 0) & (inputs["topk_idx"] < w.E)).sum()),
                           budget_s=0.3, all_cores_wall_s=0.2)
    assert r["kind"] == "oracle" and r["unit"] == "GB/s"
    assert r["cores"] == min(3, r["host"]["affinity_cpus"]) and r["host"]["threads"] == r["cores"]
    assert r["single_thread"]["cores"] == 1 and r["single_thread"]["value"] > 0 and r["value"] > 0
    assert "bitwise equal to the one-thread pass" in r["sample"]
    assert r["host"]["model"] and r["host"]["os_cpu_count"] >= 1
