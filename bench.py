"""Benchmark of the deterministic EP dispatch + combine hot path on one MI355X.

One step = layout + dispatch (scatter + copy epilogue) + combine over one batch
of seeded synthetic input already resident in HBM, enqueued as
ep_layout_dispatch (ep_layout then ep_dispatch; one kernel for a small single
source) and ep_combine.  The headline is
the DeepSeek-V3-like share of the deterministic-dispatch page's benchmark
(T=4096 tokens, hidden 7168 bf16, top-8 of 256 experts on 16 ranks, Nmax=4096,
compact layout).  Prints ONE JSON line: effective HBM GB/s on the algorithmic
bytes of the step, the same figures for every workload (``configs``), the
roofline of the dominant kernel, the cold-cache per-stage protocol, and the CPU
oracle timed on the host (one thread and all of the host's cores).

Consecutive steps rotate over two complete buffer sets (inputs, layout tables,
staging, receive rows, expert outputs, output), so no step finds the previous
step's rows still in the Infinity Cache.

    python bench.py [--steps K] [--warmup W] [--gpus 1] [--config 2] [--no-cpu-baseline] ...
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import re
import sys
import threading
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_HBM_GBPS = 8000.0  # MI355X HBM3E
METRIC = "dispatch+combine effective HBM GB/s (% of peak) at T=4096,H=7168,K=8"
PROFILES = os.path.join(ROOT, "profiles")
CSRC = os.path.join(ROOT, "combine_ep_layout_07_amd", "csrc")
STAGES = ["layout", "scatter", "epilogue", "combine"]
N_SETS = 2  # buffer sets the timed steps rotate over
# The other workloads' lines time at least this long (more steps than K when a
# step is short): the headline times exactly K steps.
MIN_TIMED_MS = 20.0
# Kernel sources per stage: a change to any of them invalidates that stage's
# stored HBM counters.
STAGE_SOURCES = {
    "layout": ["ep_layout.hip", "ep_device.h", "ep_kernels.h"],
    "scatter": ["ep_dispatch.hip", "ep_rows.h", "ep_device.h", "ep_kernels.h"],
    "epilogue": ["ep_dispatch.hip", "ep_rows.h", "ep_device.h", "ep_kernels.h"],
    "combine": ["ep_combine.hip", "ep_device.h", "ep_kernels.h"],
}
ALL_SOURCES = ["ep_layout.hip", "ep_dispatch.hip", "ep_combine.hip", "ep_api.cpp", "ep_device.h", "ep_kernels.h",
               "ep_rows.h"]


def alg_bytes(w, n_rows: int, v_rows: int, direct: bool = False, pad_rows: int = 0, n_bias: int = 0) -> dict:
    """Algorithmic bytes per stage: each mandatory input read and output write once.

    Rw row bytes, F scale bytes per row, M = 4(1+2K) staging metadata bytes,
    Y = 2H expert-output row bytes; N deduplicated rows, V valid lanes.  With
    Direct Recv X the scatter writes the hidden rows to recv_x (same bytes) and
    the epilogue moves only scales and metadata.  Expand padding rows (expert
    alignment > 1) are written like expand rows; each bias tensor adds one
    [S][T][H] bf16 read to the combine."""
    S, T, K, H = w.S, w.T, w.K, w.H
    Rw = H if w.dtype == "fp8" else 2 * H
    F = (H // 128) * 4 if w.dtype == "fp8" else 0
    M = 4 * (1 + 2 * K)
    Y = 2 * H
    lanes = S * T * K
    layout = lanes * (8 + 4) + (lanes * 4 if w.expand else 0)
    scatter = S * T * (Rw + F) + lanes * 16 + n_rows * (Rw + F + M)
    if direct:
        epilogue = n_rows * (F + M) + n_rows * (F + 4 + 8 * K)
    else:
        epilogue = n_rows * (Rw + F + M) + ((v_rows + pad_rows) * (Rw + F + 8) if w.expand
                                            else n_rows * (Rw + F + 4 + 8 * K))
    combine = lanes * 16 + (v_rows if w.expand else n_rows) * Y + S * T * Y + n_bias * S * T * Y
    return dict(layout=layout, scatter=scatter, epilogue=epilogue, combine=combine,
                total=layout + scatter + epilogue + combine)


def source_digest(paths) -> str:
    """Hash of the kernel sources with comments and whitespace removed, so that
    only a change of code (not of its comments) invalidates stored counters."""
    h = hashlib.sha256()
    for p in paths:
        with open(p) as f:
            text = f.read()
        text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
        text = re.sub(r"//[^\n]*", " ", text)
        h.update(" ".join(text.split()).encode())
    return h.hexdigest()[:16]


def stage_digest(stage: str) -> str:
    return source_digest([os.path.join(CSRC, f) for f in STAGE_SOURCES[stage]])


def library_identity() -> dict:
    """Which libep.so this run loaded: its path, a hash of the file, and the
    digest of the kernel and ABI sources in the tree."""
    import combine_ep_layout_07_amd.ep as ep
    with open(ep.LIB_PATH, "rb") as f:
        so = hashlib.sha256(f.read()).hexdigest()[:16]
    path = os.path.relpath(ep.LIB_PATH, ROOT) if ep.LIB_PATH.startswith(ROOT) else ep.LIB_PATH
    return {"path": path, "so_sha256_16": so, "sources_digest": source_digest([os.path.join(CSRC, f)
                                                                                for f in ALL_SOURCES]),
            "overridden_by_env": bool(os.environ.get("EP_LIBRARY"))}


def traffic_file(workload_name: str) -> str:
    return os.path.join(PROFILES, f"{workload_name}_traffic.md")


def read_traffic(workload_name: str, stage: str):
    """HBM bytes per launch of a stage's kernel from the committed rocprofv3
    counter summary of the workload, or None when the summary is missing or
    the kernel's sources changed since the counters were taken."""
    path = traffic_file(workload_name)
    if not os.path.exists(path):
        return None
    m = re.search(r"^\| %s \| [^|]+ \| [^|]+ \| [^|]+ \| ([0-9]+) \| [^|]+ \| [^|]+ \| ([0-9a-f]{16}) \|$"
                  % re.escape(stage), open(path).read(), flags=re.M)
    if not m or m.group(2) != stage_digest(stage):
        return None
    return float(m.group(1))


def host_cpus() -> dict:
    """The host's CPU model and the threads this process may use: the CPU
    affinity, capped by OMP_NUM_THREADS when it is set (the share of the host a
    job on it is given)."""
    model = "unknown"
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    try:
        affinity = len(os.sched_getaffinity(0))
    except AttributeError:
        affinity = os.cpu_count() or 1
    threads = affinity
    omp = os.environ.get("OMP_NUM_THREADS", "")
    if omp.isdigit() and int(omp) > 0:
        threads = min(threads, int(omp))
    return {"model": model, "os_cpu_count": os.cpu_count(), "affinity_cpus": affinity, "threads": threads}


def cpu_baseline(w, inputs, n_rows, v_rows, budget_s=6.0, all_cores_wall_s=1.5):
    """The oracle as it stands (plain single-threaded C) on the same workload:
    whole passes of layout + dispatch + combine on host arrays, about 30 s of
    CPU work in all.

    Leg 1, one thread: passes until about budget_s of CPU time; the median pass
    gives the rate.  Leg 2, all of the host's cores: one Python thread per core,
    each running the same whole passes independently (ctypes releases the GIL
    during every oracle call) until all_cores_wall_s of wall time (each thread
    finishes the pass it is in); the rate is all passes' bytes over the wall
    time, and every thread's first pass must equal the one-thread pass bit for
    bit.  The oracle itself stays unthreaded."""
    import numpy as np

    import oracle
    from combine_ep_layout_07_amd.workloads import draw_expert_outputs

    oracle.build(force=False)
    rows = n_rows if not w.expand else v_rows
    y = draw_expert_outputs(rows, w.H, 99)
    fp8 = w.dtype == "fp8"

    def one_pass():
        lay = oracle.layout(w.S, w.T, w.K, w.E, w.R, w.Nmax, inputs["topk_idx"], w.expand, w.alignment)
        disp = oracle.dispatch(w.S, w.T, w.H, w.K, w.E, w.R, w.Nmax, fp8, w.expand, w.alignment, inputs["x"],
                               inputs.get("x_sf"), inputs["topk_idx"], inputs["topk_weights"], lay)
        out = oracle.combine(w.S, w.T, w.H, w.K, w.E, w.R, w.Nmax, w.expand, inputs["topk_idx"],
                             inputs["topk_weights"], lay, y)
        keep = dict(lay)
        keep.update({k: v for k, v in disp.items() if k.startswith("recv_")}, out=out)
        return keep

    def same(a, b):
        return a.keys() == b.keys() and all(np.array_equal(a[k], b[k]) for k in a)

    times, ref = [], None
    while len(times) < 3 or sum(times) < budget_s:
        t0 = time.perf_counter()
        res = one_pass()
        times.append(time.perf_counter() - t0)
        if ref is None:
            ref = res
        del res
    t1 = float(np.median(times))
    b = alg_bytes(w, n_rows, v_rows)["total"]

    host = host_cpus()
    nthr = host["threads"]
    counts = [0] * nthr
    agree = [None] * nthr
    errors = []
    start = time.perf_counter()
    deadline = start + all_cores_wall_s

    def worker(i):
        try:
            while True:
                res = one_pass()
                if agree[i] is None:
                    agree[i] = same(res, ref)
                del res
                counts[i] += 1
                if time.perf_counter() >= deadline:
                    break
        except Exception as exc:  # reported in the JSON line, never swallowed silently
            errors.append(repr(exc))

    threads = [threading.Thread(target=worker, args=(i,)) for i in range(nthr)]
    for t in threads:
        t.start()
    for t in threads:
        t.join()
    wall = time.perf_counter() - start
    n_pass = sum(counts)
    if errors or not all(agree):
        raise RuntimeError(f"all-cores oracle leg: errors {errors}, results equal to the one-thread pass {agree}")
    all_gbps = b * n_pass / wall / 1e9
    sample = (f"full {w.name} workload (S={w.S} T={w.T} H={w.H} K={w.K}), whole layout+dispatch+combine passes on "
              f"host arrays; all cores: {nthr} threads each running independent passes of the unthreaded oracle, "
              f"{n_pass} passes in {wall:.1f} s wall, every thread's first pass bitwise equal to the one-thread "
              f"pass; one thread: median of {len(times)} passes of {t1:.2f} s ({sum(times):.1f} s of CPU work)")
    return {"value": round(all_gbps, 3), "unit": "GB/s", "cores": nthr, "kind": "oracle", "sample": sample,
            "tokens_per_s": round(w.S * w.T * n_pass / wall, 1), "host": host,
            "single_thread": {"value": round(b / t1 / 1e9, 3), "unit": "GB/s", "cores": 1,
                              "seconds_per_step": round(t1, 3), "tokens_per_s": round(w.S * w.T / t1, 1),
                              "passes": len(times)},
            "speedup_all_cores_vs_one": round(all_gbps / (b / t1 / 1e9), 2)}


COPY_CAL_BYTES = 256 * 2**20
COPY_CAL_REPS = 5


def copy_calibration(reps=COPY_CAL_REPS):
    """A plain device-to-device copy of COPY_CAL_BYTES, the reference the HBM
    byte counters are scaled by (it reads and writes exactly that many bytes)."""
    import torch
    src = torch.ones(COPY_CAL_BYTES, dtype=torch.uint8, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(reps):
        dst.copy_(src)
    torch.cuda.synchronize()


def _counter_rows(path):
    import csv
    with open(path) as f:
        return list(csv.DictReader(f))


def kernel_stage(name: str):
    """Stage a libep kernel belongs to (None for other kernels)."""
    if "ep::" not in name:
        return None
    if "k_layout" in name:
        return "layout"
    if "k_scatter" in name:
        return "scatter"
    if "k_epilogue" in name or "k_expand_padding" in name:
        return "epilogue"
    if "k_combine" in name:
        return "combine"
    return None


def _last_json(path):
    with open(path) as f:
        return json.loads([ln for ln in f.read().strip().splitlines() if ln.startswith("{")][-1])


def summarize_counters(fetch_csv: str, write_csv: str, bench_json: str, out_md: str, command: str) -> None:
    """Turn two rocprofv3 --pmc counter CSVs (FETCH_SIZE, WRITE_SIZE; KiB per
    dispatch) and the JSON line bench.py printed in the same run into the
    per-kernel traffic summary read by read_traffic()."""
    import numpy as np

    def per_kernel(path, counter):
        acc = {}
        for r in _counter_rows(path):
            if r.get("Counter_Name") != counter:
                continue
            acc.setdefault(r["Kernel_Name"], []).append(float(r["Counter_Value"]))
        return acc

    fetch, write = per_kernel(fetch_csv, "FETCH_SIZE"), per_kernel(write_csv, "WRITE_SIZE")
    b = _last_json(bench_json)
    alg = b["alg_bytes_per_step"]

    def calibration(path, counter):
        # The calibration copies (torch's device-to-device copy runs the
        # runtime's copyBuffer kernel) are the run's last COPY_CAL_REPS copy
        # dispatches; earlier ones (the benchmark's own buffer copies) differ
        # in size.  Median over them.
        rows = [r for r in _counter_rows(path) if r.get("Counter_Name") == counter and "copyBuffer" in r["Kernel_Name"]]
        rows.sort(key=lambda r: int(r.get("Dispatch_Id") or 0))
        vals = [float(r["Counter_Value"]) for r in rows[-COPY_CAL_REPS:]]
        return float(np.median(vals)) if vals else float("nan")

    cf, cw = calibration(fetch_csv, "FETCH_SIZE"), calibration(write_csv, "WRITE_SIZE")
    f_scale = COPY_CAL_BYTES / (cf * 1024.0)
    w_scale = COPY_CAL_BYTES / (cw * 1024.0)
    lines = [
        f"# HBM traffic per kernel launch ({b['config']['workload']})",
        "",
        "Counters from two rocprofv3 --pmc runs (FETCH_SIZE, then WRITE_SIZE), KiB per dispatch, median over",
        "each kernel's dispatches; scaled by what the same counters read for a plain device copy of 256 MiB",
        "(the run's calibration copy). alg = the stage's algorithmic bytes of the bench line of the same run.",
        "",
        "command: " + command,
        "",
        f"copy_fetch_kib_per_dispatch: {cf:.1f}",
        f"copy_write_kib_per_dispatch: {cw:.1f}",
        f"fetch_scale: {f_scale:.4f}",
        f"write_scale: {w_scale:.4f}",
        "",
        "| stage | kernel | fetch KiB | write KiB | traffic bytes per launch | alg bytes per launch | traffic / alg "
        "| kernel sources digest |",
        "|---|---|---|---|---|---|---|---|",
    ]
    for k in sorted(set(fetch) | set(write)):
        st = kernel_stage(k)
        if st is None or st == "layout":
            continue
        fk = float(np.median(fetch.get(k, [np.nan])))
        wk = float(np.median(write.get(k, [np.nan])))
        traffic = fk * 1024.0 * f_scale + wk * 1024.0 * w_scale
        short = re.sub(r"\(anonymous namespace\)::", "", k)[:70]
        lines.append(f"| {st} | `{short}` | {fk:.1f} | {wk:.1f} | {traffic:.0f} | {alg[st]} | "
                     f"{traffic / alg[st]:.4f} | {stage_digest(st)} |")
    os.makedirs(os.path.dirname(out_md) or ".", exist_ok=True)
    with open(out_md, "w") as f:
        f.write("\n".join(lines) + "\n")
    print("\n".join(lines))


def kernel_runs(trace_csv: str, match) -> dict:
    """Dispatches of the kernels `match(name)` accepts in a rocprofv3 kernel
    trace (kernel_trace.csv), split by what ran around them: "back_to_back" =
    launches in a run of two or more consecutive such dispatches (bench.py's
    roofline loop), "in_step" = the rest.  For each group: count, mean
    duration (us) and, for the back-to-back runs, the mean time per launch from
    the first start to the last end of each run, the interval the bench's two
    HIP events bracket."""
    rows = sorted(_counter_rows(trace_csv), key=lambda r: int(r["Start_Timestamp"]))
    hit = [match(r["Kernel_Name"]) for r in rows]
    groups = {"back_to_back": [], "in_step": []}
    spans = []
    i = 0
    while i < len(rows):
        if not hit[i]:
            i += 1
            continue
        j = i
        while j + 1 < len(rows) and hit[j + 1]:
            j += 1
        run = rows[i:j + 1]
        durs = [(int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3 for r in run]
        if len(run) >= 2:
            groups["back_to_back"] += durs
            spans.append(((int(run[-1]["End_Timestamp"]) - int(run[0]["Start_Timestamp"])) / 1e3, len(run)))
        else:
            groups["in_step"] += durs
        i = j + 1
    out = {k: {"n": len(v), "avg_us": (sum(v) / len(v)) if v else None} for k, v in groups.items()}
    n_span = sum(n for _, n in spans)
    out["back_to_back"]["span_us_per_launch"] = (sum(s for s, _ in spans) / n_span) if n_span else None
    return out


def summarize_trace(stats_csv: str, bench_json: str, out_md: str, command: str) -> None:
    """Turn a rocprofv3 --kernel-trace --stats summary (kernel_stats.csv) and the
    JSON line bench.py printed in the same run into a short markdown summary;
    with the run's kernel_trace.csv beside the stats file, the roofline
    kernel's back-to-back launches (the ones bench.py's roofline times) are
    also summarised on their own."""
    rows = [r for r in _counter_rows(stats_csv) if "ep::" in r["Name"]]
    b = _last_json(bench_json)
    roof = b["roofline"]
    lines = [f"# Kernel trace: {b['config']['workload']}", "", "command: " + command, "",
             "rocprofv3 --stats summary (kernel_stats.csv), libep kernels only. Durations in microseconds.", "",
             "| kernel | calls | avg us | min us | max us | share of GPU time |", "|---|---|---|---|---|---|"]
    for r in rows:
        name = r["Name"].replace("(anonymous namespace)::", "")
        lines.append(f"| `{name}` | {r['Calls']} | {float(r['AverageNs']) / 1e3:.2f} | {float(r['MinNs']) / 1e3:.2f} "
                     f"| {float(r['MaxNs']) / 1e3:.2f} | {float(r['Percentage']):.2f}% |")
    lines += ["", f"bench.py line of the same (profiled) run: value {b['value']} GB/s, ms_per_step {b['ms_per_step']}, "
                  f"stage_us {b['stage_us']}; roofline kernel {roof['kernel']}: achieved {roof['achieved']} GB/s, "
                  f"frac {roof['frac']} ({roof.get('timing', 'HIP events')})."]
    stage = roof.get("stage", "epilogue")
    kname = roof["kernel"].split(" ")[0]
    trace_csv = stats_csv.replace("kernel_stats.csv", "kernel_trace.csv")
    if trace_csv != stats_csv and os.path.exists(trace_csv):
        g = kernel_runs(trace_csv, lambda n: kname in n)
        bb, ins = g["back_to_back"], g["in_step"]
        ev = b["stage_us"].get(f"{stage}_back_to_back")
        alg = roof["alg_bytes_per_launch"]
        lines += ["", f"Dispatches of the roofline kernel `{kname}` by what ran around them (kernel_trace.csv):", "",
                  "| launches | count | rocprofv3 mean duration us | rocprofv3 first start to last end, per launch us "
                  "| bench.py HIP events us |", "|---|---|---|---|---|"]
        if bb["n"]:
            lines.append(f"| back to back (roofline loop) | {bb['n']} | {bb['avg_us']:.2f} | "
                         f"{bb['span_us_per_launch']:.2f} | {ev} |")
        if ins["n"]:
            lines.append(f"| inside steps | {ins['n']} | {ins['avg_us']:.2f} | — | "
                         f"{b['stage_us'].get(stage)} (event pair around the launch) |")
        if bb["n"]:
            g_rp = alg / bb["avg_us"] / 1e3
            lines += ["", f"Roofline from the profiler: {alg} algorithmic bytes per launch over the rocprofv3 mean "
                          f"duration of the back-to-back launches ({bb['avg_us']:.2f} us): {g_rp:.1f} GB/s = "
                          f"{g_rp / PEAK_HBM_GBPS * 100:.1f}% of 8 TB/s (bench.py's events: {roof['achieved']} GB/s)."]
    with open(out_md, "w") as f:
        f.write("\n".join(lines) + "\n")
    print("\n".join(lines))


def measure_ceilings(reps: int = 10) -> dict:
    """Practical HBM ceilings of this device for context: torch's own device
    kernels on 1 GiB buffers (copy_ reads and writes, fill_ writes), timed
    between events on the current stream."""
    import torch

    n = 1 << 30
    stream = torch.cuda.current_stream()
    a = torch.ones(n // 4, dtype=torch.float32, device="cuda")
    b = torch.empty_like(a)
    ops = {"copy": (lambda: b.copy_(a), 2 * n), "write": (lambda: b.fill_(2.0), n)}
    res = {}
    for name, (fn, nbytes) in ops.items():
        fn()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(reps):
            fn()
        e1.record(stream)
        torch.cuda.synchronize()
        gbps = nbytes * reps / (e0.elapsed_time(e1) * 1e-3) / 1e9
        res[name] = {"GB/s": round(gbps, 1), "frac": round(gbps / PEAK_HBM_GBPS, 4)}
    del a, b
    torch.cuda.empty_cache()
    res["what"] = "torch copy_ (read + write) and fill_ (write) on 1 GiB, 10 back-to-back launches"
    return res


class BufferSet:
    """One complete, independent set of device buffers for a step: inputs
    (hidden rows and scales; routing and weights are shared, read-only),
    layout tables, staging and receive buffers, expert outputs y (seeded
    N(0,1) bf16 rows, a stand-in for the experts) and the combine output."""

    def __init__(self, w, cfg, x, x_sf, seed):
        import torch

        import combine_ep_layout_07_amd.ep as ep
        self.x = x.clone()
        self.x_sf = x_sf.clone() if x_sf is not None else None
        self.L = ep.alloc_layout(cfg)
        self.R = ep.alloc_recv(cfg)
        rows = int(ep.ep_query_sizes(cfg).recv_rows)
        gen = torch.Generator(device="cuda")
        gen.manual_seed(seed)
        self.y = torch.randn((max(rows, 1), w.H), generator=gen, device="cuda").to(torch.bfloat16)
        self.out = torch.empty((w.S * w.T, w.H), dtype=torch.bfloat16, device="cuda")


def measure_workload(w, inputs, steps, warmup, direct=False, n_sets=N_SETS, min_timed_ms=0.0):
    """Time a workload: K steps back to back rotating over n_sets buffer sets
    (between two HIP events on the launch stream, synchronised on both sides);
    the same steps with an event between stages (stage_us); and each stage's
    kernel alone, K launches back to back over the rotating sets (the
    roofline's durations).  With min_timed_ms, K is raised so that the timed
    steps take at least that long (a few-microsecond step timed 20 times is
    mostly the events' own jitter).  Returns the timings and the sets (still
    holding the last results)."""
    import numpy as np
    import torch

    import combine_ep_layout_07_amd.ep as ep

    cfg = ep.config_for(w, direct_recv_x=direct)
    stream = torch.cuda.current_stream()
    topk = torch.from_numpy(inputs["topk_idx"]).cuda()
    wts = torch.from_numpy(inputs["topk_weights"]).cuda()
    x = torch.from_numpy(inputs["x"].reshape(w.S * w.T, -1)).cuda()
    x_sf = torch.from_numpy(inputs["x_sf"]).cuda() if w.dtype == "fp8" else None
    sets = [BufferSet(w, cfg, x, x_sf, 12345 + i) for i in range(n_sets)]
    del x, x_sf

    calls = {
        "layout": lambda b: ep.ep_layout(cfg, topk, b.L, stream),
        "scatter": lambda b: ep.ep_dispatch(cfg, b.x, b.x_sf, topk, wts, b.L, b.R, ep.EP_PHASE_SCATTER, stream),
        "epilogue": lambda b: ep.ep_dispatch(cfg, b.x, b.x_sf, topk, wts, b.L, b.R, ep.EP_PHASE_EPILOGUE, stream),
        "combine": lambda b: ep.ep_combine(cfg, b.L, topk, wts, b.y, b.out, stream),
    }

    def step(b):
        ep.ep_layout_dispatch(cfg, b.x, b.x_sf, topk, wts, b.L, b.R, stream)
        ep.ep_combine(cfg, b.L, topk, wts, b.y, b.out, stream)

    for i in range(max(warmup, n_sets)):
        step(sets[i % n_sets])
    torch.cuda.synchronize()

    def timed_steps(k):
        t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        t0.record(stream)
        for i in range(k):
            step(sets[i % n_sets])
        t1.record(stream)
        torch.cuda.synchronize()
        return t0.elapsed_time(t1) / k

    ms = timed_steps(steps)
    if ms * steps < min_timed_ms:
        steps = int(math.ceil(min_timed_ms / ms))
        ms = timed_steps(steps)

    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(5)] for _ in range(steps)]
    for i in range(steps):
        b = sets[i % n_sets]
        for j, n in enumerate(STAGES):
            evs[i][j].record(stream)
            calls[n](b)
        evs[i][4].record(stream)
    torch.cuda.synchronize()
    stage_ms = {n: float(np.mean([e[j].elapsed_time(e[j + 1]) for e in evs])) for j, n in enumerate(STAGES)}

    # Each stage's kernels alone, K launches back to back over the rotating
    # sets: each launch's dispatch overlaps the previous one's tail, so the
    # mean is the kernels' own duration (what rocprofv3 reports per dispatch).
    for n in STAGES:
        b0, b1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        b0.record(stream)
        for i in range(steps):
            calls[n](sets[i % n_sets])
        b1.record(stream)
        torch.cuda.synchronize()
        stage_ms[f"{n}_back_to_back"] = b0.elapsed_time(b1) / steps
    L = sets[0].L
    n_rows = int(L.recv_base[-1].item())
    v_rows = int(((topk >= 0) & (topk < w.E)).sum().item())
    pad = int(L.expert_base[-1].item()) - v_rows if w.expand else 0
    return dict(cfg=cfg, sets=sets, topk=topk, wts=wts, calls=calls, step=step, stream=stream, ms=ms,
                stage_ms=stage_ms, n_rows=n_rows, v_rows=v_rows, pad=pad, steps=steps)


def workload_summary(w, m, direct=False) -> dict:
    """GB/s, % of peak, tokens/s, stage times and the dominant kernel's
    roofline of one measured workload."""
    b = alg_bytes(w, m["n_rows"], m["v_rows"], direct=direct, pad_rows=m["pad"])
    ms, st = m["ms"], m["stage_ms"]
    value = b["total"] / (ms * 1e-3) / 1e9
    dom = max(STAGES, key=lambda n: st[n])
    dom_gbps = b[dom] / (st[f"{dom}_back_to_back"] * 1e-3) / 1e9
    return {
        "workload": f"{w.name}: S={w.S} T={w.T} H={w.H} {w.dtype} K={w.K} E={w.E} R={w.R} Nmax={w.Nmax} "
                    f"{'expand A=%d' % w.alignment if w.expand else 'compact'} layout, {w.routing} routing"
                    f"{', Direct Recv X' if direct else ''}",
        "value": round(value, 2), "unit": "GB/s", "pct_of_peak": round(100.0 * value / PEAK_HBM_GBPS, 2),
        "ms_per_step": round(ms, 5), "steps": m["steps"], "tokens_per_s": round(w.S * w.T / (ms * 1e-3), 1),
        "alg_bytes_per_step": b, "rows": {"dedup_N": m["n_rows"], "valid_V": m["v_rows"], "padding": m["pad"]},
        "stage_us": {k: round(v * 1e3, 2) for k, v in st.items()},
        "stage_gbps_back_to_back": {n: round(b[n] / (st[f"{n}_back_to_back"] * 1e-3) / 1e9, 1) for n in STAGES},
        "dominant": {"stage": dom, "achieved": round(dom_gbps, 1), "frac": round(dom_gbps / PEAK_HBM_GBPS, 4)},
    }


def cold_stages(w, m, reps=20, warm=3):
    """Each stage alone after a clean flush of L2 and the Infinity Cache: a 1 GiB
    fill followed by a 1 GiB read of another buffer (the read evicts the fill's
    dirty lines, so their write-back is over before the timed stage starts).
    Median and minimum over `reps` runs."""
    import numpy as np
    import torch

    stream = m["stream"]
    fill = torch.empty((1 << 30) // 4, dtype=torch.int32, device="cuda")
    other = torch.ones((1 << 30) // 4, dtype=torch.int32, device="cuda")
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    times = {n: [] for n in STAGES}
    b = m["sets"][0]
    for r in range(warm + reps):
        for n in STAGES:
            fill.fill_(r)
            other.sum()
            e0.record(stream)
            m["calls"][n](b)
            e1.record(stream)
            torch.cuda.synchronize()
            if r >= warm:
                times[n].append(e0.elapsed_time(e1))
    del fill, other
    return {n: (float(np.median(v)), float(np.min(v))) for n, v in times.items()}


def graph_replay(m, steps, warmup):
    """The step captured once in a HIP graph per buffer set and replayed,
    rotating over the sets."""
    import torch
    gs = torch.cuda.Stream()
    gs.wait_stream(m["stream"])
    graphs = []
    import combine_ep_layout_07_amd.ep as ep
    cfg, topk, wts = m["cfg"], m["topk"], m["wts"]
    with torch.cuda.stream(gs):
        for b in m["sets"]:
            def on(b=b):
                ep.ep_layout_dispatch(cfg, b.x, b.x_sf, topk, wts, b.L, b.R, gs)
                ep.ep_combine(cfg, b.L, topk, wts, b.y, b.out, gs)
            on()
            torch.cuda.synchronize()
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g, stream=gs):
                on()
            graphs.append(g)
    torch.cuda.synchronize()
    for i in range(warmup):
        graphs[i % len(graphs)].replay()
    torch.cuda.synchronize()
    g0, g1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    g0.record()
    for i in range(steps):
        graphs[i % len(graphs)].replay()
    g1.record()
    torch.cuda.synchronize()
    return g0.elapsed_time(g1) / steps


def measure_extras(steps: int, warmup: int) -> dict:
    """The API's further modes at the headline shape (4096 tokens, H=7168 bf16,
    top-8 of 256 experts on 16 ranks), each timed as whole steps rotating over
    two buffer sets, on its own byte count:
      bias2          combine adds two bias tensors (ep_combine_bias);
      cached_layout  dispatch + combine replaying a layout computed once;
      expand_a128    expand layout, expert alignment 128 with zero padding;
      hybrid_2x8     hybrid row form: 16 sources = 2 scale-out x 8 scale-up
                     ranks of 256 tokens each, Nmax = 256."""
    import torch

    import combine_ep_layout_07_amd.ep as ep
    from combine_ep_layout_07_amd.workloads import WORKLOADS, generate, seed_for

    stream = torch.cuda.current_stream()
    base = WORKLOADS[2]
    cases = {
        "bias2": base,
        "cached_layout": base,
        "expand_a128": base.with_(name="dsv3_share_expand_a128", expand=True, alignment=128),
        "hybrid_2x8": base.with_(name="hybrid_2x8", S=16, T=256, Nmax=256, n_out=2),
    }
    res = {}
    for name, w in cases.items():
        print(f"[bench] extra: {name}", file=sys.stderr, flush=True)
        d = generate(w, seed_for(2, 5))
        topk = torch.from_numpy(d["topk_idx"]).cuda()
        wts = torch.from_numpy(d["topk_weights"]).cuda()
        x = torch.from_numpy(d["x"].reshape(w.S * w.T, -1)).cuda()
        cfg = ep.config_for(w)
        sets = [BufferSet(w, cfg, x, None, 777 + i) for i in range(N_SETS)]
        gen = torch.Generator(device="cuda")
        gen.manual_seed(778)
        bias = [torch.randn((w.S * w.T, w.H), generator=gen, device="cuda").to(torch.bfloat16) for _ in range(2)]
        for b in sets:
            ep.ep_layout(cfg, topk, b.L, stream)

        def step(b):
            if name == "cached_layout":
                ep.ep_dispatch(cfg, b.x, None, topk, wts, b.L, b.R, ep.EP_PHASE_ALL, stream)
            else:
                ep.ep_layout_dispatch(cfg, b.x, None, topk, wts, b.L, b.R, stream)
            if name == "bias2":
                ep.ep_combine_bias(cfg, b.L, topk, wts, b.y, bias[0], bias[1], b.out, stream)
            else:
                ep.ep_combine(cfg, b.L, topk, wts, b.y, b.out, stream)

        for i in range(max(warmup, N_SETS)):
            step(sets[i % N_SETS])
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for i in range(steps):
            step(sets[i % N_SETS])
        e1.record(stream)
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1) / steps
        L = sets[0].L
        n_rows = int(L.recv_base[-1].item())
        v_rows = int(((topk >= 0) & (topk < w.E)).sum().item())
        pad = int(L.expert_base[-1].item()) - v_rows if w.expand else 0
        b = alg_bytes(w, n_rows, v_rows, pad_rows=pad, n_bias=2 if name == "bias2" else 0)
        total = b["total"] - (b["layout"] if name == "cached_layout" else 0)
        res[name] = {"workload": f"{w.name}: S={w.S} T={w.T} H={w.H} K={w.K} E={w.E} R={w.R} Nmax={w.Nmax}"
                                 f"{' expand A=%d' % w.alignment if w.expand else ''}"
                                 f"{' n_out=%d' % w.n_out if w.n_out > 1 else ''}",
                     "value": round(total / (ms * 1e-3) / 1e9, 2), "unit": "GB/s",
                     "pct_of_peak": round(100.0 * total / (ms * 1e-3) / 1e9 / PEAK_HBM_GBPS, 2),
                     "ms_per_step": round(ms, 5), "steps": steps, "tokens_per_s": round(w.S * w.T / (ms * 1e-3), 1),
                     "alg_bytes_per_step": total, "rows": {"dedup_N": n_rows, "valid_V": v_rows, "padding": pad}}
        del sets, bias, x
        torch.cuda.empty_cache()
    return res


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--config", type=int, default=2, help="workload of the headline line")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-configs", action="store_true", help="skip the other workloads' measurements")
    ap.add_argument("--no-direct", action="store_true", help="skip the Direct Recv X variant")
    ap.add_argument("--no-graph", action="store_true", help="skip the HIP-graph replay measurement")
    ap.add_argument("--no-cold", action="store_true", help="skip the cold-cache per-stage timing")
    ap.add_argument("--no-extras", action="store_true",
                    help="skip the bias / cached-layout / expand-alignment / hybrid measurements and ceilings")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="also run a plain 256 MiB device copy (the reference for the byte counters)")
    ap.add_argument("--summarize-counters", nargs=4, metavar=("FETCH_CSV", "WRITE_CSV", "BENCH_JSON", "OUT_MD"),
                    help="write the traffic summary from two rocprofv3 --pmc CSVs and exit (no GPU use)")
    ap.add_argument("--summarize-trace", nargs=3, metavar=("STATS_CSV", "BENCH_JSON", "OUT_MD"),
                    help="write a kernel-trace summary from rocprofv3 --stats output and exit (no GPU use)")
    ap.add_argument("--command", default="", help="profiling command recorded in the summary")
    args = ap.parse_args()
    if args.summarize_counters:
        summarize_counters(*args.summarize_counters, command=args.command)
        return
    if args.summarize_trace:
        summarize_trace(*args.summarize_trace, command=args.command)
        return
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py runs one GPU's share only (--gpus {args.gpus}, WORLD_SIZE {world}): the ranks of this "
              "workload are emulated as partitions of one GPU's HBM; there is no multi-GPU path.", file=sys.stderr)
        sys.exit(2)

    import torch

    from combine_ep_layout_07_amd.workloads import WORKLOADS, generate, seed_for

    w = WORKLOADS[args.config]
    inputs = generate(w, seed_for(args.config))
    print(f"[bench] {w.name}: warmup {args.warmup}, timing {args.steps} steps over {N_SETS} buffer sets",
          file=sys.stderr, flush=True)
    m = measure_workload(w, inputs, args.steps, args.warmup)
    head = workload_summary(w, m)
    b = head["alg_bytes_per_step"]
    dom = head["dominant"]["stage"]
    dom_kernel = {"layout": "k_layout", "scatter": "k_scatter", "combine": "k_combine",
                  "epilogue": ("k_epilogue_expand_indexed" if w.alignment == 1 else "k_epilogue_expand_pieces")
                  if w.expand else "k_epilogue_indexed"}[dom]
    res = {
        "metric": METRIC,
        "value": head["value"],
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": head["ms_per_step"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.dtype,
        "data": "synthetic",
        "config": {"workload": head["workload"],
                   "source_partitions": w.S, "tokens_per_source": w.T, "hidden": w.H, "top_k": w.K,
                   "experts": w.E, "destination_ranks": w.R, "num_max_tokens_per_rank": w.Nmax,
                   "layout": "expand" if w.expand else "compact",
                   "emulation": f"{w.S} source and {w.R} destination ranks as partitions of one GPU's HBM",
                   "timing": f"{args.steps} steps back to back rotating over {N_SETS} complete buffer sets"},
        "pct_of_peak": head["pct_of_peak"],
        "tokens_per_s": head["tokens_per_s"],
        "alg_bytes_per_step": b,
        "rows": head["rows"],
        "stage_us": head["stage_us"],
        "stage_gbps_back_to_back": head["stage_gbps_back_to_back"],
        "roofline": {"bound": "hbm", "kernel": f"{dom_kernel} ({dom})", "stage": dom,
                     "achieved": head["dominant"]["achieved"], "peak": PEAK_HBM_GBPS, "unit": "GB/s",
                     "frac": head["dominant"]["frac"], "alg_bytes_per_launch": b[dom],
                     "traffic": read_traffic(w.name, dom),
                     "timing": f"mean of {args.steps} launches back to back, rotating over {N_SETS} buffer sets, "
                               "between two HIP events on the launch stream"},
        "library": library_identity(),
    }
    if not args.no_cold:
        print("[bench] cold per-stage timing (clean flush)", file=sys.stderr, flush=True)
        cold = cold_stages(w, m)
        cold_ms = sum(v[0] for v in cold.values())
        res["cold_per_stage"] = {
            "protocol": "each stage alone after a 1 GiB fill then a 1 GiB read of another buffer (L2 and Infinity "
                        "Cache flushed, the fill's write-back done), 3 warm-up + 20 runs",
            "median_us": {k: round(v[0] * 1e3, 2) for k, v in cold.items()},
            "min_us": {k: round(v[1] * 1e3, 2) for k, v in cold.items()},
            "value": round(b["total"] / (cold_ms * 1e-3) / 1e9, 2), "unit": "GB/s",
            "pct_of_peak": round(100.0 * b["total"] / (cold_ms * 1e-3) / 1e9 / PEAK_HBM_GBPS, 2),
            "ms_per_step": round(cold_ms, 5)}
    if not args.no_graph:
        print("[bench] graph replay", file=sys.stderr, flush=True)
        ms_g = graph_replay(m, args.steps, args.warmup)
        res["graph_replay"] = {"value": round(b["total"] / (ms_g * 1e-3) / 1e9, 2), "unit": "GB/s",
                               "ms_per_step": round(ms_g, 5), "tokens_per_s": round(w.S * w.T / (ms_g * 1e-3), 1)}
    n_rows, v_rows = m["n_rows"], m["v_rows"]
    del m
    torch.cuda.empty_cache()
    if not w.expand and not args.no_direct:
        # Direct Recv X (the scatter writes hidden rows straight into recv_x):
        # a different byte count, reported beside the headline, never as it.
        print("[bench] direct recv_x variant", file=sys.stderr, flush=True)
        md = measure_workload(w, inputs, args.steps, args.warmup, direct=True)
        d = workload_summary(w, md, direct=True)
        d["speedup_vs_staging"] = round(head["ms_per_step"] / d["ms_per_step"], 3)
        res["direct_recv_x"] = d
        del md
        torch.cuda.empty_cache()
    if not args.no_configs:
        res["configs"] = {}
        for cid in sorted(WORKLOADS):
            if cid == args.config:
                res["configs"][str(cid)] = head
                continue
            wc = WORKLOADS[cid]
            print(f"[bench] workload {cid} ({wc.name})", file=sys.stderr, flush=True)
            inp = generate(wc, seed_for(cid))
            mc = measure_workload(wc, inp, args.steps, args.warmup, min_timed_ms=MIN_TIMED_MS)
            res["configs"][str(cid)] = workload_summary(wc, mc)
            del mc, inp
            torch.cuda.empty_cache()
    if args.config == 2 and not args.no_extras:
        res["extras"] = measure_extras(args.steps, args.warmup)
    if not args.no_extras:
        res["ceilings"] = measure_ceilings()
    if args.copy_calibration:
        copy_calibration()
    if not args.no_cpu_baseline:
        print("[bench] cpu baseline (oracle): one thread, then all cores", file=sys.stderr, flush=True)
        res["cpu_baseline"] = cpu_baseline(w, inputs, n_rows, v_rows)
    else:
        res["cpu_baseline"] = None
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
