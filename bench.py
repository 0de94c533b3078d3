"""Benchmark of the deterministic EP dispatch + combine hot path on one MI355X.

One step = ep_layout + ep_dispatch (scatter + copy epilogue) + ep_combine over
one batch of seeded synthetic input already resident in HBM: the DeepSeek-V3-
like share of the deterministic-dispatch page's benchmark (T=4096 tokens,
hidden 7168 bf16, top-8 of 256 experts on 16 ranks, Nmax=4096, compact
layout).  Prints ONE JSON line with effective HBM GB/s on the algorithmic bytes
of the step, the roofline of the dominant kernel (the copy epilogue) and the
CPU oracle timed on the host as a reported baseline.

    python bench.py [--steps K] [--warmup W] [--gpus 1] [--config 2] [--no-cpu-baseline]
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_HBM_GBPS = 8000.0  # MI355X HBM3E
METRIC = "dispatch+combine effective HBM GB/s (% of peak) at T=4096,H=7168,K=8"
PROFILES = os.path.join(ROOT, "profiles")
TRAFFIC_FILE = os.path.join(PROFILES, "epilogue_dsv3_share_traffic.md")
EPILOGUE_SOURCES = [os.path.join(ROOT, "combine_ep_layout_07_amd", "csrc", f)
                    for f in ("ep_dispatch.hip", "ep_device.h", "ep_kernels.h")]


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


def read_traffic(per_launch_alg: float):
    """HBM bytes per epilogue launch from the committed rocprofv3 counter summary,
    or None when the summary is missing or the kernel source changed since."""
    if not os.path.exists(TRAFFIC_FILE):
        return None
    text = open(TRAFFIC_FILE).read()

    def field(name):
        m = re.search(r"^%s:\s*([0-9.eE+-]+|[0-9a-f]+)\s*$" % re.escape(name), text, flags=re.M)
        return m.group(1) if m else None

    if field("kernel_source_sha256_16") != source_digest(EPILOGUE_SOURCES):
        return None
    try:
        return float(field("traffic_bytes_per_launch"))
    except (TypeError, ValueError):
        return None


def cpu_baseline(w, inputs, n_rows, v_rows, max_passes=100, budget_s=12.0):
    """The oracle as it stands, single-threaded, on the same workload: whole
    passes (layout + dispatch + combine) until about budget_s of CPU time."""
    import numpy as np
    import oracle
    from combine_ep_layout_07_amd.workloads import draw_expert_outputs

    oracle.build(force=False)
    times = []
    rows = n_rows if not w.expand else v_rows
    y = draw_expert_outputs(rows, w.H, 99)
    while len(times) < max_passes and (len(times) < 3 or sum(times) < budget_s):
        t0 = time.perf_counter()
        lay = oracle.layout(w.S, w.T, w.K, w.E, w.R, w.Nmax, inputs["topk_idx"], w.expand, w.alignment)
        disp = oracle.dispatch(w.S, w.T, w.H, w.K, w.E, w.R, w.Nmax, w.dtype == "fp8", w.expand, w.alignment,
                               inputs["x"], inputs.get("x_sf"), inputs["topk_idx"], inputs["topk_weights"], lay)
        del disp
        oracle.combine(w.S, w.T, w.H, w.K, w.E, w.R, w.Nmax, w.expand, inputs["topk_idx"], inputs["topk_weights"],
                       lay, y)
        times.append(time.perf_counter() - t0)
    t = float(np.median(times))
    b = alg_bytes(w, n_rows, v_rows)["total"]
    return {"value": round(b / t / 1e9, 3), "unit": "GB/s", "cores": 1, "kind": "oracle",
            "sample": f"full {w.name} workload (S={w.S} T={w.T} H={w.H} K={w.K}), layout+dispatch+combine, "
                      f"median of {len(times)} passes of {t:.2f} s ({sum(times):.1f} s of CPU work), single thread",
            "seconds_per_step": round(t, 3), "tokens_per_s": round(w.S * w.T / t, 1)}


COPY_CAL_BYTES = 256 * 2**20


def copy_calibration(reps=5):
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


def summarize_counters(fetch_csv: str, write_csv: str, out_md: str, command: str) -> None:
    """Turn two rocprofv3 --pmc counter CSVs (FETCH_SIZE, WRITE_SIZE; KiB per
    dispatch) into the traffic summary read by read_traffic()."""
    import numpy as np

    def per_kernel(path, counter):
        acc = {}
        for r in _counter_rows(path):
            if r.get("Counter_Name") != counter:
                continue
            acc.setdefault(r["Kernel_Name"], []).append(float(r["Counter_Value"]))
        return acc

    fetch, write = per_kernel(fetch_csv, "FETCH_SIZE"), per_kernel(write_csv, "WRITE_SIZE")

    def pick(acc, key, largest=False):
        vals = [v for k, vs in acc.items() if key in k for v in vs]
        if not vals:
            return float("nan")
        return float(max(vals)) if largest else float(np.median(vals))

    # The calibration copy (torch's device-to-device copy runs the runtime's
    # copyBuffer kernel) is the largest copy dispatch of the run.
    cf, cw = pick(fetch, "copyBuffer", True), pick(write, "copyBuffer", True)
    ef, ew = pick(fetch, "k_epilogue"), pick(write, "k_epilogue")
    # counters are KiB per dispatch; a copy of COPY_CAL_BYTES must read and write that many bytes
    f_scale = COPY_CAL_BYTES / (cf * 1024.0)
    w_scale = COPY_CAL_BYTES / (cw * 1024.0)
    traffic = ef * 1024.0 * f_scale + ew * 1024.0 * w_scale
    lines = [
        "# Copy-epilogue HBM traffic (dsv3_share: T=4096 H=7168 bf16 K=8 E=256 R=16)",
        "",
        "Counters from two rocprofv3 --pmc runs (FETCH_SIZE, then WRITE_SIZE), KiB per dispatch, median over",
        "dispatches; scaled by what the same counters read for a plain device copy of 256 MiB.",
        "",
        "command: " + command,
        "",
        f"copy_fetch_kib_per_dispatch: {cf:.1f}",
        f"copy_write_kib_per_dispatch: {cw:.1f}",
        f"fetch_scale: {f_scale:.4f}",
        f"write_scale: {w_scale:.4f}",
        f"epilogue_fetch_kib_per_dispatch: {ef:.1f}",
        f"epilogue_write_kib_per_dispatch: {ew:.1f}",
        f"traffic_bytes_per_launch: {traffic:.0f}",
        f"kernel_source_sha256_16: {source_digest(EPILOGUE_SOURCES)}",
        "",
        "Other kernels (median KiB per dispatch, fetch / write):",
    ]
    for k in sorted(set(fetch) | set(write)):
        if "ep::" in k or "copy" in k:
            lines.append(f"- {k[:90]}: {np.median(fetch.get(k, [np.nan])):.1f} / {np.median(write.get(k, [np.nan])):.1f}")
    with open(out_md, "w") as f:
        f.write("\n".join(lines) + "\n")
    print("\n".join(lines))


def is_copy_epilogue(name: str) -> bool:
    return "k_epilogue" in name and "meta" not in name


def epilogue_runs(trace_csv: str) -> dict:
    """Copy-epilogue dispatches of a rocprofv3 kernel trace (kernel_trace.csv),
    split by what ran around them: "back_to_back" = launches in a run of two or
    more consecutive epilogue dispatches (bench.py's roofline loop),
    "in_step" = the rest (between a scatter and a combine).  For each group:
    count, mean duration (us) and, for the back-to-back runs, the mean time per
    launch from the first start to the last end of each run, the interval the
    bench's two HIP events bracket."""
    rows = sorted(_counter_rows(trace_csv), key=lambda r: int(r["Start_Timestamp"]))
    epi = [is_copy_epilogue(r["Kernel_Name"]) for r in rows]
    groups = {"back_to_back": [], "in_step": []}
    spans = []
    i = 0
    while i < len(rows):
        if not epi[i]:
            i += 1
            continue
        j = i
        while j + 1 < len(rows) and epi[j + 1]:
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
    with the run's kernel_trace.csv beside the stats file, the copy epilogue's
    back-to-back launches (the roofline's) are also summarised on their own."""
    rows = [r for r in _counter_rows(stats_csv) if "ep::" in r["Name"]]
    with open(bench_json) as f:
        b = json.loads(f.read().strip().splitlines()[-1])
    lines = [f"# Kernel trace: {b['config']['workload']}", "", "command: " + command, "",
             "rocprofv3 --stats summary (kernel_stats.csv), libep kernels only. Durations in microseconds.", "",
             "| kernel | calls | avg us | min us | max us | share of GPU time |", "|---|---|---|---|---|---|"]
    for r in rows:
        name = r["Name"].replace("(anonymous namespace)::", "")
        lines.append(f"| `{name}` | {r['Calls']} | {float(r['AverageNs']) / 1e3:.2f} | {float(r['MinNs']) / 1e3:.2f} "
                     f"| {float(r['MaxNs']) / 1e3:.2f} | {float(r['Percentage']):.2f}% |")
    lines += ["", f"bench.py line of the same (profiled) run: value {b['value']} GB/s, ms_per_step {b['ms_per_step']}, "
                  f"stage_us {b['stage_us']}, epilogue achieved {b['roofline']['achieved']} GB/s "
                  f"({b['roofline'].get('timing', 'HIP events')})."]
    epi = [r for r in rows if is_copy_epilogue(r["Name"])]
    if epi:
        avg = float(epi[0]["AverageNs"]) / 1e3
        alg = b["roofline"]["alg_bytes_per_launch"]
        lines.append(f"The same algorithmic bytes ({alg} B per launch) over the rocprofv3 average duration of the "
                     f"copy epilogue ({avg:.2f} us): {alg / avg / 1e3:.1f} GB/s = "
                     f"{alg / avg / 1e3 / PEAK_HBM_GBPS * 100:.1f}% of 8 TB/s.")
    trace_csv = stats_csv.replace("kernel_stats.csv", "kernel_trace.csv")
    if epi and trace_csv != stats_csv and os.path.exists(trace_csv):
        g = epilogue_runs(trace_csv)
        bb, ins = g["back_to_back"], g["in_step"]
        ev = b["stage_us"].get("epilogue_back_to_back")
        lines += ["", "Copy-epilogue dispatches of the same run by what ran around them (kernel_trace.csv):", "",
                  "| launches | count | rocprofv3 mean duration us | rocprofv3 first start to last end, per launch us "
                  "| bench.py HIP events us |", "|---|---|---|---|---|"]
        if bb["n"]:
            lines.append(f"| back to back (roofline loop) | {bb['n']} | {bb['avg_us']:.2f} | "
                         f"{bb['span_us_per_launch']:.2f} | {ev} |")
        if ins["n"]:
            lines.append(f"| inside steps (after the scatter) | {ins['n']} | {ins['avg_us']:.2f} | — | "
                         f"{b['stage_us'].get('epilogue')} (event pair around the launch) |")
    with open(out_md, "w") as f:
        f.write("\n".join(lines) + "\n")
    print("\n".join(lines))


def measure_ceilings(reps: int = 10) -> dict:
    """Practical HBM ceilings of this device for context: torch's own device
    kernels on 1 GiB buffers (copy_ reads and writes, fill_ writes), timed
    between events on the current stream.  (torch's reductions are not
    read-bound enough to serve as a read ceiling.)"""
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


def measure_extras(steps: int, warmup: int) -> dict:
    """The API's further modes at the headline shape (4096 tokens, H=7168 bf16,
    top-8 of 256 experts on 16 ranks), each timed as whole steps between two
    events on the launch stream, on its own byte count:
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
        L, R = ep.alloc_layout(cfg), ep.alloc_recv(cfg)
        rows_cap = int(ep.ep_query_sizes(cfg).recv_rows)
        gen = torch.Generator(device="cuda")
        gen.manual_seed(777)
        y = torch.randn((rows_cap, w.H), generator=gen, device="cuda").to(torch.bfloat16)
        out = torch.empty((w.S * w.T, w.H), dtype=torch.bfloat16, device="cuda")
        bias = [torch.randn((w.S * w.T, w.H), generator=gen, device="cuda").to(torch.bfloat16) for _ in range(2)]
        ep.ep_layout(cfg, topk, L, stream)

        def step():
            if name != "cached_layout":
                ep.ep_layout(cfg, topk, L, stream)
            ep.ep_dispatch(cfg, x, None, topk, wts, L, R, ep.EP_PHASE_ALL, stream)
            if name == "bias2":
                ep.ep_combine_bias(cfg, L, topk, wts, y, bias[0], bias[1], out, stream)
            else:
                ep.ep_combine(cfg, L, topk, wts, y, out, stream)

        for _ in range(warmup):
            step()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(steps):
            step()
        e1.record(stream)
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1) / steps
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
                     "ms_per_step": round(ms, 5), "tokens_per_s": round(w.S * w.T / (ms * 1e-3), 1),
                     "alg_bytes_per_step": total, "rows": {"dedup_N": n_rows, "valid_V": v_rows, "padding": pad}}
        del L, R, y, out, bias, x
        torch.cuda.empty_cache()
    return res


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--config", type=int, default=2)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-direct", action="store_true", help="skip the Direct Recv X variant")
    ap.add_argument("--no-graph", action="store_true", help="skip the HIP-graph replay measurement")
    ap.add_argument("--no-cold", action="store_true", help="skip the cold-cache per-stage timing")
    ap.add_argument("--no-extras", action="store_true",
                    help="skip the bias / cached-layout / expand-alignment / hybrid measurements")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="also run a plain 256 MiB device copy (the reference for the byte counters)")
    ap.add_argument("--summarize-counters", nargs=3, metavar=("FETCH_CSV", "WRITE_CSV", "OUT_MD"),
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

    import numpy as np
    import torch

    import combine_ep_layout_07_amd.ep as ep
    from combine_ep_layout_07_amd.workloads import WORKLOADS, generate, seed_for

    w = WORKLOADS[args.config]
    inputs = generate(w, seed_for(args.config))
    dev = "cuda"
    topk = torch.from_numpy(inputs["topk_idx"]).to(dev)
    wts = torch.from_numpy(inputs["topk_weights"]).to(dev)
    x = torch.from_numpy(inputs["x"].reshape(w.S * w.T, -1)).to(dev)
    x_sf = torch.from_numpy(inputs["x_sf"]).to(dev) if w.dtype == "fp8" else None
    cfg = ep.config_for(w)
    L = ep.alloc_layout(cfg, dev)
    R = ep.alloc_recv(cfg, dev)
    rows_cap = int(ep.ep_query_sizes(cfg).recv_rows)
    gen = torch.Generator(device=dev)
    gen.manual_seed(12345)
    y = torch.randn((rows_cap, w.H), generator=gen, device=dev).to(torch.bfloat16)
    out = torch.empty((w.S * w.T, w.H), dtype=torch.bfloat16, device=dev)
    stream = torch.cuda.current_stream()

    def step(c, recv, phased=False, ev=None):
        if ev is not None:
            ev[0].record(stream)
        ep.ep_layout(c, topk, L, stream)
        if ev is not None:
            ev[1].record(stream)
        if phased:
            ep.ep_dispatch(c, x, x_sf, topk, wts, L, recv, ep.EP_PHASE_SCATTER, stream)
            if ev is not None:
                ev[2].record(stream)
            ep.ep_dispatch(c, x, x_sf, topk, wts, L, recv, ep.EP_PHASE_EPILOGUE, stream)
        else:
            ep.ep_dispatch(c, x, x_sf, topk, wts, L, recv, ep.EP_PHASE_ALL, stream)
        if ev is not None:
            ev[3].record(stream)
        ep.ep_combine(c, L, topk, wts, y, out, stream)
        if ev is not None:
            ev[4].record(stream)

    names = ["layout", "scatter", "epilogue", "combine"]

    def measure(c, recv):
        """K back-to-back steps between two events (synchronised on both sides),
        then the same steps again with an event between stages."""
        for _ in range(args.warmup):
            step(c, recv)
        torch.cuda.synchronize()
        t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        t0.record(stream)
        for _ in range(args.steps):
            step(c, recv)
        t1.record(stream)
        torch.cuda.synchronize()
        ms = t0.elapsed_time(t1) / args.steps
        evs = [[torch.cuda.Event(enable_timing=True) for _ in range(5)] for _ in range(args.steps)]
        torch.cuda.synchronize()
        for i in range(args.steps):
            step(c, recv, phased=True, ev=evs[i])
        torch.cuda.synchronize()
        stage_ms = {n: float(np.mean([e[i].elapsed_time(e[i + 1]) for e in evs])) for i, n in enumerate(names)}
        # The copy epilogue alone, K launches back to back between two events:
        # each launch's dispatch overlaps the previous one's tail, so the mean
        # is the kernel's own duration (what rocprofv3 reports per dispatch).
        b0, b1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        b0.record(stream)
        for _ in range(args.steps):
            ep.ep_dispatch(c, x, x_sf, topk, wts, L, recv, ep.EP_PHASE_EPILOGUE, stream)
        b1.record(stream)
        torch.cuda.synchronize()
        stage_ms["epilogue_back_to_back"] = b0.elapsed_time(b1) / args.steps
        return ms, stage_ms

    def cold_stages(c, recv, reps=20, warm=3):
        """Each stage alone, after a 1 GiB device fill has flushed L2 and the
        Infinity Cache; median and minimum over `reps` runs."""
        flush = torch.empty((1 << 30) // 4, dtype=torch.int32, device=dev)
        calls = {
            "layout": lambda: ep.ep_layout(c, topk, L, stream),
            "scatter": lambda: ep.ep_dispatch(c, x, x_sf, topk, wts, L, recv, ep.EP_PHASE_SCATTER, stream),
            "epilogue": lambda: ep.ep_dispatch(c, x, x_sf, topk, wts, L, recv, ep.EP_PHASE_EPILOGUE, stream),
            "combine": lambda: ep.ep_combine(c, L, topk, wts, y, out, stream),
        }
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        times = {n: [] for n in names}
        for r in range(warm + reps):
            for n in names:
                flush.fill_(r)
                e0.record(stream)
                calls[n]()
                e1.record(stream)
                torch.cuda.synchronize()
                if r >= warm:
                    times[n].append(e0.elapsed_time(e1))
        del flush
        return {n: (float(np.median(v)), float(np.min(v))) for n, v in times.items()}

    print(f"[bench] {w.name}: warmup {args.warmup}, timing {args.steps} steps", file=sys.stderr, flush=True)
    ms, stage_ms = measure(cfg, R)
    cold = None
    if not args.no_cold:
        print("[bench] cold per-stage timing", file=sys.stderr, flush=True)
        cold = cold_stages(cfg, R)
    n_rows = int(L.recv_base[-1].item())
    v_rows = int(((topk >= 0) & (topk < w.E)).sum().item())
    b = alg_bytes(w, n_rows, v_rows)

    value = b["total"] / (ms * 1e-3) / 1e9
    epi_alg = b["epilogue"]
    epi_gbps = epi_alg / (stage_ms["epilogue_back_to_back"] * 1e-3) / 1e9
    traffic = read_traffic(epi_alg)
    res = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.dtype,
        "data": "synthetic",
        "config": {"workload": f"{w.name}: S={w.S} T={w.T} H={w.H} {w.dtype} K={w.K} E={w.E} R={w.R} "
                               f"Nmax={w.Nmax} {'expand' if w.expand else 'compact'} layout, {w.routing} routing",
                   "source_partitions": w.S, "tokens_per_source": w.T, "hidden": w.H, "top_k": w.K,
                   "experts": w.E, "destination_ranks": w.R, "num_max_tokens_per_rank": w.Nmax,
                   "layout": "expand" if w.expand else "compact",
                   "emulation": f"{w.S} source and {w.R} destination ranks as partitions of one GPU's HBM"},
        "pct_of_peak": round(100.0 * value / PEAK_HBM_GBPS, 2),
        "tokens_per_s": round(w.S * w.T / (ms * 1e-3), 1),
        "alg_bytes_per_step": b,
        "rows": {"dedup_N": n_rows, "valid_V": v_rows},
        "stage_us": {k: round(v * 1e3, 2) for k, v in stage_ms.items()},
        "stage_gbps": {k: round(b[k] / (stage_ms[k] * 1e-3) / 1e9, 1) for k in names},
        "roofline": {"bound": "hbm", "kernel": "k_epilogue_pf (copy epilogue)", "achieved": round(epi_gbps, 1),
                     "peak": PEAK_HBM_GBPS, "unit": "GB/s", "frac": round(epi_gbps / PEAK_HBM_GBPS, 4),
                     "alg_bytes_per_launch": epi_alg, "traffic": traffic,
                     "timing": "mean of K epilogue launches back to back between two HIP events on the launch "
                               "stream"},
    }
    if cold is not None:
        cold_ms = sum(v[0] for v in cold.values())
        res["cold_per_stage"] = {
            "protocol": "each stage alone after a 1 GiB fill (L2 and Infinity Cache flushed), 3 warm-up + 20 runs",
            "median_us": {k: round(v[0] * 1e3, 2) for k, v in cold.items()},
            "min_us": {k: round(v[1] * 1e3, 2) for k, v in cold.items()},
            "value": round(b["total"] / (cold_ms * 1e-3) / 1e9, 2), "unit": "GB/s",
            "ms_per_step": round(cold_ms, 5)}
    if not args.no_graph:
        # The same step captured once in a HIP graph and replayed K times.
        print("[bench] graph replay", file=sys.stderr, flush=True)
        gs = torch.cuda.Stream()
        gs.wait_stream(stream)
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.stream(gs):
            step_on = lambda: (ep.ep_layout(cfg, topk, L, gs),  # noqa: E731
                               ep.ep_dispatch(cfg, x, x_sf, topk, wts, L, R, ep.EP_PHASE_ALL, gs),
                               ep.ep_combine(cfg, L, topk, wts, y, out, gs))
            step_on()
            torch.cuda.synchronize()
            with torch.cuda.graph(graph, stream=gs):
                step_on()
        torch.cuda.synchronize()
        for _ in range(args.warmup):
            graph.replay()
        torch.cuda.synchronize()
        g0, g1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        g0.record()
        for _ in range(args.steps):
            graph.replay()
        g1.record()
        torch.cuda.synchronize()
        ms_g = g0.elapsed_time(g1) / args.steps
        res["graph_replay"] = {"value": round(b["total"] / (ms_g * 1e-3) / 1e9, 2), "unit": "GB/s",
                               "ms_per_step": round(ms_g, 5), "tokens_per_s": round(w.S * w.T / (ms_g * 1e-3), 1)}
    if not w.expand and not args.no_direct:
        # Direct Recv X (the scatter writes hidden rows straight into recv_x):
        # a different byte count, reported beside the headline, never as it.
        cfg_d = ep.config_for(w, direct_recv_x=True)
        del R
        R_d = ep.alloc_recv(cfg_d, dev)
        print("[bench] direct recv_x variant", file=sys.stderr, flush=True)
        ms_d, stage_d = measure(cfg_d, R_d)
        bd = alg_bytes(w, n_rows, v_rows, direct=True)
        res["direct_recv_x"] = {
            "value": round(bd["total"] / (ms_d * 1e-3) / 1e9, 2), "unit": "GB/s",
            "ms_per_step": round(ms_d, 5), "tokens_per_s": round(w.S * w.T / (ms_d * 1e-3), 1),
            "alg_bytes_per_step": bd, "stage_us": {k: round(v * 1e3, 2) for k, v in stage_d.items()},
            "speedup_vs_staging": round(ms / ms_d, 3)}
    if args.config == 2 and not args.no_extras:
        res["extras"] = measure_extras(args.steps, args.warmup)
    if not args.no_extras:
        res["ceilings"] = measure_ceilings()
    if args.copy_calibration:
        copy_calibration()
    if not args.no_cpu_baseline:
        print("[bench] cpu baseline (oracle)", file=sys.stderr, flush=True)
        res["cpu_baseline"] = cpu_baseline(w, inputs, n_rows, v_rows)
    else:
        res["cpu_baseline"] = None
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
