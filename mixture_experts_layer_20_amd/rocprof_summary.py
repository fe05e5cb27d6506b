"""Summarise rocprofv3 output of bench.py runs into the text kept under profiles/.

Inputs (all written by rocprofv3 with --output-format csv):
  <trace dir>/run_kernel_stats.csv, run_kernel_trace.csv   from  --kernel-trace --stats
  <pmc dir>/run_counter_collection.csv                      from  --pmc FETCH_SIZE  (one pass)
  <pmc dir>/run_counter_collection.csv                      from  --pmc WRITE_SIZE  (one pass)
  <pmc dir>/run_counter_collection.csv                      from  --pmc <other counters>
                                                            (optional, --pmc, repeatable)
The bench run must include `--copy-probe-mb N`: one plain device copy of N MiB whose counter
readings calibrate FETCH_SIZE / WRITE_SIZE (KiB per dispatch) to bytes.

Each GEMM stage of a layer step is one launch covering the routed experts and the shared expert
(--sets-per-stage 1, the default), or two launches, routed then shared (--sets-per-stage 2, a
bench run with --no-merge); dispatches are labelled by that order.

Usage:
  python -m mixture_experts_layer_20_amd.rocprof_summary --trace T --fetch F --write W \
      --workload tiny64e_random --copy-mb 256 --command "<the rocprofv3 commands>" \
      --out profiles/<name>.md [--traffic-json profiles/traffic.json]
"""
from __future__ import annotations

import argparse
import collections
import csv
import hashlib
import json
import os
import re

MODES = ["gate_up_fwd", "down_fwd", "down_bwd", "gate_up_dgrad", "down_wgrad", "gate_up_wgrad"]
PKG = os.path.dirname(os.path.abspath(__file__))


GEMM_SOURCES = ("common.h", "gemm_common.h", "grouped_gemm.hip", "grouped_gemm_pipe.hip")


def kernel_source_sha() -> str:
    """Hash of the grouped-GEMM sources: counter readings are valid only for the code they came from."""
    h = hashlib.sha256()
    for name in GEMM_SOURCES:
        h.update(open(os.path.join(PKG, "csrc", name), "rb").read())
    return h.hexdigest()[:16]


def short_name(name: str) -> str:
    m = re.search(r"grouped_gemm_bf16<(\d), [^>]*Cfg<(\d+), (\d+), (\d), (\d)>", name)
    if m:
        return f"grouped_gemm_bf16[{MODES[int(m.group(1))]}, {m.group(2)}x{m.group(3)}, {int(m.group(4)) * int(m.group(5))} waves]"
    m = re.search(r"(mx_gemm_pipe_kernel|mx_gemm_kernel)<(\d), (true|false)(?:, (\d+))?>", name)
    if m:
        epi = "wgrad" if m.group(3) == "true" else ("store", "swiglu", "swiglu_bwd")[int(m.group(2))]
        sw = f", {m.group(4)}-byte scales" if m.group(4) else ""
        return f"{m.group(1).replace('_kernel', '')}[{epi}{sw}]"
    m = re.search(r"(grouped_gemm_pipe|grouped_gemm_bf16_dma|splitk_reduce)<(\d)>", name)
    if m:
        return f"{m.group(1)}[{MODES[int(m.group(2))]}]"
    n = re.sub(r"void |moe::|\(anonymous namespace\)::", "", name)
    n = re.sub(r"\(.*", "", n)
    return n.strip()


def gemm_mode(name: str) -> str | None:
    m = re.search(r"grouped_gemm_(?:bf16|bf16_dma|pipe|f32)<(\d)[,>]", name)
    return MODES[int(m.group(1))] if m else None


def labelled_dispatches(rows, name_key, id_key, sets_per_stage=1):
    """Label GEMM dispatches by expert set: 'routed+shared' (one launch per stage) or
    'routed'/'shared' by their order within a step."""
    seen = collections.Counter()
    out = []
    for r in sorted(rows, key=lambda r: int(r[id_key])):
        n = r[name_key]
        mode = gemm_mode(n)
        label = None
        if mode:
            label = "routed+shared" if sets_per_stage == 1 else ("routed", "shared")[seen[n] % 2]
            seen[n] += 1
        out.append((r, mode, label))
    return out


def copy_scale(pmc_csv: str, counter: str, copy_mb: int) -> float | None:
    vals = [float(r["Counter_Value"]) for r in csv.DictReader(open(pmc_csv))
            if r["Counter_Name"] == counter and "copyBuffer" in r["Kernel_Name"] and int(r["Grid_Size"]) > 4096]
    if not vals:
        return None
    return copy_mb * 1024.0 / (sum(vals) / len(vals))


def per_stage_counter(pmc_csv: str, counter: str, sets_per_stage: int):
    rows = [r for r in csv.DictReader(open(pmc_csv)) if r["Counter_Name"] == counter]
    acc = collections.defaultdict(list)
    for r, mode, label in labelled_dispatches(rows, "Kernel_Name", "Dispatch_Id", sets_per_stage):
        if mode:
            acc[(mode, label)].append(float(r["Counter_Value"]))
    return {k: sum(v) / len(v) for k, v in acc.items()}


SIMDS = 1024   # 256 CUs x 4


def counter_section(dirs, durs, sets_per_stage):
    """Per-stage means of every counter of the extra passes, plus the L2 hit rate and the MFMA
    busy cycles per SIMD per second of the stage."""
    vals = collections.defaultdict(dict)
    names = []
    for d in dirs:
        path = os.path.join(d, "run_counter_collection.csv")
        for c in sorted({r["Counter_Name"] for r in csv.DictReader(open(path))}):
            names.append(c)
            for key, v in per_stage_counter(path, c, sets_per_stage).items():
                vals[key][c] = v
    out = ["", "## Grouped GEMM stages: cache and issue counters (mean per launch)", "",
           "| stage | expert set | " + " | ".join(names) + " | L2 hit % | MFMA busy G cycles/s per SIMD |",
           "|---|---|" + "---:|" * (len(names) + 2)]
    for key in sorted(vals, key=lambda k: (MODES.index(k[0]), k[1])):
        v = vals[key]
        dur = sum(durs[key]) / len(durs[key]) * 1e-6 if durs.get(key) else float("nan")
        hit = miss = float("nan")
        if "TCC_HIT_sum" in v and "TCC_MISS_sum" in v:
            hit, miss = v["TCC_HIT_sum"], v["TCC_MISS_sum"]
        rate = v.get("SQ_VALU_MFMA_BUSY_CYCLES", float("nan")) / SIMDS / dur / 1e9
        out.append(f"| {key[0]} | {key[1]} | " + " | ".join(f"{v.get(c, float('nan')):.4g}" for c in names)
                   + f" | {100.0 * hit / (hit + miss):.1f} | {rate:.3f} |")
    out += ["", "L2 hit % = TCC_HIT / (TCC_HIT + TCC_MISS). MFMA busy rate = SQ_VALU_MFMA_BUSY_CYCLES per SIMD "
            f"({SIMDS} SIMDs) over the stage's trace duration: divided by the shader clock it is the share of "
            "time the matrix unit was busy (0.35 of 2.4 GHz, 0.41 of 2.06 GHz for 0.85)."]
    return out


def main(argv=None) -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("--trace", required=True)
    ap.add_argument("--fetch", help="FETCH_SIZE pass (omit both counter passes for a trace-only summary)")
    ap.add_argument("--write")
    ap.add_argument("--workload", required=True)
    ap.add_argument("--copy-mb", type=int, default=0)
    ap.add_argument("--command", required=True)
    ap.add_argument("--out", required=True)
    ap.add_argument("--traffic-json")
    ap.add_argument("--sets-per-stage", type=int, choices=(1, 2), default=1)
    ap.add_argument("--pmc", action="append", default=[],
                    help="a further counter pass (cache and issue counters), repeatable")
    a = ap.parse_args(argv)

    stats = list(csv.DictReader(open(os.path.join(a.trace, "run_kernel_stats.csv"))))
    trace = list(csv.DictReader(open(os.path.join(a.trace, "run_kernel_trace.csv"))))
    # per-stage durations from the trace
    durs = collections.defaultdict(list)
    for r, mode, label in labelled_dispatches(trace, "Kernel_Name", "Dispatch_Id", a.sets_per_stage):
        if mode:
            durs[(mode, label)].append((int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3)
    if not (a.fetch and a.write):
        lines = [f"# rocprofv3 summary: kernels of one layer step, workload {a.workload}", "",
                 "Command (run from the repository root on one MI355X):", "", "```", a.command, "```", "",
                 "## Kernel statistics (--kernel-trace --stats)", "",
                 "| kernel | calls | avg us | total us | % |", "|---|---:|---:|---:|---:|"]
        for r in stats:
            lines.append(f"| {short_name(r['Name'])} | {r['Calls']} | {float(r['AverageNs']) / 1e3:.1f} | "
                         f"{float(r['TotalDurationNs']) / 1e3:.1f} | {float(r['Percentage']):.2f} |")
        open(a.out, "w").write("\n".join(lines) + "\n")
        print("\n".join(lines))
        return 0
    fcsv = os.path.join(a.fetch, "run_counter_collection.csv")
    wcsv = os.path.join(a.write, "run_counter_collection.csv")
    fs = copy_scale(fcsv, "FETCH_SIZE", a.copy_mb)
    ws = copy_scale(wcsv, "WRITE_SIZE", a.copy_mb)
    fetch = per_stage_counter(fcsv, "FETCH_SIZE", a.sets_per_stage)
    write = per_stage_counter(wcsv, "WRITE_SIZE", a.sets_per_stage)

    lines = [f"# rocprofv3 summary: grouped GEMM and other kernels, workload {a.workload}", "",
             "Command (run from the repository root on one MI355X):", "", "```", a.command, "```", "",
             f"grouped-GEMM sources ({', '.join(GEMM_SOURCES)}) sha256[:16] = {kernel_source_sha()}", "",
             "## Kernel statistics (--kernel-trace --stats)", "",
             "| kernel | calls | avg us | total us | % |", "|---|---:|---:|---:|---:|"]
    for r in stats:
        lines.append(f"| {short_name(r['Name'])} | {r['Calls']} | {float(r['AverageNs']) / 1e3:.1f} | "
                     f"{float(r['TotalDurationNs']) / 1e3:.1f} | {float(r['Percentage']):.2f} |")
    lines += ["", "## Grouped GEMM stages: duration and HBM traffic per launch", "",
              f"Counter calibration with a plain {a.copy_mb} MiB device copy: FETCH_SIZE x{fs:.3f}, "
              f"WRITE_SIZE x{ws:.3f} (KiB per dispatch -> bytes = KiB x 1024 x factor).", "",
              "| stage | expert set | avg us (trace) | HBM read MB | HBM write MB |",
              "|---|---|---:|---:|---:|"]
    traffic = {}
    for key in sorted(durs, key=lambda k: (MODES.index(k[0]), k[1])):
        d = sum(durs[key]) / len(durs[key])
        rd = fetch.get(key, float("nan")) * 1024 * (fs or 1)
        wr = write.get(key, float("nan")) * 1024 * (ws or 1)
        lines.append(f"| {key[0]} | {key[1]} | {d:.1f} | {rd / 1e6:.1f} | {wr / 1e6:.1f} |")
        stage = "shared_" + key[0] if key[1] == "shared" else key[0]
        traffic[stage] = {"bytes_per_launch": rd + wr, "read_bytes": rd, "write_bytes": wr,
                          "avg_us_trace": d, "kernel_source_sha": kernel_source_sha()}
    if a.pmc:
        lines += counter_section(a.pmc, durs, a.sets_per_stage)
    open(a.out, "w").write("\n".join(lines) + "\n")
    if a.traffic_json:
        allt = json.load(open(a.traffic_json)) if os.path.exists(a.traffic_json) else {}
        allt[a.workload] = traffic
        json.dump(allt, open(a.traffic_json, "w"), indent=1, sort_keys=True)
    print("\n".join(lines))
    return 0


if __name__ == "__main__":
    raise SystemExit(main())
