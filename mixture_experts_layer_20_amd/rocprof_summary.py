"""Summarise rocprofv3 output of bench.py runs into the text kept under profiles/.

Inputs (all written by rocprofv3 with --output-format csv):
  <trace dir>/run_kernel_stats.csv, run_kernel_trace.csv   from  --kernel-trace --stats
  <pmc dir>/run_counter_collection.csv                      from  --pmc FETCH_SIZE  (one pass)
  <pmc dir>/run_counter_collection.csv                      from  --pmc WRITE_SIZE  (one pass)
  <pmc dir>/run_counter_collection.csv                      from  --pmc <other counters>
                                                            (optional, --pmc, repeatable)
The bench runs must include `--copy-probe-mb N`: one plain device copy of N MiB whose counter
readings calibrate FETCH_SIZE / WRITE_SIZE (KiB per dispatch) to bytes.

Every kernel of the layer is attributed to the library call (stage) that launches it.  Each grouped
GEMM stage is one launch over the routed experts and the shared expert (a split weight-gradient
reduction adds a reduce launch).  Per stage: launch durations from the trace, HBM bytes per launch
from the counters, and the algorithmic work (FLOPs of the GEMM stages, bytes of the
bandwidth-bound ones) of the workload.

Usage:
  python -m mixture_experts_layer_20_amd.rocprof_summary --trace T [--fetch F --write W] \
      --workload large_e128 --copy-mb 256 --command "<the rocprofv3 commands>" \
      --out profiles/<name>.md [--traffic-json profiles/traffic.json] [--pmc P ...]
"""
from __future__ import annotations

import argparse
import collections
import statistics
import csv
import hashlib
import json
import os
import re
import sys

MODES = ["gate_up_fwd", "down_fwd", "down_bwd", "gate_up_dgrad", "down_wgrad", "gate_up_wgrad"]
PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)

GEMM_SOURCES = ("common.h", "gemm_common.h", "grouped_gemm.hip", "grouped_gemm_pipe.hip")
PEAK_BF16_TFLOPS = 2500.0
PEAK_HBM_GBS = 8000.0
SIMDS = 1024   # 256 CUs x 4

# kernel name pattern -> stage (library call) that launches it; first match wins
STAGE_OF = [
    (r"router_logits|topk_gate", "route"),
    (r"local_rank|scan_lds|scan_kernel|scatter_gather|scan_gather|rank_scan", "permute"),
    (r"combine_bwd(_k)?_kernel", "combine_bwd"),
    (r"combine(_k)?_kernel", "combine"),
    (r"route_bwd|route_dx|route_dw", "route_bwd"),
    (r"permute_bwd(_k)?_kernel", "permute_bwd"),
    (r"aux_", "router_aux"),
    (r"mx_", "mxfp8"),
]


def kernel_source_sha() -> str:
    """Hash of the grouped-GEMM sources: counter readings are valid only for the code they came from."""
    h = hashlib.sha256()
    for name in GEMM_SOURCES:
        h.update(open(os.path.join(PKG, "csrc", name), "rb").read())
    return h.hexdigest()[:16]


def gemm_mode(name: str) -> str | None:
    m = re.search(r"(?:grouped_gemm_(?:bf16|bf16_dma|pipe|f32)|splitk_reduce)<(\d)[,>]", name)
    return MODES[int(m.group(1))] if m else None


def stage_of(name: str) -> str | None:
    mode = gemm_mode(name)
    if mode:
        return mode
    for pat, st in STAGE_OF:
        if re.search(pat, name):
            return st
    return None


def short_name(name: str) -> str:
    m = re.search(r"grouped_gemm_bf16<(\d), [^>]*Cfg<(\d+), (\d+), (\d), (\d)>", name)
    if m:
        return f"grouped_gemm_bf16[{MODES[int(m.group(1))]}, {m.group(2)}x{m.group(3)}, {int(m.group(4)) * int(m.group(5))} waves]"
    m = re.search(r"(mx_gemm_pipe_kernel|mx_gemm_kernel)<(\d), (true|false)(?:, (\d+))?>", name)
    if m:
        epi = "wgrad" if m.group(3) == "true" else ("store", "swiglu", "swiglu_bwd")[int(m.group(2))]
        sw = f", {m.group(4)}-byte scales" if m.group(4) else ""
        return f"{m.group(1)}[{epi}{sw}]"
    m = re.search(r"(grouped_gemm_pipe|grouped_gemm_bf16_dma|splitk_reduce)<(\d)>", name)
    if m:
        return f"{m.group(1)}[{MODES[int(m.group(2))]}]"
    n = re.sub(r"void |moe::|\(anonymous namespace\)::", "", name)
    n = re.sub(r"\(.*", "", n)
    return n.strip()


def copy_scale(pmc_csv: str, counter: str, copy_mb: int) -> float | None:
    vals = [float(r["Counter_Value"]) for r in csv.DictReader(open(pmc_csv))
            if r["Counter_Name"] == counter and "copyBuffer" in r["Kernel_Name"] and int(r["Grid_Size"]) > 4096]
    if not vals:
        return None
    return copy_mb * 1024.0 / (sum(vals) / len(vals))


def per_kernel_counter(pmc_csv: str, counter: str):
    """Mean of a counter per launch of each kernel (short name)."""
    acc = collections.defaultdict(list)
    for r in csv.DictReader(open(pmc_csv)):
        if r["Counter_Name"] == counter:
            acc[short_name(r["Kernel_Name"])].append(float(r["Counter_Value"]))
    return {k: sum(v) / len(v) for k, v in acc.items()}


def algorithmic(workload: str):
    """FLOPs of each GEMM stage and bytes of each bandwidth-bound stage of one step (bench.py's
    formulas, imported so the two cannot drift apart)."""
    if ROOT not in sys.path:
        sys.path.insert(0, ROOT)
    import bench
    from mixture_experts_layer_20_amd import inputs as I
    cfg = I.CONFIGS[workload]
    return bench.stage_flops(cfg), bench.stage_bytes(cfg)


def counter_section(dirs, kdur):
    """Mean per launch of every counter of the extra passes, per kernel, plus the L2 hit rate and
    the MFMA busy cycles per SIMD per second of the launch."""
    vals = collections.defaultdict(dict)
    names = []
    for d in dirs:
        path = os.path.join(d, "run_counter_collection.csv")
        for c in sorted({r["Counter_Name"] for r in csv.DictReader(open(path))}):
            names.append(c)
            for k, v in per_kernel_counter(path, c).items():
                vals[k][c] = v
    out = ["", "## Cache and issue counters (mean per launch)", "",
           "| kernel | " + " | ".join(names) + " | L2 hit % | MFMA busy G cycles/s per SIMD |",
           "|---|" + "---:|" * (len(names) + 2)]
    for k in sorted(vals, key=lambda k: -kdur.get(k, 0.0)):
        v = vals[k]
        dur = kdur.get(k, float("nan")) * 1e-6
        hit = miss = float("nan")
        if "TCC_HIT_sum" in v and "TCC_MISS_sum" in v:
            hit, miss = v["TCC_HIT_sum"], v["TCC_MISS_sum"]
        rate = v.get("SQ_VALU_MFMA_BUSY_CYCLES", float("nan")) / SIMDS / dur / 1e9
        hitp = 100.0 * hit / (hit + miss) if hit + miss > 0 else float("nan")
        out.append(f"| {k} | " + " | ".join(f"{v.get(c, float('nan')):.4g}" for c in names)
                   + f" | {hitp:.1f} | {rate:.3f} |")
    out += ["", "L2 hit % = TCC_HIT / (TCC_HIT + TCC_MISS). MFMA busy rate = SQ_VALU_MFMA_BUSY_CYCLES per SIMD "
            f"({SIMDS} SIMDs) over the launch's trace duration: divided by the shader clock it is the share of "
            "time the matrix unit was busy."]
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
    ap.add_argument("--pmc", action="append", default=[],
                    help="a further counter pass (cache and issue counters), repeatable")
    a = ap.parse_args(argv)

    stats = list(csv.DictReader(open(os.path.join(a.trace, "run_kernel_stats.csv"))))
    trace = list(csv.DictReader(open(os.path.join(a.trace, "run_kernel_trace.csv"))))
    kd = collections.defaultdict(list)      # short kernel name -> launch durations (us)
    kstage = {}
    for r in trace:
        n = short_name(r["Kernel_Name"])
        kd[n].append((int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3)
        kstage[n] = stage_of(r["Kernel_Name"])
    # Median launch duration: the profiled command's first launches (warm-up, cold caches) and the
    # per-call pass (events around every call, slowed by the tracer) would pull a mean away from the
    # steady state that bench.py's events measure.
    kdur = {k: statistics.median(v) for k, v in kd.items()}
    flops, hbm_bytes = algorithmic(a.workload)

    lines = [f"# rocprofv3 summary: kernels of the layer step, workload {a.workload}", "",
             "Command (run from the repository root on one MI355X):", "", "```", a.command, "```", "",
             f"grouped-GEMM sources ({', '.join(GEMM_SOURCES)}) sha256[:16] = {kernel_source_sha()}", "",
             "## Kernel statistics (--kernel-trace --stats)", "",
             "| kernel | stage | calls | avg us | total us | % |", "|---|---|---:|---:|---:|---:|"]
    for r in stats:
        n = short_name(r["Name"])
        lines.append(f"| {n} | {kstage.get(n) or '-'} | {r['Calls']} | {float(r['AverageNs']) / 1e3:.1f} | "
                     f"{float(r['TotalDurationNs']) / 1e3:.1f} | {float(r['Percentage']):.2f} |")

    # The GEMM launches: the grouped GEMM kernel of each stage (its split reduce listed apart).
    gemm_k = {k: s for k, s in kstage.items() if s in MODES and not k.startswith("splitk_reduce")}
    lines += ["", "## Grouped GEMM launches (one per stage: routed experts + shared expert)", "",
              "Duration: the median of the kernel's launches in the trace.", "",
              "| stage | kernel | median us | algorithmic TFLOP | TFLOP/s | of 2.5 PFLOP/s bf16 |",
              "|---|---|---:|---:|---:|---:|"]
    best = None
    for k, s in sorted(gemm_k.items(), key=lambda kv: MODES.index(kv[1])):
        if s not in flops:
            continue
        rate = flops[s] / (kdur[k] * 1e-6) / 1e12
        lines.append(f"| {s} | {k} | {kdur[k]:.1f} | {flops[s] / 1e12:.3f} | {rate:.1f} | {rate / PEAK_BF16_TFLOPS:.3f} |")
        if best is None or kdur[k] > kdur[best[0]]:
            best = (k, s, rate)
    if best:
        lines += ["", f"Dominant kernel (longest launch): {best[0]} ({best[1]}), {kdur[best[0]]:.1f} us, "
                      f"{best[2]:.1f} TFLOP/s = {best[2] / PEAK_BF16_TFLOPS:.3f} of the bf16 peak."]

    traffic = {}
    if a.fetch and a.write:
        fcsv = os.path.join(a.fetch, "run_counter_collection.csv")
        wcsv = os.path.join(a.write, "run_counter_collection.csv")
        fs = copy_scale(fcsv, "FETCH_SIZE", a.copy_mb)
        ws = copy_scale(wcsv, "WRITE_SIZE", a.copy_mb)
        fetch = per_kernel_counter(fcsv, "FETCH_SIZE")
        write = per_kernel_counter(wcsv, "WRITE_SIZE")
        lines += ["", "## HBM traffic per launch (FETCH_SIZE, WRITE_SIZE)", "",
                  f"Calibration with a plain {a.copy_mb} MiB device copy: FETCH_SIZE x{fs:.3f}, "
                  f"WRITE_SIZE x{ws:.3f} (KiB per dispatch -> bytes = KiB x 1024 x factor).", "",
                  "| kernel | stage | median us | read MB | write MB | GB/s (counters) | of 8 TB/s |",
                  "|---|---|---:|---:|---:|---:|---:|"]
        per_stage = collections.defaultdict(lambda: [0.0, 0.0, 0.0])   # us, read, write per step-call
        for k in sorted(kdur, key=lambda k: -kdur[k]):
            st = kstage.get(k)
            if st is None or k not in fetch:
                continue
            rd = fetch[k] * 1024 * (fs or 1)
            wr = write.get(k, float("nan")) * 1024 * (ws or 1)
            gbs = (rd + wr) / (kdur[k] * 1e-6) / 1e9
            lines.append(f"| {k} | {st} | {kdur[k]:.1f} | {rd / 1e6:.1f} | {wr / 1e6:.1f} | {gbs:.0f} | "
                         f"{gbs / PEAK_HBM_GBS:.3f} |")
            if st in hbm_bytes or st in MODES:
                # launches per call of the stage: GEMM stages and the data-movement calls launch
                # each of their kernels once per call
                ps = per_stage[st]
                ps[0] += kdur[k]
                ps[1] += rd
                ps[2] += wr
        lines += ["", "## Bandwidth-bound stages: counters against the algorithmic bytes", "",
                  "| stage | kernels us | counter MB | algorithmic MB | ratio | GB/s (algorithmic) | of 8 TB/s |",
                  "|---|---:|---:|---:|---:|---:|---:|"]
        for st in ("permute", "combine", "combine_bwd", "permute_bwd"):
            if st in per_stage and st in hbm_bytes:
                us, rd, wr = per_stage[st]
                alg = hbm_bytes[st]
                gbs = alg / (us * 1e-6) / 1e9
                lines.append(f"| {st} | {us:.1f} | {(rd + wr) / 1e6:.1f} | {alg / 1e6:.1f} | {(rd + wr) / alg:.2f} | "
                             f"{gbs:.0f} | {gbs / PEAK_HBM_GBS:.3f} |")
        for k, s in gemm_k.items():
            rd = fetch.get(k, 0.0) * 1024 * (fs or 1)
            wr = write.get(k, 0.0) * 1024 * (ws or 1)
            traffic[s] = {"bytes_per_launch": rd + wr, "read_bytes": rd, "write_bytes": wr,
                          "avg_us_trace": kdur[k], "kernel_source_sha": kernel_source_sha()}
    if a.pmc:
        lines += counter_section(a.pmc, kdur)
    open(a.out, "w").write("\n".join(lines) + "\n")
    if a.traffic_json and traffic:
        allt = json.load(open(a.traffic_json)) if os.path.exists(a.traffic_json) else {}
        allt[a.workload] = traffic
        json.dump(allt, open(a.traffic_json, "w"), indent=1, sort_keys=True)
    print("\n".join(lines))
    return 0


if __name__ == "__main__":
    raise SystemExit(main())
