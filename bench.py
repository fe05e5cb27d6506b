"""Benchmark: one GPU's MoE layer, forward+backward, on device-resident synthetic inputs.

Default workload `large_e128`: one 8192-token sequence, d_model 4096, 128 experts, top-4 learned
softmax router, expert d_ff 2048 plus one shared expert of d_ff 4096, bf16 storage with fp32
accumulation -- the 128-expert operating point of the Olmo-core DDP MoE examples ("Production
throughput runs": sequence 8192, top-4, one shared expert) and the largest workload that runs
here.  A step is one full pass of the path: route -> permute -> grouped SwiGLU experts + shared
expert -> combine -> combine backward -> router backward -> expert and shared dgrad/wgrad ->
permute backward.

Timing: W untimed warm-up steps, then K timed steps, each preceded by a write of a 512 MiB
scratch buffer that evicts the L2 caches and the 256 MiB last-level cache, with HIP events on the
launch stream around every step (not around the flush); `ms_per_step` is the median of those K
step times and `value` the tokens per second it gives.  A second loop of K steps without flushes
gives the warm-cache numbers.  Per-call times come from a separate pass with events around every
library call, so the timed steps carry no per-call events.  Practical ceilings measured in the same
process: a device-to-device copy (bandwidth) and a square bf16 matrix product (matrix units).

Prints one JSON line.  `--gpus N` with N > 1 is not supported: libmoe runs on one GPU.
"""
from __future__ import annotations

import argparse
import json
import os
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "MoE-layer tokens/s fwd+bwd on 1 GPU; grouped-GEMM TFLOP/s (% bf16 MFMA peak)"
PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16 MFMA
PEAK_FP8_TFLOPS = 5000.0    # MI355X dense fp8 MFMA
PEAK_HBM_GBS = 8000.0

GEMM_STAGES = ("gate_up_fwd", "down_fwd", "down_bwd", "down_wgrad", "gate_up_dgrad", "gate_up_wgrad")


def stage_flops(cfg, merged=True, recompute=False):
    """Algorithmic FLOPs of each GEMM stage call of one step (2 per multiply-add, no padding).
    Merged: each stage runs the routed experts and the shared expert in one call.  Recompute: the
    backward repeats the gate/up GEMM (the recompute variant's extra work)."""
    Tk, T, d, f, fs = cfg.T * cfg.k, cfg.T, cfg.d, cfg.f, cfg.fs
    per_row = {"gate_up_fwd": 4.0, "down_fwd": 2.0, "down_bwd": 2.0, "down_wgrad": 2.0,
               "gate_up_dgrad": 4.0, "gate_up_wgrad": 4.0}
    stages = GEMM_STAGES if cfg.backward else ("gate_up_fwd", "down_fwd")
    fl = {}
    for s in stages:
        fl[s] = per_row[s] * Tk * d * f
        if fs:
            key = s if merged else "shared_" + s
            fl[key] = fl.get(key, 0.0) + per_row[s] * T * d * fs
    if recompute and cfg.backward:
        fl["gate_up_recompute"] = per_row["gate_up_fwd"] * Tk * d * f
        if fs:
            key = "gate_up_recompute" if merged else "shared_gate_up_recompute"
            fl[key] = fl.get(key, 0.0) + per_row["gate_up_fwd"] * T * d * fs
    return fl


def stage_bytes(cfg):
    """Algorithmic HBM bytes of the bandwidth-bound calls (each tensor read or written once)."""
    es = 2 if cfg.dtype == "bf16" else 4
    T, Tk, d = cfg.T, cfg.T * cfg.k, cfg.d
    row, perm = T * d * es, Tk * d * es
    shared = cfg.fs > 0
    learned = cfg.routing == "learned"
    b = {"permute": row + perm + 3 * Tk * 4,
         "combine": perm + row * (2 if shared else 1) + Tk * 8}
    if cfg.backward:
        b["combine_bwd"] = row + perm * (2 if learned else 1) + Tk * 8 + (Tk * 4 if learned else 0)
        b["permute_bwd"] = perm + row * (1 + int(shared) + int(learned)) + Tk * 4
    return b


def cpu_baseline(cfg, inp, sample_tokens, min_seconds=10.0, max_runs=4):
    """The oracle (as it stands) on the first `sample_tokens` tokens of the same workload, repeated
    until about `min_seconds` of CPU work have been timed (at most `max_runs` runs)."""
    from mixture_experts_layer_20_amd import inputs as I
    from oracle import moe_oracle as O
    vals = I.values(inp)
    n = min(sample_tokens, cfg.T)
    sub = dict(vals)
    for key in ("x", "logits", "dout"):
        if sub.get(key) is not None:
            sub[key] = vals[key][:n]
    c = cfg.with_(T=n)
    runs, total = 0, 0.0
    while runs < max_runs and (runs == 0 or total < min_seconds):
        t0 = time.perf_counter()
        O.run_layer(c, sub)
        total += time.perf_counter() - t0
        runs += 1
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:
        threads = len(os.sched_getaffinity(0))
    return {"value": n * runs / total, "unit": "tokens/s", "cores": int(threads), "kind": "oracle",
            "sample": f"first {n} of {cfg.T} tokens of the same workload, "
                      f"{'forward+backward' if cfg.backward else 'forward'}, numpy float64 oracle, "
                      f"{runs} run(s), {total:.1f} s total"}


def cpu_small_configs():
    """The oracle on the tiny fp32 workload (median of 5, all cores and one thread) and on a
    512-token sample of the Tiny-64E workload with one thread: fixed small reference points."""
    from threadpoolctl import threadpool_limits
    from mixture_experts_layer_20_amd import inputs as I
    from oracle import moe_oracle as O
    out = {}
    c0 = I.CONFIGS["tiny_fp32"]
    v0 = I.values(I.make_inputs(c0))
    for label, limit in (("all_cores", None), ("one_thread", 1)):
        times = []
        with threadpool_limits(limits=limit):
            for _ in range(5):
                t0 = time.perf_counter()
                O.run_layer(c0, v0)
                times.append(time.perf_counter() - t0)
        out[f"tiny_fp32_{label}"] = {"tokens_per_s": c0.T / statistics.median(times),
                                     "median_s": statistics.median(times), "runs": 5}
    c1 = I.CONFIGS["tiny64e_random"]
    v1 = I.values(I.make_inputs(c1))
    n = 512
    sub = dict(v1)
    for key in ("x", "logits", "dout"):
        sub[key] = v1[key][:n]
    with threadpool_limits(limits=1):
        O.run_layer(c1.with_(T=n), sub)
        t0 = time.perf_counter()
        O.run_layer(c1.with_(T=n), sub)
        dt = time.perf_counter() - t0
    out["tiny64e_random_one_thread"] = {"tokens_per_s": n / dt, "seconds": dt,
                                        "sample": f"first {n} of {c1.T} tokens, forward+backward"}
    return out


def pct(xs, q):
    """q-th percentile (linear interpolation) of a non-empty list."""
    s = sorted(xs)
    i = (len(s) - 1) * q / 100.0
    lo = int(i)
    hi = min(lo + 1, len(s) - 1)
    return s[lo] + (s[hi] - s[lo]) * (i - lo)


def timed_steps(lay, steps, flush):
    """K steps with events around each (flush before each when given); per-step ms and wall s."""
    import torch
    evs = []
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        if flush is not None:
            flush.fill_(1)
        s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        s.record()
        lay.step()
        e.record()
        evs.append((s, e))
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    return [s.elapsed_time(e) for s, e in evs], wall


def ceilings(dev):
    """Practical ceilings on this GPU: device copy bandwidth (torch copy of 2 GiB) and a square
    bf16 matrix product (torch.matmul, 8192^3), each the best of 10 event-timed runs."""
    import torch
    out = {}
    n = 2 << 30
    src = torch.empty(n, dtype=torch.uint8, device=dev)
    dst = torch.empty_like(src)
    best = float("inf")
    for _ in range(12):
        s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        s.record()
        dst.copy_(src)
        e.record()
        torch.cuda.synchronize()
        best = min(best, s.elapsed_time(e))
    out["device_copy_GBps"] = 2 * n / (best * 1e-3) / 1e9
    del src, dst
    m = 8192
    a = torch.randn(m, m, device=dev, dtype=torch.bfloat16)
    b = torch.randn(m, m, device=dev, dtype=torch.bfloat16)
    best = float("inf")
    for _ in range(12):
        s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        s.record()
        torch.matmul(a, b)
        e.record()
        torch.cuda.synchronize()
        best = min(best, s.elapsed_time(e))
    out["torch_matmul_bf16_8192_TFLOPs"] = 2 * m ** 3 / (best * 1e-3) / 1e12
    # the same product through libmoe's grouped GEMM (one group of 8192 rows, the down stage)
    from mixture_experts_layer_20_amd import libmoe as L
    offs = torch.tensor([0, m], dtype=torch.int32, device=dev)
    ws = torch.empty(max(256, L.moe_grouped_mlp_fwd_workspace_size(m, 1, m, m)), dtype=torch.uint8, device=dev)
    y = torch.empty(m, m, device=dev, dtype=torch.bfloat16)
    best = float("inf")
    for _ in range(12):
        s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        s.record()
        L.moe_expert_down_fwd(a, offs, 1, m, m, m, b, L.MOE_BF16, y, ws, ws.numel())
        e.record()
        torch.cuda.synchronize()
        best = min(best, s.elapsed_time(e))
    out["libmoe_grouped_gemm_bf16_8192_TFLOPs"] = 2 * m ** 3 / (best * 1e-3) / 1e12
    return out


def main(argv=None) -> int:
    ap = argparse.ArgumentParser(description=__doc__)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="large_e128")
    ap.add_argument("--flush-mb", type=int, default=512,
                    help="MiB of scratch written before each timed step to evict the caches (0: none)")
    ap.add_argument("--stage-steps", type=int, default=10,
                    help="steps of the separate pass with events around every library call")
    ap.add_argument("--cpu-sample-tokens", type=int, default=0,
                    help="tokens of the workload the oracle runs for cpu_baseline (0: a size that takes "
                         "about 10-30 s)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-ceilings", action="store_true")
    ap.add_argument("--cpu-small-configs", action="store_true",
                    help="also time the oracle on the tiny fp32 workload and a Tiny-64E sample, with one "
                         "thread and all cores")
    ap.add_argument("--lbl", type=float, default=0.0,
                    help="weight of the router's load-balancing loss (learned-routing workloads; 0: off)")
    ap.add_argument("--recompute", action="store_true",
                    help="per-layer recompute variant: no A/B stash in the forward, gate/up GEMM rerun in "
                         "the backward")
    ap.add_argument("--precision", choices=("bf16", "mxfp8"), default="bf16",
                    help="expert products in bf16, or in MXFP8 (E4M3 with one E8M0 scale per 32 elements)")
    ap.add_argument("--mx-cached-weights", action="store_true",
                    help="MXFP8: quantize the expert weights once before the timed steps (the optimizer-step "
                         "cadence, with several micro-batches per weight update) instead of in every pass")
    ap.add_argument("--no-merge", action="store_true",
                    help="one GEMM call per expert set instead of routed + shared in one call")
    ap.add_argument("--copy-probe-mb", type=int, default=0,
                    help="run one plain device copy of this many MiB first (counter calibration)")
    ap.add_argument("--traffic-json", default=os.path.join(ROOT, "profiles", "traffic.json"),
                    help="measured HBM bytes per launch (from rocprofv3 counters), if present")
    a = ap.parse_args(argv)
    if a.gpus != 1:
        print(f"bench.py runs one GPU's share of the layer only; --gpus {a.gpus} is not supported "
              "(libmoe has no multi-GPU path).", file=sys.stderr)
        return 2

    import torch
    from mixture_experts_layer_20_amd import inputs as I
    from mixture_experts_layer_20_amd import layer as LY
    from mixture_experts_layer_20_amd import libmoe

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        return 1
    libmoe.lib()   # fails loudly if the HIP library is missing
    cfg = I.CONFIGS[a.workload]
    print(f"[bench] generating inputs for {cfg.name}", file=sys.stderr, flush=True)
    inp = I.make_inputs(cfg)
    dev = torch.device("cuda:0")
    mx = a.precision == "mxfp8"
    merged = not (a.no_merge or mx)
    lay = LY.MoELayer(cfg, LY.upload_inputs(inp, dev), merge_shared=merged, recompute=a.recompute,
                      lbl_weight=a.lbl, precision=a.precision, mx_cached_weights=a.mx_cached_weights)
    if a.copy_probe_mb > 0:
        src = torch.empty(a.copy_probe_mb << 20, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
    flush = torch.empty(a.flush_mb << 20, dtype=torch.uint8, device=dev) if a.flush_mb > 0 else None
    print("[bench] warmup", file=sys.stderr, flush=True)
    for _ in range(a.warmup):
        lay.step()
    torch.cuda.synchronize()
    print("[bench] timing", file=sys.stderr, flush=True)
    cold, cold_wall = timed_steps(lay, a.steps, flush)
    warm, warm_wall = timed_steps(lay, a.steps, None)
    ms_per_step = statistics.median(cold)

    # Separate pass: events around every library call, on the launch stream.
    print("[bench] per-call pass", file=sys.stderr, flush=True)
    lay.events = {}
    for _ in range(a.stage_steps):
        lay.step()
    torch.cuda.synchronize()
    stages = {}
    for name, pairs in lay.events.items():
        ms = [s.elapsed_time(e) for s, e in pairs]
        stages[name] = sum(ms) / len(ms)
    lay.events = None
    flops = stage_flops(cfg, merged=merged, recompute=a.recompute)
    peak = PEAK_FP8_TFLOPS if mx else PEAK_BF16_TFLOPS
    gemm_ms = sum(stages[s] for s in flops if s in stages)
    gemm_flop = sum(flops.values())
    stage_tflops = {s: flops[s] / (stages[s] * 1e-3) / 1e12 for s in flops if s in stages}
    # The dominant kernel: the longest GEMM stage, weight gradients included.  Each stage is one
    # grouped-GEMM launch (a weight gradient whose reduction is split adds its reduce launch).
    dom = max((s for s in flops if s in stages), key=lambda s: stages[s])
    achieved = stage_tflops[dom]
    traffic = None
    if os.path.exists(a.traffic_json):
        try:
            tj = json.load(open(a.traffic_json))
            ent = tj.get(cfg.name, {}).get(dom)
            if ent and not mx and ent.get("kernel_source_sha") == _kernel_source_sha():
                traffic = ent["bytes_per_launch"]
        except Exception:
            traffic = None
    line = {
        "metric": METRIC,
        "value": cfg.T / (ms_per_step * 1e-3),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": a.steps,
        "warmup": a.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "mxfp8-e4m3 products, bf16 storage" if mx else cfg.dtype,
        "data": "synthetic (seeded Gaussian inputs and weights; random routing logits drawn per token)"
        if cfg.routing == "random" else "synthetic (seeded Gaussian inputs and weights, learned router)",
        "config": {"workload": cfg.name, "tokens": cfg.T, "d_model": cfg.d, "experts": cfg.E, "top_k": cfg.k,
                   "expert_d_ff": cfg.f, "shared_d_ff": cfg.fs, "routing": cfg.routing,
                   "backward": cfg.backward, "recompute": a.recompute, "precision": a.precision,
                   "mx_weights": ("quantized once (optimizer-step cadence)" if a.mx_cached_weights
                                  else "quantized every pass") if mx else None,
                   "lbl_weight": a.lbl if cfg.routing == "learned" else 0.0},
        "step_ms": {"median": ms_per_step, "p10": pct(cold, 10), "p90": pct(cold, 90),
                    "mean": statistics.fmean(cold), "caches_flushed_mb": a.flush_mb,
                    "wall_s_incl_flushes": cold_wall,
                    "warm_median": statistics.median(warm), "warm_p10": pct(warm, 10), "warm_p90": pct(warm, 90),
                    "warm_wall_ms_per_step": warm_wall * 1e3 / a.steps},
        "roofline": {"bound": "mfma", "kernel": dom, "achieved": achieved, "peak": peak,
                     "unit": "TFLOP/s", "frac": achieved / peak, "traffic": traffic},
        "grouped_gemm": {"tflops": gemm_flop / (gemm_ms * 1e-3) / 1e12,
                         "frac_peak": gemm_flop / (gemm_ms * 1e-3) / 1e12 / peak,
                         "ms": gemm_ms, "per_stage_tflops": stage_tflops},
        "stages_ms": stages,
        "hbm_bound_stages": {s: {"gbs": by / (stages[s] * 1e-3) / 1e9,
                                 "frac_hbm": by / (stages[s] * 1e-3) / 1e9 / PEAK_HBM_GBS,
                                 "bytes": by}
                             for s, by in stage_bytes(cfg).items() if s in stages},
    }
    if mx:
        # MXFP8 quantization passes (activations each product, weights in both orientations).
        qs = {k: v for k, v in stages.items() if k.startswith("q_") or k.startswith("shared_q_")}
        line["mxfp8_quantize_ms"] = sum(qs.values())
    del lay, flush
    torch.cuda.empty_cache()
    if not a.no_ceilings:
        print("[bench] ceilings", file=sys.stderr, flush=True)
        line["ceilings"] = ceilings(dev)
    if not a.no_cpu_baseline:
        print("[bench] cpu baseline (oracle)", file=sys.stderr, flush=True)
        n = a.cpu_sample_tokens or (512 if cfg.d * cfg.f * cfg.E > (1 << 28) else 8192)
        line["cpu_baseline"] = cpu_baseline(cfg, inp, n)
        if a.cpu_small_configs:
            line["cpu_baseline"]["small_configs"] = cpu_small_configs()
    print(json.dumps(line), flush=True)
    return 0


def _kernel_source_sha() -> str:
    from mixture_experts_layer_20_amd.rocprof_summary import kernel_source_sha
    return kernel_source_sha()


if __name__ == "__main__":
    sys.exit(main())
