"""Benchmark: one GPU's MoE layer, forward+backward, on device-resident synthetic inputs.

Default workload: one 8192-token sequence, d_model 2048, 64 experts, top-4 random routing, expert
and shared-expert d_ff 1024, bf16 storage with fp32 accumulation (the Tiny-64E operating point of
the Olmo-core DDP MoE examples, "Production throughput runs").  A step is one full pass of the
path: route -> permute -> grouped SwiGLU experts + shared expert -> combine -> combine backward ->
expert and shared dgrad/wgrad -> permute backward (+ router backward for learned routing).

Prints one JSON line.  `--gpus N` with N > 1 is not supported: libmoe runs on one GPU.
"""
from __future__ import annotations

import argparse
import json
import os
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


def main(argv=None) -> int:
    ap = argparse.ArgumentParser(description=__doc__)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="tiny64e_random")
    ap.add_argument("--cpu-sample-tokens", type=int, default=8192)
    ap.add_argument("--no-cpu-baseline", action="store_true")
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
    lay = LY.MoELayer(cfg, LY.upload_inputs(inp, dev), merge_shared=not (a.no_merge or mx), recompute=a.recompute,
                      lbl_weight=a.lbl, precision=a.precision, mx_cached_weights=a.mx_cached_weights)
    if a.copy_probe_mb > 0:
        src = torch.empty(a.copy_probe_mb << 20, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
    print("[bench] warmup", file=sys.stderr, flush=True)
    for _ in range(a.warmup):
        lay.step()
    torch.cuda.synchronize()
    lay.events = {}
    print("[bench] timing", file=sys.stderr, flush=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(a.steps):
        lay.step()
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    ms_per_step = elapsed * 1e3 / a.steps

    # Per-call device durations from the events recorded on the launch stream.
    stages = {}
    for name, pairs in lay.events.items():
        ms = [s.elapsed_time(e) for s, e in pairs]
        stages[name] = sum(ms) / len(ms)
    flops = stage_flops(cfg, merged=not (a.no_merge or mx), recompute=a.recompute)
    peak = PEAK_FP8_TFLOPS if mx else PEAK_BF16_TFLOPS
    gemm_ms = sum(stages[s] for s in flops if s in stages)
    gemm_flop = sum(flops.values())
    stage_tflops = {s: flops[s] / (stages[s] * 1e-3) / 1e12 for s in flops if s in stages}
    # The dominant GEMM kernel: the longest stage that is one kernel launch (a weight-gradient
    # stage is the GEMM plus its split-reduction pass).
    dom = max((s for s in GEMM_STAGES if s in stages and (mx or "wgrad" not in s)), key=lambda s: stages[s])
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
        "value": cfg.T * a.steps / elapsed,
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
    if not a.no_cpu_baseline:
        print("[bench] cpu baseline (oracle)", file=sys.stderr, flush=True)
        line["cpu_baseline"] = cpu_baseline(cfg, inp, a.cpu_sample_tokens)
    print(json.dumps(line), flush=True)
    return 0


def _kernel_source_sha() -> str:
    from mixture_experts_layer_20_amd.rocprof_summary import kernel_source_sha
    return kernel_source_sha()


if __name__ == "__main__":
    sys.exit(main())
