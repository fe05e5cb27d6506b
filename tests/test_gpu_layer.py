"""Whole-layer parity of the HIP path against the CPU oracle (GPU): small workloads compared element by
element, the full-size workloads (in the launch configuration the benchmark times) compared bit for
bit on routing and permutation and on sampled tokens and experts for the floating-point results,
edge cases, and run-to-run bitwise determinism."""
import numpy as np
import pytest
import torch

from mixture_experts_layer_20_amd import inputs as I
from oracle import moe_oracle as O
from mixture_experts_layer_20_amd import layer as LY
from tests.gpu_helpers import (DEV, TOL, assert_close, expert_weight_grads, full_routing, log, run_layer_gpu,
                               sampled_token_oracle, tnp)

pytestmark = pytest.mark.gpu

SMALL = {
    # name: config
    "tiny_fp32": I.CONFIGS["tiny_fp32"],
    "fp32_fwd_bwd_learned_bias": I.CONFIGS["tiny_fp32"].with_(name="f32bwd", T=300, E=8, k=2, f=256, fs=128,
                                                               bias_std=1.0, backward=True),
    "bf16_random_ragged": I.CONFIGS["tiny64e_random"].with_(name="bf16r", T=1000, d=256, E=16, f=256, fs=256),
    "bf16_learned_skew": I.CONFIGS["tiny64e_learned_skew"].with_(name="bf16s", T=777, d=384, E=32, f=384,
                                                                  fs=128),
    "bf16_top8_e256": I.CONFIGS["tiny64e_random"].with_(name="top8", T=200, d=128, E=256, k=8, f=128, fs=128),
    "bf16_single_token": I.CONFIGS["tiny64e_learned_skew"].with_(name="one", T=1, d=128, E=4, k=1, f=128,
                                                                  fs=128),
    "bf16_one_expert": I.CONFIGS["tiny64e_learned_skew"].with_(name="e1", T=130, d=128, E=1, k=1, f=256, fs=0),
    "bf16_all_to_few_experts": I.CONFIGS["tiny64e_learned_skew"].with_(name="few", T=600, d=256, E=16, k=2,
                                                                        f=128, fs=128, bias_std=40.0),
}


def compare_layer(cfg, lay, fwd, bwd):
    tol = TOL[cfg.dtype]
    b = lay.bufs
    for key in ("topk_idx", "counts", "offsets", "dest_pos", "src_row"):
        assert np.array_equal(tnp(b[key]).reshape(-1), np.asarray(fwd[key]).reshape(-1)), key
    if cfg.routing == "learned":
        assert np.array_equal(tnp(b["logits"]).view(np.uint32), fwd["logits"].view(np.uint32)), "logits"
    assert np.array_equal(tnp(b["x_perm"]), fwd["X_perm"].astype(np.float32)), "x_perm"
    assert_close("gates", tnp(b["gate"]), fwd["gates"], 1e-6)
    assert_close("out", tnp(b["out"]), fwd["out"], tol)
    if bwd is None:
        return
    assert_close("dx", tnp(b["dx"]), bwd["dx"], tol)
    for g, r in (("dw1", "dW1"), ("dw3", "dW3"), ("dw2", "dW2")):
        assert_close(g, tnp(b[g]), bwd[r], tol)
    if cfg.fs:
        for g, r in (("dws1", "dWs1"), ("dws3", "dWs3"), ("dws2", "dWs2")):
            assert_close(g, tnp(b[g]), bwd[r], tol)
    if cfg.routing == "learned":
        assert_close("dgate", tnp(b["dgate"]), bwd["dgates"], max(tol, 1e-5))
        assert_close("dwr", tnp(b["dwr"]), bwd["dWr"], tol)


@pytest.mark.parametrize("name", list(SMALL))
def test_small_layer_matches_oracle(name):
    cfg = SMALL[name]
    log(f"layer {name}: {cfg}")
    inp = I.make_inputs(cfg)
    lay = run_layer_gpu(cfg, inp)
    fwd, bwd = O.run_layer(cfg, I.values(inp))
    compare_layer(cfg, lay, fwd, bwd)


def test_layer_is_bitwise_deterministic():
    cfg = SMALL["bf16_learned_skew"]
    inp = I.make_inputs(cfg)
    lay = run_layer_gpu(cfg, inp)
    first = {k: v.clone() for k, v in lay.bufs.t.items() if not k.startswith("ws")}
    for _ in range(2):
        lay.step()
        torch.cuda.synchronize()
        for k, v in first.items():
            assert torch.equal(v, lay.bufs[k]), k


def test_layer_step_replays_as_hip_graph():
    """The whole step captured once as a HIP graph (nothing in the path allocates, clears memory or
    synchronizes): every replay, with eager steps in between, reproduces the eager step bit for bit,
    also after its outputs were overwritten."""
    cfg = SMALL["bf16_learned_skew"]
    inp = I.make_inputs(cfg)
    lay = run_layer_gpu(cfg, inp)
    keys = [k for k in lay.bufs.t if not k.startswith("ws") and k != "shared_offsets"]
    ref = {k: lay.bufs[k].clone() for k in keys}
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        lay.step()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        lay.step()
    torch.cuda.synchronize()
    for rep in range(3):
        for k in keys:
            lay.bufs[k].fill_(float("nan") if lay.bufs[k].is_floating_point() else -1)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for k in keys:
            assert torch.equal(lay.bufs[k], ref[k]), f"replay {rep}: {k}"
        lay.step()
        torch.cuda.synchronize()
        for k in keys:
            assert torch.equal(lay.bufs[k], ref[k]), f"eager step after replay {rep}: {k}"


@pytest.mark.parametrize("name", ["fp32_fwd_bwd_learned_bias", "bf16_random_ragged", "bf16_learned_skew"])
def test_recompute_layer_matches_oracle(name):
    """Per-layer recompute variant (no A/B stash in the forward, gate/up GEMM rerun in the backward)
    against the oracle, which keeps the stash."""
    cfg = SMALL[name]
    log(f"layer {name} with recompute: {cfg}")
    inp = I.make_inputs(cfg)
    lay = run_layer_gpu(cfg, inp, recompute=True)
    fwd, bwd = O.run_layer(cfg, I.values(inp))
    compare_layer(cfg, lay, fwd, bwd)


def test_recompute_is_bitwise_the_stashing_pass():
    """At the benchmark's shape and launch configuration the recompute variant reproduces every
    output of the stashing pass bit for bit (the kernels are deterministic)."""
    cfg = I.CONFIGS["tiny64e_random"]
    log(f"recompute vs stash, full size: {cfg}")
    inp = I.make_inputs(cfg)
    ref = run_layer_gpu(cfg, inp)
    keep = {k: ref.bufs[k].clone() for k in ("out", "dx", "dw1", "dw3", "dw2", "dws1", "dws3", "dws2", "a", "b", "h")}
    del ref
    torch.cuda.empty_cache()
    lay = run_layer_gpu(cfg, inp, recompute=True)
    for k, v in keep.items():
        assert torch.equal(v, lay.bufs[k]), k


@pytest.mark.parametrize("name", ["fp32_fwd_bwd_learned_bias", "bf16_learned_skew", "bf16_all_to_few_experts"])
def test_layer_with_load_balancing_loss_matches_oracle(name):
    cfg = SMALL[name]
    w = 0.05
    log(f"layer {name} with load-balancing loss {w}: {cfg}")
    inp = I.make_inputs(cfg)
    params = LY.upload_inputs(inp, DEV)
    lay = LY.MoELayer(cfg, params, lbl_weight=w)
    lay.step()
    torch.cuda.synchronize()
    fwd, bwd = O.run_layer(cfg, I.values(inp), lbl_weight=w)
    compare_layer(cfg, lay, fwd, bwd)
    assert_close("P", tnp(lay.bufs["prob_mean"]), fwd["P"], 1e-5)
    assert_close("f", tnp(lay.bufs["load_frac"]), fwd["f"], 1e-6)
    assert abs(tnp(lay.bufs["lbl_loss"])[0] - fwd["lbl"]) <= 1e-5 * abs(fwd["lbl"])


FULL = ["tiny64e_random", "tiny64e_learned_skew", "e128_2seq", "e32_2seq", "e8_2seq", "large_e128"]


@pytest.mark.parametrize("name", FULL)
def test_full_size_layer_sampled(name):
    cfg = I.CONFIGS[name]
    log(f"full-size layer {name}: {cfg}")
    inp = I.make_inputs(cfg)
    vals = I.values(inp)
    lay = run_layer_gpu(cfg, inp)
    b = lay.bufs
    tol = TOL[cfg.dtype]
    # Routing, dispatch and the row copy over the whole batch: bit-exact.
    R = full_routing(cfg, vals)
    for key in ("topk_idx", "counts", "offsets", "dest_pos", "src_row"):
        assert np.array_equal(tnp(b[key]).reshape(-1), np.asarray(R[key]).reshape(-1)), key
    if cfg.routing == "learned":
        assert np.array_equal(tnp(b["logits"]).view(np.uint32), R["logits"].view(np.uint32)), "logits"
    xp = b["x_perm"]
    rows = np.random.default_rng(0).choice(cfg.Tk, 512, replace=False)
    got_rows = tnp(xp[torch.from_numpy(rows).to(xp.device)])
    assert np.array_equal(got_rows, vals["x"][R["src_row"][rows] // cfg.k]), "x_perm rows"
    assert_close("gates", tnp(b["gate"]), R["gates"], 1e-6)
    # Per-token results on a sample of tokens.
    toks = np.sort(np.random.default_rng(1).choice(cfg.T, 48, replace=False))
    sf, sb = sampled_token_oracle(cfg, vals, toks)
    tt = torch.from_numpy(toks).to(xp.device)
    assert_close("out[sample]", tnp(b["out"][tt]), sf["out"], tol)
    assert_close("dx[sample]", tnp(b["dx"][tt]), sb["dx"], tol)
    if cfg.routing == "learned":
        assert_close("dgate[sample]", tnp(b["dgate"][tt]), sb["dgates"], tol)
    # Weight gradients of the busiest, the least busy non-empty and the median-load expert, and of
    # one expert of 257..320 rows if there is one (a single 320-row tile in the forward products).
    counts = R["counts"]
    nz = np.nonzero(counts)[0]
    pick = {int(nz[np.argmax(counts[nz])]), int(nz[np.argmin(counts[nz])]),
            int(nz[np.argsort(counts[nz])[len(nz) // 2]])}
    mid = np.nonzero((counts > 256) & (counts <= 320))[0]
    if len(mid):
        pick.add(int(mid[0]))
    for e in sorted(pick):
        dW1, dW3, dW2 = expert_weight_grads(cfg, vals, R, e, None)
        assert_close(f"dw1[{e}]", tnp(b["dw1"][e]), dW1, tol)
        assert_close(f"dw3[{e}]", tnp(b["dw3"][e]), dW3, tol)
        assert_close(f"dw2[{e}]", tnp(b["dw2"][e]), dW2, tol)
    for e in np.nonzero(counts == 0)[0]:
        assert bool((b["dw1"][int(e)] == 0).all()), f"empty expert {e} has a nonzero gradient"
    # Router weight gradient of the least busy non-empty expert: it depends only on the tokens
    # that chose that expert, so the oracle runs on exactly those tokens.
    if cfg.routing == "learned":
        e = int(nz[np.argmin(counts[nz])])
        toks_e = np.nonzero((R["topk_idx"] == e).any(axis=1))[0]
        _, eb = sampled_token_oracle(cfg, vals, toks_e)
        dwr_e = eb["dlogits"][:, e] @ vals["x"][toks_e].astype(np.float64)
        assert_close(f"dwr[{e}]", tnp(b["dwr"][e]), dwr_e, tol)
    # Shared expert weight gradients on sampled rows / columns (exact over all tokens).
    if cfg.fs:
        x = vals["x"].astype(np.float64)
        dout = vals["dout"].astype(np.float64)
        ws1, ws3, ws2 = (vals[k].astype(np.float64) for k in ("ws1", "ws3", "ws2"))
        cols = np.random.default_rng(2).choice(cfg.fs, 4, replace=False)
        As = x @ ws1[cols].T
        Bs = x @ ws3[cols].T
        s = O.sigmoid(As)
        dHs = dout @ ws2[:, cols]
        dAs = dHs * Bs * s * (1 + As * (1 - s))
        dBs = dHs * As * s
        assert_close("dws1[rows]", tnp(b["dws1"][torch.from_numpy(cols).to(xp.device)]), dAs.T @ x, tol)
        assert_close("dws3[rows]", tnp(b["dws3"][torch.from_numpy(cols).to(xp.device)]), dBs.T @ x, tol)
        Hs = As * s * Bs
        assert_close("dws2[:,cols]", tnp(b["dws2"][:, torch.from_numpy(cols).to(xp.device)]), dout.T @ Hs, tol)
