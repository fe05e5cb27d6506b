"""Helpers for the GPU parity tests: run the HIP path through the C-ABI and fetch its results, and
compute oracle values for sampled tokens / experts of full-size workloads."""
from __future__ import annotations

import sys

import numpy as np
import torch

from mixture_experts_layer_20_amd import inputs as I
from mixture_experts_layer_20_amd import layer as LY
from oracle import moe_oracle as O

DEV = torch.device("cuda:0")
TOL = {"f32": 1e-5, "bf16": 2e-2}


def log(msg: str) -> None:
    print(msg, flush=True)
    sys.stdout.flush()


def tnp(t: torch.Tensor) -> np.ndarray:
    """Device tensor -> numpy (bf16 widened exactly to fp32)."""
    if t.dtype == torch.bfloat16:
        return t.float().cpu().numpy()
    return t.cpu().numpy()


def dev_tensor(a: np.ndarray, dtype: str) -> torch.Tensor:
    """Upload values that are exactly representable in `dtype` ("bf16" values are rounded first)."""
    a = np.ascontiguousarray(a, np.float32)
    if dtype == "bf16":
        bits = I.bf16_bits_from_f32(a)
        return torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to(DEV)
    return torch.from_numpy(a).to(DEV)


def as_dtype_values(a: np.ndarray, dtype: str) -> np.ndarray:
    """The fp32 values the device sees after upload in `dtype`."""
    a = np.ascontiguousarray(a, np.float32)
    return I.f32_from_bf16_bits(I.bf16_bits_from_f32(a)) if dtype == "bf16" else a


def run_layer_gpu(cfg, inp, renormalize=1, recompute=False):
    params = LY.upload_inputs(inp, DEV)
    lay = LY.MoELayer(cfg, params, renormalize=renormalize, recompute=recompute)
    lay.step()
    torch.cuda.synchronize()
    return lay


def err(got, ref) -> float:
    return O.max_abs_rel_err(got, ref)


def assert_close(name, got, ref, tol):
    e = err(got, ref)
    assert e <= tol, f"{name}: max-abs-relative error {e:.3e} > {tol:.0e}"
    return e


def sampled_token_oracle(cfg, vals, tokens):
    """Oracle forward+backward restricted to the given tokens.  The layer acts on every token
    independently, so per-token outputs (out, gates, dgates, dx) of the sub-batch equal those of
    the full batch; weight gradients do not and are checked separately."""
    sub = dict(vals)
    for key in ("x", "logits", "dout"):
        if vals.get(key) is not None:
            sub[key] = vals[key][tokens]
    c = cfg.with_(T=len(tokens))
    return O.run_layer(c, sub)


def expert_weight_grads(cfg, vals, fwd_full_routing, e, gpu_gate):
    """Exact dW1[e], dW3[e], dW2[e] of the full batch: only the tokens routed to expert e matter.
    Uses the oracle's routing (bit-exact with the GPU's) and the oracle's own gates."""
    idx = fwd_full_routing["topk_idx"]
    gates = fwd_full_routing["gates"]
    tok, slot = np.nonzero(idx == e)
    order = np.argsort(tok * cfg.k + slot, kind="stable")
    tok, slot = tok[order], slot[order]
    X = vals["x"][tok].astype(np.float64)
    dY = gates[tok, slot][:, None] * vals["dout"][tok].astype(np.float64)
    A, B, H, Y = O.swiglu_forward(X, vals["w1"][e], vals["w3"][e], vals["w2"][e])
    dX, dW1, dW3, dW2, dA, dB = O.swiglu_backward(dY, X, A, B, H, vals["w1"][e], vals["w3"][e], vals["w2"][e])
    return dW1, dW3, dW2


def full_routing(cfg, vals):
    """Oracle routing of the whole batch: logits (canonical fp32), top-k, gates, dispatch."""
    if cfg.routing == "learned":
        logits = O.canonical_router_logits(vals["x"], vals["w_router"], vals["bias"])
    else:
        logits = vals["logits"]
    idx = O.select_topk(logits, cfg.k)
    gates = O.gate_weights(logits, idx)
    counts, offsets, dest_pos, src_row = O.dispatch_plan(idx, cfg.E)
    return dict(logits=logits, topk_idx=idx, gates=gates, counts=counts, offsets=offsets,
                dest_pos=dest_pos, src_row=src_row)
