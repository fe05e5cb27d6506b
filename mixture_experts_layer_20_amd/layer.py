"""The MoE layer (router -> dispatch -> grouped SwiGLU experts + shared expert -> combine, and the
backward) driven through libmoe's C-ABI.

This module only sequences library calls and owns the device buffers (allocated once with torch,
which serves as the device-memory and stream provider).  Every arithmetic step runs in libmoe's
HIP kernels.
"""
from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np
import torch

from . import libmoe as L
from .inputs import MoEConfig, Tensor


def to_device(t: Tensor | None, device) -> torch.Tensor | None:
    """Upload one input tensor (bf16 bit patterns become a bfloat16 tensor, fp32 stays fp32)."""
    if t is None:
        return None
    if t.is_bf16:
        return torch.from_numpy(np.ascontiguousarray(t.bits).view(np.int16)).view(torch.bfloat16).to(device)
    return torch.from_numpy(np.ascontiguousarray(t.value, np.float32)).to(device)


def upload_inputs(inp: dict, device) -> dict:
    return {k: to_device(v, device) for k, v in inp.items()}


@dataclass
class Buffers:
    """Every activation, gradient and workspace buffer of one layer pass, allocated once."""
    cfg: MoEConfig
    device: torch.device
    t: dict = field(default_factory=dict)

    @staticmethod
    def allocate(cfg: MoEConfig, device) -> "Buffers":
        T, d, E, k, f, fs = cfg.T, cfg.d, cfg.E, cfg.k, cfg.f, cfg.fs
        Tk = T * k
        dt = torch.bfloat16 if cfg.dtype == "bf16" else torch.float32
        e = lambda *s: torch.empty(*s, dtype=dt, device=device)
        i32 = lambda *s: torch.empty(*s, dtype=torch.int32, device=device)
        f32 = lambda *s: torch.empty(*s, dtype=torch.float32, device=device)
        u8 = lambda n: torch.empty(max(int(n), 256), dtype=torch.uint8, device=device)
        b = {}
        b["logits"] = f32(T, cfg.E)
        b["topk_idx"] = i32(T, k)
        b["gate"] = f32(T, k)
        b["counts"] = i32(E)
        b["offsets"] = i32(E + 1)
        b["dest_pos"] = i32(Tk)
        b["src_row"] = i32(Tk)
        b["x_perm"] = e(Tk, d)
        b["a"] = e(Tk, f)
        b["b"] = e(Tk, f)
        b["h"] = e(Tk, f)
        b["y"] = e(Tk, d)
        b["out"] = e(T, d)
        b["ws_perm"] = u8(L.moe_permute_workspace_size(T, E, k))
        sizing = [L.expert_set(None, E, Tk, f)] + ([L.expert_set(None, 1, T, fs)] if fs > 0 else [])
        b["ws_fwd"] = u8(L.moe_expert_stage_workspace_size(sizing, d))
        if fs > 0:
            b["shared_offsets"] = torch.tensor([0, T], dtype=torch.int32, device=device)
            b["as"] = e(T, fs)
            b["bs"] = e(T, fs)
            b["hs"] = e(T, fs)
            b["s"] = e(T, d)
        if cfg.backward:
            # Backward GEMM workspace: tile prefix plus room for split weight-gradient partials.
            b["ws_bwd"] = u8(L.moe_expert_stage_workspace_size(sizing, d))
            b["dy"] = e(Tk, d)
            b["dgate"] = f32(T, k)
            b["dab"] = e(Tk, 2 * f)
            b["dx_perm"] = e(Tk, d)
            b["dw1"] = e(E, f, d)
            b["dw3"] = e(E, f, d)
            b["dw2"] = e(E, d, f)
            b["dx"] = e(T, d)
            if fs > 0:
                b["dabs"] = e(T, 2 * fs)
                b["dx_shared"] = e(T, d)
                b["dws1"] = e(fs, d)
                b["dws3"] = e(fs, d)
                b["dws2"] = e(d, fs)
            if cfg.routing == "learned":
                b["dwr"] = f32(E, d)
                b["dx_router"] = e(T, d)
                b["ws_route"] = u8(L.moe_route_bwd_workspace_size(T, d, E, k))
        return Buffers(cfg, torch.device(device), b)

    def __getitem__(self, k):
        return self.t[k]


class MxSet:
    """Buffers and calls of one expert set (routed experts, or the shared expert as one group) in
    MXFP8: every product quantizes both operands along its contraction axis (E4M3 codes, one E8M0
    scale per 32 elements) and multiplies them on the block-scaled matrix instruction.  Weights are
    quantized once per pass in each orientation the products need."""

    KPAD = 128   # weight gradients: each group's rows padded to a multiple of this

    def __init__(self, offsets, G, M, d, f, device, backward):
        self.offsets, self.G, self.M, self.d, self.f = offsets, G, M, d, f
        u8 = lambda *s: torch.empty(*s, dtype=torch.uint8, device=device)
        q = lambda R, K: (u8(max(R, 1), K), u8(max(R, 1), K // 32))
        self.xq = q(M, d)
        self.w1q, self.w3q, self.w2q = q(G * f, d), q(G * f, d), q(G * d, f)
        self.hq = q(M, f)
        self.ws = u8(max(L.moe_mx_gemm_workspace_size(G), 256))
        if backward:
            self.dyq = q(M, d)
            self.dabq = q(M, 2 * f)
            self.w2t = q(f, G * d)          # W2 along d: [f, G d]
            self.w1t, self.w3t = q(d, G * f), q(d, G * f)   # W1, W3 along f: [d, G f]
            self.ld = max(int(L.moe_mx_quantize_cols_ld(M, G, self.KPAD)), self.KPAD)
            self.dyc, self.hc = q(d, self.ld), q(f, self.ld)
            self.abc, self.xc = q(2 * f, self.ld), q(d, self.ld)
            self.kbase = torch.empty(G + 1, dtype=torch.int32, device=device)
            self.kbase_w = torch.empty(G + 1, dtype=torch.int32, device=device)
            # weight gradients: split-K partials when the product has few output tiles
            nws = max(L.moe_mx_gemm_k_workspace_size(G, d, f), L.moe_mx_gemm_k_workspace_size(G, 2 * f, d))
            self.ws_k = u8(max(nws, 256))


class MoELayer:
    """One GPU's MoE layer pass over device-resident inputs.

    ``params`` holds device tensors: x, logits (random routing) or w_router (+ bias), w1, w3, w2,
    ws1, ws3, ws2 (shared expert, may be None), dout (backward).
    ``events``: if given a dict, a (start, end) pair of CUDA events is recorded on the current
    stream around every library call, keyed by stage name.
    ``merge_shared``: run each GEMM stage of the routed experts and the shared expert as one
    two-set call (one launch where the kernel allows); False makes one call per set.
    ``recompute``: the per-layer recompute variant of the Ultra runs ("Olmo-core 3 Opens Large MoE
    Training", "Technical Deep Dive"): the forward keeps no SwiGLU pre-activation stash (it writes
    H only), and the backward runs the gate/up GEMM again to regenerate A, B and H before the
    down-projection dgrad.  The kernels are deterministic, so the results are bitwise those of the
    stashing pass.
    ``precision``: "bf16" (bf16 MFMA products) or "mxfp8" (the MXFP8 recipe of the Ultra runs, "Olmo-core
    DDP MoE examples", "Production throughput runs": every expert product on MX-quantized E4M3
    operands with fp32 accumulation; stored activations and gradients stay bf16).
    ``mx_cached_weights``: quantize the expert weights (both orientations) on the first pass and
    reuse them until ``refresh_mx_weights()`` is called, as when the weights change once per
    optimizer step and several micro-batches pass through the layer in between; otherwise every
    pass quantizes them.
    """

    def __init__(self, cfg: MoEConfig, params: dict, bufs: Buffers | None = None, renormalize: int = 1,
                 merge_shared: bool = True, recompute: bool = False, lbl_weight: float = 0.0,
                 precision: str = "bf16", mx_cached_weights: bool = False):
        self.cfg = cfg
        self.p = params
        self.bufs = bufs or Buffers.allocate(cfg, params["x"].device)
        self.renorm = renormalize
        self.merge = merge_shared
        self.recompute = recompute
        # Auxiliary load-balancing loss of the learned router (weight 0: off): its statistics and
        # loss in the forward, its gradient added to the router gradients in the backward.
        self.lbl = float(lbl_weight) if cfg.routing == "learned" else 0.0
        if self.lbl > 0:
            dev, t = params["x"].device, self.bufs.t
            t["lbl_loss"] = torch.empty(1, dtype=torch.float32, device=dev)
            t["prob_mean"] = torch.empty(cfg.E, dtype=torch.float32, device=dev)
            t["load_frac"] = torch.empty(cfg.E, dtype=torch.float32, device=dev)
            t["ws_aux"] = torch.empty(max(1, L.moe_router_aux_workspace_size(cfg.T, cfg.E)), dtype=torch.uint8,
                                      device=dev)
            if cfg.backward:
                t["ws_aux_bwd"] = torch.empty(max(1, L.moe_router_aux_bwd_workspace_size(cfg.T, cfg.d, cfg.E)),
                                              dtype=torch.uint8, device=dev)
        self.dt = L.MOE_BF16 if cfg.dtype == "bf16" else L.MOE_F32
        self.events: dict | None = None
        if precision not in ("bf16", "mxfp8"):
            raise ValueError(f"unknown precision {precision!r}")
        self.precision = precision
        self.mx = None
        self.mx_cached = bool(mx_cached_weights)
        self._mx_w_fresh = False   # quantized weights valid (cached mode)
        if precision == "mxfp8":
            if cfg.dtype != "bf16" or recompute:
                raise ValueError("the MXFP8 expert path takes bf16 workloads without recompute")
            dev, b = params["x"].device, self.bufs
            self.mx = [MxSet(b["offsets"], cfg.E, cfg.T * cfg.k, cfg.d, cfg.f, dev, cfg.backward)]
            if cfg.fs > 0:
                self.mx.append(MxSet(b["shared_offsets"], 1, cfg.T, cfg.d, cfg.fs, dev, cfg.backward))

    def _sets(self, dout=None, stash=True):
        """The routed experts and (if any) the shared expert as expert sets; stash=False leaves out
        the pre-activation outputs A and B."""
        c, p, b = self.cfg, self.p, self.bufs
        T, E, k, f, fs = c.T, c.E, c.k, c.f, c.fs
        bw = c.backward and stash
        g = lambda name: b.t.get(name)
        routed = L.expert_set(b["offsets"], E, T * k, f, x=b["x_perm"], w1=p["w1"], w3=p["w3"], w2=p["w2"],
                              a=b["a"] if bw else None, b=b["b"] if bw else None, h=b["h"], y=b["y"],
                              dy=g("dy"), dab=g("dab"), dx=g("dx_perm"), dw1=g("dw1"), dw3=g("dw3"),
                              dw2=g("dw2"))
        if fs == 0:
            return [routed]
        shared = L.expert_set(b["shared_offsets"], 1, T, fs, x=p["x"], w1=p["ws1"], w3=p["ws3"], w2=p["ws2"],
                              a=b["as"] if bw else None, b=b["bs"] if bw else None, h=b["hs"], y=b["s"],
                              dy=dout, dab=g("dabs"), dx=g("dx_shared"), dw1=g("dws1"), dw3=g("dws3"),
                              dw2=g("dws2"))
        return [routed, shared]

    def _gemm(self, name, stage, sets, ws):
        """One GEMM stage over the expert sets: a single call, or one call per set."""
        d, dt = self.cfg.d, self.dt
        if self.merge or len(sets) == 1:
            self._stage(name, L.moe_expert_stage, stage, sets, d, dt, ws, ws.numel())
        else:
            for i, s in enumerate(sets):
                self._stage(name if i == 0 else "shared_" + name, L.moe_expert_stage, stage, [s], d, dt, ws,
                            ws.numel())

    def _stage(self, name, fn, *args):
        if self.events is None:
            fn(*args)
            return
        s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        s.record()
        fn(*args)
        e.record()
        self.events.setdefault(name, []).append((s, e))

    def forward(self):
        c, p, b, dt = self.cfg, self.p, self.bufs, self.dt
        T, d, E, k, f, fs = c.T, c.d, c.E, c.k, c.f, c.fs
        Tk = T * k
        learned = c.routing == "learned"
        logits = b["logits"] if learned else p["logits"]
        self._stage("route", L.moe_route, p["x"], p.get("w_router") if learned else None,
                    p.get("bias") if learned else None, logits, T, d, E, k, self.renorm, dt,
                    b["topk_idx"], b["gate"])
        self._stage("permute", L.moe_permute, p["x"], b["topk_idx"], T, d, E, k, dt, b["counts"],
                    b["offsets"], b["dest_pos"], b["src_row"], b["x_perm"], b["ws_perm"],
                    b["ws_perm"].numel())
        if self.lbl > 0:
            self._stage("router_aux", L.moe_router_aux, logits, b["counts"], T, E, k, self.lbl, b["lbl_loss"],
                        b["prob_mean"], b["load_frac"], b["ws_aux"], b["ws_aux"].numel())
        if self.mx is not None:
            self._mx_forward()
        else:
            sets = self._sets(stash=not self.recompute)
            self._gemm("gate_up_fwd", L.MOE_STAGE_GATE_UP_FWD, sets, b["ws_fwd"])
            self._gemm("down_fwd", L.MOE_STAGE_DOWN_FWD, sets, b["ws_fwd"])
        shared = b["s"] if fs > 0 else None
        self._stage("combine", L.moe_combine, b["y"], b["gate"], b["dest_pos"], shared, T, d, k, dt, b["out"])
        return b["out"]

    def backward(self, dout=None):
        c, p, b, dt = self.cfg, self.p, self.bufs, self.dt
        T, d, E, k, f, fs = c.T, c.d, c.E, c.k, c.f, c.fs
        Tk = T * k
        dout = p["dout"] if dout is None else dout
        learned = c.routing == "learned"
        self._stage("combine_bwd", L.moe_combine_bwd, dout, b["y"], b["gate"], b["dest_pos"], T, d, k, dt,
                    b["dy"], b["dgate"] if learned else None)
        dx_router = None
        if learned:
            self._stage("route_bwd", L.moe_route_bwd, b["dgate"], b["gate"], b["topk_idx"], b["offsets"],
                        b["src_row"], p["x"], p["w_router"], T, d, E, k, self.renorm, dt, b["dwr"],
                        b["dx_router"], b["ws_route"], b["ws_route"].numel())
            dx_router = b["dx_router"]
            if self.lbl > 0:
                self._stage("router_aux_bwd", L.moe_router_aux_bwd, b["logits"], b["load_frac"], p["x"],
                            p["w_router"], T, d, E, self.lbl, dt, b["dwr"], b["dx_router"], b["ws_aux_bwd"],
                            b["ws_aux_bwd"].numel())
        dx_shared = b["dx_shared"] if fs > 0 else None
        if self.mx is not None:
            self._mx_dgrad(dout)
            self._stage("permute_bwd", L.moe_permute_bwd, b["dx_perm"], b["dest_pos"], dx_shared, dx_router, T,
                        d, k, dt, b["dx"])
            self._mx_wgrad(dout)
            return b["dx"]
        ws = b["ws_bwd"]
        sets = self._sets(dout)
        if self.recompute:
            self._gemm("gate_up_recompute", L.MOE_STAGE_GATE_UP_FWD, sets, b["ws_fwd"])
        # Each activation gradient is consumed right after it is produced, while it still sits in
        # the last-level cache (dA/dB by the gate/up dgrad, dX_perm by the permute backward); the
        # weight gradients, which nothing downstream reads, go last.
        self._gemm("down_bwd", L.MOE_STAGE_DOWN_BWD, sets, ws)
        self._gemm("gate_up_dgrad", L.MOE_STAGE_GATE_UP_DGRAD, sets, ws)
        self._stage("permute_bwd", L.moe_permute_bwd, b["dx_perm"], b["dest_pos"], dx_shared, dx_router, T, d,
                    k, dt, b["dx"])
        self._gemm("down_wgrad", L.MOE_STAGE_DOWN_WGRAD, sets, ws)
        self._gemm("gate_up_wgrad", L.MOE_STAGE_GATE_UP_WGRAD, sets, ws)
        return b["dx"]

    # ---- MXFP8 expert products -------------------------------------------------------------
    def _mx_tensors(self, i, dout=None):
        """Input, weights, stash and gradient buffers of expert set i (0: routed, 1: shared)."""
        p, b, t = self.p, self.bufs, self.bufs.t
        if i == 0:
            return dict(x=b["x_perm"], w1=p["w1"], w3=p["w3"], w2=p["w2"], a=t.get("a"), b=t.get("b"), h=b["h"],
                        y=b["y"], dy=t.get("dy"), dab=t.get("dab"), dx=t.get("dx_perm"), dw1=t.get("dw1"),
                        dw3=t.get("dw3"), dw2=t.get("dw2"))
        return dict(x=p["x"], w1=p["ws1"], w3=p["ws3"], w2=p["ws2"], a=t.get("as"), b=t.get("bs"), h=b["hs"],
                    y=b["s"], dy=dout, dab=t.get("dabs"), dx=t.get("dx_shared"), dw1=t.get("dws1"),
                    dw3=t.get("dws3"), dw2=t.get("dws2"))

    @staticmethod
    def _pfx(i, name):
        return name if i == 0 else "shared_" + name

    def refresh_mx_weights(self):
        """Cached mode: the weights changed; the next pass quantizes them again."""
        self._mx_w_fresh = False

    def _mx_quantize_weights(self):
        """Expert weights of both sets in MXFP8: along d / f (forward), and transposed along f / d
        (data gradients, when the layer has a backward)."""
        d = self.cfg.d
        for i, m in enumerate(self.mx):
            t, G, f = self._mx_tensors(i), m.G, m.f
            q = lambda name, x, R, K, out: self._stage(self._pfx(i, name), L.moe_mx_quantize_rows, x, R, K, K,
                                                       out[0], out[1])
            q("q_w1", t["w1"], G * f, d, m.w1q)
            q("q_w3", t["w3"], G * f, d, m.w3q)
            q("q_w2", t["w2"], G * d, f, m.w2q)
            if self.cfg.backward:
                qt = lambda name, x, R, N, rows, out, ld: self._stage(
                    self._pfx(i, name), L.moe_mx_quantize_cols, x, R, N, N, None, G, rows, m.KPAD, out[0], out[1],
                    ld, m.kbase_w)
                qt("q_w2t", t["w2"], G * d, f, d, m.w2t, G * d)
                qt("q_w1t", t["w1"], G * f, d, f, m.w1t, G * f)
                qt("q_w3t", t["w3"], G * f, d, f, m.w3t, G * f)
        self._mx_w_fresh = True

    def _mx_forward(self):
        d, bw = self.cfg.d, self.cfg.backward
        if not (self.mx_cached and self._mx_w_fresh):
            self._mx_quantize_weights()
        for i, m in enumerate(self.mx):
            t, G, M, f = self._mx_tensors(i), m.G, m.M, m.f
            q = lambda name, x, R, K, out: self._stage(self._pfx(i, name), L.moe_mx_quantize_rows, x, R, K, K,
                                                       out[0], out[1])
            q("q_x", t["x"], M, d, m.xq)
            self._stage(self._pfx(i, "gate_up_fwd"), L.moe_mx_gemm_rows, m.xq[0], m.xq[1], m.w1q[0], m.w1q[1], d,
                        f * d, m.w3q[0], m.w3q[1], 0, m.offsets, G, M, f, d, L.MOE_MX_EPI_SWIGLU,
                        t["a"] if bw else None, t["b"] if bw else None, t["h"], None, None, m.hq[0], m.hq[1],
                        m.ws, m.ws.numel())   # H also comes out quantized (rows along f)
            self._stage(self._pfx(i, "down_fwd"), L.moe_mx_gemm_rows, m.hq[0], m.hq[1], m.w2q[0], m.w2q[1], f,
                        d * f, None, None, 0, m.offsets, G, M, d, f, L.MOE_MX_EPI_STORE, t["y"], None, None, None,
                        None, None, None, m.ws, m.ws.numel())

    def _mx_dgrad(self, dout):
        d = self.cfg.d
        for i, m in enumerate(self.mx):
            t, G, M, f = self._mx_tensors(i, dout), m.G, m.M, m.f
            q = lambda name, x, R, K, out: self._stage(self._pfx(i, name), L.moe_mx_quantize_rows, x, R, K, K,
                                                       out[0], out[1])
            q("q_dy", t["dy"], M, d, m.dyq)
            self._stage(self._pfx(i, "down_bwd"), L.moe_mx_gemm_rows, m.dyq[0], m.dyq[1], m.w2t[0], m.w2t[1], G * d,
                        d, None, None, 0, m.offsets, G, M, f, d, L.MOE_MX_EPI_SWIGLU_BWD, t["dab"], None, None,
                        t["a"], t["b"], m.dabq[0], m.dabq[1], m.ws, m.ws.numel())   # [dA | dB] also quantized
            self._stage(self._pfx(i, "gate_up_dgrad"), L.moe_mx_gemm_rows, m.dabq[0], m.dabq[1], m.w1t[0],
                        m.w1t[1], G * f, f, m.w3t[0], m.w3t[1], f, m.offsets, G, M, d, 2 * f, L.MOE_MX_EPI_STORE,
                        t["dx"], None, None, None, None, None, None, m.ws, m.ws.numel())

    def _mx_wgrad(self, dout):
        d = self.cfg.d
        for i, m in enumerate(self.mx):
            t, G, M, f = self._mx_tensors(i, dout), m.G, m.M, m.f
            qc = lambda name, x, N, out: self._stage(self._pfx(i, name), L.moe_mx_quantize_cols, x, M, N, N,
                                                     m.offsets, G, 0, m.KPAD, out[0], out[1], m.ld, m.kbase)
            qc("q_dy_cols", t["dy"], d, m.dyc)
            qc("q_h_cols", t["h"], f, m.hc)
            self._stage(self._pfx(i, "down_wgrad"), L.moe_mx_gemm_k, m.dyc[0], m.dyc[1], m.ld, m.hc[0], m.hc[1],
                        m.ld, m.kbase, G, d, f, d, t["dw2"], None, m.ws_k, m.ws_k.numel())
            qc("q_dab_cols", t["dab"], 2 * f, m.abc)
            qc("q_x_cols", t["x"], d, m.xc)
            self._stage(self._pfx(i, "gate_up_wgrad"), L.moe_mx_gemm_k, m.abc[0], m.abc[1], m.ld, m.xc[0],
                        m.xc[1], m.ld, m.kbase, G, 2 * f, d, f, t["dw1"], t["dw3"], m.ws_k,
                        m.ws_k.numel())

    def step(self):
        """One pass of the whole path: forward, then backward when the workload has one."""
        self.forward()
        if self.cfg.backward:
            self.backward()
