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
        gws = max(L.moe_grouped_mlp_fwd_workspace_size(Tk, E, d, f),
                  L.moe_grouped_mlp_fwd_workspace_size(T, 1, d, max(fs, 128)))
        b["ws_fwd"] = u8(gws)
        if fs > 0:
            b["shared_offsets"] = torch.tensor([0, T], dtype=torch.int32, device=device)
            b["as"] = e(T, fs)
            b["bs"] = e(T, fs)
            b["hs"] = e(T, fs)
            b["s"] = e(T, d)
        if cfg.backward:
            # Backward GEMM workspace: tile prefix plus room for split weight-gradient partials.
            b["ws_bwd"] = u8(max(L.moe_grouped_mlp_bwd_workspace_size(Tk, E, d, f),
                                 L.moe_grouped_mlp_bwd_workspace_size(T, 1, d, max(fs, 128))))
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


class MoELayer:
    """One GPU's MoE layer pass over device-resident inputs.

    ``params`` holds device tensors: x, logits (random routing) or w_router (+ bias), w1, w3, w2,
    ws1, ws3, ws2 (shared expert, may be None), dout (backward).
    ``events``: if given a dict, a (start, end) pair of CUDA events is recorded on the current
    stream around every library call, keyed by stage name.
    """

    def __init__(self, cfg: MoEConfig, params: dict, bufs: Buffers | None = None, renormalize: int = 1):
        self.cfg = cfg
        self.p = params
        self.bufs = bufs or Buffers.allocate(cfg, params["x"].device)
        self.renorm = renormalize
        self.dt = L.MOE_BF16 if cfg.dtype == "bf16" else L.MOE_F32
        self.events: dict | None = None

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
        stash_a = b["a"] if c.backward else None
        stash_b = b["b"] if c.backward else None
        self._stage("gate_up_fwd", L.moe_expert_gate_up_fwd, b["x_perm"], b["offsets"], E, Tk, d, f,
                    p["w1"], p["w3"], dt, stash_a, stash_b, b["h"], b["ws_fwd"], b["ws_fwd"].numel())
        self._stage("down_fwd", L.moe_expert_down_fwd, b["h"], b["offsets"], E, Tk, d, f, p["w2"], dt,
                    b["y"], b["ws_fwd"], b["ws_fwd"].numel())
        shared = None
        if fs > 0:
            self._stage("shared_fwd", L.moe_grouped_mlp_fwd, p["x"], b["shared_offsets"], 1, T, d, fs,
                        p["ws1"], p["ws3"], p["ws2"], dt, b["as"] if c.backward else None,
                        b["bs"] if c.backward else None, b["hs"], b["s"], b["ws_fwd"], b["ws_fwd"].numel())
            shared = b["s"]
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
        ws, wsn = b["ws_bwd"], b["ws_bwd"].numel()
        self._stage("down_bwd", L.moe_expert_down_bwd, b["dy"], b["a"], b["b"], b["offsets"], E, Tk, d, f,
                    p["w2"], dt, b["dab"], ws, wsn)
        self._stage("down_wgrad", L.moe_expert_down_wgrad, b["dy"], b["h"], b["offsets"], E, Tk, d, f, dt,
                    b["dw2"], ws, wsn)
        self._stage("gate_up_dgrad", L.moe_expert_gate_up_dgrad, b["dab"], b["offsets"], E, Tk, d, f,
                    p["w1"], p["w3"], dt, b["dx_perm"], ws, wsn)
        self._stage("gate_up_wgrad", L.moe_expert_gate_up_wgrad, b["dab"], b["x_perm"], b["offsets"], E, Tk,
                    d, f, dt, b["dw1"], b["dw3"], ws, wsn)
        dx_shared = None
        if fs > 0:
            so = b["shared_offsets"]
            self._stage("shared_down_bwd", L.moe_expert_down_bwd, dout, b["as"], b["bs"], so, 1, T, d, fs,
                        p["ws2"], dt, b["dabs"], ws, wsn)
            self._stage("shared_down_wgrad", L.moe_expert_down_wgrad, dout, b["hs"], so, 1, T, d, fs, dt,
                        b["dws2"], ws, wsn)
            self._stage("shared_gate_up_dgrad", L.moe_expert_gate_up_dgrad, b["dabs"], so, 1, T, d, fs,
                        p["ws1"], p["ws3"], dt, b["dx_shared"], ws, wsn)
            self._stage("shared_gate_up_wgrad", L.moe_expert_gate_up_wgrad, b["dabs"], p["x"], so, 1, T, d, fs,
                        dt, b["dws1"], b["dws3"], ws, wsn)
            dx_shared = b["dx_shared"]
        self._stage("permute_bwd", L.moe_permute_bwd, b["dx_perm"], b["dest_pos"], dx_shared, dx_router, T, d,
                    k, dt, b["dx"])
        return b["dx"]

    def step(self):
        """One pass of the whole path: forward, then backward when the workload has one."""
        self.forward()
        if self.cfg.backward:
            self.backward()
