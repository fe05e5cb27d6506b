"""Seeded synthetic inputs for the MoE layer, shared by the oracle-side tests and the GPU path.

This module holds workload shapes and random draws only: none of the layer's arithmetic.
Both sides receive the same bytes from here and nothing else in common.

Workload shapes follow the operating points of the Olmo-core DDP MoE examples README
("Production throughput runs": sequence length 8192, top-4 routing, one shared expert,
random or learned routing, 64-128 experts; "Other experiments in the report": the
8-to-128-expert sweep and the rank micro-batch of 2 sequences). The real training data the
pages name is not available, so Gaussian activations stand in for post-norm hidden states.

Weight layouts (every weight is [out_features, in_features], row-major, contiguous):
  w_router [E, d]       router
  w1, w3   [E, f, d]    gate and up projections of each routed expert
  w2       [E, d, f]    down projection of each routed expert
  ws1, ws3 [fs, d]      shared expert gate / up
  ws2      [d, fs]      shared expert down
"""
from __future__ import annotations

import dataclasses
from dataclasses import dataclass

import numpy as np


@dataclass(frozen=True)
class MoEConfig:
    name: str
    T: int           # tokens
    d: int           # d_model
    E: int           # routed experts
    k: int           # experts per token
    f: int           # routed expert hidden size
    fs: int          # shared expert hidden size (0: no shared expert)
    dtype: str       # "f32" or "bf16": storage and compute type of activations and weights
    routing: str     # "learned" (logits = x . w_router^T + bias) or "random" (logits drawn)
    bias_std: float  # std of the per-expert logit bias; 0 means no bias
    backward: bool   # forward+backward (True) or forward only
    seed: int = 0
    x_std: float = 1.0
    w_std: float = 0.02
    logit_std: float = 1.0
    dout_std: float = 1.0

    @property
    def Tk(self) -> int:
        return self.T * self.k

    def with_(self, **kw) -> "MoEConfig":
        return dataclasses.replace(self, **kw)


# The five workloads.  Sizes are the pages' operating points (sequence 8192, top-4, one shared
# expert, 64 or 128 experts); the tiny fp32 case is small enough for the oracle in seconds.
CONFIGS: dict[str, MoEConfig] = {
    # T=512, d=256, E=8, top-2 learned softmax router, d_ff=512, no shared expert, fp32, fwd only.
    "tiny_fp32": MoEConfig("tiny_fp32", 512, 256, 8, 2, 512, 0, "f32", "learned", 0.0, False),
    # One 8192-token sequence, d=2048, E=64, top-4 random routing, d_ff=1024 + shared 1024.
    "tiny64e_random": MoEConfig("tiny64e_random", 8192, 2048, 64, 4, 1024, 1024, "bf16", "random",
                                0.0, True),
    # Same shapes, learned router with a per-expert logit bias ~ N(0, 1.5): skewed expert loads.
    "tiny64e_learned_skew": MoEConfig("tiny64e_learned_skew", 8192, 2048, 64, 4, 1024, 1024,
                                      "bf16", "learned", 1.5, True),
    # Two 8192-token sequences, E=128 (and the 8/32-expert points of the same active size).
    "e128_2seq": MoEConfig("e128_2seq", 16384, 2048, 128, 4, 1024, 1024, "bf16", "random", 0.0, True),
    "e32_2seq": MoEConfig("e32_2seq", 16384, 2048, 32, 4, 1024, 1024, "bf16", "random", 0.0, True),
    "e8_2seq": MoEConfig("e8_2seq", 16384, 2048, 8, 4, 1024, 1024, "bf16", "random", 0.0, True),
    # Larger layer: d=4096, E=128, top-4 learned, d_ff=2048, shared d_ff=4096.
    "large_e128": MoEConfig("large_e128", 8192, 4096, 128, 4, 2048, 4096, "bf16", "learned", 0.0,
                            True),
}


def bf16_bits_from_f32(a: np.ndarray) -> np.ndarray:
    """Round fp32 values to bfloat16 (round to nearest, ties to even); returns the uint16 bit patterns."""
    u = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32)
    lsb = (u >> np.uint32(16)) & np.uint32(1)
    return ((u + np.uint32(0x7FFF) + lsb) >> np.uint32(16)).astype(np.uint16)


def f32_from_bf16_bits(b: np.ndarray) -> np.ndarray:
    """Widen bfloat16 bit patterns to fp32 (exact)."""
    return (np.ascontiguousarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


@dataclass
class Tensor:
    """One input tensor: fp32 values plus, for bf16 storage, the bf16 bit patterns they came from.

    ``value`` always holds the exact value both sides compute with (for bf16, the widened bf16).
    """
    value: np.ndarray
    bits: np.ndarray | None = None   # uint16 bf16 bit patterns when stored as bf16

    @property
    def is_bf16(self) -> bool:
        return self.bits is not None


def _draw(rng: np.random.Generator, shape, std: float, as_bf16: bool, chunk_rows: int = 1 << 14) -> Tensor:
    """Draw N(0, std) in fp32 (row chunks keep peak host memory bounded), then round to bf16 if asked."""
    shape = tuple(int(s) for s in shape)
    rows = shape[0]
    inner = shape[1:]
    vals = np.empty(shape, np.float32)
    bits = np.empty(shape, np.uint16) if as_bf16 else None
    for r0 in range(0, rows, chunk_rows):
        r1 = min(rows, r0 + chunk_rows)
        v = rng.standard_normal((r1 - r0,) + inner, dtype=np.float32)
        v *= np.float32(std)
        if as_bf16:
            b = bf16_bits_from_f32(v)
            bits[r0:r1] = b
            vals[r0:r1] = f32_from_bf16_bits(b)
        else:
            vals[r0:r1] = v
    return Tensor(vals, bits)


def make_inputs(cfg: MoEConfig, seed: int | None = None) -> dict[str, Tensor | None]:
    """All inputs of one layer pass, drawn in a fixed order from numpy's PCG64 with the given seed.

    Order: x, then (logits) for random routing or (w_router, bias) for learned routing, then
    w1, w3, w2, ws1, ws3, ws2, dout.  Random logits and the bias stay fp32; everything else is
    stored in the configuration's dtype.
    """
    rng = np.random.default_rng(cfg.seed if seed is None else seed)
    bf = cfg.dtype == "bf16"
    out: dict[str, Tensor | None] = {}
    out["x"] = _draw(rng, (cfg.T, cfg.d), cfg.x_std, bf)
    if cfg.routing == "random":
        out["logits"] = _draw(rng, (cfg.T, cfg.E), cfg.logit_std, False)
        out["w_router"] = None
        out["bias"] = None
    elif cfg.routing == "learned":
        out["logits"] = None
        out["w_router"] = _draw(rng, (cfg.E, cfg.d), cfg.w_std, bf)
        out["bias"] = _draw(rng, (cfg.E,), cfg.bias_std, False) if cfg.bias_std > 0 else None
    else:
        raise ValueError(f"unknown routing mode {cfg.routing!r}")
    out["w1"] = _draw(rng, (cfg.E, cfg.f, cfg.d), cfg.w_std, bf, chunk_rows=1)
    out["w3"] = _draw(rng, (cfg.E, cfg.f, cfg.d), cfg.w_std, bf, chunk_rows=1)
    out["w2"] = _draw(rng, (cfg.E, cfg.d, cfg.f), cfg.w_std, bf, chunk_rows=1)
    if cfg.fs > 0:
        out["ws1"] = _draw(rng, (cfg.fs, cfg.d), cfg.w_std, bf)
        out["ws3"] = _draw(rng, (cfg.fs, cfg.d), cfg.w_std, bf)
        out["ws2"] = _draw(rng, (cfg.d, cfg.fs), cfg.w_std, bf)
    else:
        out["ws1"] = out["ws3"] = out["ws2"] = None
    out["dout"] = _draw(rng, (cfg.T, cfg.d), cfg.dout_std, bf) if cfg.backward else None
    return out


def values(inp: dict[str, Tensor | None]) -> dict[str, np.ndarray | None]:
    """The exact values of every input (fp32 arrays), for the oracle."""
    return {k: (None if v is None else v.value) for k, v in inp.items()}
