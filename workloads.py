"""Seeded synthetic inputs for the int8-weight MoE feed-forward layer.

This module only draws numbers. It holds none of the layer's arithmetic (no
routing, no quantization, no contraction), so both the CPU oracle and the HIP
path can take their inputs from here without sharing any of the method.

Workloads are shaped like the MoE layer of the Jamba models (Jamba-1.5 paper,
"Model Architecture": n=16 experts, top K=2, MoE in place of the MLP every
e=2 layers, hidden size 8192 for Jamba-1.5-Large). The expert width, the Mini
hidden size and the value distributions are synthetic stand-ins: the paper
prints no kernel-level workload.

Recipe (per workload, base seed 0):
  * x        [T, d]   ~ N(0, 1), drawn in fp32 on the host, then rounded (RNE)
                      to the activation dtype.
  * router_w [E, d]   ~ N(0, 0.02), same handling. Layout is (out, in).
  * bias     [E] fp32 zeros except +2.0 on experts 0 and 1 for the skewed
                      workload, None otherwise.
  * w_gate, w_up [E, f, d] and w_down [E, d, f] ~ N(0, 0.02): the unquantized
                      expert weights in the checkpoint dtype (fp32 for the tiny
                      workload, bf16 otherwise), (out, in) layout. Small sets
                      are drawn on the host with numpy; multi-GB sets with
                      torch's generator on the device that will hold them, so
                      they never pass through the host.
Each tensor has its own stream: numpy SeedSequence(seed).spawn for host draws,
and a seed taken from the same SeedSequence for torch's device generator.
"""
from __future__ import annotations

import dataclasses
from typing import Optional

import numpy as np
import torch


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    T: int
    d: int
    f: int
    E: int = 16
    K: int = 2
    act: str = "bf16"      # dtype of x, router_w and y: "f32" or "bf16"
    scale: str = "bf16"    # dtype of the per-channel scales: "f32" or "bf16"
    weight_src: str = "bf16"  # dtype of the unquantized expert weights
    hot_bias: float = 0.0  # added to the router logits of experts 0 and 1
    seed: int = 0

    @property
    def has_bias(self) -> bool:
        return self.hot_bias != 0.0

    def with_(self, **kw) -> "Workload":
        return dataclasses.replace(self, **kw)


# The five workloads: shapes follow the Jamba MoE layer (16 experts, top-2).
TINY = Workload("tiny", T=64, d=256, f=512, act="f32", scale="f32", weight_src="f32")
MINI_DECODE = Workload("mini-decode", T=32, d=4096, f=14336)
MINI_PREFILL = Workload("mini-prefill", T=8192, d=4096, f=14336)
LARGE_DECODE = Workload("large-decode", T=64, d=8192, f=24576)
LARGE_PREFILL_SKEWED = Workload("large-prefill-skewed", T=16384, d=8192, f=24576, hot_bias=2.0)

WORKLOADS = {w.name: w for w in (TINY, MINI_DECODE, MINI_PREFILL, LARGE_DECODE, LARGE_PREFILL_SKEWED)}

# Dense MLP layers of the same model (ExpertsInt8 covers them too): one expert,
# every token, no router. Their FFN width is taken equal to the experts'.
LARGE_MLP_DECODE = Workload("large-mlp-decode", T=64, d=8192, f=24576, E=1, K=1)
LARGE_MLP_PREFILL = Workload("large-mlp-prefill", T=8192, d=8192, f=24576, E=1, K=1)
DENSE_WORKLOADS = {w.name: w for w in (LARGE_MLP_DECODE, LARGE_MLP_PREFILL)}

# One GPU's share of the Large layer under 8-way tensor parallelism over the
# expert width: every GPU routes all tokens and holds f/8 = 3072 channels of
# every expert's gate and up and the matching columns of down, so it runs the
# same layer at f = 3072 and produces a partial y (summed across GPUs by one
# all-reduce, not part of this single-GPU build).
LARGE_DECODE_TP8 = Workload("large-decode-tp8", T=64, d=8192, f=3072)
LARGE_PREFILL_SKEWED_TP8 = Workload("large-prefill-skewed-tp8", T=16384, d=8192, f=3072, hot_bias=2.0)
SHARD_WORKLOADS = {w.name: w for w in (LARGE_DECODE_TP8, LARGE_PREFILL_SKEWED_TP8)}
ALL_WORKLOADS = {**WORKLOADS, **DENSE_WORKLOADS, **SHARD_WORKLOADS}

TORCH_DTYPE = {"f32": torch.float32, "bf16": torch.bfloat16}

# stream ids inside the SeedSequence spawn
_X, _ROUTER, _GATE, _UP, _DOWN = range(5)


def _children(seed: int):
    return np.random.SeedSequence(seed).spawn(5)


def _host_normal(ss: np.random.SeedSequence, shape, std: float) -> np.ndarray:
    g = np.random.Generator(np.random.PCG64(ss))
    a = g.standard_normal(size=shape, dtype=np.float32)
    if std != 1.0:
        a *= np.float32(std)
    return a


def draw_activations(w: Workload, T: Optional[int] = None, seed: Optional[int] = None) -> torch.Tensor:
    """x [T, d] on the host, in the workload's activation dtype."""
    T = w.T if T is None else T
    ch = _children(w.seed if seed is None else seed)
    a = _host_normal(ch[_X], (T, w.d), 1.0)
    return torch.from_numpy(a).to(TORCH_DTYPE[w.act])


def draw_router(w: Workload) -> tuple[torch.Tensor, Optional[torch.Tensor]]:
    """router_w [E, d] (host, activation dtype) and the optional fp32 bias [E]."""
    ch = _children(w.seed)
    r = torch.from_numpy(_host_normal(ch[_ROUTER], (w.E, w.d), 0.02)).to(TORCH_DTYPE[w.act])
    bias = None
    if w.has_bias:
        bias = torch.zeros(w.E, dtype=torch.float32)
        bias[0] = w.hot_bias
        bias[1] = w.hot_bias
    return r, bias


def _device_seed(ss: np.random.SeedSequence) -> int:
    return int(ss.generate_state(1, dtype=np.uint64)[0] & ((1 << 63) - 1))


HOST_DRAW_LIMIT = 1 << 26   # expert-weight elements drawn on the host with numpy


def draw_expert_weights(w: Workload, device="cpu") -> dict[str, torch.Tensor]:
    """Unquantized expert weights (checkpoint dtype) on `device`.

    w_gate, w_up: [E, f, d]; w_down: [E, d, f]; (out, in) layout.
    Up to HOST_DRAW_LIMIT elements in total they are drawn on the host with
    numpy's PCG64 (reproducible on any machine); larger sets are drawn with
    torch's generator directly on `device`, one expert at a time.
    """
    ch = _children(w.seed)
    dt = TORCH_DTYPE[w.weight_src]
    host = 3 * w.E * w.d * w.f <= HOST_DRAW_LIMIT
    out = {}
    for name, idx, shape in (("w_gate", _GATE, (w.E, w.f, w.d)),
                             ("w_up", _UP, (w.E, w.f, w.d)),
                             ("w_down", _DOWN, (w.E, w.d, w.f))):
        if host:
            a = _host_normal(ch[idx], shape, 0.02)
            out[name] = torch.from_numpy(a).to(dt).to(device)
            continue
        g = torch.Generator(device=device)
        g.manual_seed(_device_seed(ch[idx]))
        t = torch.empty(shape, dtype=dt, device=device)
        for e in range(w.E):
            buf = torch.randn(shape[1:], generator=g, dtype=torch.float32, device=device)
            buf.mul_(0.02)
            t[e].copy_(buf)
            del buf
        out[name] = t
    return out


def workload_bytes(w: Workload) -> dict[str, int]:
    """Sizes in bytes of the layer's resident tensors (for memory planning)."""
    act = 4 if w.act == "f32" else 2
    sc = 4 if w.scale == "f32" else 2
    return {
        "x": w.T * w.d * act,
        "router_w": w.E * w.d * act,
        "int8_weights": 3 * w.E * w.d * w.f,
        "scales": w.E * (2 * w.f + w.d) * sc,
        "y": w.T * w.d * act,
    }
