"""Seeded synthetic inputs for the MoE layer forward pass.

This module holds no part of the method's arithmetic: it only draws
Gaussian tensors with the stated standard deviations, rounds them to bf16
storage, and names the five workloads.  Both the GPU library's callers and
the CPU oracle's tests take their inputs from here.

Every tensor is drawn from its own ``torch.Generator`` seeded with
``seed * 64 + tensor_id``, so a tensor's values depend only on (seed, tensor
id, shape, device type).  Large expert weights are drawn one expert at a time
to bound temporary memory.  Values differ between ``device="cpu"`` and a GPU
device (different generator algorithms); each parity test feeds the same
tensors to both sides, so that never matters.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field, replace

import torch

BASE_SEED = 20261203


@dataclass(frozen=True)
class MoEConfig:
    """Shape, placement and input distribution of one workload."""

    name: str
    T: int          # tokens on this device
    d: int          # hidden size
    E: int          # routed experts
    k: int          # experts per token
    H: int          # SwiGLU hidden size of one expert
    cf: float       # capacity factor; inf = dropless
    D: int          # logical destination ranks (E % D == 0)
    x_std: float
    wg_std: float
    w_std: float
    bias: dict = field(default_factory=dict)  # expert -> logit bias
    my_rank: int = 0
    seed: int = BASE_SEED
    drop_policy: int = 0   # 0: overflow dropped in token order; 1: by gate value
    min_capacity: int = 0  # lower bound on the capacity C (capacity mode)
    dispatch_fp8: int = 0  # 1: dispatch payload as E4M3 rows with fp32 row scales
    n_groups: int = 0      # expert groups for group-limited routing (<= 1: none)
    group_limit: int = 0   # groups a token may use
    shared_H: int = 0      # hidden size of a shared (replicated) expert; 0: none

    def with_(self, **kw) -> "MoEConfig":
        return replace(self, **kw)


def _cfg(idx, name, T, d, E, k, H, cf, D, x_std, wg_std, w_std, bias=None):
    return MoEConfig(name=name, T=T, d=d, E=E, k=k, H=H, cf=cf, D=D, x_std=x_std,
                     wg_std=wg_std, w_std=w_std, bias=dict(bias or {}),
                     seed=BASE_SEED + idx)


INF = float("inf")

# The five workloads.  x and W_g standard deviations: "N(0,1)/sqrt(d)" is
# std 1/sqrt(d); "N(0, 1/d)" is variance 1/d; "N(0, 0.02)" is std 0.02.
CONFIGS = {
    c.name: c
    for c in (
        _cfg(0, "tiny", 256, 512, 8, 2, 1024, 1.25, 2,
             1 / math.sqrt(512), 1 / math.sqrt(512), 0.02),
        _cfg(1, "mixtral", 4096, 4096, 8, 2, 14336, 1.0, 8, 1.0, 0.02, 0.02),
        _cfg(2, "dsv3_prefill", 4096, 7168, 256, 8, 2048, INF, 8,
             1.0, 1 / math.sqrt(7168), 0.02),
        _cfg(3, "dsv3_decode", 64, 7168, 256, 8, 2048, INF, 8,
             1.0, 1 / math.sqrt(7168), 0.02),
        _cfg(4, "skewed", 8192, 4096, 64, 2, 8192, 1.25, 8,
             1.0, 1 / math.sqrt(4096), 0.02, bias={2: 3.0}),
    )
}

_X, _WG, _W1, _W3, _W2, _W1S, _W3S, _W2S = range(8)


def _gen(seed: int, tid: int, device) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(seed * 64 + tid)
    return g


def _normal_bf16(shape, std, g, device) -> torch.Tensor:
    t = torch.randn(shape, generator=g, device=device, dtype=torch.float32)
    return t.mul_(std).to(torch.bfloat16)


def _normal_bf16_stacked(n, shape, std, g, device) -> torch.Tensor:
    out = torch.empty((n, *shape), dtype=torch.bfloat16, device=device)
    for i in range(n):
        out[i].copy_(_normal_bf16(shape, std, g, device))
    return out


def make_inputs(cfg: MoEConfig, device="cpu", *, experts: bool = True) -> dict:
    """Draw x [T,d], w_gate [d,E], bias [E] fp32 (or None), w1/w3 [E,H,d], w2 [E,d,H],
    and with a shared expert w1s/w3s [shared_H,d], w2s [d,shared_H].

    ``experts=False`` skips the expert weights (routing-only tests).
    """
    dev = torch.device(device)
    out = {
        "x": _normal_bf16((cfg.T, cfg.d), cfg.x_std, _gen(cfg.seed, _X, dev), dev),
        "w_gate": _normal_bf16((cfg.d, cfg.E), cfg.wg_std, _gen(cfg.seed, _WG, dev), dev),
        "bias": None,
    }
    if cfg.bias:
        b = torch.zeros(cfg.E, dtype=torch.float32)
        for e, v in cfg.bias.items():
            b[e] = v
        out["bias"] = b.to(dev)
    if experts:
        out["w1"] = _normal_bf16_stacked(cfg.E, (cfg.H, cfg.d), cfg.w_std,
                                         _gen(cfg.seed, _W1, dev), dev)
        out["w3"] = _normal_bf16_stacked(cfg.E, (cfg.H, cfg.d), cfg.w_std,
                                         _gen(cfg.seed, _W3, dev), dev)
        out["w2"] = _normal_bf16_stacked(cfg.E, (cfg.d, cfg.H), cfg.w_std,
                                         _gen(cfg.seed, _W2, dev), dev)
        if cfg.shared_H > 0:
            out["w1s"] = _normal_bf16((cfg.shared_H, cfg.d), cfg.w_std,
                                      _gen(cfg.seed, _W1S, dev), dev)
            out["w3s"] = _normal_bf16((cfg.shared_H, cfg.d), cfg.w_std,
                                      _gen(cfg.seed, _W3S, dev), dev)
            out["w2s"] = _normal_bf16((cfg.d, cfg.shared_H), cfg.w_std,
                                      _gen(cfg.seed, _W2S, dev), dev)
    return out


def bf16_bits(t: torch.Tensor):
    """Raw bf16 bits of a tensor as a host numpy uint16 array."""
    import numpy as np

    return t.detach().contiguous().cpu().view(torch.int16).numpy().view(np.uint16)


def from_bf16_bits(a, device="cpu") -> torch.Tensor:
    import numpy as np

    return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).to(device)
