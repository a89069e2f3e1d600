"""Comparison helpers shared by the GPU parity tests (test code only)."""
from __future__ import annotations

import numpy as np
import torch

from expert_token_routing_moe_amd.inputs import bf16_bits

# Output tolerance for bf16 results with fp32 accumulation: elementwise
# |a - b| <= REL * (|b| + rms(b)) and relative Frobenius <= FROB.
REL = 2e-2
FROB = 5e-3
# A routing flip between the GPU and the oracle is accepted only where the
# oracle's top-k boundary gap is below this.
GAP = 1e-5


def bits_to_f64(bits: np.ndarray) -> np.ndarray:
    return (bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def t2f(t: torch.Tensor) -> np.ndarray:
    return bits_to_f64(bf16_bits(t))


def assert_bf16_close(got: np.ndarray, ref: np.ndarray, what: str):
    """got/ref: float64 arrays of bf16 values."""
    assert got.shape == ref.shape, what
    if ref.size == 0:
        return
    rms = float(np.sqrt(np.mean(ref * ref)))
    err = np.abs(got - ref)
    bound = REL * (np.abs(ref) + rms)
    bad = err > bound
    frob = float(np.linalg.norm(got - ref) / max(np.linalg.norm(ref), 1e-300))
    assert not bad.any(), (
        f"{what}: {int(bad.sum())} elements beyond {REL}*(|ref|+rms); worst "
        f"{float((err / np.maximum(bound, 1e-300)).max()):.3g}x of the bound")
    assert frob <= FROB, f"{what}: relative Frobenius error {frob:.3g} > {FROB}"
    return dict(frob=frob, exact=float(np.mean(got == ref)))


def logit_tolerance(x_f64: np.ndarray, wg_f64: np.ndarray) -> np.ndarray:
    """Bound on fp32-accumulation error of x W_g: 8 sqrt(d) u sum_j |x_j w_je| + 1e-6."""
    d = x_f64.shape[1]
    mag = np.abs(x_f64) @ np.abs(wg_f64)
    return 8 * np.sqrt(d) * 2.0 ** -24 * mag + 1e-6
