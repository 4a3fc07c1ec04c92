"""Rounding points of the oracle's numerical model (test infrastructure only).

The oracle computes in float64.  In its "bf16" model it rounds a value to
bfloat16 (round to nearest even) exactly where the GPU path stores that tensor
in bfloat16; everything between two stores is float64 here.  The "exact" model
(used for the float32 tiny case) rounds nothing.

The list of rounding points is a declared reading (the pages fix no storage
precision): c (normalised concat), x_a (attention-norm output), q, k, v
(after RoPE), o, y (FFN-norm output), the SwiGLU product, h^k, and x_hat
(output-norm output).  The residual stream u -> a -> h stays wide until h^k
is stored.
"""
from __future__ import annotations

import numpy as np


def bf16_round(x: np.ndarray) -> np.ndarray:
    """Round float64/float32 values to the nearest bfloat16 (ties to even),
    returned as float64.  Written out on the float32 bit pattern: a float64
    value is first rounded to float32 (exact for values already representable
    there), then the low 16 bits are rounded away."""
    f = np.asarray(x, dtype=np.float32)
    u = f.view(np.uint32).astype(np.uint64)
    lsb = (u >> np.uint64(16)) & np.uint64(1)
    u = (u + np.uint64(0x7FFF) + lsb) >> np.uint64(16)
    out = (u.astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)
    nan = np.isnan(f)
    if nan.any():
        out[nan] = np.nan
    return out


class Model:
    """A numerical model: ``store(x)`` is applied at every rounding point."""

    def __init__(self, kind: str):
        if kind not in ("exact", "bf16"):
            raise ValueError("model must be 'exact' or 'bf16'")
        self.kind = kind

    def store(self, x: np.ndarray) -> np.ndarray:
        x = np.asarray(x, dtype=np.float64)
        return bf16_round(x) if self.kind == "bf16" else x


EXACT = Model("exact")
BF16 = Model("bf16")
