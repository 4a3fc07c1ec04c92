"""Helpers for the GPU parity tests: device copies of the seeded inputs and
comparisons with the oracle (test-only)."""
from __future__ import annotations

import numpy as np
import torch

DEV = "cuda:0"


def tdev(a: np.ndarray, dtype) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a)).to(device=DEV).to(dtype)


def chain_tensors(inp, dtype):
    """torch device tensors of make_chain_inputs(...) output."""
    t = dict(tokens=tdev(inp["tokens"].astype(np.int32), torch.int32),
             segment_ids=tdev(inp["segment_ids"].astype(np.int32), torch.int32),
             h0=tdev(inp["h0"], dtype), E=tdev(inp["E"], dtype),
             W_out=tdev(inp["W_out"], dtype) if inp["W_out"] is not None else None,
             g_out=tdev(inp["g_out"], torch.float32))
    t["depths"] = [dict(g_h=tdev(w["g_h"], torch.float32), g_e=tdev(w["g_e"], torch.float32),
                        M=tdev(w["M"], dtype), g_a=tdev(w["g_a"], torch.float32),
                        Wqkv=tdev(w["Wqkv"], dtype), Wo=tdev(w["Wo"], dtype),
                        g_f=tdev(w["g_f"], torch.float32), Wgate=tdev(w["Wgate"], dtype),
                        Wup=tdev(w["Wup"], dtype), Wdown=tdev(w["Wdown"], dtype))
                   for w in inp["depths"]]
    return t


def bf16_ulp(x: np.ndarray) -> np.ndarray:
    ax = np.maximum(np.abs(x), 2.0 ** -126)
    return 2.0 ** (np.floor(np.log2(ax)) - 7)


def compare(gpu: np.ndarray, ref: np.ndarray, atol: float, bf16_store: bool = False, ulps: int = 1):
    """Max-abs comparison.  With ``bf16_store`` a difference of ``ulps`` bf16
    ulps of the reference (at the element's row scale, for 2-D arrays) is
    also admitted: the two sides rounded nearly equal values to neighbouring
    bf16 numbers at the stores before it.  Returns (max_err, n_over_atol, ok)."""
    gpu = np.asarray(gpu, np.float64)
    ref = np.asarray(ref, np.float64)
    err = np.abs(gpu - ref)
    allowed = np.full_like(err, atol)
    if bf16_store:
        # the ulp is taken at the larger of the element and its row's RMS: a
        # small element of a large-scale row carries the row's absolute noise
        scale = np.abs(ref)
        if ref.ndim == 2:
            scale = np.maximum(scale, np.sqrt(np.mean(ref * ref, axis=1, keepdims=True)))
        allowed = np.maximum(allowed, ulps * bf16_ulp(scale) * 1.0001)
    bad = ~(err <= allowed)
    return float(err.max()) if err.size else 0.0, int((err > atol).sum()), not bad.any()


def rel_fro(gpu: np.ndarray, ref: np.ndarray) -> float:
    n = np.linalg.norm(np.asarray(ref, np.float64))
    return float(np.linalg.norm(np.asarray(gpu, np.float64) - ref) / max(n, 1e-300))


def to_np(t: torch.Tensor) -> np.ndarray:
    return t.detach().float().cpu().numpy() if t.dtype in (torch.bfloat16, torch.float16) \
        else t.detach().cpu().numpy()
