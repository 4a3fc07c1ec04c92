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


# Hidden states h^k (bf16 stores, R22's rule).  An element passes at max-abs
# 2e-2 or within one bf16 ulp of the larger of |ref| and |gpu| (the two sides
# rounded nearly equal fp32/fp64 values to neighbouring bf16 numbers at the
# h^k store).  From depth 2 on, the module also reads the earlier depths'
# store flips, whose effect is absolute noise at the row's scale (relative
# Frobenius error ~1.7e-3 per depth), so a capped fraction of elements may
# exceed both.  Per depth: no element beyond H_MAX_ABS; at most H_FRAC_CAP
# of the elements over 2e-2; none beyond one ulp and 2e-2 at depth 1, at most
# H_DEEP_FRAC_CAP from depth 2 on; relative Frobenius error below
# H_RELF_PER_DEPTH * k.
H_ATOL = 2e-2
H_MAX_ABS = 4e-2
H_FRAC_CAP = 2e-3
H_DEEP_FRAC_CAP = 5e-4
H_RELF_PER_DEPTH = 2.5e-3


def compare_h(gpu: np.ndarray, ref: np.ndarray, depth: int):
    """The hidden-state rule at depth ``depth`` (1-based).  Returns a dict of
    the statistics and ``ok``."""
    gpu = np.asarray(gpu, np.float64)
    ref = np.asarray(ref, np.float64)
    err = np.abs(gpu - ref)
    ulp = bf16_ulp(np.maximum(np.abs(ref), np.abs(gpu))) * 1.0001
    over_atol = err > H_ATOL
    beyond_one = over_atol & (err > ulp)
    n = max(err.size, 1)
    st = dict(max_err=float(err.max()) if err.size else 0.0, n=err.size, n_over_atol=int(over_atol.sum()),
              frac_over_atol=float(over_atol.sum()) / n, n_beyond_one_ulp=int(beyond_one.sum()),
              frac_beyond_one_ulp=float(beyond_one.sum()) / n, relF=rel_fro(gpu, ref))
    cap_deep = 0.0 if depth == 1 else H_DEEP_FRAC_CAP
    st["ok"] = (st["max_err"] <= H_MAX_ABS and st["frac_over_atol"] <= H_FRAC_CAP
                and st["frac_beyond_one_ulp"] <= cap_deep and st["relF"] < H_RELF_PER_DEPTH * depth)
    return st


def fmt_h(st) -> str:
    return (f"max|err| {st['max_err']:.3e}, over 2e-2: {st['n_over_atol']} of {st['n']} "
            f"({100 * st['frac_over_atol']:.3f}%), beyond one ulp and 2e-2: {st['n_beyond_one_ulp']} "
            f"({100 * st['frac_beyond_one_ulp']:.4f}%), relF {st['relF']:.2e}")


def rel_fro(gpu: np.ndarray, ref: np.ndarray) -> float:
    n = np.linalg.norm(np.asarray(ref, np.float64))
    return float(np.linalg.norm(np.asarray(gpu, np.float64) - ref) / max(n, 1e-300))


def to_np(t: torch.Tensor) -> np.ndarray:
    return t.detach().float().cpu().numpy() if t.dtype in (torch.bfloat16, torch.float16) \
        else t.detach().cpu().numpy()
