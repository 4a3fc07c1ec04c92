"""Seeded synthetic inputs for the MTP depth chain, the shared-head CE and verify.

This module draws random numbers and lays them out. It holds none of the
method's arithmetic (no normalisation, projection, attention, loss or
acceptance rule): both the CPU oracle and the HIP path receive the arrays it
returns, and neither is imported from here.

Recipe (one ``numpy.random.SeedSequence(base_seed + config_index)`` spawned
into child streams in a fixed order, so adding a tensor never shifts another):

* tokens: uniform over [0, V) for the tiny case, otherwise bounded Zipf(1.1)
  over ranks 1..V with token id = rank - 1, drawn by inverse CDF;
* segments: per batch row, lengths uniform (inclusive) in [lo, hi], filled left
  to right with ids 0, 1, 2, ...; the last segment is truncated to the space
  left.  The tiny case uses the fixed layout of its description (row 0 = one
  segment of 10 then padding; row 1 = segments of 7 and 9);
* h^0 ~ N(0, 1); E, W_out and every per-depth matrix ~ N(0, sigma_w);
  every RMSNorm gain ~ 1 + N(0, 0.1), drawn independently;
* every floating-point array is drawn in float32 and rounded once to bfloat16
  (round to nearest even) for the bf16 cases; the tiny case stays float32.
"""
from __future__ import annotations

import dataclasses
from typing import Dict, List

import numpy as np

BASE_SEED = 20261202


@dataclasses.dataclass(frozen=True)
class ChainConfig:
    name: str
    index: int
    B: int
    T: int
    d: int
    n_heads: int
    head_dim: int
    ffn: int
    V: int
    D: int
    dtype: str            # "f32" or "bf16"
    sigma_w: float
    seg_lo: int           # packed segment length range (inclusive); 0 = fixed layout
    seg_hi: int
    zipf: bool
    lam: float = 0.1
    eps: float = 1e-6
    rope_theta: float = 10000.0

    @property
    def N(self) -> int:
        return self.B * self.T

    @property
    def A_w(self) -> int:
        return self.n_heads * self.head_dim


TINY = ChainConfig("tiny_f32", 0, B=2, T=16, d=64, n_heads=4, head_dim=16, ffn=172,
                   V=512, D=1, dtype="f32", sigma_w=0.02, seg_lo=0, seg_hi=0, zipf=False)
D1 = ChainConfig("d1_bf16", 1, B=4, T=1024, d=1024, n_heads=8, head_dim=128, ffn=2816,
                 V=32768, D=1, dtype="bf16", sigma_w=0.02, seg_lo=64, seg_hi=1024, zipf=True)
D3 = ChainConfig("d3_bf16", 2, B=8, T=2048, d=2048, n_heads=16, head_dim=128, ffn=5632,
                 V=65536, D=3, dtype="bf16", sigma_w=0.02, seg_lo=128, seg_hi=2048, zipf=True)
V3 = ChainConfig("v3width_bf16", 3, B=1, T=4096, d=7168, n_heads=128, head_dim=128,
                 ffn=18432, V=129280, D=1, dtype="bf16", sigma_w=0.006,
                 seg_lo=4096, seg_hi=4096, zipf=True)

CHAIN_CONFIGS = {c.name: c for c in (TINY, D1, D3, V3)}


def scaled(cfg: ChainConfig, **kw) -> ChainConfig:
    """A copy of ``cfg`` with some fields replaced (smaller parity cases of the
    same structure)."""
    return dataclasses.replace(cfg, **kw)


# ----------------------------------------------------------------------------
# bfloat16 storage helpers (input preparation only)
# ----------------------------------------------------------------------------

def to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """float32 -> bfloat16 bit patterns (uint16), round to nearest even."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32)
    rounding = ((u >> 16) & 1) + np.uint32(0x7FFF)
    out = ((u + rounding) >> 16).astype(np.uint16)
    nan = np.isnan(x)
    if nan.any():
        out[nan] = 0x7FC0
    return out


def from_bf16_bits(b: np.ndarray) -> np.ndarray:
    return (b.astype(np.uint32) << 16).view(np.float32)


def round_bf16(x: np.ndarray) -> np.ndarray:
    """float32 array rounded to bfloat16 values (nearest even), in place for
    finite float32 input (returned), else via a copy."""
    if x.dtype != np.float32 or not x.flags.c_contiguous or not np.isfinite(x).all():
        return from_bf16_bits(to_bf16_bits(x))
    u = x.view(np.uint32)
    t = u >> 16
    t &= 1
    t += 0x7FFF
    u += t
    u &= 0xFFFF0000
    return x


# ----------------------------------------------------------------------------
# structure: tokens and segments
# ----------------------------------------------------------------------------

def zipf_tokens(rng: np.random.Generator, V: int, size, s: float = 1.1) -> np.ndarray:
    """Bounded Zipf(s) over ranks 1..V; token id = rank - 1; inverse CDF."""
    ranks = np.arange(1, V + 1, dtype=np.float64)
    w = ranks ** (-s)
    cdf = np.cumsum(w)
    cdf /= cdf[-1]
    u = rng.random(size)
    return np.minimum(np.searchsorted(cdf, u, side="right"), V - 1).astype(np.int32)


def packed_segments(rng: np.random.Generator, B: int, T: int, lo: int, hi: int) -> np.ndarray:
    seg = np.empty((B, T), dtype=np.int32)
    for b in range(B):
        t, sid = 0, 0
        while t < T:
            L = int(rng.integers(lo, hi + 1))
            L = min(L, T - t)
            seg[b, t:t + L] = sid
            t += L
            sid += 1
    return seg


def tiny_segments() -> np.ndarray:
    seg = np.full((2, 16), -1, dtype=np.int32)
    seg[0, 0:10] = 0
    seg[1, 0:7] = 0
    seg[1, 7:16] = 1
    return seg


# ----------------------------------------------------------------------------
# full chain inputs
# ----------------------------------------------------------------------------

DEPTH_FIELDS = ("g_h", "g_e", "M", "g_a", "Wqkv", "Wo", "g_f", "Wgate", "Wup", "Wdown")


def _normal(rng, shape, sigma, mean=0.0):
    x = rng.standard_normal(shape, dtype=np.float32)
    if sigma != 1.0:
        x *= np.float32(sigma)
    if mean != 0.0:
        x += np.float32(mean)
    return x


def make_chain_inputs(cfg: ChainConfig, seed_offset: int = 0, with_head: bool = True) -> Dict[str, object]:
    """All inputs of one step of ``cfg``.

    Floating arrays are float32 numpy arrays whose values are exactly
    representable in the config's dtype (bf16-rounded for bf16 cases).
    Per-depth weights are a list of dicts (``DEPTH_FIELDS``).  With
    ``with_head=False`` W_out is not drawn (None); every other array is the
    same, since each tensor has its own child stream."""
    ss = np.random.SeedSequence(BASE_SEED + cfg.index + 1000 * seed_offset)
    n_children = 6 + len(DEPTH_FIELDS) * cfg.D
    kids = ss.spawn(n_children)
    gens = [np.random.Generator(np.random.PCG64(k)) for k in kids]
    it = iter(gens)
    B, T, d, V = cfg.B, cfg.T, cfg.d, cfg.V
    A_w, f = cfg.A_w, cfg.ffn
    rnd = round_bf16 if cfg.dtype == "bf16" else (lambda a: a)

    g_tok = next(it)
    tokens = (zipf_tokens(g_tok, V, (B, T)) if cfg.zipf
              else g_tok.integers(0, V, size=(B, T)).astype(np.int32))
    g_seg = next(it)
    if cfg.seg_lo == 0:
        segment_ids = tiny_segments()
        assert segment_ids.shape == (B, T)
    else:
        segment_ids = packed_segments(g_seg, B, T, cfg.seg_lo, cfg.seg_hi)
    h0 = rnd(_normal(next(it), (B * T, d), 1.0))
    E = rnd(_normal(next(it), (V, d), cfg.sigma_w))
    g_w = next(it)
    W_out = rnd(_normal(g_w, (V, d), cfg.sigma_w)) if with_head else None
    g_out = _normal(next(it), (d,), 0.1, 1.0)
    depths: List[Dict[str, np.ndarray]] = []
    for _ in range(cfg.D):
        w = {}
        w["g_h"] = _normal(next(it), (d,), 0.1, 1.0)
        w["g_e"] = _normal(next(it), (d,), 0.1, 1.0)
        w["M"] = rnd(_normal(next(it), (d, 2 * d), cfg.sigma_w))
        w["g_a"] = _normal(next(it), (d,), 0.1, 1.0)
        w["Wqkv"] = rnd(_normal(next(it), (3 * A_w, d), cfg.sigma_w))
        w["Wo"] = rnd(_normal(next(it), (d, A_w), cfg.sigma_w))
        w["g_f"] = _normal(next(it), (d,), 0.1, 1.0)
        w["Wgate"] = rnd(_normal(next(it), (f, d), cfg.sigma_w))
        w["Wup"] = rnd(_normal(next(it), (f, d), cfg.sigma_w))
        w["Wdown"] = rnd(_normal(next(it), (d, f), cfg.sigma_w))
        depths.append(w)
    return dict(cfg=cfg, tokens=tokens, segment_ids=segment_ids, h0=h0, E=E,
                W_out=W_out, g_out=g_out, depths=depths)


def make_head_inputs(cfg: ChainConfig, seed_offset: int = 0, h_sigma: float = 1.0):
    """Inputs of the shared-head CE alone: D hidden-state arrays h^k drawn
    N(0, h_sigma) (stand-ins for chain outputs), W_out, g_out, tokens and
    segments.  Labels are made by the caller from tokens/segments."""
    ss = np.random.SeedSequence(BASE_SEED + 500 + cfg.index + 1000 * seed_offset)
    gens = [np.random.Generator(np.random.PCG64(k)) for k in ss.spawn(4 + cfg.D)]
    B, T, d, V = cfg.B, cfg.T, cfg.d, cfg.V
    rnd = round_bf16 if cfg.dtype == "bf16" else (lambda a: a)
    tokens = (zipf_tokens(gens[0], V, (B, T)) if cfg.zipf
              else gens[0].integers(0, V, size=(B, T)).astype(np.int32))
    if cfg.seg_lo == 0:
        segment_ids = tiny_segments()
    else:
        segment_ids = packed_segments(gens[1], B, T, cfg.seg_lo, cfg.seg_hi)
    W_out = rnd(_normal(gens[2], (V, d), cfg.sigma_w))
    g_out = _normal(gens[3], (d,), 0.1, 1.0)
    hs = [rnd(_normal(gens[4 + k], (B * T, d), h_sigma)) for k in range(cfg.D)]
    return dict(cfg=cfg, tokens=tokens, segment_ids=segment_ids, W_out=W_out,
                g_out=g_out, h=hs)


# ----------------------------------------------------------------------------
# verify inputs
# ----------------------------------------------------------------------------

@dataclasses.dataclass(frozen=True)
class VerifyConfig:
    name: str
    R: int
    gamma: int
    V: int
    temperature: float = 1.0
    target_sigma: float = 2.0
    draft_noise: float = 0.5


def verify_config(gamma: int, R: int = 256, V: int = 129280) -> VerifyConfig:
    return VerifyConfig(f"verify_g{gamma}", R=R, gamma=gamma, V=V)


def make_verify_logits(vc: VerifyConfig, seed_offset: int = 0):
    """Target logits zt ~ N(0, 2) (float32, then bf16) and draft logits
    zd = bf16(zt_f32 + N(0, 0.5)); uniforms for the accept tests and for the
    emission slot.  Draft tokens are NOT drawn here: they must be sampled from
    the draft distribution, which the caller computes (see
    ``sample_draft_tokens``)."""
    ss = np.random.SeedSequence(BASE_SEED + 4 + 100 * vc.gamma + 1000 * seed_offset)
    g = [np.random.Generator(np.random.PCG64(k)) for k in ss.spawn(5)]
    R, G, V = vc.R, vc.gamma, vc.V
    zt32 = _normal(g[0], (R, G + 1, V), vc.target_sigma)
    noise = _normal(g[1], (R, G, V), vc.draft_noise)
    zt = round_bf16(zt32.copy())
    noise += zt32[:, :G, :]
    zd = round_bf16(noise)
    u_accept = g[2].random((R, G), dtype=np.float32)
    u_sample = g[3].random((R, G + 1), dtype=np.float32)
    return dict(vc=vc, zt=zt, zd=zd, u_accept=u_accept, u_sample=u_sample,
                draft_rng=g[4])


def sample_from_probs(rng: np.random.Generator, probs: np.ndarray) -> np.ndarray:
    """Draw one index per row of ``probs`` (rows sum to 1) by inverse CDF.
    Used only to produce draft tokens y ~ q as an input."""
    u = rng.random(probs.shape[:-1])
    cdf = np.cumsum(probs, axis=-1)
    idx = (cdf < u[..., None] * cdf[..., -1:]).sum(axis=-1)
    return np.minimum(idx, probs.shape[-1] - 1).astype(np.int32)
