"""Forward of one MTP module and of the depth chain (test infrastructure only).

Follows M7.6:

* 0x03 / 0x03C: h_bar = RMSNorm_{h,k}(h^(k-1)_i), e_bar = RMSNorm_{e,k}(E(x_(i+k))),
  c = [h_bar; e_bar] in "he" order (hidden block first, 0x07B),
  u = M_k c with M_k in R^{d x 2d}, no bias;
  RMSNorm_g(z) = g * z / sqrt(mean(z^2) + eps);
* 0x03C: a pre-norm block, a = u + Attention(Norm_a(u); causal mask),
  h^(k) = a + FFN(Norm_f(a));
* 0x04C / 0x06A: the causal mask is segment-aware -- row i sees keys j of its
  own run with j <= i -- and positions are semantic (offset inside the run).

Declared readings where the pages leave the block open: multi-head attention
with H heads of width head_dim, no biases, scores scaled by 1/sqrt(head_dim);
rotate-half RoPE over the whole head with theta given (theta 0 = none) at
position i - run_start(i); FFN = SwiGLU, (silu(y Wg^T) * (y Wu^T)) Wd^T; block
norms are RMSNorms with their own gains.

Rows whose state is not supported at depth k (see ``rows``) are still
computed (the dense layout keeps them) with the shifted-token index clamped to
the last position; their values are unspecified and never compared.  A
padding row is its own one-key attention window.

Parity: RMSNorm, RoPE, attention and SwiGLU are pinned by closed forms and a
library attention routine in the tests; the block composition itself (order
of the sub-layers, choice of MHA/SwiGLU) is a declared reading the pages do
not fix numerically -- parity unpinned beyond those sub-step pins.
"""
from __future__ import annotations

from typing import Dict, List

import numpy as np

from .numerics import EXACT, Model
from .rows import run_bounds


def rmsnorm(z: np.ndarray, g: np.ndarray, eps: float) -> np.ndarray:
    """RMSNorm_g(z) = g * z / sqrt(mean_j z_j^2 + eps), row-wise (M7.6 0x03C)."""
    z = np.asarray(z, dtype=np.float64)
    ms = np.mean(z * z, axis=-1, keepdims=True)
    return np.asarray(g, dtype=np.float64) * z / np.sqrt(ms + eps)


def rms_inverse(z: np.ndarray, eps: float) -> np.ndarray:
    """1 / sqrt(mean(z^2) + eps) per row."""
    z = np.asarray(z, dtype=np.float64)
    return 1.0 / np.sqrt(np.mean(z * z, axis=-1) + eps)


def rope(x: np.ndarray, pos: np.ndarray, theta: float) -> np.ndarray:
    """Rotate-half rotary embedding of x [..., L, hd] at integer positions
    pos [L]: for j < hd/2, with w_j = theta^(-2j/hd) and angle = pos * w_j,
    out_j = x_j cos - x_(j+hd/2) sin and out_(j+hd/2) = x_(j+hd/2) cos + x_j sin."""
    if theta == 0:
        return x
    hd = x.shape[-1]
    half = hd // 2
    j = np.arange(half, dtype=np.float64)
    w = theta ** (-2.0 * j / hd)
    ang = np.asarray(pos, dtype=np.float64)[:, None] * w[None, :]
    cos, sin = np.cos(ang), np.sin(ang)
    x1, x2 = x[..., :half], x[..., half:]
    return np.concatenate([x1 * cos - x2 * sin, x2 * cos + x1 * sin], axis=-1)


def segment_causal_attention(q: np.ndarray, k: np.ndarray, v: np.ndarray,
                             segment_row: np.ndarray) -> np.ndarray:
    """q, k, v: [T, H, hd] of one batch row.  o_i = sum over keys j of i's run
    with j <= i of softmax_j(q_i . k_j / sqrt(hd)) v_j; a padding row attends
    to itself only."""
    T, H, hd = q.shape
    out = np.zeros_like(q, dtype=np.float64)
    rs, _ = run_bounds(np.asarray(segment_row)[None, :])
    rs = rs[0]
    seg = np.asarray(segment_row)
    scale = 1.0 / np.sqrt(hd)
    # Group rows by window start: a run is one contiguous block of queries
    # whose keys are the same block restricted to j <= i.
    i = 0
    while i < T:
        if seg[i] < 0:
            out[i] = v[i]
            i += 1
            continue
        r0 = i
        r1 = i
        while r1 + 1 < T and rs[r1 + 1] == r0:
            r1 += 1
        L = r1 - r0 + 1
        causal = np.tril(np.ones((L, L), dtype=bool))
        for h in range(H):
            s = (q[r0:r1 + 1, h, :] @ k[r0:r1 + 1, h, :].T) * scale
            s = np.where(causal, s, -np.inf)
            s = s - s.max(axis=1, keepdims=True)
            p = np.exp(s)
            p /= p.sum(axis=1, keepdims=True)
            out[r0:r1 + 1, h, :] = p @ v[r0:r1 + 1, h, :]
        i = r1 + 1
    return out


def silu(x: np.ndarray) -> np.ndarray:
    return x / (1.0 + np.exp(-x))


def module_forward(h_prev: np.ndarray, tokens: np.ndarray, segment_ids: np.ndarray,
                   depth: int, w: Dict[str, np.ndarray], E: np.ndarray,
                   n_heads: int, head_dim: int, eps: float, rope_theta: float,
                   model: Model = EXACT, keep: bool = False):
    """One MTP module on the dense [B, T] layout.

    h_prev: [B*T, d] (row b*T + i).  Returns h^(k) [B*T, d] (and the named
    intermediates when ``keep``)."""
    B, T = segment_ids.shape
    N = B * T
    d = h_prev.shape[1]
    A_w = n_heads * head_dim
    st = model.store
    h_prev = np.asarray(h_prev, dtype=np.float64)

    # shifted ground-truth token x_(i+k) (clamped for rows that have none)
    idx = np.minimum(np.arange(T) + depth, T - 1)
    shifted = np.clip(np.asarray(tokens)[:, idx], 0, E.shape[0] - 1).reshape(N)
    e = np.asarray(E, dtype=np.float64)[shifted]

    h_bar = rmsnorm(h_prev, w["g_h"], eps)
    e_bar = rmsnorm(e, w["g_e"], eps)
    c = st(np.concatenate([h_bar, e_bar], axis=1))                      # [N, 2d]
    u = c @ np.asarray(w["M"], np.float64).T                             # [N, d], wide

    x_a = st(rmsnorm(u, w["g_a"], eps))
    qkv = x_a @ np.asarray(w["Wqkv"], np.float64).T                      # [N, 3A]
    q = qkv[:, :A_w].reshape(B, T, n_heads, head_dim)
    k = qkv[:, A_w:2 * A_w].reshape(B, T, n_heads, head_dim)
    v = qkv[:, 2 * A_w:].reshape(B, T, n_heads, head_dim)
    rs, _ = run_bounds(segment_ids)
    pos = np.arange(T)[None, :] - rs                                     # [B, T]
    o = np.empty((B, T, n_heads, head_dim), dtype=np.float64)
    qr = np.empty_like(q)
    kr = np.empty_like(k)
    for b in range(B):
        # RoPE acts per head on [T, hd]; move heads first
        qb = rope(np.transpose(q[b], (1, 0, 2)), pos[b], rope_theta)
        kb = rope(np.transpose(k[b], (1, 0, 2)), pos[b], rope_theta)
        qr[b] = st(np.transpose(qb, (1, 0, 2)))
        kr[b] = st(np.transpose(kb, (1, 0, 2)))
    v = st(v)
    for b in range(B):
        o[b] = segment_causal_attention(qr[b], kr[b], v[b], segment_ids[b])
    o = st(o.reshape(N, A_w))
    a = u + o @ np.asarray(w["Wo"], np.float64).T                        # wide

    y = st(rmsnorm(a, w["g_f"], eps))
    gate = y @ np.asarray(w["Wgate"], np.float64).T
    up = y @ np.asarray(w["Wup"], np.float64).T
    gsw = st(silu(gate) * up)
    h = st(a + gsw @ np.asarray(w["Wdown"], np.float64).T)
    if keep:
        return h, dict(c=c, u=u, x_a=x_a, q=qr.reshape(N, A_w), k=kr.reshape(N, A_w),
                       v=v.reshape(N, A_w), o=o, a=a, y=y, gsw=gsw, h=h)
    return h


def chain_forward(h0: np.ndarray, tokens: np.ndarray, segment_ids: np.ndarray,
                  depths: List[Dict[str, np.ndarray]], E: np.ndarray,
                  n_heads: int, head_dim: int, eps: float, rope_theta: float,
                  model: Model = EXACT) -> List[np.ndarray]:
    """h^(1..D): depth k consumes h^(k-1) and x_(i+k) (M7.6 0x02, 0x06A).
    Row i of depth k reads row i of depth k-1 (dense layout: the predecessor
    of a state row is always present, since state(k,i) implies
    state(k-1,i))."""
    hs = []
    h = np.asarray(h0, dtype=np.float64)
    for k, w in enumerate(depths, start=1):
        h = module_forward(h, tokens, segment_ids, k, w, E, n_heads, head_dim,
                           eps, rope_theta, model)
        hs.append(h)
    return hs


# ----------------------------------------------------------------------------
# Compact packed-stream form (M7.6 0x04C gather rules, 0x06A training loop)
# ----------------------------------------------------------------------------

def compact_module_forward(previous: np.ndarray, shifted_tokens: np.ndarray,
                           positions: np.ndarray, segments: np.ndarray,
                           w: Dict[str, np.ndarray], E: np.ndarray, n_heads: int,
                           head_dim: int, eps: float, rope_theta: float) -> np.ndarray:
    """The module on compact rows (exact model): row r may attend to row s iff
    both carry the same segment and position[s] <= position[r].  Written with
    per-row loops, independently of the dense path."""
    n, d = previous.shape
    A_w = n_heads * head_dim
    e = np.asarray(E, np.float64)[np.asarray(shifted_tokens)]
    c = np.concatenate([rmsnorm(previous, w["g_h"], eps), rmsnorm(e, w["g_e"], eps)], axis=1)
    u = c @ np.asarray(w["M"], np.float64).T
    x_a = rmsnorm(u, w["g_a"], eps)
    qkv = x_a @ np.asarray(w["Wqkv"], np.float64).T
    q = qkv[:, :A_w].reshape(n, n_heads, head_dim).transpose(1, 0, 2)
    k = qkv[:, A_w:2 * A_w].reshape(n, n_heads, head_dim).transpose(1, 0, 2)
    v = qkv[:, 2 * A_w:].reshape(n, n_heads, head_dim).transpose(1, 0, 2)
    q = rope(q, positions, rope_theta)
    k = rope(k, positions, rope_theta)
    o = np.zeros((n, n_heads, head_dim))
    for r in range(n):
        keys = [s for s in range(n)
                if segments[s] == segments[r] and positions[s] <= positions[r]]
        for hh in range(n_heads):
            sc = np.array([q[hh, r] @ k[hh, s] for s in keys]) / np.sqrt(head_dim)
            p = np.exp(sc - sc.max())
            p /= p.sum()
            o[r, hh] = sum(p[t] * v[hh, s] for t, s in enumerate(keys))
    a = u + o.reshape(n, A_w) @ np.asarray(w["Wo"], np.float64).T
    y = rmsnorm(a, w["g_f"], eps)
    gsw = silu(y @ np.asarray(w["Wgate"], np.float64).T) * (y @ np.asarray(w["Wup"], np.float64).T)
    return a + gsw @ np.asarray(w["Wdown"], np.float64).T


def compact_training_step(tokens_row, segment_row, h0_rows, depths, E, W_out, g_out,
                          n_heads, head_dim, eps, rope_theta, lam, T_fixed):
    """The packed-stream training loop of M7.6 0x06A on one stream, exact
    model: per depth compile rows, gather previous rows by physical row,
    shifted tokens by packed address and positions by semantic position, run
    the module, carry (state, state_bases) and add token_loss_sum / T; an
    empty depth adds a zero term that stays in the D-way mean.  Returns the
    per-depth compact states with their bases, the per-depth loss terms and
    lam * mean(terms)."""
    from .rows import compile_mtp_rows
    from .head import output_norm, logsumexp_rows
    n = len(tokens_row)
    valid = [s >= 0 for s in segment_row]
    state = np.asarray(h0_rows, np.float64)
    bases = list(range(n))
    terms, states = [], []
    for k, w in enumerate(depths, start=1):
        assert state.shape[0] == len(bases)
        rows_k = compile_mtp_rows(list(tokens_row), list(segment_row), valid, k, bases)
        if not rows_k:
            terms.append(0.0)
            state, bases = state[:0], []
            states.append((state, bases))
            continue
        prev = state[[r["previous_depth_row"] for r in rows_k]]
        shifted = np.array([tokens_row[r["shifted_token_index"]] for r in rows_k])
        pos = np.array([r["position"] for r in rows_k])
        segs = np.array([r["segment"] for r in rows_k])
        cur = compact_module_forward(prev, shifted, pos, segs, w, E, n_heads, head_dim,
                                     eps, rope_theta)
        state = cur
        bases = [r["base"] for r in rows_k]
        states.append((state, bases))
        loss_rows = [j for j, r in enumerate(rows_k) if r["loss_valid"]]
        if loss_rows:
            labels = np.array([tokens_row[rows_k[j]["label_index"]] for j in loss_rows])
            x_hat, _, _ = output_norm(cur[loss_rows], g_out, eps)
            z = x_hat @ np.asarray(W_out, np.float64).T
            ell = logsumexp_rows(z) - z[np.arange(len(loss_rows)), labels]
            terms.append(ell.sum() / T_fixed)
        else:
            terms.append(0.0)
    return states, terms, lam * float(np.mean(terms))
