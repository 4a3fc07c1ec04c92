"""Independent prediction horizons on one trunk state (test infrastructure
only).

Follows M7.4:

* 0x02: head k receives the representation of the causal prefix and
  predicts the token k positions ahead; the weighted objective sums
  -log p^(k)(x_(t+k) | x_<=t) over the positions that have that label;
* 0x02A / 0x01A: horizon k has a label at t only when t + k stays inside
  the sequence -- here inside t's segment run (the packed two-row fixture's
  horizon pairs (t, t+k) inside one segment);
* 0x06A: each head's forward and backward finish before the next head's,
  and the trunk receives the sum of the heads' gradients once.

Two head forms:

* ``independent_heads`` -- g_k = identity (0x02 allows it for a head), so
  every horizon applies the shared head Norm_out + W_U to the trunk state h
  itself;
* ``block_heads`` -- g_k a Transformer block of its own (0x05B: each horizon
  gets an independent transformer head, the vocabulary projection is
  shared): u^(k) = Block_k(h) with the MTP module's block (pre-norm
  segment-causal multi-head attention with RoPE, then SwiGLU, residual adds;
  the same block as ``chain.module_forward`` without eh_proj), then the
  shared head on u^(k).  Each head's forward and backward run in turn and
  the trunk gradient is the sum of the heads' (0x06A).

Both use lambda_k = lambda / K and the fixed denominator B*T -- the chain
objective's scaling with D = K.

Pins (tests/test_oracle_horizons.py): the fixture's horizon counts 9 / 6 / 3;
horizon k+1's labels equal the dense chain rows' depth-k labels (a separate
implementation of the run rule); central finite differences of the summed
objective with respect to h (both forms) and to every block weight, gain,
W_out and g_out (block heads); block heads whose output projections W_o and
W_down are zero reduce exactly to the identity heads.
"""
from __future__ import annotations

import numpy as np

from . import head
from .backward import block_backward
from .chain import rmsnorm, rope, segment_causal_attention, silu
from .numerics import EXACT, Model
from .rows import run_bounds

BLOCK_PARAMS = ("g_a", "Wqkv", "Wo", "g_f", "Wgate", "Wup", "Wdown")


def horizon_labels(tokens: np.ndarray, segment_ids: np.ndarray, K: int) -> np.ndarray:
    """[K, B*T]: row k-1 holds x_(t+k) where t is in a run and t + k <= the
    run's end, else -1."""
    tokens = np.asarray(tokens)
    seg = np.asarray(segment_ids)
    B, T = seg.shape
    _, re = run_bounds(seg)
    out = np.full((K, B, T), -1, dtype=np.int64)
    for k in range(1, K + 1):
        for b in range(B):
            for t in range(T):
                if seg[b, t] >= 0 and t + k <= re[b, t]:
                    out[k - 1, b, t] = tokens[b, t + k]
    return out.reshape(K, B * T)


def independent_heads(h: np.ndarray, tokens: np.ndarray, segment_ids: np.ndarray, K: int, W_out: np.ndarray,
                      g_out: np.ndarray, eps: float, lam: float, model: Model = EXACT, grads: bool = True):
    """The K horizons' losses on one trunk state h [B*T, d]; with grads, the
    per-horizon gradients and dh_trunk = their sum."""
    labels = horizon_labels(tokens, segment_ids, K)
    out = head.head_ce([h] * K, labels, W_out, g_out, eps, lam, "fixed", None, model, grads=grads)
    out["labels"] = labels
    if grads:
        out["dh_trunk"] = np.sum(out["dh"], axis=0)
    return out


def block_forward(h: np.ndarray, segment_ids: np.ndarray, w, n_heads: int, head_dim: int, eps: float,
                  rope_theta: float, model: Model = EXACT, keep: bool = False):
    """Block_k(h) on the dense [B, T] layout (M7.6 0x03C's block, read as in
    ``chain.module_forward``): a = h + Attn(Norm_a(h)), u = a + FFN(Norm_f(a)),
    stored at the model's rounding points; h [B*T, d]."""
    B, T = np.asarray(segment_ids).shape
    N = B * T
    A_w = n_heads * head_dim
    st = model.store
    h = np.asarray(h, np.float64)
    x_a = st(rmsnorm(h, w["g_a"], eps))
    qkv = x_a @ np.asarray(w["Wqkv"], np.float64).T
    q = qkv[:, :A_w].reshape(B, T, n_heads, head_dim)
    k = qkv[:, A_w:2 * A_w].reshape(B, T, n_heads, head_dim)
    v = st(qkv[:, 2 * A_w:].reshape(B, T, n_heads, head_dim))
    rs, _ = run_bounds(np.asarray(segment_ids))
    pos = np.arange(T)[None, :] - rs
    qr = np.empty_like(q)
    kr = np.empty_like(k)
    o = np.empty_like(q)
    for b in range(B):
        qr[b] = st(np.transpose(rope(np.transpose(q[b], (1, 0, 2)), pos[b], rope_theta), (1, 0, 2)))
        kr[b] = st(np.transpose(rope(np.transpose(k[b], (1, 0, 2)), pos[b], rope_theta), (1, 0, 2)))
        o[b] = segment_causal_attention(qr[b], kr[b], v[b], np.asarray(segment_ids)[b])
    o = st(o.reshape(N, A_w))
    a = h + o @ np.asarray(w["Wo"], np.float64).T
    y = st(rmsnorm(a, w["g_f"], eps))
    gate = y @ np.asarray(w["Wgate"], np.float64).T
    up = y @ np.asarray(w["Wup"], np.float64).T
    gsw = st(silu(gate) * up)
    u = st(a + gsw @ np.asarray(w["Wdown"], np.float64).T)
    if keep:
        return u, dict(u_in=h, x_a=x_a, q=qr.reshape(N, A_w), k=kr.reshape(N, A_w), v=v.reshape(N, A_w), o=o,
                       a=a, y=y, gsw=gsw)
    return u


def block_heads(h: np.ndarray, tokens: np.ndarray, segment_ids: np.ndarray, blocks, W_out: np.ndarray,
                g_out: np.ndarray, n_heads: int, head_dim: int, eps: float, rope_theta: float, lam: float,
                model: Model = EXACT, grads: bool = True, denom: float = None):
    """K = len(blocks) horizons, head k = the shared head on Block_k(h);
    denom: the fixed denominator (default B*T of these rows).
    Returns the head CE's outputs (loss, loss_mtp, counts, dW_out, dg_out)
    and, with grads, dh_trunk = sum over heads of dL/dh through head k and
    ``blocks_grad`` = per-head dicts of block-parameter gradients."""
    K = len(blocks)
    labels = horizon_labels(tokens, segment_ids, K)
    outs, acts = [], []
    for w in blocks:
        u, act = block_forward(h, segment_ids, w, n_heads, head_dim, eps, rope_theta, model, keep=True)
        outs.append(u)
        acts.append(act)
    out = head.head_ce(outs, labels, W_out, g_out, eps, lam, "fixed", denom, model, grads=grads)
    out["labels"] = labels
    if grads:
        dh = np.zeros_like(np.asarray(h, np.float64))
        bg = []
        for k, w in enumerate(blocks):
            r = block_backward(acts[k], segment_ids, w, n_heads, head_dim, eps, rope_theta, out["dh"][k], model)
            dh += r.pop("du_in")
            bg.append(r)
        out["dh_trunk"] = dh
        out["blocks_grad"] = bg
    return out
