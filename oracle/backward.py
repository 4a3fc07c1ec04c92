"""Gradients of L_MTP through the whole depth chain (test infrastructure only).

Follows M7.6:

* 0x05A ("The MTP gradient reaches"): the MTP loss reaches the module's own
  parameters (enorm, hnorm, eh_proj, the Transformer block), the shared
  token embedding and output head, and the main model through h^(0); a
  deeper loss reaches h^(0) through every module before it, as the product
  of the per-depth Jacobians dh^(k)/dh^(k-1);
* 0x05B: the ledger -- a depth-j module's parameters receive
  sum_{k=j..D} (lambda/D) dL^(k)/dtheta_j (its own loss and every deeper
  loss that traverses it, none from shallower ones), and the shared
  embedding sums every depth's contribution.

The chain gradient is the reverse of ``chain.module_forward`` taken one
depth at a time, from D down to 1.  The gradient arriving at h^(k) is the
head's (``head.head_ce``'s dh for depth k) plus what depth k+1 sends back
through its hnorm input; depth 1 sends its share to h^(0).  Each module's
reverse pass, written from the forward's definitions (y = x W^T gives
dx = dy W and dW = dy^T x; a residual add passes its gradient to both
terms):

* SwiGLU: with s = silu(a), silu'(a) = sig(a) (1 + a (1 - sig(a))),
  d gate = d(gsw) * up * silu'(gate), d up = d(gsw) * silu(gate);
* RMSNorm_g(z) = g z r with r = 1/sqrt(mean(z^2) + eps) and x_n = z r:
  dz = r (g dy - x_n mean(x_n g dy)), dg = sum over rows of dy x_n;
* attention per head and run window (P = softmax(S), S = Q K^T / sqrt(hd),
  causal inside the run): dV = P^T dO, dP = dO V^T,
  dS = P (dP - rowsum(P dP)), dQ = dS K / sqrt(hd), dK = dS^T Q / sqrt(hd);
* rotate-half RoPE is a rotation per (j, j + hd/2) pair, so its reverse is
  the rotation by the opposite angle;
* the gathered embedding row E[x_(i+k)] passes its gradient back to that
  row of E (a scatter-add over every row and depth that read it).

Numerical model: with ``model = BF16`` the recomputed forward rounds at the
forward's storage points (``numerics``) and the reverse pass rounds, like
the GPU, every gradient it hands to a matrix product as an operand: the
gradient entering a module, d(gsw), d gate and d up, da, dO, the RoPE'd
dq/dk/dv and du.  Residual sums, norm statistics and accumulated weight
gradients stay wide.  EXACT rounds nothing.

Pins (tests/test_oracle_backward.py): central finite differences of L_MTP in
float64 (M7.4 0x04C's reconciliation) for h^(0), E, every per-depth weight
and gain at D = 2 on the tiny packed layout, including rows and embedding
entries whose gradient is exactly 0 (padding, tokens never read); the 0x05B
ledger structure (a depth-2 module receives nothing from a depth-1-only
loss, a depth-1 module receives the depth-2 loss); the attention reverse
against brute-force differences of a standalone attention.
"""
from __future__ import annotations

from typing import Dict, List, Sequence

import numpy as np

from .chain import module_forward, rms_inverse, silu
from .head import head_ce
from .numerics import EXACT, Model
from .rows import dense_rows, run_bounds

PARAMS = ("g_h", "g_e", "M", "g_a", "Wqkv", "Wo", "g_f", "Wgate", "Wup", "Wdown")


def rmsnorm_backward(z: np.ndarray, g: np.ndarray, eps: float, dy: np.ndarray):
    """Reverse of y = g * z * r (row-wise RMSNorm).  Returns (dz, dg)."""
    z = np.asarray(z, np.float64)
    r = rms_inverse(z, eps)[:, None]
    x_n = z * r
    gdy = np.asarray(g, np.float64)[None, :] * dy
    dz = r * (gdy - x_n * np.mean(x_n * gdy, axis=1, keepdims=True))
    dg = np.sum(dy * x_n, axis=0)
    return dz, dg


def silu_grad(x: np.ndarray) -> np.ndarray:
    sig = 1.0 / (1.0 + np.exp(-x))
    return sig * (1.0 + x * (1.0 - sig))


def rope_reverse(dx: np.ndarray, pos: np.ndarray, theta: float) -> np.ndarray:
    """Gradient through rotate-half RoPE: rotate each (j, j + hd/2) pair of
    dx [..., L, hd] by the opposite angle pos * theta^(-2j/hd)."""
    if theta == 0:
        return dx
    hd = dx.shape[-1]
    half = hd // 2
    w = theta ** (-2.0 * np.arange(half, dtype=np.float64) / hd)
    ang = np.asarray(pos, np.float64)[:, None] * w[None, :]
    cos, sin = np.cos(ang), np.sin(ang)
    d1, d2 = dx[..., :half], dx[..., half:]
    return np.concatenate([d1 * cos + d2 * sin, d2 * cos - d1 * sin], axis=-1)


def attention_backward(q: np.ndarray, k: np.ndarray, v: np.ndarray, do: np.ndarray,
                       segment_row: np.ndarray):
    """Reverse of ``chain.segment_causal_attention`` for one batch row:
    q, k, v, do [T, H, hd].  Returns (dq, dk, dv)."""
    T, H, hd = q.shape
    dq = np.zeros((T, H, hd))
    dk = np.zeros((T, H, hd))
    dv = np.zeros((T, H, hd))
    seg = np.asarray(segment_row)
    rs, re = run_bounds(seg[None, :])
    rs, re = rs[0], re[0]
    scale = 1.0 / np.sqrt(hd)
    i = 0
    while i < T:
        if seg[i] < 0:            # padding: o_i = v_i
            dv[i] += do[i]
            i += 1
            continue
        r0, r1 = i, int(re[i])
        L = r1 - r0 + 1
        causal = np.tril(np.ones((L, L), dtype=bool))
        for h in range(H):
            Q, K, Vv, dO = q[r0:r1 + 1, h], k[r0:r1 + 1, h], v[r0:r1 + 1, h], do[r0:r1 + 1, h]
            s = np.where(causal, (Q @ K.T) * scale, -np.inf)
            p = np.exp(s - s.max(axis=1, keepdims=True))
            p /= p.sum(axis=1, keepdims=True)
            dv[r0:r1 + 1, h] += p.T @ dO
            dp = dO @ Vv.T
            ds = p * (dp - np.sum(p * dp, axis=1, keepdims=True))
            dq[r0:r1 + 1, h] += (ds @ K) * scale
            dk[r0:r1 + 1, h] += (ds.T @ Q) * scale
        i = r1 + 1
    return dq, dk, dv


def block_backward(act: Dict[str, np.ndarray], segment_ids: np.ndarray, w: Dict[str, np.ndarray], n_heads: int,
                   head_dim: int, eps: float, rope_theta: float, dh: np.ndarray, model: Model = EXACT):
    """Reverse of the block a = u + Attn(Norm_a(u)), h = a + FFN(Norm_f(a))
    given dL/dh = dh, from the forward's stored activations ``act`` (u_in,
    x_a, q, k, v after RoPE, o, a, y, gsw).  Returns dict(du_in = dL/du and the
    gradients of g_a, Wqkv, Wo, g_f, Wgate, Wup, Wdown)."""
    B, T = np.asarray(segment_ids).shape
    N = B * T
    A_w = n_heads * head_dim
    st = model.store
    W = {n: np.asarray(w[n], np.float64) for n in ("g_a", "Wqkv", "Wo", "g_f", "Wgate", "Wup", "Wdown")}
    out: Dict[str, np.ndarray] = {}
    # h = a + gsw Wd^T
    g = st(np.asarray(dh, np.float64))
    out["Wdown"] = g.T @ act["gsw"]
    dgsw = st(g @ W["Wdown"])
    gate = act["y"] @ W["Wgate"].T
    up = act["y"] @ W["Wup"].T
    dgate = st(dgsw * up * silu_grad(gate))
    dup = st(dgsw * silu(gate))
    out["Wgate"] = dgate.T @ act["y"]
    out["Wup"] = dup.T @ act["y"]
    dy = dgate @ W["Wgate"] + dup @ W["Wup"]
    # y = RMSNorm_{g_f}(a); the residual passes dh to a
    da_norm, out["g_f"] = rmsnorm_backward(act["a"], W["g_f"], eps, dy)
    da = np.asarray(dh, np.float64) + da_norm
    # a = u + o Wo^T
    dab = st(da)
    out["Wo"] = dab.T @ act["o"]
    do = st(dab @ W["Wo"])
    # attention on the RoPE'd q, k and on v, per batch row
    rs, _ = run_bounds(segment_ids)
    pos = np.arange(T)[None, :] - rs
    q = act["q"].reshape(B, T, n_heads, head_dim)
    k = act["k"].reshape(B, T, n_heads, head_dim)
    v = act["v"].reshape(B, T, n_heads, head_dim)
    dO = do.reshape(B, T, n_heads, head_dim)
    dqkv = np.zeros((N, 3 * A_w))
    for b in range(B):
        dq, dk, dv = attention_backward(q[b], k[b], v[b], dO[b], segment_ids[b])
        dq = np.transpose(rope_reverse(np.transpose(dq, (1, 0, 2)), pos[b], rope_theta), (1, 0, 2))
        dk = np.transpose(rope_reverse(np.transpose(dk, (1, 0, 2)), pos[b], rope_theta), (1, 0, 2))
        rows = slice(b * T, (b + 1) * T)
        dqkv[rows, :A_w] = dq.reshape(T, A_w)
        dqkv[rows, A_w:2 * A_w] = dk.reshape(T, A_w)
        dqkv[rows, 2 * A_w:] = dv.reshape(T, A_w)
    dqkv = st(dqkv)
    out["Wqkv"] = dqkv.T @ act["x_a"]
    dxa = dqkv @ W["Wqkv"]
    # x_a = RMSNorm_{g_a}(u); the residual passes da to u
    du_norm, out["g_a"] = rmsnorm_backward(act["u_in"], W["g_a"], eps, dxa)
    out["du_in"] = da + du_norm
    return out


def module_backward(h_prev: np.ndarray, tokens: np.ndarray, segment_ids: np.ndarray, depth: int,
                    w: Dict[str, np.ndarray], E: np.ndarray, n_heads: int, head_dim: int, eps: float,
                    rope_theta: float, dh: np.ndarray, model: Model = EXACT):
    """Gradients of one module (M7.6 0x03/0x03C forward) given dL/dh^(k) = dh
    [B*T, d] at its output.  Returns dict(dh_prev [B*T, d], dE [V, d],
    and one entry per parameter name in PARAMS)."""
    B, T = segment_ids.shape
    N = B * T
    A_w = n_heads * head_dim
    st = model.store
    W = {n: np.asarray(w[n], np.float64) for n in PARAMS}
    _, act = module_forward(h_prev, tokens, segment_ids, depth, w, E, n_heads, head_dim, eps,
                            rope_theta, model, keep=True)
    h_prev = np.asarray(h_prev, np.float64)
    idx = np.minimum(np.arange(T) + depth, T - 1)
    shifted = np.clip(np.asarray(tokens)[:, idx], 0, E.shape[0] - 1).reshape(N)
    e = np.asarray(E, np.float64)[shifted]
    out: Dict[str, np.ndarray] = {}

    act = dict(act, u_in=act["u"])
    r = block_backward(act, segment_ids, w, n_heads, head_dim, eps, rope_theta, dh, model)
    du = r.pop("du_in")
    out.update(r)
    # u = M [h_bar; e_bar]
    dub = st(du)
    out["M"] = dub.T @ act["c"]
    dc = dub @ W["M"]
    d = h_prev.shape[1]
    out["dh_prev"], out["g_h"] = rmsnorm_backward(h_prev, W["g_h"], eps, dc[:, :d])
    de, out["g_e"] = rmsnorm_backward(e, W["g_e"], eps, dc[:, d:])
    dE = np.zeros(np.asarray(E).shape)
    np.add.at(dE, shifted, de)
    out["dE"] = dE
    return out


def chain_backward(h0: np.ndarray, tokens: np.ndarray, segment_ids: np.ndarray,
                   depths: List[Dict[str, np.ndarray]], E: np.ndarray, n_heads: int, head_dim: int,
                   eps: float, rope_theta: float, dh_head: Sequence[np.ndarray], model: Model = EXACT):
    """Reverse of ``chain.chain_forward`` given the head's gradients dh_head[k]
    = dL_MTP/dh^(k+1) through the head alone.  Returns dict(dh0, dE, depths =
    list of per-depth parameter-gradient dicts)."""
    D = len(depths)
    hs = [np.asarray(h0, np.float64)]
    for k in range(1, D + 1):
        hs.append(module_forward(hs[-1], tokens, segment_ids, k, depths[k - 1], E, n_heads, head_dim,
                                 eps, rope_theta, model))
    dE = np.zeros(np.asarray(E).shape)
    grads: List[Dict[str, np.ndarray]] = [None] * D
    g = np.asarray(dh_head[D - 1], np.float64)
    for k in range(D, 0, -1):
        res = module_backward(hs[k - 1], tokens, segment_ids, k, depths[k - 1], E, n_heads, head_dim,
                              eps, rope_theta, g, model)
        dE += res.pop("dE")
        dprev = res.pop("dh_prev")
        grads[k - 1] = res
        g = dprev + (np.asarray(dh_head[k - 2], np.float64) if k > 1 else 0.0)
    return dict(dh0=g, dE=dE, depths=grads, h=hs[1:])


def mtp_gradients(h0, tokens, segment_ids, depths, E, W_out, g_out, n_heads, head_dim, eps, rope_theta,
                  lam, reduce="fixed", denom=None, model: Model = EXACT, labels=None):
    """The whole MTP objective's gradients: chain forward, head CE (its loss
    and its gradients at each h^(k), W_out and g_out), then the chain reverse.
    ``labels`` [D, B*T] overrides the rows' labels (e.g. to keep a subset)."""
    D = len(depths)
    B, T = np.asarray(segment_ids).shape
    if labels is None:
        _, _, labels, _ = dense_rows(tokens, segment_ids, D)
    labels = np.asarray(labels).reshape(D, B * T)
    hs = [np.asarray(h0, np.float64)]
    for k in range(1, D + 1):
        hs.append(module_forward(hs[-1], tokens, segment_ids, k, depths[k - 1], E, n_heads, head_dim,
                                 eps, rope_theta, model))
    head = head_ce(hs[1:], labels, W_out, g_out, eps, lam, reduce, denom, model)
    back = chain_backward(h0, tokens, segment_ids, depths, E, n_heads, head_dim, eps, rope_theta,
                          head["dh"], model)
    back.update(loss_mtp=head["loss_mtp"], dW_out=head["dW_out"], dg_out=head["dg_out"], head=head)
    return back
