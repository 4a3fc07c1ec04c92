"""One recurrent draft step of a retained MTP module (test infrastructure only).

Follows M7.6:

* 0x09: the proposal for the position after the incoming token f is seeded by
  the saved parent hidden state and E(f), and y is sampled from the module's
  normalised distribution q, which verification then uses;
* 0x09A: a module served autoregressively keeps its own K/V cache -- the keys
  and values of earlier positions are that module's own projections of its
  inputs there;
* 0x09D: one module rolled out for several draft steps feeds back its own
  output hidden state and the newly drafted token.

Reading.  A request's module inputs are rows (h_j, x_j) for cache slots
j = 0..p, slot index = RoPE position.  The step at slot p runs the block of
the chain (pre-norm attention and SwiGLU, the storage rounding points of the
chain oracle) with the query of slot p attending to slots 0..p; the keys and
values of slots < p are those the same module computed from their rows.  So
the step equals the module evaluated on the whole row sequence, read at its
last row -- this file computes exactly that, with per-row loops.  Then
logits = store(W_out RMSNorm_{g_out}(h_p)) -- stored values, since they are
what verification reads -- and y = the inverse CDF of softmax(logits / tau)
with u (the verify oracle's rule).

Pins (tests/test_oracle_propose.py): the step at every slot of a prefix,
cache built slot by slot, equals the dense chain oracle's teacher-forced rows
of one segment (a different implementation: vectorised, dense layout,
shifted-token gather); a one-slot step attends only to itself, so its
attention output is its own value row; logits with one dominant entry draw
it for every u, equal logits draw floor(u V).
"""
from __future__ import annotations

from typing import Dict, List, Sequence

import numpy as np

from .chain import rmsnorm, rope, silu
from .numerics import EXACT, Model
from .verify import inverse_cdf, softmax64

OK, BAD_UNIFORM, BAD_TOKEN, NONFINITE, BAD_POSITION = 0, 1, 2, 5, 6


def module_rows(h_rows: np.ndarray, tok_rows: Sequence[int], w: Dict[str, np.ndarray], E: np.ndarray,
                n_heads: int, head_dim: int, eps: float, theta: float, model: Model = EXACT):
    """Block output of every slot j = 0..p of one request (slot j attends to
    slots 0..j).  h_rows [p+1, d]; tok_rows [p+1].  Returns (h [p+1, d],
    k [p+1, A], v [p+1, A]) -- k after RoPE, both as stored."""
    st = model.store
    n = len(tok_rows)
    A = n_heads * head_dim
    Wq = np.asarray(w["Wqkv"], np.float64)
    out = np.zeros((n, h_rows.shape[1]))
    qs = np.zeros((n, A))
    ks = np.zeros((n, A))
    vs = np.zeros((n, A))
    us = []
    for j in range(n):
        hb = rmsnorm(np.asarray(h_rows[j], np.float64)[None, :], w["g_h"], eps)
        eb = rmsnorm(np.asarray(E[int(tok_rows[j])], np.float64)[None, :], w["g_e"], eps)
        c = st(np.concatenate([hb, eb], axis=1))
        u = c @ np.asarray(w["M"], np.float64).T
        xa = st(rmsnorm(u, w["g_a"], eps))
        qkv = (xa @ Wq.T)[0]
        for hh in range(n_heads):
            sl = slice(hh * head_dim, (hh + 1) * head_dim)
            q = rope(qkv[None, None, sl], np.array([j]), theta)[0, 0]
            k = rope(qkv[None, None, A + hh * head_dim: A + (hh + 1) * head_dim], np.array([j]), theta)[0, 0]
            qs[j, sl], ks[j, sl] = st(q), st(k)
        vs[j] = st(qkv[2 * A:])
        us.append(u[0])
    for j in range(n):
        o = np.zeros(A)
        for hh in range(n_heads):
            sl = slice(hh * head_dim, (hh + 1) * head_dim)
            sc = np.array([qs[j, sl] @ ks[s, sl] for s in range(j + 1)]) / np.sqrt(head_dim)
            p = np.exp(sc - sc.max())
            p /= p.sum()
            o[sl] = sum(p[s] * vs[s, sl] for s in range(j + 1))
        o = st(o)
        a = us[j] + o @ np.asarray(w["Wo"], np.float64).T
        y = st(rmsnorm(a[None, :], w["g_f"], eps))
        gsw = st(silu(y @ np.asarray(w["Wgate"], np.float64).T) * (y @ np.asarray(w["Wup"], np.float64).T))
        out[j] = st(a + (gsw @ np.asarray(w["Wdown"], np.float64).T)[0])
    return out, ks, vs


def step_from_cache(h: np.ndarray, tok: int, p: int, k_cache: np.ndarray, v_cache: np.ndarray,
                    w: Dict[str, np.ndarray], E: np.ndarray, W_out: np.ndarray, g_out: np.ndarray,
                    n_heads: int, head_dim: int, eps: float, theta: float, tau: float, u: float,
                    model: Model = EXACT):
    """The step at slot p (0x09A: the module serves from its own cache) with
    the keys and values of slots 0..p-1 given as stored rows (k after RoPE),
    not recomputed from earlier module inputs: the row (h, tok) is normalised
    and projected as in module_rows, its query attends to the given slots and
    to its own key and value, and the block and the head follow.  Returns
    dict(h, logits, token, margin, k, v) with k, v this slot's stored key and
    value rows.  Weights may be passed in float64 to skip the conversions."""
    st = model.store
    A = n_heads * head_dim
    f64 = lambda a: np.asarray(a, np.float64)
    hb = rmsnorm(f64(h)[None, :], w["g_h"], eps)
    eb = rmsnorm(f64(E[int(tok)])[None, :], w["g_e"], eps)
    c = st(np.concatenate([hb, eb], axis=1))
    u_row = (c @ f64(w["M"]).T)[0]
    xa = st(rmsnorm(u_row[None, :], w["g_a"], eps))
    qkv = f64(w["Wqkv"]) @ xa[0]
    q = np.zeros(A)
    k = np.zeros(A)
    for hh in range(n_heads):
        sl = slice(hh * head_dim, (hh + 1) * head_dim)
        q[sl] = st(rope(qkv[None, None, sl], np.array([p]), theta)[0, 0])
        k[sl] = st(rope(qkv[None, None, A + hh * head_dim: A + (hh + 1) * head_dim], np.array([p]), theta)[0, 0])
    v = st(qkv[2 * A:])
    keys = np.concatenate([f64(k_cache[:p]), k[None, :]], axis=0)     # slots 0..p
    vals = np.concatenate([f64(v_cache[:p]), v[None, :]], axis=0)
    o = np.zeros(A)
    for hh in range(n_heads):
        sl = slice(hh * head_dim, (hh + 1) * head_dim)
        sc = keys[:, sl] @ q[sl] / np.sqrt(head_dim)
        pr = np.exp(sc - sc.max())
        pr /= pr.sum()
        o[sl] = pr @ vals[:, sl]
    o = st(o)
    a = u_row + f64(w["Wo"]) @ o
    y = st(rmsnorm(a[None, :], w["g_f"], eps))[0]
    gsw = st(silu(f64(w["Wgate"]) @ y) * (f64(w["Wup"]) @ y))
    h_out = st(a + f64(w["Wdown"]) @ gsw)
    z = head_logits(h_out, W_out, g_out, eps, model)
    p_soft, _ = softmax64(z, tau)
    token, margin = inverse_cdf(p_soft, u)
    return dict(h=h_out, logits=z, token=token, margin=margin, k=k, v=v)


def head_logits(h: np.ndarray, W_out: np.ndarray, g_out: np.ndarray, eps: float, model: Model = EXACT):
    """Stored logits store(W_out store(RMSNorm_{g_out}(h))) of one row."""
    st = model.store
    x = st(rmsnorm(np.asarray(h, np.float64)[None, :], g_out, eps))
    return st((x @ np.asarray(W_out, np.float64).T)[0])


def draw(logits: np.ndarray, u: float, tau: float):
    """(token, status, margin): the inverse CDF of softmax(logits / tau) at u."""
    if not (0.0 <= u < 1.0):
        return -1, BAD_UNIFORM, 0.0
    p, ok = softmax64(logits, tau)
    if not ok:
        return -1, NONFINITE, 0.0
    tok, margin = inverse_cdf(p, u)
    return tok, OK, margin


def propose_step(h_rows: np.ndarray, tok_rows: Sequence[int], w: Dict[str, np.ndarray], E: np.ndarray,
                 W_out: np.ndarray, g_out: np.ndarray, n_heads: int, head_dim: int, eps: float,
                 theta: float, tau: float, u: float, model: Model = EXACT):
    """One request's step at slot p = len(tok_rows) - 1, given the module
    input rows of slots 0..p.  Returns dict(h, logits, token, status,
    margin)."""
    V = E.shape[0]
    if not (0.0 <= u < 1.0):
        return dict(h=None, logits=None, token=-1, status=BAD_UNIFORM, margin=0.0)
    if any(not (0 <= int(t) < V) for t in tok_rows):
        return dict(h=None, logits=None, token=-1, status=BAD_TOKEN, margin=0.0)
    h, _, _ = module_rows(h_rows, tok_rows, w, E, n_heads, head_dim, eps, theta, model)
    z = head_logits(h[-1], W_out, g_out, eps, model)
    tok, status, margin = draw(z, u, tau)
    return dict(h=h[-1], logits=z, token=tok, status=status, margin=margin)


def rollout(h_prefix: np.ndarray, tok_prefix: Sequence[int], h_seed: np.ndarray, f: int, steps: int,
            w, E, W_out, g_out, n_heads, head_dim, eps, theta, tau, us: Sequence[float],
            model: Model = EXACT, tokens: Sequence[int] = None) -> List[dict]:
    """Recurrent rollout of one module (0x09D): slots 0..P-1 hold the
    committed prefix rows (h_prefix, tok_prefix); step 0 at slot P takes the
    parent state h_seed and the incoming token f; step s > 0 takes step s-1's
    output state and drafted token (or ``tokens[s]`` when given, so that two
    implementations can be driven along one token path)."""
    rows_h = [np.asarray(x, np.float64) for x in h_prefix] + [np.asarray(h_seed, np.float64)]
    rows_t = list(tok_prefix) + [int(f)]
    res = []
    for s in range(steps):
        r = propose_step(np.array(rows_h), rows_t, w, E, W_out, g_out, n_heads, head_dim, eps, theta, tau,
                         us[s], model)
        res.append(r)
        if r["status"] != OK:
            break
        nxt = r["token"] if tokens is None else int(tokens[s + 1])
        rows_h.append(r["h"])
        rows_t.append(nxt)
    return res
