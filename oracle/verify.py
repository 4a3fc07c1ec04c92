"""Draft verification: accept / correct / bonus (test infrastructure only).

Follows the one-proposal selector of M7.6 0x09 (accept the drafted y iff
u < min(1, p[y] / q[y]); on rejection draw from the normalised positive part
(p - q)+; on acceptance a bonus from the next target distribution; its input
checks) generalised to gamma drafts by the speculative-decoding explainer
page (test left to right; the first rejection takes a correction from the
normalised residual and drops the rest; if all gamma pass, one extra token is
drawn from the target's next distribution; N_emit = A + 1).

Declared readings: p_j = softmax(zt_j / tau), q_j = softmax(zd_j / tau);
strict "<" with u in [0, 1); one uniform per position: u_accept[j] for the
test at j and u_sample[A] for the emission at slot A; "sample" is the inverse
CDF over ascending token ids with a strict ">": the smallest i with
cumsum(w)[i] > u * sum(w).  EOS and output-budget truncation stay with the
caller.

Arithmetic is float64 with numpy's pairwise sums; the bound on its error
(~1e-15 relative) is far below the GPU's (~1e-6), so a decision whose margin
exceeds the latter is fixed.

Status codes (per request, first failing check wins): 1 a uniform outside
[0, 1) or NaN; 2 a draft token outside [0, V); 5 a used logit row that is
not finite (NaN or +inf, or all -inf); 3 a tested draft token with q = 0;
4 a rejection with zero residual mass.  On error A = 0 and token = -1.

Pins: the single-token invariant min(p,q) + (1 - sum min) norm((p-q)+) = p at
p = [0.6, 0.3, 0.1], q = [0.4, 0.4, 0.2] (explainer page); emitted-token
frequencies reproduce p on exhaustive uniform grids; E[N_emit] =
(1 - a^(g+1)) / (1 - a) by Monte Carlo (2.533 at a = 0.7, g = 3), and 1 + a
at g = 1 (M7.6 0x0A).
"""
from __future__ import annotations

import numpy as np

OK, BAD_UNIFORM, BAD_TOKEN, ZERO_DRAFT_PROB, ZERO_RESIDUAL, NONFINITE = 0, 1, 2, 3, 4, 5


def softmax64(z: np.ndarray, tau: float):
    """Returns (probabilities, ok) of one logit row at temperature tau."""
    s = np.asarray(z, dtype=np.float64) / tau
    if np.isnan(s).any() or np.isposinf(s).any():
        return None, False
    m = s.max()
    if not np.isfinite(m):
        return None, False
    e = np.exp(s - m)
    return e / e.sum(), True


def inverse_cdf(w: np.ndarray, u: float):
    """Smallest i with cumsum(w)[i] > u * sum(w); also the decision margin
    (distance of u * sum(w) to the nearer bracketing CDF step, relative to the
    sum)."""
    cdf = np.cumsum(w)
    total = cdf[-1]
    target = u * total
    i = int(np.searchsorted(cdf, target, side="right"))
    i = min(i, len(w) - 1)
    lo = cdf[i - 1] if i > 0 else 0.0
    margin = min(target - lo, cdf[i] - target) / total
    return i, margin


def verify_request(zt: np.ndarray, zd: np.ndarray, y: np.ndarray, u_accept: np.ndarray,
                   u_sample: np.ndarray, tau: float = 1.0):
    """zt [g+1, V], zd [g, V], y [g], u_accept [g], u_sample [g+1].

    Returns dict(A, token, status, accept_margin, sample_margin)."""
    G = zd.shape[0]
    V = zt.shape[1]
    res = dict(A=0, token=-1, status=OK, accept_margin=np.inf, sample_margin=np.inf)
    u_all = np.concatenate([np.asarray(u_accept, np.float64).ravel(),
                            np.asarray(u_sample, np.float64).ravel()])
    if np.isnan(u_all).any() or (u_all < 0).any() or (u_all >= 1).any():
        res["status"] = BAD_UNIFORM
        return res
    y = np.asarray(y).astype(np.int64)
    if (y < 0).any() or (y >= V).any():
        res["status"] = BAD_TOKEN
        return res
    A = G
    p_at = None
    q_at = None
    for j in range(G):
        p, okp = softmax64(zt[j], tau)
        q, okq = softmax64(zd[j], tau)
        if not (okp and okq):
            res["status"] = NONFINITE
            return res
        if q[y[j]] <= 0:
            res["status"] = ZERO_DRAFT_PROB
            return res
        ratio = p[y[j]] / q[y[j]]
        res["accept_margin"] = min(res["accept_margin"], abs(float(u_accept[j]) - ratio))
        if float(u_accept[j]) < ratio:      # min(1, ratio) is redundant: u < 1
            continue
        A = j
        p_at, q_at = p, q
        break
    if A < G:
        w = np.maximum(p_at - q_at, 0.0)
        if w.sum() <= 0:
            res["status"] = ZERO_RESIDUAL
            return res
        tok, marg = inverse_cdf(w, float(u_sample[A]))
    else:
        p, okp = softmax64(zt[G], tau)
        if not okp:
            res["status"] = NONFINITE
            return res
        tok, marg = inverse_cdf(p, float(u_sample[G]))
    res.update(A=A, token=tok, sample_margin=marg)
    return res


def verify(zt: np.ndarray, zd: np.ndarray, y: np.ndarray, u_accept: np.ndarray,
           u_sample: np.ndarray, tau: float = 1.0):
    """Batched over requests R: zt [R, g+1, V], zd [R, g, V], y [R, g],
    u_accept [R, g], u_sample [R, g+1]."""
    R = zt.shape[0]
    A = np.zeros(R, np.int32)
    tok = np.full(R, -1, np.int32)
    st = np.zeros(R, np.int32)
    am = np.full(R, np.inf)
    sm = np.full(R, np.inf)
    for r in range(R):
        o = verify_request(zt[r], zd[r], y[r], u_accept[r], u_sample[r], tau)
        A[r], tok[r], st[r] = o["A"], o["token"], o["status"]
        am[r], sm[r] = o["accept_margin"], o["sample_margin"]
    return dict(A=A, token=tok, status=st, accept_margin=am, sample_margin=sm)


def draft_probs(zd: np.ndarray, tau: float = 1.0) -> np.ndarray:
    """q for every draft row (used by the harness to sample y ~ q)."""
    s = np.asarray(zd, dtype=np.float64) / tau
    s = s - s.max(axis=-1, keepdims=True)
    e = np.exp(s)
    return e / e.sum(axis=-1, keepdims=True)
