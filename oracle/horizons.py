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

Reading: g_k = identity (0x02 allows it for a head), so every horizon applies
the shared head Norm_out + W_U to the trunk state h itself, with
lambda_k = lambda / K and the fixed denominator B*T -- the chain objective's
scaling with D = K.  Heads that are Transformer blocks need the block
backward and are not modelled.

Pins (tests/test_oracle_horizons.py): the fixture's horizon counts 9 / 6 / 3;
horizon k+1's labels equal the dense chain rows' depth-k labels (a separate
implementation of the run rule); central finite differences of the summed
objective with respect to h equal the summed gradient.
"""
from __future__ import annotations

import numpy as np

from . import head
from .numerics import EXACT, Model
from .rows import run_bounds


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
