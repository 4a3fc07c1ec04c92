"""Shared output head, masked cross-entropy and its gradients (test
infrastructure only).

Follows M7.6:

* 0x03 / 0x04B: the shared head is Norm_out followed by W_U (not a bare
  projection): p^(k)_(i+k+1) = softmax(W_U Norm_out(h^(k)_i));
* 0x05: per-depth loss over the valid rows V_k, either with the paper's fixed
  denominator T or as a masked mean over |V_k|; an empty depth contributes a
  zero term that stays in the D-way mean; L_MTP = (lambda / D) sum_k L^(k);
* 0x05A-0x05B: the shared head's gradient sums the depths' contributions,
  accumulated exactly once; the gradient reaching h^(k) through the head.

Returned gradients are those of L_MTP only (the main loss is the caller's).
With x_n = r * h, r = 1 / sqrt(mean(h^2) + eps) and x_hat = g_out * x_n:

  dz     = c_k (softmax(z) - onehot(label))  on loss rows, 0 elsewhere,
           c_k = lambda / (D * denom_k)
  dx_hat = dz W_out
  dW_out = sum_k dz^T x_hat
  dg_out = sum_k sum_rows dx_hat * x_n
  dh     = r (g_out * dx_hat - x_n * mean(x_n * g_out * dx_hat))

(the RMSNorm derivative written out; x_hat's storage rounding is treated as
the identity, as any straight-through store is).

Top-1 accuracy by depth (M7.6 0x0E and M7.4 0x0C list it among the
training metrics without defining it further; read here as the plain
definition): pred_i = argmax_v z_iv on each loss row, the lowest id among
equal maxima; correct_k = #{loss rows with pred_i = label_i};
accuracy_k = correct_k / |V_k|, 0 for an empty depth.

Pins: W_out = 0 gives loss log V per row and dz = c (1/V - onehot); central
finite differences of L_MTP in float64 for h, W_out and g_out (M7.4 0x04C);
each dz row sums to 0 so sum_v dW_out[v, :] = 0; L_paper = (|V_k| / T) L_valid
(M7.6 0x05); accuracy: rows of W_out parallel to one vector put the
argmax at the largest or smallest scale by the sign of the projection,
W_out = 0 ties every logit (pred 0), brute-force loops on a tiny case.
"""
from __future__ import annotations

from typing import List, Sequence

import numpy as np

from .numerics import EXACT, Model
from .chain import rms_inverse


def logsumexp_rows(z: np.ndarray) -> np.ndarray:
    m = z.max(axis=1)
    return m + np.log(np.exp(z - m[:, None]).sum(axis=1))


def output_norm(h: np.ndarray, g_out: np.ndarray, eps: float, model: Model = EXACT):
    """x_hat = store(g_out * h * r) and r = 1/rms, per row."""
    h = np.asarray(h, dtype=np.float64)
    r = rms_inverse(h, eps)
    x_n = h * r[:, None]
    return model.store(np.asarray(g_out, np.float64) * x_n), r, x_n


def row_lse(h_rows: np.ndarray, W_out: np.ndarray, g_out: np.ndarray, eps: float,
            model: Model = EXACT) -> np.ndarray:
    """log-sum-exp of the shared-head logits of the given rows."""
    x_hat, _, _ = output_norm(h_rows, g_out, eps, model)
    return logsumexp_rows(x_hat @ np.asarray(W_out, np.float64).T)


def head_ce(hs: Sequence[np.ndarray], labels: np.ndarray, W_out: np.ndarray,
            g_out: np.ndarray, eps: float, lam: float, reduce: str = "fixed",
            denom: float = None, model: Model = EXACT, grads: bool = True):
    """Shared-head CE over D depths.

    hs: D arrays [N, d]; labels: [D, N] int (-1 = no loss on that row);
    reduce: "fixed" (divide depth k by ``denom``, default N = B*T) or
    "valid_mean" (divide by |V_k|; an empty depth contributes 0)."""
    D = len(hs)
    labels = np.asarray(labels).reshape(D, -1)
    N = labels.shape[1]
    W = np.asarray(W_out, dtype=np.float64)
    V, d = W.shape
    g = np.asarray(g_out, dtype=np.float64)
    if reduce not in ("fixed", "valid_mean"):
        raise ValueError("reduce must be 'fixed' or 'valid_mean'")
    if denom is None:
        denom = float(N)

    loss_sum = np.zeros(D)
    counts = np.zeros(D, dtype=np.int64)
    loss_k = np.zeros(D)
    lse_all = np.full((D, N), np.nan)
    pred = np.full((D, N), -1, dtype=np.int64)
    correct = np.zeros(D, dtype=np.int64)
    accuracy = np.zeros(D)
    dW = np.zeros((V, d))
    dg = np.zeros(d)
    dhs: List[np.ndarray] = []
    for k in range(D):
        rows = np.nonzero(labels[k] >= 0)[0]
        y = labels[k, rows].astype(np.int64)
        counts[k] = rows.size
        dh = np.zeros((N, d))
        if rows.size == 0:
            dhs.append(dh)
            continue
        x_hat, r, x_n = output_norm(np.asarray(hs[k])[rows], g, eps, model)
        z = x_hat @ W.T
        lse = logsumexp_rows(z)
        lse_all[k, rows] = lse
        # np.argmax returns the first index among equal maxima
        pk = np.argmax(z, axis=1)
        pred[k, rows] = pk
        correct[k] = int((pk == y).sum())
        accuracy[k] = correct[k] / rows.size
        ell = lse - z[np.arange(rows.size), y]
        loss_sum[k] = ell.sum()
        den = denom if reduce == "fixed" else float(rows.size)
        loss_k[k] = loss_sum[k] / den
        if grads:
            c = lam / (D * den)
            dz = np.exp(z - lse[:, None])
            dz[np.arange(rows.size), y] -= 1.0
            dz *= c
            dx_hat = dz @ W
            dW += dz.T @ x_hat
            dg += (dx_hat * x_n).sum(axis=0)
            t = x_n * g * dx_hat
            dh[rows] = r[:, None] * (g * dx_hat - x_n * t.mean(axis=1, keepdims=True))
        dhs.append(dh)
    loss_mtp = lam / D * loss_k.sum()
    out = dict(loss_sum=loss_sum, counts=counts, loss=loss_k, loss_mtp=loss_mtp, lse=lse_all,
               pred=pred, correct=correct, accuracy=accuracy)
    if grads:
        out.update(dh=dhs, dW_out=dW, dg_out=dg)
    return out


def mtp_objective(hs, labels, W_out, g_out, eps, lam, reduce="fixed", denom=None):
    """Scalar L_MTP (exact model) -- the function the finite-difference pins
    differentiate."""
    return head_ce(hs, labels, W_out, g_out, eps, lam, reduce, denom, EXACT,
                   grads=False)["loss_mtp"]
