"""Pins of the oracle's shared-head CE and its gradients."""
import numpy as np
import pytest
import torch
import torch.nn.functional as F

from oracle import head, rows
from oracle.numerics import EXACT


def _setup(seed, D=2, B=2, T=9, d=6, V=11):
    rng = np.random.default_rng(seed)
    seg = np.zeros((B, T), np.int32)
    seg[0, 6:] = -1
    seg[1, 4:] = 1
    toks = rng.integers(0, V, (B, T))
    _, _, labels, counts = rows.dense_rows(toks, seg, D)
    hs = [rng.standard_normal((B * T, d)) for _ in range(D)]
    W = 0.7 * rng.standard_normal((V, d))
    g = 1.0 + 0.2 * rng.standard_normal(d)
    return hs, labels.reshape(D, -1), counts, W, g


def test_zero_head_gives_log_v():
    hs, labels, counts, W, g = _setup(0)
    V = W.shape[0]
    D = len(hs)
    out = head.head_ce(hs, labels, np.zeros_like(W), g, 1e-6, 0.1)
    np.testing.assert_allclose(out["loss_sum"], counts * np.log(V), rtol=1e-14)
    N = labels.shape[1]
    # dz = c (1/V - onehot), dx_hat = dz W = 0 when W = 0 -> dh = 0, dg = 0
    for k in range(D):
        np.testing.assert_array_equal(out["dh"][k], 0.0)
    np.testing.assert_array_equal(out["dg_out"], 0.0)
    # dW = sum_k c_k sum_rows (1/V - onehot(y)) x_hat
    exp = np.zeros_like(W)
    for k in range(D):
        c = 0.1 / (D * N)
        rws = np.nonzero(labels[k] >= 0)[0]
        xh, _, _ = head.output_norm(hs[k][rws], g, 1e-6)
        dz = np.full((rws.size, V), 1.0 / V)
        dz[np.arange(rws.size), labels[k, rws]] -= 1.0
        exp += c * dz.T @ xh
    np.testing.assert_allclose(out["dW_out"], exp, rtol=1e-12, atol=1e-16)


def test_ce_forward_vs_library():
    hs, labels, counts, W, g = _setup(1)
    out = head.head_ce(hs, labels, W, g, 1e-6, 0.1)
    for k in range(len(hs)):
        rws = np.nonzero(labels[k] >= 0)[0]
        x = F.rms_norm(torch.tensor(hs[k][rws]), (W.shape[1],), torch.tensor(g), 1e-6)
        z = x @ torch.tensor(W).T
        ref = F.cross_entropy(z, torch.tensor(labels[k, rws], dtype=torch.long), reduction="sum").item()
        np.testing.assert_allclose(out["loss_sum"][k], ref, rtol=1e-13)
        np.testing.assert_allclose(out["lse"][k, rws], torch.logsumexp(z, 1).numpy(), rtol=1e-13)


def test_reductions_paper_vs_valid_mean():
    hs, labels, counts, W, g = _setup(2, D=3)
    N = labels.shape[1]
    fixed = head.head_ce(hs, labels, W, g, 1e-6, 0.1, "fixed", grads=False)
    vm = head.head_ce(hs, labels, W, g, 1e-6, 0.1, "valid_mean", grads=False)
    for k in range(3):
        if counts[k]:
            # L_paper = (|V_k| / T) L_valid
            np.testing.assert_allclose(fixed["loss"][k], counts[k] / N * vm["loss"][k], rtol=1e-14)
    # the two reductions differ once counts differ across depths
    assert counts[0] != counts[1]
    assert abs(fixed["loss_mtp"] - vm["loss_mtp"]) > 1e-6
    np.testing.assert_allclose(fixed["loss_mtp"], 0.1 / 3 * fixed["loss"].sum(), rtol=1e-15)


def test_empty_depth_is_zero_term_kept_in_mean():
    hs, labels, counts, W, g = _setup(3, D=2)
    labels = labels.copy()
    labels[1] = -1
    for red in ("fixed", "valid_mean"):
        out = head.head_ce(hs, labels, W, g, 1e-6, 0.1, red)
        assert out["loss"][1] == 0.0 and out["counts"][1] == 0
        np.testing.assert_allclose(out["loss_mtp"], 0.1 / 2 * out["loss"][0])
        np.testing.assert_array_equal(out["dh"][1], 0.0)


@pytest.mark.parametrize("reduce", ["fixed", "valid_mean"])
def test_gradients_by_central_differences(reduce):
    """M7.4 0x04C: summed per-depth gradients must equal a finite-difference
    derivative of the aggregate objective."""
    hs, labels, counts, W, g = _setup(4, D=2, d=5, V=7)
    out = head.head_ce(hs, labels, W, g, 1e-6, 0.1, reduce)
    f = lambda hs_, W_, g_: head.mtp_objective(hs_, labels, W_, g_, 1e-6, 0.1, reduce)
    step = 1e-6
    # h^k
    for k in range(2):
        for (i, j) in [(0, 0), (3, 2), (10, 4), (15, 1), (7, 3)]:
            hp = [h.copy() for h in hs]
            hm = [h.copy() for h in hs]
            hp[k][i, j] += step
            hm[k][i, j] -= step
            fd = (f(hp, W, g) - f(hm, W, g)) / (2 * step)
            assert abs(fd - out["dh"][k][i, j]) < 1e-8, (k, i, j)
    for (v, j) in [(0, 0), (3, 4), (6, 2)]:
        Wp, Wm = W.copy(), W.copy()
        Wp[v, j] += step
        Wm[v, j] -= step
        fd = (f(hs, Wp, g) - f(hs, Wm, g)) / (2 * step)
        assert abs(fd - out["dW_out"][v, j]) < 1e-8
    for j in range(5):
        gp, gm = g.copy(), g.copy()
        gp[j] += step
        gm[j] -= step
        fd = (f(hs, W, gp) - f(hs, W, gm)) / (2 * step)
        assert abs(fd - out["dg_out"][j]) < 1e-8


def test_gradient_invariants():
    hs, labels, counts, W, g = _setup(5, D=2)
    out = head.head_ce(hs, labels, W, g, 1e-6, 0.1)
    # every dz row sums to zero -> the columns of dW_out sum to zero
    np.testing.assert_allclose(out["dW_out"].sum(axis=0), 0.0, atol=1e-15)
    # rows without a label receive no gradient
    for k in range(2):
        no = labels[k] < 0
        np.testing.assert_array_equal(out["dh"][k][no], 0.0)
    # RMSNorm's scale invariance: dh is orthogonal to h on every row (eps -> 0)
    out0 = head.head_ce(hs, labels, W, g, 0.0, 0.1)
    for k in range(2):
        np.testing.assert_allclose((out0["dh"][k] * hs[k]).sum(axis=1), 0.0, atol=1e-15)


def test_gradients_vs_autograd():
    hs, labels, counts, W, g = _setup(6, D=2)
    out = head.head_ce(hs, labels, W, g, 1e-6, 0.1)
    ht = [torch.tensor(h, requires_grad=True) for h in hs]
    Wt = torch.tensor(W, requires_grad=True)
    gt = torch.tensor(g, requires_grad=True)
    N = labels.shape[1]
    total = 0
    for k in range(2):
        rws = np.nonzero(labels[k] >= 0)[0]
        x = F.rms_norm(ht[k][rws], (W.shape[1],), gt, 1e-6)
        total = total + F.cross_entropy(x @ Wt.T, torch.tensor(labels[k, rws], dtype=torch.long), reduction="sum") / N
    (0.1 / 2 * total).backward()
    for k in range(2):
        np.testing.assert_allclose(out["dh"][k], ht[k].grad.numpy(), rtol=1e-11, atol=1e-15)
    np.testing.assert_allclose(out["dW_out"], Wt.grad.numpy(), rtol=1e-11, atol=1e-15)
    np.testing.assert_allclose(out["dg_out"], gt.grad.numpy(), rtol=1e-11, atol=1e-15)


def test_accuracy_parallel_head_rows():
    """W_out[v] = s_v u: z_iv = s_v (x_hat_i . u), so the argmax is the largest
    scale where the projection is positive and the smallest where negative."""
    hs, labels, counts, W, g = _setup(5, D=2, V=13)
    rng = np.random.default_rng(7)
    V, d = W.shape
    u = rng.standard_normal(d)
    s = rng.permutation(V).astype(np.float64) - 4.0
    Wp = s[:, None] * u[None, :]
    out = head.head_ce(hs, labels, Wp, g, 1e-6, 0.1, grads=False)
    for k in range(len(hs)):
        rws = np.nonzero(labels[k] >= 0)[0]
        xh, _, _ = head.output_norm(hs[k][rws], g, 1e-6)
        proj = xh @ u
        exp = np.where(proj > 0, np.argmax(s), np.argmin(s))
        np.testing.assert_array_equal(out["pred"][k, rws], exp)
        assert np.all(out["pred"][k, labels[k] < 0] == -1)
        assert out["correct"][k] == int((exp == labels[k, rws]).sum())
    # labels set to the known argmax: every loss row is correct
    lab2 = labels.copy()
    for k in range(len(hs)):
        rws = np.nonzero(labels[k] >= 0)[0]
        xh, _, _ = head.output_norm(hs[k][rws], g, 1e-6)
        lab2[k, rws] = np.where(xh @ u > 0, np.argmax(s), np.argmin(s))
    out2 = head.head_ce(hs, lab2, Wp, g, 1e-6, 0.1, grads=False)
    np.testing.assert_array_equal(out2["correct"], counts)
    np.testing.assert_array_equal(out2["accuracy"], np.where(counts > 0, 1.0, 0.0))


def test_accuracy_ties_take_the_lowest_id():
    hs, labels, counts, W, g = _setup(6, D=2)
    out = head.head_ce(hs, labels, np.zeros_like(W), g, 1e-6, 0.1, grads=False)
    for k in range(len(hs)):
        rws = labels[k] >= 0
        assert np.all(out["pred"][k, rws] == 0)
        assert out["correct"][k] == int((labels[k, rws] == 0).sum())
    # two equal maxima at ids 3 and 7 on every row: 3 wins
    V, d = W.shape
    W2 = np.full((V, d), 0.0)
    W2[3] = W2[7] = 1.0
    pos = [np.abs(h) + 0.1 for h in hs]        # x_hat . 1 > 0
    out = head.head_ce(pos, labels, W2, np.abs(g), 1e-6, 0.1, grads=False)
    for k in range(len(hs)):
        assert np.all(out["pred"][k, labels[k] >= 0] == 3)


def test_accuracy_brute_force_loops():
    hs, labels, counts, W, g = _setup(8, D=2, T=7, d=4, V=9)
    out = head.head_ce(hs, labels, W, g, 1e-6, 0.1, grads=False)
    D, N = labels.shape
    for k in range(D):
        correct = 0
        for i in range(N):
            if labels[k, i] < 0:
                assert out["pred"][k, i] == -1
                continue
            h = hs[k][i]
            ms = sum(float(x) * float(x) for x in h) / len(h)
            xh = [g[j] * h[j] / np.sqrt(ms + 1e-6) for j in range(len(h))]
            best, arg = None, -1
            for v in range(W.shape[0]):
                zv = sum(xh[j] * W[v, j] for j in range(len(h)))
                if best is None or zv > best:
                    best, arg = zv, v
            assert out["pred"][k, i] == arg
            correct += int(arg == labels[k, i])
        assert out["correct"][k] == correct
        assert out["accuracy"][k] == (correct / counts[k] if counts[k] else 0.0)


def test_accuracy_of_an_empty_depth_is_zero():
    hs, labels, counts, W, g = _setup(9, D=2)
    labels = labels.copy()
    labels[1] = -1
    out = head.head_ce(hs, labels, W, g, 1e-6, 0.1, grads=False)
    assert out["correct"][1] == 0 and out["accuracy"][1] == 0.0
    assert np.all(out["pred"][1] == -1)
    assert 0 <= out["correct"][0] <= out["counts"][0]
