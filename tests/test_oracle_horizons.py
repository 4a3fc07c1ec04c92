"""Pins of the independent-horizon oracle (M7.4 0x02, 0x02A, 0x06A)."""
import json
import os

import numpy as np

from oracle import horizons, rows

GOLD = os.path.join(os.path.dirname(__file__), "golden", "packed_two_row.json")


def test_fixture_horizon_counts():
    g = json.load(open(GOLD))
    tok = np.array(g["tokens"])
    seg = np.array(g["segment"])
    lab = horizons.horizon_labels(np.where(tok < 0, 0, tok), seg, 3)
    counts = (lab >= 0).sum(axis=1)
    assert counts.tolist() == [g["horizon_valid_pairs"][str(k)] for k in (1, 2, 3)]
    # horizon 1 of the first row: the next token inside the 5-token segment
    assert lab[0, :7].tolist() == [12, 13, 14, 15, -1, -1, -1]


def test_horizon_k_plus_1_is_chain_depth_k():
    rng = np.random.default_rng(0)
    for _ in range(20):
        B, T, D = 2, 17, 3
        seg = np.zeros((B, T), np.int32)
        for b in range(B):
            cuts = np.sort(rng.choice(np.arange(1, T), 3, replace=False))
            for i, c in enumerate(cuts):
                seg[b, c:] = i + 1
            seg[b, T - rng.integers(0, 4):] = -1
        tok = rng.integers(0, 50, (B, T))
        _, _, lab_chain, _ = rows.dense_rows(tok, seg, D)
        lab_h = horizons.horizon_labels(tok, seg, D + 1)
        np.testing.assert_array_equal(lab_h[1:], lab_chain.reshape(D, -1))


def test_trunk_gradient_by_central_differences():
    rng = np.random.default_rng(3)
    B, T, d, V, K = 2, 9, 6, 11, 3
    seg = np.zeros((B, T), np.int32)
    seg[0, 6:] = -1
    seg[1, 4:] = 1
    tok = rng.integers(0, V, (B, T))
    h = rng.standard_normal((B * T, d))
    W = 0.7 * rng.standard_normal((V, d))
    g = 1.0 + 0.2 * rng.standard_normal(d)
    out = horizons.independent_heads(h, tok, seg, K, W, g, 1e-6, 0.3)
    f = lambda hh: horizons.independent_heads(hh, tok, seg, K, W, g, 1e-6, 0.3, grads=False)["loss_mtp"]
    num = np.zeros_like(h)
    e = 1e-6
    for i in range(h.shape[0]):
        for j in range(d):
            hp, hm = h.copy(), h.copy()
            hp[i, j] += e
            hm[i, j] -= e
            num[i, j] = (f(hp) - f(hm)) / (2 * e)
    np.testing.assert_allclose(out["dh_trunk"], num, rtol=1e-6, atol=1e-9)
