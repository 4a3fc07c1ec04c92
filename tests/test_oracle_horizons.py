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


def _block_case(seed=5, K=2):
    from deepseek_sequential_mtp_amd import synth
    cfg = synth.scaled(synth.TINY, D=1, sigma_w=0.2)
    inp = synth.make_chain_inputs(cfg, seed_offset=seed)
    rng = np.random.default_rng(seed)
    d, A, f = cfg.d, cfg.A_w, cfg.ffn
    blocks = []
    for _ in range(K):
        blocks.append(dict(g_a=1 + 0.1 * rng.standard_normal(d), Wqkv=0.2 * rng.standard_normal((3 * A, d)),
                           Wo=0.2 * rng.standard_normal((d, A)), g_f=1 + 0.1 * rng.standard_normal(d),
                           Wgate=0.2 * rng.standard_normal((f, d)), Wup=0.2 * rng.standard_normal((f, d)),
                           Wdown=0.2 * rng.standard_normal((d, f))))
    h = np.asarray(inp["h0"], np.float64)
    W = np.asarray(inp["W_out"], np.float64)
    g = np.asarray(inp["g_out"], np.float64)
    return cfg, inp, blocks, h, W, g


def test_block_heads_gradients_by_central_differences():
    """Every block weight and gain of both heads, the trunk state, W_out and
    g_out against central differences of the summed objective."""
    cfg, inp, blocks, h, W, g = _block_case()
    kw = dict(n_heads=cfg.n_heads, head_dim=cfg.head_dim, eps=cfg.eps, rope_theta=cfg.rope_theta, lam=0.3)
    out = horizons.block_heads(h, inp["tokens"], inp["segment_ids"], blocks, W, g, **kw)
    f = lambda: horizons.block_heads(h, inp["tokens"], inp["segment_ids"], blocks, W, g, grads=False,
                                     **kw)["loss_mtp"]
    rng = np.random.default_rng(9)

    def check(x, gx, n=5):
        flat = np.abs(gx).ravel()
        for j in np.concatenate([np.argsort(flat)[-n:], rng.choice(flat.size, n, replace=False)]):
            idx = np.unravel_index(j, x.shape)
            x0 = x[idx]
            x[idx] = x0 + 1e-5
            lp = f()
            x[idx] = x0 - 1e-5
            lm = f()
            x[idx] = x0
            num = (lp - lm) / 2e-5
            assert abs(num - gx[idx]) <= 1e-6 * abs(num) + 1e-10, (idx, num, gx[idx])

    check(h, out["dh_trunk"])
    check(W, out["dW_out"], 3)
    check(g, out["dg_out"], 3)
    for k in range(len(blocks)):
        for n in horizons.BLOCK_PARAMS:
            assert np.abs(out["blocks_grad"][k][n]).max() > 0, (k, n)
            check(blocks[k][n], out["blocks_grad"][k][n], 3)


def test_block_heads_with_zero_output_projections_are_identity_heads():
    cfg, inp, blocks, h, W, g = _block_case(seed=6, K=3)
    for b in blocks:
        b["Wo"][:] = 0.0
        b["Wdown"][:] = 0.0
    kw = dict(n_heads=cfg.n_heads, head_dim=cfg.head_dim, eps=cfg.eps, rope_theta=cfg.rope_theta, lam=0.3)
    blk = horizons.block_heads(h, inp["tokens"], inp["segment_ids"], blocks, W, g, **kw)
    idn = horizons.independent_heads(h, inp["tokens"], inp["segment_ids"], 3, W, g, cfg.eps, 0.3)
    np.testing.assert_allclose(blk["loss"], idn["loss"], rtol=1e-12)
    np.testing.assert_allclose(blk["dW_out"], idn["dW_out"], rtol=1e-10, atol=1e-16)
    # the trunk gradient passes the residual stream of each block unchanged
    np.testing.assert_allclose(blk["dh_trunk"], idn["dh_trunk"], rtol=1e-10, atol=1e-16)
