"""Pins of the oracle's module forward: closed forms, special cases, library
routines (torch CPU float64 functional ops) and the literal compact training
loop of M7.6 0x06A by brute force."""
import numpy as np
import pytest
import torch
import torch.nn.functional as F

from oracle import chain, rows
from oracle.numerics import BF16, EXACT, bf16_round


def _rand_weights(rng, d, A_w, f, sigma=0.2):
    g = lambda n: 1.0 + 0.1 * rng.standard_normal(n)
    return dict(g_h=g(d), g_e=g(d), M=sigma * rng.standard_normal((d, 2 * d)), g_a=g(d),
                Wqkv=sigma * rng.standard_normal((3 * A_w, d)),
                Wo=sigma * rng.standard_normal((d, A_w)), g_f=g(d),
                Wgate=sigma * rng.standard_normal((f, d)),
                Wup=sigma * rng.standard_normal((f, d)),
                Wdown=sigma * rng.standard_normal((d, f)))


def test_rmsnorm_closed_forms():
    g = np.array([0.5, 2.0, -1.0, 3.0])
    z = np.full((1, 4), 3.0)
    eps = 1e-6
    np.testing.assert_allclose(chain.rmsnorm(z, g, eps)[0], g * 3.0 / np.sqrt(9.0 + eps), rtol=1e-15)
    rng = np.random.default_rng(0)
    z = rng.standard_normal((5, 16))
    # scale invariance when eps = 0; mean of squares of the normalised row is 1
    np.testing.assert_allclose(chain.rmsnorm(7.5 * z, np.ones(16), 0.0), chain.rmsnorm(z, np.ones(16), 0.0), rtol=1e-13)
    np.testing.assert_allclose((chain.rmsnorm(z, np.ones(16), 0.0) ** 2).mean(axis=1), 1.0, rtol=1e-13)
    # torch's functional rms_norm (library routine)
    gt = rng.standard_normal(16)
    ref = F.rms_norm(torch.tensor(z), (16,), torch.tensor(gt), eps=1e-6).numpy()
    np.testing.assert_allclose(chain.rmsnorm(z, gt, 1e-6), ref, rtol=1e-12, atol=1e-14)


def test_rope_textbook_rotation_and_relativity():
    # head_dim 2: a plain 2-D rotation by pos * theta^0 = pos radians
    x = np.array([[[1.0, 0.0], [0.3, -0.7]]])   # [1 head, L=2, hd=2]
    pos = np.array([0.5, 2.0])
    out = chain.rope(x, pos, 10000.0)
    for t in range(2):
        c, s = np.cos(pos[t]), np.sin(pos[t])
        R = np.array([[c, -s], [s, c]])
        np.testing.assert_allclose(out[0, t], R @ x[0, t], rtol=1e-15, atol=1e-15)
    # the score of a rotated pair depends only on the position difference
    rng = np.random.default_rng(1)
    q = rng.standard_normal((1, 1, 16))
    k = rng.standard_normal((1, 1, 16))
    for p, pp, delta in ((3, 1, 17), (0, 0, 40), (9, 2, 5)):
        s0 = chain.rope(q, np.array([p]), 1e4)[0, 0] @ chain.rope(k, np.array([pp]), 1e4)[0, 0]
        s1 = chain.rope(q, np.array([p + delta]), 1e4)[0, 0] @ chain.rope(k, np.array([pp + delta]), 1e4)[0, 0]
        assert abs(s0 - s1) < 1e-12
    # theta = 0 switches RoPE off
    assert chain.rope(q, np.array([5]), 0.0) is q


def test_segment_causal_attention_vs_library():
    rng = np.random.default_rng(2)
    T, H, hd = 13, 3, 8
    seg = np.array([0, 0, 0, 0, 0, 1, 1, 1, -1, -1, 2, 2, 2])
    q, k, v = (rng.standard_normal((T, H, hd)) for _ in range(3))
    out = chain.segment_causal_attention(q, k, v, seg)
    # library routine with an explicit boolean mask
    rs, _ = rows.run_bounds(seg[None])
    rs = rs[0]
    mask = np.zeros((T, T), bool)
    for i in range(T):
        for j in range(T):
            mask[i, j] = (rs[i] <= j <= i)
    ref = F.scaled_dot_product_attention(
        torch.tensor(q).permute(1, 0, 2), torch.tensor(k).permute(1, 0, 2),
        torch.tensor(v).permute(1, 0, 2), attn_mask=torch.tensor(mask)).permute(1, 0, 2).numpy()
    np.testing.assert_allclose(out, ref, rtol=1e-12, atol=1e-12)
    # padding rows see only themselves; no row reads another segment
    np.testing.assert_allclose(out[8], v[8])
    v2 = v.copy()
    v2[5:8] += 100.0                 # perturb segment 1 only
    out2 = chain.segment_causal_attention(q, k, v2, seg)
    np.testing.assert_allclose(out2[:5], out[:5])
    np.testing.assert_allclose(out2[10:], out[10:])


def test_silu_library():
    from scipy.special import expit
    x = np.linspace(-30, 30, 101)
    np.testing.assert_allclose(chain.silu(x), x * expit(x), rtol=1e-14, atol=1e-300)


def _tiny_setup(seed, B=2, T=12, d=16, H=2, hd=8, f=24, V=40, D=1):
    rng = np.random.default_rng(seed)
    seg = np.full((B, T), -1, np.int32)
    seg[0, :7] = 0
    seg[1, :4] = 0
    seg[1, 4:] = 1
    toks = rng.integers(0, V, (B, T))
    h0 = rng.standard_normal((B * T, d))
    E = 0.5 * rng.standard_normal((V, d))
    depths = [_rand_weights(rng, d, H * hd, f) for _ in range(D)]
    return rng, seg, toks, h0, E, depths


def test_eh_proj_column_order_and_gains():
    rng, seg, toks, h0, E, depths = _tiny_setup(3)
    w = dict(depths[0])
    d = h0.shape[1]
    # M = [I | 0]: u is the normalised hidden path, independent of tokens
    w["M"] = np.concatenate([np.eye(d), np.zeros((d, d))], axis=1)
    _, it = chain.module_forward(h0, toks, seg, 1, w, E, 2, 8, 1e-6, 1e4, EXACT, keep=True)
    np.testing.assert_allclose(it["u"], chain.rmsnorm(h0, w["g_h"], 1e-6), rtol=1e-13)
    _, it2 = chain.module_forward(h0, (toks + 1) % E.shape[0], seg, 1, w, E, 2, 8, 1e-6, 1e4, EXACT, keep=True)
    np.testing.assert_allclose(it2["u"], it["u"])
    # M = [0 | I]: u is the normalised embedding of x_(i+k)
    w["M"] = np.concatenate([np.zeros((d, d)), np.eye(d)], axis=1)
    _, it = chain.module_forward(h0, toks, seg, 1, w, E, 2, 8, 1e-6, 1e4, EXACT, keep=True)
    B, T = seg.shape
    i = np.arange(T)
    shifted = toks[:, np.minimum(i + 1, T - 1)].reshape(-1)
    np.testing.assert_allclose(it["u"], chain.rmsnorm(E[shifted], w["g_e"], 1e-6), rtol=1e-13)


def test_block_residual_wiring():
    rng, seg, toks, h0, E, depths = _tiny_setup(4)
    w = dict(depths[0])
    w["Wo"] = np.zeros_like(w["Wo"])
    w["Wdown"] = np.zeros_like(w["Wdown"])
    h, it = chain.module_forward(h0, toks, seg, 1, w, E, 2, 8, 1e-6, 1e4, EXACT, keep=True)
    np.testing.assert_allclose(h, it["u"])          # both sub-layers switched off
    w = dict(depths[0])
    w["Wdown"] = np.zeros_like(w["Wdown"])
    h, it = chain.module_forward(h0, toks, seg, 1, w, E, 2, 8, 1e-6, 1e4, EXACT, keep=True)
    np.testing.assert_allclose(h, it["a"])


def _torch_block(h_prev, e, w, pos, mask, H, hd, eps, theta):
    """The same module written with torch CPU float64 library ops."""
    t = lambda a: torch.tensor(np.asarray(a, np.float64))
    d = h_prev.shape[1]
    hb = F.rms_norm(t(h_prev), (d,), t(w["g_h"]), eps)
    eb = F.rms_norm(t(e), (d,), t(w["g_e"]), eps)
    u = F.linear(torch.cat([hb, eb], 1), t(w["M"]))
    x = F.rms_norm(u, (d,), t(w["g_a"]), eps)
    qkv = F.linear(x, t(w["Wqkv"]))
    A = H * hd
    n = u.shape[0]
    q, k, v = (qkv[:, i * A:(i + 1) * A].reshape(n, H, hd).permute(1, 0, 2) for i in range(3))
    half = hd // 2
    inv = theta ** (-torch.arange(half, dtype=torch.float64) * 2 / hd)
    ang = t(pos)[:, None] * inv[None]
    cos = torch.cat([torch.cos(ang)] * 2, -1)
    sin = torch.cat([torch.sin(ang)] * 2, -1)
    rot = lambda z: torch.cat([-z[..., half:], z[..., :half]], -1)
    q = q * cos + rot(q) * sin
    k = k * cos + rot(k) * sin
    o = F.scaled_dot_product_attention(q, k, v, attn_mask=torch.tensor(mask)).permute(1, 0, 2).reshape(n, A)
    a = u + F.linear(o, t(w["Wo"]))
    y = F.rms_norm(a, (d,), t(w["g_f"]), eps)
    hk = a + F.linear(F.silu(F.linear(y, t(w["Wgate"]))) * F.linear(y, t(w["Wup"])), t(w["Wdown"]))
    return hk.numpy()


def test_module_vs_torch_functional_block():
    rng, seg, toks, h0, E, depths = _tiny_setup(5)
    B, T = seg.shape
    h = chain.module_forward(h0, toks, seg, 1, depths[0], E, 2, 8, 1e-6, 1e4, EXACT)
    rs, re = rows.run_bounds(seg)
    state, _, _, _ = rows.dense_rows(toks, seg, 1)
    for b in range(B):
        i = np.arange(T)
        shifted = toks[b, np.minimum(i + 1, T - 1)]
        mask = (rs[b][None, :] <= i[:, None]) & (i[None, :] <= i[:, None]) & (rs[b][None, :] == rs[b][:, None])
        mask |= np.eye(T, dtype=bool)
        pos = i - rs[b]
        ref = _torch_block(h0[b * T:(b + 1) * T], E[shifted], depths[0], pos, mask, 2, 8, 1e-6, 1e4)
        st = state[0, b].astype(bool)
        np.testing.assert_allclose(h[b * T:(b + 1) * T][st], ref[st], rtol=1e-10, atol=1e-11)


@pytest.mark.parametrize("seed", range(4))
def test_dense_chain_equals_literal_compact_loop(seed):
    """M7.6 0x06A literal loop (compact rows, gathers, positions = packed base)
    versus the dense masked chain, float64, D = 2 and 3."""
    D = 2 + seed % 2
    rng = np.random.default_rng(100 + seed)
    B, T, d, H, hd, f, V = 2, 14, 12, 2, 4, 20, 30
    seg = np.full((B, T), -1, np.int32)
    for b in range(B):
        t, sid = int(rng.integers(0, 2)), 0
        while t < T:
            L = int(rng.integers(2, 8))
            seg[b, t:min(T, t + L)] = sid
            sid += 1
            t += L + int(rng.integers(0, 2))
    toks = rng.integers(0, V, (B, T))
    h0 = rng.standard_normal((B * T, d))
    E = 0.5 * rng.standard_normal((V, d))
    W_out = 0.3 * rng.standard_normal((V, d))
    g_out = 1.0 + 0.1 * rng.standard_normal(d)
    depths = [_rand_weights(rng, d, H * hd, f) for _ in range(D)]
    hs = chain.chain_forward(h0, toks, seg, depths, E, H, hd, 1e-6, 1e4, EXACT)
    state, loss, labels, counts = rows.dense_rows(toks, seg, D)
    from oracle import head
    dense_terms = []
    for b in range(B):
        states, terms, total = chain.compact_training_step(
            list(toks[b]), list(seg[b]), h0[b * T:(b + 1) * T], depths, E, W_out, g_out,
            H, hd, 1e-6, 1e4, 0.1, float(T))
        for k in range(D):
            st_k, bases = states[k]
            assert bases == list(np.nonzero(state[k, b])[0])
            if bases:
                np.testing.assert_allclose(hs[k][b * T + np.array(bases)], st_k, rtol=1e-9, atol=1e-10)
        # per-stream objective equals the dense head CE restricted to this stream
        lab_b = np.full((D, B * T), -1)
        lab_b[:, b * T:(b + 1) * T] = labels[:, b, :]
        out = head.head_ce(hs, lab_b, W_out, g_out, 1e-6, 0.1, "fixed", float(T), EXACT, grads=False)
        np.testing.assert_allclose(out["loss"], terms, rtol=1e-10, atol=1e-14)
        np.testing.assert_allclose(out["loss_mtp"], total, rtol=1e-10, atol=1e-14)


def test_bf16_model_rounds_only_at_declared_points():
    rng, seg, toks, h0, E, depths = _tiny_setup(6)
    h_ex = chain.module_forward(h0, toks, seg, 1, depths[0], E, 2, 8, 1e-6, 1e4, EXACT)
    h_bf, it = chain.module_forward(h0, toks, seg, 1, depths[0], E, 2, 8, 1e-6, 1e4, BF16, keep=True)
    for name in ("c", "x_a", "q", "k", "v", "o", "y", "gsw", "h"):
        np.testing.assert_array_equal(bf16_round(it[name]), it[name])
    st = rows.dense_rows(toks, seg, 1)[0][0].reshape(-1).astype(bool)
    err = np.abs(h_ex[st] - h_bf[st]).max()
    assert 0 < err < 0.1


def test_bf16_round_ties_and_specials():
    x = np.array([1.0, 1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, -2.5, 0.0, np.inf, -np.inf])
    got = bf16_round(x)
    # 1 + 2^-8 is a tie between 1 and 1 + 2^-7: even mantissa (1.0) wins;
    # 1 + 3*2^-8 ties between 1+2^-7 and 1+2^-6 -> 1 + 2^-6 (even)
    np.testing.assert_array_equal(got, [1.0, 1.0, 1.0 + 2 ** -6, -2.5, 0.0, np.inf, -np.inf])
    assert np.isnan(bf16_round(np.array([np.nan])))[0]
    # agrees with torch's bfloat16 conversion (library routine)
    r = np.random.default_rng(0).standard_normal(10000) * 10
    np.testing.assert_array_equal(bf16_round(r), torch.tensor(r, dtype=torch.float32).to(torch.bfloat16).double().numpy())
