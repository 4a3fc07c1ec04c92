"""GPU parity of the whole-chain gradient (mtp_chain_backward after
mtp_chain_forward and mtp_head_ce_fwd_bwd) at the full workload sizes, in
the launch configuration a training step would use.

The GPU runs every row of the batch; the head's labels are kept on one
window only (the longest D=1 or D=3 segment, or the first 128 positions of
the single V3-width segment) and set to -1 elsewhere.  Every gradient then comes
from the window's losses: under the segment-causal mask a window row depends
on nothing after it, so dh^(0) on the window, and dE and every per-depth
weight and gain gradient in full, equal the oracle's on the window run
standalone (oracle.backward.mtp_gradients, bf16 model, with the batch's fixed
denominator B*T).  Rows outside the window get exactly 0.  Gate: relative
Frobenius error below 1e-2 per tensor."""
import numpy as np
import pytest
import torch

from deepseek_sequential_mtp_amd import _lib, synth
from oracle import backward as ob, horizons, rows as orows
from oracle.numerics import BF16
from tests.gpu_util import chain_tensors, rel_fro, tdev, to_np
from tests.test_gpu_full import _segments

pytestmark = [pytest.mark.gpu, pytest.mark.slow]

NAMES = ("g_h", "g_e", "g_a", "g_f", "M", "Wqkv", "Wo", "Wgate", "Wup", "Wdown")


def _case(cfg, b, s0, s1, keep_end):
    """Window rows [s0, s1) of batch row b; labels kept on rows [s0, keep_end)."""
    print(f"[full-bwd] {cfg.name}: drawing inputs; window row {b} [{s0}, {s1}), labels to {keep_end}", flush=True)
    inp = synth.make_chain_inputs(cfg)
    t = chain_tensors(inp, torch.bfloat16)
    kw = dict(n_heads=cfg.n_heads, head_dim=cfg.head_dim, eps=cfg.eps, rope_theta=cfg.rope_theta)
    fw = _lib.chain_forward(t["tokens"], t["segment_ids"], t["h0"], t["E"], t["depths"], **kw)
    labels = fw["labels"].clone()
    keep = torch.zeros_like(labels, dtype=torch.bool)
    keep[:, b, s0:keep_end] = True
    labels[~keep] = -1
    ce = _lib.head_ce_fwd_bwd(fw["h"], labels, t["W_out"], t["g_out"], lam=cfg.lam, eps=cfg.eps)
    bw = _lib.chain_backward(t["tokens"], t["segment_ids"], t["h0"], t["E"], t["depths"], fw["h"], ce["dh"], **kw)
    torch.cuda.synchronize()
    lab_win = to_np(labels)[:, b, s0:s1].reshape(cfg.D, -1)
    dh0 = to_np(bw["dh0"]).reshape(cfg.B, cfg.T, cfg.d)
    dE = to_np(bw["dE"])
    dw = [{n: to_np(g[n]) for n in NAMES} for g in bw["dw"]]
    assert int(to_np(bw["device_error"])[0]) == 0
    del t, fw, ce, bw
    torch.cuda.empty_cache()

    outside = np.ones((cfg.B, cfg.T), dtype=bool)
    outside[b, s0:s1] = False
    assert np.all(dh0[outside] == 0.0)
    L = s1 - s0
    rows = b * cfg.T + np.arange(s0, s1)
    print(f"[full-bwd] {cfg.name}: oracle on {L} rows", flush=True)
    ref = ob.mtp_gradients(inp["h0"][rows], inp["tokens"][b:b + 1, s0:s1], np.zeros((1, L), np.int32),
                           inp["depths"], inp["E"], inp["W_out"], inp["g_out"], cfg.n_heads, cfg.head_dim, cfg.eps,
                           cfg.rope_theta, cfg.lam, denom=float(cfg.B * cfg.T), model=BF16, labels=lab_win)
    rf = rel_fro(dh0[b, s0:s1], ref["dh0"])
    print(f"  dh0 relF {rf:.2e}", flush=True)
    assert rf < 1e-2
    rf = rel_fro(dE, ref["dE"])
    print(f"  dE relF {rf:.2e}", flush=True)
    assert rf < 1e-2
    for k in range(cfg.D):
        for n in NAMES:
            rf = rel_fro(dw[k][n], ref["depths"][k][n])
            print(f"  depth {k + 1} d{n}: relF {rf:.2e}", flush=True)
            assert np.isfinite(dw[k][n]).all() and rf < 1e-2, (k, n, rf)


@pytest.mark.timeout(900)
def test_full_chain_backward_d3_longest_segment():
    cfg = synth.D3
    seg = synth.make_chain_inputs(synth.scaled(cfg, d=8, n_heads=1, head_dim=8, ffn=8, V=cfg.V),
                                  with_head=False)["segment_ids"]
    b, s0, s1 = max(((bb, s, e) for bb in range(cfg.B) for (s, e) in _segments(seg[bb])),
                    key=lambda w: (w[2] - w[1], -w[0]))
    # the whole run: its own labels everywhere (the standalone run has the same ones)
    _case(cfg, b, s0, s1, s1)


@pytest.mark.timeout(900)
def test_full_chain_backward_v3width_prefix():
    cfg = synth.V3
    P = 128
    # window [0, P + D): labels on rows [0, P); every label index i + k + 1 stays inside it
    _case(cfg, 0, 0, P + cfg.D, P)


@pytest.mark.timeout(900)
def test_full_chain_backward_d1_longest_segment():
    cfg = synth.D1
    seg = synth.make_chain_inputs(synth.scaled(cfg, d=8, n_heads=1, head_dim=8, ffn=8, V=cfg.V),
                                  with_head=False)["segment_ids"]
    b, s0, s1 = max(((bb, s, e) for bb in range(cfg.B) for (s, e) in _segments(seg[bb])),
                    key=lambda w: (w[2] - w[1], -w[0]))
    _case(cfg, b, s0, s1, s1)


@pytest.mark.timeout(900)
def test_full_width_horizon_block_heads_window():
    """mtp_horizon_heads at V3 width (d 7168, 128x128 heads, ffn 18432,
    V 129280, T 4096) with K = 2 block heads: one run of W tokens and padding
    elsewhere, so every row goes through the full-size GEMMs while only the
    run has labels.  Padding rows attend to themselves only, so the run's
    losses and every gradient equal the oracle's on the run alone (with the
    batch's denominator B*T); padding rows get exactly 0."""
    K, W = 2, 96
    cfg = synth.scaled(synth.V3, D=K)
    print(f"[full-bwd] horizon heads at V3 width: drawing inputs, run of {W} tokens", flush=True)
    inp = synth.make_chain_inputs(cfg)
    seg = np.full((cfg.B, cfg.T), -1, dtype=inp["segment_ids"].dtype)
    seg[0, :W] = 0
    names = ("g_a", "Wqkv", "Wo", "g_f", "Wgate", "Wup", "Wdown")
    blocks = [{n: w[n] for n in names} for w in inp["depths"]]
    bt = [{n: tdev(b[n], torch.float32 if n.startswith("g_") else torch.bfloat16) for n in b} for b in blocks]
    res = _lib.horizon_heads(tdev(inp["tokens"].astype(np.int32), torch.int32), tdev(seg.astype(np.int32), torch.int32),
                             tdev(inp["h0"], torch.bfloat16), bt, tdev(inp["W_out"], torch.bfloat16),
                             tdev(inp["g_out"], torch.float32), n_heads=cfg.n_heads, head_dim=cfg.head_dim,
                             lam=cfg.lam, eps=cfg.eps, rope_theta=cfg.rope_theta)
    torch.cuda.synchronize()
    got = {"loss": to_np(res["loss"]), "counts": to_np(res["counts"]), "dh": to_np(res["dh"]),
           "dW_out": to_np(res["dW_out"]), "dg_out": to_np(res["dg_out"]),
           "dw": [{n: to_np(res["dw"][k][n]) for n in _lib.BLOCK_FIELDS} for k in range(K)]}
    assert int(to_np(res["device_error"])[0]) == 0
    del res, bt
    torch.cuda.empty_cache()
    assert np.all(got["dh"][W:] == 0.0)
    print(f"[full-bwd] horizon heads: oracle on {W} rows", flush=True)
    ref = horizons.block_heads(inp["h0"][:W], inp["tokens"][:, :W], seg[:, :W], blocks, inp["W_out"], inp["g_out"],
                               cfg.n_heads, cfg.head_dim, cfg.eps, cfg.rope_theta, cfg.lam, model=BF16,
                               denom=float(cfg.B * cfg.T))
    np.testing.assert_array_equal(got["counts"], ref["counts"])
    np.testing.assert_allclose(got["loss"], ref["loss"], rtol=2e-3)
    checks = [("dh", got["dh"][:W], ref["dh_trunk"]), ("dW_out", got["dW_out"], ref["dW_out"]),
              ("dg_out", got["dg_out"], ref["dg_out"])]
    checks += [(f"head {k + 1} d{n}", got["dw"][k][n], ref["blocks_grad"][k][n]) for k in range(K)
               for n in _lib.BLOCK_FIELDS]
    for name, g, r in checks:
        rf = rel_fro(g, r)
        print(f"  {name}: relF {rf:.2e}", flush=True)
        assert np.isfinite(g).all() and rf < 1e-2, (name, rf)
