"""GPU parity of mtp_horizon_heads (K independent horizon heads, each a
Transformer block followed by the shared head, run head after head) against
oracle.horizons.block_heads (bf16 model): per-head losses (relative 2e-3),
label counts (exact), and the summed trunk gradient, dW_out, dg_out and every
head's block gradients (relative Frobenius error below 1e-2: their entries
are far below the 2e-2 max-abs bar)."""
import numpy as np
import pytest
import torch

from deepseek_sequential_mtp_amd import _lib, synth
from oracle import horizons
from oracle.numerics import BF16
from tests.gpu_util import rel_fro, tdev, to_np

pytestmark = pytest.mark.gpu


def _blocks(inp):
    return [{n: w[n] for n in ("g_a", "Wqkv", "Wo", "g_f", "Wgate", "Wup", "Wdown")} for w in inp["depths"]]


@pytest.mark.parametrize("hd,K,theta", [(128, 2, 10000.0), (64, 3, 10000.0), (128, 2, 0.0)])
def test_horizon_block_heads(hd, K, theta):
    cfg = synth.scaled(synth.D1, name=f"horizon_hd{hd}_K{K}", B=2, T=260, d=256, n_heads=256 // hd, head_dim=hd,
                       ffn=688, V=1000, D=K, seg_lo=20, seg_hi=180, sigma_w=0.05, rope_theta=theta)
    inp = synth.make_chain_inputs(cfg)
    seg = inp["segment_ids"].copy()
    seg[1, 230:] = -1                                   # a padded tail
    inp["segment_ids"] = seg
    blocks = _blocks(inp)
    print(f"[horizon] {cfg.name}: B={cfg.B} T={cfg.T} d={cfg.d} H={cfg.n_heads}x{hd} K={K}", flush=True)
    bt = [{n: tdev(b[n], torch.float32 if n.startswith("g_") else torch.bfloat16) for n in b} for b in blocks]
    res = _lib.horizon_heads(tdev(inp["tokens"].astype(np.int32), torch.int32),
                             tdev(seg.astype(np.int32), torch.int32), tdev(inp["h0"], torch.bfloat16), bt,
                             tdev(inp["W_out"], torch.bfloat16), tdev(inp["g_out"], torch.float32),
                             n_heads=cfg.n_heads, head_dim=hd, lam=cfg.lam, eps=cfg.eps, rope_theta=theta)
    torch.cuda.synchronize()
    ref = horizons.block_heads(inp["h0"], inp["tokens"], seg, blocks, inp["W_out"], inp["g_out"], cfg.n_heads, hd,
                               cfg.eps, theta, cfg.lam, model=BF16)
    assert int(to_np(res["device_error"])[0]) == 0
    np.testing.assert_array_equal(to_np(res["counts"]), ref["counts"])
    np.testing.assert_allclose(to_np(res["loss"]), ref["loss"], rtol=2e-3)
    np.testing.assert_allclose(float(to_np(res["loss_total"])[0]), ref["loss_mtp"], rtol=2e-3)
    checks = [("dh", to_np(res["dh"]), ref["dh_trunk"]), ("dW_out", to_np(res["dW_out"]), ref["dW_out"]),
              ("dg_out", to_np(res["dg_out"]), ref["dg_out"])]
    for k in range(K):
        for n in _lib.BLOCK_FIELDS:
            checks.append((f"head {k + 1} d{n}", to_np(res["dw"][k][n]), ref["blocks_grad"][k][n]))
    for name, g, r in checks:
        assert np.isfinite(g).all(), name
        rf = rel_fro(g, r)
        print(f"  {name}: relF {rf:.2e}", flush=True)
        assert rf < 1e-2, (name, rf)
    # rows with no label in any horizon and no later row of their run get no gradient
    assert np.all(to_np(res["dh"]).reshape(cfg.B, cfg.T, cfg.d)[1, 230:] == 0.0)
