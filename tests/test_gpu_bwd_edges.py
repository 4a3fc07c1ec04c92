"""Degenerate inputs of the reverse pass and of the block horizon heads on
the GPU: a batch that is all padding, rows of a single token (no state row
at any depth), and a horizon that no position can label.  Where no loss
reaches a tensor its gradient is exactly 0, dE (which the call adds to) is
left as it was, and no error is flagged; the labelled horizons still match
the oracle."""
import numpy as np
import pytest
import torch

from deepseek_sequential_mtp_amd import _lib, synth
from oracle import horizons
from oracle.numerics import BF16
from tests.gpu_util import chain_tensors, rel_fro, tdev, to_np

pytestmark = pytest.mark.gpu


def _cfg(**kw):
    base = dict(name="edge", B=2, T=160, d=128, n_heads=1, head_dim=128, ffn=256, V=512, D=2, seg_lo=10, seg_hi=90,
                sigma_w=0.05)
    base.update(kw)
    return synth.scaled(synth.D1, **base)


def _run_chain(cfg, inp):
    t = chain_tensors(inp, torch.bfloat16)
    kw = dict(n_heads=cfg.n_heads, head_dim=cfg.head_dim, eps=cfg.eps, rope_theta=cfg.rope_theta)
    fw = _lib.chain_forward(t["tokens"], t["segment_ids"], t["h0"], t["E"], t["depths"], **kw)
    ce = _lib.head_ce_fwd_bwd(fw["h"], fw["labels"], t["W_out"], t["g_out"], lam=cfg.lam, eps=cfg.eps)
    g = torch.Generator(device="cuda").manual_seed(5)
    dE0 = torch.randn((cfg.V, cfg.d), generator=g, device="cuda")
    out = dict(dh0=torch.full((cfg.B * cfg.T, cfg.d), 7.0, device="cuda"), dE=dE0.clone(),
               dw=[{n: torch.full(w[n].shape, 7.0, device="cuda") for n in _lib.GRAD_FIELDS} for w in t["depths"]],
               device_error=torch.full((1,), 3, dtype=torch.int32, device="cuda"))
    bw = _lib.chain_backward(t["tokens"], t["segment_ids"], t["h0"], t["E"], t["depths"], fw["h"], ce["dh"], out=out,
                             **kw)
    torch.cuda.synchronize()
    return fw, ce, bw, dE0


def _assert_no_gradient(cfg, fw, ce, bw, dE0):
    assert int(to_np(fw["counts"]).sum()) == 0
    assert int(to_np(ce["counts"]).sum()) == 0
    assert int(to_np(bw["device_error"])[0]) == 0
    assert torch.equal(bw["dh0"], torch.zeros_like(bw["dh0"]))
    assert torch.equal(bw["dE"], dE0)                        # nothing added
    for k in range(cfg.D):
        for n in _lib.GRAD_FIELDS:
            assert torch.equal(bw["dw"][k][n], torch.zeros_like(bw["dw"][k][n])), (k, n)


def test_chain_backward_all_padding():
    cfg = _cfg()
    inp = synth.make_chain_inputs(cfg)
    inp["segment_ids"] = np.full_like(inp["segment_ids"], -1)
    print(f"[bwd-edge] all padding B={cfg.B} T={cfg.T} D={cfg.D}", flush=True)
    _assert_no_gradient(cfg, *_run_chain(cfg, inp))


def test_chain_backward_one_token_rows():
    cfg = _cfg(B=5, T=1, D=3)
    inp = synth.make_chain_inputs(cfg)
    inp["segment_ids"] = np.arange(cfg.B, dtype=inp["segment_ids"].dtype).reshape(cfg.B, 1)
    print(f"[bwd-edge] one-token rows B={cfg.B} T={cfg.T} D={cfg.D}", flush=True)
    _assert_no_gradient(cfg, *_run_chain(cfg, inp))


def test_horizon_heads_with_an_empty_horizon():
    # runs of 1, 2 and 3 tokens: horizon 3 (t + 3 inside t's run) never has a label
    K = 3
    cfg = _cfg(B=2, T=96, D=K)
    inp = synth.make_chain_inputs(cfg)
    lens = np.resize([1, 2, 3, 2, 3, 1, 3], 64)
    seg_row = np.repeat(np.arange(lens.size), lens)[:cfg.T]
    seg = np.stack([seg_row, seg_row[::-1].copy()]).astype(inp["segment_ids"].dtype)
    blocks = [{n: w[n] for n in ("g_a", "Wqkv", "Wo", "g_f", "Wgate", "Wup", "Wdown")} for w in inp["depths"]]
    bt = [{n: tdev(b[n], torch.float32 if n.startswith("g_") else torch.bfloat16) for n in b} for b in blocks]
    print(f"[bwd-edge] horizon heads K={K} on runs of 1-3 tokens", flush=True)
    res = _lib.horizon_heads(tdev(inp["tokens"].astype(np.int32), torch.int32), tdev(seg.astype(np.int32), torch.int32),
                             tdev(inp["h0"], torch.bfloat16), bt, tdev(inp["W_out"], torch.bfloat16),
                             tdev(inp["g_out"], torch.float32), n_heads=cfg.n_heads, head_dim=cfg.head_dim,
                             lam=cfg.lam, eps=cfg.eps, rope_theta=cfg.rope_theta)
    torch.cuda.synchronize()
    ref = horizons.block_heads(inp["h0"], inp["tokens"], seg, blocks, inp["W_out"], inp["g_out"], cfg.n_heads,
                               cfg.head_dim, cfg.eps, cfg.rope_theta, cfg.lam, model=BF16)
    counts = to_np(res["counts"])
    np.testing.assert_array_equal(counts, ref["counts"])
    assert counts[2] == 0 and counts[0] > 0 and counts[1] > 0
    assert float(to_np(res["loss"])[2]) == 0.0
    assert int(to_np(res["device_error"])[0]) == 0
    for n in _lib.BLOCK_FIELDS:                              # no loss reaches head 3's block
        assert np.all(to_np(res["dw"][2][n]) == 0.0), n
    np.testing.assert_allclose(to_np(res["loss"])[:2], ref["loss"][:2], rtol=2e-3)
    for name, g, r in [("dh", to_np(res["dh"]), ref["dh_trunk"]), ("dW_out", to_np(res["dW_out"]), ref["dW_out"])] + \
            [(f"head {k + 1} d{n}", to_np(res["dw"][k][n]), ref["blocks_grad"][k][n]) for k in range(2)
             for n in _lib.BLOCK_FIELDS]:
        rf = rel_fro(g, r)
        print(f"  {name}: relF {rf:.2e}", flush=True)
        assert np.isfinite(g).all() and rf < 1e-2, (name, rf)
