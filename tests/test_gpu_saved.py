"""Saved activations: mtp_chain_forward with a saved-activation buffer keeps
every depth's activations, and mtp_chain_backward reading them instead of
recomputing gives bitwise the same results (the same kernels run on the same
inputs either way).  The forward's own outputs do not change either."""
import numpy as np
import pytest
import torch

from deepseek_sequential_mtp_amd import _lib, synth
from tests.gpu_util import chain_tensors, to_np

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("hd,D,theta", [(128, 2, 10000.0), (64, 3, 0.0)])
def test_saved_activations_give_the_same_bits(hd, D, theta):
    cfg = synth.scaled(synth.D1, name=f"saved_hd{hd}_D{D}", B=2, T=300, d=256, n_heads=256 // hd, head_dim=hd,
                       ffn=688, V=1000, D=D, seg_lo=20, seg_hi=200, sigma_w=0.05, rope_theta=theta)
    inp = synth.make_chain_inputs(cfg)
    seg = inp["segment_ids"].copy()
    seg[1, 260:] = -1
    inp["segment_ids"] = seg
    print(f"[saved] {cfg.name}", flush=True)
    t = chain_tensors(inp, torch.bfloat16)
    kw = dict(n_heads=cfg.n_heads, head_dim=hd, eps=cfg.eps, rope_theta=theta)
    plain = _lib.chain_forward(t["tokens"], t["segment_ids"], t["h0"], t["E"], t["depths"], **kw)
    kept = _lib.chain_forward(t["tokens"], t["segment_ids"], t["h0"], t["E"], t["depths"], save=True, **kw)
    torch.cuda.synchronize()
    for k in range(D):
        assert torch.equal(plain["h"][k], kept["h"][k]), k
    for name in ("state_mask", "loss_mask", "labels", "counts", "device_error"):
        assert torch.equal(plain[name], kept[name]), name
    ce = _lib.head_ce_fwd_bwd(kept["h"], kept["labels"], t["W_out"], t["g_out"], lam=cfg.lam, eps=cfg.eps)
    a = _lib.chain_backward(t["tokens"], t["segment_ids"], t["h0"], t["E"], t["depths"], kept["h"], ce["dh"], **kw)
    b = _lib.chain_backward(t["tokens"], t["segment_ids"], t["h0"], t["E"], t["depths"], kept["h"], ce["dh"],
                            saved=kept["saved"], **kw)
    torch.cuda.synchronize()
    assert int(to_np(b["device_error"])[0]) == 0
    assert torch.equal(a["dh0"], b["dh0"]) and torch.equal(a["dE"], b["dE"])
    assert torch.abs(b["dh0"]).max() > 0
    for k in range(D):
        for n in _lib.GRAD_FIELDS:
            assert torch.equal(a["dw"][k][n], b["dw"][k][n]), (k, n)
