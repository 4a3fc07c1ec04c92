"""The entry points under HIP graph capture.  They launch kernels only
on the caller's stream, allocate nothing and clear their buffers with fill
kernels (no memset nodes), so a captured step replays the same work: each
replay here is compared bit for bit with the eager result, with eager steps
and host synchronisations between the replays.  Every reduction of the path
has a fixed order, so equal inputs give equal bits."""
import numpy as np
import pytest
import torch

from deepseek_sequential_mtp_amd import _lib, synth
from tests.gpu_util import chain_tensors, tdev

pytestmark = pytest.mark.gpu


def _snapshot(chain, ce, ver, prop):
    keys = [chain["labels"], chain["state_mask"], chain["counts"], *chain["h"],
            ce["loss_sum"], ce["loss"], ce["loss_mtp"], *ce["dh"], ce["dW_out"], ce["dg_out"],
            ce["pred"], ce["correct"], ce["accuracy"],
            ver["accepted_len"], ver["next_token"], ver["status"], ver["margin"],
            prop["h_out"], prop["logits"], prop["draft_token"], prop["status"]]
    return [k.clone() for k in keys]


@pytest.mark.parametrize("name,kw", [
    # 128x128 tiles, two depths
    ("graph_small", dict(B=2, T=512, d=512, n_heads=4, head_dim=128, ffn=1408, V=2048, D=2,
                         seg_lo=64, seg_hi=400)),
    # 256x256 tiles with the balanced schedule (1024 CE tiles) and K-split dx
    ("graph_big", dict(B=2, T=1024, d=1024, n_heads=8, head_dim=128, ffn=2816, V=32768, D=1,
                       seg_lo=100, seg_hi=900)),
])
def test_captured_step_replays_bitwise(name, kw):
    cfg = synth.scaled(synth.D1, name=name, **kw)
    print(f"[graph] {name}: {kw}", flush=True)
    t = chain_tensors(synth.make_chain_inputs(cfg), torch.bfloat16)
    vc = synth.verify_config(3, R=32, V=4096)
    vd = synth.make_verify_logits(vc)
    vy = np.random.default_rng(5).integers(0, vc.V, (vc.R, vc.gamma)).astype(np.int32)
    vt = dict(zt=tdev(vd["zt"], torch.bfloat16), zd=tdev(vd["zd"], torch.bfloat16),
              y=tdev(vy, torch.int32), ua=tdev(vd["u_accept"], torch.float32),
              us=tdev(vd["u_sample"], torch.float32))
    # proposer: 8 requests of the chain's first module at slot 40 of a random cache
    R = 8
    A = cfg.n_heads * cfg.head_dim
    gen = torch.Generator(device="cuda").manual_seed(3)
    kv = torch.randn((R, 2, 64, A), generator=gen, device="cuda").to(torch.bfloat16)
    pt = dict(h=t["h0"][:R].contiguous(), tok=t["tokens"].reshape(-1)[:R].clone(),
              pos=torch.full((R,), 40, dtype=torch.int32, device="cuda"),
              u=torch.rand((R,), generator=gen, device="cuda"))
    cache = {}
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        chain = _lib.chain_forward(t["tokens"], t["segment_ids"], t["h0"], t["E"], t["depths"],
                                   n_heads=cfg.n_heads, head_dim=cfg.head_dim, eps=cfg.eps,
                                   rope_theta=cfg.rope_theta, cache=cache)
        ce = _lib.head_ce_fwd_bwd(chain["h"], chain["labels"], t["W_out"], t["g_out"], lam=cfg.lam,
                                  eps=cfg.eps, want_accuracy=True, cache=cache)
        ver = _lib.verify(vt["zt"], vt["zd"], vt["y"], vt["ua"], vt["us"], cache=cache)
        prop = _lib.propose_step(pt["h"], pt["tok"], pt["pos"], pt["u"], kv, t["depths"][0], t["E"], t["W_out"],
                                 t["g_out"], n_heads=cfg.n_heads, head_dim=cfg.head_dim, eps=cfg.eps,
                                 rope_theta=cfg.rope_theta, cache=cache)

        def step():
            _lib.chain_forward(t["tokens"], t["segment_ids"], t["h0"], t["E"], t["depths"],
                               n_heads=cfg.n_heads, head_dim=cfg.head_dim, eps=cfg.eps,
                               rope_theta=cfg.rope_theta, out=chain, cache=cache)
            _lib.head_ce_fwd_bwd(chain["h"], chain["labels"], t["W_out"], t["g_out"], lam=cfg.lam,
                                 eps=cfg.eps, out=ce, cache=cache)
            _lib.verify(vt["zt"], vt["zd"], vt["y"], vt["ua"], vt["us"], out=ver, cache=cache)
            _lib.propose_step(pt["h"], pt["tok"], pt["pos"], pt["u"], kv, t["depths"][0], t["E"], t["W_out"],
                              t["g_out"], n_heads=cfg.n_heads, head_dim=cfg.head_dim, eps=cfg.eps,
                              rope_theta=cfg.rope_theta, out=prop, cache=cache)

        step()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    assert int(chain["device_error"][0]) == 0 and int(ce["device_error"][0]) == 0
    ref = _snapshot(chain, ce, ver, prop)

    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    torch.cuda.synchronize()
    for r in range(4):
        # clobber the outputs, replay, compare; then an eager step in between
        for x in (*chain["h"], *ce["dh"], ce["dW_out"], ce["pred"], ver["next_token"], prop["logits"],
                  prop["draft_token"]):
            x.fill_(-7)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        got = _snapshot(chain, ce, ver, prop)
        for i, (a, b) in enumerate(zip(got, ref)):
            assert torch.equal(a, b), f"replay {r}: output {i} differs"
        print(f"  replay {r}: every output bitwise equal to the eager step", flush=True)
        step()
        torch.cuda.synchronize()
