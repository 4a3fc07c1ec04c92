"""GPU parity of mtp_propose_step at the size bench.py times: the V3-width
retained module and shared head, R = 64 requests, 2048 cached slots of
random keys and values (drawn on the device with a seeded generator, as the
benchmark does), most requests at slot 2048 and a few at slots 0, 1 and 777.
The GPU runs every request; the oracle (oracle.propose.step_from_cache)
recomputes five of them one by one from the same cache rows.

Checked per sampled request: the output state and the stored logits (bf16
max-abs 2e-2 or one bf16 ulp at the row scale, as the small proposer cases),
the key and value the step writes into its slot (same rule), and the draft
token: exact where the oracle's draw is clear of its CDF steps by more than
the logits' rounding can move them, else bracketing u * mass within that
window.  Every request's status must be 0."""
import numpy as np
import pytest
import torch

from deepseek_sequential_mtp_amd import _lib, synth
from oracle import propose
from oracle.numerics import BF16
from oracle.verify import softmax64
from tests.gpu_util import bf16_ulp, chain_tensors, compare, tdev, to_np

pytestmark = [pytest.mark.gpu, pytest.mark.slow]


def test_propose_step_at_v3_width():
    cfg = synth.V3
    R, prefix = 64, 2048
    L_max = prefix + 64
    A = cfg.n_heads * cfg.head_dim
    tau = 1.0
    print(f"[full-propose] {cfg.name}: R={R} slots={prefix} d={cfg.d} H={cfg.n_heads}x{cfg.head_dim} "
          f"ffn={cfg.ffn} V={cfg.V}: drawing inputs", flush=True)
    inp = synth.make_chain_inputs(cfg)
    t = chain_tensors(inp, torch.bfloat16)
    g = torch.Generator(device="cuda").manual_seed(4321)
    kv = (torch.randn((R, 2, L_max, A), generator=g, device="cuda", dtype=torch.float32) * 0.5).to(torch.bfloat16)
    pos = np.full(R, prefix, np.int32)
    pos[1], pos[2], pos[3] = 0, 1, 777
    toks = inp["tokens"].reshape(-1)[1:R + 1].astype(np.int32)
    us = np.random.default_rng(11).random(R).astype(np.float32)
    sample = [0, 1, 3, 5, R - 1]
    # the cache rows the sampled requests read (slots before their own)
    kc = {r: to_np(kv[r, 0, :pos[r]].float()) for r in sample}
    vc = {r: to_np(kv[r, 1, :pos[r]].float()) for r in sample}
    out = _lib.propose_step(t["h0"][:R].contiguous(), tdev(toks, torch.int32), tdev(pos, torch.int32),
                            tdev(us, torch.float32), kv, t["depths"][0], t["E"], t["W_out"], t["g_out"],
                            n_heads=cfg.n_heads, head_dim=cfg.head_dim, eps=cfg.eps, rope_theta=cfg.rope_theta,
                            temperature=tau)
    torch.cuda.synchronize()
    st = to_np(out["status"])
    assert np.all(st == 0), st
    h_gpu = to_np(out["h_out"].float())
    z_gpu = to_np(out["logits"].float())
    tok_gpu = to_np(out["draft_token"])
    k_new = {r: to_np(kv[r, 0, pos[r]].float()) for r in sample}
    v_new = {r: to_np(kv[r, 1, pos[r]].float()) for r in sample}
    del t, kv, out
    torch.cuda.empty_cache()
    print("[full-propose] oracle on sampled requests", flush=True)
    w64 = {k: np.asarray(v, np.float64) for k, v in inp["depths"][0].items()}
    W_out64 = np.asarray(inp["W_out"], np.float64)
    h0 = inp["h0"]
    for r in sample:
        ref = propose.step_from_cache(h0[r], int(toks[r]), int(pos[r]), kc[r], vc[r], w64, inp["E"], W_out64,
                                      inp["g_out"], cfg.n_heads, cfg.head_dim, cfg.eps, cfg.rope_theta, tau,
                                      float(us[r]), BF16)
        checks = [("h", h_gpu[r], ref["h"]), ("logits", z_gpu[r], ref["logits"]), ("k", k_new[r], ref["k"]),
                  ("v", v_new[r], ref["v"])]
        for name, got, want in checks:
            err, nover, ok = compare(got[None, :], want[None, :], 2e-2, bf16_store=True)
            print(f"  request {r} slot {pos[r]}: {name} max err {err:.3e} ({nover} over 2e-2)", flush=True)
            assert ok, (r, name, err)
        p, finite = softmax64(ref["logits"], tau)
        assert finite
        window = float(np.sum(p * np.expm1(2.0 * bf16_ulp(ref["logits"]) / tau)))
        if ref["margin"] > window:
            assert tok_gpu[r] == ref["token"], (r, tok_gpu[r], ref["token"], ref["margin"])
        else:
            cdf = np.cumsum(p)
            tk = int(tok_gpu[r])
            lo = cdf[tk - 1] if tk > 0 else 0.0
            assert lo - window <= us[r] * cdf[-1] <= cdf[tk] + window, r
        print(f"  request {r}: token {tok_gpu[r]} (oracle {ref['token']}, margin {ref['margin']:.2e})", flush=True)
