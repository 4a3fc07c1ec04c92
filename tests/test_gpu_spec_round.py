"""One self-speculative round on the GPU, end to end (M7.6 0x09, 0x09D; the
explainer page's gamma-draft round): a retained module's cache is filled
slot by slot, the module rolls out gamma drafts feeding back its own state
and draws (mtp_propose_step), verification tests them against target logits
(mtp_verify) and the round is committed (mtp_round_commit).  The oracle runs
the same composition from its own values.  f32, so the drafts, decisions and
bookkeeping agree exactly wherever a decision is clear of its threshold by
more than the f32 logits' error (1e-5); a request whose draw or test is
closer than that is reported and left out of the later comparisons."""
import numpy as np
import pytest
import torch

from deepseek_sequential_mtp_amd import _lib, synth
from oracle import propose, rounds, verify as ov
from oracle.numerics import EXACT
from tests.gpu_util import chain_tensors, tdev, to_np

pytestmark = pytest.mark.gpu


def test_self_speculative_round_f32():
    R, P, G, L_max, tau, eos = 6, 10, 3, 32, 1.0, 5
    cfg = synth.scaled(synth.TINY, name="spec_round", B=R, T=P + 8, D=1, seg_lo=P + 8, seg_hi=P + 8)
    inp = synth.make_chain_inputs(cfg, 4)
    t = chain_tensors(inp, torch.float32)
    A_w = cfg.n_heads * cfg.head_dim
    kv = torch.zeros((R, 2, L_max, A_w), dtype=torch.float32, device="cuda")
    w, wt = inp["depths"][0], t["depths"][0]
    toks = inp["tokens"]
    h0 = inp["h0"].reshape(R, cfg.T, cfg.d)
    h0_dev = t["h0"].reshape(R, cfg.T, cfg.d)
    rng = np.random.default_rng(11)
    cache = {}
    kw = dict(n_heads=cfg.n_heads, head_dim=cfg.head_dim, eps=cfg.eps, rope_theta=cfg.rope_theta,
              temperature=tau, cache=cache)
    for s in range(P):                                   # committed prefix
        _lib.propose_step(h0_dev[:, s].contiguous(), tdev(toks[:, s + 1].astype(np.int32), torch.int32),
                          tdev(np.full(R, s, np.int32), torch.int32),
                          tdev(np.full(R, 0.5, np.float32), torch.float32), kv, wt, t["E"], t["W_out"],
                          t["g_out"], **kw)
    us_draft = rng.random((G, R)).astype(np.float32)
    h_prev, tok_in = h0_dev[:, P].contiguous(), toks[:, P + 1].astype(np.int32)
    zd_gpu, y_gpu = [], []
    for g in range(G):                                   # rollout on the GPU's own states and draws
        o = _lib.propose_step(h_prev, tdev(tok_in, torch.int32), tdev(np.full(R, P + g, np.int32), torch.int32),
                              tdev(us_draft[g], torch.float32), kv, wt, t["E"], t["W_out"], t["g_out"], **kw)
        zd_gpu.append(o["logits"].clone())
        y_gpu.append(o["draft_token"].clone())
        h_prev, tok_in = o["h_out"].clone(), to_np(o["draft_token"]).astype(np.int32)
    zd = torch.stack(zd_gpu, dim=1).contiguous()         # [R, G, V]
    y = torch.stack(y_gpu, dim=1).contiguous()           # [R, G]
    zt_np = (2.0 * rng.standard_normal((R, G + 1, cfg.V))).astype(np.float32)
    ua = rng.random((R, G)).astype(np.float32)
    us = rng.random((R, G + 1)).astype(np.float32)
    rem = rng.integers(1, G + 3, R).astype(np.int32)
    ver = _lib.verify(tdev(zt_np, torch.float32), zd, y, tdev(ua, torch.float32), tdev(us, torch.float32),
                      temperature=tau)
    com = _lib.round_commit(y, ver["accepted_len"], ver["next_token"], ver["status"], tdev(rem, torch.int32),
                            eos=eos)
    torch.cuda.synchronize()
    y_g, A_g, tok_g = to_np(y), to_np(ver["accepted_len"]), to_np(ver["next_token"])
    nt, nn = to_np(com["new_tokens"]), to_np(com["n_new"])
    kp, pf, sp = to_np(com["rows_to_keep"]), to_np(com["pending_frontier"]), to_np(com["stopped"])
    compared = 0
    for r in range(R):
        orc = propose.rollout(h0[r, :P], toks[r, 1:P + 1], h0[r, P], int(toks[r, P + 1]), G, w, inp["E"],
                              inp["W_out"], inp["g_out"], cfg.n_heads, cfg.head_dim, cfg.eps, cfg.rope_theta,
                              tau, us_draft[:, r], EXACT)
        if min(x["margin"] for x in orc) < 1e-5:
            print(f"  request {r}: a draft draw within 1e-5 of a CDF step; left out", flush=True)
            continue
        y_o = [x["token"] for x in orc]
        assert y_g[r].tolist() == y_o, r
        zd_o = np.stack([x["logits"] for x in orc])
        vo = ov.verify_request(zt_np[r], zd_o, np.array(y_o), ua[r], us[r], tau)
        if min(vo["accept_margin"], vo["sample_margin"]) < 1e-5:
            print(f"  request {r}: a verify decision within 1e-5 of its threshold; left out", flush=True)
            continue
        assert (A_g[r], tok_g[r]) == (vo["A"], vo["token"]), r
        ref = rounds.commit(y_o, vo["A"], vo["token"], vo["status"], int(rem[r]), eos)
        n = len(ref["new_tokens"])
        assert nn[r] == n and nt[r, :n].tolist() == ref["new_tokens"], r
        assert (kp[r], pf[r], sp[r]) == (ref["keep"], ref["pending"], ref["stopped"]), r
        compared += 1
        print(f"  request {r}: drafts {y_o}, A={vo['A']}, token {vo['token']}, emitted {ref['new_tokens']}",
              flush=True)
    assert compared >= R - 1
