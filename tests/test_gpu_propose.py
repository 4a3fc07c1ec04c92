"""GPU parity of mtp_propose_step (one recurrent draft step of a retained
module with its own K/V cache) against oracle/propose.py.

* Prefill by decode: slot by slot from an empty cache, step s of every
  request takes the teacher-forced row (h0_s, x_(s+1)) at position s; its
  output must be the oracle module's row s over slots 0..s.
* Rollout: after the prefix, gamma steps feed back the step's own output
  state; both sides follow one token path (the oracle's draws).
* Statuses per request.

Tolerances: h and the stored logits as the chain (bf16 max-abs 2e-2, one bf16
ulp at the row scale admitted: both sides round nearly equal values at the
same storage points); f32 1e-4.  The draft token is exact where the oracle's
draw is clear of its CDF steps by more than the logits' rounding can move
them; elsewhere the GPU's token must bracket u * mass within that window."""
import numpy as np
import pytest
import torch

from deepseek_sequential_mtp_amd import _lib, synth
from oracle import propose
from oracle.numerics import BF16, EXACT
from oracle.verify import softmax64
from tests.gpu_util import bf16_ulp, chain_tensors, compare, tdev, to_np

pytestmark = pytest.mark.gpu


def _setup(dtype, seed=0, R=3, P=24, L_max=64, hd=128):
    if dtype == "bf16":
        cfg = synth.scaled(synth.D1, name=f"prop_bf16_hd{hd}", B=R, T=P + 8, d=256, n_heads=256 // hd,
                           head_dim=hd, ffn=704, V=1024, D=1, seg_lo=P + 8, seg_hi=P + 8, sigma_w=0.05)
    else:
        cfg = synth.scaled(synth.TINY, name="prop_f32", B=R, T=P + 8, D=1, seg_lo=P + 8, seg_hi=P + 8)
    inp = synth.make_chain_inputs(cfg, seed)
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float32
    t = chain_tensors(inp, tdt)
    A = cfg.n_heads * cfg.head_dim
    cache = torch.zeros((R, 2, L_max, A), dtype=tdt, device="cuda")
    model = BF16 if dtype == "bf16" else EXACT
    return cfg, inp, t, cache, model


def _draw_ok(z_ref, tok, u, tau, window):
    """The GPU's token brackets u * mass on the oracle's CDF within window."""
    p, ok = softmax64(z_ref, tau)
    cdf = np.cumsum(p)
    lo = cdf[tok - 1] if tok > 0 else 0.0
    return ok and lo - window <= u * cdf[-1] <= cdf[tok] + window


def _check_step(cfg, out, ref_h, ref_z, us, tau, model, tag):
    f32 = model is EXACT
    h = to_np(out["h_out"]).astype(np.float64)
    z = to_np(out["logits"]).astype(np.float64)
    tok = to_np(out["draft_token"])
    st = to_np(out["status"])
    assert np.all(st == 0), (tag, st)
    err_h, _, ok_h = compare(h, ref_h, 1e-4 if f32 else 2e-2, bf16_store=not f32)
    err_z, _, ok_z = compare(z, ref_z, 1e-4 if f32 else 2e-2, bf16_store=not f32)
    assert ok_h and ok_z, (tag, err_h, err_z)
    exact = 0
    for r in range(len(tok)):
        p, _ = softmax64(ref_z[r], tau)
        # how far the CDF can move: every stored logit within 1e-5 (f32) or
        # two bf16 ulps (bf16) of the oracle's -- from the oracle's logits only
        dz = np.full(len(p), 1e-5) if f32 else 2.0 * bf16_ulp(ref_z[r])
        window = float(np.sum(p * np.expm1(dz / tau)))
        otok, margin = propose.inverse_cdf(p, float(us[r]))
        if margin > window:
            assert tok[r] == otok, (tag, r, tok[r], otok, margin)
            exact += 1
        else:
            assert _draw_ok(ref_z[r], int(tok[r]), float(us[r]), tau, window), (tag, r)
    return err_h, err_z, exact


@pytest.mark.parametrize("dtype,hd,tau,theta", [("f32", 16, 1.0, None), ("bf16", 128, 1.0, None),
                                              ("bf16", 64, 1.0, None), ("bf16", 32, 1.0, None),
                                              ("f32", 16, 0.7, 0.0), ("bf16", 128, 1.6, 0.0)])
def test_prefill_by_decode_then_rollout(dtype, hd, tau, theta):
    cfg, inp, t, cache, model = _setup(dtype, hd=hd)
    if theta is not None:                 # RoPE off
        cfg = synth.scaled(cfg, rope_theta=theta)
    R, P, G = cfg.B, 24, 3
    w = inp["depths"][0]
    wt = t["depths"][0]
    toks = inp["tokens"]
    h0 = inp["h0"].reshape(R, cfg.T, cfg.d)
    h0_dev = t["h0"].reshape(R, cfg.T, cfg.d)
    rng = np.random.default_rng(7)
    print(f"[propose] {cfg.name} tau={tau} theta={cfg.rope_theta} R={R} P={P} gamma={G} d={cfg.d} H={cfg.n_heads}x{cfg.head_dim} V={cfg.V}",
          flush=True)
    # oracle rows of every request over slots 0..P-1 (teacher-forced inputs)
    ref = [propose.module_rows(h0[r, :P], toks[r, 1:P + 1], w, inp["E"], cfg.n_heads, cfg.head_dim, cfg.eps,
                               cfg.rope_theta, model)[0] for r in range(R)]
    wcache = {}
    worst = [0.0, 0.0]
    for s in range(P):
        us = rng.random(R).astype(np.float32)
        out = _lib.propose_step(h0_dev[:, s].contiguous(), tdev(toks[:, s + 1].astype(np.int32), torch.int32),
                                tdev(np.full(R, s, np.int32), torch.int32), tdev(us, torch.float32), cache, wt,
                                t["E"], t["W_out"], t["g_out"], n_heads=cfg.n_heads, head_dim=cfg.head_dim,
                                eps=cfg.eps, rope_theta=cfg.rope_theta, temperature=tau, cache=wcache)
        torch.cuda.synchronize()
        ref_h = np.stack([ref[r][s] for r in range(R)])
        ref_z = np.stack([propose.head_logits(ref_h[r], inp["W_out"], inp["g_out"], cfg.eps, model)
                          for r in range(R)])
        eh, ez, _ = _check_step(cfg, out, ref_h, ref_z, us, tau, model, f"prefill slot {s}")
        worst = [max(worst[0], eh), max(worst[1], ez)]
    print(f"  prefill: max |h err| {worst[0]:.3e}, max |logit err| {worst[1]:.3e}", flush=True)

    # one launch with the requests at different slots (each rewrites its slot
    # with the same teacher-forced row, so the cache is unchanged)
    sl = np.array([P - 1, 5, 0][:R] + [3] * max(0, R - 3), np.int32)
    us = rng.random(R).astype(np.float32)
    hsel = torch.stack([h0_dev[r, sl[r]] for r in range(R)]).contiguous()
    out = _lib.propose_step(hsel, tdev(np.array([toks[r, sl[r] + 1] for r in range(R)], np.int32), torch.int32),
                            tdev(sl, torch.int32), tdev(us, torch.float32), cache, wt, t["E"], t["W_out"],
                            t["g_out"], n_heads=cfg.n_heads, head_dim=cfg.head_dim, eps=cfg.eps,
                            rope_theta=cfg.rope_theta, temperature=tau, cache=wcache)
    torch.cuda.synchronize()
    ref_h = np.stack([ref[r][sl[r]] for r in range(R)])
    ref_z = np.stack([propose.head_logits(ref_h[r], inp["W_out"], inp["g_out"], cfg.eps, model) for r in range(R)])
    _check_step(cfg, out, ref_h, ref_z, us, tau, model, f"slots {sl.tolist()}")

    # rollout from slot P: seed = (h0_P, x_(P+1)); the oracle's draws set the token path
    us_roll = rng.random((G, R)).astype(np.float32)
    orc = [propose.rollout(h0[r, :P], toks[r, 1:P + 1], h0[r, P], int(toks[r, P + 1]), G, w, inp["E"],
                           inp["W_out"], inp["g_out"], cfg.n_heads, cfg.head_dim, cfg.eps, cfg.rope_theta, tau,
                           us_roll[:, r], model) for r in range(R)]
    h_prev = h0_dev[:, P].contiguous()
    tok_in = toks[:, P + 1].astype(np.int32)
    n_exact = 0
    for g in range(G):
        out = _lib.propose_step(h_prev, tdev(tok_in, torch.int32), tdev(np.full(R, P + g, np.int32), torch.int32),
                                tdev(us_roll[g], torch.float32), cache, wt, t["E"], t["W_out"], t["g_out"],
                                n_heads=cfg.n_heads, head_dim=cfg.head_dim, eps=cfg.eps,
                                rope_theta=cfg.rope_theta, temperature=tau, cache=wcache)
        torch.cuda.synchronize()
        ref_h = np.stack([orc[r][g]["h"] for r in range(R)])
        ref_z = np.stack([orc[r][g]["logits"] for r in range(R)])
        eh, ez, ex = _check_step(cfg, out, ref_h, ref_z, us_roll[g], tau, model, f"rollout step {g}")
        n_exact += ex
        print(f"  rollout step {g}: |h err| {eh:.3e}, |logit err| {ez:.3e}", flush=True)
        h_prev = out["h_out"].clone()
        tok_in = np.array([orc[r][g]["token"] for r in range(R)], np.int32)
    if dtype == "f32":
        assert n_exact >= G * R - 1


def test_statuses_per_request():
    cfg, inp, t, cache, model = _setup("bf16", R=5, P=4, L_max=16)
    R = cfg.B
    wt = t["depths"][0]
    h = t["h0"].reshape(R, cfg.T, cfg.d)[:, 0].contiguous()
    # a recognisable cache: requests rejected before the step must leave it as it is
    cache.copy_(torch.randn(cache.shape, generator=torch.Generator(device=cache.device).manual_seed(5),
                            device=cache.device).to(cache.dtype))
    before = cache.clone()
    toks = np.array([1, cfg.V, 3, 4, -1], np.int32)           # request 1 and 4: bad token
    pos = np.array([0, 0, 16, 0, 0], np.int32)               # request 2: position = L_max
    us = np.array([0.5, 0.5, 0.5, 1.0, 0.5], np.float32)     # request 3: u = 1
    out = _lib.propose_step(h, tdev(toks, torch.int32), tdev(pos, torch.int32), tdev(us, torch.float32), cache,
                            wt, t["E"], t["W_out"], t["g_out"], n_heads=cfg.n_heads, head_dim=cfg.head_dim,
                            eps=cfg.eps, rope_theta=cfg.rope_theta)
    torch.cuda.synchronize()
    st = to_np(out["status"])
    tok = to_np(out["draft_token"])
    np.testing.assert_array_equal(st, [0, 2, 6, 1, 2])
    assert tok[0] >= 0 and np.all(tok[1:] == -1)
    # rejected before the step (bad token, bad position): no slot written, slot 0 included
    for r in (1, 2, 4):
        assert torch.equal(cache[r], before[r]), r
    # accepted requests wrote exactly their own slot
    changed = (cache[0] != before[0]).reshape(2, 16, -1).any(dim=2)
    assert changed[:, 0].all() and not changed[:, 1:].any()
