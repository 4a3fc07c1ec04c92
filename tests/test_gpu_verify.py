"""GPU parity of mtp_verify against the oracle: accepted prefix length,
emitted token and status bit-exact.  A decision whose margin (distance of the
uniform from its threshold) is below 1e-9 would be a floating-point tie; the
fixed seeds are required to produce none, and any would be reported.  Both
sides work in float64 (GPU error ~1e-13), so a margin above 1e-9 fixes the
decision."""
import numpy as np
import pytest
import torch

from deepseek_sequential_mtp_amd import _lib, synth
from oracle import verify as ov
from tests.gpu_util import tdev, to_np

pytestmark = pytest.mark.gpu

TIE = 1e-9


def _inputs(gamma, R, V, seed=0):
    vc = synth.verify_config(gamma, R=R, V=V)
    d = synth.make_verify_logits(vc, seed)
    q = ov.draft_probs(d["zd"])
    y = synth.sample_from_probs(d["draft_rng"], q)
    return vc, d, y


def _gpu(d, y, dtype=torch.bfloat16):
    res = _lib.verify(tdev(d["zt"], dtype), tdev(d["zd"], dtype), tdev(y.astype(np.int32), torch.int32),
                      tdev(d["u_accept"], torch.float32), tdev(d["u_sample"], torch.float32))
    torch.cuda.synchronize()
    return {k: to_np(v) for k, v in res.items() if k != "_keep" and v is not None}


def _compare(d, y, g, req=None):
    R = d["zt"].shape[0]
    req = np.arange(R) if req is None else req
    ties = 0
    for r in req:
        o = ov.verify_request(d["zt"][r], d["zd"][r], y[r], d["u_accept"][r], d["u_sample"][r])
        if min(o["accept_margin"], o["sample_margin"]) < TIE:
            ties += 1
            print(f"  tie at request {r}: margins {o['accept_margin']:.2e} {o['sample_margin']:.2e}")
            continue
        assert (g["status"][r], g["accepted_len"][r], g["next_token"][r]) == \
            (o["status"], o["A"], o["token"]), r
    return ties


@pytest.mark.parametrize("gamma", [1, 2, 3, 4])
def test_verify_small_vocab(gamma):
    vc, d, y = _inputs(gamma, R=128, V=1000)
    print(f"[verify] gamma={gamma} R=128 V=1000", flush=True)
    g = _gpu(d, y)
    assert _compare(d, y, g) == 0
    assert (g["status"] == 0).all()


@pytest.mark.parametrize("gamma", [1, 2, 3, 4])
def test_verify_full_vocab_every_request(gamma):
    # the full launch (R = 256, V = 129280); the oracle checks every request
    vc, d, y = _inputs(gamma, R=256, V=129280)
    print(f"[verify] gamma={gamma} R=256 V=129280", flush=True)
    g = _gpu(d, y)
    assert _compare(d, y, g) == 0
    assert (g["status"] == 0).all()
    assert ((g["accepted_len"] >= 0) & (g["accepted_len"] <= gamma)).all()


@pytest.mark.parametrize("dtype,V", [(torch.bfloat16, 1003), (torch.float32, 997)])
def test_verify_vocab_not_a_chunk_multiple(dtype, V):
    # V not a multiple of a 16-byte chunk (8 bf16 or 4 float32 logits): the
    # rows are read logit by logit
    vc, d, y = _inputs(3, R=64, V=V, seed=5)
    print(f"[verify] gamma=3 R=64 V={V} {dtype}", flush=True)
    g = _gpu(d, y, dtype)
    assert _compare(d, y, g) == 0
    assert (g["status"] == 0).all()


def test_verify_float32_logits_and_statuses():
    R, G, V = 8, 2, 64
    rng = np.random.default_rng(5)
    zt = rng.standard_normal((R, G + 1, V)).astype(np.float32) * 2
    zd = (zt[:, :G] + 0.5 * rng.standard_normal((R, G, V))).astype(np.float32)
    q = ov.draft_probs(zd)
    y = synth.sample_from_probs(rng, q)
    ua = rng.random((R, G), dtype=np.float32)
    us = rng.random((R, G + 1), dtype=np.float32)
    ua[1, 0] = 1.0                         # bad uniform
    y[2, 1] = V                            # bad token id
    zt[3, 0, 7] = np.nan                   # non-finite used row
    zd[4, 0, :] = -np.inf                  # all -inf draft row -> non-finite
    zd[5, 0, y[5, 0]] = -np.inf            # q(y) = 0
    zt[6, 1, :] = np.nan                   # row never reached if position 0 rejects
    ua[6, 0] = 0.999999
    d = dict(zt=zt, zd=zd, u_accept=ua, u_sample=us)
    g = _gpu(d, y, torch.float32)
    assert _compare(d, y, g) == 0
    assert list(g["status"][:6]) == [0, 1, 2, 5, 5, 3]


def test_verify_extreme_logits_and_temperature():
    # float32 logits spread over most of the float range with a temperature of
    # 1e36, so z / temperature lies within +-300 and the log-sum-exp loop's
    # float clamp of the logits (bounded at -FLT_MAX) is exercised at its
    # limits; -inf logits contribute nothing; decisions match the oracle's
    R, G, V = 16, 2, 256
    tau = 1e36
    rng = np.random.default_rng(11)
    zt = (rng.uniform(-1.0, 1.0, (R, G + 1, V)) * 3.0e38).astype(np.float32)
    zd = (zt[:, :G].astype(np.float64) * 0.9 + rng.uniform(-1.0, 1.0, (R, G, V)) * 2.0e37).astype(np.float32)
    zt[:, :, 3] = -np.inf
    zd[:, :, 7] = -np.inf
    q = ov.draft_probs(zd, tau)
    y = synth.sample_from_probs(rng, q)
    ua = rng.random((R, G), dtype=np.float32)
    us = rng.random((R, G + 1), dtype=np.float32)
    res = _lib.verify(tdev(zt, torch.float32), tdev(zd, torch.float32), tdev(y.astype(np.int32), torch.int32),
                      tdev(ua, torch.float32), tdev(us, torch.float32), temperature=tau)
    torch.cuda.synchronize()
    g = {k: to_np(v) for k, v in res.items() if k != "_keep" and v is not None}
    for r in range(R):
        o = ov.verify_request(zt[r], zd[r], y[r], ua[r], us[r], tau)
        if min(o["accept_margin"], o["sample_margin"]) < TIE:
            continue
        assert (g["status"][r], g["accepted_len"][r], g["next_token"][r]) == (o["status"], o["A"], o["token"]), r
    assert (g["status"] == 0).all()


def test_verify_single_token_invariant_on_grid():
    """The explainer page's example through the GPU: y enumerated with weight
    q(y), uniforms on a midpoint grid; emitted-token law = p."""
    p = np.array([0.6, 0.3, 0.1])
    q = np.array([0.4, 0.4, 0.2])
    M = 64
    grid = (np.arange(M) + 0.5) / M
    ys, ua, us = np.meshgrid(np.arange(3), grid, grid, indexing="ij")
    R = ys.size
    zt = np.broadcast_to(np.log(p)[None, None, :], (R, 2, 3)).astype(np.float32)
    zd = np.broadcast_to(np.log(q)[None, None, :], (R, 1, 3)).astype(np.float32)
    d = dict(zt=np.ascontiguousarray(zt), zd=np.ascontiguousarray(zd),
             u_accept=ua.reshape(R, 1).astype(np.float32), u_sample=np.repeat(us.reshape(R, 1), 2, 1).astype(np.float32))
    y = ys.reshape(R, 1).astype(np.int32)
    g = _gpu(d, y, torch.float32)
    emitted = np.where(g["accepted_len"] == 0, g["next_token"], y[:, 0])
    w = q[y[:, 0]] / (M * M)
    freq = np.array([w[emitted == t].sum() for t in range(3)])
    np.testing.assert_allclose(freq, p, atol=2.0 / M)
