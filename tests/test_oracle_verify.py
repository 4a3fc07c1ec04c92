"""Pins of the oracle's verify (accept / correct / bonus)."""
import json
import os
from fractions import Fraction

import numpy as np
import pytest

from oracle import verify as ov

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def _gold():
    with open(os.path.join(GOLD, "verify_single_token.json")) as f:
        return json.load(f)


def test_single_token_invariant_exact_rationals():
    g = _gold()
    p = [Fraction(x) for x in g["p"]]
    q = [Fraction(x) for x in g["q"]]
    mn = [min(a, b) for a, b in zip(p, q)]
    assert mn == [Fraction(x) for x in g["min_pq"]]
    assert sum(mn) == Fraction(g["accept_total"])
    res = [max(a - b, 0) for a, b in zip(p, q)]
    assert res == [Fraction(x) for x in g["residual"]]
    norm = [r / sum(res) for r in res]
    assert norm == [Fraction(x) for x in g["residual_normalised"]]
    recon = [m + (1 - sum(mn)) * r for m, r in zip(mn, norm)]
    assert recon == p


def _logits(probs):
    with np.errstate(divide="ignore"):
        return np.log(np.asarray(probs, np.float64))


def test_single_token_emission_frequencies_on_grid():
    """Integrate the oracle's decision over y ~ q and a uniform midpoint grid
    of (u_accept, u_sample): the emitted-token law must be p."""
    g = _gold()
    p = np.array([float(Fraction(x)) for x in g["p"]])
    q = np.array([float(Fraction(x)) for x in g["q"]])
    zt = np.stack([_logits(p), _logits(p)])      # row 1 = bonus distribution
    zd = _logits(q)[None]
    M = 200
    grid = (np.arange(M) + 0.5) / M
    freq = np.zeros(3)
    for y in range(3):
        for ua in grid:
            for us in grid[::4]:
                o = ov.verify_request(zt, zd, np.array([y]), np.array([ua]), np.array([us, us]))
                assert o["status"] == 0
                if o["A"] == 0:
                    freq[o["token"]] += q[y] / (M * len(grid[::4]))
                else:
                    freq[y] += q[y] / (M * len(grid[::4]))
    np.testing.assert_allclose(freq, p, atol=2.0 / M)


def test_exhaustive_two_position_losslessness():
    """gamma = 2, V = 3: the first emitted token follows p_0 and, given that
    the first draft was accepted, the second emitted token follows p_1."""
    rng = np.random.default_rng(7)
    V = 3
    p0, p1, p2 = (rng.dirichlet(np.ones(V)) for _ in range(3))
    q0, q1 = (rng.dirichlet(np.ones(V)) for _ in range(2))
    zt = np.stack([_logits(p0), _logits(p1), _logits(p2)])
    zd = np.stack([_logits(q0), _logits(q1)])
    M = 40
    grid = (np.arange(M) + 0.5) / M
    first = np.zeros(V)
    second = np.zeros(V)
    second_mass = 0.0
    for y0 in range(V):
        for y1 in range(V):
            wy = q0[y0] * q1[y1]
            for ua0 in grid:
                for ua1 in grid:
                    for us in grid[::5]:
                        w = wy / (M * M * len(grid[::5]))
                        o = ov.verify_request(zt, zd, np.array([y0, y1]), np.array([ua0, ua1]),
                                              np.array([us, us, us]))
                        A, tok = o["A"], o["token"]
                        first[tok if A == 0 else y0] += w
                        if A >= 1:
                            second_mass += w
                            second[tok if A == 1 else y1] += w
    np.testing.assert_allclose(first, p0, atol=0.03)
    np.testing.assert_allclose(second / second_mass, p1, atol=0.03)


@pytest.mark.parametrize("gamma,alpha", [(3, 0.7), (1, 0.7), (2, 0.85)])
def test_expected_emitted_tokens_monte_carlo(gamma, alpha):
    """E[N_emit] = (1 - a^(g+1)) / (1 - a); 2.533 at a = 0.7, g = 3 (explainer
    page), 1 + a at g = 1 (M7.6 0x0A).  Positions are built with
    sum_v min(p, q) = a exactly: V = 2, p = [1, 0], q = [a, 1 - a]."""
    g = _gold()
    rng = np.random.default_rng(11 + gamma)
    V = 2
    p = np.array([1.0, 0.0])
    q = np.array([alpha, 1 - alpha])
    zt = np.stack([_logits(p)] * (gamma + 1))
    zd = np.stack([_logits(q)] * gamma)
    n = 40000
    total = 0
    for _ in range(n):
        y = (rng.random(gamma) >= alpha).astype(np.int64)   # y ~ q
        o = ov.verify_request(zt, zd, y, rng.random(gamma), rng.random(gamma + 1))
        total += o["A"] + 1
    mean = total / n
    exp = (1 - alpha ** (gamma + 1)) / (1 - alpha)
    if gamma == 3 and alpha == 0.7:
        assert round(exp, 3) == g["e_n_emit"]["value_printed"]
        # the page's idealised speedup (context only)
        assert round(exp / (1 + 3 * g["ideal_speedup_context"]["draft_step_cost"]), 2) == \
            g["ideal_speedup_context"]["value_printed"]
    if gamma == 1:
        assert abs(exp - (1 + alpha)) < 1e-15
    # std of N_emit is below gamma; 4 sigma
    assert abs(mean - exp) < 4 * gamma / np.sqrt(n)


def test_inverse_cdf_convention():
    w = np.array([0.0, 0.25, 0.0, 0.75])
    assert ov.inverse_cdf(w, 0.0)[0] == 1          # zero-mass token 0 never returned
    assert ov.inverse_cdf(w, 0.2499)[0] == 1
    assert ov.inverse_cdf(w, 0.25)[0] == 3         # strict ">" at the step
    assert ov.inverse_cdf(w, 0.999999)[0] == 3


def test_error_statuses():
    zt = np.zeros((2, 4))
    zd = np.zeros((1, 4))
    base = dict(zt=zt, zd=zd, y=np.array([1]), u_accept=np.array([0.5]), u_sample=np.array([0.1, 0.2]))

    def run(**kw):
        a = dict(base)
        a.update(kw)
        return ov.verify_request(a["zt"], a["zd"], a["y"], a["u_accept"], a["u_sample"])

    assert run()["status"] == ov.OK
    assert run(u_accept=np.array([1.0]))["status"] == ov.BAD_UNIFORM
    assert run(u_sample=np.array([-0.1, 0.2]))["status"] == ov.BAD_UNIFORM
    assert run(y=np.array([4]))["status"] == ov.BAD_TOKEN
    zd2 = zd.copy()
    zd2[0, 1] = -np.inf
    assert run(zd=zd2)["status"] == ov.ZERO_DRAFT_PROB
    zt2 = zt.copy()
    zt2[0, 2] = np.nan
    assert run(zt=zt2)["status"] == ov.NONFINITE
    # p == q everywhere: a rejection is impossible (ratio 1 > u) -> all accepted
    o = run()
    assert o["A"] == 1
    # a row never reached is not checked
    zt3 = zt.copy()
    zt3[1, :] = np.nan
    zd3 = np.log(np.array([[0.1, 0.7, 0.1, 0.1]]))
    zt4 = np.log(np.array([[0.7, 0.1, 0.1, 0.1]] * 2))
    zt4[1] = np.nan
    o = ov.verify_request(zt4, zd3, np.array([1]), np.array([0.9]), np.array([0.5, 0.5]))
    assert o["status"] == ov.OK and o["A"] == 0 and o["token"] == 0


def test_rejection_samples_only_positive_residual():
    p = np.array([0.1, 0.6, 0.1, 0.2])
    q = np.array([0.4, 0.2, 0.3, 0.1])
    zt = np.stack([_logits(p)] * 2)
    zd = _logits(q)[None]
    for us in np.linspace(0.001, 0.999, 50):
        o = ov.verify_request(zt, zd, np.array([0]), np.array([0.9]), np.array([us, 0.0]))
        assert o["A"] == 0
        assert o["token"] in (1, 3)       # (p - q)+ = [0, 0.4, 0, 0.1]
