"""Pins of the round bookkeeping oracle: the one-proposal selector's branches
(M7.6 0x09) written out case by case, and invariants at gamma drafts."""
import numpy as np

from oracle.rounds import commit


def test_one_proposal_branches():
    # accepted y with room for the bonus: [y, b], rows of f and y kept, b pending
    assert commit([7], 1, 9, 0, remaining=5) == dict(new_tokens=[7, 9], keep=2, pending=9, stopped=0)
    # accepted y at the last budget slot: no bonus, nothing pending, stopped
    assert commit([7], 1, 9, 0, remaining=1) == dict(new_tokens=[7], keep=2, pending=-1, stopped=1)
    # accepted EOS: no bonus
    assert commit([2], 1, 9, 0, remaining=5, eos=2) == dict(new_tokens=[2], keep=2, pending=-1, stopped=1)
    # rejection: the correction only, the row of f only, the correction pending
    assert commit([7], 0, 4, 0, remaining=5) == dict(new_tokens=[4], keep=1, pending=4, stopped=0)
    # rejection with one slot left: the correction fills it
    assert commit([7], 0, 4, 0, remaining=1) == dict(new_tokens=[4], keep=1, pending=4, stopped=1)
    # a correction that is EOS stops the request
    assert commit([7], 0, 2, 0, remaining=5, eos=2)["stopped"] == 1
    # bonus EOS: emitted and stops
    assert commit([7], 1, 2, 0, remaining=5, eos=2) == dict(new_tokens=[7, 2], keep=2, pending=2, stopped=1)
    # verification error, no slot left, an impossible A: nothing emitted
    for args in (([7], 0, -1, 3, 5), ([7], 1, 9, 0, 0), ([7], 2, 9, 0, 5), ([7], -1, 9, 0, 5)):
        assert commit(*args) == dict(new_tokens=[], keep=0, pending=-1, stopped=1)


def test_invariants_at_gamma_drafts():
    rng = np.random.default_rng(0)
    for _ in range(2000):
        g = int(rng.integers(1, 6))
        drafts = rng.integers(0, 6, g).tolist()
        A = int(rng.integers(0, g + 1))
        tok = int(rng.integers(0, 6))
        rem = int(rng.integers(1, 8))
        eos = int(rng.integers(-1, 6))
        r = commit(drafts, A, tok, 0, rem, eos)
        out = r["new_tokens"]
        assert 1 <= len(out) <= min(rem, A + 1)
        assert r["keep"] == A + 1
        n_acc = min(len(out), A)
        assert out[:n_acc] == drafts[:n_acc]
        if r["pending"] >= 0:
            assert len(out) == A + 1 and out[-1] == tok == r["pending"]
        # stopped iff the budget is used up or the last emitted token is EOS
        assert r["stopped"] == int(len(out) == rem or (eos >= 0 and out[-1] == eos))
        # nothing after an emitted EOS
        if eos >= 0 and eos in out:
            assert out.index(eos) == len(out) - 1
