"""The backward oracle's pins catch plausible mistakes.

Each case plants one mistake into a copy of oracle/backward.py built in
memory (the file itself is untouched): a flipped RoPE rotation sign, the
row term of dS dropped, silu' replaced by the sigmoid, the mean term of the
RMSNorm reverse taken without x_n, the residual gradient dropped, dK taken
without its transpose, and the gradient carried between depths replaced
instead of summed.  The pins of tests/test_oracle_backward.py then run
against the planted copy, and at least one of them must fail.
"""
import inspect
import types

import numpy as np
import pytest

from deepseek_sequential_mtp_amd import synth
from oracle import backward as ob
from tests import test_oracle_backward as tob

PLANTS = {
    "rope sign": ("d2 * cos - d1 * sin", "d2 * cos + d1 * sin"),
    "dS row term": ("ds = p * (dp - np.sum(p * dp, axis=1, keepdims=True))", "ds = p * dp"),
    "silu derivative": ("sig * (1.0 + x * (1.0 - sig))", "sig"),
    "rmsnorm mean term": ("x_n * np.mean(x_n * gdy, axis=1, keepdims=True)", "x_n * np.mean(gdy, axis=1, keepdims=True)"),
    "residual": ("da = np.asarray(dh, np.float64) + da_norm", "da = da_norm"),
    "dK transpose": ("dk[r0:r1 + 1, h] += (ds.T @ Q) * scale", "dk[r0:r1 + 1, h] += (ds @ Q) * scale"),
    "depth carry": ("g = dprev + (np.asarray(dh_head[k - 2], np.float64) if k > 1 else 0.0)",
                    "g = (np.asarray(dh_head[k - 2], np.float64) if k > 1 else dprev)"),
}


def _planted(old, new):
    src = inspect.getsource(ob)
    assert src.count(old) == 1, old
    mod = types.ModuleType("oracle.backward_planted")
    mod.__package__ = "oracle"
    mod.__file__ = ob.__file__
    exec(compile(src.replace(old, new), ob.__file__, "exec"), mod.__dict__)
    return mod


def _pins(setup):
    yield lambda: tob.test_h0_and_embedding_gradients_match_finite_differences(setup)
    for depth in (1, 2):
        for name in ob.PARAMS:
            yield lambda name=name, depth=depth: tob.test_param_gradients_match_finite_differences(setup, name, depth)
    yield lambda: tob.test_exact_zeros_where_no_loss_reaches(setup)
    yield lambda: tob.test_gradient_ledger_by_depth(setup)
    yield tob.test_attention_reverse_matches_finite_differences
    yield tob.test_rmsnorm_and_rope_reverse_match_finite_differences


@pytest.mark.parametrize("plant", sorted(PLANTS))
def test_planted_mistake_fails_a_pin(plant, monkeypatch):
    monkeypatch.setattr(tob, "ob", _planted(*PLANTS[plant]))
    cfg = tob._cfg()
    inp = synth.make_chain_inputs(cfg)
    inp = {k: (np.asarray(v, np.float64) if isinstance(v, np.ndarray) and v.dtype.kind == "f" else v)
           for k, v in inp.items()}
    inp["depths"] = [{n: np.asarray(a, np.float64) for n, a in w.items()} for w in inp["depths"]]
    try:
        setup = (cfg, inp, tob._grads(inp, cfg))
    except (AssertionError, ValueError, FloatingPointError):
        return                                   # the planted copy already breaks
    for pin in _pins(setup):
        try:
            pin()
        except AssertionError:
            return                               # caught
    pytest.fail(f"no pin fails with the planted mistake: {plant}")
