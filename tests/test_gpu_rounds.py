"""GPU parity of mtp_round_commit against oracle/rounds.py: bit-exact on
every output of every request (random accepted counts, tokens, verify
statuses, budgets including 0, with and without an EOS id)."""
import numpy as np
import pytest
import torch

from deepseek_sequential_mtp_amd import _lib
from oracle.rounds import commit
from tests.gpu_util import tdev, to_np

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("gamma,eos", [(1, -1), (4, 3), (4, -1), (7, 0)])
def test_round_commit_bitexact(gamma, eos):
    R = 4096
    rng = np.random.default_rng(gamma * 10 + eos + 1)
    drafts = rng.integers(0, 8, (R, gamma)).astype(np.int32)
    A = rng.integers(0, gamma + 1, R).astype(np.int32)
    A[::97] = gamma + 1                                  # impossible counts: treated as errors
    tok = rng.integers(0, 8, R).astype(np.int32)
    st = np.where(rng.random(R) < 0.05, rng.integers(1, 6, R), 0).astype(np.int32)
    rem = rng.integers(0, 7, R).astype(np.int32)
    print(f"[rounds] R={R} gamma={gamma} eos={eos}", flush=True)
    out = _lib.round_commit(tdev(drafts, torch.int32), tdev(A, torch.int32), tdev(tok, torch.int32),
                            tdev(st, torch.int32), tdev(rem, torch.int32), eos=eos)
    torch.cuda.synchronize()
    nt, nn = to_np(out["new_tokens"]), to_np(out["n_new"])
    kp, pf, sp = to_np(out["rows_to_keep"]), to_np(out["pending_frontier"]), to_np(out["stopped"])
    for r in range(R):
        ref = commit(drafts[r].tolist(), int(A[r]), int(tok[r]), int(st[r]), int(rem[r]), eos)
        n = len(ref["new_tokens"])
        assert nn[r] == n and nt[r, :n].tolist() == ref["new_tokens"] and np.all(nt[r, n:] == -1), r
        assert (kp[r], pf[r], sp[r]) == (ref["keep"], ref["pending"], ref["stopped"]), r
