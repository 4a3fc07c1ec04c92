"""Bookkeeping of one carried-frontier speculative round (test infrastructure
only).

Follows M7.6 0x09: the one-proposal selector's outputs -- the new output
tokens, the number of target rows to keep, the pending frontier and the stop
flag -- and its truncation rules: output stops at the available budget and
after an emitted EOS, and an accepted EOS or last-budget proposal gets no
bonus; the target row of the incoming frontier is always kept, a draft's row
only when that draft was accepted; the correction (or the bonus) is carried as
the next pending frontier, never appended to the target state in this round.
Generalised to gamma drafts with the speculative-decoding explainer page's
round: the accepted drafts y_0 .. y_(A-1) come first, then the correction or
bonus token t.

Reading for a verification error (status != 0), for no output slot left
(remaining < 1) and for an accepted count outside [0, gamma] (where the page
raises): the request emits nothing, keeps no row, has no pending frontier and
stops.

Pins (tests/test_oracle_rounds.py): the selector's branches at gamma = 1
written out from the page (accept with bonus, accept at the last budget slot,
accepted EOS, rejection with correction, a correction that is EOS), and
invariants at any gamma (n_new <= remaining, n_new <= A + 1, the emitted
prefix equals the accepted drafts, keep = A + 1).
"""
from __future__ import annotations

from typing import Dict, Sequence


def commit(drafts: Sequence[int], A: int, token: int, status: int, remaining: int, eos: int = -1) -> Dict:
    """One request.  drafts: the gamma draft tokens; A: accepted count;
    token: the correction (A < gamma) or bonus (A == gamma); remaining: new
    output slots available (>= 1); eos: the EOS id, -1 for none."""
    if status != 0 or remaining < 1 or not (0 <= A <= len(drafts)):
        return dict(new_tokens=[], keep=0, pending=-1, stopped=1)
    out = []
    stopped = False
    for y in list(drafts)[:A]:
        out.append(int(y))
        if len(out) == remaining or (eos >= 0 and y == eos):
            stopped = True
            break
    pending = -1
    if not stopped:
        out.append(int(token))
        pending = int(token)
        stopped = len(out) == remaining or (eos >= 0 and token == eos)
    return dict(new_tokens=out, keep=A + 1, pending=pending, stopped=int(stopped))
