"""State rows, loss rows and labels of each MTP depth (test infrastructure only).

Follows M7.6 0x02 (depth k reads h^(k-1)_i and x_(i+k) and predicts
x_(i+k+1)), 0x04 (tensor alignment, the final row at each depth has no label)
and 0x04C (compile state support before loss rows; a state needs every
teacher-forced input base..base+k active and in one document occurrence; its
label may be missing; a missing predecessor is an error).

Two forms:

* ``compile_mtp_rows`` -- compact rows of one packed stream (M7.6 0x04C),
  written from the rules stated there (a state needs its whole teacher-forced
  chain inside one document occurrence; a label is optional; a missing
  predecessor is an error) over the end of each position's occurrence;
* ``dense_rows`` -- the same sets on the dense [B, T] layout.  A *run* is a
  maximal stretch of one non-negative segment id inside a batch row; padding
  (id < 0) belongs to no run.  For position i in run [r0, r1]:
  state(k, i) <=> i + k <= r1 and loss(k, i) <=> i + k + 1 <= r1.
  The interval test of 0x04C makes contiguity the meaning of "same document
  occurrence", so an id that reappears after a gap starts a new run.

Pins: the [A..F] trace (M7.6 0x09G), the two four-token segments
(M7.6 0x04C), the two-row packed fixture and its 9/6/3 support counts
(M7.4 0x01A, 0x02C), the label-count closed form D(T-1) - D(D+1)/2 with the
T=2, D=3 -> [0,0,0] case (M7.6 0x05A), and dense == compact by brute force.
"""
from __future__ import annotations

from typing import Dict, List, Sequence, Tuple

import numpy as np


def _occurrence_ends(segment_ids: Sequence[int], valid: Sequence[bool]) -> List[int]:
    """For every position j, the last position of the stretch of available
    inputs that continues j's document occurrence (j itself when the next
    position is unavailable or belongs to another segment); -1 where j is not
    available.  Built by one sweep from the end of the stream."""
    n = len(segment_ids)
    ends = [-1] * n
    for j in range(n - 1, -1, -1):
        if not valid[j]:
            continue
        continues = j + 1 < n and valid[j + 1] and segment_ids[j + 1] == segment_ids[j]
        ends[j] = ends[j + 1] if continues else j
    return ends


def compile_mtp_rows(tokens: Sequence[int], segment_ids: Sequence[int],
                     valid: Sequence[bool], depth: int,
                     previous_bases: Sequence[int]) -> List[Dict[str, object]]:
    """Compact rows of one packed stream at depth ``depth`` (M7.6 0x04C).

    The rules: base b is a state row iff every teacher-forced input b..b+depth
    is available and in b's document occurrence, i.e. b + depth does not pass
    the end of b's occurrence; it carries a loss iff its label position
    b + depth + 1 is inside the occurrence too, else it is kept state-only.
    The row reads the previous depth's output at the physical row whose base
    is b (``previous_bases`` lists the base of every previous-depth row in
    row order); a state row without such a row is an error, as are misaligned
    inputs, a depth below one and invalid or repeated previous bases.
    Rows come out in ascending base order.
    """
    if type(depth) is not int or depth < 1:
        raise ValueError("depth must be positive (an int >= 1)")
    n = len(tokens)
    if len(segment_ids) != n or len(valid) != n:
        raise ValueError("tokens, segment ids and validity flags are unaligned")
    prev_row: Dict[int, int] = {}
    for r, b in enumerate(previous_bases):
        if type(b) is not int or not 0 <= b < n:
            raise ValueError(f"invalid previous base {b!r}")
        if b in prev_row:
            raise ValueError(f"duplicate previous base {b}")
        prev_row[b] = r

    ends = _occurrence_ends(segment_ids, valid)
    out: List[Dict[str, object]] = []
    for b, end in enumerate(ends):
        if end < 0 or b + depth > end:
            continue                      # no complete teacher-forced chain from b
        if b not in prev_row:
            raise ValueError(f"required predecessor state is missing for base {b}")
        has_label = b + depth + 1 <= end
        out.append(dict(base=b, previous_depth_row=prev_row[b],
                        shifted_token_index=b + depth,
                        label_index=b + depth + 1 if has_label else None,
                        loss_valid=has_label, position=b, segment=segment_ids[b]))
    return out


def runs(segment_row: Sequence[int]) -> List[Tuple[int, int]]:
    """Maximal runs [r0, r1] (inclusive) of one non-negative id."""
    seg = list(segment_row)
    out = []
    i, T = 0, len(seg)
    while i < T:
        if seg[i] < 0:
            i += 1
            continue
        j = i
        while j + 1 < T and seg[j + 1] == seg[i]:
            j += 1
        out.append((i, j))
        i = j + 1
    return out


def run_bounds(segment_ids: np.ndarray) -> Tuple[np.ndarray, np.ndarray]:
    """Per position: start and end (inclusive) of its run; a padding position
    is its own one-element window."""
    B, T = segment_ids.shape
    rs = np.arange(T)[None, :].repeat(B, 0).astype(np.int64)
    re = rs.copy()
    for b in range(B):
        for r0, r1 in runs(segment_ids[b]):
            rs[b, r0:r1 + 1] = r0
            re[b, r0:r1 + 1] = r1
    return rs, re


def dense_rows(tokens: np.ndarray, segment_ids: np.ndarray, D: int):
    """Dense masks for depths 1..D on [B, T].

    Returns state_mask, loss_mask (uint8 [D,B,T]), labels (int32 [D,B,T], -1
    where no loss) and counts (int64 [D], loss-valid rows per depth)."""
    if D < 1:
        raise ValueError("depth must be positive")
    tokens = np.asarray(tokens)
    seg = np.asarray(segment_ids)
    B, T = seg.shape
    rs, re = run_bounds(seg)
    active = seg >= 0
    pos = np.arange(T)[None, :]
    state = np.zeros((D, B, T), np.uint8)
    loss = np.zeros((D, B, T), np.uint8)
    labels = np.full((D, B, T), -1, np.int32)
    for k in range(1, D + 1):
        st = active & (pos + k <= re)
        ls = active & (pos + k + 1 <= re)
        state[k - 1] = st
        loss[k - 1] = ls
        for b in range(B):
            for i in np.nonzero(ls[b])[0]:
                labels[k - 1, b, i] = tokens[b, i + k + 1]
    counts = loss.reshape(D, -1).sum(axis=1).astype(np.int64)
    return state, loss, labels, counts


def compact_chain_rows(tokens_row, segment_row, D: int):
    """Run ``compile_mtp_rows`` depth after depth on one packed stream, carrying
    the state bases forward (M7.6 0x06A).  Returns the per-depth row lists."""
    n = len(tokens_row)
    valid = [s >= 0 for s in segment_row]
    bases = list(range(n))
    per_depth = []
    for k in range(1, D + 1):
        rows_k = compile_mtp_rows(list(tokens_row), list(segment_row), valid, k, bases)
        per_depth.append(rows_k)
        bases = [r["base"] for r in rows_k]
    return per_depth
