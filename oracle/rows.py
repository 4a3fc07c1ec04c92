"""State rows, loss rows and labels of each MTP depth (test infrastructure only).

Follows M7.6 0x02 (depth k reads h^(k-1)_i and x_(i+k) and predicts
x_(i+k+1)), 0x04 (tensor alignment, the final row at each depth has no label)
and 0x04C (compile state support before loss rows; a state needs every
teacher-forced input base..base+k active and in one document occurrence; its
label may be missing; a missing predecessor is an error).

Two forms:

* ``compile_mtp_rows`` -- the compact packed-stream compiler of M7.6 0x04C,
  written from its stated semantics, with the same error conditions;
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


def compile_mtp_rows(tokens: Sequence[int], segment_ids: Sequence[int],
                     valid: Sequence[bool], depth: int,
                     previous_bases: Sequence[int]) -> List[Dict[str, object]]:
    """Compact row compiler for one packed stream (M7.6 0x04C).

    For each base position (ascending) whose teacher-forced chain
    base..base+depth lies inside the stream, is all valid and all carries the
    base's segment id, emit a state row.  Its label index is base+depth+1 when
    that position exists, is valid and has the same segment id; otherwise the
    row is a state-only row (loss_valid False).  ``previous_bases`` lists the
    base of every row of the previous depth's tensor in physical row order.
    """
    n = len(tokens)
    if len(segment_ids) != n or len(valid) != n:
        raise ValueError("unaligned packed inputs")
    if type(depth) is not int or depth < 1:
        raise ValueError("depth must be positive")
    for b in previous_bases:
        if type(b) is not int or b < 0 or b >= n:
            raise ValueError("invalid previous base")
    if len(set(previous_bases)) != len(previous_bases):
        raise ValueError("duplicate previous base")
    row_of_base = {}
    for r, b in enumerate(previous_bases):
        row_of_base[b] = r

    out: List[Dict[str, object]] = []
    for base in range(n):
        teacher = base + depth
        if teacher >= n:
            continue
        sid = segment_ids[base]
        chain_ok = True
        for j in range(base, teacher + 1):
            if not valid[j] or segment_ids[j] != sid:
                chain_ok = False
                break
        if not chain_ok:
            continue
        if base not in row_of_base:
            raise ValueError("required predecessor state is missing")
        lab = teacher + 1
        has_label = lab < n and bool(valid[lab]) and segment_ids[lab] == sid
        out.append({
            "base": base,
            "previous_depth_row": row_of_base[base],
            "shifted_token_index": teacher,
            "label_index": lab if has_label else None,
            "loss_valid": bool(has_label),
            "position": base,
            "segment": sid,
        })
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
