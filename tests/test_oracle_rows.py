"""Pins of the oracle's row/label compiler against what the pages print."""
import json
import os

import numpy as np
import pytest

from oracle import rows

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def _load(name):
    with open(os.path.join(GOLD, name)) as f:
        return json.load(f)


def test_af_trace_depth_alignment():
    g = _load("depth_trace_AF.json")
    names = g["tokens"]
    toks = list(range(len(names)))
    seg = g["segment"]
    per_depth = rows.compact_chain_rows(toks, seg, 2)
    for k, key in ((1, "depth_1_labelled_rows"), (2, "depth_2_labelled_rows")):
        got = [(names[r["base"]], names[toks[r["shifted_token_index"]]],
                names[toks[r["label_index"]]]) for r in per_depth[k - 1] if r["loss_valid"]]
        assert got == [tuple(t) for t in g[key]]
    # dense form agrees: label(k, i) = x_(i+k+1)
    _, loss, labels, _ = rows.dense_rows(np.array([toks]), np.array([seg]), 2)
    for k, key in ((1, "depth_1_labelled_rows"), (2, "depth_2_labelled_rows")):
        dense = [(names[i], names[i + k], names[labels[k - 1, 0, i]])
                 for i in range(6) if loss[k - 1, 0, i]]
        assert dense == [tuple(t) for t in g[key]]


def test_two_four_token_segments():
    g = _load("two_segments.json")
    seg = g["segment"]
    toks = list(range(100, 108))
    d1, d2 = rows.compact_chain_rows(toks, seg, 2)
    assert [r["base"] for r in d1] == g["depth_1"]["state_bases"]
    assert [r["base"] for r in d1 if r["loss_valid"]] == g["depth_1"]["supervised_bases"]
    assert [r["base"] for r in d2] == g["depth_2"]["state_bases"]
    assert [r["previous_depth_row"] for r in d2] == g["depth_2"]["previous_physical_rows"]
    assert [r["base"] for r in d2 if r["loss_valid"]] == g["depth_2"]["supervised_bases"]
    state, loss, _, _ = rows.dense_rows(np.array([toks]), np.array([seg]), 2)
    assert list(np.nonzero(state[0, 0])[0]) == g["depth_1"]["state_bases"]
    assert list(np.nonzero(loss[0, 0])[0]) == g["depth_1"]["supervised_bases"]
    assert list(np.nonzero(state[1, 0])[0]) == g["depth_2"]["state_bases"]
    assert list(np.nonzero(loss[1, 0])[0]) == g["depth_2"]["supervised_bases"]


def test_packed_two_row_fixture_counts():
    g = _load("packed_two_row.json")
    toks = np.array(g["tokens"])
    seg = np.array(g["segment"])
    state, loss, labels, counts = rows.dense_rows(toks, seg, 3)
    for k in (1, 2, 3):
        assert int(state[k - 1].sum()) == g["horizon_valid_pairs"][str(k)]
    assert int(state.sum()) == g["horizon_total"]
    # loss rows = sum over segments of max(L - k - 1, 0) for lengths [5], [3, 4]
    lengths = [5, 3, 4]
    for k in (1, 2, 3):
        assert counts[k - 1] == sum(max(L - k - 1, 0) for L in lengths)
    assert list(counts) == [6, 3, 1]
    # labels never cross a packed boundary or read padding
    for k in (1, 2, 3):
        for b in range(2):
            for i in range(7):
                if loss[k - 1, b, i]:
                    j = i + k + 1
                    assert seg[b, j] == seg[b, i] >= 0
                    assert labels[k - 1, b, i] == toks[b, j]
                else:
                    assert labels[k - 1, b, i] == -1
    # the shape-only slice would expose 12/10/8 rows
    for k in (1, 2, 3):
        assert 2 * (7 - k - 1 + 1) == g["shape_only_rows"][str(k)]


def test_label_count_closed_form():
    g = _load("label_counts.json")
    ex = g["example"]
    toks = np.zeros((1, ex["T"]), np.int32)
    seg = np.zeros((1, ex["T"]), np.int32)
    _, _, _, counts = rows.dense_rows(toks, seg, ex["D"])
    assert list(counts) == ex["counts"]
    D, T = ex["D"], ex["T"]
    assert D * (T - 1) - D * (D + 1) // 2 == ex["unrestricted_polynomial"]
    for T in range(2, 12):
        for D in range(1, T):
            toks = np.zeros((1, T), np.int32)
            seg = np.zeros((1, T), np.int32)
            _, _, _, counts = rows.dense_rows(toks, seg, D)
            assert counts.sum() == D * (T - 1) - D * (D + 1) // 2
            assert list(counts) == [max(T - k - 1, 0) for k in range(1, D + 1)]


def test_tiny_config_counts():
    # row 0: one segment of 10 then padding; row 1: segments of 7 and 9
    seg = np.full((2, 16), -1, np.int32)
    seg[0, :10] = 0
    seg[1, :7] = 0
    seg[1, 7:] = 1
    state, loss, _, counts = rows.dense_rows(np.zeros((2, 16), np.int32), seg, 1)
    assert int(state.sum()) == 9 + 6 + 8 == 23
    assert int(counts[0]) == 8 + 5 + 7 == 20


def test_compiler_errors():
    t = [1, 2, 3]
    s = [0, 0, 0]
    v = [True] * 3
    with pytest.raises(ValueError, match="unaligned"):
        rows.compile_mtp_rows(t, s[:2], v, 1, [0, 1, 2])
    with pytest.raises(ValueError, match="positive"):
        rows.compile_mtp_rows(t, s, v, 0, [0, 1, 2])
    with pytest.raises(ValueError, match="invalid previous base"):
        rows.compile_mtp_rows(t, s, v, 1, [0, 1, 3])
    with pytest.raises(ValueError, match="duplicate"):
        rows.compile_mtp_rows(t, s, v, 1, [0, 0, 1])
    with pytest.raises(ValueError, match="predecessor"):
        rows.compile_mtp_rows(t, s, v, 1, [1, 2])


def test_gap_reused_id_is_a_new_occurrence():
    # id 0 reappears after a padding hole: the interval test forbids chains across it
    seg = [0, 0, -1, 0, 0, 0]
    d1 = rows.compact_chain_rows(list(range(6)), seg, 1)[0]
    assert [r["base"] for r in d1] == [0, 3, 4]
    state, loss, _, _ = rows.dense_rows(np.arange(6)[None], np.array([seg]), 1)
    assert list(np.nonzero(state[0, 0])[0]) == [0, 3, 4]
    assert list(np.nonzero(loss[0, 0])[0]) == [3]


@pytest.mark.parametrize("seed", range(20))
def test_dense_equals_compact_random_packings(seed):
    rng = np.random.default_rng(seed)
    B, T, D = 3, int(rng.integers(2, 40)), int(rng.integers(1, 5))
    seg = np.full((B, T), -1, np.int32)
    for b in range(B):
        t, sid = int(rng.integers(0, 3)), 0
        while t < T:
            L = int(rng.integers(1, 9))
            seg[b, t:min(T, t + L)] = sid
            sid += 1
            t += L + int(rng.integers(0, 3))   # optional padding hole
    toks = rng.integers(0, 50, (B, T))
    state, loss, labels, counts = rows.dense_rows(toks, seg, D)
    tot = np.zeros(D, np.int64)
    for b in range(B):
        per_depth = rows.compact_chain_rows(list(toks[b]), list(seg[b]), D)
        for k in range(D):
            assert [r["base"] for r in per_depth[k]] == list(np.nonzero(state[k, b])[0])
            lb = [r["base"] for r in per_depth[k] if r["loss_valid"]]
            assert lb == list(np.nonzero(loss[k, b])[0])
            for r in per_depth[k]:
                if r["loss_valid"]:
                    assert labels[k, b, r["base"]] == toks[b, r["label_index"]]
            tot[k] += len(lb)
    assert list(tot) == list(counts)
    # state at depth k implies state at depth k-1 (the predecessor exists)
    for k in range(1, D):
        assert np.all(state[k] <= state[k - 1])
