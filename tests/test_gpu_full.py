"""GPU parity at the full workload sizes, in the launch configuration that
bench.py times (256x256 tiles, K splits, the default logit slab).  The oracle
computes sampled outputs one by one:

* chain: the longest whole segment of a batch row (up to 1024 tokens at
  D=1 and 2048 at D=3), and the first 2048 positions of the single
  4096-token V3-width segment, recomputed standalone -- under the
  segment-causal mask a window's state rows depend on nothing after it, so
  the standalone result equals the batch's.  These are the attention windows
  the benchmark times: up to 64 key tiles per query tile, the lazy rescale
  and the fully visible tiles' fast path;
* head CE: the D=1 batch with every loss row labelled; the V3-width and D=3
  batches with labels kept on a sample of rows (the GPU still runs every row
  of the vocabulary GEMMs: the loss, counts, dh and the whole dW_out and
  dg_out then depend on the sampled rows only), and the log-sum-exp of every
  V3-width row (labelled or not) against the oracle's.

Tolerances as in the small cases: h^k by ``tests.gpu_util.compare_h``
(max-abs 2e-2 or one bf16 ulp of the larger magnitude, no element beyond
4e-2, at most 0.2% of a depth's elements over 2e-2 and 0.05% beyond one ulp
and 2e-2 (none at depth 1), relative Frobenius error below
2.5e-3 k); losses and lse relative 2e-3; gradients max-abs 2e-2 and relative
Frobenius 1e-2."""
import numpy as np
import pytest
import torch

from deepseek_sequential_mtp_amd import _lib, synth
from oracle import chain as ochain, head as ohead, rows as orows
from oracle.numerics import BF16
from tests.gpu_util import chain_tensors, compare, compare_h, fmt_h, rel_fro, tdev, to_np

pytestmark = [pytest.mark.gpu, pytest.mark.slow]


def _segments(seg_row):
    """(start, end) of the runs of one batch row (ids >= 0)."""
    out, t, T = [], 0, len(seg_row)
    while t < T:
        if seg_row[t] < 0:
            t += 1
            continue
        s = t
        while t < T and seg_row[t] == seg_row[s]:
            t += 1
        out.append((s, t))
    return out


def _chain_case(cfg, windows):
    """Run the full chain on the GPU; recompute each (b, s0, s1) window with
    the oracle standalone and compare h^k on the window's state rows."""
    print(f"[full-chain] {cfg.name}: drawing inputs", flush=True)
    inp = synth.make_chain_inputs(cfg, with_head=False)
    t = chain_tensors(inp, torch.bfloat16)
    out = _lib.chain_forward(t["tokens"], t["segment_ids"], t["h0"], t["E"], t["depths"],
                             n_heads=cfg.n_heads, head_dim=cfg.head_dim, eps=cfg.eps,
                             rope_theta=cfg.rope_theta)
    torch.cuda.synchronize()
    del t
    st, ls, lab, cnt = orows.dense_rows(inp["tokens"], inp["segment_ids"], cfg.D)
    np.testing.assert_array_equal(to_np(out["state_mask"]), st)
    np.testing.assert_array_equal(to_np(out["loss_mask"]), ls)
    np.testing.assert_array_equal(to_np(out["labels"]), lab)
    np.testing.assert_array_equal(to_np(out["counts"]), cnt)
    assert int(to_np(out["device_error"])[0]) == 0
    hs_gpu = [to_np(h) for h in out["h"]]
    for h in hs_gpu:
        assert np.isfinite(h).all()
    for (b, s0, s1) in windows:
        L = s1 - s0
        rows = b * cfg.T + np.arange(s0, s1)
        print(f"[full-chain] {cfg.name}: oracle on row {b} [{s0}, {s1})", flush=True)
        ref = ochain.chain_forward(inp["h0"][rows], inp["tokens"][b:b + 1, s0:s1],
                                   np.zeros((1, L), np.int32), inp["depths"], inp["E"],
                                   cfg.n_heads, cfg.head_dim, cfg.eps, cfg.rope_theta, BF16)
        for k in range(cfg.D):
            keep = st[k, b, s0:s1].astype(bool)
            # rows of a window cut short of its run end are state rows of the
            # batch but may not be in the standalone window: compare those
            # that are state rows in both
            keep &= np.arange(L) + (k + 1) <= L - 1
            g, r = hs_gpu[k][rows][keep], ref[k][keep]
            stt = compare_h(g, r, k + 1)
            print(f"  depth {k + 1}: rows {keep.sum()}, {fmt_h(stt)}", flush=True)
            assert keep.sum() > 0 and stt["ok"], (k, stt)


@pytest.mark.timeout(900)
def test_full_chain_v3width_long_window():
    cfg = synth.V3
    P = 2048
    # the single 4096-token segment: positions [0, P + D) standalone give
    # rows [0, P) exactly (causal window, shifted tokens up to P - 1 + D);
    # query rows up to 2047 attend over up to 2048 keys (32 key tiles)
    _chain_case(cfg, [(0, 0, P + cfg.D)])


@pytest.mark.timeout(900)
@pytest.mark.parametrize("cfg", [synth.D1, synth.D3], ids=["d1", "d3"])
def test_full_chain_packed_longest_segments(cfg):
    seg = synth.make_chain_inputs(synth.scaled(cfg, d=8, n_heads=1, head_dim=8, ffn=8, V=cfg.V),
                                  with_head=False)["segment_ids"]
    # the longest segment overall and the longest one of another batch row
    cands = [(b, s, e) for b in range(cfg.B) for (s, e) in _segments(seg[b])]
    cands.sort(key=lambda w: (-(w[2] - w[1]), w[0], w[1]))
    wins = [cands[0]] + [w for w in cands if w[0] != cands[0][0]][:1]
    print(f"[full-chain] {cfg.name}: windows {[(b, s, e, e - s) for b, s, e in wins]}", flush=True)
    assert wins[0][2] - wins[0][1] >= (cfg.seg_hi * 3) // 4
    _chain_case(cfg, wins)


def _ce_case(cfg, n_rows, seed=0, lse_all_rows=False):
    """n_rows labelled rows per depth (None: every loss row)."""
    print(f"[full-ce] {cfg.name}: drawing inputs", flush=True)
    inp = synth.make_head_inputs(cfg, seed)
    _, _, labels, _ = orows.dense_rows(inp["tokens"], inp["segment_ids"], cfg.D)
    labels = labels.reshape(cfg.D, -1)
    rng = np.random.default_rng(77 + cfg.index)
    keep = np.zeros_like(labels, dtype=bool)
    for k in range(cfg.D):
        cand = np.nonzero(labels[k] >= 0)[0]
        keep[k, cand if n_rows is None else rng.choice(cand, n_rows, replace=False)] = True
    labels = np.where(keep, labels, -1)
    hs = [tdev(h, torch.bfloat16) for h in inp["h"]]
    W = tdev(inp["W_out"], torch.bfloat16)
    g = tdev(inp["g_out"], torch.float32)
    lab_t = tdev(labels.reshape(cfg.D, cfg.B, cfg.T).astype(np.int32), torch.int32)
    res = _lib.head_ce_fwd_bwd(hs, lab_t, W, g, lam=cfg.lam, eps=cfg.eps, want_lse=True, want_accuracy=True)
    torch.cuda.synchronize()
    del hs, W
    print(f"[full-ce] {cfg.name}: oracle on {n_rows} labelled rows per depth", flush=True)
    ref = ohead.head_ce(inp["h"], labels, inp["W_out"], inp["g_out"], cfg.eps, cfg.lam, "fixed", None, BF16)
    np.testing.assert_array_equal(to_np(res["counts"]), ref["counts"])
    assert int(to_np(res["device_error"])[0]) == 0
    np.testing.assert_allclose(to_np(res["loss_sum"]).astype(np.float64), ref["loss_sum"], rtol=2e-3)
    np.testing.assert_allclose(to_np(res["loss"]), ref["loss"], rtol=2e-3)
    np.testing.assert_allclose(to_np(res["loss_mtp"])[0], ref["loss_mtp"], rtol=2e-3)
    lse = to_np(res["lse"])
    np.testing.assert_allclose(lse[keep], ref["lse"][keep], rtol=2e-3)
    assert np.isfinite(lse).all()
    if lse_all_rows:
        # every row's log-sum-exp, labelled or not, in chunks of rows
        for k in range(cfg.D):
            h = np.asarray(inp["h"][k])
            ref_lse = np.concatenate([ohead.row_lse(h[i:i + 256], inp["W_out"], inp["g_out"], cfg.eps, BF16)
                                      for i in range(0, h.shape[0], 256)])
            rel = np.abs(lse[k] - ref_lse) / np.abs(ref_lse)
            print(f"  lse of all {h.shape[0]} rows of depth {k + 1}: max rel err {rel.max():.2e}", flush=True)
            assert rel.max() < 2e-3
    for k in range(cfg.D):
        dh = to_np(res["dh"][k])
        assert (dh[labels[k] < 0] == 0).all()
        err, _, ok = compare(dh, ref["dh"][k], 2e-2)
        rf = rel_fro(dh, ref["dh"][k])
        print(f"  dh[{k}] max|err| {err:.3e} relF {rf:.2e}", flush=True)
        assert ok and rf < 1e-2
    dW = to_np(res["dW_out"])
    err, _, ok = compare(dW, ref["dW_out"], 2e-2)
    rf = rel_fro(dW, ref["dW_out"])
    print(f"  dW max|err| {err:.3e} relF {rf:.2e}", flush=True)
    assert ok and rf < 1e-2
    dg = to_np(res["dg_out"])
    rf = rel_fro(dg, ref["dg_out"])
    print(f"  dg relF {rf:.2e}", flush=True)
    assert compare(dg, ref["dg_out"], 2e-2)[2] and rf < 1e-2
    # top-1 accuracy by depth: the argmax of every sampled row equals the
    # oracle's, or is a near-tie of the oracle's logits (within 1e-3)
    pred = to_np(res["pred"]).reshape(cfg.D, -1).astype(np.int64)
    correct = to_np(res["correct"]).astype(np.int64)
    for k in range(cfg.D):
        m = labels[k] >= 0
        assert np.all(pred[k, ~m] == -1)
        assert correct[k] == int((pred[k, m] == labels[k, m]).sum())
        diff = np.nonzero(m & (pred[k] != ref["pred"][k]))[0]
        if diff.size:
            xh, _, _ = ohead.output_norm(np.asarray(inp["h"][k])[diff], inp["g_out"], cfg.eps, BF16)
            W64 = np.asarray(inp["W_out"], np.float64)
            gap = (np.einsum("nd,nd->n", xh, W64[ref["pred"][k, diff]]) -
                   np.einsum("nd,nd->n", xh, W64[pred[k, diff]]))
            assert np.all(gap <= 1e-3), gap
        print(f"  accuracy[{k}] {float(to_np(res['accuracy'])[k]):.4f}, {diff.size} near-tie rows", flush=True)


@pytest.mark.timeout(900)
def test_full_ce_v3width_sampled_rows_lse_all_rows():
    _ce_case(synth.V3, 40, lse_all_rows=True)


@pytest.mark.timeout(600)
def test_full_ce_d1_every_loss_row():
    _ce_case(synth.D1, None)


@pytest.mark.timeout(600)
def test_full_ce_d3_sampled_rows():
    _ce_case(synth.D3, 24)
