"""GPU parity of mtp_head_ce_fwd_bwd against the oracle: per-depth loss sums
to relative 2e-3 (float32: 1e-5); dh, dW_out, dg_out to max-abs 2e-2 plus a
relative Frobenius gate (bf16: 1e-2, float32: 1e-4); counts exact."""
import numpy as np
import pytest
import torch

from deepseek_sequential_mtp_amd import _lib, synth
from oracle import head as ohead, rows as orows
from oracle.numerics import BF16, EXACT
from tests.gpu_util import compare, rel_fro, tdev, to_np

pytestmark = pytest.mark.gpu


def _case(cfg, reduce="fixed", denom=0.0, label_rows=None, accumulate=False, seed=0, slab_rows=0,
          want_accuracy=False, mirror_head=False, plant_hits=False):
    inp = synth.make_head_inputs(cfg, seed)
    if mirror_head:                       # W_out[V-1-v] = W_out[v]: every logit appears twice
        W = inp["W_out"]
        W[cfg.V // 2:] = W[:cfg.V // 2][::-1]
    _, _, labels, _ = orows.dense_rows(inp["tokens"], inp["segment_ids"], cfg.D)
    labels = labels.reshape(cfg.D, -1)
    if label_rows is not None:            # keep labels only on these rows
        keep = np.zeros(labels.shape[1], bool)
        keep[label_rows] = True
        labels = np.where(keep[None, :], labels, -1)
    model = BF16 if cfg.dtype == "bf16" else EXACT
    if plant_hits:                        # half the loss rows labelled with the oracle's argmax
        pre = ohead.head_ce(inp["h"], labels, inp["W_out"], inp["g_out"], cfg.eps, cfg.lam, "fixed",
                            None, model, grads=False)
        rng = np.random.default_rng(seed + 11)
        labels = labels.copy()
        for k in range(cfg.D):
            rws = np.nonzero(labels[k] >= 0)[0]
            pick = rws[rng.random(rws.size) < 0.5]
            labels[k, pick] = pre["pred"][k, pick]
    dtype = torch.bfloat16 if cfg.dtype == "bf16" else torch.float32
    hs = [tdev(h, dtype) for h in inp["h"]]
    W = tdev(inp["W_out"], dtype)
    g = tdev(inp["g_out"], torch.float32)
    lab_t = tdev(labels.reshape(cfg.D, cfg.B, cfg.T).astype(np.int32), torch.int32)
    print(f"[ce] {cfg.name} N={cfg.N} d={cfg.d} V={cfg.V} D={cfg.D} reduce={reduce} "
          f"labelled={(labels >= 0).sum()} slab_rows={slab_rows or 'default'}", flush=True)
    out = None
    if accumulate:
        out = dict(loss_sum=torch.empty(cfg.D, device="cuda"), counts=torch.empty(cfg.D, dtype=torch.int32, device="cuda"),
                   loss=torch.empty(cfg.D, device="cuda"), loss_mtp=torch.empty(1, device="cuda"),
                   lse=torch.empty((cfg.D, cfg.N), device="cuda"),
                   dh=[torch.empty((cfg.N, cfg.d), device="cuda") for _ in range(cfg.D)],
                   dW_out=torch.full((cfg.V, cfg.d), 0.25, device="cuda"),
                   dg_out=torch.full((cfg.d,), -0.5, device="cuda"),
                   device_error=torch.empty(1, dtype=torch.int32, device="cuda"))
    if out is not None and want_accuracy:
        out.update(pred=torch.empty((cfg.D, cfg.N), dtype=torch.int32, device="cuda"),
                   correct=torch.empty(cfg.D, dtype=torch.int32, device="cuda"),
                   accuracy=torch.empty(cfg.D, device="cuda"))
    res = _lib.head_ce_fwd_bwd(hs, lab_t, W, g, lam=cfg.lam, eps=cfg.eps, reduce=reduce, denom=denom,
                               accumulate=accumulate, want_lse=True, want_accuracy=want_accuracy, out=out,
                               logit_slab_bytes=slab_rows * cfg.V * (2 if cfg.dtype == "bf16" else 4))
    torch.cuda.synchronize()
    ref = ohead.head_ce(inp["h"], labels, inp["W_out"], inp["g_out"], cfg.eps, cfg.lam, reduce,
                        denom if denom > 0 else None, model)
    if want_accuracy:
        _assert_accuracy(cfg, res, ref, labels, inp, model)
    return res, ref, labels


def _assert_accuracy(cfg, res, ref, labels, inp, model):
    """Top-1 accuracy by depth.  The argmax is unique where the best logit
    leads the runner-up by more than the logits' rounding difference (fp32
    vs float64 accumulation: 1e-3 in bf16 runs, 1e-5 in f32 runs); elsewhere
    the GPU's choice must be a valid maximum of the oracle's logits within
    that window.  correct is exact given the GPU's argmax."""
    pred = to_np(res["pred"]).reshape(cfg.D, -1).astype(np.int64)
    correct = to_np(res["correct"]).astype(np.int64)
    acc = to_np(res["accuracy"])
    tol = 1e-5 if cfg.dtype == "f32" else 1e-3
    W = np.asarray(inp["W_out"], np.float64)
    for k in range(cfg.D):
        m = labels[k] >= 0
        np.testing.assert_array_equal(pred[k, ~m], -1)
        assert np.all((pred[k, m] >= 0) & (pred[k, m] < cfg.V))
        assert correct[k] == int((pred[k, m] == labels[k, m]).sum())
        exp_acc = correct[k] / m.sum() if m.sum() else 0.0
        np.testing.assert_allclose(acc[k], exp_acc, rtol=1e-6)
        diff = np.nonzero(m & (pred[k] != ref["pred"][k]))[0]
        if diff.size:
            xh, _, _ = ohead.output_norm(np.asarray(inp["h"][k])[diff], inp["g_out"], cfg.eps, model)
            zo = xh @ W.T
            gap = zo[np.arange(diff.size), ref["pred"][k, diff]] - zo[np.arange(diff.size), pred[k, diff]]
            assert np.all(gap <= tol), (k, diff[:8], gap.max())
        assert abs(int(correct[k]) - int(ref["correct"][k])) <= diff.size
        print(f"  accuracy[{k}] {acc[k]:.4f} (oracle {ref['accuracy'][k]:.4f}); "
              f"{diff.size} near-tie rows of {int(m.sum())}", flush=True)


def _assert(cfg, res, ref, labels, accumulate=False):
    f32 = cfg.dtype == "f32"
    np.testing.assert_array_equal(to_np(res["counts"]), ref["counts"])
    assert int(to_np(res["device_error"])[0]) == 0
    ls = to_np(res["loss_sum"]).astype(np.float64)
    np.testing.assert_allclose(ls, ref["loss_sum"], rtol=1e-5 if f32 else 2e-3, atol=1e-6)
    np.testing.assert_allclose(to_np(res["loss"]), ref["loss"], rtol=1e-5 if f32 else 2e-3, atol=1e-9)
    np.testing.assert_allclose(to_np(res["loss_mtp"])[0], ref["loss_mtp"], rtol=1e-5 if f32 else 2e-3)
    lse = to_np(res["lse"])
    m = labels >= 0
    np.testing.assert_allclose(lse[m], ref["lse"][m], rtol=1e-5 if f32 else 2e-3)
    gate = 1e-4 if f32 else 1e-2
    for k in range(cfg.D):
        g = to_np(res["dh"][k])
        err, _, ok = compare(g, ref["dh"][k], 2e-2)
        rf = rel_fro(g, ref["dh"][k])
        print(f"  dh[{k}] max|err| {err:.3e} relF {rf:.2e}", flush=True)
        assert ok and rf < gate
    dW_ref = ref["dW_out"] + (0.25 if accumulate else 0.0)
    dg_ref = ref["dg_out"] + (-0.5 if accumulate else 0.0)
    dW = to_np(res["dW_out"])
    err, _, ok = compare(dW, dW_ref, 2e-2)
    rf = rel_fro(dW - (0.25 if accumulate else 0.0), ref["dW_out"])
    print(f"  dW max|err| {err:.3e} relF {rf:.2e}", flush=True)
    assert ok and rf < gate
    dg = to_np(res["dg_out"])
    err, _, ok = compare(dg, dg_ref, 2e-2)
    rf = rel_fro(dg - (-0.5 if accumulate else 0.0), ref["dg_out"])
    print(f"  dg max|err| {err:.3e} relF {rf:.2e}", flush=True)
    assert ok and rf < gate


@pytest.mark.parametrize("slab_rows", [0, 5])
def test_ce_tiny_f32(slab_rows):
    # slab_rows=5: 32 rows in 7 logit slabs, the last one ragged
    cfg = synth.TINY
    res, ref, labels = _case(cfg, slab_rows=slab_rows)
    _assert(cfg, res, ref, labels)


@pytest.mark.parametrize("reduce,slab_rows", [("fixed", 0), ("valid_mean", 0), ("fixed", 80),
                                              ("valid_mean", 128)])
def test_ce_bf16_ragged_two_depths(reduce, slab_rows):
    # the dx / dW GEMMs run once per logit slab (dz and the kept logits are
    # both 2 bytes wide).  slab_rows=128: 600 rows in slabs 128 x 4 and 88;
    # slab_rows=80: slabs 80 x 7 and 40; two depths
    cfg = synth.scaled(synth.D1, name="ce_ragged", B=2, T=300, d=256, V=1000, D=2, seg_lo=20,
                       seg_hi=200, sigma_w=0.05)
    res, ref, labels = _case(cfg, reduce=reduce, slab_rows=slab_rows)
    _assert(cfg, res, ref, labels)


@pytest.mark.parametrize("slab_rows", [0, 100])
def test_ce_bf16_accumulate_and_custom_denom(slab_rows):
    cfg = synth.scaled(synth.D1, name="ce_acc", B=1, T=256, d=128, V=512, D=1, seg_lo=30,
                       seg_hi=100, sigma_w=0.05)
    res, ref, labels = _case(cfg, denom=1000.0, accumulate=True, slab_rows=slab_rows)
    _assert(cfg, res, ref, labels, accumulate=True)


@pytest.mark.parametrize("slab_rows,d,V", [(1024, 1024, 16384), (256, 1024, 16384), (1024, 1056, 16384),
                                            (1024, 1024, 20480)])
def test_ce_bf16_big_tiles(slab_rows, d, V):
    # 256x256 tiles in the forward and dW GEMMs (>= 256 tiles each, balanced
    # schedule) when one slab holds all 1024 rows (an explicit bound: the
    # default one keeps at most half of the rows); slab_rows=256 runs the 1024 rows as four slabs, each its
    # own dz group; d=1056 gives the forward GEMM an odd number of 32-element K
    # slices (a half-filled last pair of 128-byte A rows); V=20480 makes 320
    # tiles: one whole round of 256, the other 64 split over K into partial
    # tiles that the fixup pass sums
    cfg = synth.scaled(synth.D1, name="ce_big", B=1, T=1024, d=d, V=V, D=1, seg_lo=100,
                       seg_hi=700, sigma_w=0.02)
    res, ref, labels = _case(cfg, slab_rows=slab_rows)
    _assert(cfg, res, ref, labels)


def test_ce_bf16_big_dx_tiles_sparse_labels():
    # 256x256 tiles in the dx GEMM, 64 of them, split 4 ways over K = V;
    # labels on 64 sampled rows keep the oracle cheap, the GPU runs every row
    cfg = synth.scaled(synth.D1, name="ce_bigdx", B=1, T=4096, d=1024, V=4096, D=1,
                       seg_lo=4096, seg_hi=4096, sigma_w=0.01)
    rows = np.random.default_rng(3).choice(4095, 64, replace=False)
    res, ref, labels = _case(cfg, label_rows=rows)
    _assert(cfg, res, ref, labels)


@pytest.mark.parametrize("slab_rows", [0, 5])
def test_ce_tiny_f32_accuracy(slab_rows):
    cfg = synth.TINY
    res, ref, labels = _case(cfg, slab_rows=slab_rows, want_accuracy=True, plant_hits=True)
    _assert(cfg, res, ref, labels)


@pytest.mark.parametrize("slab_rows,accumulate", [(0, False), (80, True)])
def test_ce_bf16_accuracy_two_depths(slab_rows, accumulate):
    cfg = synth.scaled(synth.D1, name="ce_acc_d2", B=2, T=300, d=256, V=1000, D=2, seg_lo=20,
                       seg_hi=200, sigma_w=0.05)
    res, ref, labels = _case(cfg, slab_rows=slab_rows, accumulate=accumulate, want_accuracy=True,
                             plant_hits=True)
    _assert(cfg, res, ref, labels, accumulate=accumulate)
    assert np.all(to_np(res["accuracy"]) > 0.4)


@pytest.mark.parametrize("dtype,V", [("f32", 512), ("bf16", 16384)])
def test_ce_accuracy_exact_ties_take_the_lowest_id(dtype, V):
    # the head's second half mirrors its first: each logit appears at v and
    # V-1-v, in another vocabulary tile, and the lower id must win
    cfg = synth.scaled(synth.D1, name="ce_ties", B=1, T=512, d=256, V=V, D=1, seg_lo=512,
                       seg_hi=512, sigma_w=0.05, dtype=dtype)
    res, ref, labels = _case(cfg, want_accuracy=True, mirror_head=True)
    pred = to_np(res["pred"]).reshape(-1)
    m = labels[0] >= 0
    assert np.all(pred[m] < V // 2)


@pytest.mark.parametrize("slab_rows", [1024, 256])
def test_ce_bf16_big_tiles_accuracy(slab_rows):
    cfg = synth.scaled(synth.D1, name="ce_big_acc", B=1, T=1024, d=1024, V=16384, D=1, seg_lo=100,
                       seg_hi=700, sigma_w=0.02)
    res, ref, labels = _case(cfg, slab_rows=slab_rows, want_accuracy=True, plant_hits=True)
    _assert(cfg, res, ref, labels)
    assert to_np(res["accuracy"])[0] > 0.4


def test_ce_bf16_more_rows_than_one_grid_dimension():
    # 70000 rows in one logit slab (an explicit bound of 70144 rows): the
    # softmax-gradient pass strides its rows over a grid dimension of at most
    # 65535 blocks; labels on 256 sampled rows (160 of them beyond row 65535)
    # keep the oracle cheap
    cfg = synth.scaled(synth.D1, name="ce_tall", B=1, T=70000, d=64, V=256, D=1, seg_lo=2000,
                       seg_hi=9000, sigma_w=0.05)
    rng = np.random.default_rng(4)
    rows = np.concatenate([rng.choice(65536, 96, replace=False),
                           65536 + rng.choice(70000 - 65536, 160, replace=False)])
    res, ref, labels = _case(cfg, label_rows=rows, want_accuracy=True, slab_rows=70144)
    assert int((labels[0, 65536:] >= 0).sum()) > 100
    _assert(cfg, res, ref, labels)


@pytest.mark.parametrize("d", [3072, 8200])
def test_ce_bf16_output_norm_backward_widths(d):
    # the output-norm backward keeps a row block in registers for d <= 8192
    # (d = 3072: three 4-column chunks per thread) and takes the two-pass
    # kernels beyond (d = 8200)
    cfg = synth.scaled(synth.D1, name="ce_wide", B=2, T=40, d=d, V=256, D=1, seg_lo=10, seg_hi=40,
                       sigma_w=0.02)
    res, ref, labels = _case(cfg)
    _assert(cfg, res, ref, labels)


def test_ce_empty_depth_and_bad_labels():
    cfg = synth.scaled(synth.D1, name="ce_empty", B=1, T=64, d=128, V=256, D=2, seg_lo=64,
                       seg_hi=64, sigma_w=0.05)
    inp = synth.make_head_inputs(cfg)
    _, _, labels, _ = orows.dense_rows(inp["tokens"], inp["segment_ids"], 2)
    labels = labels.reshape(2, -1)
    labels[1, :] = -1                          # depth 2 empty
    hs = [tdev(h, torch.bfloat16) for h in inp["h"]]
    W = tdev(inp["W_out"], torch.bfloat16)
    g = tdev(inp["g_out"], torch.float32)
    for reduce in ("fixed", "valid_mean"):
        lab_t = tdev(labels.reshape(2, 1, 64).astype(np.int32), torch.int32)
        res = _lib.head_ce_fwd_bwd(hs, lab_t, W, g, lam=0.1, reduce=reduce)
        torch.cuda.synchronize()
        ref = ohead.head_ce(inp["h"], labels, inp["W_out"], inp["g_out"], 1e-6, 0.1, reduce, None, BF16)
        assert to_np(res["loss"])[1] == 0.0 and to_np(res["counts"])[1] == 0
        np.testing.assert_allclose(to_np(res["loss_mtp"])[0], ref["loss_mtp"], rtol=2e-3)
        assert np.all(to_np(res["dh"][1]) == 0.0)
    bad = labels.copy()
    bad[0, 5] = 10 ** 6                        # out of range: ignored and flagged
    lab_t = tdev(bad.reshape(2, 1, 64).astype(np.int32), torch.int32)
    res = _lib.head_ce_fwd_bwd(hs, lab_t, W, g, lam=0.1)
    torch.cuda.synchronize()
    assert int(to_np(res["device_error"])[0]) == 1
    assert int(to_np(res["counts"])[0]) == int((labels[0] >= 0).sum()) - 1
