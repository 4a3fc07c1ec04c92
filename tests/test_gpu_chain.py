"""GPU parity of mtp_chain_forward against the oracle: masks, labels and
counts bit-exact; h^(k) on state rows within tolerance (float32: 1e-4
max-abs and relative Frobenius error below 4e-3 k; bf16: max-abs 2e-2 or
one bf16 ulp of the larger magnitude, no element beyond 4e-2, at most 0.2%
of a depth's elements over 2e-2 and 0.05% beyond one ulp and 2e-2 (none at
depth 1), relative Frobenius error below 2.5e-3 k -- ``tests.gpu_util.compare_h``)."""
import numpy as np
import pytest
import torch

from deepseek_sequential_mtp_amd import _lib, synth
from oracle import chain as ochain, rows as orows
from oracle.numerics import BF16, EXACT
from tests.gpu_util import chain_tensors, compare, compare_h, fmt_h, rel_fro, to_np

pytestmark = pytest.mark.gpu


def _run(cfg, seed_offset=0, seg_override=None):
    inp = synth.make_chain_inputs(cfg, seed_offset)
    if seg_override is not None:
        inp["segment_ids"] = seg_override
    dtype = torch.bfloat16 if cfg.dtype == "bf16" else torch.float32
    t = chain_tensors(inp, dtype)
    print(f"[chain] {cfg.name} B={cfg.B} T={cfg.T} d={cfg.d} H={cfg.n_heads}x{cfg.head_dim} "
          f"f={cfg.ffn} V={cfg.V} D={cfg.D}", flush=True)
    out = _lib.chain_forward(t["tokens"], t["segment_ids"], t["h0"], t["E"], t["depths"],
                             n_heads=cfg.n_heads, head_dim=cfg.head_dim, eps=cfg.eps,
                             rope_theta=cfg.rope_theta)
    torch.cuda.synchronize()
    return inp, out


def _check(cfg, inp, out, model, atol):
    st, ls, lab, cnt = orows.dense_rows(inp["tokens"], inp["segment_ids"], cfg.D)
    np.testing.assert_array_equal(to_np(out["state_mask"]), st)
    np.testing.assert_array_equal(to_np(out["loss_mask"]), ls)
    np.testing.assert_array_equal(to_np(out["labels"]), lab)
    np.testing.assert_array_equal(to_np(out["counts"]), cnt)
    assert int(to_np(out["device_error"])[0]) == 0
    hs = ochain.chain_forward(inp["h0"], inp["tokens"], inp["segment_ids"], inp["depths"],
                              inp["E"], cfg.n_heads, cfg.head_dim, cfg.eps, cfg.rope_theta, model)
    for k in range(cfg.D):
        rows_k = st[k].reshape(-1).astype(bool)
        g = to_np(out["h"][k])
        assert np.isfinite(g).all()
        if model is BF16:
            stt = compare_h(g[rows_k], hs[k][rows_k], k + 1)
            print(f"  depth {k + 1}: state rows {rows_k.sum()}, {fmt_h(stt)}", flush=True)
            assert stt["ok"], (k, stt)
            continue
        err, n_over, ok = compare(g[rows_k], hs[k][rows_k], atol)
        rf = rel_fro(g[rows_k], hs[k][rows_k])
        print(f"  depth {k + 1}: state rows {rows_k.sum()}, max|err| {err:.3e}, "
              f"over atol {n_over}, relF {rf:.2e}", flush=True)
        assert ok and rf < 4e-3 * (k + 1), (k, err, n_over, rf)


def test_chain_tiny_f32():
    cfg = synth.TINY
    inp, out = _run(cfg)
    _check(cfg, inp, out, EXACT, 1e-4)


def test_chain_tiny_f32_depth3_and_degenerate_rows():
    # D = 3 on the tiny layout plus a one-token segment and a fully padded tail
    cfg = synth.scaled(synth.TINY, D=3)
    seg = synth.tiny_segments()
    seg[0, 10] = 5          # a one-token segment: never a state row
    _inp, out = _run(cfg, seg_override=seg)
    _check(cfg, _inp, out, EXACT, 1e-4)


@pytest.mark.parametrize("hd", [128, 64, 32])
def test_chain_bf16_ragged(hd):
    # several tiles in every GEMM, ragged row / feature / vocabulary tails,
    # packed segments of mixed lengths, two depths; head_dim 32 puts the
    # rotary partner 16 lanes away (the others: in the same lane)
    cfg = synth.scaled(synth.D1, name=f"ragged_hd{hd}", B=2, T=300, d=256, n_heads=256 // hd,
                       head_dim=hd, ffn=688, V=1000, D=2, seg_lo=20, seg_hi=200, sigma_w=0.05)
    inp, out = _run(cfg)
    _check(cfg, inp, out, BF16, 2e-2)


@pytest.mark.parametrize("hd", [128, 64])
def test_chain_bf16_few_rows(hd):
    # at most 64 rows (B * T = 2 x 29): every GEMM of the chain runs on the
    # 64-row tile (its ragged row tail, three vocabulary-sized operands of
    # 256-wide column tiles plus a ragged one); two depths
    cfg = synth.scaled(synth.D1, name=f"few_rows_hd{hd}", B=2, T=29, d=256, n_heads=256 // hd, head_dim=hd,
                       ffn=688, V=1000, D=2, seg_lo=5, seg_hi=20, sigma_w=0.05)
    inp, out = _run(cfg)
    _check(cfg, inp, out, BF16, 2e-2)


def test_chain_bf16_padding_and_token_error():
    cfg = synth.scaled(synth.D1, name="padded", B=2, T=130, d=128, n_heads=1, head_dim=128,
                       ffn=256, V=512, D=1, seg_lo=10, seg_hi=60, sigma_w=0.05)
    inp = synth.make_chain_inputs(cfg)
    seg = inp["segment_ids"].copy()
    seg[1, 70:] = -1                          # padded tail
    inp["segment_ids"] = seg
    dtype = torch.bfloat16
    t = chain_tensors(inp, dtype)
    out = _lib.chain_forward(t["tokens"], t["segment_ids"], t["h0"], t["E"], t["depths"],
                             n_heads=1, head_dim=128, eps=cfg.eps, rope_theta=cfg.rope_theta)
    torch.cuda.synchronize()
    _check(cfg, inp, out, BF16, 2e-2)
    # a padding slot may hold any id; an active slot outside [0, V) raises the flag
    tok = t["tokens"].clone()
    tok[1, 100] = 10 ** 6                     # padding: ignored
    out2 = _lib.chain_forward(tok, t["segment_ids"], t["h0"], t["E"], t["depths"],
                              n_heads=1, head_dim=128, eps=cfg.eps, rope_theta=cfg.rope_theta)
    torch.cuda.synchronize()
    assert int(to_np(out2["device_error"])[0]) == 0
    tok[0, 3] = -5                            # active: flagged
    out3 = _lib.chain_forward(tok, t["segment_ids"], t["h0"], t["E"], t["depths"],
                              n_heads=1, head_dim=128, eps=cfg.eps, rope_theta=cfg.rope_theta)
    torch.cuda.synchronize()
    assert int(to_np(out3["device_error"])[0]) == 1


def test_chain_rope_off_and_deterministic():
    cfg = synth.scaled(synth.D1, name="norope", B=1, T=200, d=128, n_heads=2, head_dim=64,
                       ffn=256, V=512, D=1, seg_lo=50, seg_hi=150, sigma_w=0.05, rope_theta=0.0)
    inp, out = _run(cfg)
    _check(cfg, inp, out, BF16, 2e-2)
    t = chain_tensors(inp, torch.bfloat16)
    out2 = _lib.chain_forward(t["tokens"], t["segment_ids"], t["h0"], t["E"], t["depths"],
                              n_heads=2, head_dim=64, eps=cfg.eps, rope_theta=0.0)
    torch.cuda.synchronize()
    assert torch.equal(out["h"][0], out2["h"][0])


def test_chain_bf16_wide_tile_ragged():
    # 4000 rows x d 7000: the three NT GEMMs with d outputs (eh_proj, O-proj,
    # down) take the 256 x 224 tile (512 tiles where 256 x 256 would make 448,
    # a partly idle second round), with a ragged last row tile (4000 = 15 x 256
    # + 160) and a ragged last column tile (7000 = 31 x 224 + 56).  Weights at
    # the V3-width scale (sigma 0.006), where |h| stays near the workloads'
    # magnitudes that the bf16 rule is calibrated on
    cfg = synth.scaled(synth.D1, name="wide_tile", B=1, T=4000, d=7000, n_heads=2, head_dim=128,
                       ffn=512, V=512, D=1, seg_lo=64, seg_hi=1024, sigma_w=0.006)
    inp, out = _run(cfg)
    _check(cfg, inp, out, BF16, 2e-2)
