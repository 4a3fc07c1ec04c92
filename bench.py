"""Benchmark of one MTP training step on one MI355X.

A step is mtp_chain_forward (all D depths) followed by mtp_head_ce_fwd_bwd
(all D depths) on one stream, inputs resident in HBM.  Default workload: the
V3-width configuration (B=1, T=4096, d=7168, 128 heads x 128, ffn=18432,
V=129280, D=1, bf16) with synthetic seeded inputs of the stated
distributions, generated on the device.

Prints one JSON line: tokens/s (B*T / step time), the step's fraction of the
bf16 dense MFMA peak on algorithmic FLOPs, a roofline entry for the dominant
kernel (its launches timed with HIP events over the timed region), and the
CPU oracle timed on a bounded sample of the same workload.

    python bench.py [--gpus 1] [--steps 20] [--warmup 5] [--workload v3width_bf16]
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2500.0     # MI355X dense bf16 MFMA
PEAK_HBM_GBS = 8000.0


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="v3width_bf16")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-rows", type=int, default=2048)
    ap.add_argument("--stages", action="store_true", help="print the per-stage time table to stderr")
    ap.add_argument("--propose-only", action="store_true",
                    help="time only the retained-module proposer step and print its JSON object")
    ap.add_argument("--accuracy", action="store_true",
                    help="also compute the top-1 accuracy by depth in every step (printed to stderr)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="after the timed region, run a plain 256 MiB fp32 copy kernel 3 times (the "
                         "reference dispatch that scales FETCH_SIZE / WRITE_SIZE counters)")
    ap.add_argument("--ingest-pmc", nargs=3, metavar=("STAGE", "FETCH_CSV", "WRITE_CSV"),
                    help="no GPU: turn two rocprofv3 --pmc counter CSVs (FETCH_SIZE, WRITE_SIZE) of a "
                         "--copy-calibration run into profiles/traffic_<stage>_<workload>.json")
    ap.add_argument("--pmc-table", nargs=2, metavar=("FETCH_CSV", "WRITE_CSV"),
                    help="no GPU: print per-kernel HBM bytes per dispatch (markdown) of the step's and the "
                         "verify benchmark's kernels from the two counter CSVs of a --copy-calibration run")
    return ap.parse_args()


# Kernel-name patterns of each stage; rocprofv3 prints some names demangled
# and some mangled (templates with a _Float16 argument), so each pattern
# matches both spellings.
STAGE_KERNELS = {
    "CE_DW": r"gemm_kernel.*DmaMNMajor(<[^>]*>, mtp::|IS1_Li256ELi512EEENS_10)DmaMNMajor",
    "CE_DX": r"gemm_kernel.*DmaKMajor(<[^>]*>, mtp::|IS1_Li256ELi512EEENS_10)DmaMNMajor",
    "CE_FWD": r"gemm_kernel.*EpiCEFwd",
    "QKV": r"gemm_kernel.*EpiRope",
    "GATE_UP": r"gemm_kernel.*EpiSwiGLU",
    "ATTN": r"attention_kernel",
}
COPY_BYTES = 256 << 20          # one direction of the calibration copy
COPY_KERNEL = r"neg_kernel"
COPY_REPS = 3
FIXUP_KERNEL = r"gemm_fixup_kernel"
# Bandwidth kernels named in the per-kernel traffic table (besides the stages above).
TABLE_KERNELS = {
    "DUAL_NORM": r"dual_norm_concat_kernel",
    "NORM_A_F": r"rmsnorm_kernel",
    "OUT_NORM": r"out_norm_kernel",
    "OUT_NORM_BWD": r"out_norm_bwd",
    "CE_DZ": r"ce_dz_kernel",
    "EH_O_DOWN": r"gemm_kernel.*DmaKMajor128<[^>]*>, mtp::DmaKMajor<[^>]*>, mtp::EpiStore<",
    "GEMM_FIXUP": FIXUP_KERNEL,
    "VERIFY_LSE": r"verify_lse_kernel",
    "VERIFY_MASS": r"verify_mass_kernel",
    "VERIFY_PICK": r"verify_pick_kernel",
    "VERIFY_TESTS": r"verify_tests_kernel",
}


def _read_counter(path, counter):
    """{dispatch id: (kernel name, grid size, summed counter value in KiB)}."""
    import csv
    rows = {}
    with open(path) as fh:
        for r in csv.DictReader(fh):
            if r["Counter_Name"] != counter:
                continue
            key = int(r["Dispatch_Id"])
            name, grid, val = rows.get(key, (r["Kernel_Name"], int(r.get("Grid_Size", 0) or 0), 0.0))
            rows[key] = (name, grid, val + float(r["Counter_Value"]))
    return rows


def _phases(rows, path):
    """Split the dispatches of a --copy-calibration run at the calibration
    copies: the first COPY_REPS copies follow the timed steps, the next
    COPY_REPS follow the verify benchmark.  Returns the copy factor (counter
    bytes per byte copied) and the dispatch ids of the two phases."""
    import re
    copies = sorted(i for i, (n, _, _) in rows.items() if re.search(COPY_KERNEL, n))
    if len(copies) < COPY_REPS:
        raise SystemExit(f"{path}: fewer than {COPY_REPS} calibration copies")
    factor = float(np.median([rows[i][2] for i in copies])) * 1024.0 / COPY_BYTES
    first, last1 = copies[0], copies[COPY_REPS - 1]
    end2 = copies[2 * COPY_REPS - 1] if len(copies) >= 2 * COPY_REPS else None
    step = {i for i in rows if i < first}
    verify = {i for i in rows if end2 is not None and last1 < i < copies[COPY_REPS]}
    return factor, step, verify


def _stage_dispatches(rows, ids, stage):
    """The stage's dispatches among `ids`: its GEMM launches (the main grid and
    a split tail) and the fixup kernel that follows a split tail."""
    import re
    mine = {i for i in ids if re.search(STAGE_KERNELS[stage], rows[i][0])}
    mine |= {i for i in ids if re.search(FIXUP_KERNEL, rows[i][0]) and (i - 1) in mine}
    return mine


def ingest_pmc(stage, fetch_csv, write_csv, workload):
    """HBM bytes per step of `stage` over the timed steps (the dispatches
    before the first calibration copy), from the two counter passes, each
    scaled by the same counter's reading for the copy kernel.  The number of
    steps is the output-norm dispatch count over the depth count."""
    import re
    from deepseek_sequential_mtp_amd import synth
    D = synth.CHAIN_CONFIGS[workload].D

    def per_step(path, counter):
        rows = _read_counter(path, counter)
        factor, step, _ = _phases(rows, path)
        n_steps = sum(1 for i in step if re.search(TABLE_KERNELS["OUT_NORM"], rows[i][0])) / D
        mine = _stage_dispatches(rows, step, stage)
        if not mine or n_steps < 1:
            raise SystemExit(f"{path}: no {counter} rows for the stage kernel before the calibration copy")
        total = sum(rows[i][2] for i in mine) * 1024.0 / factor
        return total / n_steps, factor, len(mine), n_steps

    fetch, ff, nf, sf = per_step(fetch_csv, "FETCH_SIZE")
    write, fw, nw, sw = per_step(write_csv, "WRITE_SIZE")
    out = {"stage": stage, "workload": workload, "kernel_regex": STAGE_KERNELS[stage],
           "fetch_bytes_per_step": fetch, "write_bytes_per_step": write, "bytes_per_step": fetch + write,
           "copy_factor_fetch": ff, "copy_factor_write": fw, "dispatches_counted": [nf, nw], "steps": [sf, sw],
           "source_hash": _kernel_hash(stage)}
    path = os.path.join(ROOT, "profiles", f"traffic_{stage.lower()}_{workload}.json")
    with open(path, "w") as fh:
        json.dump(out, fh, indent=1)
    print(json.dumps(out))


def pmc_table(fetch_csv, write_csv):
    """Markdown table: mean HBM bytes per dispatch (FETCH_SIZE, WRITE_SIZE,
    each scaled by the copy kernel's reading) of every named kernel, grouped
    by phase (timed steps / verify benchmark) and grid size."""
    import re
    labels = dict(STAGE_KERNELS)
    labels.update(TABLE_KERNELS)
    groups = {}
    for counter, path in (("FETCH_SIZE", fetch_csv), ("WRITE_SIZE", write_csv)):
        rows = _read_counter(path, counter)
        factor, step, verify = _phases(rows, path)
        for phase, ids in (("step", step), ("verify", verify)):
            for i in ids:
                name, grid, val = rows[i]
                lab = next((k for k, rx in labels.items() if re.search(rx, name)), None)
                if lab is None:
                    continue
                g = groups.setdefault((phase, lab, grid), {"FETCH_SIZE": [], "WRITE_SIZE": []})
                g[counter].append(val * 1024.0 / factor)
    print("| phase | kernel | grid size | dispatches | fetch MB / dispatch | write MB / dispatch |")
    print("|---|---|---|---|---|---|")
    for (phase, lab, grid), g in sorted(groups.items()):
        if not g["FETCH_SIZE"] or not g["WRITE_SIZE"]:
            continue
        print(f"| {phase} | {lab} | {grid} | {len(g['FETCH_SIZE'])} | {np.mean(g['FETCH_SIZE']) / 1e6:.2f} | "
              f"{np.mean(g['WRITE_SIZE']) / 1e6:.2f} |")


# ----------------------------------------------------------------------------
# inputs (device-side generation with the synthetic recipe)
# ----------------------------------------------------------------------------
def device_inputs(cfg, torch):
    from deepseek_sequential_mtp_amd import synth
    ss = np.random.SeedSequence(synth.BASE_SEED + cfg.index)
    g_tok, g_seg = [np.random.Generator(np.random.PCG64(k)) for k in ss.spawn(2)]
    tokens = (synth.zipf_tokens(g_tok, cfg.V, (cfg.B, cfg.T)) if cfg.zipf
              else g_tok.integers(0, cfg.V, (cfg.B, cfg.T)).astype(np.int32))
    seg = synth.packed_segments(g_seg, cfg.B, cfg.T, cfg.seg_lo, cfg.seg_hi)
    dev = "cuda:0"
    gen = torch.Generator(device=dev)
    gen.manual_seed(synth.BASE_SEED + cfg.index)
    bf = torch.bfloat16

    def normal(shape, sigma, mean=0.0, dtype=bf):
        t = torch.randn(shape, generator=gen, device=dev, dtype=torch.float32)
        return (t * sigma + mean).to(dtype)

    d, V, A, f = cfg.d, cfg.V, cfg.A_w, cfg.ffn
    inp = dict(tokens=torch.from_numpy(tokens).to(dev), segment_ids=torch.from_numpy(seg).to(dev),
               h0=normal((cfg.N, d), 1.0), E=normal((V, d), cfg.sigma_w),
               W_out=normal((V, d), cfg.sigma_w), g_out=normal((d,), 0.1, 1.0, torch.float32))
    inp["depths"] = [dict(g_h=normal((d,), 0.1, 1.0, torch.float32), g_e=normal((d,), 0.1, 1.0, torch.float32),
                          M=normal((d, 2 * d), cfg.sigma_w), g_a=normal((d,), 0.1, 1.0, torch.float32),
                          Wqkv=normal((3 * A, d), cfg.sigma_w), Wo=normal((d, A), cfg.sigma_w),
                          g_f=normal((d,), 0.1, 1.0, torch.float32), Wgate=normal((f, d), cfg.sigma_w),
                          Wup=normal((f, d), cfg.sigma_w), Wdown=normal((d, f), cfg.sigma_w))
                     for _ in range(cfg.D)]
    return inp


# ----------------------------------------------------------------------------
# algorithmic work from the realised packing
# ----------------------------------------------------------------------------
def run_starts(seg):
    """First position of each position's run (a maximal stretch of one
    segment id >= 0); a padding position is its own window."""
    B, T = seg.shape
    idx = np.arange(T)[None, :].repeat(B, 0)
    new_run = np.ones((B, T), dtype=bool)
    new_run[:, 1:] = (seg[:, 1:] != seg[:, :-1]) | (seg[:, 1:] < 0)
    return np.maximum.accumulate(np.where(new_run, idx, 0), axis=1)


def algorithmic_flops(cfg, state_mask, counts, run_start_fn):
    """Per depth: state rows S_k, loss rows L_k, attention pairs P_k (sum over
    state rows of the causal window length).  FLOPs (multiply-add = 2):
    eh_proj 4 d^2 S, QKV 6 d A S, attention 4 A P, O 2 A d S, SwiGLU 6 d f S,
    head 6 d V L (2 forward + 4 backward)."""
    d, A, f, V = cfg.d, cfg.A_w, cfg.ffn, cfg.V
    per = []
    rs = run_start_fn()
    pos = np.arange(cfg.T)[None, :]
    for k in range(cfg.D):
        st = state_mask[k].astype(bool)
        S = int(st.sum())
        L = int(counts[k])
        P = int(((pos - rs + 1) * st).sum())
        per.append(dict(S=S, L=L, P=P,
                        EH_PROJ=4.0 * d * d * S, QKV=6.0 * d * A * S, ATTN=4.0 * A * P,
                        O_PROJ=2.0 * A * d * S, GATE_UP=4.0 * d * f * S, DOWN=2.0 * f * d * S,
                        CE_FWD=2.0 * d * V * L, CE_DX=2.0 * d * V * L, CE_DW=2.0 * d * V * L,
                        CE_GRAD=0.0))
    return per


def executed_tflop(cfg, run_start):
    """MFMA work the kernels execute per step (multiply-add = 2): every row of
    the dense layout, GEMM tiles padded to 256, attention over the key tiles
    each 32-query wave visits (masked pairs included), and no recomputation.""" 
    def pad(x):
        return -(-x // 256) * 256
    d, A, f, V, N, hd = cfg.d, cfg.A_w, cfg.ffn, cfg.V, cfg.N, cfg.head_dim
    gemm = 2.0 * pad(N) * (pad(d) * 2 * d + pad(3 * A) * d + pad(d) * A + pad(2 * f) * d + pad(d) * f)
    head = 3 * 2.0 * pad(N) * pad(V) * d
    T = cfg.T
    wave_tiles = 0
    for b in range(cfg.B):
        rs = run_start[b]
        for q0 in range(0, T, 256):
            kbeg = rs[q0] // 64 * 64
            for w in range(q0, min(q0 + 256, T), 32):
                hi = min(w + 31, T - 1)
                lo = rs[w]
                first = kbeg + max(0, -(-(lo - 63 - kbeg) // 64)) * 64
                wave_tiles += max(0, (hi - first) // 64 + 1)
    attn = wave_tiles * cfg.n_heads * (2.0 + 2.0) * 32 * 64 * hd
    return cfg.D * (gemm + head + attn) / 1e12


# Algorithmic HBM bytes per depth of the memory-bound stages (N rows): what
# each kernel must read and write once (bf16 activations, fp32 residual
# stream and head gradients, fp16 logits).
def stage_bytes(cfg):
    N, d, V = cfg.N, cfg.d, cfg.V
    return {"DUAL_NORM": 8.0 * N * d,      # h, gathered E rows -> [h_norm, e_norm]
            "NORM_A": 6.0 * N * d,         # u (f32) -> x_a
            "NORM_F": 6.0 * N * d,         # a (f32) -> y
            "OUT_NORM": 4.0 * N * d,       # h -> x_hat
            "CE_GRAD": 4.0 * N * V,        # fp16 logits -> bf16 softmax - onehot
            "CE_NORM_BWD": 10.0 * N * d}   # dx_hat (f32), h -> dh (f32)


def stage_table(cfg, stage_ms, per):
    """Per-stage time of one step and its roofline: algorithmic TFLOP/s
    against the bf16 MFMA peak, or algorithmic GB/s against HBM."""
    flops_keys = ("EH_PROJ", "QKV", "ATTN", "O_PROJ", "GATE_UP", "DOWN", "CE_FWD", "CE_DX", "CE_DW")
    nbytes = stage_bytes(cfg)
    out = {}
    for name, ms in stage_ms.items():
        row = {"ms": round(ms, 4)}
        if name in flops_keys:
            a = sum(p[name] for p in per) / (ms * 1e-3) / 1e12
            row.update(bound="mfma", achieved=round(a, 1), unit="TFLOP/s", frac=round(a / PEAK_BF16_TFLOPS, 4))
        elif name in nbytes:
            a = nbytes[name] * cfg.D / (ms * 1e-3) / 1e9
            row.update(bound="hbm", achieved=round(a, 1), unit="GB/s", frac=round(a / PEAK_HBM_GBS, 4))
        else:
            row.update(bound="latency")
        out[name] = row
    return out


def bench_propose(torch, _lib, cfg, inp, R=64, prefix=2048, reps=10):
    """mtp_propose_step at the workload's module width: R requests, each with
    ``prefix`` cached slots of the module's own K/V (random bf16; the step
    reads them all and writes slot ``prefix``), the retained module's weights
    and the shared head of the chain inputs.  Time from HIP events around the
    call on its stream; GB/s on the algorithmic HBM bytes of one step: the
    module and head weights once, the cached keys and values once, the
    gathered embedding rows, the state in and out, the stored logits written
    and read once by the draw."""
    dev = inp["h0"].device
    A = cfg.n_heads * cfg.head_dim
    L_max = prefix + 64
    g = torch.Generator(device=dev).manual_seed(4321)
    kv = (torch.randn((R, 2, L_max, A), generator=g, device=dev, dtype=torch.float32) * 0.5).to(torch.bfloat16)
    h = inp["h0"][:R].contiguous()
    tok = inp["tokens"].reshape(-1)[1:R + 1].clone()          # a fresh (16-byte aligned) buffer
    pos = torch.full((R,), prefix, dtype=torch.int32, device=dev)
    us = torch.rand((R,), generator=g, device=dev)
    w = inp["depths"][0]
    cache = {}
    run = lambda out=None: _lib.propose_step(h, tok, pos, us, kv, w, inp["E"], inp["W_out"], inp["g_out"],
                                             n_heads=cfg.n_heads, head_dim=cfg.head_dim, eps=cfg.eps,
                                             rope_theta=cfg.rope_theta, out=out, cache=cache)
    out = run()
    torch.cuda.synchronize()
    assert int((out["status"] != 0).sum()) == 0
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    times = []
    for _ in range(reps):
        e0.record()
        run(out)
        e1.record()
        torch.cuda.synchronize()
        times.append(e0.elapsed_time(e1))
    ms = float(np.median(times))
    d, f, V = cfg.d, cfg.ffn, cfg.V
    weights = (2 * d * d + 4 * A * d + 3 * f * d + V * d) * 2.0
    kv_bytes = R * prefix * A * 2 * 2.0 + R * A * 2 * 2.0
    rows = R * d * 2 * 3.0 + R * V * 2 * 2.0
    total = weights + kv_bytes + rows
    gbs = total / (ms * 1e-3) / 1e9
    del kv
    return {"R": R, "cached_slots": prefix, "d": d, "n_heads": cfg.n_heads, "head_dim": cfg.head_dim,
            "ffn": f, "V": V, "ms": round(ms, 4), "bytes": total, "bytes_weights": weights,
            "bytes_kv": kv_bytes, "achieved": round(gbs, 1), "unit": "GB/s",
            "frac": round(gbs / PEAK_HBM_GBS, 4)}


def bench_backward(torch, _lib, cfg, inp, chain_out, ce_out, per, cache, reps=5):
    """mtp_chain_backward after the timed step (its chain outputs and the head
    CE's dh): the gradient of L_MTP through every module to h^(0), E and the
    per-depth weights, timed with the forward's saved activations (`ms`) and
    with each depth's forward recomputed (`ms_recompute`).  Algorithmic work
    credits the products of the reverse pass once: the data and weight
    gradients of every chain GEMM (twice the forward's FLOPs) and 8 A per
    attention pair (dV, dP, dQ, dK)."""
    dev = inp["h0"].device
    out = dict(dh0=torch.empty((cfg.N, cfg.d), dtype=torch.float32, device=dev),
               dE=torch.zeros((cfg.V, cfg.d), dtype=torch.float32, device=dev),
               dw=[{n: torch.empty(w[n].shape, dtype=torch.float32, device=dev) for n in _lib.GRAD_FIELDS}
                   for w in inp["depths"]],
               device_error=torch.empty(1, dtype=torch.int32, device=dev))
    # the same forward again with its activations kept (untimed)
    kept = _lib.chain_forward(inp["tokens"], inp["segment_ids"], inp["h0"], inp["E"], inp["depths"],
                              n_heads=cfg.n_heads, head_dim=cfg.head_dim, eps=cfg.eps, rope_theta=cfg.rope_theta,
                              save=True)

    def run(saved):
        _lib.chain_backward(inp["tokens"], inp["segment_ids"], inp["h0"], inp["E"], inp["depths"], chain_out["h"],
                            ce_out["dh"], n_heads=cfg.n_heads, head_dim=cfg.head_dim, eps=cfg.eps,
                            rope_theta=cfg.rope_theta, out=out, cache=cache, saved=saved)

    def timed(saved):
        run(saved)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        timer = _lib.AllStageTimer(64 * reps)
        with timer:
            e0.record()
            for _ in range(reps):
                run(saved)
            e1.record()
            torch.cuda.synchronize()
        ms = e0.elapsed_time(e1) / reps
        return ms, {k: {"ms": round(float(np.sum(v)) / reps, 4)} for k, v in timer.by_stage().items()}

    ms, stages = timed(kept["saved"])
    ms_re, stages_re = timed(None)
    g = lambda *ks: sum(p[k] for p in per for k in ks)
    fwd_gemm = g("EH_PROJ", "QKV", "O_PROJ", "GATE_UP", "DOWN")
    attn = g("ATTN")                                        # 4 A per pair
    alg = 2.0 * fwd_gemm + 2.0 * attn
    # executed: the gate/up product again inside the MLP reverse, and the
    # attention reverse's dV pass (S, dV), dK pass (S, dP, dK) and dQ pass
    # (S, dP, dQ): 16 A per pair; the recompute adds eh_proj, QKV, O-proj
    # and the attention forward
    executed = 2.0 * fwd_gemm + g("GATE_UP") + 4.0 * attn
    executed_re = executed + g("EH_PROJ", "QKV", "O_PROJ") + attn
    tf = alg / (ms * 1e-3) / 1e12
    del out, kept
    return {"ms": round(ms, 4), "ms_recompute": round(ms_re, 4), "algorithmic_tflop": round(alg / 1e12, 3),
            "executed_tflop": round(executed / 1e12, 3), "executed_tflop_recompute": round(executed_re / 1e12, 3),
            "achieved": round(tf, 1), "unit": "TFLOP/s", "frac": round(tf / PEAK_BF16_TFLOPS, 4),
            "frac_recompute": round(alg / (ms_re * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4),
            "tokens_per_s": round(cfg.N / (ms * 1e-3), 1), "stages": stages, "stages_recompute": stages_re,
            "flops_basis": "algorithmic reverse-pass FLOPs / call time (saved activations; recompute beside it)"}


def bench_horizons(torch, _lib, cfg, inp, K=2, reps=3):
    """mtp_horizon_heads at the workload's width: K independent horizon heads
    (a Transformer block each, then the shared head), forward and backward one
    head after another on the step's trunk state h^(0).  Algorithmic work per
    head: the block's forward (6 d A + 2 A d + 6 d f per row, 4 A per attention
    pair), its backward (twice that), and the head CE's 6 d V per labelled row."""
    dev = inp["h0"].device
    g = torch.Generator(device=dev).manual_seed(777)
    d, A, f = cfg.d, cfg.A_w, cfg.ffn

    def normal(shape, sigma, mean=0.0, dtype=torch.bfloat16):
        return (torch.randn(shape, generator=g, device=dev) * sigma + mean).to(dtype)

    blocks = [dict(g_a=normal((d,), 0.1, 1.0, torch.float32), g_f=normal((d,), 0.1, 1.0, torch.float32),
                   Wqkv=normal((3 * A, d), cfg.sigma_w), Wo=normal((d, A), cfg.sigma_w),
                   Wgate=normal((f, d), cfg.sigma_w), Wup=normal((f, d), cfg.sigma_w),
                   Wdown=normal((d, f), cfg.sigma_w)) for _ in range(K)]
    cache = {}
    run = lambda out=None: _lib.horizon_heads(inp["tokens"], inp["segment_ids"], inp["h0"], blocks, inp["W_out"],
                                              inp["g_out"], n_heads=cfg.n_heads, head_dim=cfg.head_dim, lam=cfg.lam,
                                              eps=cfg.eps, rope_theta=cfg.rope_theta, out=out, cache=cache)
    out = run()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        run(out)
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / reps
    seg = inp["segment_ids"].cpu().numpy()
    rs = run_starts(seg)
    pos = np.arange(cfg.T)[None, :]
    active = seg >= 0
    pairs = float(((pos - rs + 1) * active).sum())
    N = cfg.N
    block = (6.0 * d * A + 2.0 * A * d + 6.0 * d * f) * N + 4.0 * A * pairs
    labelled = out["counts"].cpu().numpy().astype(np.float64)
    alg = K * 3.0 * block + float(labelled.sum()) * 6.0 * d * cfg.V
    tf = alg / (ms * 1e-3) / 1e12
    del blocks, out, cache
    return {"K": K, "ms": round(ms, 4), "algorithmic_tflop": round(alg / 1e12, 3), "achieved": round(tf, 1),
            "unit": "TFLOP/s", "frac": round(tf / PEAK_BF16_TFLOPS, 4),
            "flops_basis": "per head: block forward + backward (3x the forward) + head CE 6 d V per labelled row"}


def bench_verify(torch, _lib, synth, reps=20):
    """mtp_verify on the retained-module verify workload (256 requests,
    V = 129280, gamma = 1..4): kernel time from HIP events around its
    launches; GB/s on the logit rows the decisions need (and, beside it, on
    one read of every row)."""
    dev = torch.device("cuda:0")
    res = []
    for gamma in (1, 2, 3, 4):
        vc = synth.verify_config(gamma)
        R, V = vc.R, vc.V
        g = torch.Generator(device=dev).manual_seed(1234 + gamma)
        zt32 = torch.randn((R, gamma + 1, V), generator=g, device=dev) * vc.target_sigma
        zd = (zt32[:, :gamma] + vc.draft_noise * torch.randn((R, gamma, V), generator=g, device=dev))
        zd = zd.to(torch.bfloat16)
        zt = zt32.to(torch.bfloat16)
        del zt32
        q = torch.softmax(zd.float(), dim=-1).view(-1, V)
        y = torch.multinomial(q, 1, generator=g).view(R, gamma).to(torch.int32)
        del q
        ua = torch.rand((R, gamma), generator=g, device=dev)
        us = torch.rand((R, gamma + 1), generator=g, device=dev)
        cache = {}
        out = _lib.verify(zt, zd, y, ua, us, cache=cache)
        torch.cuda.synchronize()
        with _lib.StageTimer("VERIFY", 4 * reps) as tm:
            for _ in range(reps):
                _lib.verify(zt, zd, y, ua, us, out=out, cache=cache)
            torch.cuda.synchronize()
        ts = tm.times_ms()
        ms = float(np.sum(ts)) / reps
        # bytes: every logit row once (what the kernels read for the row
        # log-sum-exps), and the rows the decision needs given the realised A
        # (target and draft rows 0..min(A, gamma-1), plus target row gamma
        # when every draft is accepted)
        A = out["accepted_len"].cpu().numpy().astype(np.int64)
        rows_needed = 2 * (np.minimum(A, gamma - 1) + 1) + (A == gamma)
        full_bytes = R * (2 * gamma + 1) * V * 2.0
        needed_bytes = float(rows_needed.sum()) * V * 2.0
        gbs = needed_bytes / (ms * 1e-3) / 1e9
        res.append({"gamma": gamma, "R": R, "V": V, "ms": round(ms, 4), "achieved": round(gbs, 1),
                    "unit": "GB/s", "frac": round(gbs / PEAK_HBM_GBS, 4), "bytes": needed_bytes,
                    "bytes_full_read": full_bytes,
                    "achieved_full_read": round(full_bytes / (ms * 1e-3) / 1e9, 1),
                    "mean_accepted": round(float(A.mean()), 3)})
        del zt, zd, y, ua, us, out, cache
    return res


def main():
    args = parse()
    if args.pmc_table:
        pmc_table(args.pmc_table[0], args.pmc_table[1])
        return
    if args.ingest_pmc:
        ingest_pmc(args.ingest_pmc[0], args.ingest_pmc[1], args.ingest_pmc[2], args.workload)
        return
    if args.gpus != 1:
        print(f"bench.py runs on one GPU; --gpus {args.gpus} is not supported (the path has no "
              "multi-GPU implementation: data-parallel sharding is a design only)", file=sys.stderr)
        sys.exit(2)
    import torch

    from deepseek_sequential_mtp_amd import _lib, synth

    cfg = synth.CHAIN_CONFIGS[args.workload]
    assert cfg.dtype == "bf16"
    print(f"[bench] workload {cfg.name}: B={cfg.B} T={cfg.T} d={cfg.d} H={cfg.n_heads}x{cfg.head_dim} "
          f"ffn={cfg.ffn} V={cfg.V} D={cfg.D}", file=sys.stderr, flush=True)
    inp = device_inputs(cfg, torch)
    if args.propose_only:
        print(json.dumps(bench_propose(torch, _lib, cfg, inp)), flush=True)
        return
    dev = inp["h0"].device
    D, N = cfg.D, cfg.N
    chain_out = dict(h=[torch.empty_like(inp["h0"]) for _ in range(D)],
                     state_mask=torch.empty((D, cfg.B, cfg.T), dtype=torch.uint8, device=dev),
                     loss_mask=torch.empty((D, cfg.B, cfg.T), dtype=torch.uint8, device=dev),
                     labels=torch.empty((D, cfg.B, cfg.T), dtype=torch.int32, device=dev),
                     counts=torch.empty((D,), dtype=torch.int32, device=dev),
                     device_error=torch.empty((1,), dtype=torch.int32, device=dev))
    ce_out = dict(loss_sum=torch.empty(D, device=dev), counts=torch.empty(D, dtype=torch.int32, device=dev),
                  loss=torch.empty(D, device=dev), loss_mtp=torch.empty(1, device=dev), lse=None,
                  dh=[torch.empty((N, cfg.d), device=dev) for _ in range(D)],
                  dW_out=torch.empty((cfg.V, cfg.d), device=dev), dg_out=torch.empty((cfg.d,), device=dev),
                  device_error=torch.empty(1, dtype=torch.int32, device=dev))
    if args.accuracy:
        ce_out.update(pred=torch.empty((D, N), dtype=torch.int32, device=dev),
                      correct=torch.empty(D, dtype=torch.int32, device=dev),
                      accuracy=torch.empty(D, device=dev))
    cache = {}

    def step():
        _lib.chain_forward(inp["tokens"], inp["segment_ids"], inp["h0"], inp["E"], inp["depths"],
                           n_heads=cfg.n_heads, head_dim=cfg.head_dim, eps=cfg.eps,
                           rope_theta=cfg.rope_theta, out=chain_out, cache=cache)
        _lib.head_ce_fwd_bwd(chain_out["h"], chain_out["labels"], inp["W_out"], inp["g_out"], lam=cfg.lam,
                             eps=cfg.eps, out=ce_out, cache=cache)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    assert int(chain_out["device_error"][0]) == 0
    if args.accuracy:
        print(f"top-1 accuracy by depth {ce_out['accuracy'].tolist()} "
              f"(correct {ce_out['correct'].tolist()} of {ce_out['counts'].tolist()})", file=sys.stderr)

    # stage pass (untimed, after the warm-up): every launch of every stage
    # carries a HIP event pair on the launch stream and its stage id; it gives
    # the stage table and picks the dominant stage (the MFMA stage with the
    # most launch time).  Events on every launch cost 0.6% of the step at V3
    # width and 10% at D=1, so they stay out of the timed region.
    prof_steps = max(3, min(args.steps, 5))
    all_timer = _lib.AllStageTimer(256 * prof_steps)
    torch.cuda.synchronize()
    with all_timer:
        for _ in range(prof_steps):
            step()
        torch.cuda.synchronize()
    launches = all_timer.by_stage()
    stage_ms = {name: float(np.sum(ts)) / prof_steps for name, ts in launches.items()}
    mfma_stages = ("EH_PROJ", "QKV", "ATTN", "O_PROJ", "GATE_UP", "DOWN", "CE_FWD", "CE_DX", "CE_DW")
    dominant = max((s_ for s_ in stage_ms if s_ in mfma_stages), key=lambda s_: stage_ms[s_])

    # timed region: only the dominant stage's launches carry event pairs, so
    # its roofline comes from launches inside the timed steps
    dom_per_step = len(launches[dominant]) // prof_steps
    timer = _lib.StageTimer(dominant, dom_per_step * args.steps)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps + 1)]
    with timer:
        ev[0].record()
        for i in range(args.steps):
            step()
            ev[i + 1].record()
        torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_step = ev[0].elapsed_time(ev[-1]) / args.steps
    per_step = [ev[i].elapsed_time(ev[i + 1]) for i in range(args.steps)]
    dom_times = timer.times_ms()
    assert timer.count == len(dom_times) == dom_per_step * args.steps, (timer.count, dom_per_step)
    dom_avg_ms = float(np.mean(dom_times))
    dom_step_ms = float(np.sum(dom_times)) / args.steps

    # work accounting from the realised packing
    sm = chain_out["state_mask"].cpu().numpy()
    counts = chain_out["counts"].cpu().numpy()
    seg = inp["segment_ids"].cpu().numpy()
    per = algorithmic_flops(cfg, sm, counts, lambda: run_starts(seg))
    keys = ("EH_PROJ", "QKV", "ATTN", "O_PROJ", "GATE_UP", "DOWN", "CE_FWD", "CE_DX", "CE_DW")
    alg_step = sum(p[k] for p in per for k in keys)
    # achieved = the stage's algorithmic FLOPs of one step / its launch time in
    # one step (the launches of a step differ in size when the last logit slab
    # is short; the ratio of the sums is their duration-weighted mean)
    dom_alg_step = float(np.sum([p[dominant] for p in per]))
    dom_note = "algorithmic FLOPs per step / summed launch time per step"
    achieved = dom_alg_step / (dom_step_ms * 1e-3) / 1e12
    tokens_s = cfg.N / (ms_step * 1e-3)
    step_frac = alg_step / (ms_step * 1e-3) / 1e12 / PEAK_BF16_TFLOPS

    traffic = None
    tfile = os.path.join(ROOT, "profiles", f"traffic_{dominant.lower()}_{cfg.name}.json")
    if os.path.exists(tfile):
        try:
            with open(tfile) as fh:
                tr = json.load(fh)
            if tr.get("source_hash") == _kernel_hash(dominant) and "bytes_per_step" in tr:
                # per launch, like `achieved`: the step's bytes over the step's launches
                traffic = round(tr["bytes_per_step"] / (len(dom_times) / args.steps))
        except (OSError, ValueError):
            traffic = None

    if args.stages:
        tot = sum(stage_ms.values())
        for k, v in sorted(stage_ms.items(), key=lambda kv: -kv[1]):
            print(f"  stage {k:12s} {v:9.3f} ms  {100 * v / tot:5.1f}%", file=sys.stderr)
        print(f"  dominant {dominant}: {dom_avg_ms:.3f} ms/launch over {len(dom_times)} launches, "
              f"{dom_step_ms:.3f} ms/step, {achieved:.1f} TFLOP/s ({dom_note})", file=sys.stderr)

    def calibration_copy():
        # a plain copy of known size: the reference dispatches that scale the
        # FETCH_SIZE / WRITE_SIZE counters (and mark the phases of the run)
        src = torch.randn(COPY_BYTES // 4, device=dev)
        dst = torch.empty_like(src)
        for _ in range(COPY_REPS):
            torch.neg(src, out=dst)
        torch.cuda.synchronize()
        del src, dst

    if args.copy_calibration:
        calibration_copy()

    stages = stage_table(cfg, stage_ms, per)
    verify = bench_verify(torch, _lib, synth)
    if args.copy_calibration:
        calibration_copy()
    if args.stages:
        for v in verify:
            print(f"  verify gamma={v['gamma']}: {v['ms']:.3f} ms, {v['achieved']:.0f} GB/s on needed rows "
                  f"({100 * v['frac']:.1f}% of HBM), {v['achieved_full_read']:.0f} GB/s on all rows, "
                  f"mean accepted {v['mean_accepted']}", file=sys.stderr)

    backward = bench_backward(torch, _lib, cfg, inp, chain_out, ce_out, per, cache)
    if args.stages:
        print(f"  chain backward: {backward['ms']:.3f} ms with saved activations, {backward['achieved']:.0f} TFLOP/s "
              f"algorithmic ({100 * backward['frac']:.1f}% of peak); {backward['ms_recompute']:.3f} ms recomputing "
              f"each depth's forward", file=sys.stderr)
        for k, v in sorted(backward["stages"].items(), key=lambda kv: -kv[1]["ms"]):
            print(f"    {k:14s} {v['ms']:9.3f} ms", file=sys.stderr)

    horizons = bench_horizons(torch, _lib, cfg, inp)
    if args.stages:
        print(f"  horizon heads K={horizons['K']}: {horizons['ms']:.3f} ms, {horizons['achieved']:.0f} TFLOP/s "
              f"({100 * horizons['frac']:.1f}% of peak)", file=sys.stderr)

    propose = bench_propose(torch, _lib, cfg, inp)
    if args.stages:
        print(f"  propose R={propose['R']} cached={propose['cached_slots']}: {propose['ms']:.3f} ms, "
              f"{propose['achieved']:.0f} GB/s ({100 * propose['frac']:.1f}% of HBM)", file=sys.stderr)

    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(cfg, args.cpu_rows)

    line = {
        "metric": "MTP train tokens/s (chain fwd + head-CE fwd/bwd) and % bf16 MFMA peak, 1 GPU",
        "value": round(tokens_s, 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "ms_per_step_median": round(float(np.median(per_step)), 4),
        "ms_per_step_min": round(float(np.min(per_step)), 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded, generated on device: Zipf(1.1) tokens, N(0,1) h0, N(0,sigma) weights)",
        "config": {"workload": cfg.name, "B": cfg.B, "T": cfg.T, "d": cfg.d, "n_heads": cfg.n_heads,
                   "head_dim": cfg.head_dim, "ffn": cfg.ffn, "V": cfg.V, "D": cfg.D, "lambda": cfg.lam,
                   "reduce": "fixed (B*T)", "parallelism": "none (1 GPU)"},
        "mfma_frac_step": round(step_frac, 4),
        "algorithmic_tflop_per_step": round(alg_step / 1e12, 3),
        "executed_tflop_per_step": round(executed_tflop(cfg, run_starts(seg)), 3),
        "wall_s_timed": round(wall, 3),
        "roofline": {"bound": "mfma", "kernel": dominant, "achieved": round(achieved, 1),
                     "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s", "frac": round(achieved / PEAK_BF16_TFLOPS, 4),
                     "traffic": traffic, "launch_ms": round(dom_avg_ms, 4),
                     "launches_per_step": len(dom_times) // args.steps, "flops_basis": dom_note},
        "stages": stages,
        "verify": verify,
        "chain_backward": backward,
        "horizon_heads": horizons,
        "propose": propose,
        "cpu_baseline": cpu,
    }
    print(json.dumps(line), flush=True)


def _kernel_hash(stage: str) -> str:
    """Hash of the sources the stage's kernel is compiled from (the GEMM
    templates and the host code that picks their tiles, slabs and splits, or
    the attention kernel), so that a stored traffic figure is dropped once
    that kernel or its launch changes."""
    import hashlib
    files = (["common.hpp", "attention.hip"] if stage == "ATTN"
             else ["common.hpp", "gemm.hpp", "epilogues.hpp", "mtp_api.hip"])
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "deepseek_sequential_mtp_amd", "csrc")
    for name in files:
        with open(os.path.join(csrc, name), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def cpu_baseline(cfg, P):
    """The oracle as it stands, on the first P positions of the workload's first
    batch row (the chain sees the same prefix context), plus its head CE with
    the labels of those rows.  tokens/s = P / wall time."""
    import threadpoolctl
    from deepseek_sequential_mtp_amd import synth
    from oracle import chain as ochain, head as ohead, rows as orows
    from oracle.numerics import BF16

    sub = synth.scaled(cfg, B=1, T=P + cfg.D + 1, seg_lo=P + cfg.D + 1, seg_hi=P + cfg.D + 1)
    print(f"[bench] cpu baseline: generating {cfg.name} weights on the host", file=sys.stderr, flush=True)
    inp = synth.make_chain_inputs(sub)
    cores = len(os.sched_getaffinity(0))
    info = threadpoolctl.threadpool_info()
    blas_threads = max([i.get("num_threads", 1) for i in info] or [1])
    t0 = time.perf_counter()
    hs = ochain.chain_forward(inp["h0"], inp["tokens"], inp["segment_ids"], inp["depths"], inp["E"],
                              sub.n_heads, sub.head_dim, sub.eps, sub.rope_theta, BF16)
    _, _, labels, _ = orows.dense_rows(inp["tokens"], inp["segment_ids"], sub.D)
    lab = labels.reshape(sub.D, -1).copy()
    lab[:, P:] = -1
    ohead.head_ce([h[:] for h in hs], lab, inp["W_out"], inp["g_out"], sub.eps, sub.lam, "fixed", float(cfg.N), BF16)
    dt = time.perf_counter() - t0
    rows = P
    return {"value": round(rows / dt, 3), "unit": "tokens/s", "cores": int(min(cores, blas_threads)),
            "kind": "oracle",
            "sample": f"{cfg.name}: first {P} positions of one row (prefix attention context), "
                      f"chain fwd + head CE fwd/bwd, float64 numpy; {dt:.1f} s"}


if __name__ == "__main__":
    main()
