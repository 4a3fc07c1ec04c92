"""Host-side checks of bench.py: the one-GPU contract and the algorithmic
work it divides by (no GPU needed)."""
import os
import subprocess
import sys

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402
from deepseek_sequential_mtp_amd import synth  # noqa: E402


def test_more_than_one_gpu_is_refused_with_a_message():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr


def test_algorithmic_work_of_the_one_segment_workload():
    """V3 width, one segment of T = 4096 at depth 1: every position is a state
    row, T - 1 rows carry a label, and the causal windows hold T (T + 1) / 2
    pairs; the FLOPs are the closed forms per row."""
    cfg = synth.V3
    T, d, A, f, V = cfg.T, cfg.d, cfg.A_w, cfg.ffn, cfg.V
    state = np.ones((1, 1, T), np.uint8)
    counts = np.array([T - 1])
    per = bench.algorithmic_flops(cfg, state, counts, lambda: np.zeros((1, T), np.int64))
    p = per[0]
    assert (p["S"], p["L"], p["P"]) == (T, T - 1, T * (T + 1) // 2)
    chain = (4 * d * d + 6 * d * A + 2 * A * d + 6 * d * f) * T + 4 * A * p["P"]
    head = 6 * d * V * (T - 1)
    total = sum(v for k, v in p.items() if k not in ("S", "L", "P"))
    assert total == chain + head
    # the step's algorithmic work at this width: 31.2 TFLOP
    assert abs(total / 1e12 - 31.25) < 0.05
