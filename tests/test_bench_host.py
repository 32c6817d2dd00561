"""Host logic of the benchmark (no GPU): work accounting, the paired-batch
ratio and its classification at the 5% practical threshold, the 80-shape
grid recipe, and the one-GPU guard."""
import importlib.util
import math
import os
import subprocess
import sys

import numpy as np
import pytest

import synth

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _bench():
    spec = importlib.util.spec_from_file_location("bench_mod", os.path.join(ROOT, "bench.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


bench = _bench()


def _batches(rng, median, n_batches=10, n=30, spread=0.01):
    return [list(median * (1 + spread * rng.standard_normal(n))) for _ in range(n_batches)]


def test_paired_ratio_classifies_clear_win_loss_and_tie():
    rng = np.random.default_rng(5)
    fast = _batches(rng, 10e-6)
    slow = _batches(rng, 20e-6)
    near = _batches(rng, 10.2e-6)
    win = bench.paired_ratio(slow, fast)
    assert win["cls"] == "win" and abs(win["ratio"] - 2.0) < 0.02
    loss = bench.paired_ratio(fast, slow)
    assert loss["cls"] == "loss" and abs(loss["ratio"] - 0.5) < 0.01
    tie = bench.paired_ratio(near, fast)
    assert tie["cls"] == "tie"
    for r in (win, loss, tie):
        lo, hi = r["ci95"]
        assert lo <= r["ratio"] <= hi


def test_paired_ratio_threshold_is_five_percent():
    # a constant 4% gap is real but below the practical threshold: a tie;
    # a constant 6% gap clears it
    base = [[1.0] * 30 for _ in range(10)]
    assert bench.paired_ratio([[1.04] * 30] * 10, base)["cls"] == "tie"
    assert bench.paired_ratio([[1.06] * 30] * 10, base)["cls"] == "win"
    assert bench.paired_ratio([[1 / 1.06] * 30] * 10, base)["cls"] == "loss"


def test_paired_ratio_uses_batch_medians():
    # one wild sample per batch does not move a median of 30
    base = [[1.0] * 29 + [100.0] for _ in range(10)]
    cand = [[0.5] * 30 for _ in range(10)]
    assert bench.paired_ratio(base, cand)["ratio"] == pytest.approx(2.0)


def test_row_accounting_counts_compulsory_bytes_and_macs():
    wl = synth.WORKLOADS["c3a_grouped_g64"]
    a = bench.row_accounting(wl, 64, 64)
    x = 32 * 256 * 64 * 64
    assert a["bytes"] == 4 * (x + 256 * 4 * 9 + x)
    assert a["flops"] == 2 * x * 4 * 9
    assert a["bound"] == "hbm"
    c4 = bench.row_accounting(synth.WORKLOADS["c4_dense_5x9"], 252, 248)
    assert c4["flops"] == 92154101760 and c4["bound"] == "mfma"


def test_grid_recipe():
    g = synth.ATLAS_GRID
    assert len(g) == 80
    seeds = {wl.seed for wl in g.values()}
    assert len(seeds) == 80
    for wl in g.values():
        assert (wl.R, wl.S, wl.stride, wl.pad, wl.dil) == (3, 3, 1, 1, 1)
        assert wl.C == wl.K and wl.C % wl.groups == 0 and wl.H == wl.W
        cpg = wl.C // wl.groups
        assert cpg in synth.ATLAS_CPG
        assert wl.w_dist == ("uniform", -1 / math.sqrt(9 * cpg), 1 / math.sqrt(9 * cpg))
    small = g["g3_n1_c64_14x14_cpg4"]
    inp = synth.make_inputs(small)
    assert inp["x"].shape == (1, 64, 14, 14) and inp["w"].shape == (64, 4, 3, 3)
    assert inp["x"].min() >= -1 and inp["x"].max() < 1


def test_bench_refuses_more_than_one_gpu():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2 and "one GPU" in r.stderr
