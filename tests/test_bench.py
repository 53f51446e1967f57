"""Host-side logic of bench.py: FLOP/byte accounting and the CLI contract."""
import json
import os
import subprocess
import sys

import numpy as np

import bench

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_flop_formula_reproduces_the_printed_recipe01_numbers():
    g = json.load(open(os.path.join(ROOT, "tests", "golden", "flop_accounting.json")))
    r = g["recipe01"]
    f = bench.attention_flops(r["B"], r["H"], r["N"], r["N"], r["d"], r["causal"])
    assert round(f / (r["flash_ms"] * 1e-3) / 1e12, 3) == r["flash_tflops_printed"]
    assert round(f / (r["naive_ms"] * 1e-3) / 1e12, 3) == r["naive_tflops_printed"]
    # the naive N x N score matrix printed as 16.0 MB (4-byte scores, MiB)
    assert round(r["N"] * r["N"] * 4 / 2 ** 20, 1) == r["score_matrix_mb_printed"]
    # causal is credited half (symmetric accounting)
    assert bench.attention_flops(2, 3, 64, 64, 64, True) == \
        g["causal_factor"] * bench.attention_flops(2, 3, 64, 64, 64, False)


def test_headline_flops():
    assert bench.attention_flops(8, 16, 4096, 4096, 64, True) == 2 * 8 * 16 * 4096 ** 2 * 64


def test_decode_bytes():
    lens = np.array([16, 17])
    H, d = 2, 8
    kv = 2 * 33 * H * d * 2
    io = 2 * H * d * 2 + 2 * H * d * 4 + 2 * H * 4 + (1 + 2) * 4 + 2 * 4
    assert bench.decode_bytes(lens, H, d) == kv + io
    assert bench.decode_bytes(lens, H, d, with_io=False) == kv


def test_more_than_one_gpu_is_refused():
    out = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                         capture_output=True, text=True)
    assert out.returncode == 2 and "one GPU" in out.stderr


def test_effective_flops_counts_the_unmasked_pairs():
    """Brute-force count of the (row, key) pairs the masks leave valid."""
    rng = np.random.default_rng(0)
    for causal in (False, True):
        for Nq, Nk in ((7, 7), (5, 9), (9, 5)):
            lens = rng.integers(0, Nk + 1, size=3)
            n = 0
            for L in lens:
                for i in range(Nq):
                    for j in range(Nk):
                        n += j < L and (not causal or j <= i + Nk - Nq)
            H, d = 2, 8
            assert bench.effective_flops(3, H, Nq, Nk, d, causal, lens) == 4.0 * H * d * n
    # no padding, causal, square: half the nominal count plus the diagonal
    assert bench.effective_flops(1, 1, 8, 8, 1, True) == 4.0 * 36


def test_launch_stats():
    st = bench.launch_stats(np.arange(1.0, 101.0))
    assert st["median_ms"] == 50.5 and st["launches"] == 100
    assert abs(st["p10_ms"] - 10.9) < 1e-9 and abs(st["p90_ms"] - 90.1) < 1e-9
