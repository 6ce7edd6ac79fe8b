"""The benchmark's counting rules, checked on the CPU: the algorithmic pair and flop counts that
bench.py and the workloads divide by (4·d per (query, key) pair of the window, per query head) against
the oracle's own mask, a brute-force count and the headline figure of 0.9621 TFLOP per 16K chunk;
the tile-level (executed) count against a brute-force walk of the kernel's tile schedule; and the
one-GPU guard of the command line."""
import os
import subprocess
import sys

import numpy as np
import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402
from oracle import attention as A  # noqa: E402


def brute_pairs(n, w, pos0):
    return sum(hi - lo for lo, hi in (A.key_range(pos0 + r, w) for r in range(n)))


@pytest.mark.parametrize("n,w,pos0", [(1, 1, 0), (7, 3, 0), (64, 64, 0), (100, 32, 5), (257, 100, 300),
                                      (300, 1, 1000), (500, 4096, 0), (129, 128, 128)])
def test_swa_pairs_closed_form(n, w, pos0):
    assert bench.swa_pairs(n, w, pos0) == brute_pairs(n, w, pos0)
    if pos0 == 0:
        assert bench.swa_pairs(n, w, 0) == A.mask_nonzeros(n, w)


def test_headline_flops():
    """16K chunk, w = 4096, 32 q heads, d = 128: 58,722,304 (query, key) pairs per head,
    0.9621 TFLOP."""
    pairs = bench.swa_pairs(16384, 4096)
    assert pairs == 58_722_304
    assert 4 * 128 * 32 * pairs == A.attention_flops(16384, 0, 4096, 32, 128)
    assert abs(4 * 128 * 32 * pairs / 1e12 - 0.9621) < 1e-4


def test_workload_flops_agree():
    import long_context_swa_amd.workloads as W
    for n, pos0, w in ((16384, 0, 128), (16384, 1 << 20, 128), (300, 17, None), (16384, 16384, None)):
        assert W.flops_prefill(n, pos0, w, hq=32, d=128) == A.attention_flops(n, pos0, w, 32, 128), (n, pos0, w)


def test_executed_flops_walk_the_tile_schedule():
    """Every 64-key tile a 256-row block's band touches, masked parts and padding rows included."""
    rng = np.random.default_rng(5)
    for _ in range(20):
        n, w = int(rng.integers(1, 3000)), int(rng.integers(1, 5000))
        hq, hkv, d = 32, int(rng.choice([1, 2, 4, 8, 16, 32])), 128
        P = 256 // (hq // hkv)
        tiles = 0
        for i0 in range(0, n, P):
            i1 = min(i0 + P, n) - 1
            keys = set()
            for i in range(i0, i1 + 1):
                lo, hi = A.key_range(i, w)
                keys.update(range(lo, hi))
            tiles += len({k // 64 for k in keys})
        assert bench.prefill_executed_flops(n, w, hq, hkv, d) == hkv * tiles * 4 * d * 256 * 64, (n, w, hkv)


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=300)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
