"""The measurement's own arithmetic, on the CPU: the visible-pair counts behind every
prefill FLOP figure, and the single-GPU contract of bench.py."""
import json
import os
import subprocess
import sys

import pytest
import torch

import oracle as O

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402  (after the path insert)


@pytest.mark.parametrize("kind", ["full", "sliding"])
@pytest.mark.parametrize("sq", [1, 5, 37, 600])
@pytest.mark.parametrize("pos0", [0, 3, 511, 512, 1000])
def test_prefill_pairs_equals_brute_force_count(kind, sq, pos0):
    """bench.prefill_pairs (closed form) against counting the oracle's visibility mask over
    every (query, key) of one head: queries at pos0 .. pos0 + sq - 1, keys 0 .. their end."""
    q_pos = torch.arange(sq, dtype=torch.int64) + pos0
    k_pos = torch.arange(pos0 + sq, dtype=torch.int64)
    assert bench.prefill_pairs(sq, pos0, kind) == int(O.visible(q_pos, k_pos, kind).sum())


def test_prefill_pairs_of_the_measured_configurations():
    """The per-head pair counts of the three prefill workloads, from their closed forms:
    a 32768-token sliding prefill (window 512), a 131072-token causal prefill, and the
    4096-query chunk at 1,044,480 of the 1M context."""
    w = O.WINDOW
    assert bench.prefill_pairs(32768, 0, "sliding") == w * (w + 1) // 2 + (32768 - w) * w
    assert bench.prefill_pairs(32768, 0, "sliding") == 16_646_400
    assert bench.prefill_pairs(131072, 0, "full") == 131072 * 131073 // 2 == 8_590_000_128
    assert bench.prefill_pairs(4096, 1_044_480, "full") == 4096 * 1_044_480 + 4096 * 4097 // 2
    assert bench.prefill_pairs(4096, 1_044_480, "full") == 4_286_580_736
    # Past the first window every sliding query sees exactly WINDOW keys.
    assert bench.prefill_pairs(4096, 1_044_480, "sliding") == 4096 * w


def test_flop_per_pair_counts_both_products():
    """QK^T and PV each take 2 * head_dim flops per (query, key, head)."""
    assert bench.FLOP_PER_PAIR == 2 * 2 * 256


def test_more_than_one_gpu_is_refused():
    """`bench.py --gpus N` with N > 1 prints a one-line error and exits non-zero, before
    any device work."""
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=300, cwd=ROOT)
    assert r.returncode != 0
    line = [l for l in r.stdout.splitlines() if l.startswith("{")][-1]
    rec = json.loads(line)
    assert rec["n_gpus"] == 2 and "one GPU" in rec["error"]
