"""Host-side checks of bench.py's contract and accounting (no GPU needed)."""
from __future__ import annotations

import json
import os
import subprocess
import sys
from types import SimpleNamespace

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402


def test_more_than_one_gpu_is_refused_with_a_message():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr


def test_pair_counts_reproduce_the_blog_worked_example():
    """The bench's FLOP accounting: allowed pairs of the worked shape (p = q = 32, N = 100 x 128)
    with diagonal blocks whole are the 2.46 M the blog prints; the dense square is 12,864^2."""
    with open(os.path.join(ROOT, "tests", "golden", "blog_worked_example.json")) as f:
        g = json.load(f)
    w = SimpleNamespace(prompts=[(g["p"], [g["doc_len"]] * g["n_docs"], g["q"])])
    blk, exact = bench.pair_counts(w)
    assert round(blk / 1e6, 2) == g["allowed_pairs_printed_millions"]
    L = g["p"] + g["q"] + g["n_docs"] * g["doc_len"]
    assert L == g["dense_side_printed"] and round(L * L / 1e6, 2) == g["dense_pairs_printed_millions"]
    # exact causal count: each segment's diagonal block loses its strictly-upper triangle
    n = [g["p"], g["q"]] + [g["doc_len"]] * g["n_docs"]
    assert exact == blk - sum(x * (x - 1) // 2 for x in n)


def test_batched_pair_counts_add_over_prompts():
    one = SimpleNamespace(prompts=[(32, [64, 100, 7], 16)])
    two = SimpleNamespace(prompts=[(32, [64, 100, 7], 16), (32, [64, 100, 7], 16)])
    b1, e1 = bench.pair_counts(one)
    b2, e2 = bench.pair_counts(two)
    assert (b2, e2) == (2 * b1, 2 * e1)
