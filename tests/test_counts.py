"""Pins for the work/traffic counting used by the bench (no GPU)."""

import json
import os

import pytest

from mla_speculative_decode_verify_amd import roofline as R

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
pytestmark = pytest.mark.cpu


def test_counting_convention_reproduces_page_estimate():
    g = json.load(open(os.path.join(GOLDEN, "page1_fma_budget.json")))
    wl = g["workload"]
    n = wl["prefix"] + wl["q_len"]
    c = R.verify_counts(wl["q_len"], wl["heads"], [n] * wl["streams"], mask="causal")
    fma = c["flops"] / 2
    assert 0.97 < fma / g["fma_estimate"] < 1.06
    ideal_ms = c["flops"] / (g["fp32_tflops"] * 1e12) * 1e3
    assert abs(ideal_ms - g["theoretical_ms"]) / g["theoretical_ms"] < 0.05
    assert round(g["measured_ms"] / g["theoretical_ms"]) in (g["gap_factor"], g["gap_factor"] + 3)


def test_counts_by_hand():
    # q_len 2, H 1, prefix 3: causal visible pairs = 2*3 + (1 + 2) = 9
    c = R.verify_counts(2, 1, [5], mask="causal")
    assert c["pairs"] == 9 and c["flops"] == 2 * 1088 * 9
    assert c["bytes"] == 5 * (1152 + 4) + 2 * (1152 + 2048 + 4) + 4
    # tree [-1, 0, -1]: depths 1, 2, 1
    c = R.verify_counts(3, 2, [7], mask="tree", parents=[[-1, 0, -1]])
    assert c["pairs"] == 2 * (3 * 4 + 4)
    c = R.verify_counts(3, 2, [7], mask="none")
    assert c["pairs"] == 2 * 3 * 7
    s = R.sparse_counts(32, 1, 64, 2048)
    assert s["bytes"] == 32 * 2048 * 652 + 32 * 64 * (1152 + 2048 + 4) + 32 * 4


def test_bench_table_fixture_consistent():
    rows = [l.split() for l in open(os.path.join(GOLDEN, "page1_bench_table.txt")) if l.strip() and l[0] != "#"]
    for r in rows:
        naive, flash, sp = float(r[3]), float(r[4]), float(r[5])
        if sp == sp:
            assert abs(naive / flash - sp) < 0.06


def test_bench_refuses_more_than_one_gpu():
    # the path runs on one GPU: any other count exits at once with a message
    import subprocess
    import sys
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    for argv, env in ((["--gpus", "2"], {}), (["--gpus", "1"], {"WORLD_SIZE": "8"})):
        e = dict(os.environ, **env)
        r = subprocess.run([sys.executable, os.path.join(root, "bench.py")] + argv,
                           capture_output=True, text=True, timeout=60, env=e)
        assert r.returncode == 2, r.stderr
        assert "one GPU only" in r.stderr
        assert r.stdout == ""
