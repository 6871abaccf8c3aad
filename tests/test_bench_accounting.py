"""Host-side checks of bench.py's accounting: the algorithmic bytes and flops it
divides by a kernel's time come from the selection a step actually made, each
token counted once, and per-layer figures are weighted by how often the timed
steps ran each layer.  These run on the CPU with stand-in step objects."""
from __future__ import annotations

import subprocess
import sys
from types import SimpleNamespace

import numpy as np
import pytest

import bench
from synth import WORKLOADS


def test_attended_tokens_counts_each_token_once():
    # N = 100, B = 10: sinks [0, 5), window [80, 100); block 0 overlaps the
    # sinks, block 9 lies in the window, block 3 is selected twice, 12 is past
    # the last block and -1 is an empty entry
    rows = np.array([[0, 3, 3, 9, -1, 12]])
    assert bench.attended_tokens(100, 10, 5, 20, rows) == 10 + 10 + 20
    assert bench.attended_tokens(100, 10, 0, 0, np.array([[-1]])) == 0
    assert bench.attended_tokens(100, 10, 200, 0, np.array([[-1]])) == 100


def _step(w, idx, N, lo, hi):
    return SimpleNamespace(idx=SimpleNamespace(cpu=lambda: SimpleNamespace(numpy=lambda: idx)),
                           mem=SimpleNamespace(length=N), lo=lo, hi=hi)


def test_executed_idx_refuses_a_layer_that_never_ran():
    w = WORKLOADS["infllm_gqa_decode_128k"].scaled(n_q_heads=2, n_kv_heads=1, k=3)
    never = np.full((1, 2, 3), -1, dtype=np.int32)
    with pytest.raises(AssertionError):
        bench.executed_idx(w, _step(w, never, 4096, 1, 20))
    ran = np.array([[[4, 5, 6], [7, 8, 9]]], dtype=np.int32)
    assert bench.executed_idx(w, _step(w, ran, 4096, 1, 20)) is ran


def test_step_bytes_and_flops_follow_the_selection():
    w = WORKLOADS["infllm_gqa_decode_128k"].scaled(n_q_heads=2, n_kv_heads=1, head_dim=8, rep_dim=8, block=4, k=2,
                                                    window=4, sinks=2, n_q=3, reps_per_block=1)
    N = 40
    idx = np.array([[[1, 5], [5, 7]]], dtype=np.int32)  # the two heads share block 5
    st = _step(w, idx, N, 1, 9)
    by = bench.step_bytes(w, st)
    # union per kv head: sinks 0-1, window 36-39, blocks 1, 5, 7 -> 2 + 4 + 12 tokens
    assert by["kv"] == 18 * w.head_dim * 2 * 2
    assert by["reps"] == (9 - 1) * 1 * w.head_dim * 2
    # flops by brute force: each query j at position N - n_q + j sees the
    # tokens of its head's set at or before it
    total = 0
    for h in range(2):
        T = set(range(2)) | set(range(36, 40))
        for b in idx[0, h]:
            T |= set(range(4 * b, 4 * b + 4))
        for j in range(w.n_q):
            p = N - w.n_q + j
            total += sum(1 for t in T if t <= p)
    assert bench.step_flops(w, st) == 4.0 * w.head_dim * total


def test_weighted_follows_the_timed_steps():
    # steps 0..4 over 3 layers run layers 0, 1, 2, 0, 1
    assert bench.weighted([1.0, 2.0, 3.0], 5) == pytest.approx((1 + 2 + 3 + 1 + 2) / 5)
    out = bench.weighted([{"a": 1.0}, {"a": 3.0}], 3)
    assert out["a"] == pytest.approx((1 + 3 + 1) / 3)


def test_percentiles():
    xs = [5.0, 1.0, 3.0, 2.0, 4.0]
    assert bench.pct(xs, 0.5) == 3.0
    assert bench.pct(xs, 0.0) == 1.0 and bench.pct(xs, 1.0) == 5.0
    assert bench.pct(xs, 0.1) == pytest.approx(1.4)


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, "bench.py", "--gpus", "2"], capture_output=True, text=True, timeout=300)
    assert r.returncode != 0
    assert "one GPU" in r.stdout + r.stderr
