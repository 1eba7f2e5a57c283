"""Host-side checks of bench.py (no GPU): the one-GPU guard, the algorithmic
byte count behind the roofline figure, and the CPU-baseline record."""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402
from block_sparse_kv_stats_amd import synth  # noqa: E402


def test_more_than_one_gpu_exits_with_a_message():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout == ""


def test_step_bytes_counted_by_hand():
    """One unit, d = 64, r = 4, 1024 tokens after the append (64 blocks, the
    last one holding 16 tokens), budget 128 tokens (8 blocks):
      closed before the step: 63 blocks, each k̄ + D̄ + |b| = (64 + 4 + 1) * 4 = 276 B
      kept: 8 blocks, one of them the block the token lands in, so 7 closed ones;
      v̄ of the 63 - 7 = 56 unkept closed blocks: 56 * 64 * 4 B
      append: 15 cached tokens read and the new one written (K and V, BF16),
              the block's summary row written: (2 * 64 + 4 + 1) * 4 B
      attend: the kept blocks' tokens, 8 * 16 tokens of K and V in BF16."""
    w = synth.WORKLOADS["tiny"]
    assert (w.S, w.H, w.d, w.r, w.budget) == (1, 1, 64, 4, 128)
    score, attend = bench.step_bytes(w, 1024)
    append = 15 * 2 * 64 * 2 + 2 * 64 * 2 + (2 * 64 + 4 + 1) * 4
    assert score == 63 * 276 + 56 * 64 * 4 + append
    assert attend == 8 * 16 * 2 * 64 * 2


def test_step_bytes_partial_open_block():
    """1030 tokens after the append: 65 blocks, the open one holding 6; the
    8 kept blocks include it, so 7 of the 64 closed blocks are kept."""
    w = synth.WORKLOADS["tiny"]
    score, attend = bench.step_bytes(w, 1030)
    append = 5 * 2 * 64 * 2 + 2 * 64 * 2 + (2 * 64 + 4 + 1) * 4
    assert score == 64 * 276 + (64 - 7) * 64 * 4 + append
    assert attend == (7 * 16 + 6) * 2 * 64 * 2


def test_cpu_baseline_record():
    w = synth.WORKLOADS["tiny"]
    rec = bench.cpu_baseline(w, 0.3, pool=False)
    assert rec["kind"] == "oracle" and rec["cores"] == 1 and rec["unit"] == "steps/s"
    assert rec["value"] > 0
    assert "steps over the 1 (sequence, KV head) units" in rec["sample"]
    assert rec["host_cpu_count"] == os.cpu_count()


def test_cpu_baseline_pool_record():
    """Two units, one spawned process each, released together."""
    w = synth.WORKLOADS["tiny"].replace(H=2)
    rec = bench.cpu_baseline(w, 0.6)
    assert rec["cores"] == min(2, bench.host_cpu()["usable"])
    assert rec["value"] > 0 and rec["single_thread_steps_per_s"] > 0
    assert "one spawned process per unit" in rec["sample"]


def test_ragged_step_bytes_sum_over_sequences():
    w = synth.WORKLOADS["tiny"].replace(S=2, prefill=(1023, 1029))
    s2, a2 = bench.step_bytes(w, [1024, 1030])
    s0, a0 = bench.step_bytes(w, 1024)
    s1, a1 = bench.step_bytes(w, 1030)
    assert (s2, a2) == ((s0 + s1) // 2, (a0 + a1) // 2)
    assert bench.dense_bytes(w, [1024, 1030]) == (1024 + 1030) * 2 * 64 * 2


def test_timed_regions_start_at_the_least_recently_used_layer():
    b = bench.Bench.__new__(bench.Bench)
    b.R, b.cursor = 5, 0
    warm = b.order(3)
    timed = b.order(4)
    assert warm == [0, 1, 2] and timed == [3, 4, 0, 1]
    assert b.order(1) == [2]
