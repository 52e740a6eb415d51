"""Host-side contract of bench.py (no GPU): the timed region covers exactly
--steps calls, runs on more than one GPU are refused with a message, and the
KV byte count behind the reported rate is the cache size of the workload."""

import os
import subprocess
import sys

import numpy as np
import pytest

from conftest import ROOT

sys.path.insert(0, ROOT)
import bench  # noqa: E402


@pytest.mark.parametrize("rotate", [1, 2, 4, 8])
def test_graph_plan_times_exactly_the_requested_steps(rotate):
    for steps in range(1, 400):
        calls, reps, rem = bench.graph_plan(steps, rotate)
        assert calls * reps + rem == steps, (steps, rotate, calls, reps, rem)
        if calls:
            # the main graph cycles through whole buffer sets; the remainder is shorter than one cycle
            assert calls % rotate == 0 and calls <= 16 and reps >= 1
            assert rem < rotate
        else:
            assert reps == 0 and rem == steps < rotate


def test_graph_plan_gives_five_replays_whenever_it_can():
    # percentiles are reported only with at least 5 replays of the main graph:
    # the plan picks such a graph whenever one divides the step count
    for rotate in (1, 2, 4):
        for steps in range(5 * rotate, 400):
            calls, reps, rem = bench.graph_plan(steps, rotate)
            possible = [c for c in range(rotate, 17, rotate) if steps % c == 0 and steps // c >= 5]
            if possible:
                assert rem == 0 and calls == max(possible) and reps >= 5
    # the default run: 200 calls as 25 replays of 8 calls
    assert bench.graph_plan(200, 4) == (8, 25, 0)


def test_more_than_one_gpu_is_refused_with_a_message():
    env = dict(os.environ, WORLD_SIZE="1")
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], cwd=ROOT, env=env,
                       stdout=subprocess.PIPE, stderr=subprocess.PIPE, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout == ""  # no JSON line


def test_kv_bytes_are_the_cache_size():
    # 32 sequences x 4096 rows x (K + V) x 256 channels: 2 bytes each in bf16,
    # 1 in e4m3, 4 in fp32
    lengths = np.full(32, 4096)
    assert bench._kv_bytes(lengths, "bf16") == 32 * 4096 * 2 * 256 * 2 == 134_217_728
    assert bench._kv_bytes(lengths, "fp8_e4m3") == 32 * 4096 * 2 * 256
    assert bench._kv_bytes(lengths, "f32") == 32 * 4096 * 2 * 256 * 4
    assert bench._kv_bytes([0, 1, 7], "bf16") == 8 * 1024
