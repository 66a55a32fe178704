"""Host logic of bench.py (no GPU): the algorithmic byte model behind every reported GB/s and
roofline figure, and the code hash that ties the committed traffic counters to the kernels."""
from __future__ import annotations

import os
import sys

import pytest

sys.path.insert(0, os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
import bench  # noqa: E402


def _valid(T, K):
    # a quarter of the routes absent, as the generators draw them
    return T * K - (T * K) // 4


# (T, H, K, entry, extra kwargs, bytes): reads = valid rows + route metadata (int32 index and
# float32 scale) + shared + residual + gamma; writes = residual_out + norm_out (finalize only: its
# output; quantized: residual_out + codes + block scales with the 128x4 padding), worked out by
# hand for the decode workloads.
CASES = [
    (4, 1024, 8, "rmsnorm", {}, 84_224),
    (1, 6144, 8, "rmsnorm", {}, 135_232),
    (4, 6144, 8, "rmsnorm", {}, 504_064),
    (16, 6144, 8, "rmsnorm", {}, 1_979_392),
    (32, 7168, 8, "rmsnorm", {}, 4_603_904),
    (64, 7168, 8, "rmsnorm", {}, 9_193_472),
    (128, 7168, 8, "rmsnorm", {}, 18_372_608),
    (1, 2048, 22, "finalize", {"shared": False}, 73_904),
    (32, 2048, 22, "finalize", {"shared": False}, 2_299_392),
    (1, 3584, 16, "finalize", {"shared": False}, 93_312),
    (32, 3584, 16, "finalize", {"shared": False}, 2_985_984),
    (64, 6144, 8, "quant", {"quant": "nvfp4", "norm_out": False}, 7_340_032),
    (64, 6144, 8, "quant", {"quant": "fp8", "norm_out": False}, 7_487_488),
    (64, 6144, 8, "rmsnorm", {}, 7_880_704),
]


@pytest.mark.parametrize("T,H,K,entry,kw,want", CASES)
def test_algorithmic_bytes(T, H, K, entry, kw, want):
    shared = kw.pop("shared", True)
    assert bench.algorithmic_bytes(T, H, K, _valid(T, K), 4, shared, entry, **kw) == want


def test_headline_bytes_split():
    """The headline's reads and writes add up to its algorithmic bytes; the writes are the two
    [T, H] bf16 outputs."""
    T, H, K = 128, 7168, 8
    total = bench.algorithmic_bytes(T, H, K, _valid(T, K))
    reads = bench._read_bytes(T, H, K, _valid(T, K))
    assert total - reads == 2 * T * H * 2


def test_code_hash_ignores_comments_only():
    a = "int f(int x) {  // the sum\n  return x + 1; /* one */ }\n"
    b = "int f(int x) {\n  // a different comment\n  return x + 1;\n}\n"
    c = "int f(int x) { return x + 2; }\n"
    assert bench._code_only(a) == bench._code_only(b)
    assert bench._code_only(a) != bench._code_only(c)
    assert len(bench.kernel_source_hash()) >= 16


@pytest.mark.parametrize("steps", [1, 2, 19, 20, 95, 96, 97, 192, 960, 3201])
@pytest.mark.parametrize("warmup", [0, 1, 5, 96, 320])
def test_timing_plan_is_graph_replays_only(steps, warmup):
    """The headline's timed region is one replay of a graph of exactly `steps` calls for every
    steps >= 1 (no eager remainder), over the input copies in the order the warm-up graph read
    them, and the warm-up makes at least `warmup` calls."""
    n_sets = 96
    plan = bench.timing_plan(steps, warmup, n_sets)
    assert plan["eager_calls"] == 0
    assert plan["timed_replays"] == 1 and plan["timed_calls"] == steps
    assert len(plan["timed_sets"]) == steps
    assert plan["timed_sets"][:min(steps, n_sets)] == list(range(min(steps, n_sets)))
    assert all(0 <= i < n_sets for i in plan["timed_sets"])
    # every timed call reads a copy whose previous read was n_sets calls earlier (cold rotation:
    # the other n_sets - 1 copies were read in between)
    pre = plan["upload_replay_sets"] + plan["warmup_sets"] * plan["warmup_replays"]
    seq = pre + plan["timed_sets"]
    last = {}
    for pos, i in enumerate(seq):
        if pos >= len(pre):
            assert pos - last[i] == n_sets
        last[i] = pos
    assert plan["upload_replay_sets"] == plan["timed_sets"]
    assert plan["warmup_calls"] >= max(warmup, 1)
    assert plan["warmup_calls"] == steps + plan["warmup_replays"] * n_sets


def test_timing_plan_rejects_empty_runs():
    with pytest.raises(ValueError):
        bench.timing_plan(0, 5, 96)


def test_more_than_one_gpu_is_refused():
    """The path runs on one GPU: --gpus above 1 prints one JSON error line and exits with 2,
    before touching any device."""
    import json
    import subprocess
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    r = subprocess.run([sys.executable, os.path.join(root, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=300)
    assert r.returncode == 2
    line = json.loads(r.stdout.strip().splitlines()[-1])
    assert line["n_gpus"] == 2 and "one GPU" in line["error"]
