"""bench.py's contract on the host: the one-GPU guard and the algorithmic
counts its throughput and roofline figures divide by (no GPU needed)."""

import json
import os
import subprocess
import sys

import bench

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_exits_with_a_message():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120, cwd=ROOT)
    assert r.returncode != 0
    line = json.loads(r.stdout.strip().splitlines()[-1])
    assert line["n_gpus"] == 2 and "one GPU" in line["error"]


def test_prefill_flops_by_hand():
    # projections: 2 flops per weight per token; attention: 4 * 32 * 128 per
    # unmasked (query, key) pair (Q·K and P·V, 32 heads of width 128)
    T = 2048
    proj = 2 * T * (4096 * 4096 * 2 + 1024 * 4096 * 2)
    pairs = T * (T + 1) // 2
    assert bench.prefill_flops(1, T) == proj + 4 * 32 * 128 * pairs == 206175207424
    # a chunk after cached positions attends to all of them as well
    assert bench.prefill_flops(1, 2048, 2048) - bench.prefill_flops(1, 2048) == 4 * 32 * 128 * 2048 * 2048
    stages = bench.stage_flops(1, T)
    assert sum(stages.values()) == bench.prefill_flops(1, T)


def test_decode_bytes_by_hand():
    # B=64, 8192 cached rows (8191 old + the new one): weights, old K/V rows,
    # the new K/V row, x (bf16), Δ (fp32), one rotation row (64 pairs of fp32)
    B, S = 64, 8192
    weights = 2 * (4096 * 4096 * 2 + 1024 * 4096 * 2)
    kv = B * (S - 1) * 8 * 128 * 2 * 2
    assert bench.decode_bytes(B, S) == weights + kv + B * 1024 * 4 + B * 4096 * 6 + 512 == 2232943104


def test_sampled_rows_flops_by_hand():
    # K and V of every position; Q and the W_O product of each sampled row;
    # row t attends to t + 1 keys
    T, rows = 1000, [0, 5, 999]
    kv = 2 * T * (1024 * 4096 * 2)
    qo = 2 * 3 * (4096 * 4096 * 2)
    att = 4 * 32 * 128 * (1 + 6 + 1000)
    assert bench.rows_flops(T, rows) == kv + qo + att


def test_headline_is_the_largest_workload():
    # the line quotes the largest single-GPU prefill workload; every other
    # workload has its own entry
    sizes = {n: w[1] * w[2] for n, w in bench.WORKLOADS.items() if w[0] == "prefill"}
    assert bench.HEADLINE == max(sizes, key=sizes.get)
    assert {w[0] for w in bench.WORKLOADS.values()} == {"prefill", "decode"}
