"""CPU check of the causal prefill launch plan against what the kernels assume.

Causal launches with few query tiles run a host-made plan: per (sequence, KV
head) the key tiles of all query tiles are cut into bins, one workgroup per
bin, and the pieces of cut query tiles are merged by flash_merge_kernel.
tests/flash_plan_walk.cpp includes the launcher's own plan code
(csrc/flash_plan.h) and checks every plan it makes: table bounds, entries
inside each tile's causal key range, each query tile's key tiles covered
exactly once, cut tiles with one merge record of at most four pieces in
consecutive slots, and, in the plan's own cost model, no plan slower than the
plain launch (the walker times the plain launch with its own list scheduler).
A plan with one key tile taken away must be flagged every time.
"""

import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "grouped_query_attention_amd", "csrc")
SRC = os.path.join(ROOT, "tests", "flash_plan_walk.cpp")

pytestmark = pytest.mark.skipif(shutil.which("g++") is None, reason="g++ not available")

# offsets of the prefill chunk: none, ragged, one tile, several, long caches
OFFSETS = [0, 1, 63, 64, 100, 333, 700, 2048, 4096, 30000]


@pytest.fixture(scope="module")
def walker(tmp_path_factory):
    exe = str(tmp_path_factory.mktemp("walk") / "flash_plan_walk")
    r = subprocess.run(["g++", "-O2", "-std=c++17", "-I", CSRC, SRC, "-o", exe],
                       capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    return exe


def _run(exe, *args):
    r = subprocess.run([exe, *map(str, args)], capture_output=True, text=True, timeout=300)
    assert r.returncode == 0, r.stderr
    lines = r.stdout.strip().splitlines()
    f = lines[-1].split()
    return int(f[1]), int(f[3]), int(f[5]), float(f[7]), lines[:-1]


# the planned shapes of the GPU tests and the bench (B, T, q_pos0)
LISTED = [(1, 1000, 0), (1, 2048, 0), (1, 1024, 512), (2, 300, 700), (1, 777, 333),
          (1, 64, 2048), (1, 513, 0), (1, 2048, 2048), (2, 1024, 0)]


def test_listed_shapes_keep_the_kernel_rules(walker):
    shapes, planned, broken, worst, lines = _run(walker, "plan", *[v for s in LISTED for v in s])
    assert shapes == len(LISTED)
    assert planned == len(LISTED) - 1   # (1, 64, 2048) would need 7 pieces: plain launch
    assert broken == 0, lines
    assert worst < 1.0


def test_sweep_keeps_the_kernel_rules(walker):
    # every B <= 64 and T <= 4200 (all launches with under two workgroups per CU)
    shapes, planned, broken, worst, lines = _run(walker, "plan", "sweep", 64, 4200, *OFFSETS)
    assert shapes == 64 * 4200 * len(OFFSETS)
    assert planned > 10000
    assert broken == 0, lines[:20]
    assert worst < 1.0


def test_a_missing_key_tile_is_flagged(walker):
    shapes, planned, broken, _, lines = _run(walker, "drop", "sweep", 64, 4200, 0, 333)
    assert planned > 1000
    assert broken == planned


def test_library_sizes_the_same_plan(walker):
    # the library's own compiled plan (through its workspace query) against the
    # header the walker includes: planned exactly when the walker plans, with
    # one fp32 partial per slot, sequence and KV head
    gqa = pytest.importorskip("grouped_query_attention_amd")
    try:
        gqa.lib()
    except Exception as e:   # library not built in this checkout
        pytest.skip(f"libgqa not loadable: {e}")
    shapes = [(1, 2048), (1, 1000), (1, 700), (1, 513), (1, 321), (2, 1024), (2, 300),
              (3, 777), (1, 4032), (8, 4096), (1, 128), (4, 900), (7, 520)]
    *_, lines = _run(walker, "info", *[v for B, T in shapes for v in (B, T, 0)])
    got = {}
    for ln in lines:
        f = ln.split()
        if f[0] == "info":
            got[(int(f[1]), int(f[2]))] = (int(f[4]), int(f[5]))
    part = 4 * 64 * 128 + 2 * 4 * 64   # floats per piece partial per (sequence, KV head)
    for B, T in shapes:
        planned, slots = got[(B, T)]
        want = slots * B * 8 * part * 4 if planned else 0
        assert gqa.attention_workspace_bytes(B, T, T, True) == want, (B, T)
