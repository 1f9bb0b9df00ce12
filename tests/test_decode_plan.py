"""CPU check of the split-KV decode launch plan: every item's queries are still
in their LDS slot when the workgroup reads them.

decode_splitkv_kernel loads each item's queries into a query slot together
with the item's first tile, while the next tiles of its ring (possibly the
first tiles of later items) are already loading. tests/decode_plan_walk.cpp
includes the launcher's own plan code (csrc/decode_plan.h) and replays each
persistent workgroup's issue and read order with every load landing at issue
time, the worst case. The kernel's slot count must give no clobbered read on
any shape; two slots (an earlier layout) must, on the shapes where it raced.
"""

import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "grouped_query_attention_amd", "csrc")
SRC = os.path.join(ROOT, "tests", "decode_plan_walk.cpp")

pytestmark = pytest.mark.skipif(shutil.which("g++") is None, reason="g++ not available")


@pytest.fixture(scope="module")
def walker(tmp_path_factory):
    exe = str(tmp_path_factory.mktemp("walk") / "decode_plan_walk")
    r = subprocess.run(["g++", "-O2", "-std=c++17", "-I", CSRC, SRC, "-o", exe],
                       capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    return exe


def _run(exe, *args):
    r = subprocess.run([exe, *map(str, args)], capture_output=True, text=True, timeout=300)
    assert r.returncode == 0, r.stderr
    lines = r.stdout.strip().splitlines()
    shapes, clobbered = (int(v) for v in lines[-1].split()[1::2])
    return shapes, clobbered, lines[:-1]


# shapes with many one-tile items per workgroup (16-key chunks) and the
# workloads of the tests and the bench
SHAPES = [(6, 673), (3, 1361), (5, 817), (200, 17), (64, 8192), (1, 65536), (1, 65000),
          (3, 651), (2, 1536), (256, 1), (4096, 3)]


def test_kernel_slots_never_clobbered_listed_shapes(walker):
    args = [v for s in SHAPES for v in s]
    for n_cu in (256, 304, 80):
        shapes, bad, lines = _run(walker, "plan", n_cu, *args)
        assert shapes == len(SHAPES)
        assert bad == 0, lines


def test_kernel_slots_never_clobbered_sweep(walker):
    # every B <= 64 with every key count <= 2048 on the MI355X's 256 CUs
    shapes, bad, lines = _run(walker, "plan", 256, "sweep", 64, 2048)
    assert shapes == 64 * 2048
    assert bad == 0, lines[:10]


def test_walker_finds_the_two_slot_race(walker):
    # two alternating slots let the third item in flight overwrite the first
    # item's queries: the walker must see it on the shapes where it happened
    shapes, bad, lines = _run(walker, 2, 256, 6, 673, 3, 1361, 5, 817, 200, 17, 64, 8192)
    assert shapes == 5 and bad == 4
    assert not any("B 64 kv_len 8192" in l for l in lines)
