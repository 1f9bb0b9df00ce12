"""The direct-to-LDS loads set M0 in inline asm without the compiler knowing.
That is only sound if nothing else in the kernels uses M0: compile every
kernel source to gfx950 assembly (CPU only) and check that each write of M0
is immediately followed by its global_load_lds, and that M0 is read nowhere
else."""

import os
import re
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "grouped_query_attention_amd", "csrc")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")


@pytest.mark.skipif(not os.path.exists(HIPCC), reason="hipcc not available")
@pytest.mark.parametrize("src", ["gemm.hip", "attention.hip"])
def test_m0_only_feeds_direct_to_lds_loads(src, tmp_path):
    out = tmp_path / (src + ".s")
    cmd = [HIPCC, "--offload-arch=gfx950", "-O3", "-std=c++17", "--cuda-device-only", "-S",
           "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
           "-I", os.path.join(ROOT, "include"), "-I", CSRC, os.path.join(CSRC, src), "-o", str(out)]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-2000:]
    lines = [l.strip() for l in out.read_text().splitlines()]
    code = [l for l in lines if l and not l.startswith((";", ".", "//")) and not l.endswith(":")]
    n_dma = 0
    for i, l in enumerate(code):
        if re.search(r"\bm0\b", l):
            assert l.startswith("s_mov_b32 m0,"), f"unexpected use of m0: {l}"
            assert code[i + 1].startswith("global_load_lds_dwordx4"), \
                f"m0 write not followed by its load: {l} / {code[i + 1]}"
            n_dma += 1
        if l.startswith("global_load_lds"):
            assert code[i - 1].startswith("s_mov_b32 m0,"), f"load without its m0 write: {l}"
    assert n_dma > 0
