"""CPU-only checks of the C ABI: the library loads, exports every symbol the
header declares, and rejects bad arguments on the host before any HIP call.

No call here can reach a kernel launch: each one carries at least one
argument that the host-side validation rejects, and the fake device pointers
are never dereferenced.
"""

import ctypes
import os
import re

import numpy as np
import pytest

import grouped_query_attention_amd as gqa
from oracle import gqa_oracle as O

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "gqa.h")

OK, NULL, SHAPE, ALIGN, WORKSPACE, UNSUPPORTED, HIP, ARG, TOO_LARGE = range(9)
FAKE = 0x10000          # aligned, never dereferenced
MIS = 0x10004           # not 16-byte aligned


def _declared():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(gqa_[a-z_0-9]+)\s*\(", src)))


def test_library_exports_every_declared_symbol():
    lib = gqa.lib()
    names = _declared()
    assert len(names) >= 11
    for n in names:
        assert hasattr(lib, n), n
    assert sorted(gqa.exported_symbols()) == names


def test_status_strings_and_dims():
    lib = gqa.lib()
    for s in range(9):
        assert lib.gqa_status_string(s).decode().startswith("GQA_")
    assert lib.gqa_status_string(99).decode() == "GQA_ERR_UNKNOWN"
    assert gqa.dims() == (4096, 32, 8, 128)


def test_rope_table_matches_oracle_trig():
    pos = np.array([0, 1, 2, 127, 2047, 8191, 131071], dtype=np.int32)
    tab = gqa.rope_table(pos, 500000.0)
    c, s = O.rope_cos_sin(pos, 128, 500000.0)
    assert tab.shape == (7, 64, 2) and tab.dtype == np.float32
    assert np.max(np.abs(tab[..., 0] - c)) < 1e-7
    assert np.max(np.abs(tab[..., 1] - s)) < 1e-7
    assert np.array_equal(tab[0, :, 0], np.ones(64, np.float32))
    lib = gqa.lib()
    assert lib.gqa_rope_table(None, -1, 500000.0, None) == SHAPE
    assert lib.gqa_rope_table(None, 3, 1.0, None) == SHAPE
    assert lib.gqa_rope_table(None, 3, 500000.0, None) == NULL
    assert lib.gqa_rope_table(None, 0, 500000.0, None) == OK


def test_rope_table_from_frequencies():
    pos = np.array([0, 3, 8191, 100000], dtype=np.int32)
    w = O.rope_frequencies(128) / np.linspace(1.0, 8.0, 64)
    tab = gqa.rope_table(pos, omega=w)
    c, s = O.rope_cos_sin(pos, 128, omega=w)
    assert np.max(np.abs(tab[..., 0] - c)) < 1e-7 and np.max(np.abs(tab[..., 1] - s)) < 1e-7
    # the plain frequencies give the theta table
    assert np.array_equal(gqa.rope_table(pos, omega=O.rope_frequencies(128)), gqa.rope_table(pos))
    lib = gqa.lib()
    bad = np.full(64, np.nan)
    assert lib.gqa_rope_table_freqs(pos.ctypes.data, 4, bad.ctypes.data, tab.ctypes.data) == ARG
    assert lib.gqa_rope_table_freqs(pos.ctypes.data, 4, None, tab.ctypes.data) == NULL
    assert lib.gqa_rope_table_freqs(pos.ctypes.data, -1, w.ctypes.data, tab.ctypes.data) == SHAPE


def test_workspace_sizes():
    M = 8 * 4096   # enough query tiles: no balanced-attention partials, no split reduction
    want = sum(((M * f * 2 + 255) // 256) * 256 for f in (4096, 1024, 1024, 4096))
    # plus a class byte per 64x64 tile of an explicit mask (64 x 64 tiles)
    assert gqa.prefill_workspace_bytes(8, 4096) == want + 64 * 64
    assert gqa.prefill_workspace_bytes(0, 5) == 0
    # few query tiles, causal: fp32 partials of the cut query tiles; the prefill
    # workspace covers them; plain launches need none
    att = gqa.attention_workspace_bytes(1, 2048, 2048, True)
    assert att > 0 and att % (8 * (4 * 64 * 128 + 2 * 4 * 64) * 4) == 0
    assert gqa.prefill_workspace_bytes(1, 2048) >= 2048 * 10240 * 2 + att
    # non-causal: the explicit mask's tile classes, one byte per 64x64 tile
    assert gqa.attention_workspace_bytes(1, 2048, 2048, False) == 32 * 32
    assert gqa.attention_workspace_bytes(1, 100, 100, False) == 256   # 2 x 2 tiles, rounded
    assert gqa.attention_workspace_bytes(1, 1100, 1100, False) == 512  # 18 rows of 18 (+2 pad) tiles
    assert gqa.attention_workspace_bytes(8, 4096, 4096, True) == 0
    assert gqa.attention_workspace_bytes(1, 128, 128, True) == 0
    # M <= 64 tokens: the projections' split-reduction partials (4 x M x 6144 fp32)
    assert gqa.prefill_workspace_bytes(2, 30) >= 60 * 10240 * 2 + 4 * 60 * 6144 * 4
    # decode: Q_r and H (bf16 [B][4096] each) plus at least one fp32 partial
    # (O[4][128], max[4], sum[4]) per (sequence, KV head); more keys never need less
    for B in (1, 3, 64):
        need = 2 * B * 4096 * 2 + B * 8 * (4 * 128 + 8) * 4
        sizes = [gqa.decode_workspace_bytes(B, S) for S in (1, 64, 1000, 8192, 131072)]
        assert all(sz >= need for sz in sizes)
        assert sizes == sorted(sizes)
    assert gqa.decode_workspace_bytes(0, 10) == 0


def test_decode_plan_512_items():
    # The split-KV launch plans 512 (sequence, head half, key chunk) items (two
    # per CU): 256 chunks per sequence at B = 1, 128 at B = 2, one chunk when
    # the cache is a single 16-key tile. The workspace holds the larger of the
    # attention partials (O[4][128], max[4], sum[4] fp32 per KV head and chunk)
    # and the projections' split-K partials (4 x B x 6144 fp32), which share it.
    part = 8 * (4 * 128 + 8) * 4
    for B, chunks in ((1, 256), (2, 128)):
        small = max(B * part, 4 * B * 6144 * 4)
        assert (gqa.decode_workspace_bytes(B, 8192) - gqa.decode_workspace_bytes(B, 16)
                == B * chunks * part - small)


def _fwd(**kw):
    a = dict(x=FAKE, wq=FAKE, wk=FAKE, wv=FAKE, wo=FAKE, rope=FAKE, mask=None, causal=1,
             B=1, T=128, kv=128, out=FAKE, h=None, ws=FAKE, wsb=1 << 40, stream=None)
    a.update(kw)
    return gqa.lib().gqa_block_forward(a["x"], a["wq"], a["wk"], a["wv"], a["wo"], a["rope"],
                                       a["mask"], a["causal"], a["B"], a["T"], a["kv"], a["out"],
                                       a["h"], a["ws"], a["wsb"], a["stream"])


@pytest.mark.parametrize("kw,want", [
    (dict(x=None), NULL), (dict(wo=None), NULL), (dict(out=None), NULL), (dict(rope=None), NULL),
    (dict(B=0), SHAPE), (dict(T=0), SHAPE), (dict(kv=0), SHAPE), (dict(B=1 << 20, T=1 << 20), SHAPE),
    (dict(kv=64), UNSUPPORTED), (dict(causal=1, mask=FAKE), ARG), (dict(causal=2), ARG),
    (dict(x=MIS), ALIGN), (dict(wk=MIS), ALIGN), (dict(h=MIS), ALIGN), (dict(causal=0, mask=MIS), ALIGN),
    (dict(ws=None), WORKSPACE), (dict(wsb=1024), WORKSPACE), (dict(ws=MIS), ALIGN),
])
def test_block_forward_rejects(kw, want):
    assert _fwd(**kw) == want


def _dec(**kw):
    a = dict(x=FAKE, wq=FAKE, wk=FAKE, wv=FAKE, wo=FAKE, rope=FAKE, kc=FAKE, vc=FAKE, B=64,
             S=8192, sp=8191, out=FAKE, h=None, ws=FAKE, wsb=1 << 40, stream=None)
    a.update(kw)
    return gqa.lib().gqa_decode_forward(a["x"], a["wq"], a["wk"], a["wv"], a["wo"], a["rope"],
                                        a["kc"], a["vc"], a["B"], a["S"], a["sp"], a["out"],
                                        a["h"], a["ws"], a["wsb"], a["stream"])


@pytest.mark.parametrize("kw,want", [
    (dict(kc=None), NULL), (dict(x=None), NULL), (dict(wq=None), NULL),
    (dict(sp=8192), SHAPE), (dict(sp=-1), SHAPE), (dict(B=0), SHAPE), (dict(S=0), SHAPE),
    (dict(vc=MIS), ALIGN), (dict(out=MIS), ALIGN),
    (dict(ws=None), WORKSPACE), (dict(wsb=100), WORKSPACE),
])
def test_decode_forward_rejects(kw, want):
    assert _dec(**kw) == want


def _dec_static(**kw):
    a = dict(x=FAKE, wq=FAKE, wk=FAKE, wv=FAKE, wo=FAKE, rope=FAKE, kc=FAKE, vc=FAKE, B=64,
             S=8192, sp=8191, out=FAKE, h=None, stream=None)
    a.update(kw)
    return gqa.lib().gqa_decode_forward_static(a["x"], a["wq"], a["wk"], a["wv"], a["wo"],
                                               a["rope"], a["kc"], a["vc"], a["B"], a["S"],
                                               a["sp"], a["out"], a["h"], a["stream"])


# every check runs before the first HIP call (the scratch lookup), so these
# return without touching a GPU; B = 1024 needs more than the 32 MiB array
@pytest.mark.parametrize("kw,want", [
    (dict(kc=None), NULL), (dict(x=None), NULL), (dict(wo=None), NULL), (dict(rope=None), NULL),
    (dict(sp=8192), SHAPE), (dict(sp=-1), SHAPE), (dict(B=0), SHAPE), (dict(S=0), SHAPE),
    (dict(vc=MIS), ALIGN), (dict(out=MIS), ALIGN), (dict(h=MIS), ALIGN),
    (dict(B=1024), TOO_LARGE), (dict(B=1 << 16, S=4, sp=3), TOO_LARGE),
])
def test_decode_forward_static_rejects(kw, want):
    assert _dec_static(**kw) == want


def test_static_scratch_holds_every_batch_up_to_256():
    # the no-allocation decode entry accepts exactly the requests whose
    # workspace fits its fixed array; the header promises every B <= 256 at any
    # cache length (the split-KV partials are bounded by the 512-item plan)
    assert gqa.STATIC_SCRATCH_BYTES == 32 << 20
    for B in range(1, 257):
        for S in (1, 17, 4096, 8192, 65536, 1 << 20):
            assert gqa.decode_workspace_bytes(B, S) <= gqa.STATIC_SCRATCH_BYTES, (B, S)
    assert gqa.decode_workspace_bytes(1024, 8192) > gqa.STATIC_SCRATCH_BYTES


def _chk(**kw):
    a = dict(x=FAKE, wq=FAKE, wk=FAKE, wv=FAKE, wo=FAKE, rope=FAKE, kc=FAKE, vc=FAKE, B=2,
             T=16, S=64, sp=48, out=FAKE, h=None, ws=FAKE, wsb=1 << 40, stream=None)
    a.update(kw)
    return gqa.lib().gqa_chunk_forward(a["x"], a["wq"], a["wk"], a["wv"], a["wo"], a["rope"],
                                       a["kc"], a["vc"], a["B"], a["T"], a["S"], a["sp"],
                                       a["out"], a["h"], a["ws"], a["wsb"], a["stream"])


@pytest.mark.parametrize("kw,want", [
    (dict(kc=None), NULL), (dict(x=None), NULL), (dict(wo=None), NULL), (dict(out=None), NULL),
    (dict(sp=49), SHAPE), (dict(sp=-1), SHAPE), (dict(T=0), SHAPE), (dict(B=0), SHAPE),
    (dict(S=0), SHAPE), (dict(vc=MIS), ALIGN), (dict(h=MIS), ALIGN),
    (dict(ws=None), WORKSPACE), (dict(wsb=100), WORKSPACE), (dict(ws=MIS), ALIGN),
])
def test_chunk_forward_rejects(kw, want):
    assert _chk(**kw) == want


def test_chunk_workspace_sizes():
    # Q_r and H (bf16) plus the shared fp32 region; at start_pos 0 with enough query
    # tiles it is the prefill workspace without K_r and V
    assert gqa.chunk_workspace_bytes(8, 4096, 0) == 2 * 8 * 4096 * 4096 * 2
    assert gqa.chunk_workspace_bytes(0, 4, 0) == 0
    assert gqa.chunk_workspace_bytes(1, 4, -1) == 0
    # one position per sequence: split-K partials (4 x B x 6144 fp32)
    assert gqa.chunk_workspace_bytes(2, 1, 299) >= 2 * 2 * 4096 * 2 + 4 * 2 * 6144 * 4
    # few query tiles at an offset: the balanced plan's partials
    assert gqa.chunk_workspace_bytes(1, 1024, 512) > 2 * 1024 * 4096 * 2



def test_balanced_plan_partials_at_t2048():
    # B=1 T=2048 causal: 32 query tiles of 1..32 key tiles per KV head over 32
    # bins. The cut balances key tiles plus a fixed cost per piece, which leaves
    # bins of (19 tiles, one piece) and (14 tiles, two pieces): 14 query tiles
    # per KV head are cut in two, i.e. 28 partial slots of O[4][64][128] plus
    # max and sum per row (33280 floats) for each of the 8 KV heads.
    part = 4 * 64 * 128 + 2 * 4 * 64
    assert gqa.attention_workspace_bytes(1, 2048, 2048, True) == 28 * 8 * part * 4
    # many query tiles: the plain launch needs no workspace
    assert gqa.attention_workspace_bytes(8, 4096, 4096, True) == 0

def test_stage_entries_reject():
    lib = gqa.lib()
    assert lib.gqa_qkv_rope(FAKE, FAKE, FAKE, FAKE, FAKE, 1, 0, FAKE, FAKE, FAKE, 0, None) == SHAPE
    assert lib.gqa_qkv_rope(FAKE, FAKE, FAKE, None, FAKE, 1, 4, FAKE, FAKE, FAKE, 0, None) == NULL
    assert lib.gqa_qkv_rope(FAKE, FAKE, FAKE, FAKE, FAKE, 1, 4, MIS, FAKE, FAKE, 0, None) == ALIGN
    assert lib.gqa_qkv_rope(FAKE, FAKE, FAKE, FAKE, FAKE, 1, 4, FAKE, FAKE, FAKE, 2, None) == ARG
    assert lib.gqa_attention(FAKE, FAKE, FAKE, FAKE, 1, 1, 4, 4, FAKE, None, 0, 0, None) == ARG
    assert lib.gqa_attention(FAKE, FAKE, FAKE, None, 1, 1, 4, 4, FAKE, None, 0, 3, None) == ARG
    assert lib.gqa_attention(FAKE, FAKE, FAKE, None, 1, 1, 4, 5, FAKE, None, 0, 0, None) == UNSUPPORTED
    assert lib.gqa_attention(FAKE, FAKE, None, None, 1, 1, 4, 4, FAKE, None, 0, 0, None) == NULL
    assert lib.gqa_attention(FAKE, FAKE, FAKE, None, 1, 1, 2048, 2048, FAKE, MIS, 1 << 30, 0,
                             None) == ALIGN
    need = gqa.attention_workspace_bytes(1, 2048, 2048, True)
    assert lib.gqa_attention(FAKE, FAKE, FAKE, None, 1, 1, 2048, 2048, FAKE, FAKE, need - 1, 1,
                             None) == WORKSPACE
    assert lib.gqa_output_projection(FAKE, FAKE, 0, FAKE, None) == SHAPE
    assert lib.gqa_output_projection(FAKE, MIS, 3, FAKE, None) == ALIGN
    assert lib.gqa_decode_attention(FAKE, FAKE, FAKE, 2, 10, 11, FAKE, FAKE, 1 << 30, None) == SHAPE
    assert lib.gqa_decode_attention(FAKE, FAKE, FAKE, 2, 10, 10, FAKE, None, 0, None) == WORKSPACE


def test_prenorm_entries_reject():
    lib = gqa.lib()
    # the stage: rows, pointers, eps and alignment
    assert lib.gqa_rmsnorm(FAKE, FAKE, 1e-5, 0, FAKE, None) == SHAPE
    assert lib.gqa_rmsnorm(None, FAKE, 1e-5, 4, FAKE, None) == NULL
    assert lib.gqa_rmsnorm(FAKE, None, 1e-5, 4, FAKE, None) == NULL
    assert lib.gqa_rmsnorm(FAKE, FAKE, -1e-5, 4, FAKE, None) == ARG
    assert lib.gqa_rmsnorm(FAKE, FAKE, float("nan"), 4, FAKE, None) == ARG
    assert lib.gqa_rmsnorm(FAKE, FAKE, float("inf"), 4, FAKE, None) == ARG
    assert lib.gqa_rmsnorm(FAKE, MIS, 1e-5, 4, FAKE, None) == ALIGN
    assert lib.gqa_rmsnorm(FAKE, FAKE, 1e-5, 4, MIS, None) == ALIGN
    # the half-block forms: the gain checks come on top of the plain entry's
    blk = lambda g, eps, **kw: lib.gqa_block_forward_prenorm(
        kw.get("x", FAKE), g, eps, FAKE, FAKE, FAKE, FAKE, FAKE, None, 1, 1, kw.get("T", 128),
        kw.get("T", 128), FAKE, None, kw.get("ws", FAKE), 1 << 40, None)
    assert blk(None, 1e-5) == NULL
    assert blk(FAKE, -1.0) == ARG
    assert blk(MIS, 1e-5) == ALIGN
    assert blk(FAKE, 1e-5, x=None) == NULL
    assert blk(FAKE, 1e-5, T=0) == SHAPE
    assert blk(FAKE, 1e-5, ws=None) == WORKSPACE
    dec = lambda g, eps, sp=10: lib.gqa_decode_forward_prenorm(
        FAKE, g, eps, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 2, 16, sp, FAKE, None, FAKE,
        1 << 40, None)
    assert dec(None, 1e-5) == NULL and dec(FAKE, float("nan")) == ARG
    assert dec(FAKE, 1e-5, sp=16) == SHAPE
    chk = lambda g, eps, sp=8: lib.gqa_chunk_forward_prenorm(
        FAKE, g, eps, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 2, 8, 16, sp, FAKE, None, FAKE,
        1 << 40, None)
    assert chk(None, 1e-5) == NULL and chk(FAKE, -2.0) == ARG
    assert chk(FAKE, 1e-5, sp=9) == SHAPE


def test_mlp_entries_reject_and_sizes():
    lib = gqa.lib()
    M = 300
    need = M * 4096 * 2 + M * 14336 * 2          # x̂ and A (bf16); no split partials
    assert gqa.mlp_workspace_bytes(M) >= need
    assert gqa.mlp_workspace_bytes(M) < need + 1024
    assert gqa.mlp_workspace_bytes(60) >= 60 * (4096 + 14336) * 2 + 4 * 60 * 4096 * 4
    assert gqa.mlp_workspace_bytes(0) == 0
    f = lambda **kw: lib.gqa_mlp_forward(kw.get("x", FAKE), kw.get("w1", FAKE), FAKE, FAKE,
                                         kw.get("M", M), kw.get("out", FAKE), kw.get("a", None),
                                         kw.get("ws", FAKE), kw.get("wsb", 1 << 40), None)
    assert f(x=None) == NULL and f(w1=None) == NULL and f(out=None) == NULL
    assert f(M=0) == SHAPE and f(M=(1 << 24) + 1) == SHAPE
    assert f(x=MIS) == ALIGN and f(a=MIS) == ALIGN and f(ws=MIS) == ALIGN
    assert f(ws=None) == WORKSPACE and f(wsb=gqa.mlp_workspace_bytes(M) - 1) == WORKSPACE
    p = lambda g, eps: lib.gqa_mlp_forward_prenorm(FAKE, g, eps, FAKE, FAKE, FAKE, M, FAKE, None,
                                                   FAKE, 1 << 40, None)
    assert p(None, 1e-5) == NULL and p(FAKE, -1.0) == ARG and p(MIS, 1e-5) == ALIGN
