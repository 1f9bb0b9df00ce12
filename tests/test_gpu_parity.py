"""GPU parity: the HIP path through the C ABI against the fp64 oracle.

Tolerance for Δ (fp32 output, bf16 inputs, fp32 accumulation): relative L2
error <= 5e-3 and max abs error <= 2e-2 against the oracle. bf16 stage
outputs (Q_r, K_r, V, H) are each one bf16 rounding away from exact, so they
are held to relL2 <= 3e-3 (the rounding alone gives ~1e-3) and the same max
abs bound when checked as a stage on exact inputs; H taken out of the whole
block gets relL2 <= 5e-3 and max abs <= 4e-2. Long configurations are checked on sampled rows that the oracle
evaluates one by one.
"""

import os

import numpy as np
import pytest
import torch

import gqa_inputs as gi
import grouped_query_attention_amd as gqa
from oracle import gqa_oracle as O
from tests.gpu_util import (assert_close, bf16_to_np_f64, dev, f32_to_np_f64, to_dev_bf16,
                            to_dev_f32)

pytestmark = pytest.mark.gpu

STAGE_REL = 3e-3
# H taken from the whole block carries the upstream Q_r/K_r/V and P roundings
# as well as its own: Δ's relative bound, and about two bf16 ulps at |H| ~ 4.
BLOCK_H_REL, BLOCK_H_ABS = 5e-3, 4e-2


def _weights(inp):
    return [to_dev_bf16(a) for a in (inp.wq, inp.wk, inp.wv, inp.wo)]


def _rope(T, start=0):
    return to_dev_f32(gqa.rope_table(np.arange(start, start + T)))


def _prefill(inp, causal=True, mask=None, h=False):
    x = to_dev_bf16(inp.x)
    wq, wk, wv, wo = _weights(inp)
    B, T = inp.x.shape[:2]
    h_out = torch.empty((B, T, 32, 128), dtype=torch.bfloat16, device=dev()) if h else None
    m = None if mask is None else to_dev_f32(mask)
    out = gqa.block_forward(x, wq, wk, wv, wo, _rope(T), causal=causal, mask=m, h_out=h_out)
    torch.cuda.synchronize()
    return out, h_out


# --- stages -----------------------------------------------------------------------------

@pytest.mark.parametrize("B,T", [(1, 128), (2, 129), (1, 1), (3, 64)])
def test_qkv_rope_stage(B, T):
    print(f"[case] qkv_rope B={B} T={T}", flush=True)
    inp = gi.make_block_inputs(100 + T, B, T)
    x = to_dev_bf16(inp.x)
    wq, wk, wv, _ = _weights(inp)
    q_r, k_r, v = gqa.qkv_rope(x, wq, wk, wv, _rope(T))
    torch.cuda.synchronize()
    ref = O.block_forward(inp.x, inp.wq, inp.wk, inp.wv, inp.wo, 32, 8)
    assert_close(bf16_to_np_f64(q_r), ref["q_r"], rel=STAGE_REL, what="Q_r")
    assert_close(bf16_to_np_f64(k_r), ref["k_r"], rel=STAGE_REL, what="K_r")
    assert_close(bf16_to_np_f64(v), ref["v"], rel=STAGE_REL, what="V")


@pytest.mark.parametrize("T", [2048, 3000, 4096])
def test_qkv_rope_stage_wide_tiles_sampled(T):
    # 2048 <= M <= 4096 runs 256-token x 192-feature tiles; T = 3000 leaves a
    # ragged last token tile. The oracle projects and rotates sampled rows only
    # (tile edges included); every feature column of those rows is compared.
    print(f"[case] qkv_rope wide tiles B=1 T={T} (sampled rows)", flush=True)
    inp = gi.make_block_inputs(200 + T, 1, T)
    x = to_dev_bf16(inp.x)
    wq, wk, wv, _ = _weights(inp)
    q_r, k_r, v = gqa.qkv_rope(x, wq, wk, wv, _rope(T))
    torch.cuda.synchronize()
    edges = [0, 255, 256, 2047, T - 257, T - 256, T - 1]
    rows = np.unique(np.concatenate([edges, np.random.Generator(np.random.PCG64(T)).integers(0, T, 24)]))
    xr = O.bf16_to_f64(inp.x[0, rows])
    cos, sin = O.rope_cos_sin(rows, 128)
    want_q = O.rope_rotate(O.split_heads(O.project(xr, O.bf16_to_f64(inp.wq)), 32)[None], cos, sin)[0]
    want_k = O.rope_rotate(O.split_heads(O.project(xr, O.bf16_to_f64(inp.wk)), 8)[None], cos, sin)[0]
    want_v = O.split_heads(O.project(xr, O.bf16_to_f64(inp.wv)), 8)
    sel = torch.from_numpy(rows).to(dev())
    assert_close(bf16_to_np_f64(q_r[0, sel]), want_q, rel=STAGE_REL, what=f"Q_r T={T}")
    assert_close(bf16_to_np_f64(k_r[0, sel]), want_k, rel=STAGE_REL, what=f"K_r T={T}")
    assert_close(bf16_to_np_f64(v[0, sel]), want_v, rel=STAGE_REL, what=f"V T={T}")


def test_qkv_rope_stage_scaled_queries():
    # q_scaled: the queries come out multiplied by log2(e)/sqrt(128) before their
    # one rounding; keys and values are unchanged bit for bit
    B, T = 2, 200
    print(f"[case] qkv_rope q_scaled B={B} T={T}", flush=True)
    inp = gi.make_block_inputs(140, B, T)
    x = to_dev_bf16(inp.x)
    wq, wk, wv, _ = _weights(inp)
    q0, k0, v0 = gqa.qkv_rope(x, wq, wk, wv, _rope(T))
    q1, k1, v1 = gqa.qkv_rope(x, wq, wk, wv, _rope(T), q_scaled=True)
    torch.cuda.synchronize()
    assert torch.equal(k0, k1) and torch.equal(v0, v1)
    ref = O.block_forward(inp.x, inp.wq, inp.wk, inp.wv, inp.wo, 32, 8)
    c = np.log2(np.e) / np.sqrt(128.0)
    assert_close(bf16_to_np_f64(q1), ref["q_r"] * c, rel=STAGE_REL, mabs=STAGE_REL,
                 what="log2(e)/sqrt(128) Q_r")


@pytest.mark.parametrize("B,T,causal", [(1, 300, True), (2, 200, False), (1, 1000, True)])
def test_attention_stage_scaled_queries(B, T, causal):
    # queries given times log2(e)/sqrt(128); the oracle takes the exact
    # pre-scaled bf16 values divided by that factor
    print(f"[case] attention q_scaled B={B} T={T} causal={causal}", flush=True)
    q, k, v = _qkv_direct(900 + T, B, T)
    c = np.log2(np.e) / np.sqrt(128.0)
    qs = gi.f32_to_bf16_bits((O.bf16_to_f64(q) * c).astype(np.float32))
    h = gqa.attention(to_dev_bf16(qs), to_dev_bf16(k), to_dev_bf16(v), causal=causal,
                      q_scaled=True)
    torch.cuda.synchronize()
    mask = O.causal_mask(T) if causal else None
    want = O.grouped_attention(O.bf16_to_f64(qs) / c, O.bf16_to_f64(k), O.bf16_to_f64(v), mask)
    assert_close(bf16_to_np_f64(h), want, rel=STAGE_REL, what="H (scaled queries)")


@pytest.mark.parametrize("B,T", [(2, 300), (1, 1000)])
def test_stage_entries_with_scaled_queries_reproduce_the_block(B, T):
    # above 256 tokens the block runs exactly the kernels of its three stage
    # entries (q_scaled = 1; the balanced attention plan at T = 1000): same bits
    print(f"[case] stages vs block B={B} T={T}", flush=True)
    inp = gi.make_block_inputs(150 + T, B, T)
    x = to_dev_bf16(inp.x)
    wq, wk, wv, wo = _weights(inp)
    rope = _rope(T)
    hb = torch.empty((B, T, 32, 128), dtype=torch.bfloat16, device=dev())
    out = gqa.block_forward(x, wq, wk, wv, wo, rope, causal=True, h_out=hb)
    q, k, v = gqa.qkv_rope(x, wq, wk, wv, rope, q_scaled=True)
    h = gqa.attention(q, k, v, causal=True, q_scaled=True)
    o2 = gqa.output_projection(h, wo).view(B, T, 4096)
    torch.cuda.synchronize()
    assert torch.equal(h, hb)
    assert torch.equal(o2, out)


# M = 3000: 128x256 tiles with a ragged last token tile; 4096 and 4100: 256x256
# tiles (the second with a ragged last tile)
@pytest.mark.parametrize("M", [1, 300, 1024, 3000, 4096, 4100])
def test_output_projection_stage(M):
    print(f"[case] out_proj M={M}", flush=True)
    rng = np.random.Generator(np.random.PCG64(7 + M))
    hbits = gi.normal_bf16(rng, (M, 4096), 1.0)
    wbits = gi.normal_bf16(rng, (4096, 4096), 0.02)
    out = gqa.output_projection(to_dev_bf16(hbits), to_dev_bf16(wbits))
    torch.cuda.synchronize()
    want = O.project(O.bf16_to_f64(hbits), O.bf16_to_f64(wbits))
    assert_close(f32_to_np_f64(out), want, rel=1e-5, mabs=1e-3, what="H·W_O")


def _qkv_direct(seed, B, T):
    rng = np.random.Generator(np.random.PCG64(seed))
    q = gi.normal_bf16(rng, (B, T, 32, 128), 1.28)
    k = gi.normal_bf16(rng, (B, T, 8, 128), 1.28)
    v = gi.normal_bf16(rng, (B, T, 8, 128), 1.28)
    return q, k, v


# (1, 513) and (1, 700) run the balanced plan (cut query tiles, ragged last
# tile); (1, 321) is a shape the plan declines because in its cost model the
# cuts would make it slower than the plain launch
@pytest.mark.parametrize("B,T,causal", [(1, 128, True), (2, 127, True), (1, 129, True),
                                        (2, 200, False), (1, 1, True), (1, 64, True),
                                        (1, 513, True), (1, 700, True), (1, 321, True)])
def test_attention_stage(B, T, causal):
    print(f"[case] attention B={B} T={T} causal={causal}", flush=True)
    q, k, v = _qkv_direct(300 + T, B, T)
    h = gqa.attention(to_dev_bf16(q), to_dev_bf16(k), to_dev_bf16(v), causal=causal)
    torch.cuda.synchronize()
    mask = O.causal_mask(T) if causal and T > 1 else None
    want = O.grouped_attention(O.bf16_to_f64(q), O.bf16_to_f64(k), O.bf16_to_f64(v), mask)
    assert_close(bf16_to_np_f64(h), want, rel=STAGE_REL, what="H")


@pytest.mark.parametrize("B,T", [(1, 1000), (1, 2048)])
def test_attention_balanced_launch(B, T):
    # few causal query tiles: cut tiles computed in pieces and merged; same
    # result as the plain launch up to fp32 summation order, bitwise repeatable
    print(f"[case] attention balanced B={B} T={T}", flush=True)
    assert gqa.attention_workspace_bytes(B, T, T, True) > 0
    q, k, v = _qkv_direct(700 + T, B, T)
    qd, kd, vd = to_dev_bf16(q), to_dev_bf16(k), to_dev_bf16(v)
    h1 = gqa.attention(qd, kd, vd, causal=True)
    h2 = gqa.attention(qd, kd, vd, causal=True)
    hp = gqa.attention(qd, kd, vd, causal=True, balanced=False)
    torch.cuda.synchronize()
    assert torch.equal(h1, h2)
    want = O.grouped_attention(O.bf16_to_f64(q), O.bf16_to_f64(k), O.bf16_to_f64(v),
                               O.causal_mask(T))
    assert_close(bf16_to_np_f64(h1), want, rel=STAGE_REL, what="H balanced")
    assert_close(bf16_to_np_f64(hp), want, rel=STAGE_REL, what="H plain")
    d = (h1.float() - hp.float()).abs().max().item()
    assert d <= 2 ** -4, d   # at most one bf16 ulp: |H| stays below 16


def test_attention_explicit_mask():
    B, T = 2, 96
    print(f"[case] attention explicit mask B={B} T={T}", flush=True)
    q, k, v = _qkv_direct(411, B, T)
    rng = np.random.Generator(np.random.PCG64(412))
    mask = rng.standard_normal((T, T)).astype(np.float32)
    mask[rng.random((T, T)) < 0.3] = -np.inf
    mask[:, 0] = 0.0                                   # every row keeps a key
    h = gqa.attention(to_dev_bf16(q), to_dev_bf16(k), to_dev_bf16(v), causal=False,
                      mask=to_dev_f32(mask))
    torch.cuda.synchronize()
    want = O.grouped_attention(O.bf16_to_f64(q), O.bf16_to_f64(k), O.bf16_to_f64(v),
                               mask.astype(np.float64))
    assert_close(bf16_to_np_f64(h), want, rel=STAGE_REL, what="H (mask)")



def test_attention_window_mask_rows_start_late():
    # sliding window of 48 keys (row i sees keys i-47 .. i, -inf elsewhere): rows
    # from 111 on have no visible key in the first key tile while their wave
    # neighbours do, so such rows meet the lazy rescale with no reference max
    # yet; their first tile must leave the running sums at zero, not NaN
    B, T, W = 1, 256, 48
    print(f"[case] attention window mask B={B} T={T} W={W}", flush=True)
    q, k, v = _qkv_direct(413, B, T)
    i = np.arange(T)[:, None]
    j = np.arange(T)[None, :]
    mask = np.where((j <= i) & (j > i - W), 0.0, -np.inf).astype(np.float32)
    h = gqa.attention(to_dev_bf16(q), to_dev_bf16(k), to_dev_bf16(v), causal=False,
                      mask=to_dev_f32(mask))
    torch.cuda.synchronize()
    got = bf16_to_np_f64(h)
    assert np.all(np.isfinite(got))
    want = O.grouped_attention(O.bf16_to_f64(q), O.bf16_to_f64(k), O.bf16_to_f64(v),
                               mask.astype(np.float64))
    assert_close(got, want, rel=STAGE_REL, what="H (window mask)")

@pytest.mark.parametrize("B,T,W", [(2, 700, 160), (1, 333, 100)])
def test_attention_structured_mask_by_tile_classes(B, T, W):
    # An explicit mask is classified per 64x64 tile when the launch has a
    # workspace (all 0: the add is skipped; all -inf: the tile is skipped or
    # its keys removed; else added element by element). A sliding window of W
    # keys has all three classes, a ragged last tile in both directions, and
    # key tiles before the window that the walk skips; query tile 1 is masked
    # whole (its rows get H = 0). Without a workspace every tile takes the
    # element-wise add: both launches must agree bit for bit, and match the
    # oracle.
    print(f"[case] attention window mask classes B={B} T={T} W={W}", flush=True)
    q, k, v = _qkv_direct(416 + T, B, T)
    i = np.arange(T)[:, None]
    j = np.arange(T)[None, :]
    mask = np.where((j <= i) & (j > i - W), 0.0, -np.inf).astype(np.float32)
    mask[64:128] = -np.inf
    qd, kd, vd, md = to_dev_bf16(q), to_dev_bf16(k), to_dev_bf16(v), to_dev_f32(mask)
    assert gqa.attention_workspace_bytes(B, T, T, False) > 0
    h_cls = gqa.attention(qd, kd, vd, causal=False, mask=md)
    h_elt = gqa.attention(qd, kd, vd, causal=False, mask=md, balanced=False)
    torch.cuda.synchronize()
    assert torch.equal(h_cls, h_elt), "tile classes must not change a bit of H"
    got = bf16_to_np_f64(h_cls)
    assert np.all(got[:, 64:128] == 0.0), "a query tile masked whole must give H = 0"
    live = np.r_[0:64, 128:T]
    ok_mask = mask.astype(np.float64)
    ok_mask[64:128, 0] = 0.0                            # any defined row; not compared
    want = O.grouped_attention(O.bf16_to_f64(q), O.bf16_to_f64(k), O.bf16_to_f64(v), ok_mask)
    assert_close(got[:, live], want[:, live], rel=STAGE_REL, what="H (window mask, classes)")


@pytest.mark.parametrize("q_scaled", [False, True])
def test_attention_mask_random_tile_classes(q_scaled):
    # Each 64x64 tile of the mask drawn at random as all 0, all -inf or N(0, 1)
    # values (T = 1000: the last tiles ragged both ways), so every class sits
    # next to every other and some query tiles see only a few key tiles, not
    # the first or last ones. Bitwise against the element-wise launch; rows
    # with a visible key against the oracle, rows with none exactly zero.
    B, T = 2, 1000
    print(f"[case] attention random tile classes B={B} T={T} q_scaled={q_scaled}", flush=True)
    q, k, v = _qkv_direct(419, B, T)
    rng = np.random.Generator(np.random.PCG64(420))
    nt = (T + 63) // 64
    cls = rng.integers(0, 3, (nt, nt)).repeat(64, 0).repeat(64, 1)[:T, :T]
    mask = np.where(cls == 0, 0.0, np.where(cls == 1, -np.inf,
                                            rng.standard_normal((T, T)))).astype(np.float32)
    c = np.log2(np.e) / np.sqrt(128.0)
    qd = gi.f32_to_bf16_bits((O.bf16_to_f64(q) * c).astype(np.float32)) if q_scaled else q
    args = (to_dev_bf16(qd), to_dev_bf16(k), to_dev_bf16(v))
    md = to_dev_f32(mask)
    h_cls = gqa.attention(*args, causal=False, mask=md, q_scaled=q_scaled)
    h_elt = gqa.attention(*args, causal=False, mask=md, q_scaled=q_scaled, balanced=False)
    torch.cuda.synchronize()
    assert torch.equal(h_cls, h_elt), "tile classes must not change a bit of H"
    got = bf16_to_np_f64(h_cls)
    dead = np.all(mask == -np.inf, axis=1)
    assert np.all(got[:, dead] == 0.0)
    live = np.nonzero(~dead)[0]
    assert len(live) > T // 2
    qo = O.bf16_to_f64(qd) / c if q_scaled else O.bf16_to_f64(q)
    want = O.grouped_attention(qo[:, live], O.bf16_to_f64(k), O.bf16_to_f64(v),
                               mask[live].astype(np.float64))
    assert_close(got[:, live], want, rel=STAGE_REL, what="H (random tile classes)")


@pytest.mark.parametrize("T", [1, 63, 65])
def test_attention_mask_classes_small_shapes(T):
    # one position (a single ragged tile), one tile short of full, one key
    # past a tile: random mask with -inf entries, key 0 kept for every row
    B = 2
    print(f"[case] attention mask classes B={B} T={T}", flush=True)
    q, k, v = _qkv_direct(430 + T, B, T)
    rng = np.random.Generator(np.random.PCG64(431 + T))
    mask = rng.standard_normal((T, T)).astype(np.float32)
    mask[rng.random((T, T)) < 0.4] = -np.inf
    mask[:, 0] = 0.0
    args = (to_dev_bf16(q), to_dev_bf16(k), to_dev_bf16(v))
    md = to_dev_f32(mask)
    h_cls = gqa.attention(*args, causal=False, mask=md)
    h_elt = gqa.attention(*args, causal=False, mask=md, balanced=False)
    torch.cuda.synchronize()
    assert torch.equal(h_cls, h_elt)
    want = O.grouped_attention(O.bf16_to_f64(q), O.bf16_to_f64(k), O.bf16_to_f64(v),
                               mask.astype(np.float64))
    assert_close(bf16_to_np_f64(h_cls), want, rel=STAGE_REL, what=f"H (mask classes, T={T})")


def test_attention_mask_classes_past_256_key_tiles():
    # The attention kernel holds a query tile's mask classes 256 key tiles at a
    # time; at T = 16484 (258 key tiles, the last ragged) the last query tiles
    # move to a second window. The mask: causal, key tiles 100 and 101 all -inf
    # (inside every later query tile's walk), a mixed tile in the second window
    # (keys 16400..16419 shifted by +0.75) and one in the first (-1.5 on
    # query tile 125, key tile 2). Bitwise against the element-wise launch
    # (no workspace); sampled rows against the oracle.
    B, T = 1, 16484
    print(f"[case] attention mask classes over two windows B={B} T={T}", flush=True)
    q, k, v = _qkv_direct(418, B, T)
    m = torch.triu(torch.full((T, T), float("-inf"), device=dev()), diagonal=1)
    m[:, 6400:6528] = float("-inf")
    m[:, 16400:16420] += 0.75
    m[8000:8064, 128:192] = -1.5
    qd, kd, vd = to_dev_bf16(q), to_dev_bf16(k), to_dev_bf16(v)
    h_cls = gqa.attention(qd, kd, vd, causal=False, mask=m)
    h_elt = gqa.attention(qd, kd, vd, causal=False, mask=m, balanced=False)
    torch.cuda.synchronize()
    assert torch.equal(h_cls, h_elt), "tile classes must not change a bit of H"
    rows = np.array([0, 6399, 6400, 8000, 8063, 16383, 16384, 16419, T - 1])
    mrows = m[torch.from_numpy(rows).to(dev())].cpu().numpy().astype(np.float64)
    del m
    torch.cuda.empty_cache()
    want = O.grouped_attention(O.bf16_to_f64(q[:, rows]), O.bf16_to_f64(k), O.bf16_to_f64(v), mrows)
    got = bf16_to_np_f64(h_cls[:, torch.from_numpy(rows).to(dev())])
    assert_close(got, want, rel=STAGE_REL, what="H (two class windows, sampled rows)")


@pytest.mark.parametrize("q_scaled", [False, True])
def test_attention_fully_masked_rows_give_zero(q_scaled):
    # A row whose every key the caller's mask removes has no defined softmax
    # (reading 9): the kernels write H = 0 for it (include/gqa.h), and every
    # other row still matches the oracle. Rows 0, 63, 64 and 199 sit at tile
    # edges and the ragged end of T = 200.
    B, T = 2, 200
    print(f"[case] attention fully masked rows B={B} T={T} q_scaled={q_scaled}", flush=True)
    q, k, v = _qkv_direct(414, B, T)
    rng = np.random.Generator(np.random.PCG64(415))
    mask = rng.standard_normal((T, T)).astype(np.float32)
    mask[rng.random((T, T)) < 0.3] = -np.inf
    mask[:, 0] = 0.0
    dead = np.array([0, 5, 63, 64, 130, 199])
    mask[dead, :] = -np.inf
    c = np.log2(np.e) / np.sqrt(128.0)
    qd = gi.f32_to_bf16_bits((O.bf16_to_f64(q) * c).astype(np.float32)) if q_scaled else q
    h = gqa.attention(to_dev_bf16(qd), to_dev_bf16(k), to_dev_bf16(v), causal=False,
                      mask=to_dev_f32(mask), q_scaled=q_scaled)
    torch.cuda.synchronize()
    got = bf16_to_np_f64(h)
    assert np.all(got[:, dead] == 0.0), "fully masked rows must be exactly zero"
    live = np.setdiff1d(np.arange(T), dead)
    ok_mask = mask.copy()
    ok_mask[dead, :] = 0.0                              # any defined row; not compared
    qo = O.bf16_to_f64(qd) / c if q_scaled else O.bf16_to_f64(q)
    want = O.grouped_attention(qo, O.bf16_to_f64(k), O.bf16_to_f64(v), ok_mask.astype(np.float64))
    assert_close(got[:, live], want[:, live], rel=STAGE_REL, what="H (live rows)")


# --- whole block ---------------------------------------------------------------------

# (2, 30): 60 tokens take the projections' split-reduction path with 64-token
# tiles (M <= 64); (1, 128) and (2, 77): 128-token x 64-feature tiles in 4
# slices (M <= 128); (2, 100): 128x128 tiles in 4 slices (M <= 256); (3, 129): unsplit
@pytest.mark.parametrize("B,T,seed", [(1, 128, 1), (2, 77, 21), (3, 129, 22), (1, 1, 23),
                                      (2, 30, 24), (2, 100, 25)])
def test_block_forward_small(B, T, seed):
    print(f"[case] block_forward B={B} T={T} seed={seed}", flush=True)
    inp = gi.make_block_inputs(seed, B, T)
    out, h = _prefill(inp, h=True)
    ref = O.block_forward(inp.x, inp.wq, inp.wk, inp.wv, inp.wo, 32, 8)
    assert_close(f32_to_np_f64(out), ref["delta"], what=f"Δ B={B} T={T}")
    assert_close(bf16_to_np_f64(h).reshape(B, T, 4096), ref["h"], rel=BLOCK_H_REL,
                 mabs=BLOCK_H_ABS, what="H")


def test_block_forward_c2_full():
    print("[case] block_forward C2 B=1 T=2048 seed=2", flush=True)
    inp = gi.make_block_inputs(2, 1, 2048)
    out, _ = _prefill(inp)
    ref = O.block_forward(inp.x, inp.wq, inp.wk, inp.wv, inp.wo, 32, 8)
    assert_close(f32_to_np_f64(out), ref["delta"], what="Δ C2")


def test_causal_flag_equals_explicit_mask_and_rerun_is_bitwise():
    print("[case] causal flag vs explicit mask T=200", flush=True)
    inp = gi.make_block_inputs(31, 1, 200)
    a, ha = _prefill(inp, causal=True, h=True)
    b, hb = _prefill(inp, causal=False, mask=O.causal_mask(200).astype(np.float32), h=True)
    c, hc = _prefill(inp, causal=True, h=True)
    assert torch.equal(ha, hb) and torch.equal(a, b)
    assert torch.equal(a, c) and torch.equal(ha, hc)


def _oracle_per_sequence(inp, keys=("delta", "h")):
    """The oracle's block_forward on each sequence of a batch, several sequences at
    a time (sequences share weights, positions and mask but are otherwise
    independent, so the batch result is the per-sequence results stacked). numpy
    releases the GIL inside its BLAS calls and array loops, so worker threads
    with two BLAS threads each keep the host cores busy."""
    import threadpoolctl
    from concurrent.futures import ThreadPoolExecutor
    B = inp.x.shape[0]
    cores = len(os.sched_getaffinity(0))
    workers = max(1, min(B, cores // 2))

    def one(b):
        r = O.block_forward(inp.x[b:b + 1], inp.wq, inp.wk, inp.wv, inp.wo, 32, 8)
        print(f"[oracle] sequence {b} done", flush=True)
        return {k: r[k][0] for k in keys}

    with threadpoolctl.threadpool_limits(2), ThreadPoolExecutor(workers) as ex:
        res = list(ex.map(one, range(B)))
    return {k: np.stack([r[k] for r in res]) for k in keys}


def test_block_forward_c3_full():
    # every row of every sequence of the batched prefill, Δ and H
    print("[case] block_forward C3 B=8 T=4096 seed=3 (all rows)", flush=True)
    B, T = 8, 4096
    inp = gi.make_block_inputs(3, B, T)
    out, h = _prefill(inp, h=True)
    out = f32_to_np_f64(out)
    hh = bf16_to_np_f64(h).reshape(B, T, 4096)
    del h
    ref = _oracle_per_sequence(inp)
    for b in range(B):
        assert_close(out[b], ref["delta"][b], what=f"Δ C3 sequence {b}")
    assert_close(out, ref["delta"], what="Δ C3 (all 8 x 4096 rows)")
    assert_close(hh, ref["h"], rel=BLOCK_H_REL, mabs=BLOCK_H_ABS, what="H C3 (all rows)")


def test_block_forward_ragged_5000_sampled():
    # M = 5000: 256x256 QKV and W_O tiles with a ragged last token tile, plain
    # (unbalanced) causal attention over 79 query tiles with a ragged tail
    print("[case] block_forward B=1 T=5000 seed=36 (sampled rows)", flush=True)
    T = 5000
    inp = gi.make_block_inputs(36, 1, T)
    out, h = _prefill(inp, h=True)
    rows = np.unique(np.concatenate([[0, 63, 64, 4095, 4096, 4991, T - 1],
                                     np.random.Generator(np.random.PCG64(37)).integers(0, T, 40)]))
    ref = O.block_forward_rows(inp.x, inp.wq, inp.wk, inp.wv, inp.wo, 32, 8, rows)
    sel = torch.from_numpy(rows).to(dev())
    assert_close(f32_to_np_f64(out[0, sel]), ref["delta"], what="Δ T=5000")
    assert_close(bf16_to_np_f64(h[0, sel]).reshape(len(rows), 4096), ref["h"], rel=BLOCK_H_REL,
                 mabs=BLOCK_H_ABS, what="H T=5000")


def test_block_forward_c5_sampled():
    print("[case] block_forward C5 B=1 T=131072 seed=5 (sampled rows)", flush=True)
    T = 131072
    inp = gi.make_block_inputs(5, 1, T)
    out, h = _prefill(inp, h=True)
    rows = gi.sample_positions(5, T)
    out = f32_to_np_f64(out[0, torch.from_numpy(rows).to(dev())])
    hh = bf16_to_np_f64(h[0, torch.from_numpy(rows).to(dev())]).reshape(len(rows), 4096)
    ref = O.block_forward_rows(inp.x, inp.wq, inp.wk, inp.wv, inp.wo, 32, 8, rows)
    assert_close(out, ref["delta"], what="Δ C5")
    assert_close(hh, ref["h"], rel=BLOCK_H_REL, mabs=BLOCK_H_ABS, what="H C5")


# --- chunked prefill into a KV cache ----------------------------------------------------

def _chunk(x_bits, inp, k_cache, v_cache, start_pos, h=False):
    """x_bits [B, T, 4096] bf16 bits; caches are device tensors (updated in place)."""
    B, T = x_bits.shape[:2]
    x = to_dev_bf16(x_bits)
    wq, wk, wv, wo = _weights(inp)
    rope = to_dev_f32(gqa.rope_table(np.arange(start_pos, start_pos + T)))
    hb = torch.empty((B, T, 32, 128), dtype=torch.bfloat16, device=dev()) if h else None
    out = gqa.chunk_forward(x, wq, wk, wv, wo, rope, k_cache, v_cache, start_pos, h_out=hb)
    torch.cuda.synchronize()
    return out, hb


# (1, 1024, 2048, 512) runs the balanced attention plan with a position offset;
# (2, 300, 1024, 700) a plan whose cut query tiles have four pieces (ragged T,
# offset not a multiple of 64); (1, 777, 1110, 333) a plan with a ragged last
# query tile; (1, 64, 2176, 2048) one query tile over 33 key tiles, whose plan
# would cut it into more pieces than the merge takes and falls back to the
# plain launch; (3, 20, 64, 44) ends exactly at S_max; (2, 1, 300, 299) is a
# one-position chunk (split-K projections).
@pytest.mark.parametrize("B,T,S_max,start_pos", [(2, 37, 256, 100), (1, 128, 128, 0),
                                                 (1, 1024, 2048, 512), (2, 300, 1024, 700),
                                                 (1, 777, 1110, 333), (1, 64, 2176, 2048),
                                                 (3, 20, 64, 44), (2, 1, 300, 299)])
def test_chunk_forward(B, T, S_max, start_pos):
    print(f"[case] chunk B={B} T={T} S_max={S_max} start_pos={start_pos}", flush=True)
    inp = gi.make_block_inputs(60 + T + start_pos, B, T, cache_len=S_max)
    kc, vc = to_dev_bf16(inp.k_cache), to_dev_bf16(inp.v_cache)
    out, h = _chunk(inp.x, inp, kc, vc, start_pos, h=True)
    ref = O.block_forward(inp.x, inp.wq, inp.wk, inp.wv, inp.wo, 32, 8, start_pos=start_pos,
                          k_cache=inp.k_cache, v_cache=inp.v_cache)
    assert_close(f32_to_np_f64(out), ref["delta"], what="Δ chunk")
    assert_close(bf16_to_np_f64(h).reshape(B, T, 4096), ref["h"], rel=BLOCK_H_REL,
                 mabs=BLOCK_H_ABS, what="H chunk")
    kc_np, vc_np = bf16_to_np_f64(kc), bf16_to_np_f64(vc)
    new = slice(start_pos, start_pos + T)
    assert_close(kc_np[:, new], ref["k_r"], rel=STAGE_REL, what="cache K slots")
    assert_close(vc_np[:, new], ref["v"], rel=STAGE_REL, what="cache V slots")
    keep = np.ones(S_max, bool)
    keep[new] = False
    assert np.array_equal(kc_np[:, keep], O.bf16_to_f64(inp.k_cache)[:, keep])
    assert np.array_equal(vc_np[:, keep], O.bf16_to_f64(inp.v_cache)[:, keep])


def test_two_chunks_equal_one_prefill():
    # a prefill of 300 positions into an empty cache, then a chunk of 200 more,
    # reproduces rows 300..499 of the causal prefill of all 500 positions
    print("[case] chunk 300 then 200 vs prefill of 500", flush=True)
    T1, T2, S_max = 300, 200, 512
    inp = gi.make_block_inputs(77, 1, T1 + T2)
    kc = torch.zeros((1, S_max, 8, 128), dtype=torch.bfloat16, device=dev())
    vc = torch.zeros_like(kc)
    _chunk(inp.x[:, :T1], inp, kc, vc, 0)
    out2, _ = _chunk(inp.x[:, T1:], inp, kc, vc, T1)
    ref = O.block_forward(inp.x, inp.wq, inp.wk, inp.wv, inp.wo, 32, 8)
    assert_close(f32_to_np_f64(out2), ref["delta"][:, T1:], what="Δ second chunk")


# --- decode ------------------------------------------------------------------------

def _decode(inp, start_pos):
    B = inp.x.shape[0]
    x = to_dev_bf16(inp.x[:, 0])
    wq, wk, wv, wo = _weights(inp)
    kc, vc = to_dev_bf16(inp.k_cache), to_dev_bf16(inp.v_cache)
    h = torch.empty((B, 32, 128), dtype=torch.bfloat16, device=dev())
    rope = to_dev_f32(gqa.rope_table([start_pos])[0])
    out = gqa.decode_forward(x, wq, wk, wv, wo, rope, kc, vc, start_pos, h_out=h)
    torch.cuda.synchronize()
    return out, h, kc, vc


# (6, 700, 672) and (3, 1400, 1360): 16-key chunks, several one-tile items per
# persistent workgroup (each item's queries must survive the ring's lookahead)
# (100, 300, 299) and (200, 64, 63): projections split in 4 slices (128x64 and
# 128x128 tiles)
@pytest.mark.parametrize("B,S_max,start_pos", [(3, 700, 650), (2, 40, 0), (1, 1024, 1023),
                                               (2, 600, 511), (6, 700, 672), (3, 1400, 1360),
                                               (100, 300, 299), (200, 64, 63)])
def test_decode_forward_small(B, S_max, start_pos):
    print(f"[case] decode B={B} S_max={S_max} start_pos={start_pos}", flush=True)
    inp = gi.make_block_inputs(40 + start_pos, B, 1, cache_len=S_max)
    out, h, kc, vc = _decode(inp, start_pos)
    ref = O.decode_forward(inp.x[:, 0], inp.wq, inp.wk, inp.wv, inp.wo, 32, 8, inp.k_cache,
                           inp.v_cache, start_pos)
    assert_close(f32_to_np_f64(out), ref["delta"], what="Δ decode")
    assert_close(bf16_to_np_f64(h).reshape(B, 4096), ref["h"], rel=BLOCK_H_REL,
                 mabs=BLOCK_H_ABS, what="H decode")
    kc_np = bf16_to_np_f64(kc)
    vc_np = bf16_to_np_f64(vc)
    assert_close(kc_np[:, start_pos], ref["k_r"], rel=STAGE_REL, what="cache K slot")
    assert_close(vc_np[:, start_pos], ref["v"], rel=STAGE_REL, what="cache V slot")
    # every other slot untouched
    keep = np.ones(S_max, bool)
    keep[start_pos] = False
    assert np.array_equal(kc_np[:, keep], O.bf16_to_f64(inp.k_cache)[:, keep])
    assert np.array_equal(vc_np[:, keep], O.bf16_to_f64(inp.v_cache)[:, keep])


def test_decode_forward_c4_full():
    print("[case] decode C4 B=64 S_max=8192 start_pos=8191 seed=4", flush=True)
    B, S, sp = 64, 8192, 8191
    inp = gi.make_block_inputs(4, B, 1, cache_len=S)
    out, h, _, _ = _decode(inp, sp)
    ref = O.decode_forward(inp.x[:, 0], inp.wq, inp.wk, inp.wv, inp.wo, 32, 8, inp.k_cache,
                           inp.v_cache, sp)
    assert_close(f32_to_np_f64(out), ref["delta"], what="Δ C4")
    assert_close(bf16_to_np_f64(h).reshape(B, 4096), ref["h"], rel=BLOCK_H_REL,
                 mabs=BLOCK_H_ABS, what="H C4")


@pytest.mark.parametrize("kv_len", [1, 31, 33, 512, 513, 1500])
def test_decode_attention_stage(kv_len):
    print(f"[case] decode_attention kv_len={kv_len}", flush=True)
    B, S = 2, 1536
    rng = np.random.Generator(np.random.PCG64(500 + kv_len))
    q = gi.normal_bf16(rng, (B, 32, 128), 1.28)
    kc = gi.normal_bf16(rng, (B, S, 8, 128), 1.28)
    vc = gi.normal_bf16(rng, (B, S, 8, 128), 1.28)
    h = gqa.decode_attention(to_dev_bf16(q), to_dev_bf16(kc), to_dev_bf16(vc), kv_len)
    torch.cuda.synchronize()
    want = O.grouped_attention(O.bf16_to_f64(q)[:, None], O.bf16_to_f64(kc)[:, :kv_len],
                               O.bf16_to_f64(vc)[:, :kv_len], None)[:, 0]
    assert_close(bf16_to_np_f64(h), want, rel=STAGE_REL, what="H decode stage")


# plans whose persistent workgroups take three or more one-tile items in a
# row: a later item's query load must not overwrite an earlier item's queries
@pytest.mark.parametrize("B,kv_len", [(6, 673), (3, 1361), (5, 817), (200, 17)])
def test_decode_attention_one_tile_items(B, kv_len):
    print(f"[case] decode_attention one-tile items B={B} kv_len={kv_len}", flush=True)
    S = kv_len + 7
    rng = np.random.Generator(np.random.PCG64(1300 + B * 7 + kv_len))
    q = gi.normal_bf16(rng, (B, 32, 128), 1.28)
    kc = gi.normal_bf16(rng, (B, S, 8, 128), 1.28)
    vc = gi.normal_bf16(rng, (B, S, 8, 128), 1.28)
    h = gqa.decode_attention(to_dev_bf16(q), to_dev_bf16(kc), to_dev_bf16(vc), kv_len)
    torch.cuda.synchronize()
    want = O.grouped_attention(O.bf16_to_f64(q)[:, None], O.bf16_to_f64(kc)[:, :kv_len],
                               O.bf16_to_f64(vc)[:, :kv_len], None)[:, 0]
    assert_close(bf16_to_np_f64(h), want, rel=STAGE_REL, what=f"H decode B={B} kv_len={kv_len}")


@pytest.mark.parametrize("kv_len", [65536, 65000])
def test_decode_attention_long_context(kv_len):
    # one sequence over a long cache: the launch plans 256 key chunks of 256
    # keys (two head halves each, 512 items); 65000 leaves a short last chunk
    print(f"[case] decode_attention B=1 kv_len={kv_len}", flush=True)
    B, S = 1, 65536
    rng = np.random.Generator(np.random.PCG64(900 + kv_len))
    q = gi.normal_bf16(rng, (B, 32, 128), 1.28)
    kc = gi.normal_bf16(rng, (B, S, 8, 128), 1.28)
    vc = gi.normal_bf16(rng, (B, S, 8, 128), 1.28)
    h = gqa.decode_attention(to_dev_bf16(q), to_dev_bf16(kc), to_dev_bf16(vc), kv_len)
    torch.cuda.synchronize()
    want = O.grouped_attention(O.bf16_to_f64(q)[:, None], O.bf16_to_f64(kc)[:, :kv_len],
                               O.bf16_to_f64(vc)[:, :kv_len], None)[:, 0]
    assert_close(bf16_to_np_f64(h), want, rel=STAGE_REL, what=f"H decode B=1 kv_len={kv_len}")


def test_decode_matches_prefill_row():
    print("[case] decode vs prefill row p=300", flush=True)
    p = 300
    inp = gi.make_block_inputs(50, 2, p + 1)
    full, _ = _prefill(inp)
    # cache from the library's own projection of tokens 0..p-1
    wq, wk, wv, wo = _weights(inp)
    x = to_dev_bf16(inp.x)
    _, k_r, v = gqa.qkv_rope(x[:, :p].contiguous(), wq, wk, wv, _rope(p))
    S = 512
    kc = torch.zeros((2, S, 8, 128), dtype=torch.bfloat16, device=dev())
    vc = torch.zeros_like(kc)
    kc[:, :p] = k_r
    vc[:, :p] = v
    rope = to_dev_f32(gqa.rope_table([p])[0])
    out = gqa.decode_forward(x[:, p].contiguous(), wq, wk, wv, wo, rope, kc, vc, p)
    torch.cuda.synchronize()
    ref = O.block_forward(inp.x, inp.wq, inp.wk, inp.wv, inp.wo, 32, 8)["delta"][:, p]
    assert_close(f32_to_np_f64(out), ref, what="decode row p")
    assert_close(f32_to_np_f64(out), f32_to_np_f64(full[:, p]), what="decode vs prefill")


# --- rotation tables from explicit frequencies -------------------------------------------

def _rescaled_omega():
    # a long-context style table: low-frequency pairs divided by up to 8 (a
    # synthetic ramp; the kernels apply whatever table they are given)
    return O.rope_frequencies(128) / np.linspace(1.0, 8.0, 64)


def test_block_forward_rescaled_table():
    print("[case] block_forward B=2 T=300 rescaled frequencies", flush=True)
    B, T = 2, 300
    w = _rescaled_omega()
    inp = gi.make_block_inputs(41, B, T)
    wq, wk, wv, wo = _weights(inp)
    rope = to_dev_f32(gqa.rope_table(np.arange(T), omega=w))
    out = gqa.block_forward(to_dev_bf16(inp.x), wq, wk, wv, wo, rope)
    torch.cuda.synchronize()
    ref = O.block_forward(inp.x, inp.wq, inp.wk, inp.wv, inp.wo, 32, 8, omega=w)
    assert_close(f32_to_np_f64(out), ref["delta"], what="Δ rescaled table")
    plain = O.block_forward(inp.x, inp.wq, inp.wk, inp.wv, inp.wo, 32, 8)["delta"]
    assert np.linalg.norm(plain - ref["delta"]) > 0.05 * np.linalg.norm(plain)


def test_chunk_forward_rescaled_table_far_positions():
    # positions 20000 .. 20063 over 20000 cached ones, past the 8192 positions of
    # the unscaled catalogue entry's context
    print("[case] chunk B=1 T=64 start_pos=20000 rescaled frequencies", flush=True)
    B, T, sp = 1, 64, 20000
    w = _rescaled_omega()
    inp = gi.make_block_inputs(42, B, T, cache_len=sp + T)
    wq, wk, wv, wo = _weights(inp)
    kc, vc = to_dev_bf16(inp.k_cache), to_dev_bf16(inp.v_cache)
    rope = to_dev_f32(gqa.rope_table(np.arange(sp, sp + T), omega=w))
    out = gqa.chunk_forward(to_dev_bf16(inp.x), wq, wk, wv, wo, rope, kc, vc, sp)
    torch.cuda.synchronize()
    ref = O.block_forward(inp.x, inp.wq, inp.wk, inp.wv, inp.wo, 32, 8, start_pos=sp,
                          k_cache=inp.k_cache, v_cache=inp.v_cache, omega=w)
    assert_close(f32_to_np_f64(out), ref["delta"], what="Δ chunk rescaled")
    assert_close(bf16_to_np_f64(kc)[:, sp:], ref["k_r"], rel=STAGE_REL, what="cache K rescaled")
