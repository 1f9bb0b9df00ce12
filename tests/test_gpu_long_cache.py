"""GPU parity of a prefill chunk and a decode step whose keys run past 2^21
cached positions.

Each cached key row of one sequence is 2 KiB (8 KV heads x 128 bf16), so from
2^21 rows on a row's byte offset from the sequence base no longer fits in 32
bits. The flash kernel's K/V loads take a 64-bit tile base plus a per-lane
offset inside the tile, including the ragged last tile whose rows past the
last key are clamped; this chunk ends 37 keys into the tile after 2^21.

A 64-position chunk after 2^21 - 27 cached positions (kv_len = 2^21 + 37) is
checked on three query rows and two KV-head groups against the fp64 oracle's
definition (Grouped-query attention page, "All 13 steps": projection,
rotation, scores over every cached and new key, softmax, the weighted sum of
the values), composed from the oracle's functions. The cached keys and values
are zero: every cached key then scores 0 and adds exactly 1 to the softmax
denominator and nothing to its numerator, so H is carried by the chunk's own
64 keys, 37 of which lie past 2^21; a load that missed them (a wrapped
offset reads the zero rows near the sequence start) would change H entirely,
which the test also checks against a reference built without those keys.

With H carried by a handful of keys, the roundings of the stored Q_r, K_r and
V (one bf16 rounding each, as the kernels store them) no longer average out
over many keys: the reference applies the same single roundings to its exact
values (the block's queries are stored times log2(e)/sqrt(128)), and the
bound is the one for H out of the block.
"""

import math

import numpy as np
import pytest
import torch

import gqa_inputs as gi
import grouped_query_attention_amd as gqa
from oracle import gqa_oracle as O
from tests.gpu_util import assert_close, bf16_to_np_f64, dev, to_dev_bf16, to_dev_f32

pytestmark = pytest.mark.gpu

# H taken from the whole block: the same bound as the other chunk tests
BLOCK_H_REL, BLOCK_H_ABS = 5e-3, 4e-2


def test_chunk_keys_past_two_million():
    T = 64
    kv_len = (1 << 21) + 37
    start = kv_len - T
    print(f"[case] chunk B=1 T={T} start_pos={start} kv_len={kv_len}", flush=True)
    inp = gi.make_block_inputs(2101, 1, T)
    kc = torch.zeros((1, kv_len, 8, 128), dtype=torch.bfloat16, device=dev())
    vc = torch.zeros((1, kv_len, 8, 128), dtype=torch.bfloat16, device=dev())

    x = to_dev_bf16(inp.x)
    wq, wk, wv, wo = (to_dev_bf16(a) for a in (inp.wq, inp.wk, inp.wv, inp.wo))
    rope = to_dev_f32(gqa.rope_table(np.arange(start, start + T)))
    hb = torch.empty((1, T, 32, 128), dtype=torch.bfloat16, device=dev())
    gqa.chunk_forward(x, wq, wk, wv, wo, rope, kc, vc, start, h_out=hb)
    torch.cuda.synchronize()
    h = bf16_to_np_f64(hb)[0]                      # [T, 32, 128]
    del kc, vc
    torch.cuda.empty_cache()

    # reference: the chunk's own queries, keys and values from x, rotated at
    # their positions; the cached keys and values below start are zero
    xs = O.bf16_to_f64(inp.x[0])
    pos = np.arange(start, start + T)
    cos, sin = O.rope_cos_sin(pos, 128)
    q_r = O.rope_rotate(O.split_heads(O.project(xs, O.bf16_to_f64(inp.wq)), 32)[None], cos, sin)[0]
    k_new = O.rope_rotate(O.split_heads(O.project(xs, O.bf16_to_f64(inp.wk)), 8)[None], cos, sin)[0]
    v_new = O.split_heads(O.project(xs, O.bf16_to_f64(inp.wv)), 8)
    # the single bf16 roundings of the stored operands (queries stored scaled)
    c = 1.0 / (math.sqrt(128) * math.log(2.0))
    q_b = O.round_to_bf16(q_r * c) / c
    k_b = O.round_to_bf16(k_new)
    v_b = O.round_to_bf16(v_new)
    rows = [0, 31, T - 1]
    groups = [0, 5]
    past = (1 << 21) - start                       # chunk keys from this index on lie past 2^21

    def reference(drop_past):
        out = np.empty((len(rows), 4 * len(groups), 128))
        for gi_, grp in enumerate(groups):
            for ri, r in enumerate(rows):
                # keys 0 .. start + r: start zero keys (score 0, value 0), then the
                # chunk's keys 0 .. r (the ones past 2^21 zeroed when drop_past)
                kk = k_b[: r + 1, grp, :].copy()
                vv = v_b[: r + 1, grp, :].copy()
                if drop_past:
                    kk[past:] = 0.0
                    vv[past:] = 0.0
                s_new = (kk @ q_b[r, 4 * grp:4 * grp + 4].T).T / math.sqrt(128)
                for hh in range(4):
                    sc = np.concatenate([np.zeros(start), s_new[hh]])
                    p = O.softmax_rows(sc[None])[0]
                    out[ri, 4 * gi_ + hh] = p[start:] @ vv
        return out

    got = np.empty((len(rows), 4 * len(groups), 128))
    for gi_, grp in enumerate(groups):
        for ri, r in enumerate(rows):
            got[ri, 4 * gi_:4 * gi_ + 4] = h[r, 4 * grp:4 * grp + 4]
    want = reference(False)
    assert_close(got, want, rel=BLOCK_H_REL, mabs=BLOCK_H_ABS, what="H past 2^21 keys")
    # the rows that see keys past 2^21 are far from a result that misses them
    wrong = reference(True)
    for ri in (1, 2):
        d = np.linalg.norm(got[ri] - wrong[ri]) / np.linalg.norm(wrong[ri])
        print(f"[check] row {rows[ri]}: distance to the result without keys past 2^21 {d:.3f}",
              flush=True)
        assert d > 0.2


def test_decode_step_past_two_million():
    # one decode step of two sequences at position 2^21 + 36 in caches of
    # 2^21 + 64 rows: the new key and value go into slot 2^21 + 36 (byte offset
    # past 4 GiB from the sequence base), the second sequence starts 4 GiB
    # into the cache, and with the cached rows below zero the new key carries H
    B = 2
    S_max = (1 << 21) + 64
    start = (1 << 21) + 36
    print(f"[case] decode B={B} S_max={S_max} start_pos={start}", flush=True)
    inp = gi.make_block_inputs(2102, B, 1)
    kc = torch.zeros((B, S_max, 8, 128), dtype=torch.bfloat16, device=dev())
    vc = torch.zeros((B, S_max, 8, 128), dtype=torch.bfloat16, device=dev())
    x = to_dev_bf16(inp.x[:, 0])
    wq, wk, wv, wo = (to_dev_bf16(a) for a in (inp.wq, inp.wk, inp.wv, inp.wo))
    rope = to_dev_f32(gqa.rope_table(np.arange(start, start + 1))[0])
    hb = torch.empty((B, 32, 128), dtype=torch.bfloat16, device=dev())
    gqa.decode_forward(x, wq, wk, wv, wo, rope, kc, vc, start, h_out=hb)
    torch.cuda.synchronize()
    h = bf16_to_np_f64(hb)                          # [B, 32, 128]
    k_slot = bf16_to_np_f64(kc[:, start])           # [B, 8, 128]
    v_slot = bf16_to_np_f64(vc[:, start])
    del kc, vc
    torch.cuda.empty_cache()

    xs = O.bf16_to_f64(inp.x[:, 0])                 # [B, 4096]
    cos, sin = O.rope_cos_sin([start], 128)
    q_r = O.rope_rotate(O.split_heads(O.project(xs, O.bf16_to_f64(inp.wq)), 32)[:, None], cos, sin)[:, 0]
    k_r = O.rope_rotate(O.split_heads(O.project(xs, O.bf16_to_f64(inp.wk)), 8)[:, None], cos, sin)[:, 0]
    v = O.split_heads(O.project(xs, O.bf16_to_f64(inp.wv)), 8)
    # the slot written past 4 GiB holds the new key and value (one bf16 rounding)
    assert_close(k_slot, k_r, rel=3e-3, what="cache K slot past 2^21")
    assert_close(v_slot, v, rel=3e-3, what="cache V slot past 2^21")
    # H: start zero keys (score 0, value 0) and the new one; the decode path
    # stores Q_r unscaled, rounded once to bf16
    q_b, k_b, v_b = O.round_to_bf16(q_r), O.round_to_bf16(k_r), O.round_to_bf16(v)
    want = np.empty((B, 32, 128))
    for b in range(B):
        for hd in range(32):
            g = hd // 4
            s_new = float(q_b[b, hd] @ k_b[b, g]) / math.sqrt(128)
            # softmax over start zeros and s_new, weight of the new key
            w = 1.0 / (1.0 + start * math.exp(-s_new))
            want[b, hd] = w * v_b[b, g]
    assert_close(h, want, rel=BLOCK_H_REL, mabs=BLOCK_H_ABS, what="decode H past 2^21 keys")
