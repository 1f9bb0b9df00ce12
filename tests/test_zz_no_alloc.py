"""GPU check of gqa_decode_forward_static, the decode entry that allocates
nothing: it must return what gqa_decode_forward (with a caller workspace)
returns, bit for bit, on two calls in a row, the second smaller than the
first (the fixed scratch array then holds the first call's contents)."""

import numpy as np
import pytest
import torch

import gqa_inputs as gi
import grouped_query_attention_amd as gqa
from tests.gpu_util import assert_close, dev, f32_to_np_f64, to_dev_bf16, to_dev_f32

pytestmark = pytest.mark.gpu


def _case(seed, B, S_max, start_pos):
    inp = gi.make_block_inputs(seed, B, 1, cache_len=S_max)
    x = to_dev_bf16(inp.x[:, 0])
    w = [to_dev_bf16(a) for a in (inp.wq, inp.wk, inp.wv, inp.wo)]
    rope = to_dev_f32(gqa.rope_table([start_pos])[0])
    kc, vc = to_dev_bf16(inp.k_cache), to_dev_bf16(inp.v_cache)
    return x, w, rope, kc, vc


def _both(seed, B, S_max, start_pos):
    print(f"[case] decode_forward_static B={B} S_max={S_max} start_pos={start_pos}", flush=True)
    x, w, rope, kc, vc = _case(seed, B, S_max, start_pos)
    kc2, vc2 = kc.clone(), vc.clone()
    h_ref = torch.empty((B, 32, 128), dtype=torch.bfloat16, device=dev())
    ref = gqa.decode_forward(x, *w, rope, kc, vc, start_pos, h_out=h_ref)
    out = torch.empty((B, 4096), dtype=torch.float32, device=dev())
    h = torch.empty_like(h_ref)
    torch.cuda.synchronize()
    before = torch.cuda.memory_allocated()
    gqa.decode_forward_static(x, *w, rope, kc2, vc2, start_pos, out=out, h_out=h)
    after = torch.cuda.memory_allocated()
    torch.cuda.synchronize()
    assert after == before
    assert_close(f32_to_np_f64(out), f32_to_np_f64(ref), what=f"Δ static vs workspace B={B}")
    assert torch.equal(out, ref)
    assert torch.equal(h, h_ref)
    assert torch.equal(kc2, kc) and torch.equal(vc2, vc)


def test_static_decode_matches_workspace_entry_twice():
    # the decode workload's shape first, then a smaller call whose 16-key chunks
    # give several one-tile items per workgroup
    _both(4, 64, 8192, 8191)
    _both(44, 6, 700, 672)
