"""HIP graph capture of the block's entry points (through torch.cuda.CUDAGraph).

The library allocates nothing, never synchronises and issues no memset or
copy: a call is a fixed sequence of kernel launches on the caller's stream,
with every table it needs (the balanced attention plan included) passed by
value in the kernel arguments. A serving loop can therefore capture one block
step and replay it. Each replay here follows eager work on the same device
(the outputs are cleared in between) and must reproduce the eager result bit
for bit: every kernel reduces in a fixed order.
"""

import numpy as np
import pytest
import torch

import gqa_inputs as gi
import grouped_query_attention_amd as gqa
from tests.gpu_util import dev, to_dev_bf16, to_dev_f32

pytestmark = pytest.mark.gpu


def _check_replays(step, outs, replays=3):
    step()
    torch.cuda.synchronize()
    want = [o.clone() for o in outs]
    # warm-up on a side stream, then capture (torch's recipe; default priority)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step()
    torch.cuda.synchronize()
    a = torch.randn(512, 512, device=dev())
    for i in range(replays):
        for o in outs:
            o.zero_()
        b = a @ a                       # unrelated eager work between replays
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.isfinite(b).all()
        for o, w in zip(outs, want):
            assert torch.equal(o, w), f"replay {i} differs from the eager call"


def test_graph_replay_block_forward_balanced_plan():
    # B=1 T=1024 causal: the balanced launch (plan in the kernel arguments) + merge
    B, T = 1, 1024
    print(f"[case] graph replay block_forward B={B} T={T}", flush=True)
    inp = gi.make_block_inputs(41, B, T)
    x = to_dev_bf16(inp.x)
    w = [to_dev_bf16(m) for m in (inp.wq, inp.wk, inp.wv, inp.wo)]
    rope = to_dev_f32(gqa.rope_table(np.arange(T)))
    out = torch.empty((B, T, 4096), dtype=torch.float32, device=dev())
    h = torch.empty((B, T, 32, 128), dtype=torch.bfloat16, device=dev())
    ws = torch.empty(gqa.prefill_workspace_bytes(B, T), dtype=torch.uint8, device=dev())
    _check_replays(lambda: gqa.block_forward(x, *w, rope, causal=True, out=out, h_out=h,
                                             workspace=ws), [out, h])


def test_graph_replay_decode_forward():
    # split-K projections, split-KV attention and both merges; the call also
    # writes the new K/V row into the cache (the same values on every replay)
    B, S_max, sp = 4, 300, 200
    print(f"[case] graph replay decode_forward B={B} S_max={S_max} start_pos={sp}", flush=True)
    inp = gi.make_block_inputs(42, B, 1, cache_len=S_max)
    x = to_dev_bf16(inp.x[:, 0])
    w = [to_dev_bf16(m) for m in (inp.wq, inp.wk, inp.wv, inp.wo)]
    kc, vc = to_dev_bf16(inp.k_cache), to_dev_bf16(inp.v_cache)
    rope = to_dev_f32(gqa.rope_table([sp])[0])
    out = torch.empty((B, 4096), dtype=torch.float32, device=dev())
    ws = torch.empty(gqa.decode_workspace_bytes(B, S_max), dtype=torch.uint8, device=dev())
    _check_replays(lambda: gqa.decode_forward(x, *w, rope, kc, vc, sp, out=out, workspace=ws),
                   [out])


def test_graph_replay_mlp_split_launch():
    # M = 2048: the gate/up product runs as two launches (three whole rounds of
    # 256x256 tiles, then the last 4096 features on 256x128 tiles) before the
    # down product; the hidden activation is an output too
    M = 2048
    print(f"[case] graph replay mlp_forward M={M}", flush=True)
    m = gi.make_mlp_inputs(51, M)
    x = to_dev_bf16(m.x)
    w1, w2, w3 = (to_dev_bf16(a) for a in (m.w1, m.w2, m.w3))
    out = torch.empty((M, 4096), dtype=torch.float32, device=dev())
    act = torch.empty((M, 14336), dtype=torch.bfloat16, device=dev())
    ws = torch.empty(max(1, gqa.mlp_workspace_bytes(M)), dtype=torch.uint8, device=dev())
    _check_replays(lambda: gqa.mlp_forward(x, w1, w2, w3, out=out, a_out=act, workspace=ws),
                   [out, act])


def test_graph_replay_chunk_forward():
    # 2048 new positions after 2048 cached ones: projections with the cache
    # write (the same values on every replay), the balanced attention plan and
    # its merge, W_O
    B, T, S_max, sp = 1, 2048, 4096, 2048
    print(f"[case] graph replay chunk_forward B={B} T={T} start_pos={sp}", flush=True)
    inp = gi.make_block_inputs(52, B, T, cache_len=S_max)
    x = to_dev_bf16(inp.x)
    w = [to_dev_bf16(m) for m in (inp.wq, inp.wk, inp.wv, inp.wo)]
    kc, vc = to_dev_bf16(inp.k_cache), to_dev_bf16(inp.v_cache)
    rope = to_dev_f32(gqa.rope_table(np.arange(sp, sp + T)))
    out = torch.empty((B, T, 4096), dtype=torch.float32, device=dev())
    ws = torch.empty(max(1, gqa.chunk_workspace_bytes(B, T, sp)), dtype=torch.uint8, device=dev())
    _check_replays(lambda: gqa.chunk_forward(x, *w, rope, kc, vc, sp, out=out, workspace=ws),
                   [out])
