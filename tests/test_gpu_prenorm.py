"""GPU parity of the block's handoff: RMS pre-normalisation of the input and the
residual add (out = x + Δ(RMSNorm(x))), through the C ABI, against the fp64 oracle.

Tolerances:
  * RMSNorm alone: the kernel works in fp32 and rounds once to bf16, so each
    element is within half a bf16 ulp of the exact value plus the fp32 error
    before rounding: |y - y_exact| <= 2^-8 |y_exact| (half an ulp is at most
    2^-9 of the value's binade, i.e. <= 2^-8 |y|) + 1e-5 |y_exact|.
  * Whole half-block: the attention's input is a bf16 activation, so the
    oracle rounds x̂ to bf16 once (nearest even) before the block, as the
    kernel does. Δ = out - x (x is bf16, exact in fp32; the subtraction adds
    at most one fp32 ulp of |out|) is then held to the bar of the plain block,
    relL2 <= 5e-3 and max abs <= 2e-2. Where the kernel's fp32 x̂ and the
    oracle's fp64 x̂ fall on opposite sides of a rounding midpoint the two
    inputs differ by one bf16 ulp in that element, which the bar absorbs.
  * Against the unrounded definition (x̂ exact): the rounding of x̂ is a
    second error source as large as the plain block's own (it feeds Q, K and
    V together; the oracle alone puts it at 3.1e-3 to 3.6e-3 relL2 and 1.4e-2
    max abs on these inputs), so the bar there is twice the block's:
    relL2 <= 1e-2, max abs <= 4e-2.
"""

import numpy as np
import pytest
import torch

import gqa_inputs as gi
import grouped_query_attention_amd as gqa
from oracle import gqa_oracle as O
from tests.gpu_util import assert_close, bf16_to_np_f64, dev, f32_to_np_f64, to_dev_bf16, to_dev_f32

pytestmark = pytest.mark.gpu

BLOCK_H_REL, BLOCK_H_ABS = 5e-3, 4e-2
STAGE_REL = 3e-3


def _rows_with_scales(seed, M):
    """x [M, 4096] bf16 bits: N(0, 1) rows times per-row scales from 1e-3 to 1e3,
    with row 1 (if present) all zero."""
    rng = np.random.Generator(np.random.PCG64(seed))
    v = rng.standard_normal((M, 4096), dtype=np.float32)
    scale = np.float32(10.0) ** rng.uniform(-3, 3, size=(M, 1)).astype(np.float32)
    v *= scale
    if M > 1:
        v[1] = 0.0
    return gi.f32_to_bf16_bits(v)


@pytest.mark.parametrize("M,eps", [(1, 1e-5), (7, 1e-5), (300, 1e-5), (2048, 1e-5), (5, 0.5)])
def test_rmsnorm_stage(M, eps):
    print(f"[case] rmsnorm M={M} eps={eps}", flush=True)
    xb = _rows_with_scales(900 + M, M)
    g = gi.make_norm_weight(900 + M)
    y = gqa.rmsnorm(to_dev_bf16(xb), to_dev_bf16(g), eps)
    torch.cuda.synchronize()
    got = bf16_to_np_f64(y)
    want = O.rms_norm(xb, g, eps)
    err = np.abs(got - want)
    bound = (2.0 ** -8 + 1e-5) * np.abs(want)
    worst = float(np.max(err - bound))
    print(f"[parity] rmsnorm: max|err| {err.max():.3e}, worst excess over bound {worst:.3e}",
          flush=True)
    assert np.all(err <= bound)
    if M > 1:
        assert np.all(got[1] == 0.0)


def _block_inputs(seed, B, T, cache_len=0):
    inp = gi.make_block_inputs(seed, B, T, cache_len=cache_len)
    return inp, gi.make_norm_weight(seed)


def _w(inp):
    return [to_dev_bf16(a) for a in (inp.wq, inp.wk, inp.wv, inp.wo)]


EXACT_REL, EXACT_ABS = 1e-2, 4e-2


def _check_half_block(out, x_bits, ref, ref_exact, what):
    got = f32_to_np_f64(out)
    x = O.bf16_to_f64(x_bits)
    assert_close(got - x, ref["delta"], what=f"Δ = out - x {what}")
    assert_close(got, ref["out"], what=f"out {what}")
    assert_close(got - x, ref_exact["delta"], rel=EXACT_REL, mabs=EXACT_ABS,
                 what=f"Δ vs unrounded x̂ {what}")


# (2, 30): split-reduction projections (M <= 64); h=False puts x̂ and H in the
# same workspace region one after the other
@pytest.mark.parametrize("B,T,seed,h", [(1, 128, 1, True), (2, 77, 21, False),
                                        (2, 30, 24, False), (1, 1000, 25, True)])
def test_prenorm_block_forward(B, T, seed, h):
    print(f"[case] prenorm block B={B} T={T} seed={seed} h_out={h}", flush=True)
    inp, g = _block_inputs(seed, B, T)
    wq, wk, wv, wo = _w(inp)
    rope = to_dev_f32(gqa.rope_table(np.arange(T)))
    hb = torch.empty((B, T, 32, 128), dtype=torch.bfloat16, device=dev()) if h else None
    out = gqa.block_forward(to_dev_bf16(inp.x), wq, wk, wv, wo, rope, h_out=hb,
                            norm_w=to_dev_bf16(g))
    torch.cuda.synchronize()
    ref = O.prenorm_block_forward(inp.x, g, inp.wq, inp.wk, inp.wv, inp.wo, 32, 8)
    ref_x = O.prenorm_block_forward(inp.x, g, inp.wq, inp.wk, inp.wv, inp.wo, 32, 8,
                                    input_bf16=False)
    _check_half_block(out, inp.x, ref, ref_x, f"B={B} T={T}")
    if h:
        assert_close(bf16_to_np_f64(hb).reshape(B, T, 4096), ref["h"], rel=BLOCK_H_REL,
                     mabs=BLOCK_H_ABS, what="H")


def test_prenorm_zero_gain_returns_x_exactly():
    # gain 0: x̂ = 0, so Q = K = V = 0, H = 0 and Δ = 0 exactly; out must be x bit for bit
    print("[case] prenorm zero gain B=2 T=70", flush=True)
    inp, _ = _block_inputs(26, 2, 70)
    wq, wk, wv, wo = _w(inp)
    x = to_dev_bf16(inp.x)
    out = gqa.block_forward(x, wq, wk, wv, wo, to_dev_f32(gqa.rope_table(np.arange(70))),
                            norm_w=torch.zeros(4096, dtype=torch.bfloat16, device=dev()))
    torch.cuda.synchronize()
    assert torch.equal(out, x.float())


@pytest.mark.parametrize("B,T,S_max,start_pos", [(2, 37, 256, 100), (2, 1, 300, 299)])
def test_prenorm_chunk_forward(B, T, S_max, start_pos):
    print(f"[case] prenorm chunk B={B} T={T} S_max={S_max} start_pos={start_pos}", flush=True)
    inp, g = _block_inputs(80 + T, B, T, cache_len=S_max)
    wq, wk, wv, wo = _w(inp)
    kc, vc = to_dev_bf16(inp.k_cache), to_dev_bf16(inp.v_cache)
    rope = to_dev_f32(gqa.rope_table(np.arange(start_pos, start_pos + T)))
    out = gqa.chunk_forward(to_dev_bf16(inp.x), wq, wk, wv, wo, rope, kc, vc, start_pos,
                            norm_w=to_dev_bf16(g))
    torch.cuda.synchronize()
    kw = dict(start_pos=start_pos, k_cache=inp.k_cache, v_cache=inp.v_cache)
    ref = O.prenorm_block_forward(inp.x, g, inp.wq, inp.wk, inp.wv, inp.wo, 32, 8, **kw)
    ref_x = O.prenorm_block_forward(inp.x, g, inp.wq, inp.wk, inp.wv, inp.wo, 32, 8,
                                    input_bf16=False, **kw)
    _check_half_block(out, inp.x, ref, ref_x, "chunk")
    new = slice(start_pos, start_pos + T)
    assert_close(bf16_to_np_f64(kc)[:, new], ref["k_r"], rel=STAGE_REL, what="cache K slots")
    assert_close(bf16_to_np_f64(vc)[:, new], ref["v"], rel=STAGE_REL, what="cache V slots")


@pytest.mark.parametrize("B,S_max,start_pos", [(3, 700, 650), (64, 1024, 1000)])
def test_prenorm_decode_forward(B, S_max, start_pos):
    print(f"[case] prenorm decode B={B} S_max={S_max} start_pos={start_pos}", flush=True)
    inp, g = _block_inputs(90 + B, B, 1, cache_len=S_max)
    wq, wk, wv, wo = _w(inp)
    kc, vc = to_dev_bf16(inp.k_cache), to_dev_bf16(inp.v_cache)
    rope = to_dev_f32(gqa.rope_table([start_pos])[0])
    out = gqa.decode_forward(to_dev_bf16(inp.x[:, 0]), wq, wk, wv, wo, rope, kc, vc, start_pos,
                             norm_w=to_dev_bf16(g))
    torch.cuda.synchronize()
    args = (inp.x[:, 0], g, inp.wq, inp.wk, inp.wv, inp.wo, 32, 8, inp.k_cache, inp.v_cache,
            start_pos)
    ref = O.prenorm_decode_forward(*args)
    ref_x = O.prenorm_decode_forward(*args, input_bf16=False)
    _check_half_block(out, inp.x[:, 0], ref, ref_x, "decode")
    assert_close(bf16_to_np_f64(kc)[:, start_pos], ref["k_r"], rel=STAGE_REL,
                 what="cache K slot")
