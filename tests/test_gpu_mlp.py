"""GPU parity of the SwiGLU MLP ("Llama 3" page, SwiGLU MLP) through the C ABI
against the fp64 oracle, plain and in its pre-norm + residual form.

Tolerances: out (fp32) is held to relL2 <= 5e-3, the block's bar, and to a
max abs error of 3% of the exact output's rms. The attention block's 2e-2
max-abs bar is about 3% of its Δ's rms (0.6 to 0.75 on the block's inputs);
the MLP's output is about four times larger (rms ~2.4: 14336 terms of
N(0, 0.02^2) weights against A of rms ~1), and its error with it. That
error comes from rounding A = silu(gate)·up to bf16 before the down product
(about 2^-9/sqrt(3) relative per element, averaged over 14336 terms) and
fp32 accumulation. A itself is one bf16 rounding from the fp32
value: elementwise |A - A_exact| <= 2^-8 |A_exact| (half an ulp) + 1e-3 (the
fp32 error of gate and up over 4096 terms, and of the exponential, before the
rounding; it matters only where A is near zero). In the pre-norm
form the oracle rounds x̂ to bf16 (the MLP's input is a bf16 activation).
Long inputs are checked on sampled rows: rows of the MLP are independent, so
the oracle evaluates exactly those rows.
"""

import numpy as np
import pytest
import torch

import gqa_inputs as gi
import grouped_query_attention_amd as gqa
from oracle import gqa_oracle as O
from tests.gpu_util import assert_close, bf16_to_np_f64, dev, f32_to_np_f64, to_dev_bf16

pytestmark = pytest.mark.gpu

_W = {}


def _close(got, want, what):
    rms = float(np.sqrt(np.mean(want * want)))
    assert_close(got, want, mabs=0.03 * rms, what=f"{what} (rms {rms:.2f})")


def _weights():
    # one set of weights (352 MB of bf16) for every case; inputs vary per case
    if not _W:
        m = gi.make_mlp_inputs(10, 1)
        _W["np"] = m
        _W["dev"] = [to_dev_bf16(a) for a in (m.w1, m.w2, m.w3)]
    return _W["np"], _W["dev"]


def _x(seed, M):
    rng = np.random.Generator(np.random.PCG64(seed))
    return gi.normal_bf16(rng, (M, 4096), 1.0)


# M = 1, 60: the down product's split reduction; 64 < M: plain tiles; 300 ragged;
# 1500: the 128x256 gate/up tiles
@pytest.mark.parametrize("M", [1, 60, 65, 300, 1500])
def test_mlp_forward(M):
    print(f"[case] mlp M={M}", flush=True)
    w, (w1, w2, w3) = _weights()
    xb = _x(1000 + M, M)
    a = torch.empty((M, 14336), dtype=torch.bfloat16, device=dev())
    out = gqa.mlp_forward(to_dev_bf16(xb), w1, w2, w3, a_out=a)
    torch.cuda.synchronize()
    ref = O.mlp_forward(xb, w.w1, w.w2, w.w3)
    _close(f32_to_np_f64(out), ref["delta"], f"MLP out M={M}")
    ga = bf16_to_np_f64(a)
    err = np.abs(ga - ref["a"])
    print(f"[parity] A M={M}: max|err| {err.max():.3e}, "
          f"max rel {np.max(err / np.maximum(np.abs(ref['a']), 1e-30)):.3e}", flush=True)
    assert np.all(err <= 2.0 ** -8 * np.abs(ref["a"]) + 1e-3)


# M = 9000 takes the 256x256 gate/up tiles in one launch (36 token tiles x 112
# feature tiles make no whole number of rounds on 256 CUs) and 256x256 down
# tiles; M = 2048 and 2000 (8 token tiles, the last ragged at 2000) split the
# gate/up product into 768 tiles of 256x256 (hidden units 0 .. 12287) and 256
# of 256x128 (12288 .. 14335). The hidden activation A is compared as well.
@pytest.mark.parametrize("M", [9000, 2048, 2000])
def test_mlp_forward_large_sampled_rows(M):
    print(f"[case] mlp M={M} (sampled rows)", flush=True)
    w, (w1, w2, w3) = _weights()
    xb = _x(1999 + M, M)
    a_out = torch.empty((M, 14336), dtype=torch.bfloat16, device=dev())
    out = gqa.mlp_forward(to_dev_bf16(xb), w1, w2, w3, a_out=a_out)
    torch.cuda.synchronize()
    edges = [0, 1, 255, 256, 1791, 1792, M - 1] + ([8191, 8192] if M > 8192 else [])
    rows = np.unique(np.concatenate([edges, np.random.Generator(np.random.PCG64(5)).integers(0, M, 40)]))
    sel = torch.from_numpy(rows).to(dev())
    ref = O.mlp_forward(xb[rows], w.w1, w.w2, w.w3)
    _close(f32_to_np_f64(out[sel]), ref["delta"], f"MLP out sampled rows M={M}")
    # A is rounded to bf16 once: at most one bf16 ulp of the largest value off
    got_a = bf16_to_np_f64(a_out[sel])
    for lo, hi in ((0, 12288), (12288, 14336)):
        want_a = ref["a"][:, lo:hi]
        assert_close(got_a[:, lo:hi], want_a, mabs=float(np.abs(want_a).max()) * 2.0 ** -7,
                     what=f"MLP A units {lo}..{hi - 1} M={M}")


@pytest.mark.parametrize("M", [7, 64, 700])
def test_mlp_forward_prenorm(M):
    print(f"[case] mlp prenorm M={M}", flush=True)
    w, (w1, w2, w3) = _weights()
    xb = _x(3000 + M, M)
    g = gi.make_norm_weight(3000 + M)
    out = gqa.mlp_forward(to_dev_bf16(xb), w1, w2, w3, norm_w=to_dev_bf16(g))
    torch.cuda.synchronize()
    ref = O.prenorm_mlp_forward(xb, g, w.w1, w.w2, w.w3)
    got = f32_to_np_f64(out)
    x = O.bf16_to_f64(xb)
    _close(got - x, ref["delta"], f"MLP Δ = out - x M={M}")
    _close(got, ref["out"], f"MLP out M={M}")


def test_mlp_rerun_is_bitwise():
    _, (w1, w2, w3) = _weights()
    x = to_dev_bf16(_x(4000, 333))
    o1 = gqa.mlp_forward(x, w1, w2, w3)
    o2 = gqa.mlp_forward(x, w1, w2, w3)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2)
