"""Pins of the fp64 oracle against what the pages and the mathematics fix.

Each test would fail on a plausible slip in the oracle: a dropped scale, a
wrong rotation sign or pairing, a transposed weight, h % n_kv instead of
floor(h / n_rep), a mask off by one, an unnormalised softmax.
"""

import json
import math
import os

import numpy as np
import pytest

import gqa_inputs as gi
from oracle import gqa_oracle as O
from tests.brute_force import brute_block

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _golden(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


def _tiny(seed, B=1, T=4, d=16, H=4, G=2, dh=4, cache=0, w_std=0.3):
    rng = np.random.default_rng(seed)
    f = lambda *s: rng.standard_normal(s)
    x = f(B, T, d)
    wq, wk, wv = f(H * dh, d) * w_std, f(G * dh, d) * w_std, f(G * dh, d) * w_std
    wo = f(d, H * dh) * w_std
    kc = f(B, cache, G, dh) if cache else None
    vc = f(B, cache, G, dh) if cache else None
    return x, wq, wk, wv, wo, kc, vc


# --- values the pages print ---------------------------------------------------------

def test_parameter_counts_match_pages():
    g = _golden("llama31_8b_attention_page.json")
    pc = O.param_counts(g["dim"], g["n_heads"], g["n_kv_heads"])
    p = g["params_per_block"]
    assert pc["head_dim"] == g["head_dim"]
    assert pc["q"] == p["query_projection"]
    assert pc["k"] == p["key_projection"]
    assert pc["v"] == p["value_projection"]
    assert pc["o"] == p["output_projection"]
    assert pc["total"] == p["total"]
    assert pc["total"] * g["n_layers"] == g["params_all_blocks"]
    assert pc["q"] * g["n_layers"] == g["w_q_all_blocks"]
    assert pc["o"] * g["n_layers"] == g["w_o_all_blocks"]
    # the generator makes weights of exactly these shapes
    inp = gi.make_block_inputs(0, 1, 1)
    assert inp.wq.size == p["query_projection"] and inp.wk.size == p["key_projection"]
    assert inp.wv.size == p["value_projection"] and inp.wo.size == p["output_projection"]
    assert g["rope_pairs"] == g["head_dim"] // 2


def test_causal_mask_matches_hand_examples():
    for case in _golden("causal_mask_examples.json")["cases"]:
        want = np.array([[-np.inf if v is None else v for v in row] for row in case["mask"]])
        got = O.causal_mask(case["T"], case["start_pos"])
        assert got.shape == want.shape
        assert np.array_equal(got, want)


# --- dtype ------------------------------------------------------------------------

def test_bf16_widening_known_patterns():
    bits = np.array([0x3F80, 0xC000, 0x3F81, 0x0000, 0x8000, 0x7F80], dtype=np.uint16)
    got = O.bf16_to_f64(bits)
    assert got[0] == 1.0 and got[1] == -2.0 and got[2] == 1.0 + 2.0 ** -7
    assert got[3] == 0.0 and np.signbit(got[4]) and got[5] == np.inf


def test_generator_rounding_is_nearest_even_and_seeded():
    v = np.array([1.0 + 2.0 ** -8, 1.0 + 3 * 2.0 ** -8, -1.0 - 2.0 ** -8, 1.0 + 2.0 ** -8 + 2.0 ** -20],
                 dtype=np.float32)
    b = gi.f32_to_bf16_bits(v)
    assert list(b) == [0x3F80, 0x3F82, 0xBF80, 0x3F81]
    a = gi.make_block_inputs(5, 1, 3)
    c = gi.make_block_inputs(5, 1, 3)
    assert np.array_equal(a.x, c.x) and np.array_equal(a.wo, c.wo)
    assert not np.array_equal(a.x, gi.make_block_inputs(6, 1, 3).x)
    xs = gi.bf16_bits_to_f32(a.wq).astype(np.float64)
    assert abs(xs.std() - 0.02) < 1e-3 and abs(xs.mean()) < 1e-4


# --- rotation ---------------------------------------------------------------------

def test_rope_frequency_exponent():
    w = O.rope_frequencies(128, 500000.0)
    assert w.shape == (64,)
    assert w[0] == 1.0                                    # pair 0 turns by t radians
    assert math.isclose(w[32] ** 2, 1.0 / 500000.0, rel_tol=1e-13)
    r = w[1:] / w[:-1]
    assert np.allclose(r, r[0], rtol=1e-13, atol=0)      # geometric in j
    assert math.isclose(r[0] ** 64, 1.0 / 500000.0, rel_tol=1e-12)


def test_rope_rotation_sense_and_pairing():
    z = np.zeros((1, 1, 1, 8))
    z[..., 2] = 1.0                                       # e_2 = first member of pair 1
    cos = np.zeros((1, 4)); sin = np.zeros((1, 4))
    cos[:] = 1.0
    cos[0, 1], sin[0, 1] = 0.0, 1.0                       # quarter turn on pair 1 only
    out = O.rope_rotate(z, cos, sin)[0, 0, 0]
    assert np.array_equal(out, [0, 0, 0, 1, 0, 0, 0, 0])  # (1,0) -> (0,1): counter-clockwise
    z[..., 2] = 0.0
    z[..., 3] = 1.0
    out = O.rope_rotate(z, cos, sin)[0, 0, 0]
    assert np.array_equal(out, [0, 0, -1, 0, 0, 0, 0, 0])  # (0,1) -> (-1,0)
    # pair 0 at position 1 turns by exactly one radian
    c, s = O.rope_cos_sin([1], 128)
    assert c[0, 0] == math.cos(1.0) and s[0, 0] == math.sin(1.0)


def test_rope_preserves_pair_norm_and_identity_at_zero():
    rng = np.random.default_rng(0)
    z = rng.standard_normal((2, 5, 3, 128))
    pos = np.array([0, 1, 17, 8191, 131071])
    c, s = O.rope_cos_sin(pos, 128)
    r = O.rope_rotate(z, c, s)
    n0 = z[..., 0::2] ** 2 + z[..., 1::2] ** 2
    n1 = r[..., 0::2] ** 2 + r[..., 1::2] ** 2
    assert np.allclose(n1, n0, rtol=1e-13, atol=0)
    assert np.array_equal(r[:, 0], z[:, 0])              # t = 0 is the identity


def test_rope_relative_position():
    # q_t · k_s depends on t - s only: shift both positions by c, scores unchanged
    rng = np.random.default_rng(1)
    q = rng.standard_normal((1, 1, 1, 128))
    k = rng.standard_normal((1, 1, 1, 128))
    vals = []
    for shift in (0, 5, 1000, 70000):
        cq, sq = O.rope_cos_sin([30 + shift], 128)
        ck, sk = O.rope_cos_sin([7 + shift], 128)
        vals.append(float(np.sum(O.rope_rotate(q, cq, sq) * O.rope_rotate(k, ck, sk))))
    assert np.allclose(vals, vals[0], rtol=1e-9, atol=1e-9)


# --- softmax / scale / mask ---------------------------------------------------------

def test_softmax_rows_normalised_and_masked_entries_zero():
    x, wq, wk, wv, wo, _, _ = _tiny(3, B=2, T=6)
    r = O.block_forward(x, wq, wk, wv, wo, 4, 2, causal=True, return_probs=True)
    a = r["probs"]
    assert np.all(a >= 0)
    assert np.allclose(a.sum(-1), 1.0, rtol=0, atol=1e-12)
    iu = np.triu_indices(6, 1)
    assert np.all(a[:, :, iu[0], iu[1]] == 0.0)


def test_scale_is_inverse_sqrt_head_dim():
    # two keys whose scores differ by sqrt(128)*ln 3: weights 3/4 and 1/4 exactly
    dh = 128
    q = np.zeros((1, 1, 1, dh)); q[..., 0] = 1.0
    k = np.zeros((1, 2, 1, dh)); k[0, 0, 0, 0] = math.sqrt(dh) * math.log(3.0)
    v = np.zeros((1, 2, 1, dh)); v[0, 0, 0, 0] = 1.0; v[0, 1, 0, 1] = 1.0
    h = O.grouped_attention(q, k, v, None)
    assert math.isclose(h[0, 0, 0, 0], 0.75, rel_tol=1e-14)
    assert math.isclose(h[0, 0, 0, 1], 0.25, rel_tol=1e-14)


def test_fully_masked_row_raises():
    q = np.ones((1, 1, 1, 4)); k = np.ones((1, 2, 1, 4)); v = np.ones((1, 2, 1, 4))
    with pytest.raises(ValueError):
        O.grouped_attention(q, k, v, np.full((1, 2), -np.inf))


def test_mask_equivalences():
    x, wq, wk, wv, wo, _, _ = _tiny(4, T=5)
    a = O.block_forward(x, wq, wk, wv, wo, 4, 2, causal=True)["delta"]
    b = O.block_forward(x, wq, wk, wv, wo, 4, 2, causal=False, mask=O.causal_mask(5))["delta"]
    assert np.array_equal(a, b)
    c = O.block_forward(x, wq, wk, wv, wo, 4, 2, causal=False, mask=np.zeros((5, 5)))["delta"]
    d = O.block_forward(x, wq, wk, wv, wo, 4, 2, causal=False, mask=None)["delta"]
    assert np.array_equal(c, d)
    assert not np.allclose(a, d)


# --- whole-block closed forms at the real dims ---------------------------------------

def test_causal_row0_is_own_value_through_wo():
    inp = gi.make_block_inputs(11, 2, 3)
    r = O.block_forward(inp.x, inp.wq, inp.wk, inp.wv, inp.wo, 32, 8)
    x0 = O.bf16_to_f64(inp.x)[:, 0, :]                    # [B, 4096]
    wv = O.bf16_to_f64(inp.wv)
    wo = O.bf16_to_f64(inp.wo)
    for b in range(2):
        v0 = np.einsum("k,nk->n", x0[b], wv)                 # the token's own value row
        heads = [v0[128 * (h // 4): 128 * (h // 4) + 128] for h in range(32)]
        merged = np.concatenate(heads)                     # feature 128*h + d
        want = np.einsum("k,nk->n", merged, wo)
        assert np.allclose(r["delta"][b, 0], want, rtol=1e-12, atol=1e-12)


def test_gqa_equals_mha_with_interleaved_kv():
    x, wq, wk, wv, wo, _, _ = _tiny(5, B=2, T=5, d=16, H=4, G=2, dh=4)
    g = O.block_forward(x, wq, wk, wv, wo, 4, 2)["delta"]
    rep = lambda w: np.concatenate([w[4 * (h // 2): 4 * (h // 2) + 4] for h in range(4)])
    m = O.block_forward(x, wq, rep(wk), rep(wv), wo, 4, 4)["delta"]
    assert np.allclose(g, m, rtol=1e-12, atol=1e-13)
    # the other grouping (h mod n_kv) gives a different answer
    alt = lambda w: np.concatenate([w[4 * (h % 2): 4 * (h % 2) + 4] for h in range(4)])
    wrong = O.block_forward(x, wq, alt(wk), alt(wv), wo, 4, 4)["delta"]
    assert not np.allclose(g, wrong)


def test_uniform_attention_gives_prefix_mean():
    inp = gi.make_block_inputs(12, 1, 6)
    wk0 = np.zeros_like(inp.wk)                          # all scores 0
    r = O.block_forward(inp.x, inp.wq, wk0, inp.wv, inp.wo, 32, 8)
    v = r["v"][0]                                         # [T, 8, 128]
    for t in range(6):
        mean = v[: t + 1].mean(axis=0)                    # [8, 128]
        want = np.concatenate([mean[h // 4] for h in range(32)])
        assert np.allclose(r["h"][0, t], want, rtol=1e-12, atol=1e-13)


def test_causal_prefix_property():
    x, wq, wk, wv, wo, _, _ = _tiny(6, B=2, T=7)
    full = O.block_forward(x, wq, wk, wv, wo, 4, 2)["delta"]
    part = O.block_forward(x[:, :4], wq, wk, wv, wo, 4, 2)["delta"]
    assert np.allclose(full[:, :4], part, rtol=1e-13, atol=1e-14)


def test_decode_equals_prefill_row():
    x, wq, wk, wv, wo, _, _ = _tiny(7, B=2, T=6)
    pre = O.block_forward(x, wq, wk, wv, wo, 4, 2)
    p = 5
    first = O.block_forward(x[:, :p], wq, wk, wv, wo, 4, 2)
    kc = first["k_r"]; vc = first["v"]                    # rotated keys / raw values of 0..p-1
    # a cache longer than start_pos: trailing rows must be ignored / overwritten
    pad = np.full((2, 3, 2, 4), 1e3)
    dec = O.decode_forward(x[:, p], wq, wk, wv, wo, 4, 2, np.concatenate([kc, pad], 1),
                           np.concatenate([vc, pad], 1), start_pos=p)
    assert np.allclose(dec["delta"], pre["delta"][:, p], rtol=1e-12, atol=1e-13)
    # chunked prefill over a cache gives the same rows too
    ch = O.block_forward(x[:, 3:], wq, wk, wv, wo, 4, 2, start_pos=3,
                         k_cache=pre["k_r"][:, :3], v_cache=pre["v"][:, :3])
    assert np.allclose(ch["delta"], pre["delta"][:, 3:], rtol=1e-12, atol=1e-13)


def test_linear_in_wo_and_wv():
    x, wq, wk, wv, wo, _, _ = _tiny(8, T=4)
    a = O.block_forward(x, wq, wk, wv, wo, 4, 2)["delta"]
    assert np.allclose(O.block_forward(x, wq, wk, wv, 2 * wo, 4, 2)["delta"], 2 * a, rtol=1e-13)
    assert np.allclose(O.block_forward(x, wq, wk, 3 * wv, wo, 4, 2)["delta"], 3 * a, rtol=1e-13)


# --- brute force on tiny shapes ----------------------------------------------------

@pytest.mark.parametrize("case", ["causal", "causal_cache", "explicit_mask", "no_mask", "single"])
def test_brute_force_tiny(case):
    B, T, d, H, G, dh = 2, 5, 16, 4, 2, 4
    sp = 3 if case == "causal_cache" else 0
    if case == "single":
        T = 1
    x, wq, wk, wv, wo, kc, vc = _tiny(20 + len(case), B=B, T=T, d=d, H=H, G=G, dh=dh, cache=sp)
    mask = None
    causal = case in ("causal", "causal_cache", "single")
    if case == "explicit_mask":
        rng = np.random.default_rng(99)
        mask = rng.standard_normal((T, T))
        mask[1, 3] = -np.inf
    want = O.block_forward(x, wq, wk, wv, wo, H, G, causal=causal, mask=mask, start_pos=sp,
                           k_cache=kc, v_cache=vc, theta=10000.0)["delta"]
    ck = None if not sp else kc.reshape(B, sp, G * dh).tolist()
    cv = None if not sp else vc.reshape(B, sp, G * dh).tolist()
    got = brute_block(x.tolist(), wq.tolist(), wk.tolist(), wv.tolist(), wo.tolist(), H, G,
                      start_pos=sp, cache_k=ck, cache_v=cv,
                      mask=None if mask is None else mask.tolist(), causal=causal, theta=10000.0)
    assert np.allclose(np.array(got), want, rtol=1e-12, atol=1e-12)


def test_brute_force_real_theta_long_positions():
    # real theta and large positions, where the rotation angle is far from zero
    x, wq, wk, wv, wo, kc, vc = _tiny(31, B=1, T=3, d=8, H=2, G=1, dh=4, cache=0)
    sp = 5000
    rng = np.random.default_rng(2)
    kc = rng.standard_normal((1, sp, 1, 4)); vc = rng.standard_normal((1, sp, 1, 4))
    want = O.block_forward(x, wq, wk, wv, wo, 2, 1, start_pos=sp, k_cache=kc, v_cache=vc)["delta"]
    got = brute_block(x.tolist(), wq.tolist(), wk.tolist(), wv.tolist(), wo.tolist(), 2, 1,
                      start_pos=sp, cache_k=kc.reshape(1, sp, 4).tolist(),
                      cache_v=vc.reshape(1, sp, 4).tolist())
    assert np.allclose(np.array(got), want, rtol=1e-10, atol=1e-12)


def test_sampled_rows_match_full_oracle():
    inp = gi.make_block_inputs(13, 2, 40)
    full = O.block_forward(inp.x, inp.wq, inp.wk, inp.wv, inp.wo, 32, 8)
    rows = [0, 1, 17, 39]
    for b in range(2):
        r = O.block_forward_rows(inp.x, inp.wq, inp.wk, inp.wv, inp.wo, 32, 8, rows, batch_index=b)
        assert np.allclose(r["delta"], full["delta"][b, rows], rtol=1e-12, atol=1e-12)
        assert np.allclose(r["h"], full["h"][b, rows], rtol=1e-12, atol=1e-12)


# --- pre-norm and residual (the block's handoff) ------------------------------------

def test_rms_norm_one_hot_closed_form():
    # x = a·e_k in n features: mean square a²/n, so with eps = 0 the output is
    # sign(a)·sqrt(n)·w_k at feature k and zero elsewhere. A sum in place of the
    # mean, a missing root or a gain taken from another feature all fail here.
    n = 16
    w = 1.0 + np.arange(n) / 8.0
    for k, a in ((0, 3.0), (5, -0.25), (15, 1e-3)):
        x = np.zeros(n)
        x[k] = a
        y = O.rms_norm(x, w, eps=0.0)
        want = np.zeros(n)
        want[k] = math.copysign(math.sqrt(n), a) * w[k]
        assert np.allclose(y, want, rtol=1e-14, atol=0)


def test_rms_norm_eps_sits_under_the_root():
    # a constant row c: y = w·c/sqrt(c² + eps). At c = 1e-3 and eps = 1e-5 that is
    # 1e-3/sqrt(1.1e-5) = 0.30151..., far from c/(|c| + eps) = 0.990 or
    # c/sqrt(c²) = 1 (eps added outside the root, or dropped).
    c, eps = 1e-3, 1e-5
    y = O.rms_norm(np.full((2, 8), c), np.ones(8), eps=eps)
    assert np.allclose(y, 0.30151134457776363, rtol=1e-12)
    assert O.NORM_EPS == 1e-5


def test_rms_norm_unit_mean_square_and_scale_invariance():
    rng = np.random.default_rng(11)
    x = rng.standard_normal((3, 5, 64)) * 7.0
    y = O.rms_norm(x, np.ones(64), eps=0.0)
    assert np.allclose(np.mean(y * y, axis=-1), 1.0, rtol=1e-13)
    assert np.all(np.sign(y) == np.sign(x))          # a positive rescaling per row
    assert np.allclose(O.rms_norm(x * 0.01, np.ones(64), eps=0.0), y, rtol=1e-12)
    # rows are normalised independently
    assert np.allclose(O.rms_norm(x[1:2], np.ones(64), eps=0.0), y[1:2], rtol=1e-13)


def test_prenorm_zero_gain_leaves_the_input():
    # gain 0: the normalised input is 0, so Q = K = V = 0, every head averages zero
    # values and Δ = 0: the residual must give back x exactly (not x̂, not Δ alone).
    x, wq, wk, wv, wo, _, _ = _tiny(21, B=2, T=5)
    r = O.prenorm_block_forward(x, np.zeros(16), wq, wk, wv, wo, 4, 2)
    assert np.array_equal(r["out"], x)
    assert np.array_equal(r["delta"], np.zeros_like(x))


def test_prenorm_residual_adds_x_to_the_normalised_block():
    # out − x is the block applied to the normalised rows; scaling x by α > 0
    # leaves that part unchanged (eps = 0), so out(αx) − αx = out(x) − x.
    x, wq, wk, wv, wo, kc, vc = _tiny(22, B=1, T=6)
    g = 1.0 + np.random.default_rng(5).standard_normal(16) * 0.3
    r1 = O.prenorm_block_forward(x, g, wq, wk, wv, wo, 4, 2, eps=0.0, input_bf16=False)
    r2 = O.prenorm_block_forward(3.5 * x, g, wq, wk, wv, wo, 4, 2, eps=0.0, input_bf16=False)
    assert np.allclose(r2["out"] - 3.5 * x, r1["out"] - x, rtol=1e-10, atol=1e-12)
    assert not np.allclose(r1["out"] - x, O.block_forward(x, wq, wk, wv, wo, 4, 2)["delta"])
    # with the bf16 input reading, the block sees the rounded x̂
    r3 = O.prenorm_block_forward(x, g, wq, wk, wv, wo, 4, 2, eps=0.0)
    xr = O.round_to_bf16(O.rms_norm(x, g, eps=0.0))
    assert np.array_equal(r3["x_norm"], xr)
    assert np.allclose(r3["out"] - x, O.block_forward(xr, wq, wk, wv, wo, 4, 2)["delta"],
                       rtol=1e-12, atol=1e-14)
    # decode form: same block at one position over the cache
    x, wq, wk, wv, wo, kc, vc = _tiny(23, B=2, T=1, cache=4)
    d = O.prenorm_decode_forward(x[:, 0], g, wq, wk, wv, wo, 4, 2, kc, vc, 3)
    p = O.prenorm_block_forward(x, g, wq, wk, wv, wo, 4, 2, start_pos=3, k_cache=kc,
                                v_cache=vc)
    assert np.allclose(d["out"], p["out"][:, 0], rtol=1e-12, atol=1e-14)


def test_norm_gain_generator_is_seeded_and_centred():
    g1, g2 = gi.make_norm_weight(3), gi.make_norm_weight(3)
    assert g1.dtype == np.uint16 and g1.shape == (4096,) and np.array_equal(g1, g2)
    v = O.bf16_to_f64(g1)
    assert abs(v.mean() - 1.0) < 0.02 and 0.17 < v.std() < 0.23
    assert not np.array_equal(g1, gi.make_norm_weight(4))


def test_round_to_bf16_known_values_and_ties_to_even():
    # bf16 spacing is 2^-7 in [1, 2): 1 + 2^-8 is a tie and goes to the even
    # neighbour 1; 1 + 3·2^-8 is a tie between 1 + 2^-7 (odd) and 1 + 2^-6 (even)
    cases = {1.0: 1.0, 1.0 + 2 ** -8: 1.0, 1.0 + 3 * 2 ** -8: 1.0 + 2 ** -6,
             1.0 + 2 ** -8 + 2 ** -30: 1.0 + 2 ** -7, -(1.0 + 2 ** -8 + 2 ** -30): -(1.0 + 2 ** -7),
             0.0: 0.0, 3.0: 3.0, 255.5: 256.0, 2.0 ** -130: 2.0 ** -130, 1e-3: 0.00099945068359375}
    for a, want in cases.items():
        assert O.round_to_bf16(np.array([a]))[0] == want, a
    # agrees with the generator's float32 -> bf16 rounding wherever float32 is exact
    rng = np.random.default_rng(3)
    v = (rng.standard_normal(20000) * np.exp(rng.uniform(-20, 20, 20000))).astype(np.float32)
    assert np.array_equal(O.round_to_bf16(v.astype(np.float64)),
                          O.bf16_to_f64(gi.f32_to_bf16_bits(v)))
    # and lands within half a bf16 ulp of fp64 inputs that float32 cannot hold
    w = rng.standard_normal(20000) * 10.0
    r = O.round_to_bf16(w)
    _, e = np.frexp(w)
    assert np.all(np.abs(r - w) <= np.ldexp(0.5, e - 8))


def test_rope_explicit_frequencies():
    # the table is an input of the block: explicit frequencies replace θ^(-2j/d)
    x, wq, wk, wv, wo, _, _ = _tiny(31, B=1, T=5)
    base = O.block_forward(x, wq, wk, wv, wo, 4, 2)
    same = O.block_forward(x, wq, wk, wv, wo, 4, 2, omega=O.rope_frequencies(4))
    assert np.array_equal(base["delta"], same["delta"])
    # zero frequencies: no rotation at any position
    flat = O.block_forward(x, wq, wk, wv, wo, 4, 2, omega=np.zeros(2))
    assert np.array_equal(flat["q_r"], flat["q"]) and np.array_equal(flat["k_r"], flat["k"])
    # dividing every frequency by 8 (exact in binary) turns position 8t into t
    w = O.rope_frequencies(128)
    t = np.array([0, 1, 5, 1000, 8191])
    c1, s1 = O.rope_cos_sin(8 * t, 128, omega=w / 8)
    c2, s2 = O.rope_cos_sin(t, 128)
    assert np.array_equal(c1, c2) and np.array_equal(s1, s2)


# --- SwiGLU MLP -------------------------------------------------------------------------

def test_silu_minimum_matches_page():
    # the page prints that SiLU dips to about -0.28 near g = -1.28
    from scipy.optimize import minimize_scalar
    gold = _golden("llama3_swiglu_page.json")
    r = minimize_scalar(lambda g: float(O.silu(g)), bounds=(-5, 5), method="bounded",
                        options={"xatol": 1e-10})
    nd = gold["printed_decimals"]
    assert round(r.x, nd) == gold["silu_min_at_about"]
    assert round(r.fun, nd) == gold["silu_min_value_about"]
    assert O.D_FF == gold["d_ff"]


def test_silu_identities():
    g = np.linspace(-30, 30, 601)
    # sigma(g) + sigma(-g) = 1  =>  silu(g) - silu(-g) = g
    assert np.allclose(O.silu(g) - O.silu(-g), g, rtol=1e-13, atol=1e-13)
    assert O.silu(0.0) == 0.0
    assert O.silu(50.0) == 50.0                       # sigma(50) rounds to 1
    assert O.silu(-800.0) == 0.0                      # the limit, no overflow error
    # slope 1/2 at 0 (sigma(0) = 1/2)
    e = 1e-6
    assert abs((O.silu(e) - O.silu(-e)) / (2 * e) - 0.5) < 1e-9
    assert abs(O.silu(1.0) - 1.0 / (1.0 + math.exp(-1.0))) < 1e-15


def test_mlp_brute_force_tiny():
    from tests.brute_force import brute_mlp
    rng = np.random.default_rng(17)
    T, d, f = 3, 5, 7     # non-square: a transposed weight cannot pass
    x = rng.standard_normal((T, d))
    w1, w3 = rng.standard_normal((f, d)), rng.standard_normal((f, d))
    w2 = rng.standard_normal((d, f))
    want = np.array(brute_mlp(x.tolist(), w1.tolist(), w2.tolist(), w3.tolist()))
    got = O.mlp_forward(x, w1, w2, w3)["delta"]
    assert np.allclose(got, want, rtol=1e-12, atol=1e-12)
    # gate and up are not interchangeable (silu is not symmetric)
    assert not np.allclose(O.mlp_forward(x, w3, w2, w1)["delta"], want)


def test_mlp_structure():
    rng = np.random.default_rng(18)
    x = rng.standard_normal((4, 6))
    w1, w3, w2 = rng.standard_normal((9, 6)), rng.standard_normal((9, 6)), rng.standard_normal((6, 9))
    r = O.mlp_forward(x, w1, w2, w3)
    # linear in w2 and in w3; zero up projection gives zero output
    assert np.allclose(O.mlp_forward(x, w1, 2.5 * w2, w3)["delta"], 2.5 * r["delta"], rtol=1e-13)
    assert np.allclose(O.mlp_forward(x, w1, w2, -3 * w3)["delta"], -3 * r["delta"], rtol=1e-13)
    assert np.array_equal(O.mlp_forward(x, w1, w2, 0 * w3)["delta"], np.zeros((4, 6)))
    # rows are independent: one row alone gives the same row
    assert np.allclose(O.mlp_forward(x[2:3], w1, w2, w3)["delta"], r["delta"][2:3], rtol=1e-13)
    # pre-norm form: zero gain leaves h unchanged (silu(0)·0 = 0)
    p = O.prenorm_mlp_forward(x, np.zeros(6), w1, w2, w3)
    assert np.array_equal(p["out"], x)


def test_mlp_generator_shapes():
    m = gi.make_mlp_inputs(1, 3)
    assert m.w1.shape == (14336, 4096) and m.w3.shape == (14336, 4096)
    assert m.w2.shape == (4096, 14336) and m.x.shape == (3, 4096)
    small = gi.make_mlp_inputs(1, 3, d=32, d_ff=64)
    assert np.array_equal(small.x, gi.make_mlp_inputs(1, 3, d=32, d_ff=64).x)
