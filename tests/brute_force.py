"""Scalar pure-Python evaluation of the grouped-query-attention block, for tiny shapes.

Written from the equations on the "Llama 3.1 8B · Grouped-query attention"
page ("All 13 steps") with plain loops and the math module, independent of
the vectorised oracle, to pin it. Inputs are nested lists of floats.
"""

import math

NEG_INF = float("-inf")


def _linear(vec, W):
    # out[n] = sum_k vec[k] * W[n][k]  (weights stored [out, in])
    return [sum(vec[k] * W[n][k] for k in range(len(vec))) for n in range(len(W))]


def _rotate(vec, dh, pos, theta):
    out = list(vec)
    n_heads = len(vec) // dh
    for h in range(n_heads):
        for j in range(dh // 2):
            w = theta ** (-(2.0 * j) / dh)
            c, s = math.cos(pos * w), math.sin(pos * w)
            a = vec[h * dh + 2 * j]
            b = vec[h * dh + 2 * j + 1]
            out[h * dh + 2 * j] = c * a - s * b
            out[h * dh + 2 * j + 1] = s * a + c * b
    return out


def brute_block(x, wq, wk, wv, wo, n_heads, n_kv, start_pos=0, cache_k=None,
                cache_v=None, mask=None, causal=True, theta=500000.0):
    """x: [B][T][d]; cache_k/cache_v: [B][start_pos][n_kv*dh] (rotated keys, raw values).

    Returns delta [B][T][d].
    """
    B, T = len(x), len(x[0])
    dh = len(wq) // n_heads
    rep = n_heads // n_kv
    out = []
    for b in range(B):
        qs, ks, vs = [], [], []
        for t in range(T):
            pos = start_pos + t
            qs.append(_rotate(_linear(x[b][t], wq), dh, pos, theta))
            ks.append(_rotate(_linear(x[b][t], wk), dh, pos, theta))
            vs.append(_linear(x[b][t], wv))
        keys = (list(cache_k[b][:start_pos]) if start_pos else []) + ks
        vals = (list(cache_v[b][:start_pos]) if start_pos else []) + vs
        rows = []
        for t in range(T):
            merged = []
            for h in range(n_heads):
                g = h // rep
                scores = []
                for j in range(len(keys)):
                    s = sum(qs[t][h * dh + e] * keys[j][g * dh + e] for e in range(dh))
                    s = s / math.sqrt(dh)
                    if causal:
                        if T > 1 and j > start_pos + t:
                            s = NEG_INF
                    elif mask is not None:
                        s = s + mask[t][j]
                    scores.append(s)
                mx = max(scores)
                ex = [math.exp(s - mx) if s != NEG_INF else 0.0 for s in scores]
                tot = sum(ex)
                for e in range(dh):
                    merged.append(sum(ex[j] / tot * vals[j][g * dh + e] for j in range(len(keys))))
            rows.append(_linear(merged, wo))
        out.append(rows)
    return out


def brute_mlp(x, w1, w2, w3):
    """x: [T][d] lists; w1, w3: [f][d]; w2: [d][f]. Written from the "Llama 3"
    page's SwiGLU MLP (w2(silu(w1 x) * w3 x), silu(g) = g * sigma(g),
    sigma(z) = 1/(1 + e^-z)) with loops. Returns [T][d]."""
    out = []
    for row in x:
        gate = _linear(row, w1)
        up = _linear(row, w3)
        a = [gi * (1.0 / (1.0 + math.exp(-gi))) * ui for gi, ui in zip(gate, up)]
        out.append(_linear(a, w2))
    return out
