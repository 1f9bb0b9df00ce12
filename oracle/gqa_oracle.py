"""Plain fp64 CPU oracle for the forward pass of one grouped-query-attention block.

TEST INFRASTRUCTURE ONLY. This module exists to check the GPU library. Only
tests/, __graft_entry__.smoke() and the cpu_baseline leg of bench.py may
import or call it; the library and its Python binding never do, and this
module imports nothing from them.

What it computes follows the OpenModelAtlas page "Llama 3.1 8B · Grouped-query
attention", section "All 13 steps" (Q, K, V projections; the pair rotation of
queries and keys; the group head map K_G[h] = K_r[floor(h/4)], V_G likewise;
scores, scale by sqrt(128), additive mask, softmax over keys, A·V_G, merge of
heads, output projection), with the storage conventions of the "Llama 3 8B ·
Query projection" page (weights held [out, in], applied as x·Wᵀ, no bias) and
the mask construction shown in that page's model.py excerpt (minus infinity
where key j > start_pos + i; no mask when one position is decoded).

Everything is float64: bf16 inputs are widened exactly, and no intermediate is
rounded. The function is generic over (d, n_heads, n_kv, d_head) so that tiny
shapes can be brute-forced.

Readings taken where the pages leave a step open (each also listed in the
design notes):
  * x·W means x·Wᵀ with W stored [out, in] (Query projection page, storage
    note; the fairscale excerpt's comment that F.linear computes X·Aᵀ).
  * The rotation acts on adjacent pairs (z_{2j}, z_{2j+1}) inside each head,
    by the angle t·ω_j with ω_j = θ^(-2j/d_head), θ = 500000 (rope_theta of
    the catalogue entry); the prime on ω is read as the unscaled frequency.
  * Position t of query row i is start_pos + i; keys in a cache are already
    rotated at their own positions; values are never rotated.
  * Softmax runs over every key of the row (cache keys included); masked keys
    contribute exp(-inf) = 0. A row with every key masked has no defined
    softmax and raises.
"""

from __future__ import annotations

import math
from typing import Optional

import numpy as np

ROPE_THETA = 500000.0
NORM_EPS = 1e-5     # norm_eps of the Llama 3 / 3.1 8B catalogue entries


# --- dtype -------------------------------------------------------------------

def bf16_to_f64(bits: np.ndarray) -> np.ndarray:
    """bf16 bit patterns -> float64. A bf16 value is the top 16 bits of a float32."""
    b = np.asarray(bits)
    if b.dtype != np.uint16:
        raise TypeError("expected uint16 bf16 bit patterns")
    return (b.astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)


def round_to_bf16(a) -> np.ndarray:
    """Nearest bf16 value of each float64, ties to even, returned as float64.

    bf16 keeps 8 significant bits (the top half of an IEEE float32): with
    a = m·2^e, 0.5 <= |m| < 1, the result is rint(m·2^8)·2^(e-8), rint rounding
    halves to even. Exact in fp64 (one rounding, no pass through float32);
    values here stay far from bf16's overflow and subnormal range.
    """
    a = np.asarray(a, dtype=np.float64)
    m, e = np.frexp(a)
    return np.ldexp(np.rint(m * 256.0), e - 8)


def _f64(a) -> np.ndarray:
    """bf16 bit patterns (uint16) or any float array -> float64."""
    a = np.asarray(a)
    return bf16_to_f64(a) if a.dtype == np.uint16 else a.astype(np.float64)


# --- steps 1-3: projections ----------------------------------------------------

def project(x: np.ndarray, w: np.ndarray) -> np.ndarray:
    """Q = x·W_Q (and K, V alike), with W stored [out, in]: out[t, n] = sum_k x[t, k] W[n, k].

    Grouped-query attention page, "All 13 steps", the three projection
    equations; Query projection page, the [out, in] storage note.
    """
    return np.asarray(x, dtype=np.float64) @ np.asarray(w, dtype=np.float64).T


def split_heads(z: np.ndarray, n_heads: int) -> np.ndarray:
    """[..., T, n_heads*d_head] -> [..., T, n_heads, d_head]; feature n = d_head*h + d.

    Grouped-query attention page, model.py excerpt: the .view into heads.
    """
    *lead, f = z.shape
    return z.reshape(*lead, n_heads, f // n_heads)


# --- steps 4-5: pair rotation -------------------------------------------------

def rope_frequencies(d_head: int, theta: float = ROPE_THETA) -> np.ndarray:
    """ω_j = θ^(-2j/d_head) for j = 0 .. d_head/2 - 1 (catalogue rope_theta = 500000)."""
    j = np.arange(d_head // 2, dtype=np.float64)
    return np.exp(-(2.0 * j / d_head) * math.log(theta))


def rope_cos_sin(positions, d_head: int, theta: float = ROPE_THETA, omega=None):
    """cos(t·ω_j), sin(t·ω_j) in fp64, shape [len(positions), d_head/2].

    `omega` (d_head/2 frequencies) replaces θ^(-2j/d_head) when given: the
    block takes the table R as an input (Grouped-query attention page, in/out
    header), and the prime on ω in "All 13 steps" allows frequencies other
    than the plain ones (the 3.1 catalogue entry sets use_scaled_rope).
    """
    t = np.asarray(positions, dtype=np.float64)
    w = rope_frequencies(d_head, theta) if omega is None else np.asarray(omega, np.float64)
    ang = np.outer(t, w)
    return np.cos(ang), np.sin(ang)


def rope_rotate(z: np.ndarray, cos: np.ndarray, sin: np.ndarray) -> np.ndarray:
    """Rotate each adjacent pair (z_2j, z_2j+1) by the angle whose cos/sin are given.

    Grouped-query attention page, "All 13 steps", the 2x2 rotation display:
    z'_2j = cos·z_2j - sin·z_2j+1 and z'_2j+1 = sin·z_2j + cos·z_2j+1.
    z is [B, T, heads, d_head]; cos/sin are [T, d_head/2] and broadcast over
    batch and heads.
    """
    ze = z[..., 0::2]
    zo = z[..., 1::2]
    c = cos[None, :, None, :]
    s = sin[None, :, None, :]
    out = np.empty_like(z, dtype=np.float64)
    out[..., 0::2] = c * ze - s * zo
    out[..., 1::2] = s * ze + c * zo
    return out


# --- mask ------------------------------------------------------------------------

def causal_mask(T: int, start_pos: int = 0) -> np.ndarray:
    """Additive mask [T, start_pos+T]: -inf where key j > start_pos + i, else 0.

    Grouped-query attention page, model.py excerpt of the mask construction
    (upper triangle above the diagonal, with start_pos zero columns in front).
    """
    i = np.arange(T)[:, None]
    j = np.arange(start_pos + T)[None, :]
    m = np.zeros((T, start_pos + T), dtype=np.float64)
    m[j > start_pos + i] = -np.inf
    return m


# --- steps 6-11: grouped attention -------------------------------------------------

def softmax_rows(s: np.ndarray) -> np.ndarray:
    """A = exp(S)/sum_u exp(S) along the last axis (max subtracted first: same value)."""
    mx = np.max(s, axis=-1, keepdims=True)
    if not np.all(np.isfinite(mx)):
        raise ValueError("softmax of a row whose every key is masked is undefined")
    e = np.exp(s - mx)
    return e / np.sum(e, axis=-1, keepdims=True)


def grouped_attention(q_r: np.ndarray, k_all: np.ndarray, v_all: np.ndarray,
                      mask: Optional[np.ndarray], q_block: int = 512,
                      return_probs: bool = False):
    """H[b,:,h,:] = softmax(Q_r[b,:,h,:]·K_G[h]ᵀ/sqrt(d_head) + M)·V_G[h].

    Grouped-query attention page, "All 13 steps": K_G[h] = K_r[floor(h/4)],
    V_G[h] = V[floor(h/4)] (the group map; in general floor(h/n_rep) with
    n_rep = n_heads/n_kv, the repeat_kv excerpt's repeat_interleave), then
    S = Q_r K_Gᵀ, S_s = S/sqrt(128), S_m = S_s + M, A = softmax over keys,
    H = A V_G.

    q_r [B, T, n_heads, d_head]; k_all, v_all [B, S, n_kv, d_head];
    mask [T, S] additive or None. Queries are taken q_block rows at a time
    so the score block stays small. Returns H [B, T, n_heads, d_head]
    (and A [B, n_heads, T, S] if asked, for tiny shapes).
    """
    B, T, H, dh = q_r.shape
    G = k_all.shape[2]
    n_rep = H // G
    inv_sqrt = 1.0 / math.sqrt(dh)
    out = np.empty((B, T, H, dh), dtype=np.float64)
    probs = np.empty((B, H, T, k_all.shape[1])) if return_probs else None
    for b in range(B):
        for h in range(H):
            g = h // n_rep
            kg = k_all[b, :, g, :]
            vg = v_all[b, :, g, :]
            for t0 in range(0, T, q_block):
                t1 = min(T, t0 + q_block)
                s = (q_r[b, t0:t1, h, :] @ kg.T) * inv_sqrt
                if mask is not None:
                    s = s + mask[t0:t1]
                a = softmax_rows(s)
                if return_probs:
                    probs[b, h, t0:t1] = a
                out[b, t0:t1, h, :] = a @ vg
    return (out, probs) if return_probs else out


def merge_heads(h: np.ndarray) -> np.ndarray:
    """[B, T, n_heads, d_head] -> [B, T, n_heads*d_head], feature = d_head*h + d.

    Merge and project page, Explanation; the transpose(1, 2).view excerpt.
    """
    B, T, H, dh = h.shape
    return h.reshape(B, T, H * dh)


# --- whole block -----------------------------------------------------------------

def block_forward(x, wq, wk, wv, wo, n_heads: int, n_kv: int, *, causal: bool = True,
                  mask: Optional[np.ndarray] = None, start_pos: int = 0,
                  k_cache=None, v_cache=None, theta: float = ROPE_THETA,
                  return_probs: bool = False, omega=None) -> dict:
    """Δ_attn for x [B, T, d] (bf16 bits or float arrays), all in fp64.

    causal=True builds the mask of the model.py excerpt for this T and
    start_pos; causal=False uses `mask` ([T, start_pos+T] additive) or none.
    With start_pos > 0, k_cache/v_cache [B, >= start_pos, n_kv, d_head] hold
    the rotated keys and raw values of positions 0 .. start_pos-1.
    Returns the intermediates too: q, k, v, q_r, k_r, h (merged), delta.
    """
    def f64(a):
        a = np.asarray(a)
        return bf16_to_f64(a) if a.dtype == np.uint16 else a.astype(np.float64)

    x, wq, wk, wv, wo = (f64(a) for a in (x, wq, wk, wv, wo))
    B, T, _ = x.shape
    q = split_heads(project(x, wq), n_heads)
    k = split_heads(project(x, wk), n_kv)
    v = split_heads(project(x, wv), n_kv)
    dh = q.shape[-1]
    cos, sin = rope_cos_sin(np.arange(start_pos, start_pos + T), dh, theta, omega)
    q_r = rope_rotate(q, cos, sin)
    k_r = rope_rotate(k, cos, sin)
    if start_pos > 0:
        kc = f64(k_cache)[:, :start_pos]
        vc = f64(v_cache)[:, :start_pos]
        k_all = np.concatenate([kc, k_r], axis=1)
        v_all = np.concatenate([vc, v], axis=1)
    else:
        k_all, v_all = k_r, v
    if causal:
        m = causal_mask(T, start_pos) if T > 1 else None
    else:
        m = None if mask is None else np.asarray(mask, dtype=np.float64)
    res = grouped_attention(q_r, k_all, v_all, m, return_probs=return_probs)
    if return_probs:
        hh, probs = res
    else:
        hh, probs = res, None
    hm = merge_heads(hh)
    delta = project(hm, wo)
    out = dict(q=q, k=k, v=v, q_r=q_r, k_r=k_r, h=hm, delta=delta)
    if return_probs:
        out["probs"] = probs
    return out


def decode_forward(x, wq, wk, wv, wo, n_heads: int, n_kv: int, k_cache, v_cache,
                   start_pos: int, theta: float = ROPE_THETA) -> dict:
    """One new position per sequence at start_pos, attending over cache rows
    0 .. start_pos-1 plus the new token's own rotated key and value.

    x is [B, d]. The mask of the model.py excerpt is absent for a single
    position. Returns q_r [B, n_heads, d_head], the new k_r/v
    [B, n_kv, d_head], h [B, n_heads*d_head] and delta [B, d].
    """
    x = np.asarray(x)
    r = block_forward(x[:, None, :], wq, wk, wv, wo, n_heads, n_kv, causal=True,
                      start_pos=start_pos, k_cache=k_cache, v_cache=v_cache, theta=theta)
    return dict(q_r=r["q_r"][:, 0], k_r=r["k_r"][:, 0], v=r["v"][:, 0],
                h=r["h"][:, 0], delta=r["delta"][:, 0])


def block_forward_rows(x, wq, wk, wv, wo, n_heads: int, n_kv: int, rows,
                       theta: float = ROPE_THETA, batch_index: int = 0) -> dict:
    """Causal prefill (start_pos 0) evaluated only at the listed query positions
    of one sequence: keys and values are projected for every position up to the
    largest listed one, queries only for the listed rows. Same definition as
    block_forward; rows are checked one by one.

    Returns h [R, n_heads*d_head] and delta [R, d] for the sorted rows.
    """
    def f64(a):
        a = np.asarray(a)
        return bf16_to_f64(a) if a.dtype == np.uint16 else a.astype(np.float64)

    rows = np.asarray(sorted(set(int(r) for r in rows)), dtype=np.int64)
    last = int(rows[-1]) + 1
    xs = x[batch_index]
    wq, wk, wv, wo = (f64(a) for a in (wq, wk, wv, wo))
    dh = wq.shape[0] // n_heads
    # keys/values of positions 0..last-1, projected in slabs to bound memory
    k_r = np.empty((last, n_kv, dh))
    v = np.empty((last, n_kv, dh))
    slab = 8192
    for t0 in range(0, last, slab):
        t1 = min(last, t0 + slab)
        xb = f64(xs[t0:t1])
        kb = split_heads(project(xb, wk), n_kv)
        v[t0:t1] = split_heads(project(xb, wv), n_kv)
        cos, sin = rope_cos_sin(np.arange(t0, t1), dh, theta)
        k_r[t0:t1] = rope_rotate(kb[None], cos, sin)[0]
    xq = f64(xs[rows])
    q = split_heads(project(xq, wq), n_heads)
    cos, sin = rope_cos_sin(rows, dh, theta)
    q_r = rope_rotate(q[None], cos, sin)[0]           # [R, H, dh]
    n_rep = n_heads // n_kv
    inv_sqrt = 1.0 / math.sqrt(dh)
    h = np.empty((len(rows), n_heads, dh))
    keys = np.arange(last)
    for g in range(n_kv):
        kg = np.ascontiguousarray(k_r[:, g, :])        # [last, dh]
        vg = np.ascontiguousarray(v[:, g, :])
        for r0 in range(0, len(rows), 64):
            r1 = min(len(rows), r0 + 64)
            # additive causal mask of the sampled rows: -inf where key j > position t
            m = np.where(keys[None, :] > rows[r0:r1, None], -np.inf, 0.0)
            for hd in range(g * n_rep, (g + 1) * n_rep):
                s = (q_r[r0:r1, hd, :] @ kg.T) * inv_sqrt + m
                h[r0:r1, hd] = softmax_rows(s) @ vg
    hm = h.reshape(len(rows), n_heads * dh)
    return dict(rows=rows, h=hm, delta=project(hm, wo))


# --- the block's handoff: pre-norm and residual --------------------------------------
#
# The "Llama 3.1 8B · Merge and project" page, section "Contextual evidence from
# Output projection" (the model.py handoff excerpt), feeds the attention the
# normalised input attention_norm(x) and adds its update to x itself. The module
# there is RMSNorm(dim, eps=norm_eps) with norm_eps = 1e-5 (catalogue entry), but
# no page writes its formula out. Reading taken: root-mean-square layer
# normalisation (Zhang & Sennrich, 2019) with a learned per-feature gain and eps
# added under the root, evaluated exactly.
#
# The attention module's input is an activation of the model's bf16 data flow
# (as x itself is at this boundary), so by default x̂ is rounded once to bf16
# (nearest even) before the block; input_bf16=False keeps it exact.

def rms_norm(x, weight, eps: float = NORM_EPS) -> np.ndarray:
    """y[..., i] = weight[i] · x[..., i] / sqrt(mean over j of x[..., j]^2 + eps), fp64.

    Merge and project page, handoff excerpt (attention_norm), with the
    definition stated above.
    """
    x = _f64(x)
    w = _f64(weight)
    ms = np.mean(x * x, axis=-1, keepdims=True)
    return x / np.sqrt(ms + eps) * w


def prenorm_block_forward(x, norm_w, wq, wk, wv, wo, n_heads: int, n_kv: int, *,
                          eps: float = NORM_EPS, input_bf16: bool = True, **kw) -> dict:
    """out = x + Δ_attn(x̂), x̂ = rms_norm(x) (bf16-rounded when input_bf16): the
    attention half of the block with its handoff (Merge and project page,
    handoff excerpt). Other keyword arguments go to block_forward (causal,
    mask, start_pos, caches). Returns block_forward's intermediates plus
    x_norm (x̂ as fed to the block) and out."""
    x = _f64(x)
    xn = rms_norm(x, norm_w, eps)
    if input_bf16:
        xn = round_to_bf16(xn)
    r = block_forward(xn, wq, wk, wv, wo, n_heads, n_kv, **kw)
    r["x_norm"] = xn
    r["out"] = x + r["delta"]
    return r


def prenorm_decode_forward(x, norm_w, wq, wk, wv, wo, n_heads: int, n_kv: int, k_cache,
                           v_cache, start_pos: int, eps: float = NORM_EPS,
                           theta: float = ROPE_THETA, input_bf16: bool = True) -> dict:
    """decode_forward on x̂ = rms_norm(x) (bf16-rounded when input_bf16) plus the
    residual: out = x + Δ, x [B, d]."""
    x = _f64(x)
    xn = rms_norm(x, norm_w, eps)
    if input_bf16:
        xn = round_to_bf16(xn)
    r = decode_forward(xn, wq, wk, wv, wo, n_heads, n_kv, k_cache, v_cache, start_pos, theta)
    r["x_norm"] = xn
    r["out"] = x + r["delta"]
    return r


# --- the other half of the block: SwiGLU MLP ---------------------------------------------
#
# "Llama 3" page, section "SwiGLU MLP": three bias-free projections w1, w3
# (d -> d_ff) and w2 (d_ff -> d), stored [out, in] like the attention weights;
# output w2(silu(w1 x) * w3 x), silu(g) = g·σ(g), σ(z) = 1/(1 + e^-z); d_ff =
# 14336 (the SiLU panel's shapes). The block feeds it ffn_norm(h) and adds its
# update to h (Merge and project page, handoff excerpt): the same RMS
# normalisation and residual as the attention half.

D_FF = 14336


def silu(g) -> np.ndarray:
    """silu(g) = g / (1 + e^-g) in fp64 ("Llama 3" page, SiLU explanation).
    For g below about -709, e^-g overflows to inf and the value is -0, the limit."""
    g = np.asarray(g, dtype=np.float64)
    with np.errstate(over="ignore"):
        return g / (1.0 + np.exp(-g))


def mlp_forward(x, w1, w2, w3) -> dict:
    """out = w2(silu(w1 x) · w3 x) for x [..., d], all in fp64.
    Returns the gate g = x·w1ᵀ, up u = x·w3ᵀ, a = silu(g)·u and delta = a·w2ᵀ."""
    x, w1, w2, w3 = (_f64(t) for t in (x, w1, w2, w3))
    g = project(x, w1)
    u = project(x, w3)
    a = silu(g) * u
    return dict(g=g, u=u, a=a, delta=project(a, w2))


def prenorm_mlp_forward(h, norm_w, w1, w2, w3, eps: float = NORM_EPS,
                        input_bf16: bool = True) -> dict:
    """out = h + mlp(ĥ), ĥ = rms_norm(h) (bf16-rounded when input_bf16, the MLP's
    input being a bf16 activation), h [..., d]."""
    h = _f64(h)
    hn = rms_norm(h, norm_w, eps)
    if input_bf16:
        hn = round_to_bf16(hn)
    r = mlp_forward(hn, w1, w2, w3)
    r["x_norm"] = hn
    r["out"] = h + r["delta"]
    return r


def param_counts(d: int, n_heads: int, n_kv: int) -> dict:
    """Weight-element counts of one block for the given dims (head width d/n_heads)."""
    dh = d // n_heads
    q = (n_heads * dh) * d
    k = (n_kv * dh) * d
    v = (n_kv * dh) * d
    o = d * (n_heads * dh)
    return dict(q=q, k=k, v=v, o=o, total=q + k + v + o, head_dim=dh)
