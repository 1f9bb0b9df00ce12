"""Seeded synthetic inputs for the grouped-query-attention block.

This module holds random-number generation and float32 -> bf16 rounding only.
It contains none of the block's arithmetic (no projection, rotation, softmax
or mask), so the oracle side and the GPU side can both take their inputs from
here without sharing any of the method.

Value recipe (Llama 3.1 8B attention block shapes from the "Grouped-query
attention" page, parameter table and in/out header):
  * weights W_Q [4096,4096], W_K [1024,4096], W_V [1024,4096], W_O [4096,4096],
    stored [out, in] as the "Query projection" page notes; N(0, 0.02^2);
  * block input x [B, T, 4096] ~ N(0, 1);
  * decode K/V cache [B, S_max, 8, 128] ~ N(0, 1);
  * gain of the pre-attention RMS normalisation [4096] ~ 1 + N(0, 0.2^2), from
    a stream of its own (make_norm_weight);
  * SwiGLU MLP ("Llama 3" page): w1, w3 [14336, 4096], w2 [4096, 14336] ~
    N(0, 0.02^2), input [M, 4096] ~ N(0, 1), from a stream of their own
    (make_mlp_inputs).
Each value is drawn as a float32 standard normal from numpy's PCG64 generator,
scaled by the standard deviation in float32 and rounded to bf16 with
round-to-nearest-even. Generation order: W_Q, W_K, W_V, W_O, x, cache K,
cache V. Arrays are returned as uint16 bf16 bit patterns.
"""

from __future__ import annotations

from dataclasses import dataclass
from typing import Optional

import numpy as np

D_MODEL = 4096
N_HEADS = 32
N_KV_HEADS = 8
D_HEAD = 128
D_FF = 14336

_CHUNK = 1 << 24  # values drawn per step, bounds the float32 temporaries


def f32_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """Round float32 values to bf16 (nearest, ties to even); return uint16 bits."""
    a = np.ascontiguousarray(a, dtype=np.float32)
    u = a.view(np.uint32)
    bias = np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))
    return ((u + bias) >> np.uint32(16)).astype(np.uint16)


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    """Widen bf16 bit patterns to float32 (exact)."""
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def normal_bf16(rng: np.random.Generator, shape, std: float) -> np.ndarray:
    """Draw N(0, std^2) float32 values in chunks and round them to bf16 bits."""
    n = int(np.prod(shape))
    out = np.empty(n, dtype=np.uint16)
    s = np.float32(std)
    for lo in range(0, n, _CHUNK):
        hi = min(n, lo + _CHUNK)
        v = rng.standard_normal(hi - lo, dtype=np.float32)
        if s != np.float32(1.0):
            v *= s
        out[lo:hi] = f32_to_bf16_bits(v)
    return out.reshape(shape)


@dataclass
class BlockInputs:
    """bf16 bit patterns (uint16) of one block's weights and input."""

    x: np.ndarray            # [B, T, d]
    wq: np.ndarray           # [n_heads*d_head, d]
    wk: np.ndarray           # [n_kv*d_head, d]
    wv: np.ndarray           # [n_kv*d_head, d]
    wo: np.ndarray           # [d, n_heads*d_head]
    k_cache: Optional[np.ndarray] = None  # [B, S_max, n_kv, d_head]
    v_cache: Optional[np.ndarray] = None  # [B, S_max, n_kv, d_head]


def make_block_inputs(seed: int, B: int, T: int, *, d: int = D_MODEL,
                      n_heads: int = N_HEADS, n_kv: int = N_KV_HEADS,
                      d_head: int = D_HEAD, w_std: float = 0.02,
                      x_std: float = 1.0, cache_len: int = 0,
                      cache_std: float = 1.0) -> BlockInputs:
    """Seeded weights, block input and (if cache_len > 0) a K/V cache."""
    rng = np.random.Generator(np.random.PCG64(seed))
    wq = normal_bf16(rng, (n_heads * d_head, d), w_std)
    wk = normal_bf16(rng, (n_kv * d_head, d), w_std)
    wv = normal_bf16(rng, (n_kv * d_head, d), w_std)
    wo = normal_bf16(rng, (d, n_heads * d_head), w_std)
    x = normal_bf16(rng, (B, T, d), x_std)
    kc = vc = None
    if cache_len > 0:
        kc = normal_bf16(rng, (B, cache_len, n_kv, d_head), cache_std)
        vc = normal_bf16(rng, (B, cache_len, n_kv, d_head), cache_std)
    return BlockInputs(x=x, wq=wq, wk=wk, wv=wv, wo=wo, k_cache=kc, v_cache=vc)


@dataclass
class MlpInputs:
    """bf16 bit patterns (uint16) of the SwiGLU MLP's weights and input."""

    x: np.ndarray            # [M, d]
    w1: np.ndarray           # [d_ff, d]  gate
    w3: np.ndarray           # [d_ff, d]  up
    w2: np.ndarray           # [d, d_ff]  down


def make_mlp_inputs(seed: int, M: int, *, d: int = D_MODEL, d_ff: int = D_FF,
                    w_std: float = 0.02, x_std: float = 1.0) -> MlpInputs:
    """Seeded MLP weights N(0, w_std^2) and input N(0, x_std^2), bf16 (nearest
    even). Generation order: w1, w3, w2, x."""
    rng = np.random.Generator(np.random.PCG64(seed + 15485863))
    w1 = normal_bf16(rng, (d_ff, d), w_std)
    w3 = normal_bf16(rng, (d_ff, d), w_std)
    w2 = normal_bf16(rng, (d, d_ff), w_std)
    x = normal_bf16(rng, (M, d), x_std)
    return MlpInputs(x=x, w1=w1, w3=w3, w2=w2)


def make_norm_weight(seed: int, d: int = D_MODEL, std: float = 0.2) -> np.ndarray:
    """Gain of the pre-attention RMS normalisation: bf16 bits of 1 + N(0, std^2)
    per feature (float32, rounded to nearest even). A trained gain is not all
    ones; the spread makes a gain applied to the wrong feature visible. Drawn
    from its own stream so that the block inputs of a seed are unchanged."""
    rng = np.random.Generator(np.random.PCG64(seed + 104729))
    v = np.float32(1.0) + rng.standard_normal(d, dtype=np.float32) * np.float32(std)
    return f32_to_bf16_bits(v)


def sample_positions(seed: int, T: int, per_group: int = 64, n_groups: int = N_KV_HEADS,
                     tile_edges=(127, 128, 4095, 4096, 65535, 65536)) -> np.ndarray:
    """Sorted distinct query positions to check at long T.

    per_group seeded positions for each KV-head group, plus 0, 1, T-1 and
    the listed tile edges that fall inside [0, T).
    """
    rng = np.random.Generator(np.random.PCG64(seed + 7919))
    fixed = [p for p in (0, 1, T - 1, *tile_edges) if 0 <= p < T]
    rand = rng.integers(0, T, size=per_group * n_groups)
    return np.unique(np.concatenate([np.asarray(fixed, dtype=np.int64), rand]))
