"""Python binding of libgqa, the MI355X (gfx950) grouped-query-attention block library.

Argument marshalling only: every step of the block runs in the library's HIP
kernels. torch supplies device memory and the current stream; tensors are
passed to the C ABI as raw pointers. There is no fallback: if libgqa.so is
missing or cannot be loaded, every call raises.

Names follow include/gqa.h:
    block_forward, chunk_forward, decode_forward (each with a pre-norm and
    residual form: norm_w=... ), qkv_rope, attention, output_projection,
    decode_attention, rmsnorm, rope_table, the *_workspace_bytes sizes, dims.
"""

from __future__ import annotations

import ctypes
import os
from typing import Optional

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libgqa.so")

D_MODEL, N_HEADS, N_KV_HEADS, D_HEAD, N_PAIRS = 4096, 32, 8, 128, 64
D_FF = 14336
ROPE_THETA = 500000.0
NORM_EPS = 1e-5

_lib = None


class GQAError(RuntimeError):
    """A libgqa entry point returned a non-zero status."""

    def __init__(self, fn: str, status: int):
        msg = _load().gqa_status_string(status).decode()
        super().__init__(f"{fn}: {msg} (status {status})")
        self.status = status


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"libgqa.so not built at {LIB_PATH}; run "
                           "`python -m grouped_query_attention_amd.build`")
    lib = ctypes.CDLL(LIB_PATH)
    P, I, Z, D = ctypes.c_void_p, ctypes.c_int, ctypes.c_size_t, ctypes.c_double
    F = ctypes.c_float
    sig = {
        "gqa_status_string": (ctypes.c_char_p, [I]),
        "gqa_dims": (None, [P, P, P, P]),
        "gqa_rope_table": (I, [P, I, D, P]),
        "gqa_rope_table_freqs": (I, [P, I, P, P]),
        "gqa_prefill_workspace_bytes": (Z, [I, I]),
        "gqa_decode_workspace_bytes": (Z, [I, I]),
        "gqa_attention_workspace_bytes": (Z, [I, I, I, I]),
        "gqa_chunk_workspace_bytes": (Z, [I, I, I]),
        "gqa_chunk_forward": (I, [P, P, P, P, P, P, P, P, I, I, I, I, P, P, P, Z, P]),
        "gqa_block_forward": (I, [P, P, P, P, P, P, P, I, I, I, I, P, P, P, Z, P]),
        "gqa_decode_forward": (I, [P, P, P, P, P, P, P, P, I, I, I, P, P, P, Z, P]),
        "gqa_decode_forward_static": (I, [P, P, P, P, P, P, P, P, I, I, I, P, P, P]),
        "gqa_qkv_rope": (I, [P, P, P, P, P, I, I, P, P, P, I, P]),
        "gqa_attention": (I, [P, P, P, P, I, I, I, I, P, P, Z, I, P]),
        "gqa_output_projection": (I, [P, P, I, P, P]),
        "gqa_decode_attention": (I, [P, P, P, I, I, I, P, P, Z, P]),
        "gqa_block_forward_prenorm": (I, [P, P, F, P, P, P, P, P, P, I, I, I, I, P, P, P, Z,
                                          P]),
        "gqa_chunk_forward_prenorm": (I, [P, P, F, P, P, P, P, P, P, P, I, I, I, I, P, P, P,
                                          Z, P]),
        "gqa_decode_forward_prenorm": (I, [P, P, F, P, P, P, P, P, P, P, I, I, I, P, P, P, Z,
                                           P]),
        "gqa_rmsnorm": (I, [P, P, F, I, P, P]),
        "gqa_mlp_workspace_bytes": (Z, [I]),
        "gqa_mlp_forward": (I, [P, P, P, P, I, P, P, P, Z, P]),
        "gqa_mlp_forward_prenorm": (I, [P, P, F, P, P, P, I, P, P, P, Z, P]),
    }
    for name, (res, args) in sig.items():
        f = getattr(lib, name)
        f.restype = res
        f.argtypes = args
    _lib = lib
    return lib


def lib():
    """The loaded ctypes library (raises if it is not built)."""
    return _load()


def exported_symbols():
    return ["gqa_status_string", "gqa_dims", "gqa_rope_table", "gqa_rope_table_freqs",
            "gqa_prefill_workspace_bytes",
            "gqa_decode_workspace_bytes", "gqa_attention_workspace_bytes",
            "gqa_chunk_workspace_bytes", "gqa_block_forward", "gqa_chunk_forward",
            "gqa_decode_forward", "gqa_decode_forward_static",
            "gqa_qkv_rope", "gqa_attention", "gqa_output_projection", "gqa_decode_attention",
            "gqa_block_forward_prenorm", "gqa_chunk_forward_prenorm",
            "gqa_decode_forward_prenorm", "gqa_rmsnorm", "gqa_mlp_workspace_bytes",
            "gqa_mlp_forward", "gqa_mlp_forward_prenorm"]


# --- helpers -------------------------------------------------------------------------

def _ptr(t) -> Optional[int]:
    if t is None:
        return None
    return t.data_ptr()


def _stream(stream) -> Optional[int]:
    import torch
    if stream is None:
        stream = torch.cuda.current_stream()
    return stream.cuda_stream


def _check(fn: str, st: int):
    if st != 0:
        raise GQAError(fn, st)


def _req(t, dtype, shape, name):
    import torch
    if t.dtype != dtype:
        raise TypeError(f"{name}: expected {dtype}, got {t.dtype}")
    if not t.is_cuda:
        raise ValueError(f"{name}: expected a device tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name}: expected a contiguous tensor")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name}: expected shape {tuple(shape)}, got {tuple(t.shape)}")
    return t


# --- host-side entries ----------------------------------------------------------------

def dims():
    a, b, c, d = (ctypes.c_int() for _ in range(4))
    _load().gqa_dims(ctypes.byref(a), ctypes.byref(b), ctypes.byref(c), ctypes.byref(d))
    return a.value, b.value, c.value, d.value


def rope_table(positions, theta: float = ROPE_THETA, omega=None) -> np.ndarray:
    """(cos, sin) table [n, 64, 2] float32 for the given positions (host computation).

    omega: optional 64 explicit per-pair frequencies in place of theta^(-2j/128).
    """
    pos = np.ascontiguousarray(np.asarray(positions, dtype=np.int32))
    out = np.empty((pos.size, N_PAIRS, 2), dtype=np.float32)
    pp = pos.ctypes.data if pos.size else None
    po = out.ctypes.data if pos.size else None
    if omega is None:
        _check("gqa_rope_table", _load().gqa_rope_table(pp, int(pos.size), float(theta), po))
    else:
        w = np.ascontiguousarray(np.asarray(omega, dtype=np.float64))
        if w.shape != (N_PAIRS,):
            raise ValueError(f"omega: expected {N_PAIRS} frequencies, got shape {w.shape}")
        _check("gqa_rope_table_freqs",
               _load().gqa_rope_table_freqs(pp, int(pos.size), w.ctypes.data, po))
    return out


def prefill_workspace_bytes(B: int, T: int) -> int:
    return int(_load().gqa_prefill_workspace_bytes(B, T))


def decode_workspace_bytes(B: int, S_max: int) -> int:
    return int(_load().gqa_decode_workspace_bytes(B, S_max))


def chunk_workspace_bytes(B: int, T: int, start_pos: int) -> int:
    return int(_load().gqa_chunk_workspace_bytes(B, T, int(start_pos)))


def attention_workspace_bytes(B: int, T: int, kv_len: int, causal: bool = True) -> int:
    return int(_load().gqa_attention_workspace_bytes(B, T, kv_len, int(bool(causal))))


# --- device entries -------------------------------------------------------------------

def block_forward(x, w_q, w_k, w_v, w_o, rope, *, causal: bool = True, mask=None,
                  out=None, h_out=None, workspace=None, norm_w=None, eps: float = NORM_EPS,
                  stream=None):
    """Δ = GQA block forward for x [B, T, 4096] bf16; returns out [B, T, 4096] fp32.

    With norm_w ([4096] bf16 gain) the block reads RMSNorm(x) and returns x + Δ.
    """
    import torch
    B, T, _ = x.shape
    _req(x, torch.bfloat16, (B, T, D_MODEL), "x")
    _req(rope, torch.float32, (T, N_PAIRS, 2), "rope")
    if mask is not None:
        _req(mask, torch.float32, (T, T), "mask")
    if out is None:
        out = torch.empty((B, T, D_MODEL), dtype=torch.float32, device=x.device)
    _req(out, torch.float32, (B, T, D_MODEL), "out")
    if h_out is not None:
        _req(h_out, torch.bfloat16, (B, T, N_HEADS, D_HEAD), "h_out")
    need = prefill_workspace_bytes(B, T)
    if workspace is None:
        workspace = torch.empty(need, dtype=torch.uint8, device=x.device)
    args = (_ptr(w_q), _ptr(w_k), _ptr(w_v), _ptr(w_o), _ptr(rope), _ptr(mask),
            int(bool(causal)), B, T, T, _ptr(out), _ptr(h_out), _ptr(workspace),
            workspace.numel() * workspace.element_size(), _stream(stream))
    if norm_w is None:
        _check("gqa_block_forward", _load().gqa_block_forward(_ptr(x), *args))
    else:
        _req(norm_w, torch.bfloat16, (D_MODEL,), "norm_w")
        _check("gqa_block_forward_prenorm",
               _load().gqa_block_forward_prenorm(_ptr(x), _ptr(norm_w), float(eps), *args))
    return out


def decode_forward(x, w_q, w_k, w_v, w_o, rope, k_cache, v_cache, start_pos: int, *,
                   out=None, h_out=None, workspace=None, norm_w=None, eps: float = NORM_EPS,
                   stream=None):
    """One new position per sequence at start_pos; x [B, 4096]; returns out [B, 4096] fp32.

    Writes the new rotated key and value into cache slot start_pos. With norm_w
    the block reads RMSNorm(x) and returns x + Δ.
    """
    import torch
    B = x.shape[0]
    S_max = k_cache.shape[1]
    _req(x, torch.bfloat16, (B, D_MODEL), "x")
    _req(rope, torch.float32, (N_PAIRS, 2), "rope")
    _req(k_cache, torch.bfloat16, (B, S_max, N_KV_HEADS, D_HEAD), "k_cache")
    _req(v_cache, torch.bfloat16, (B, S_max, N_KV_HEADS, D_HEAD), "v_cache")
    if out is None:
        out = torch.empty((B, D_MODEL), dtype=torch.float32, device=x.device)
    if workspace is None:
        workspace = torch.empty(decode_workspace_bytes(B, S_max), dtype=torch.uint8,
                                device=x.device)
    args = (_ptr(w_q), _ptr(w_k), _ptr(w_v), _ptr(w_o), _ptr(rope), _ptr(k_cache),
            _ptr(v_cache), B, S_max, int(start_pos), _ptr(out), _ptr(h_out), _ptr(workspace),
            workspace.numel() * workspace.element_size(), _stream(stream))
    if norm_w is None:
        _check("gqa_decode_forward", _load().gqa_decode_forward(_ptr(x), *args))
    else:
        _req(norm_w, torch.bfloat16, (D_MODEL,), "norm_w")
        _check("gqa_decode_forward_prenorm",
               _load().gqa_decode_forward_prenorm(_ptr(x), _ptr(norm_w), float(eps), *args))
    return out


STATIC_SCRATCH_BYTES = 32 << 20


def decode_forward_static(x, w_q, w_k, w_v, w_o, rope, k_cache, v_cache, start_pos: int, *,
                          out=None, h_out=None, stream=None):
    """decode_forward without a workspace: the library's fixed per-GPU device
    array (STATIC_SCRATCH_BYTES) holds the step's scratch, so the call allocates
    nothing when `out` is given. Calls that overlap in time on one GPU race."""
    import torch
    B = x.shape[0]
    S_max = k_cache.shape[1]
    _req(x, torch.bfloat16, (B, D_MODEL), "x")
    _req(rope, torch.float32, (N_PAIRS, 2), "rope")
    _req(k_cache, torch.bfloat16, (B, S_max, N_KV_HEADS, D_HEAD), "k_cache")
    _req(v_cache, torch.bfloat16, (B, S_max, N_KV_HEADS, D_HEAD), "v_cache")
    if out is None:
        out = torch.empty((B, D_MODEL), dtype=torch.float32, device=x.device)
    _req(out, torch.float32, (B, D_MODEL), "out")
    if h_out is not None:
        _req(h_out, torch.bfloat16, (B, N_HEADS, D_HEAD), "h_out")
    _check("gqa_decode_forward_static", _load().gqa_decode_forward_static(
        _ptr(x), _ptr(w_q), _ptr(w_k), _ptr(w_v), _ptr(w_o), _ptr(rope), _ptr(k_cache),
        _ptr(v_cache), B, S_max, int(start_pos), _ptr(out), _ptr(h_out), _stream(stream)))
    return out


def chunk_forward(x, w_q, w_k, w_v, w_o, rope, k_cache, v_cache, start_pos: int, *,
                  out=None, h_out=None, workspace=None, norm_w=None, eps: float = NORM_EPS,
                  stream=None):
    """T new positions per sequence at start_pos .. start_pos+T-1 over a KV cache
    holding positions 0 .. start_pos-1; x [B, T, 4096]; returns out [B, T, 4096] fp32.

    Writes the new rotated keys and values into cache slots start_pos .. start_pos+T-1.
    With norm_w the block reads RMSNorm(x) and returns x + Δ.
    """
    import torch
    B, T, _ = x.shape
    S_max = k_cache.shape[1]
    _req(x, torch.bfloat16, (B, T, D_MODEL), "x")
    _req(rope, torch.float32, (T, N_PAIRS, 2), "rope")
    _req(k_cache, torch.bfloat16, (B, S_max, N_KV_HEADS, D_HEAD), "k_cache")
    _req(v_cache, torch.bfloat16, (B, S_max, N_KV_HEADS, D_HEAD), "v_cache")
    if out is None:
        out = torch.empty((B, T, D_MODEL), dtype=torch.float32, device=x.device)
    if workspace is None:
        workspace = torch.empty(chunk_workspace_bytes(B, T, start_pos), dtype=torch.uint8,
                                device=x.device)
    args = (_ptr(w_q), _ptr(w_k), _ptr(w_v), _ptr(w_o), _ptr(rope), _ptr(k_cache),
            _ptr(v_cache), B, T, S_max, int(start_pos), _ptr(out), _ptr(h_out),
            _ptr(workspace), workspace.numel() * workspace.element_size(), _stream(stream))
    if norm_w is None:
        _check("gqa_chunk_forward", _load().gqa_chunk_forward(_ptr(x), *args))
    else:
        _req(norm_w, torch.bfloat16, (D_MODEL,), "norm_w")
        _check("gqa_chunk_forward_prenorm",
               _load().gqa_chunk_forward_prenorm(_ptr(x), _ptr(norm_w), float(eps), *args))
    return out


def rmsnorm(x, norm_w, eps: float = NORM_EPS, *, y=None, stream=None):
    """y = RMSNorm(x) (bf16, same shape) for x [..., 4096] bf16 and gain norm_w [4096]."""
    import torch
    _req(x, torch.bfloat16, None, "x")
    _req(norm_w, torch.bfloat16, (D_MODEL,), "norm_w")
    if x.shape[-1] != D_MODEL:
        raise ValueError(f"x: last dimension must be {D_MODEL}")
    M = x.numel() // D_MODEL
    if y is None:
        y = torch.empty_like(x)
    _req(y, torch.bfloat16, tuple(x.shape), "y")
    _check("gqa_rmsnorm", _load().gqa_rmsnorm(_ptr(x), _ptr(norm_w), float(eps), M, _ptr(y),
                                              _stream(stream)))
    return y


def mlp_workspace_bytes(M: int) -> int:
    return int(_load().gqa_mlp_workspace_bytes(M))


def mlp_forward(x, w1, w2, w3, *, norm_w=None, eps: float = NORM_EPS, out=None, a_out=None,
                workspace=None, stream=None):
    """SwiGLU MLP: out = w2(silu(x·w1ᵀ)·(x·w3ᵀ)) for x [..., 4096] bf16; fp32 out of
    the same leading shape. With norm_w the MLP reads RMSNorm(x) and out = x + MLP."""
    import torch
    _req(x, torch.bfloat16, None, "x")
    if x.shape[-1] != D_MODEL:
        raise ValueError(f"x: last dimension must be {D_MODEL}")
    M = x.numel() // D_MODEL
    _req(w1, torch.bfloat16, (D_FF, D_MODEL), "w1")
    _req(w3, torch.bfloat16, (D_FF, D_MODEL), "w3")
    _req(w2, torch.bfloat16, (D_MODEL, D_FF), "w2")
    if out is None:
        out = torch.empty(tuple(x.shape), dtype=torch.float32, device=x.device)
    _req(out, torch.float32, tuple(x.shape), "out")
    if a_out is not None:
        _req(a_out, torch.bfloat16, None, "a_out")
        if a_out.numel() != M * D_FF:
            raise ValueError(f"a_out: expected {M * D_FF} elements")
    if workspace is None:
        workspace = torch.empty(mlp_workspace_bytes(M), dtype=torch.uint8, device=x.device)
    wsb = workspace.numel() * workspace.element_size()
    if norm_w is None:
        _check("gqa_mlp_forward", _load().gqa_mlp_forward(
            _ptr(x), _ptr(w1), _ptr(w2), _ptr(w3), M, _ptr(out), _ptr(a_out), _ptr(workspace),
            wsb, _stream(stream)))
    else:
        _req(norm_w, torch.bfloat16, (D_MODEL,), "norm_w")
        _check("gqa_mlp_forward_prenorm", _load().gqa_mlp_forward_prenorm(
            _ptr(x), _ptr(norm_w), float(eps), _ptr(w1), _ptr(w2), _ptr(w3), M, _ptr(out),
            _ptr(a_out), _ptr(workspace), wsb, _stream(stream)))
    return out


def qkv_rope(x, w_q, w_k, w_v, rope, *, q_r=None, k_r=None, v=None, q_scaled: bool = False,
             stream=None):
    """Q_r [B,T,32,128], K_r [B,T,8,128], V [B,T,8,128] (bf16) for x [B,T,4096].

    q_scaled: Q_r comes out multiplied by log2(e)/sqrt(128), the form the block's
    own attention stage takes (attention(..., q_scaled=True)).
    """
    import torch
    B, T, _ = x.shape
    _req(x, torch.bfloat16, (B, T, D_MODEL), "x")
    dev = x.device
    if q_r is None:
        q_r = torch.empty((B, T, N_HEADS, D_HEAD), dtype=torch.bfloat16, device=dev)
    if k_r is None:
        k_r = torch.empty((B, T, N_KV_HEADS, D_HEAD), dtype=torch.bfloat16, device=dev)
    if v is None:
        v = torch.empty((B, T, N_KV_HEADS, D_HEAD), dtype=torch.bfloat16, device=dev)
    st = _load().gqa_qkv_rope(_ptr(x), _ptr(w_q), _ptr(w_k), _ptr(w_v), _ptr(rope), B, T,
                              _ptr(q_r), _ptr(k_r), _ptr(v), int(bool(q_scaled)),
                              _stream(stream))
    _check("gqa_qkv_rope", st)
    return q_r, k_r, v


def attention(q_r, k_r, v, *, causal: bool = True, mask=None, h_out=None, workspace=None,
              balanced: bool = True, q_scaled: bool = False, stream=None):
    """H [B,T,32,128] bf16 from rotated queries/keys and values. With `balanced`
    (default) a causal launch of few query tiles gets its workspace (allocated
    here unless given); balanced=False runs the plain launch. q_scaled: the
    queries carry the factor log2(e)/sqrt(128) (qkv_rope(..., q_scaled=True)),
    the kernel the block runs."""
    import torch
    B, T = q_r.shape[:2]
    kv_len = k_r.shape[1]
    if h_out is None:
        h_out = torch.empty((B, T, N_HEADS, D_HEAD), dtype=torch.bfloat16, device=q_r.device)
    if balanced and workspace is None:
        nb = attention_workspace_bytes(B, T, kv_len, causal)
        if nb:
            workspace = torch.empty(nb, dtype=torch.uint8, device=q_r.device)
    if not balanced:
        workspace = None
    wsb = 0 if workspace is None else workspace.numel() * workspace.element_size()
    st = _load().gqa_attention(_ptr(q_r), _ptr(k_r), _ptr(v), _ptr(mask), int(bool(causal)),
                               B, T, kv_len, _ptr(h_out), _ptr(workspace), wsb,
                               int(bool(q_scaled)), _stream(stream))
    _check("gqa_attention", st)
    return h_out


def output_projection(h, w_o, *, out=None, stream=None):
    """out [M,4096] fp32 = h [M,4096] bf16 · w_oᵀ (h may be [B,T,32,128])."""
    import torch
    M = h.numel() // D_MODEL
    if out is None:
        out = torch.empty((M, D_MODEL), dtype=torch.float32, device=h.device)
    st = _load().gqa_output_projection(_ptr(h), _ptr(w_o), M, _ptr(out), _stream(stream))
    _check("gqa_output_projection", st)
    return out


def decode_attention(q_r, k_cache, v_cache, kv_len: int, *, h_out=None, workspace=None,
                     stream=None):
    """H [B,32,128] bf16 for queries q_r [B,32,128] over cache keys 0..kv_len-1."""
    import torch
    B, S_max = k_cache.shape[:2]
    if h_out is None:
        h_out = torch.empty((B, N_HEADS, D_HEAD), dtype=torch.bfloat16, device=q_r.device)
    if workspace is None:
        workspace = torch.empty(decode_workspace_bytes(B, S_max), dtype=torch.uint8,
                                device=q_r.device)
    st = _load().gqa_decode_attention(_ptr(q_r), _ptr(k_cache), _ptr(v_cache), B, S_max,
                                      int(kv_len), _ptr(h_out), _ptr(workspace),
                                      workspace.numel() * workspace.element_size(),
                                      _stream(stream))
    _check("gqa_decode_attention", st)
    return h_out
