"""Helpers shared by the GPU tests: host <-> device transfer of bf16 bit
patterns and the comparison metrics (no arithmetic of the block)."""

import numpy as np
import torch


def dev():
    if not torch.cuda.is_available():
        raise RuntimeError("GPU tests need a visible MI355X")
    return torch.device("cuda:0")


def to_dev_bf16(bits: np.ndarray) -> torch.Tensor:
    """uint16 bf16 bit patterns -> device bf16 tensor of the same shape."""
    t = torch.from_numpy(np.ascontiguousarray(bits).view(np.int16))
    return t.to(dev()).view(torch.bfloat16)


def to_dev_f32(a: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(dev())


def bf16_to_np_f64(t: torch.Tensor) -> np.ndarray:
    bits = t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)
    return (bits.astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)


def f32_to_np_f64(t: torch.Tensor) -> np.ndarray:
    return t.detach().cpu().numpy().astype(np.float64)


def rel_l2(got: np.ndarray, want: np.ndarray) -> float:
    return float(np.linalg.norm((got - want).ravel()) / np.linalg.norm(want.ravel()))


def max_abs(got: np.ndarray, want: np.ndarray) -> float:
    return float(np.max(np.abs(got - want)))


# Tolerances of the block output Δ against the fp64 oracle (bf16 inputs,
# fp32 accumulation): relative L2 error and largest absolute error.
REL_L2_TOL = 5e-3
MAX_ABS_TOL = 2e-2


def assert_close(got, want, rel=REL_L2_TOL, mabs=MAX_ABS_TOL, what=""):
    assert np.all(np.isfinite(got)), f"{what}: non-finite values"
    r, m = rel_l2(got, want), max_abs(got, want)
    print(f"[parity] {what}: relL2={r:.3e} maxabs={m:.3e}", flush=True)
    assert r <= rel, f"{what}: relL2 {r:.3e} > {rel}"
    assert m <= mabs, f"{what}: max abs {m:.3e} > {mabs}"
    return r, m
