"""Helpers shared by the GPU parity tests: run the HIP path, compare with the
fp64 oracle element by element and report the worst element."""
from __future__ import annotations

import math

import numpy as np
import torch

# Tolerances (max-abs): fp32 path 1e-5 (the atol of the page's own fp32
# comparison in "Efficient Attention"), bf16 inputs with fp32 accumulation
# 2e-2, float32 LSE 1e-4.
TOL_F32 = 1e-5
TOL_BF16 = 2e-2
TOL_LSE = 1e-4


def tol_for(dtype: torch.dtype) -> float:
    return TOL_F32 if dtype == torch.float32 else TOL_BF16


def require_gpu() -> torch.device:
    if not torch.cuda.is_available():
        raise RuntimeError("GPU tests need a visible MI355X (torch.cuda.is_available() is False)")
    return torch.device("cuda:0")


def np64(t: torch.Tensor) -> np.ndarray:
    return t.detach().to("cpu", torch.float64).numpy()


# bf16 backward bound outside the workloads.  Each gradient is a sum of
# products whose bf16-rounded factor (P or dS) carries a relative error up to
# 2^-9, and the result is rounded to bf16 once more (2^-9 of its magnitude,
# which is at most the sum of the absolute terms).  Both together are bounded
# by 2^-8 * sum |terms|; the tests allow twice that on top of the 2e-2 set for
# the O(1) gradients of the workloads.  The sums of absolute terms are
#   dQ: scale |dS| |K|,  dK: scale |dS|^T |Q|,  dV: |P|^T |dO|.
RTOL_BF16_TERMS = 2.0 ** -7


def fp32_score_tol(q, k, v, scale) -> float:
    """fp32 max-abs bound for inputs whose scores are far from N(0, 1).

    A float32 dot product of d terms carries a rounding error of about
    sqrt(d) * 2^-24 * sum_c |q_c k_c|; after scaling, that error moves each
    probability by the same relative amount, so O moves by up to that much
    times max |V|.  Returns max(1e-5, 8x that estimate).
    """
    qa, ka = np.abs(np64(q)), np.abs(np64(k))
    d = qa.shape[-1]
    worst = float(np.max(np.matmul(qa, np.swapaxes(ka, -1, -2)))) * scale
    return max(TOL_F32, 8 * math.sqrt(d) * 2.0 ** -24 * worst * float(np.max(np.abs(np64(v)))))


def assert_close(name: str, got, ref, tol: float, rtol: float = 0.0, mag=None) -> float:
    """Element-wise |got - ref| <= tol + rtol * mag (mag defaults to |ref|);
    prints the worst element."""
    got = np64(got) if isinstance(got, torch.Tensor) else np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert got.shape == ref.shape, f"{name}: shape {got.shape} vs {ref.shape}"
    assert np.all(np.isfinite(got)), f"{name}: non-finite values"
    err = np.abs(got - ref)
    mag = np.abs(ref) if mag is None else np.asarray(mag, dtype=np.float64)
    excess = err - (tol + rtol * mag)
    idx = np.unravel_index(int(np.argmax(excess)), err.shape)
    worst = float(np.max(err))
    msg = (f"{name}: max |err| {worst:.3e}; worst vs bound at {tuple(int(i) for i in idx)} "
           f"(got {got[idx]:.6g}, ref {ref[idx]:.6g}, err {err[idx]:.3e}), tol {tol:.1e} rtol {rtol:.1e}")
    print(msg)
    assert float(excess[idx]) <= 0.0, msg
    return worst
