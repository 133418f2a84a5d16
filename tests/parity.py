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


# bf16 backward bound for shapes whose keys gather many query rows
# (group * n_q >= MANY_ROWS_PER_KEY * n_k, e.g. 600 queries on 5 keys): there
# a key's dK and dV are sums whose absolute terms add up to ~20 or more,
# beyond the O(1) gradients the 2e-2 bound is set for.  Each gradient is a sum
# of products whose bf16-rounded factor (P or dS) carries a relative error up
# to 2^-9, and the result is rounded to bf16 once more (2^-9 of its magnitude,
# which is at most the sum of the absolute terms).  Both together are bounded
# by 2^-8 * sum |terms|; those shapes are allowed twice that on top of 2e-2.
# The sums of absolute terms are
#   dQ: scale |dS| |K|,  dK: scale |dS|^T |Q|,  dV: |P|^T |dO|.
# Every other shape is held to the plain bounds.
RTOL_BF16_TERMS = 2.0 ** -7
MANY_ROWS_PER_KEY = 16
# Under a mask the same regime can hold for single elements of shapes the
# rule above does not cover: the first keys of a causal window are seen by
# up to w + 1 rows of each query head of their group, whose early
# probabilities (and dS) are large.  The band checks therefore give the same
# allowance to every element whose sum of absolute terms, computed from the
# oracle, reaches MANY_TERMS_SUM (the "~20 or more" of the rule above), and
# hold every other element to the plain bound.
MANY_TERMS_SUM = 20.0


def bf16_grad_rtol(dtype: torch.dtype, n_q: int, n_k: int, group: int = 1) -> float:
    """RTOL_BF16_TERMS for bf16 shapes with many query rows per key, else 0."""
    if dtype != torch.bfloat16:
        return 0.0
    return RTOL_BF16_TERMS if group * n_q >= MANY_ROWS_PER_KEY * n_k else 0.0


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


def half_ulp_bf16(x) -> np.ndarray:
    """Half a unit in the last place of bfloat16 at |x| (8 significant bits:
    2^(e - 8) for |x| in [2^e, 2^(e+1))), the largest rounding error of a
    round-to-nearest-even conversion to bfloat16; 0 at x = 0."""
    a = np.abs(np.asarray(x, dtype=np.float64))
    e = np.floor(np.log2(np.where(a > 0, a, 1.0)))
    return np.where(a > 0, np.exp2(e - 8.0), 0.0)


def assert_close(name: str, got, ref, tol: float, rtol: float = 0.0, mag=None, rounded_bf16=None,
                 rtol_from: float = 0.0) -> float:
    """Element-wise |got - ref| <= tol + rtol * mag (mag defaults to |ref|;
    the rtol term only where mag >= rtol_from),
    plus, for a bfloat16 result, the rounding of that result to bfloat16 (half
    an ulp at max(|got|, |ref|)): tol bounds the arithmetic, and the output
    format adds its own rounding on top, which alone passes 2e-2 once
    |x| >= 8.  ``rounded_bf16`` says whether ``got`` was a bfloat16 result
    (default: whether it is a bfloat16 tensor).  Prints the worst element."""
    if rounded_bf16 is None:
        rounded_bf16 = isinstance(got, torch.Tensor) and got.dtype == torch.bfloat16
    got = np64(got) if isinstance(got, torch.Tensor) else np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert got.shape == ref.shape, f"{name}: shape {got.shape} vs {ref.shape}"
    assert np.all(np.isfinite(got)), f"{name}: non-finite values"
    if got.size == 0:  # e.g. the finite LSE of a call in which no row sees a key
        print(f"{name}: no elements")
        return 0.0
    err = np.abs(got - ref)
    mag = np.abs(ref) if mag is None else np.asarray(mag, dtype=np.float64)
    bound = tol + np.where(mag >= rtol_from, rtol * mag, 0.0)
    if rounded_bf16:
        bound = bound + half_ulp_bf16(np.maximum(np.abs(got), np.abs(np.where(np.isfinite(ref), ref, 0.0))))
    excess = err - bound
    idx = np.unravel_index(int(np.argmax(excess)), err.shape)
    worst = float(np.max(err))
    msg = (f"{name}: max |err| {worst:.3e}; worst vs bound at {tuple(int(i) for i in idx)} "
           f"(got {got[idx]:.6g}, ref {ref[idx]:.6g}, err {err[idx]:.3e}, bound {float(bound[idx] if np.ndim(bound) else bound):.3e}), "
           f"tol {tol:.1e} rtol {rtol:.1e}{f' where mag >= {rtol_from:g}' if rtol_from else ''}"
           f"{' +half-ulp bf16' if rounded_bf16 else ''}")
    print(msg)
    assert float(excess[idx]) <= 0.0, msg
    return worst
