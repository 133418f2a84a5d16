"""GPU parity of the query offset and the sliding window (fa_forward_ext /
fa_backward_ext) against the fp64 oracle."""
import math

import numpy as np
import pytest
import torch

import exact_attention_05_amd as fa
import oracle
import workloads
from parity import (MANY_TERMS_SUM, RTOL_BF16_TERMS, TOL_LSE, assert_close, bf16_grad_rtol, np64,
                    require_gpu, tol_for)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dev():
    return require_gpu()


def draw(seed, B, H, h_kv, n_q, n_k, d, dtype):
    q, _, _, do = workloads.random_qkv(seed, B, H, n_q, n_k, d, dtype, with_do=True)
    _, k, v = workloads.random_qkv(seed + 1, B, h_kv, n_q, n_k, d, dtype)
    return q, k, v, do


def run(dev, q, k, v, do, scale, causal, off, w):
    qd, kd, vd, dod = (t.to(dev) for t in (q, k, v, do))
    o, lse = fa.forward(qd, kd, vd, causal=causal, scale=scale, q_offset=off, window=w)
    dq, dk, dv = fa.backward(qd, kd, vd, o, dod, lse, causal=causal, scale=scale, q_offset=off, window=w)
    torch.cuda.synchronize()
    return o.cpu(), lse.cpu(), dq.cpu(), dk.cpu(), dv.cpu()


def check(tag, got, q, k, v, do, scale, causal, off, w, dtype):
    o, lse, dq, dk, dv = got
    q64, k64, v64, do64 = np64(q), np64(k), np64(v), np64(do)
    ro, rl = oracle.attention_fwd_band(q64, k64, v64, scale, causal, off, w)
    assert_close(f"O {tag}", o, ro, tol_for(dtype))
    fin = np.isfinite(rl)
    assert np.array_equal(np.isfinite(np64(lse)), fin), f"LSE {tag}: rows without keys differ"
    assert_close(f"LSE {tag}", np64(lse)[fin], rl[fin], TOL_LSE)
    rq, rk, rv = oracle.attention_bwd_band(q64, k64, v64, do64, scale, causal, off, w)
    if dtype == torch.bfloat16:
        # the sums of absolute terms, as for ordinary heads (see parity.py):
        # dQ: scale |dS| |K|, dK: scale |dS|^T |Q|, dV: |P|^T |dO|, with P and
        # dS of the banded oracle (K/V heads repeated, then folded).
        H, h_kv = q64.shape[1], k64.shape[1]
        ke, ve = oracle.expand_kv_heads(k64, H), oracle.expand_kv_heads(v64, H)
        vis = oracle.band_visible(q64.shape[2], k64.shape[2], causal, off, w)
        s = np.where(vis, scale * q64 @ np.swapaxes(ke, -1, -2), -np.inf)
        m = np.max(s, -1, keepdims=True)
        m = np.where(np.isfinite(m), m, 0.0)
        e = np.where(vis, np.exp(s - m), 0.0)
        z = e.sum(-1, keepdims=True)
        p = e / np.where(z > 0, z, 1.0)
        ds = p * (do64 @ np.swapaxes(ve, -1, -2) - np.sum(do64 * (p @ ve), -1, keepdims=True))
        t = lambda x: np.swapaxes(x, -1, -2)  # noqa: E731
        g = H // h_kv

        def fold(x):
            return x.reshape(x.shape[:-3] + (h_kv, g) + x.shape[-2:]).sum(axis=-3)

        mags = (scale * np.abs(ds) @ np.abs(ke), fold(scale * t(np.abs(ds)) @ np.abs(q64)),
                fold(t(p) @ np.abs(do64)))
        tol, rtol = tol_for(dtype), bf16_grad_rtol(dtype, q64.shape[2], k64.shape[2], g)
        # shapes outside that rule: only elements whose absolute terms sum to
        # MANY_TERMS_SUM or more (see parity.py)
        rtol, rfrom = (rtol, 0.0) if rtol > 0 else (RTOL_BF16_TERMS, MANY_TERMS_SUM)
    else:
        tol, rtol, rfrom, mags = tol_for(dtype), 0.0, 0.0, (None, None, None)
    for name, g, r, m in zip(("dQ", "dK", "dV"), (dq, dk, dv), (rq, rk, rv), mags):
        assert_close(f"{name} {tag}", g, r, tol, rtol, mag=m, rtol_from=rfrom)


CASES = [  # B, H, H_kv, n_q, n_k, causal, q_offset, window
    (1, 2, 2, 200, 200, True, 0, 0),
    (1, 2, 2, 200, 200, True, 0, 31),
    (1, 2, 1, 300, 300, False, 0, 64),
    (2, 2, 2, 257, 300, True, 43, 100),
    (1, 2, 2, 129, 600, True, 471, -1),
    (1, 4, 2, 333, 333, False, -20, 150),
    (1, 2, 2, 150, 150, True, -40, -1),
    (1, 2, 2, 64, 1000, False, 500, 90),
]


def test_causal_window_gqa_many_terms(dev):
    # 24 query heads per K/V head under a causal +-108 window: the first keys
    # are seen by up to 109 rows of each of 24 heads whose early probabilities
    # are large, so their dK is a sum whose absolute terms reach ~65 and
    # cancel to ~0.07.  Rounding dS to bf16, as the bf16 path does for
    # dK += dS^T Q, moves such an element by ~0.012 in an fp64 simulation
    # (0.023 on the GPU), beyond 2e-2 + rounding for the output; those
    # elements take the derived bound, every other element the plain one.
    B, H, h_kv, n_q, n_k, d, w = 1, 48, 2, 633, 1240, 64, 108
    q, k, v, do = draw(7006, B, H, h_kv, n_q, n_k, d, torch.bfloat16)
    scale = 1 / math.sqrt(d)
    got = run(dev, q, k, v, do, scale, True, 0, w)
    check("GQA 24 heads per K/V head, causal w=108", got, q, k, v, do, scale, True, 0, w, torch.bfloat16)


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("case", CASES, ids=lambda c: "B{}H{}kv{}_{}x{}_c{}_off{}_w{}".format(*c))
def test_band_parity(dev, case, d, dtype):
    B, H, h_kv, n_q, n_k, causal, off, w = case
    q, k, v, do = draw(4000 + n_q + n_k + d + (w % 97), B, H, h_kv, n_q, n_k, d, dtype)
    scale = 1 / math.sqrt(d)
    got = run(dev, q, k, v, do, scale, causal, off, w)
    check(f"{case} d{d} {dtype}", got, q, k, v, do, scale, causal, off, w, dtype)


def test_wide_window_and_zero_offset_equal_plain_attention_bitwise(dev):
    q, k, v, do = draw(4100, 1, 4, 4, 300, 300, 128, torch.bfloat16)
    qd, kd, vd, dod = (t.to(dev) for t in (q, k, v, do))
    for causal in (False, True):
        o1, l1 = fa.forward(qd, kd, vd, causal=causal)
        o2, l2 = fa.forward(qd, kd, vd, causal=causal, window=10000)
        g1 = fa.backward(qd, kd, vd, o1, dod, l1, causal=causal)
        g2 = fa.backward(qd, kd, vd, o2, dod, l2, causal=causal, window=10000)
        torch.cuda.synchronize()
        assert torch.equal(o1, o2) and torch.equal(l1, l2)
        for a, b in zip(g1, g2):
            assert torch.equal(a, b)


def test_sliding_window_workload_size(dev):
    # n = 4096, 32 heads, causal sliding window of 512 keys (+-512 before the
    # diagonal), bf16; four whole heads against the oracle.
    B, H, n, d, w = 1, 32, 4096, 128, 512
    q, k, v, _ = draw(4200, B, H, H, n, n, d, torch.bfloat16)
    o, lse = fa.forward(q.to(dev), k.to(dev), v.to(dev), causal=True, window=w)
    torch.cuda.synchronize()
    o, lse = o.cpu(), lse.cpu()
    for h in (0, 9, 22, 31):
        ro, rl = oracle.attention_fwd_band(np64(q[0, h]), np64(k[0, h]), np64(v[0, h]), 1 / math.sqrt(d), True, 0, w)
        assert_close(f"O head {h}", o[0, h], ro, 2e-2)
        assert_close(f"LSE head {h}", lse[0, h], rl, TOL_LSE)


# Few query tiles but many keys: the forward runs these on a split-key
# kernel (keys spread over the waves of a workgroup and merged in LDS):
# bf16 on the decoding kernel with one chunk, float32 on the key-split
# float32 kernel; the backward is unchanged.
STARVED = [  # B, H, H_kv, n_q, n_k, causal, q_offset, window, d
    (1, 1, 1, 2048, 2048, True, 0, -1, 128),
    (1, 2, 2, 1000, 3000, False, 500, 300, 64),
    (1, 4, 1, 700, 1500, True, 800, -1, 32),
    (2, 1, 1, 300, 4100, False, 0, -1, 128),
    (1, 2, 1, 33, 2500, True, 2467, 700, 64),
]


# Float32 shapes with at most 128 tiles of 128 rows but more than 128 blocks
# of 32: the forward takes the 32-row key-split kernel (the shapes above take
# the 16-row one).
F32_SPLIT32 = [  # B, H, H_kv, n_q, n_k, causal, q_offset, window, d
    (1, 2, 2, 4096, 4096, True, 0, -1, 64),
    (2, 4, 2, 1000, 1500, False, 300, 200, 128),
    (1, 8, 8, 600, 2000, False, 0, -1, 32),
]


@pytest.mark.parametrize("case", F32_SPLIT32, ids=lambda c: "B{}H{}kv{}_{}x{}_c{}_off{}_w{}_d{}".format(*c))
def test_fp32_32_row_key_split_parity(dev, case):
    B, H, h_kv, n_q, n_k, causal, off, w, d = case
    assert B * H * -(-n_q // 128) <= 128 < B * H * -(-n_q // 32)
    q, k, v, do = draw(4900 + n_q + n_k + d, B, H, h_kv, n_q, n_k, d, torch.float32)
    scale = 1 / math.sqrt(d)
    got = run(dev, q, k, v, do, scale, causal, off, w)
    check(f"{case}", got, q, k, v, do, scale, causal, off, w, torch.float32)


# Float32 shapes with at most 128 blocks of 32 rows (the 16-row key-split
# kernel): at d <= 64 from 1024 keys on its eight-wave form (the keys spread
# over eight waves, two per SIMD), below that and at d = 128 its four-wave
# form; both sides of the 1024-key boundary, masks, offsets, a window and
# shared K/V heads.
F32_SPLIT16 = [  # B, H, H_kv, n_q, n_k, causal, q_offset, window, d
    (1, 1, 1, 4096, 4096, False, 0, -1, 64),
    (1, 1, 1, 1500, 1024, True, 0, -1, 64),
    (1, 1, 1, 1500, 1023, True, 0, -1, 64),
    (1, 2, 1, 700, 3001, False, 0, -1, 32),
    (2, 1, 1, 257, 2000, True, 1743, -1, 32),
    (1, 2, 2, 900, 5000, False, 2000, 600, 64),
    (1, 4, 2, 500, 1100, True, -17, -1, 64),
    (1, 1, 1, 2000, 2000, False, 0, -1, 128),
]


@pytest.mark.parametrize("case", F32_SPLIT16, ids=lambda c: "B{}H{}kv{}_{}x{}_c{}_off{}_w{}_d{}".format(*c))
def test_fp32_16_row_key_split_parity(dev, case):
    B, H, h_kv, n_q, n_k, causal, off, w, d = case
    assert B * H * -(-n_q // 32) <= 128
    q, k, v, do = draw(5300 + n_q + n_k + d, B, H, h_kv, n_q, n_k, d, torch.float32)
    scale = 1 / math.sqrt(d)
    got = run(dev, q, k, v, do, scale, causal, off, w)
    check(f"{case}", got, q, k, v, do, scale, causal, off, w, torch.float32)


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32], ids=["bf16", "fp32"])
@pytest.mark.parametrize("case", STARVED, ids=lambda c: "B{}H{}kv{}_{}x{}_c{}_off{}_w{}_d{}".format(*c))
def test_starved_shapes_parity(dev, case, dtype):
    B, H, h_kv, n_q, n_k, causal, off, w, d = case
    q, k, v, do = draw(4700 + n_q + n_k + d, B, H, h_kv, n_q, n_k, d, dtype)
    scale = 1 / math.sqrt(d)
    got = run(dev, q, k, v, do, scale, causal, off, w)
    check(f"{case}", got, q, k, v, do, scale, causal, off, w, dtype)
