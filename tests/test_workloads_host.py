"""CPU tests of the seeded input recipe (workloads.py): the shapes, dtypes,
scales, masks, seeds and draw order that the tests, smoke() and bench.py
rely on, and that the bf16 inputs are round-to-nearest-even casts of the
float32 draws (checked against a bit-level rounding written here)."""
import math

import numpy as np
import torch

import workloads


def _rne_bf16_bits(x: torch.Tensor) -> np.ndarray:
    # round-to-nearest-even of float32 to its upper 16 bits (finite values)
    u = x.contiguous().view(torch.int32).numpy().astype(np.int64) & 0xFFFFFFFF
    return ((u + 0x7FFF + ((u >> 16) & 1)) >> 16) & 0xFFFF


def _bits(x: torch.Tensor) -> np.ndarray:
    return x.contiguous().view(torch.int16).numpy().astype(np.int64) & 0xFFFF


def test_c1_is_the_seed_9_stream():
    w = workloads.c1()
    g = torch.Generator().manual_seed(9)
    for t in (w.q, w.k, w.v):
        assert t.dtype == torch.float32 and t.shape == (2, 3, 128, 32)
        assert torch.equal(t, torch.randn(2, 3, 128, 32, generator=g))
    assert w.scale == 1 / math.sqrt(32) and not w.causal and w.do is None


def test_c2_continues_the_c1_stream_and_its_bf16_is_the_rne_cast():
    w, wb = workloads.c2(), workloads.c2(torch.bfloat16)
    g = torch.Generator().manual_seed(9)
    for _ in range(3):
        torch.randn(2, 3, 128, 32, generator=g)
    for t, tb in zip((w.q, w.k, w.v), (wb.q, wb.k, wb.v)):
        assert t.shape == tb.shape == (1, 1, 4096, 64)
        assert torch.equal(t.reshape(4096, 64), torch.randn(4096, 64, generator=g))
        assert tb.dtype == torch.bfloat16
        assert np.array_equal(_bits(tb), _rne_bf16_bits(t))
    assert w.scale == wb.scale == 1 / 8 and not w.causal


def test_c3_and_its_training_step_share_q_k_v():
    a, b, t = workloads.c3(False), workloads.c3(True), workloads.c3_train()
    for x, y, z in zip((a.q, a.k, a.v), (b.q, b.k, b.v), (t.q, t.k, t.v)):
        assert x.shape == (1, 32, 4096, 128) and x.dtype == torch.bfloat16
        assert torch.equal(x, y) and torch.equal(x, z)
    assert not a.causal and b.causal and not t.causal
    assert t.do.shape == (1, 32, 4096, 128) and t.do.dtype == torch.bfloat16
    # dO is the fourth draw of the seed-3 stream, cast by RNE
    g = torch.Generator().manual_seed(3)
    for _ in range(3):
        torch.randn(1, 32, 4096, 128, generator=g)
    assert np.array_equal(_bits(t.do), _rne_bf16_bits(torch.randn(1, 32, 4096, 128, generator=g)))


def test_c4_rows_are_256_distinct_rows_of_the_long_head_set():
    rows = workloads.c4_rows()
    assert len(rows) == 256 and len(set(rows)) == 256
    assert all(b == 0 and 0 <= h < 32 and 0 <= i < 16384 for b, h, i in rows)
    assert rows == workloads.c4_rows()


def test_c5_and_decode_shapes():
    w = workloads.c5()
    assert w.q.shape == w.k.shape == w.v.shape == w.do.shape == (2, 16, 4096, 128)
    assert w.causal and w.q.dtype == torch.bfloat16 and w.scale == 1 / math.sqrt(128)
    d = workloads.decode_gqa(B=2, H=8, H_kv=2, n_k=300, d=64)
    assert d.q.shape == (2, 8, 1, 64) and d.k.shape == d.v.shape == (2, 2, 300, 64)
    assert d.causal and d.scale == 1 / 8


def test_random_qkv_is_seeded_and_scales_only_the_scores():
    a = workloads.random_qkv(5, 1, 2, 30, 40, 32, torch.float32, with_do=True)
    b = workloads.random_qkv(5, 1, 2, 30, 40, 32, torch.float32, with_do=True)
    c = workloads.random_qkv(5, 1, 2, 30, 40, 32, torch.float32, with_do=True, std=4.0)
    assert all(torch.equal(x, y) for x, y in zip(a, b))
    assert torch.equal(c[0], 4 * a[0]) and torch.equal(c[1], 4 * a[1])
    assert torch.equal(c[2], a[2]) and torch.equal(c[3], a[3])
    assert [t.shape for t in a] == [(1, 2, 30, 32), (1, 2, 40, 32), (1, 2, 40, 32), (1, 2, 30, 32)]
