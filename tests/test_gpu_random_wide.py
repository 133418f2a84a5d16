"""Seeded random ragged shapes large enough for the wide routes against the
fp64 oracle: more than 512 query rows and enough heads that the forward and
dQ run 256-row workgroups (the d = 128 ping-pong kernels, the forward's
persistent tile loop once there are more tiles than compute units) and dK/dV
runs 128-key workgroups, mixed with causal masks, query offsets, windows and
shared K/V heads.  The oracle checks the gradients and outputs of a few
sampled K/V heads (with all query heads of their groups) and one sampled
batch entry; the smaller random shapes of test_gpu_random_shapes.py take the
narrow routes."""
import math
import random

import pytest
import torch

from parity import require_gpu
from test_gpu_band import check, draw, run

pytestmark = pytest.mark.gpu


def _cases(seed=11, count=16):
    # Every case takes the wide routes: 256-row forward and dQ workgroups
    # need more than 512 query rows and more than 128 of them without the
    # mask (at least 512 with it, so that the costliest-first order has
    # enough tiles); no window (windows always take the narrow routes).
    r = random.Random(seed)
    out = []
    for _ in range(count):
        d = r.choice([128, 128, 64, 32])
        causal = r.random() < 0.5
        if causal:
            B, H = 2, 48
            n_q = r.randint(1300, 1700)
        else:
            B, H = 2, 32
            n_q = r.randint(513, 1700)
        h_kv = H if r.random() < 0.7 else H // r.choice([2, 8, 16])
        n_k = n_q if r.random() < 0.5 else r.randint(64, 1700)
        off = 0 if r.random() < 0.7 else r.randint(-n_q // 2, n_k)
        dtype = "bf16" if r.random() < 0.8 else "fp32"
        pick = r.random()
        out.append((B, H, h_kv, n_q, n_k, causal, off, -1, d, dtype, pick))
    return out


@pytest.fixture(scope="module")
def dev():
    return require_gpu()


@pytest.mark.parametrize("case", _cases(),
                         ids=lambda c: "B{}H{}kv{}_{}x{}_c{:d}_off{}_w{}_d{}_{}".format(*c[:10]))
def test_random_wide_shape_parity(dev, case):
    B, H, h_kv, n_q, n_k, causal, off, w, d, dt, pick = case
    dtype = torch.bfloat16 if dt == "bf16" else torch.float32
    q, k, v, do = draw(12000 + n_q * 7 + n_k + d, B, H, h_kv, n_q, n_k, d, dtype)
    scale = 1 / math.sqrt(d)
    o, lse, dq, dk, dv = run(dev, q, k, v, do, scale, causal, off, w)
    # first, last and one middle K/V head, with all query heads of their groups
    g = H // h_kv
    kvs = sorted({0, h_kv - 1, int(pick * h_kv)})
    while len(kvs) * g > 8 and len(kvs) > 1:
        kvs = kvs[:-1]
    qs = [j * g + i for j in kvs for i in range(g)]
    b = int(pick * B)

    def sl(t, idx):
        return t[b:b + 1, idx]

    got = (sl(o, qs), sl(lse, qs), sl(dq, qs), sl(dk, kvs), sl(dv, kvs))
    check(f"{case[:10]} batch {b} K/V heads {kvs}", got, sl(q, qs), sl(k, kvs), sl(v, kvs), sl(do, qs),
          scale, causal, off, w, dtype)
