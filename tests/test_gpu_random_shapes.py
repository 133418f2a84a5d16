"""Seeded random shapes through the whole path (fa_forward_ext /
fa_backward_ext, the most general entry points) against the fp64 oracle:
batch, query and K/V heads, ragged row and key counts, head dimension, dtype,
causal mask, query offset and window drawn from a fixed seed.  The cases mix
unmasked and masked key blocks in every order and length, both workgroup
heights and shared K/V heads, beyond the hand-picked cases of the other
parity tests."""
import math
import random

import pytest
import torch

from test_gpu_band import check, draw, run
from parity import require_gpu

pytestmark = pytest.mark.gpu


def _size(r):
    lo, hi = r.choice([(1, 70), (60, 520), (500, 1100)])
    return r.randint(lo, hi)


def _cases(seed=2024, count=40):
    r = random.Random(seed)
    out = []
    for _ in range(count):
        h_kv = r.choice([1, 2])
        group = r.choice([1, 2, 3])
        n_q, n_k = _size(r), _size(r)
        B = r.choice([1, 2])
        while B * h_kv * group * n_q * n_k > 2_500_000 and (B > 1 or group > 1 or h_kv > 1):
            B, group, h_kv = (1, group, h_kv) if B > 1 else ((B, 1, h_kv) if group > 1 else (B, group, 1))
        causal = r.random() < 0.5
        off = 0 if r.random() < 0.5 else r.randint(-n_q, n_k)
        w = -1 if r.random() < 0.4 else r.randint(0, 400)
        d = r.choice([32, 64, 128])
        dtype = r.choice(["bf16", "fp32"])
        out.append((B, h_kv * group, h_kv, n_q, n_k, causal, off, w, d, dtype))
    return out


@pytest.fixture(scope="module")
def dev():
    return require_gpu()


@pytest.mark.parametrize("case", _cases(), ids=lambda c: "B{}H{}kv{}_{}x{}_c{:d}_off{}_w{}_d{}_{}".format(*c))
def test_random_shape_parity(dev, case):
    B, H, h_kv, n_q, n_k, causal, off, w, d, dt = case
    dtype = torch.bfloat16 if dt == "bf16" else torch.float32
    q, k, v, do = draw(9000 + n_q * 31 + n_k + d, B, H, h_kv, n_q, n_k, d, dtype)
    scale = 1 / math.sqrt(d)
    got = run(dev, q, k, v, do, scale, causal, off, w)
    check(f"{case}", got, q, k, v, do, scale, causal, off, w, dtype)
