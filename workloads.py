"""Seeded synthetic inputs for the attention workloads.

This module only draws random tensors and casts them; it holds none of the
attention arithmetic.  It is the one piece shared by the tests, the bench and
the smoke check: the HIP path and the fp64 oracle both consume exactly the
tensors returned here (the oracle upcasts them to float64, which is exact).

Recipe (all draws are float32 ``torch.randn`` on the CPU generator, in the
order q, k, v[, dO]; bf16 tensors are the round-to-nearest-even cast of those
float32 draws):

* ``c1``: non-causal forward, fp32, (B, H, n, d) = (2, 3, 128, 32), seed 9,
  scale 1/sqrt(32).  Same seed, shapes and draw order as the script of
  "Efficient Attention" (section "Mengapa Memori Attention Tumbuh
  Kuadratik"), so these are that script's tensors.
* ``c2``: single head, n = 4096, d = 64, non-causal, scale 1/8, fp32 and its
  bf16 cast.  The draws continue the same seed-9 stream after ``c1``, as the
  script's third part does.
* ``c3``: (1, 32, 4096, 128) bf16, seed 3, scale 1/sqrt(128), both causal and
  non-causal.
* ``c3_train``: ``c3`` plus dO drawn fourth from the seed-3 stream: one
  forward + backward step (the bench workload).
* ``c4``: (1, 32, 16384, 128) bf16, seed 4, causal, scale 1/sqrt(128); the
  256 checked rows are the first 256 entries of ``torch.randperm(32 * 16384)``
  under seed 4004, row r -> (h, i) = (r // 16384, r % 16384).
* ``c5``: (2, 16, 4096, 128) bf16, seed 5, causal; draws q, k, v, dO.
* ``decode_gqa``: one decoding step of a grouped-K/V attention layer at long
  context, the shape "Attention Mechanism" uses for its KV-cache arithmetic
  (section 12: a 70B-class model at 32K context; 64 query heads over 8 K/V
  heads, head width 128): 4 sequences, one new query row each, against
  32768 cached keys; bf16, seed 8, draws q (4, 64, 1, 128) then k and v
  (4, 8, 32768, 128); causal with the query on the last key, scale
  1/sqrt(128).

All values are i.i.d. N(0, 1), so with scale 1/sqrt(d) the scores are close
to N(0, 1): dense heads, no padding, no variable lengths.
"""
from __future__ import annotations

import math
from dataclasses import dataclass

import torch

__all__ = ["Workload", "c1", "c2", "c3", "c3_train", "c4", "c4_rows", "c5", "decode_gqa", "random_qkv"]


@dataclass
class Workload:
    name: str
    q: torch.Tensor
    k: torch.Tensor
    v: torch.Tensor
    scale: float
    causal: bool
    do: torch.Tensor | None = None


def _draw(gen: torch.Generator, shape, n: int):
    return [torch.randn(*shape, generator=gen, dtype=torch.float32) for _ in range(n)]


def c1() -> Workload:
    gen = torch.Generator().manual_seed(9)
    q, k, v = _draw(gen, (2, 3, 128, 32), 3)
    return Workload("c1 fwd fp32 B2 H3 n128 d32", q, k, v, 1.0 / math.sqrt(32), False)


def c2(dtype: torch.dtype = torch.float32) -> Workload:
    gen = torch.Generator().manual_seed(9)
    _draw(gen, (2, 3, 128, 32), 3)  # the c1 draws come first in the same stream
    q, k, v = (t.reshape(1, 1, 4096, 64).to(dtype) for t in _draw(gen, (4096, 64), 3))
    tag = "fp32" if dtype == torch.float32 else "bf16"
    return Workload(f"c2 fwd {tag} B1 H1 n4096 d64", q, k, v, 1.0 / 8.0, False)


def c3(causal: bool = False) -> Workload:
    gen = torch.Generator().manual_seed(3)
    q, k, v = (t.to(torch.bfloat16) for t in _draw(gen, (1, 32, 4096, 128), 3))
    return Workload(f"c3 fwd bf16 B1 H32 n4096 d128 {'causal' if causal else 'noncausal'}",
                    q, k, v, 1.0 / math.sqrt(128), causal)


def c3_train(causal: bool = False) -> Workload:
    """``c3`` plus an output gradient dO, drawn fourth from the same stream
    (q, k, v are identical to ``c3``'s): the input of one forward + backward
    step at B=1, H=32, n=4096, d=128."""
    gen = torch.Generator().manual_seed(3)
    q, k, v, do = (t.to(torch.bfloat16) for t in _draw(gen, (1, 32, 4096, 128), 4))
    return Workload(f"c3 fwd+bwd bf16 B1 H32 n4096 d128 {'causal' if causal else 'noncausal'}",
                    q, k, v, 1.0 / math.sqrt(128), causal, do)


def c4() -> Workload:
    gen = torch.Generator().manual_seed(4)
    q, k, v = (t.to(torch.bfloat16) for t in _draw(gen, (1, 32, 16384, 128), 3))
    return Workload("c4 fwd bf16 B1 H32 n16384 d128 causal", q, k, v, 1.0 / math.sqrt(128), True)


def c4_rows(count: int = 256):
    """The checked (b, h, i) rows of ``c4``."""
    gen = torch.Generator().manual_seed(4004)
    r = torch.randperm(32 * 16384, generator=gen)[:count].tolist()
    return [(0, x // 16384, x % 16384) for x in r]


def c5() -> Workload:
    gen = torch.Generator().manual_seed(5)
    q, k, v, do = (t.to(torch.bfloat16) for t in _draw(gen, (2, 16, 4096, 128), 4))
    return Workload("c5 bwd bf16 B2 H16 n4096 d128 causal", q, k, v, 1.0 / math.sqrt(128), True, do)


def decode_gqa(B: int = 4, H: int = 64, H_kv: int = 8, n_k: int = 32768, d: int = 128) -> Workload:
    gen = torch.Generator().manual_seed(8)
    q = torch.randn(B, H, 1, d, generator=gen).to(torch.bfloat16)
    k = torch.randn(B, H_kv, n_k, d, generator=gen).to(torch.bfloat16)
    v = torch.randn(B, H_kv, n_k, d, generator=gen).to(torch.bfloat16)
    return Workload(f"decode bf16 B{B} H{H} Hkv{H_kv} n_q1 n_k{n_k} d{d}", q, k, v, 1.0 / math.sqrt(d), True)


def random_qkv(seed: int, B: int, H: int, n_q: int, n_k: int, d: int,
               dtype: torch.dtype = torch.bfloat16, with_do: bool = False, std: float = 1.0):
    """Generic seeded draws for test shapes, in the order q (B,H,n_q,d), k,
    v (B,H,n_k,d) and optionally dO (B,H,n_q,d): q and k N(0, std^2) (std
    sets the score magnitude), v and dO N(0, 1)."""
    gen = torch.Generator().manual_seed(seed)
    q = torch.randn(B, H, n_q, d, generator=gen) * std
    k = torch.randn(B, H, n_k, d, generator=gen) * std
    v = torch.randn(B, H, n_k, d, generator=gen)
    out = [q.to(dtype), k.to(dtype), v.to(dtype)]
    if with_do:
        out.append(torch.randn(B, H, n_q, d, generator=gen).to(dtype))
    return out
