"""GPU parity of split-KV decoding (fa_decode) and of the merge of results
over disjoint key sets (fa_lse_merge) against the fp64 oracle."""
import math
import random

import numpy as np
import pytest
import torch

import exact_attention_05_amd as fa
import oracle
import workloads
from parity import TOL_LSE, assert_close, np64, require_gpu, tol_for

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dev():
    return require_gpu()


def draw(seed, B, H, h_kv, n_q, n_k, d, dtype=torch.bfloat16):
    q, _, _ = workloads.random_qkv(seed, B, H, n_q, 1, d, dtype)
    _, k, v = workloads.random_qkv(seed + 1, B, h_kv, 1, n_k, d, dtype)
    return q, k, v


def check_band(tag, o, lse, q, k, v, scale, causal, off, w, tol):
    ro, rl = oracle.attention_fwd_band(np64(q), np64(k), np64(v), scale, causal, off, w)
    assert_close(f"O {tag}", o, ro, tol)
    fin = np.isfinite(rl)
    assert np.array_equal(np.isfinite(np64(lse)), fin), f"LSE {tag}: rows without keys differ"
    assert_close(f"LSE {tag}", np64(lse)[fin], rl[fin], TOL_LSE)


DECODE = [  # B, H, H_kv, n_q, n_k, d, causal, q_offset (None: n_k - n_q), window, n_splits
    (2, 8, 2, 1, 1000, 128, True, None, None, None),
    (1, 8, 2, 1, 1000, 64, True, None, None, 1),
    (1, 8, 2, 3, 777, 128, True, None, None, 3),
    (2, 16, 1, 4, 600, 64, True, None, None, 2),      # 64 packed rows: two row blocks
    (1, 4, 4, 9, 300, 128, False, 0, None, 2),
    (1, 8, 2, 1, 5000, 128, True, None, 100, None),   # window: most chunks see nothing
    (1, 8, 8, 5, 129, 32, True, None, None, 1),
    (1, 6, 2, 11, 1, 64, True, None, None, 1),        # rows before the only key see nothing
    (1, 4, 2, 20, 500, 64, True, None, 50, 2),        # a row block that wraps across heads
    (1, 2, 1, 40, 3000, 128, True, 2960, None, 7),
]


def check_decode_case(dev, case):
    B, H, h_kv, n_q, n_k, d, causal, off, w, splits = case
    q, k, v = draw(5000 + n_k + d + n_q, B, H, h_kv, n_q, n_k, d)
    scale = 1 / math.sqrt(d)
    o, lse = fa.decode(q.to(dev), k.to(dev), v.to(dev), causal=causal, scale=scale, q_offset=off,
                       window=w, n_splits=splits)
    torch.cuda.synchronize()
    off_ = n_k - n_q if off is None else off
    check_band(str(case), o.cpu(), lse.cpu(), q, k, v, scale, causal, off_, -1 if w is None else w, 2e-2)


@pytest.mark.parametrize("case", DECODE, ids=lambda c: "B{}H{}kv{}_q{}_k{}_d{}_c{}_off{}_w{}_s{}".format(*c))
def test_decode_parity(dev, case):
    check_decode_case(dev, case)


def _random_decode_cases(seed=23, count=14):
    # Seeded shapes around the fixed cases above: several batch entries and
    # group sizes (up to 64 query heads, so up to two 32-row blocks per K/V
    # head and step), 1-40 new rows, caches from one key to several thousand
    # (ragged against the 128-key chunk blocks), offsets that put rows before
    # the first key, windows, and chunk counts up to more than the cache holds.
    r = random.Random(seed)
    out = []
    for i in range(count):
        h_kv = r.choice([1, 2, 3, 4, 8])
        group = r.choice([g for g in (1, 2, 4, 5, 8, 16) if h_kv * g <= 64])
        n_q = r.randint(1, 16) if r.random() < 0.8 else r.randint(17, 40)
        n_k = r.randint(1, 6000)
        causal = i % 3 != 2
        u = r.random()
        off = None if u < 0.45 else -r.randint(1, n_q) if u < 0.6 else r.randint(0, n_k)
        w = None if r.random() < 0.7 else r.randint(0, 400)
        splits = None if r.random() < 0.5 else r.randint(1, 12)
        out.append((r.randint(1, 3), h_kv * group, h_kv, n_q, n_k, r.choice([32, 64, 128]), causal, off, w,
                    splits))
    return out


@pytest.mark.parametrize("case", _random_decode_cases(),
                         ids=lambda c: "B{}H{}kv{}_q{}_k{}_d{}_c{}_off{}_w{}_s{}".format(*c))
def test_decode_random_cases(dev, case):
    check_decode_case(dev, case)


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("n_q,splits", [(1, None), (1, 1), (3, 5)])
def test_decode_running_max_stress(dev, d, n_q, splits):
    # The decoding kernel keeps a reference maximum per row and rescales its
    # sums only when a block's maximum passes it by a margin; the query rows
    # of a K/V group share a wave, so one row's jump rescales all of them.
    # K/V head 0: key j scores c * f(j) for a query row of constant c, with f
    # rising slowly (well under the margin per 32 keys), a jump past the
    # margin at key 1800 and a spike near the end; its four query heads rise
    # at different rates or fall (c = -1).  K/V head 1: scores near -30.
    B, H, h_kv, n_k = 1, 8, 2, 3000
    scale = 1 / math.sqrt(d)
    q, k, v = draw(5900 + d + n_q, B, H, h_kv, n_q, n_k, d, torch.float32)
    j = torch.arange(n_k, dtype=torch.float32)
    f = 0.012 * j + 12.0 * (j >= 1800).float() + 15.0 * (j == n_k - 5).float()
    k[0, 0] = (f / (d * scale))[:, None].expand(n_k, d)
    for h, c in enumerate((1.0, 0.5, -1.0, 1.5)):
        q[0, h] = c
    q[0, 4:] = -q[0, 4:].abs() * 2.0
    k[0, 1] = k[0, 1].abs() * 2.0
    q, k, v = (t.to(torch.bfloat16) for t in (q, k, v))
    o, lse = fa.decode(q.to(dev), k.to(dev), v.to(dev), causal=True, scale=scale, n_splits=splits)
    torch.cuda.synchronize()
    check_band(f"d={d} n_q={n_q} splits={splits}", o.cpu(), lse.cpu(), q, k, v, scale, True, n_k - n_q, -1,
               2e-2)


def test_decode_workload_size_sampled_heads(dev):
    # One decoding step at 32K context, 64 query heads over 8 K/V heads.
    wl = workloads.decode_gqa()
    n_k = wl.k.shape[2]
    o, lse = fa.decode(wl.q.to(dev), wl.k.to(dev), wl.v.to(dev), causal=True, scale=wl.scale)
    torch.cuda.synchronize()
    o, lse = o.cpu(), lse.cpu()
    for b, h in ((0, 0), (1, 37), (3, 63), (2, 8)):
        kv = h // 8
        ro, rl = oracle.attention_fwd_band(np64(wl.q[b, h]), np64(wl.k[b, kv]), np64(wl.v[b, kv]),
                                           wl.scale, True, n_k - 1)
        assert_close(f"decode O ({b},{h})", o[b, h], ro, 2e-2)
        assert_close(f"decode LSE ({b},{h})", lse[b, h], rl, TOL_LSE)


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
@pytest.mark.parametrize("causal,off,w", [(True, 500, -1), (False, 0, -1), (True, 480, 120)])
def test_merge_of_key_chunks_equals_attention_over_all_keys(dev, dtype, causal, off, w):
    # The one-GPU half of sequence-parallel attention: each key chunk [a, b)
    # is attended separately (query offset shifted by -a), the parts merged.
    B, H, h_kv, n_q, n_k, d = 1, 4, 2, 200, 700, 64
    q, k, v = draw(5100, B, H, h_kv, n_q, n_k, d, dtype)
    scale = 1 / math.sqrt(d)
    qd, kd, vd = q.to(dev), k.to(dev), v.to(dev)
    cuts = [(0, 250), (250, 251), (251, 640), (640, 700)]
    parts_o = torch.empty((len(cuts), B, H, n_q, d), dtype=dtype, device=dev)
    parts_l = torch.empty((len(cuts), B, H, n_q), dtype=torch.float32, device=dev)
    for p, (a, b) in enumerate(cuts):
        fa.forward(qd, kd[:, :, a:b].contiguous(), vd[:, :, a:b].contiguous(), causal=causal, scale=scale,
                   q_offset=off - a, window=None if w < 0 else w, out=parts_o[p], lse=parts_l[p])
    o, lse = fa.lse_merge(parts_o, parts_l)
    torch.cuda.synchronize()
    tag = f"{dtype} causal={causal} off={off} w={w}"
    # against the plain definition over all keys
    check_band(tag, o.cpu(), lse.cpu(), q, k, v, scale, causal, off, w, tol_for(dtype))
    # and, tightly, against the oracle's merge of the very same GPU parts
    mo, ml = oracle.lse_merge(np64(parts_o.cpu()), np64(parts_l.cpu()))
    assert_close(f"merge O {tag}", o.cpu(), mo, 1e-2 if dtype == torch.bfloat16 else 2e-6)
    fin = np.isfinite(ml)
    assert np.array_equal(np.isfinite(np64(lse.cpu())), fin)
    assert_close(f"merge LSE {tag}", np64(lse.cpu())[fin], ml[fin], 2e-6)


@pytest.mark.parametrize("d", [32, 64, 128])
@pytest.mark.parametrize("pdt,odt", [(torch.float32, torch.float32), (torch.float32, torch.bfloat16),
                                     (torch.bfloat16, torch.bfloat16), (torch.bfloat16, torch.float32)])
def test_merge_against_oracle(dev, d, pdt, odt):
    gen = torch.Generator().manual_seed(5200 + d)
    P, rows = 5, 333
    o_parts = torch.randn(P, rows, d, generator=gen).to(pdt)
    lse_parts = (torch.randn(P, rows, generator=gen) * 4).float()
    lse_parts[1, :50] = -math.inf          # parts without keys for some rows
    lse_parts[:, 7] = -math.inf            # a row with no keys anywhere
    o, lse = fa.lse_merge(o_parts.to(dev), lse_parts.to(dev), out_dtype=odt)
    torch.cuda.synchronize()
    mo, ml = oracle.lse_merge(np64(o_parts), np64(lse_parts))
    assert_close(f"merge O d{d} {pdt}->{odt}", o.cpu(), mo, 1e-2 if odt == torch.bfloat16 else 2e-6)
    got_l = np64(lse.cpu())
    fin = np.isfinite(ml)
    assert np.array_equal(np.isfinite(got_l), fin) and not fin[7]
    assert np.all(np64(o.cpu())[7] == 0)
    assert_close(f"merge LSE d{d}", got_l[fin], ml[fin], 2e-6)
