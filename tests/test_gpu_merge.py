"""GPU parity of the forward pass merged into a prior result
(fa_forward_merge): attention over keys that arrive in chunks, the one-GPU
step of ring attention, against the fp64 oracle over all keys and against
the oracle's own merge rule."""
import math

import numpy as np
import pytest
import torch

import exact_attention_05_amd as fa
import oracle
import workloads
from parity import TOL_LSE, assert_close, half_ulp_bf16, np64, require_gpu, tol_for

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dev():
    return require_gpu()


def draw(seed, B, H, h_kv, n_q, n_k, d, dtype):
    q, _, _, do = workloads.random_qkv(seed, B, H, n_q, n_k, d, dtype, with_do=True)
    _, k, v = workloads.random_qkv(seed + 1, B, h_kv, n_q, n_k, d, dtype)
    return q, k, v, do


def check_band(tag, o, lse, q, k, v, scale, causal, off, w, tol, rounded_bf16=None):
    ro, rl = oracle.attention_fwd_band(np64(q), np64(k), np64(v), scale, causal, off, w)
    assert_close(f"O {tag}", o, ro, tol, rounded_bf16=rounded_bf16)
    got_l = np64(lse)
    fin = np.isfinite(rl)
    assert np.array_equal(np.isfinite(got_l), fin), f"LSE {tag}: rows without keys differ"
    assert_close(f"LSE {tag}", got_l[fin], rl[fin], TOL_LSE)


CUTS = [(0, 250), (250, 251), (251, 640), (640, 700)]


@pytest.mark.parametrize("dtype,acc", [(torch.bfloat16, torch.bfloat16), (torch.bfloat16, torch.float32),
                                       (torch.float32, torch.float32)])
@pytest.mark.parametrize("causal,off,w", [(True, 500, -1), (False, 0, -1), (True, 480, 120)])
def test_chained_key_chunks_equal_attention_over_all_keys(dev, dtype, acc, causal, off, w):
    # Ring attention's forward on one GPU: the query rows visit the key chunks
    # [a, b) one after the other (query offset shifted by -a), each call
    # merging into the running result in place; the first starts from
    # lse = -inf and a running output full of NaN, which must never be read.
    B, H, h_kv, n_q, n_k, d = 1, 4, 2, 200, 700, 64
    q, k, v, _ = draw(5100, B, H, h_kv, n_q, n_k, d, dtype)
    scale = 1 / math.sqrt(d)
    qd, kd, vd = q.to(dev), k.to(dev), v.to(dev)
    o = torch.full(q.shape, float("nan"), dtype=acc, device=dev)
    lse = torch.full(q.shape[:3], -math.inf, dtype=torch.float32, device=dev)
    for a, b in CUTS:
        fa.forward_merge(qd, kd[:, :, a:b].contiguous(), vd[:, :, a:b].contiguous(), o, lse, causal=causal,
                         scale=scale, q_offset=off - a, window=None if w < 0 else w, out=o, lse=lse)
    torch.cuda.synchronize()
    tag = f"{dtype} acc {acc} causal={causal} off={off} w={w}"
    check_band(tag, o.cpu(), lse.cpu(), q, k, v, scale, causal, off, w, tol_for(dtype))
    # the same as the separate forward + fa_lse_merge route, within rounding
    parts_o = torch.empty((len(CUTS), B, H, n_q, d), dtype=torch.float32, device=dev)
    parts_l = torch.empty((len(CUTS), B, H, n_q), dtype=torch.float32, device=dev)
    for p, (a, b) in enumerate(CUTS):
        po, pl = fa.forward(qd, kd[:, :, a:b].contiguous(), vd[:, :, a:b].contiguous(), causal=causal,
                            scale=scale, q_offset=off - a, window=None if w < 0 else w)
        parts_o[p] = po.float()
        parts_l[p] = pl
    mo, ml = fa.lse_merge(parts_o, parts_l)
    torch.cuda.synchronize()
    fin = torch.isfinite(ml)
    assert torch.equal(torch.isfinite(lse), fin)
    assert_close(f"LSE vs forward + lse_merge {tag}", np64(lse.cpu())[np64(fin.cpu()) > 0],
                 np64(ml.cpu())[np64(fin.cpu()) > 0], 2e-6)


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
@pytest.mark.parametrize("d", [32, 64, 128])
@pytest.mark.parametrize("causal", [False, True])
def test_merge_step_against_the_oracle_merge_rule(dev, dtype, d, causal):
    # One step against a random prior: the result must be oracle.lse_merge of
    # (prior, this chunk's exact attention).  Some rows have no prior
    # (lse = -inf), some see no key in this chunk (the window), and the
    # prior LSE values are spread wide (+-8) so both sides dominate somewhere.
    B, H, n_q, n_k, w, off = 2, 3, 333, 300, 90, 150
    q, k, v, _ = draw(5300 + d, B, H, H, n_q, n_k, d, dtype)
    scale = 1 / math.sqrt(d)
    gen = torch.Generator().manual_seed(5400 + d)
    o_p = torch.randn(B, H, n_q, d, generator=gen).to(dtype)
    l_p = torch.randn(B, H, n_q, generator=gen) * 8.0
    l_p[0, 1, :40] = -math.inf
    o_p[0, 1, :40] = float("nan")   # never read: that prior holds no keys
    l_p[1, 2, 250:260] = -math.inf  # rows 240.. see no key of this chunk either
    o, lse = fa.forward_merge(q.to(dev), k.to(dev), v.to(dev), o_p.to(dev), l_p.to(dev), causal=causal,
                              scale=scale, q_offset=off, window=w)
    torch.cuda.synchronize()
    co, cl = oracle.attention_fwd_band(np64(q), np64(k), np64(v), scale, causal, off, w)
    prior = np.where(np.isfinite(np64(l_p))[..., None], np64(o_p), 0.0)  # a part without keys has no O
    ro, rl = oracle.lse_merge(np.stack([prior, co]), np.stack([np64(l_p), cl]))
    tag = f"d{d} {dtype} causal={causal}"
    assert_close(f"O {tag}", o.cpu(), ro, tol_for(dtype))
    got_l = np64(lse.cpu())
    fin = np.isfinite(rl)
    assert np.array_equal(np.isfinite(got_l), fin)
    assert_close(f"LSE {tag}", got_l[fin], rl[fin], TOL_LSE)
    # rows with neither a prior nor a visible key: O = 0, LSE = -inf
    empty = ~fin
    assert empty.sum() == 10 and np.all(np64(o.cpu())[empty] == 0.0)


def test_in_place_equals_out_of_place_bitwise(dev):
    B, H, n_q, n_k, d = 1, 4, 300, 500, 128
    q, k, v, _ = draw(5500, B, H, H, n_q, n_k, d, torch.bfloat16)
    gen = torch.Generator().manual_seed(5501)
    o_p = torch.randn(B, H, n_q, d, generator=gen).to(torch.bfloat16).to(dev)
    l_p = (torch.randn(B, H, n_q, generator=gen) * 3.0).to(dev)
    qd, kd, vd = q.to(dev), k.to(dev), v.to(dev)
    for causal in (False, True):
        o1, l1 = fa.forward_merge(qd, kd, vd, o_p, l_p, causal=causal, q_offset=200)
        o2, l2 = o_p.clone(), l_p.clone()
        fa.forward_merge(qd, kd, vd, o2, l2, causal=causal, q_offset=200, out=o2, lse=l2)
        torch.cuda.synchronize()
        assert torch.equal(o1, o2) and torch.equal(l1, l2)


def test_no_prior_equals_plain_forward(dev):
    # With lse_prior = -inf everywhere the merged result is this call's own:
    # fa_forward's O and LSE, up to the rounding of the merge weights (the
    # output is scaled by 2^(m - LSE_n) / sum instead of 1 / l).  Both O are
    # bf16 roundings of float32 values a few float32 ulps apart: they agree
    # or are neighbours on the bf16 grid (one ulp).
    B, H, n_q, n_k, d = 2, 8, 700, 700, 128
    q, k, v, _ = draw(5600, B, H, H, n_q, n_k, d, torch.bfloat16)
    qd, kd, vd = q.to(dev), k.to(dev), v.to(dev)
    for causal in (False, True):
        o0, l0 = fa.forward(qd, kd, vd, causal=causal)
        o_p = torch.zeros_like(qd)
        l_p = torch.full(q.shape[:3], -math.inf, device=dev)
        o1, l1 = fa.forward_merge(qd, kd, vd, o_p, l_p, causal=causal)
        torch.cuda.synchronize()
        a, b = np64(o1.cpu()), np64(o0.cpu())
        one_ulp = 2.0 * half_ulp_bf16(np.maximum(np.abs(a), np.abs(b)))
        assert np.all(np.abs(a - b) <= one_ulp), f"O causal={causal}: more than one bf16 ulp apart"
        print(f"O causal={causal}: {np.mean(a == b):.4f} of the elements bitwise equal")
        assert_close(f"LSE causal={causal}", l1.cpu(), np64(l0.cpu()), 2e-6)


def test_ring_attention_backward_by_chunks(dev):
    # The backward over key chunks: with the final o and lse over all keys,
    # fa_backward_ext on one chunk gives that chunk's exact dK, dV and its
    # share of dQ (the probabilities exp(S - LSE) are the global ones); the
    # chunks' dQ sum to the full dQ.  Forward by chained fa_forward_merge.
    B, H, n, d = 1, 4, 640, 128
    q, k, v, do = draw(5700, B, H, H, n, n, d, torch.bfloat16)
    scale = 1 / math.sqrt(d)
    qd, kd, vd, dod = (t.to(dev) for t in (q, k, v, do))
    cuts = [(0, 160), (160, 320), (320, 480), (480, 640)]
    o = torch.zeros(q.shape, dtype=torch.float32, device=dev)
    lse = torch.full(q.shape[:3], -math.inf, device=dev)
    for a, b in cuts:
        fa.forward_merge(qd, kd[:, :, a:b].contiguous(), vd[:, :, a:b].contiguous(), o, lse, causal=True,
                         q_offset=-a, out=o, lse=lse)
    o16 = o.to(torch.bfloat16)
    dq = torch.zeros(q.shape, dtype=torch.float32, device=dev)
    dks, dvs = [], []
    for a, b in cuts:
        gq, gk, gv = fa.backward(qd, kd[:, :, a:b].contiguous(), vd[:, :, a:b].contiguous(), o16, dod, lse,
                                 causal=True, q_offset=-a)
        dq += gq.float()
        dks.append(gk)
        dvs.append(gv)
    torch.cuda.synchronize()
    rq, rk, rv = oracle.attention_bwd(np64(q), np64(k), np64(v), np64(do), scale, True)
    check_band("ring forward", o16.cpu(), lse.cpu(), q, k, v, scale, True, 0, -1, 2e-2)
    # dQ is a sum of four bf16-rounded shares: each carries half an ulp
    assert_close("ring dQ", dq.cpu(), rq, 2e-2 + 4 * 2.0 ** -9 * float(np.max(np.abs(rq))))
    assert_close("ring dK", torch.cat(dks, dim=2).cpu(), rk, 2e-2)
    assert_close("ring dV", torch.cat(dvs, dim=2).cpu(), rv, 2e-2)


@pytest.mark.parametrize("acc", [torch.bfloat16, torch.float32])
@pytest.mark.parametrize("causal", [False, True])
def test_chained_key_chunks_on_the_wide_kernels(dev, acc, causal):
    # Shapes large enough for 256-row workgroups (the d = 128 ping-pong
    # kernel with its merging epilogue, and for the non-causal pass its
    # persistent tile loop): three chunks, the last ragged, merged in place;
    # a few heads against the oracle over all keys.
    B, H, n_q, n_k, d = 2, 48, 1400, 1500, 128
    cuts = [(0, 640), (640, 1281), (1281, 1500)]
    off = n_k - n_q if causal else 0
    q, k, v, _ = draw(5300 + int(causal), B, H, H, n_q, n_k, d, torch.bfloat16)
    scale = 1 / math.sqrt(d)
    qd, kd, vd = q.to(dev), k.to(dev), v.to(dev)
    o = torch.full(q.shape, float("nan"), dtype=acc, device=dev)
    lse = torch.full(q.shape[:3], -math.inf, dtype=torch.float32, device=dev)
    for a, b in cuts:
        fa.forward_merge(qd, kd[:, :, a:b].contiguous(), vd[:, :, a:b].contiguous(), o, lse, causal=causal,
                         scale=scale, q_offset=off - a, out=o, lse=lse)
    torch.cuda.synchronize()
    oc, lc = o.cpu(), lse.cpu()
    for b, h in ((0, 0), (1, 47), (1, 20)):
        check_band(f"acc {acc} causal={causal} ({b}, {h})", oc[b:b + 1, h:h + 1], lc[b:b + 1, h:h + 1],
                   q[b:b + 1, h:h + 1], k[b:b + 1, h:h + 1], v[b:b + 1, h:h + 1], scale, causal, off, -1,
                   tol_for(torch.bfloat16), rounded_bf16=(acc == torch.bfloat16))
