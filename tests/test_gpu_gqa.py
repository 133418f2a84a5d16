"""GPU parity of grouped-query and multi-query attention (shared K/V heads)
against the fp64 oracle, through fa_forward_gqa / fa_backward_gqa."""
import math

import numpy as np
import pytest
import torch

import exact_attention_05_amd as fa
import oracle
import workloads
from parity import TOL_F32, TOL_LSE, assert_close, bf16_grad_rtol, np64, require_gpu, tol_for

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dev():
    return require_gpu()


def draw(seed, B, H, h_kv, n_q, n_k, d, dtype):
    q, _, _, do = workloads.random_qkv(seed, B, H, n_q, n_k, d, dtype, with_do=True)
    _, k, v = workloads.random_qkv(seed + 1, B, h_kv, n_q, n_k, d, dtype)
    return q, k, v, do


CASES = [(1, 8, 8, 65, 65), (2, 8, 4, 200, 333), (1, 8, 2, 300, 257), (1, 8, 1, 129, 129),
         (1, 4, 1, 17, 600)]


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("case", CASES, ids=lambda c: "B{}H{}kv{}_{}x{}".format(*c))
def test_gqa_forward_backward(dev, case, causal, dtype, d):
    B, H, h_kv, n_q, n_k = case
    q, k, v, do = draw(3000 + H * 31 + h_kv * 7 + n_q + d, B, H, h_kv, n_q, n_k, d, dtype)
    scale = 1 / math.sqrt(d)
    qd, kd, vd, dod = (t.to(dev) for t in (q, k, v, do))
    o, lse = fa.forward(qd, kd, vd, causal=causal, scale=scale)
    dq, dk, dv = fa.backward(qd, kd, vd, o, dod, lse, causal=causal, scale=scale)
    torch.cuda.synchronize()
    assert dk.shape == k.shape and dv.shape == v.shape
    q64, k64, v64, do64 = np64(q), np64(k), np64(v), np64(do)
    ro, rl = oracle.attention_fwd_gqa(q64, k64, v64, scale, causal)
    tag = f"{case} d{d} {dtype} causal={causal}"
    tol = tol_for(dtype)
    assert_close(f"O {tag}", o, ro, tol_for(dtype))
    assert_close(f"LSE {tag}", lse, rl, TOL_LSE)
    rq, rk, rv = oracle.attention_bwd_gqa(q64, k64, v64, do64, scale, causal)
    if dtype == torch.bfloat16:
        # bound from the sums of absolute terms, as for ordinary heads; a
        # shared K/V head gathers the terms of all heads in its group.
        ke, ve = oracle.expand_kv_heads(k64, H), oracle.expand_kv_heads(v64, H)
        _, _, _, mid = oracle.attention_bwd(q64, ke, ve, do64, scale, causal, intermediates=True)
        t = lambda x: np.swapaxes(x, -1, -2)  # noqa: E731
        ads, ap = np.abs(mid["ds"]), np.abs(mid["p"])
        g = H // h_kv

        def fold(x):
            return x.reshape(x.shape[:-3] + (h_kv, g) + x.shape[-2:]).sum(axis=-3)

        mags = (scale * ads @ np.abs(ke), fold(scale * t(ads) @ np.abs(q64)), fold(t(ap) @ np.abs(do64)))
        rtol = bf16_grad_rtol(dtype, n_q, n_k, g)
    else:
        mags, rtol = (None, None, None), 0.0
    for name, got, ref, m in zip(("dQ", "dK", "dV"), (dq, dk, dv), (rq, rk, rv), mags):
        assert_close(f"{name} {tag}", got, ref, tol, rtol, mag=m)


def test_gqa_forward_equals_mha_on_repeated_heads_bitwise(dev):
    # The kernels read the shared head where multi-head attention reads its
    # copy: the same arithmetic in the same order (on the forward kernel; a
    # shape with few query tiles and >= 1024 keys runs on the split-key
    # kernel, which packs a group's rows together and agrees within rounding).
    q, k, v, _ = draw(3100, 2, 8, 2, 333, 333, 128, torch.bfloat16)
    qd, kd, vd = (t.to(dev) for t in (q, k, v))
    for causal in (False, True):
        o1, l1 = fa.forward(qd, kd, vd, causal=causal)
        o2, l2 = fa.forward(qd, kd.repeat_interleave(4, dim=1).contiguous(),
                            vd.repeat_interleave(4, dim=1).contiguous(), causal=causal)
        torch.cuda.synchronize()
        assert torch.equal(o1, o2) and torch.equal(l1, l2)


def test_gqa_backward_equals_group_sum_of_mha(dev):
    q, k, v, do = draw(3200, 1, 8, 2, 256, 256, 64, torch.float32)
    qd, kd, vd, dod = (t.to(dev) for t in (q, k, v, do))
    ke, ve = (x.repeat_interleave(4, dim=1).contiguous() for x in (kd, vd))
    for causal in (False, True):
        o, lse = fa.forward(qd, kd, vd, causal=causal)
        dq, dk, dv = fa.backward(qd, kd, vd, o, dod, lse, causal=causal)
        dq2, dke, dve = fa.backward(qd, ke, ve, o, dod, lse, causal=causal)
        torch.cuda.synchronize()
        assert torch.equal(dq, dq2)
        assert_close("dK group sum", dk, np64(dke.view(1, 2, 4, 256, 64).sum(2)), TOL_F32)
        assert_close("dV group sum", dv, np64(dve.view(1, 2, 4, 256, 64).sum(2)), TOL_F32)


def test_gqa_workload_size_sampled_heads(dev):
    # n = 4096, 32 query heads over 8 K/V heads, causal, bf16; four whole
    # query heads against the oracle.
    B, H, h_kv, n, d = 1, 32, 8, 4096, 128
    q, k, v, _ = draw(3300, B, H, h_kv, n, n, d, torch.bfloat16)
    o, lse = fa.forward(q.to(dev), k.to(dev), v.to(dev), causal=True)
    torch.cuda.synchronize()
    o, lse = o.cpu(), lse.cpu()
    for h in (0, 3, 17, 31):
        j = h // (H // h_kv)
        ro, rl = oracle.attention_fwd(np64(q[0, h]), np64(k[0, j]), np64(v[0, j]), 1 / math.sqrt(d), True)
        assert_close(f"O head {h}", o[0, h], ro, 2e-2)
        assert_close(f"LSE head {h}", lse[0, h], rl, TOL_LSE)


def _oracle_bwd_one_kv_head(q, k, v, do, scale, causal, off, w, chunk=8):
    """oracle.attention_bwd_band for one shared K/V head, taken over the
    query heads `chunk` at a time (the repeated K/V of all 64 heads at
    65664 keys would need ~9 GB of fp64): dQ per head, dK and dV summed over
    the chunks, which is the sum over the whole group."""
    q64, k64, v64, do64 = np64(q), np64(k), np64(v), np64(do)
    H = q64.shape[1]
    dqs, dk, dv = [], 0.0, 0.0
    for h0 in range(0, H, chunk):
        sl = slice(h0, h0 + chunk)
        a, b, c = oracle.attention_bwd_band(q64[:, sl], k64, v64, do64[:, sl], scale, causal, off, w)
        dqs.append(a)
        dk, dv = dk + b, dv + c
    return np.concatenate(dqs, axis=1), dk, dv


# One K/V head for 64 query heads at n_k = 65664: one-head runs would need
# more than 4 GiB of partial sums, so the dK/dV workgroups take runs of two
# heads (the head-loop variant).  Plain, causal with the queries at the end
# of the keys, and a window; ragged n_q.
MULTI_RUN = [  # n_q, causal, q_offset, window
    (16, False, 0, -1),
    (17, True, 65664 - 17, -1),
    (33, False, 30000, 3000),
]


@pytest.mark.parametrize("case", MULTI_RUN, ids=lambda c: "nq{}_c{:d}_off{}_w{}".format(*c))
def test_gqa_backward_with_multi_head_runs(dev, case):
    n_q, causal, off, w = case
    B, H, n_k, d = 1, 64, 65664, 128
    assert fa.lib().fa_backward_gqa_workspace_size(B, H, 1, n_q, n_k, d, 1) < \
        fa.backward_workspace_size(B, H, n_q, n_k, d, torch.bfloat16) + 2 * 64 * n_k * d * 4
    q, k, v, do = draw(3400 + n_q, B, H, 1, n_q, n_k, d, torch.bfloat16)
    scale = 1 / math.sqrt(d)
    qd, kd, vd, dod = (t.to(dev) for t in (q, k, v, do))
    window = None if w < 0 else w
    o, lse = fa.forward(qd, kd, vd, causal=causal, q_offset=off, window=window)
    dq, dk, dv = fa.backward(qd, kd, vd, o, dod, lse, causal=causal, q_offset=off, window=window)
    torch.cuda.synchronize()
    rq, rk, rv = _oracle_bwd_one_kv_head(q, k, v, do, scale, causal, off, w)
    tag = f"runs of two heads {case}"
    rtol = bf16_grad_rtol(torch.bfloat16, n_q, n_k, H)
    for name, got, ref in (("dQ", dq, rq), ("dK", dk, rk), ("dV", dv, rv)):
        assert_close(f"{name} {tag}", got.cpu(), ref, tol_for(torch.bfloat16), rtol if name != "dQ" else 0.0)
