"""Pins for the fp64 oracle: values it must reproduce that do not come from
the oracle itself -- brute force, closed forms, invariants, finite
differences, torch autograd of the definition, and the numbers the pages
print (tests/golden/)."""
import json
import math
import os

import numpy as np
import pytest
import torch

import oracle
import workloads

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _rng(seed):
    return np.random.default_rng(seed)


def _head(seed, n_q, n_k, d, std=1.0):
    r = _rng(seed)
    return (r.standard_normal((n_q, d)) * std, r.standard_normal((n_k, d)) * std,
            r.standard_normal((n_k, d)))


# ----------------------------------------------------------------- forward

@pytest.mark.parametrize("n_q,n_k,d", [(1, 1, 1), (5, 5, 3), (7, 4, 2), (4, 9, 5), (16, 16, 8)])
@pytest.mark.parametrize("causal", [False, True])
def test_forward_matches_bruteforce(n_q, n_k, d, causal):
    q, k, v = _head(n_q * 100 + n_k * 10 + d, n_q, n_k, d)
    scale = 1.0 / math.sqrt(d)
    o, lse = oracle.attention_fwd(q, k, v, scale, causal)
    ob, lb = oracle.attention_fwd_bruteforce(q, k, v, scale, causal)
    np.testing.assert_allclose(o, ob, rtol=0, atol=1e-13)
    np.testing.assert_allclose(lse, lb, rtol=0, atol=1e-13)


def test_two_keys_closed_form():
    # With two visible keys the softmax is a logistic function of the score
    # difference: O = sigma(s0 - s1) V0 + sigma(s1 - s0) V1.
    q, k, v = _head(11, 3, 2, 4)
    scale = 0.7
    o, lse = oracle.attention_fwd(q, k, v, scale, False)
    s0 = scale * q @ k[0]
    s1 = scale * q @ k[1]
    w0 = 1.0 / (1.0 + np.exp(s1 - s0))
    expect = w0[:, None] * v[0] + (1.0 - w0)[:, None] * v[1]
    np.testing.assert_allclose(o, expect, atol=1e-14)
    np.testing.assert_allclose(lse, np.logaddexp(s0, s1), atol=1e-14)


@pytest.mark.parametrize("n_q,n_k", [(6, 6), (4, 9), (9, 4)])
@pytest.mark.parametrize("causal", [False, True])
def test_zero_query_gives_mean_of_visible_values(n_q, n_k, causal):
    # Q = 0 makes every visible score 0: uniform weights over visible keys.
    _, k, v = _head(3, n_q, n_k, 5)
    q = np.zeros((n_q, 5))
    o, lse = oracle.attention_fwd(q, k, v, 0.3, causal)
    for i in range(n_q):
        cnt = min(i + 1, n_k) if causal else n_k
        np.testing.assert_allclose(o[i], v[:cnt].mean(axis=0), atol=1e-14)
        assert abs(lse[i] - math.log(cnt)) < 1e-14


def test_scale_zero_equals_uniform():
    q, k, v = _head(4, 5, 7, 3)
    o, _ = oracle.attention_fwd(q, k, v, 0.0, False)
    np.testing.assert_allclose(o, np.broadcast_to(v.mean(axis=0), o.shape), atol=1e-14)


def test_causal_first_row_sees_only_key_zero():
    q, k, v = _head(5, 8, 8, 6)
    scale = 0.4
    o, lse = oracle.attention_fwd(q, k, v, scale, True)
    np.testing.assert_array_equal(o[0], v[0])
    assert abs(lse[0] - scale * q[0] @ k[0]) < 1e-14


def test_single_key():
    q, k, v = _head(6, 5, 1, 4)
    o, lse = oracle.attention_fwd(q, k, v, 0.5, False)
    np.testing.assert_allclose(o, np.broadcast_to(v[0], o.shape), atol=1e-15)
    np.testing.assert_allclose(lse, 0.5 * q @ k[0], atol=1e-14)


def test_constant_value_rows_return_that_value():
    q, k, _ = _head(7, 6, 9, 4)
    c = np.array([0.25, -1.5, 3.0, 7.0])
    v = np.tile(c, (9, 1))
    for causal in (False, True):
        o, _ = oracle.attention_fwd(q, k, v, 0.5, causal)
        np.testing.assert_allclose(o, np.broadcast_to(c, o.shape), atol=1e-14)


def test_probability_rows_sum_to_one_and_are_nonnegative():
    # "Attention Mechanism", section 3: each weight row is a probability
    # distribution over keys.
    q, k, _ = _head(8, 12, 10, 4)
    for causal in (False, True):
        p, _ = oracle.softmax_rows(oracle.scores(q, k, 0.5, causal))
        assert np.all(p >= 0)
        np.testing.assert_allclose(p.sum(axis=-1), 1.0, atol=1e-15)
        if causal:
            assert np.all(p[~oracle.causal_visible(12, 10)] == 0)


def test_causal_mask_is_lower_triangular_top_left():
    vis = oracle.causal_visible(4, 6)
    expect = np.array([[1, 0, 0, 0, 0, 0],
                       [1, 1, 0, 0, 0, 0],
                       [1, 1, 1, 0, 0, 0],
                       [1, 1, 1, 1, 0, 0]], dtype=bool)
    np.testing.assert_array_equal(vis, expect)


# ----------------------------------------------------------- invariances

def test_joint_key_value_permutation_invariance():
    q, k, v = _head(9, 7, 11, 4)
    perm = _rng(1).permutation(11)
    o1, l1 = oracle.attention_fwd(q, k, v, 0.5, False)
    o2, l2 = oracle.attention_fwd(q, k[perm], v[perm], 0.5, False)
    np.testing.assert_allclose(o1, o2, atol=1e-14)
    np.testing.assert_allclose(l1, l2, atol=1e-14)


def test_key_shift_moves_lse_not_output():
    q, k, v = _head(10, 7, 11, 4)
    c = np.array([0.5, -2.0, 1.0, 3.0])
    scale = 0.5
    o1, l1 = oracle.attention_fwd(q, k, v, scale, False)
    o2, l2 = oracle.attention_fwd(q, k + c, v, scale, False)
    np.testing.assert_allclose(o1, o2, atol=1e-13)
    np.testing.assert_allclose(l2, l1 + scale * q @ c, atol=1e-13)


def test_query_permutation_permutes_output():
    q, k, v = _head(12, 9, 6, 4)
    perm = _rng(2).permutation(9)
    o1, l1 = oracle.attention_fwd(q, k, v, 0.5, False)
    o2, l2 = oracle.attention_fwd(q[perm], k, v, 0.5, False)
    np.testing.assert_allclose(o2, o1[perm], atol=1e-15)
    np.testing.assert_allclose(l2, l1[perm], atol=1e-15)


def test_causal_future_keys_do_not_matter():
    q, k, v = _head(13, 10, 10, 4)
    o1, l1 = oracle.attention_fwd(q, k, v, 0.5, True)
    i = 4
    k2, v2 = k.copy(), v.copy()
    k2[i + 1:] += 100.0
    v2[i + 1:] -= 50.0
    o2, l2 = oracle.attention_fwd(q, k2, v2, 0.5, True)
    np.testing.assert_array_equal(o1[: i + 1], o2[: i + 1])
    np.testing.assert_array_equal(l1[: i + 1], l2[: i + 1])


def test_batch_and_heads_are_independent():
    r = _rng(14)
    q, k, v = (r.standard_normal((2, 3, 8, 4)) for _ in range(3))
    o, lse = oracle.attention_fwd(q, k, v, 0.5, True)
    for b in range(2):
        for h in range(3):
            ob, lb = oracle.attention_fwd_bruteforce(q[b, h], k[b, h], v[b, h], 0.5, True)
            np.testing.assert_allclose(o[b, h], ob, atol=1e-13)
            np.testing.assert_allclose(lse[b, h], lb, atol=1e-13)


# --------------------------------------------------- tiling and online form

def test_row_tiling_is_bitwise_identical_at_n4096_d64():
    # "Efficient Attention": 128-row query blocks over all keys give exactly
    # the full result (the script's third part, at its n = 4096, d = 64).
    w = workloads.c2()
    q, k, v = (t[0, 0].numpy().astype(np.float64) for t in (w.q, w.k, w.v))
    o, lse = oracle.attention_fwd(q, k, v, w.scale, False)
    ot, lt = oracle.attention_fwd_row_tiled(q, k, v, w.scale, False, block=128)
    assert np.array_equal(o, ot)
    assert np.array_equal(lse, lt)


def test_row_tiling_causal_small():
    q, k, v = _head(15, 37, 37, 8)
    o, lse = oracle.attention_fwd(q, k, v, 0.3, True)
    ot, lt = oracle.attention_fwd_row_tiled(q, k, v, 0.3, True, block=8)
    np.testing.assert_allclose(o, ot, atol=1e-15)
    np.testing.assert_allclose(lse, lt, atol=1e-15)


@pytest.mark.parametrize("block_k", [1, 7, 32, 64, 200])
@pytest.mark.parametrize("causal", [False, True])
def test_online_blocked_equals_full(block_k, causal):
    q, k, v = _head(16, 150, 150, 16, std=1.5)
    o, lse = oracle.attention_fwd(q, k, v, 0.25, causal)
    ob, lb = oracle.online_softmax_blocked(q, k, v, 0.25, causal, block_k=block_k)
    np.testing.assert_allclose(ob, o, atol=1e-12)
    np.testing.assert_allclose(lb, lse, atol=1e-12)


def test_page_printed_online_update_is_wrong():
    # The update printed in "Attention Mechanism", section 13, drops the
    # exp(m_old - m_new) factor on the old output; with scores whose running
    # maximum moves between blocks it does not reproduce attention.
    w = workloads.c2()
    q, k, v = (t[0, 0, :256].numpy().astype(np.float64) for t in (w.q, w.k, w.v))
    o, _ = oracle.attention_fwd(q, k, v, w.scale, False)
    good, _ = oracle.online_softmax_blocked(q, k, v, w.scale, False, block_k=32)
    bad, _ = oracle.online_softmax_blocked(q, k, v, w.scale, False, block_k=32,
                                           literal_page_rule=True)
    assert np.max(np.abs(good - o)) < 1e-13
    assert np.max(np.abs(bad - o)) > 1e-2


def test_online_blocked_rising_scores_stress():
    # Scores that rise along the keys move the running max in every block.
    n, d = 96, 4
    q = np.ones((n, d))
    k = np.outer(np.arange(n) / 4.0, np.ones(d))
    v = _rng(17).standard_normal((n, d))
    for causal in (False, True):
        o, lse = oracle.attention_fwd(q, k, v, 1.0, causal)
        ob, lb = oracle.online_softmax_blocked(q, k, v, 1.0, causal, block_k=16)
        np.testing.assert_allclose(ob, o, atol=1e-12)
        np.testing.assert_allclose(lb, lse, rtol=1e-14)


def test_rows_entry_matches_full():
    r = _rng(18)
    q, k, v = (r.standard_normal((1, 3, 40, 8)) for _ in range(3))
    rows = [(0, 0, 0), (0, 1, 17), (0, 2, 39), (0, 2, 5)]
    for causal in (False, True):
        o, lse = oracle.attention_fwd(q, k, v, 0.35, causal)
        orow, lrow = oracle.attention_rows(q, k, v, rows, 0.35, causal)
        for n, (b, h, i) in enumerate(rows):
            np.testing.assert_allclose(orow[n], o[b, h, i], atol=1e-14)
            assert abs(lrow[n] - lse[b, h, i]) < 1e-13


# ----------------------------------------------------------------- backward

def _loss(q, k, v, do, scale, causal):
    o, _ = oracle.attention_fwd(q, k, v, scale, causal)
    return float(np.sum(do * o))


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("n_q,n_k", [(5, 5), (3, 6)])
def test_backward_finite_differences(causal, n_q, n_k):
    d = 3
    r = _rng(19 + n_q)
    q, k, v = r.standard_normal((n_q, d)), r.standard_normal((n_k, d)), r.standard_normal((n_k, d))
    do = r.standard_normal((n_q, d))
    scale = 0.6
    dq, dk, dv = oracle.attention_bwd(q, k, v, do, scale, causal)
    h = 1e-6
    for x, g in ((q, dq), (k, dk), (v, dv)):
        num = np.zeros_like(x)
        for idx in np.ndindex(x.shape):
            old = x[idx]
            x[idx] = old + h
            lp = _loss(q, k, v, do, scale, causal)
            x[idx] = old - h
            lm = _loss(q, k, v, do, scale, causal)
            x[idx] = old
            num[idx] = (lp - lm) / (2 * h)
        np.testing.assert_allclose(g, num, rtol=1e-6, atol=1e-8)


@pytest.mark.parametrize("causal", [False, True])
def test_backward_matches_scalar_bruteforce(causal):
    r = _rng(23)
    q, k, v, do = (r.standard_normal((6, 4)) for _ in range(4))
    got = oracle.attention_bwd(q, k, v, do, 0.45, causal)
    ref = oracle.attention_bwd_bruteforce(q, k, v, do, 0.45, causal)
    for a, b in zip(got, ref):
        np.testing.assert_allclose(a, b, atol=1e-13)


@pytest.mark.parametrize("causal", [False, True])
def test_backward_matches_torch_autograd_of_definition(causal):
    # torch differentiates the forward definition by itself (fp64, CPU);
    # the oracle's explicit chain rule must agree.
    r = _rng(29)
    n_q, n_k, d = 33, 33, 8
    q, k, v, do = (r.standard_normal(s) for s in ((2, n_q, d), (2, n_k, d), (2, n_k, d), (2, n_q, d)))
    tq, tk, tv = (torch.tensor(x, requires_grad=True) for x in (q, k, v))
    s = 0.35 * tq @ tk.transpose(-1, -2)
    if causal:
        mask = torch.ones(n_q, n_k, dtype=torch.bool).tril()
        s = s.masked_fill(~mask, float("-inf"))
    o = torch.softmax(s, dim=-1) @ tv
    o.backward(torch.tensor(do))
    dq, dk, dv = oracle.attention_bwd(q, k, v, do, 0.35, causal)
    np.testing.assert_allclose(dq, tq.grad.numpy(), atol=1e-12)
    np.testing.assert_allclose(dk, tk.grad.numpy(), atol=1e-12)
    np.testing.assert_allclose(dv, tv.grad.numpy(), atol=1e-12)


@pytest.mark.parametrize("causal", [False, True])
def test_backward_identities(causal):
    r = _rng(31)
    n, d = 64, 16
    q, k, v, do = (r.standard_normal((n, d)) for _ in range(4))
    scale = 0.25
    dq, dk, dv = oracle.attention_bwd(q, k, v, do, scale, causal)
    # Softmax rows sum to one, so their gradient rows sum to zero; hence the
    # key gradients sum to zero and the value gradients sum to sum_i dO_i.
    np.testing.assert_allclose(dk.sum(axis=0), 0.0, atol=1e-12)
    np.testing.assert_allclose(dv.sum(axis=0), do.sum(axis=0), atol=1e-12)
    # rowsum(dO o O) equals rowsum(P o dP).
    p, _ = oracle.softmax_rows(oracle.scores(q, k, scale, causal))
    o = p @ v
    np.testing.assert_allclose(np.sum(do * o, axis=1), np.sum(p * (do @ v.T), axis=1), atol=1e-12)


def test_backward_constant_values_give_zero_q_k_gradients():
    r = _rng(37)
    q, k, do = (r.standard_normal((9, 4)) for _ in range(3))
    v = np.tile(np.array([1.0, -2.0, 0.5, 4.0]), (9, 1))
    for causal in (False, True):
        dq, dk, dv = oracle.attention_bwd(q, k, v, do, 0.5, causal)
        np.testing.assert_allclose(dq, 0.0, atol=1e-13)
        np.testing.assert_allclose(dk, 0.0, atol=1e-13)


# ------------------------------------------------- values the pages print

def test_page_script_inputs_and_manual_vs_sdpa_difference():
    # Provenance of the c1 inputs: "Efficient Attention" prints the largest
    # difference between an fp32 attention computed step by step (scores
    # divided by sqrt(d), row softmax, weighted sum) and PyTorch's fused
    # scaled_dot_product_attention on its seed-9 tensors.  Recomputing that
    # difference on c1's tensors must give the printed value, so c1's tensors
    # are the page's.  The fp32 reference is taken here with einsum products;
    # the score count is the oracle's closed form.
    g = json.load(open(os.path.join(GOLDEN, "efficient_attention_script_output.json")))["manual_vs_sdpa"]
    w = workloads.c1()
    B, H, n, d = w.q.shape
    assert oracle.score_bytes(B, H, n, 4) == g["score_bytes"]
    weights = torch.softmax(torch.einsum("bhid,bhjd->bhij", w.q, w.k) / math.sqrt(d), dim=-1)
    stepwise = torch.einsum("bhij,bhjd->bhid", weights, w.v)
    fused = torch.nn.functional.scaled_dot_product_attention(w.q, w.k, w.v)
    gap = float((stepwise - fused).abs().max())
    assert f"{gap:.2e}" == g["max_abs_diff_printed"]
    assert gap <= g["allclose_atol"]
    # The fp64 oracle sits within the page's fp32 tolerance of both.
    o, _ = oracle.attention_fwd(w.q.double().numpy(), w.k.double().numpy(), w.v.double().numpy(), w.scale)
    for name, t in (("step by step", stepwise), ("fused", fused)):
        assert np.max(np.abs(o - t.double().numpy())) < g["allclose_atol"], name


def test_score_memory_closed_forms():
    g = json.load(open(os.path.join(GOLDEN, "efficient_attention_script_output.json")))
    assert oracle.score_bytes(2, 3, 128, 4) == g["manual_vs_sdpa"]["score_bytes"]
    # The page prints sizes in binary units ("MB" = 2^20 bytes, "GB" = 2^30)
    # rounded to the digits shown: each printed figure must be the closed
    # form's byte count in that unit, to within half its last digit.
    def matches(nbytes, printed):
        number, unit = printed.split()
        digits = len(number.split(".")[1]) if "." in number else 0
        scale = {"MB": 2.0 ** 20, "GB": 2.0 ** 30}[unit]
        return abs(nbytes / scale - float(number)) <= 0.5 * 10.0 ** -digits

    for row in g["score_memory_table_fp32_b1_h1"]:
        assert row["n"] ** 2 == row["elements"]
        b = oracle.score_bytes(1, 1, row["n"], 4)
        assert b == row["bytes"]
        assert matches(b, row["printed"]), row
    t = g["row_tiling"]
    full = oracle.score_bytes(1, 1, t["n"], 4)
    block = t["block"] * t["n"] * 4
    assert (full, block, full // block) == (t["full_bytes"], t["block_bytes"], t["saving_factor"])
    assert matches(full, t["full_printed"]) and matches(block, t["block_printed"])


def test_memory_calculator_worked_example():
    g = json.load(open(os.path.join(GOLDEN, "attention_memory_calculator_example.json")))
    e = g["worked_example"]
    b = oracle.score_bytes(e["batch"], e["heads"], e["seq_len"], e["bytes_per_element"])
    assert b == e["bytes"]
    assert f"{b / 1e9:.2f}" == e["printed_gb"]
    e2 = g["doubled_context"]
    b2 = oracle.score_bytes(e2["batch"], e2["heads"], e2["seq_len"], e2["bytes_per_element"])
    assert f"{b2 / 1e9:.2f}" == e2["printed_gb"]
    assert b2 == 4 * b


def test_flop_count_matches_visible_pairs():
    for n_q, n_k in ((7, 7), (5, 9), (9, 5)):
        vis = oracle.causal_visible(n_q, n_k).sum()
        assert oracle.attention_flops(2, 3, n_q, n_k, 8, True) == 2 * 3 * vis * 4 * 8
        assert oracle.attention_flops(2, 3, n_q, n_k, 8, True, backward=True) == 2 * 3 * vis * 10 * 8
        assert oracle.attention_flops(1, 1, n_q, n_k, 8, False) == n_q * n_k * 32
    # The forward count at the headline shape.
    assert oracle.attention_flops(1, 32, 4096, 4096, 128, False) == 274877906944
