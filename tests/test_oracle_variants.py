"""Pins for the oracle's attention variants (shared K/V heads, ...): each is
checked against something other than its own definition -- brute force per
head, finite differences of its own forward, and the special cases that
reduce it to ordinary multi-head attention."""
import numpy as np
import pytest

import oracle


def _rng(seed):
    return np.random.default_rng(seed)


# ------------------------------------------------------ grouped K/V heads

def test_expand_kv_heads_groups_consecutive_query_heads():
    # section 12's picture: 8 query heads over 2 K/V heads -> Q0..Q3 use K0,
    # Q4..Q7 use K1.
    k = np.stack([np.full((3, 2), j, dtype=float) for j in range(2)])  # (2, 3, 2), head j filled with j
    e = oracle.expand_kv_heads(k, 8)
    assert e.shape == (8, 3, 2)
    assert [int(e[h, 0, 0]) for h in range(8)] == [0, 0, 0, 0, 1, 1, 1, 1]
    with pytest.raises(ValueError):
        oracle.expand_kv_heads(np.zeros((3, 4, 2)), 8)


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("h_kv", [1, 2, 4])
def test_gqa_forward_matches_per_head_bruteforce(h_kv, causal):
    r = _rng(41 + h_kv)
    H, n_q, n_k, d = 4, 6, 7, 3
    q = r.standard_normal((H, n_q, d))
    k = r.standard_normal((h_kv, n_k, d))
    v = r.standard_normal((h_kv, n_k, d))
    o, lse = oracle.attention_fwd_gqa(q, k, v, 0.7, causal)
    for h in range(H):
        j = h // (H // h_kv)
        ob, lb = oracle.attention_fwd_bruteforce(q[h], k[j], v[j], 0.7, causal)
        np.testing.assert_allclose(o[h], ob, atol=1e-13)
        np.testing.assert_allclose(lse[h], lb, atol=1e-13)


def test_gqa_with_one_group_per_head_is_multi_head():
    r = _rng(43)
    q, k, v, do = (r.standard_normal((3, 5, 4)) for _ in range(4))
    o1, l1 = oracle.attention_fwd_gqa(q, k, v, 0.5, True)
    o2, l2 = oracle.attention_fwd(q, k, v, 0.5, True)
    np.testing.assert_array_equal(o1, o2)
    np.testing.assert_array_equal(l1, l2)
    got = oracle.attention_bwd_gqa(q, k, v, do, 0.5, True)
    for h in range(3):
        ref = oracle.attention_bwd_bruteforce(q[h], k[h], v[h], do[h], 0.5, True)
        for a, b in zip(got, ref):
            np.testing.assert_allclose(a[h], b, atol=1e-12)


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("h_kv", [1, 2])
def test_gqa_backward_finite_differences(h_kv, causal):
    # the loss sum(dO * O) of the grouped forward, differentiated numerically
    # in every element of q, of the shared k and of the shared v.
    r = _rng(47 + h_kv)
    H, n_q, n_k, d = 4, 4, 5, 2
    q = r.standard_normal((H, n_q, d))
    k = r.standard_normal((h_kv, n_k, d))
    v = r.standard_normal((h_kv, n_k, d))
    do = r.standard_normal((H, n_q, d))
    scale = 0.8
    dq, dk, dv = oracle.attention_bwd_gqa(q, k, v, do, scale, causal)
    assert dk.shape == k.shape and dv.shape == v.shape

    def loss():
        o, _ = oracle.attention_fwd_gqa(q, k, v, scale, causal)
        return float(np.sum(do * o))

    h = 1e-6
    for x, g in ((q, dq), (k, dk), (v, dv)):
        num = np.zeros_like(x)
        for idx in np.ndindex(x.shape):
            old = x[idx]
            x[idx] = old + h
            lp = loss()
            x[idx] = old - h
            lm = loss()
            x[idx] = old
            num[idx] = (lp - lm) / (2 * h)
        np.testing.assert_allclose(g, num, rtol=1e-6, atol=1e-8)


def test_mqa_value_gradient_is_sum_over_heads_of_p_transpose_do():
    # dV of the single shared head equals sum_h P_h^T dO_h, with each P_h
    # from the scalar brute-force softmax.
    r = _rng(53)
    H, n, d = 3, 5, 2
    q = r.standard_normal((H, n, d))
    k = r.standard_normal((1, n, d))
    v = r.standard_normal((1, n, d))
    do = r.standard_normal((H, n, d))
    _, _, dv = oracle.attention_bwd_gqa(q, k, v, do, 0.9, False)
    ref = np.zeros((n, d))
    for h in range(H):
        for i in range(n):
            s = [0.9 * float(np.dot(q[h, i], k[0, j])) for j in range(n)]
            m = max(s)
            e = [np.exp(x - m) for x in s]
            z = sum(e)
            for j in range(n):
                ref[j] += (e[j] / z) * do[h, i]
    np.testing.assert_allclose(dv[0], ref, atol=1e-12)


# ------------------------------------------- query offset and sliding window

def _band_bruteforce(q, k, v, scale, causal, off, w):
    """Scalar loops with the visibility rule written out per pair."""
    n_q, n_k = len(q), len(k)
    o = np.zeros((n_q, v.shape[1]))
    lse = np.full(n_q, -np.inf)
    for i in range(n_q):
        p = i + off
        keys = [j for j in range(n_k) if (not causal or j <= p) and (w < 0 or abs(p - j) <= w)]
        if not keys:
            continue
        s = [scale * float(np.dot(q[i], k[j])) for j in keys]
        m = max(s)
        e = [np.exp(x - m) for x in s]
        z = sum(e)
        o[i] = sum(e[a] * v[j] for a, j in enumerate(keys)) / z
        lse[i] = m + np.log(z)
    return o, lse


def test_band_without_offset_or_window_is_the_top_left_causal_mask():
    for n_q, n_k in ((5, 5), (3, 7), (8, 2)):
        np.testing.assert_array_equal(oracle.band_visible(n_q, n_k, True), oracle.causal_visible(n_q, n_k))
        assert oracle.band_visible(n_q, n_k, False).all()


@pytest.mark.parametrize("n,w", [(10, 0), (10, 3), (10, 9), (17, 4)])
def test_window_pair_count_closed_form(n, w):
    # +-w neighbours of every row, clipped at both ends: n(2w+1) - w(w+1).
    assert int(oracle.band_visible(n, n, False, 0, w).sum()) == n * (2 * w + 1) - w * (w + 1)
    # causal: the w previous keys and the key itself, clipped at the start.
    assert int(oracle.band_visible(n, n, True, 0, w).sum()) == n * (w + 1) - w * (w + 1) // 2


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("off,w", [(0, 2), (3, 1), (-2, 3), (4, -1), (0, 0), (-6, -1)])
def test_band_forward_matches_bruteforce(causal, off, w):
    r = _rng(61 + off * 7 + w)
    q, k, v = r.standard_normal((6, 3)), r.standard_normal((8, 3)), r.standard_normal((8, 2))
    o, lse = oracle.attention_fwd_band(q, k, v, 0.8, causal, off, w)
    ob, lb = _band_bruteforce(q, k, v, 0.8, causal, off, w)
    np.testing.assert_allclose(o, ob, atol=1e-13)
    np.testing.assert_array_equal(np.isfinite(lse), np.isfinite(lb))
    np.testing.assert_allclose(lse[np.isfinite(lse)], lb[np.isfinite(lb)], atol=1e-13)


def test_window_zero_causal_returns_the_aligned_value_row():
    # Each row sees exactly key i + off: O_i = V_{i+off}, LSE_i = scale q_i.k_{i+off}.
    r = _rng(67)
    q, k, v = r.standard_normal((4, 3)), r.standard_normal((9, 3)), r.standard_normal((9, 2))
    o, lse = oracle.attention_fwd_band(q, k, v, 0.5, True, 5, 0)
    for i in range(4):
        np.testing.assert_allclose(o[i], v[i + 5], atol=1e-15)
        np.testing.assert_allclose(lse[i], 0.5 * np.dot(q[i], k[i + 5]), atol=1e-14)


def test_last_query_on_last_key_sees_everything():
    # One query at offset n_k - 1 with the causal mask is plain attention
    # over all keys; a window at least n_k wide changes nothing.
    r = _rng(71)
    q, k, v = r.standard_normal((1, 4)), r.standard_normal((20, 4)), r.standard_normal((20, 4))
    o1, l1 = oracle.attention_fwd_band(q, k, v, 0.4, True, 19, -1)
    o2, l2 = oracle.attention_fwd(q, k, v, 0.4, False)
    np.testing.assert_allclose(o1, o2, atol=1e-14)
    np.testing.assert_allclose(l1, l2, atol=1e-14)
    o3, l3 = oracle.attention_fwd_band(q, k, v, 0.4, False, 7, 25)
    np.testing.assert_allclose(o3, o2, atol=1e-14)


def test_rows_that_see_no_key_are_zero_with_minus_infinite_lse():
    r = _rng(73)
    q, k, v = r.standard_normal((5, 2)), r.standard_normal((5, 2)), r.standard_normal((5, 2))
    o, lse = oracle.attention_fwd_band(q, k, v, 1.0, True, -3, -1)  # rows 0..2 sit before key 0
    assert np.all(o[:3] == 0) and np.all(np.isneginf(lse[:3]))
    assert np.all(np.isfinite(lse[3:]))
    _, _, dv = oracle.attention_bwd_band(q, k, v, np.ones((5, 2)), 1.0, True, -3, -1)
    # only rows 3, 4 contribute: dV sums their probabilities
    assert abs(float(dv.sum()) - 2 * 2) < 1e-12


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("off,w,h_kv", [(0, 1, 2), (2, 2, 1), (-1, -1, 2)])
def test_band_backward_finite_differences(causal, off, w, h_kv):
    r = _rng(79 + w + 3 * off)
    H, n_q, n_k, d = 2, 4, 5, 2
    q = r.standard_normal((H, n_q, d))
    k = r.standard_normal((h_kv, n_k, d))
    v = r.standard_normal((h_kv, n_k, d))
    do = r.standard_normal((H, n_q, d))
    dq, dk, dv = oracle.attention_bwd_band(q, k, v, do, 0.7, causal, off, w)

    def loss():
        o, _ = oracle.attention_fwd_band(q, k, v, 0.7, causal, off, w)
        return float(np.sum(do * o))

    h = 1e-6
    for x, g in ((q, dq), (k, dk), (v, dv)):
        num = np.zeros_like(x)
        for idx in np.ndindex(x.shape):
            old = x[idx]
            x[idx] = old + h
            lp = loss()
            x[idx] = old - h
            lm = loss()
            x[idx] = old
            num[idx] = (lp - lm) / (2 * h)
        np.testing.assert_allclose(g, num, rtol=1e-6, atol=1e-8)


# ------------------------------------------------ merging key-split results

def _chunks(n_k, cuts):
    edges = [0] + list(cuts) + [n_k]
    return [(a, b) for a, b in zip(edges[:-1], edges[1:])]


@pytest.mark.parametrize("causal,off,w", [(False, 0, -1), (True, 0, -1), (True, 37, -1), (True, 5, 9),
                                          (False, -3, 6)])
@pytest.mark.parametrize("cuts", [(17,), (1, 2, 30), (11, 11, 40)])
def test_merge_of_key_chunks_is_the_attention_over_all_keys(causal, off, w, cuts):
    # Each chunk [a, b) is attention over keys a..b-1 alone, with the query
    # offset shifted by -a so that positions stay absolute; merged, the chunks
    # must give the plain definition over all keys (brute force).
    rng = _rng(70)
    n_q, n_k, d, scale = 9, 48, 5, 0.4
    q, k, v = rng.standard_normal((n_q, d)), rng.standard_normal((n_k, d)), rng.standard_normal((n_k, d))
    parts = [oracle.attention_fwd_band(q, k[a:b], v[a:b], scale, causal, off - a, w) for a, b in _chunks(n_k, cuts)]
    o, lse = oracle.lse_merge(np.stack([p[0] for p in parts]), np.stack([p[1] for p in parts]))
    ro, rl = _band_bruteforce(q, k, v, scale, causal, off, w)
    assert np.array_equal(np.isfinite(lse), np.isfinite(rl))
    np.testing.assert_allclose(o, ro, atol=1e-12)
    fin = np.isfinite(rl)
    np.testing.assert_allclose(lse[fin], rl[fin], atol=1e-12)


def test_merge_of_a_random_key_partition_non_causal():
    # Without a mask any partition of the keys works, not just contiguous
    # chunks: softmax is a sum over a set.
    rng = _rng(71)
    q, k, v = rng.standard_normal((6, 4)), rng.standard_normal((30, 4)), rng.standard_normal((30, 4))
    perm = rng.permutation(30)
    sets = [perm[:7], perm[7:8], perm[8:]]
    parts = [oracle.attention_fwd(q, k[s], v[s], 0.7) for s in sets]
    o, lse = oracle.lse_merge(np.stack([p[0] for p in parts]), np.stack([p[1] for p in parts]))
    ro, rl = _band_bruteforce(q, k, v, 0.7, False, 0, -1)
    np.testing.assert_allclose(o, ro, atol=1e-12)
    np.testing.assert_allclose(lse, rl, atol=1e-12)


def test_merge_special_cases():
    rng = _rng(72)
    o1, l1 = rng.standard_normal((4, 3)), rng.standard_normal(4)
    # one part: unchanged
    o, l = oracle.lse_merge(o1[None], l1[None])
    np.testing.assert_array_equal(o, o1)
    np.testing.assert_array_equal(l, l1)
    # two equal parts: same O, LSE + ln 2
    o, l = oracle.lse_merge(np.stack([o1, o1]), np.stack([l1, l1]))
    np.testing.assert_allclose(o, o1, atol=1e-15)
    np.testing.assert_allclose(l, l1 + np.log(2.0), atol=1e-15)
    # a part without visible keys (O = 0, LSE = -inf) changes nothing
    o, l = oracle.lse_merge(np.stack([np.zeros_like(o1), o1]), np.stack([np.full(4, -np.inf), l1]))
    np.testing.assert_array_equal(o, o1)
    np.testing.assert_array_equal(l, l1)
    # no part with visible keys: O = 0, LSE = -inf
    o, l = oracle.lse_merge(np.zeros((3, 4, 3)), np.full((3, 4), -np.inf))
    assert np.all(o == 0) and np.all(l == -np.inf)
    # weights: parts with LSE a and b weigh e^a : e^b
    o, l = oracle.lse_merge(np.stack([np.ones((1, 1)), np.zeros((1, 1))]), np.array([[0.0], [np.log(3.0)]]))
    np.testing.assert_allclose(o, [[0.25]], atol=1e-15)
    np.testing.assert_allclose(l, [np.log(4.0)], atol=1e-15)


def test_merge_of_decode_chunks_with_shared_heads():
    # The decode shape: a few new queries at the end of a long cache
    # (q_offset = n_k - n_q, causal), 4 query heads on 2 K/V heads, the cache
    # split in uneven chunks.
    rng = _rng(73)
    H, h_kv, n_q, n_k, d = 4, 2, 3, 70, 8
    q = rng.standard_normal((H, n_q, d))
    k, v = rng.standard_normal((h_kv, n_k, d)), rng.standard_normal((h_kv, n_k, d))
    off = n_k - n_q
    parts = [oracle.attention_fwd_band(q, k[:, a:b], v[:, a:b], 0.35, True, off - a) for a, b in _chunks(n_k, (20, 21, 64))]
    o, lse = oracle.lse_merge(np.stack([p[0] for p in parts]), np.stack([p[1] for p in parts]))
    for h in range(H):
        ro, rl = _band_bruteforce(q[h], k[h // 2], v[h // 2], 0.35, True, off, -1)
        np.testing.assert_allclose(o[h], ro, atol=1e-12)
        np.testing.assert_allclose(lse[h], rl, atol=1e-12)
