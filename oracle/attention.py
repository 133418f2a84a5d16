"""Plain fp64 CPU oracle for exact scaled dot-product attention.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path may import, call or
execute this module: only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` use it.  It shares no code with the HIP
library (no kernels, headers, helpers or constants) and never imports it.

Everything here is the textbook definition written out in numpy float64, with
the full score matrix materialised, so that a reader can check it against the
pages by eye:

* the formula softmax(Q K^T / sqrt(d_k)) V and its four steps (score, scale,
  row softmax whose rows sum to one, weighted sum of value rows) --
  "Attention Mechanism: Revolusi Representasi Sequence", section 3
  "Scaled Dot-Product Attention: Formula Inti";
* the causal mask M[i][j] = 0 for j <= i and -inf for j > i, added after the
  scaling -- same page, section 4.4 "Causal / Masked Attention";
* Q is (n_q, d_k), K is (n_k, d_k), V is (n_k, d_v) with d_v = d_k here --
  same page, section 3, component table;
* the per-row log-sum-exp kept for the backward pass -- "Flash Attention
  Nedir? Transformer Bellek Optimizasyonu", section "Online Softmax";
* the backward pass, which the pages describe only as recomputing the
  softmax blocks ("Apa itu FlashAttention", section "Cara kerja teknik
  Tiling dan Recomputation"; "Flash Attention Nedir?", section
  "Recomputation"), written as the explicit chain rule through
  O = P V and P = softmax(S):  dV = P^T dO, dP = dO V^T,
  D_i = sum_k dO_ik O_ik, dS = P o (dP - D), dQ = scale dS K,
  dK = scale dS^T Q.

Readings where the pages are silent or garbled:

* the scale is an explicit argument; every workload uses 1/sqrt(d);
* causal alignment when n_q != n_k is top-left: key j is hidden from query i
  exactly when j > i in absolute indices, so every row sees key 0;
* the LSE uses the natural logarithm of sum_j exp(S_ij) over scaled, masked
  scores;
* the online-softmax output update printed in "Attention Mechanism",
  section 13 "FlashAttention -- How It Works", omits the factor
  exp(m_old - m_new) on the old output; ``online_softmax_blocked`` applies the
  corrected update and can also run the printed one (``literal_page_rule``)
  so that a test shows it is wrong.

Every function here is pinned by ``tests/test_oracle_pins.py`` and
``tests/test_oracle_variants.py`` against brute force, closed forms,
invariants, finite differences and the values the pages print.
"""
from __future__ import annotations

import math

import numpy as np

__all__ = [
    "causal_visible",
    "scores",
    "softmax_rows",
    "attention_fwd",
    "attention_bwd",
    "attention_rows",
    "attention_fwd_row_tiled",
    "online_softmax_blocked",
    "attention_fwd_bruteforce",
    "attention_bwd_bruteforce",
    "score_bytes",
    "attention_flops",
    "expand_kv_heads",
    "attention_fwd_gqa",
    "attention_bwd_gqa",
    "band_visible",
    "attention_fwd_band",
    "attention_bwd_band",
    "lse_merge",
]


def _f64(x) -> np.ndarray:
    a = np.asarray(x)
    if a.dtype != np.float64:
        a = a.astype(np.float64)
    return a


def causal_visible(n_q: int, n_k: int) -> np.ndarray:
    """Boolean (n_q, n_k) matrix: True where key j is visible to query i.

    The mask of "Attention Mechanism", section 4.4: j <= i is kept, j > i is
    hidden (top-left alignment when n_q != n_k).
    """
    i = np.arange(n_q)[:, None]
    j = np.arange(n_k)[None, :]
    return j <= i


def scores(q, k, scale: float, causal: bool) -> np.ndarray:
    """S = scale * Q K^T with -inf on hidden positions; shape (..., n_q, n_k)."""
    q = _f64(q)
    k = _f64(k)
    s = float(scale) * np.matmul(q, np.swapaxes(k, -1, -2))
    if causal:
        s = np.where(causal_visible(q.shape[-2], k.shape[-2]), s, -np.inf)
    return s


def softmax_rows(s: np.ndarray):
    """Row softmax of a score matrix and its natural-log log-sum-exp.

    Returns (P, LSE) with P = exp(S - LSE) row by row.  The row maximum is
    subtracted before exponentiating; rows are never fully masked under the
    top-left causal reading, so the maximum is always finite.
    """
    m = np.max(s, axis=-1, keepdims=True)
    e = np.exp(s - m)
    l = np.sum(e, axis=-1, keepdims=True)
    p = e / l
    lse = (m + np.log(l))[..., 0]
    return p, lse


def attention_fwd(q, k, v, scale: float, causal: bool = False):
    """Full forward pass: (O, LSE).

    q: (..., n_q, d); k, v: (..., n_k, d).  O has q's shape; LSE is (..., n_q).
    The score matrix S and probabilities P are materialised in full.
    """
    v = _f64(v)
    p, lse = softmax_rows(scores(q, k, scale, causal))
    o = np.matmul(p, v)
    return o, lse


def attention_bwd(q, k, v, do, scale: float, causal: bool = False, intermediates: bool = False):
    """Explicit backward pass from the oracle's own fp64 forward: (dQ, dK, dV).

    Uses the materialised P and O (no recomputation shortcut), then the chain
    rule listed in the module docstring.  Hidden positions have P = 0 and so
    dS = 0.  With ``intermediates=True`` a fourth element, the dict
    {"p": P, "ds": dS}, is returned as well.
    """
    q = _f64(q)
    k = _f64(k)
    v = _f64(v)
    do = _f64(do)
    p, _ = softmax_rows(scores(q, k, scale, causal))
    o = np.matmul(p, v)
    dv = np.matmul(np.swapaxes(p, -1, -2), do)
    dp = np.matmul(do, np.swapaxes(v, -1, -2))
    dsum = np.sum(do * o, axis=-1, keepdims=True)
    ds = p * (dp - dsum)
    dq = float(scale) * np.matmul(ds, k)
    dk = float(scale) * np.matmul(np.swapaxes(ds, -1, -2), q)
    if intermediates:
        return dq, dk, dv, {"p": p, "ds": ds}
    return dq, dk, dv


def attention_rows(q, k, v, rows, scale: float, causal: bool = False):
    """Forward pass for a chosen list of query rows only.

    q: (B, H, n_q, d); k, v: (B, H, n_k, d); rows: iterable of (b, h, i).
    Each row is the definition applied to one query: scores against the
    visible keys (all keys, or keys 0..i when causal), softmax, weighted sum.
    Returns (O_rows (R, d), LSE_rows (R,)).
    """
    q = np.asarray(q)
    k = np.asarray(k)
    v = np.asarray(v)
    rows = list(rows)
    d = q.shape[-1]
    out = np.empty((len(rows), d), dtype=np.float64)
    lse = np.empty((len(rows),), dtype=np.float64)
    for r, (b, h, i) in enumerate(rows):
        kk = _f64(k[b, h])
        vv = _f64(v[b, h])
        if causal:
            kk = kk[: i + 1]
            vv = vv[: i + 1]
        s = float(scale) * (kk @ _f64(q[b, h, i]))
        m = np.max(s)
        e = np.exp(s - m)
        l = np.sum(e)
        out[r] = (e / l) @ vv
        lse[r] = m + np.log(l)
    return out, lse


def attention_fwd_row_tiled(q, k, v, scale: float, causal: bool = False, block: int = 128):
    """Forward pass computed one block of query rows at a time.

    Each block of ``block`` query rows takes a full-row softmax over all keys
    and the blocks are concatenated: the row-tiling demonstration of
    "Efficient Attention", section "Mengapa Memori Attention Tumbuh
    Kuadratik" (script part 3).  Rows never interact, so the result must equal
    ``attention_fwd``.
    """
    q = _f64(q)
    n_q = q.shape[-2]
    outs, lses = [], []
    for start in range(0, n_q, block):
        qb = q[..., start : start + block, :]
        s = float(scale) * np.matmul(qb, np.swapaxes(_f64(k), -1, -2))
        if causal:
            i = np.arange(start, start + qb.shape[-2])[:, None]
            j = np.arange(s.shape[-1])[None, :]
            s = np.where(j <= i, s, -np.inf)
        p, lse = softmax_rows(s)
        outs.append(np.matmul(p, _f64(v)))
        lses.append(lse)
    return np.concatenate(outs, axis=-2), np.concatenate(lses, axis=-1)


def online_softmax_blocked(q, k, v, scale: float, causal: bool = False, block_k: int = 128,
                           literal_page_rule: bool = False):
    """Key-blocked online softmax, as sketched in "Attention Mechanism",
    section 13 "FlashAttention -- How It Works" (tiling plus running max and
    running sum), in that page's notation m, l, P, O.

    State per query row starts at m = -inf, l = 0, O = 0.  For each key block:
      S     = scale * Q K_blk^T   (masked)
      m_new = max(m_old, rowmax S)
      P     = exp(S - m_new)
      l_new = exp(m_old - m_new) * l_old + rowsum P
      O     = (exp(m_old - m_new) * l_old / l_new) * O + (P V_blk) / l_new
    The page prints the last line without the exp(m_old - m_new) factor;
    ``literal_page_rule=True`` runs that printed form instead.  When
    m_new = -inf (no visible key yet) the reference 0 is used so that
    exp(-inf - (-inf)) never occurs.

    Returns (O, LSE) with LSE = m + ln l.
    """
    q = _f64(q)
    k = _f64(k)
    v = _f64(v)
    n_q = q.shape[-2]
    n_k = k.shape[-2]
    lead = q.shape[:-2]
    m = np.full(lead + (n_q, 1), -np.inf)
    l = np.zeros(lead + (n_q, 1))
    o = np.zeros(lead + (n_q, v.shape[-1]))
    vis = causal_visible(n_q, n_k) if causal else None
    for start in range(0, n_k, block_k):
        kb = k[..., start : start + block_k, :]
        vb = v[..., start : start + block_k, :]
        s = float(scale) * np.matmul(q, np.swapaxes(kb, -1, -2))
        if causal:
            s = np.where(vis[:, start : start + kb.shape[-2]], s, -np.inf)
        m_new = np.maximum(m, np.max(s, axis=-1, keepdims=True))
        ref = np.where(np.isneginf(m_new), 0.0, m_new)
        p = np.exp(s - ref)
        alpha = np.exp(m - ref)
        l_new = alpha * l + np.sum(p, axis=-1, keepdims=True)
        safe = np.where(l_new == 0.0, 1.0, l_new)
        pv = np.matmul(p, vb)
        if literal_page_rule:
            o = (l / safe) * o + pv / safe
        else:
            o = (alpha * l / safe) * o + pv / safe
        m, l = m_new, l_new
    lse = (m + np.log(l))[..., 0]
    return o, lse


# --------------------------------------------------------------------------
# Pure-Python brute force, for tiny shapes only.  Independent of numpy's BLAS
# and reductions: each score, exponential and sum is an explicit loop with
# math.exp and math.fsum (correctly rounded summation).
# --------------------------------------------------------------------------

def attention_fwd_bruteforce(q, k, v, scale: float, causal: bool = False):
    """O and LSE for one (n_q, d) / (n_k, d) head with explicit loops."""
    q = [[float(x) for x in row] for row in np.asarray(q)]
    k = [[float(x) for x in row] for row in np.asarray(k)]
    v = [[float(x) for x in row] for row in np.asarray(v)]
    n_q, n_k, d = len(q), len(k), len(q[0])
    out = [[0.0] * d for _ in range(n_q)]
    lse = [0.0] * n_q
    for i in range(n_q):
        keys = [j for j in range(n_k) if (not causal or j <= i)]
        s = [scale * math.fsum(q[i][t] * k[j][t] for t in range(d)) for j in keys]
        mx = max(s)
        e = [math.exp(x - mx) for x in s]
        tot = math.fsum(e)
        for c in range(d):
            out[i][c] = math.fsum(e[a] * v[j][c] for a, j in enumerate(keys)) / tot
        lse[i] = mx + math.log(tot)
    return np.array(out), np.array(lse)


def attention_bwd_bruteforce(q, k, v, do, scale: float, causal: bool = False):
    """dQ, dK, dV for one head by differentiating element by element.

    Written from the scalar chain rule rather than matrix identities:
    O_ic = sum_j P_ij V_jc, P_ij = exp(S_ij) / sum_t exp(S_it),
    S_ij = scale * sum_c Q_ic K_jc, and L = sum_ic dO_ic O_ic, so
    dL/dP_ij = sum_c dO_ic V_jc, dL/dS_ij = P_ij (dL/dP_ij - sum_t P_it dL/dP_it).
    """
    qf = [[float(x) for x in row] for row in np.asarray(q)]
    kf = [[float(x) for x in row] for row in np.asarray(k)]
    vf = [[float(x) for x in row] for row in np.asarray(v)]
    dof = [[float(x) for x in row] for row in np.asarray(do)]
    n_q, n_k, d = len(qf), len(kf), len(qf[0])
    p = [[0.0] * n_k for _ in range(n_q)]
    for i in range(n_q):
        keys = [j for j in range(n_k) if (not causal or j <= i)]
        s = {j: scale * math.fsum(qf[i][t] * kf[j][t] for t in range(d)) for j in keys}
        mx = max(s.values())
        tot = math.fsum(math.exp(x - mx) for x in s.values())
        for j in keys:
            p[i][j] = math.exp(s[j] - mx) / tot
    dq = [[0.0] * d for _ in range(n_q)]
    dk = [[0.0] * d for _ in range(n_k)]
    dv = [[0.0] * d for _ in range(n_k)]
    for i in range(n_q):
        gp = [math.fsum(dof[i][c] * vf[j][c] for c in range(d)) for j in range(n_k)]
        expect = math.fsum(p[i][t] * gp[t] for t in range(n_k))
        gs = [p[i][j] * (gp[j] - expect) for j in range(n_k)]
        for j in range(n_k):
            for c in range(d):
                dv[j][c] += p[i][j] * dof[i][c]
                dq[i][c] += scale * gs[j] * kf[j][c]
                dk[j][c] += scale * gs[j] * qf[i][c]
    return np.array(dq), np.array(dk), np.array(dv)


# --------------------------------------------------------------------------
# Closed forms
# --------------------------------------------------------------------------

def score_bytes(batch: int, heads: int, seq_len: int, elem_bytes: int) -> int:
    """Bytes of a materialised score matrix: batch * heads * seq_len^2 * elem_bytes.

    The formula of "Calculateur de memoire d'attention", section "La formule".
    """
    return int(batch) * int(heads) * int(seq_len) ** 2 * int(elem_bytes)


def attention_flops(batch: int, heads: int, n_q: int, n_k: int, d: int, causal: bool,
                    backward: bool = False) -> int:
    """Algorithmic FLOP count of the path.

    Each visible (query, key) pair costs 2*d for its score and 2*d for its
    share of P V in the forward pass; the backward pass performs five such
    products per visible pair (S recomputed, dV, dP, dQ, dK), 10*d in all.
    With the top-left causal mask, query i sees min(i + 1, n_k) keys.
    """
    if causal:
        i = np.arange(n_q, dtype=np.int64)
        pairs = int(np.sum(np.minimum(i + 1, n_k)))
    else:
        pairs = int(n_q) * int(n_k)
    per_pair = 10 * d if backward else 4 * d
    return int(batch) * int(heads) * pairs * per_pair


# ------------------------------------------------------ grouped K/V heads


def expand_kv_heads(x, n_heads: int) -> np.ndarray:
    """K or V of shape (..., H_kv, n, d) repeated to (..., H, n, d).

    "Attention Mechanism", section 12 "GQA vs MQA -- KV Cache Optimization":
    the H query heads fall into H_kv consecutive groups of H / H_kv, and every
    head of group j uses K/V head j; the page computes this by repeating each
    K/V head H / H_kv times along the head axis (H_kv = H is ordinary
    multi-head attention, H_kv = 1 is multi-query attention).
    """
    x = _f64(x)
    h_kv = x.shape[-3]
    if h_kv < 1 or n_heads % h_kv != 0:
        raise ValueError(f"{h_kv} K/V heads do not divide {n_heads} query heads")
    return np.repeat(x, n_heads // h_kv, axis=-3)


def attention_fwd_gqa(q, k, v, scale: float, causal: bool = False):
    """Forward pass with shared K/V heads: q (..., H, n_q, d), k and v
    (..., H_kv, n_k, d).  Defined as attention_fwd on the repeated K/V."""
    h = np.shape(q)[-3]
    return attention_fwd(q, expand_kv_heads(k, h), expand_kv_heads(v, h), scale, causal)


def attention_bwd_gqa(q, k, v, do, scale: float, causal: bool = False):
    """Backward pass of attention_fwd_gqa: (dQ, dK, dV) with dK, dV shaped
    like k.  The repetition is linear, so the gradient of a shared K/V head is
    the sum of the gradients of its copies, i.e. over the query heads of its
    group."""
    h = np.shape(q)[-3]
    h_kv = np.shape(k)[-3]
    dq, dk, dv = attention_bwd(q, expand_kv_heads(k, h), expand_kv_heads(v, h), do, scale, causal)
    g = h // h_kv

    def fold(x):
        return x.reshape(x.shape[:-3] + (h_kv, g) + x.shape[-2:]).sum(axis=-3)

    return dq, fold(dk), fold(dv)


# ------------------------------------------- query offset and sliding window


def band_visible(n_q: int, n_k: int, causal: bool, q_offset: int = 0, window: int = -1) -> np.ndarray:
    """Boolean (n_q, n_k): True where key j is visible to query row i.

    Row i sits at absolute position p = i + q_offset on the key axis.  The
    causal mask ("Attention Mechanism", section 4.4) hides j > p -- with
    q_offset = 0 this is causal_visible's top-left alignment, and
    q_offset = n_k - n_q puts the last query on the last key.  A sliding
    window of half-width w >= 0 (same page, section 4.5 "Sparse Attention":
    each query sees only its +-w neighbours) hides |p - j| > w; w < 0 means no
    window.
    """
    p = np.arange(n_q)[:, None] + int(q_offset)
    j = np.arange(n_k)[None, :]
    vis = np.ones((n_q, n_k), dtype=bool)
    if causal:
        vis &= j <= p
    if window >= 0:
        vis &= np.abs(p - j) <= window
    return vis


def _band_probs(q, k, scale, causal, q_offset, window):
    """P (rows summing to one, or all zero for a row that sees no key) and
    LSE (-inf for such a row) under band_visible."""
    q = _f64(q)
    k = _f64(k)
    vis = band_visible(q.shape[-2], k.shape[-2], causal, q_offset, window)
    s = float(scale) * np.matmul(q, np.swapaxes(k, -1, -2))
    s = np.where(vis, s, -np.inf)
    m = np.max(s, axis=-1, keepdims=True, initial=-np.inf)  # no keys at all: -inf
    empty = ~np.isfinite(m)
    m = np.where(empty, 0.0, m)
    e = np.where(vis, np.exp(s - m), 0.0)
    l = np.sum(e, axis=-1, keepdims=True)
    p = np.where(empty, 0.0, e / np.where(empty, 1.0, l))
    with np.errstate(divide="ignore"):
        lse = np.where(empty, -np.inf, m + np.log(np.where(empty, 1.0, l)))[..., 0]
    return p, lse


def attention_fwd_band(q, k, v, scale: float, causal: bool = False, q_offset: int = 0,
                       window: int = -1):
    """Forward pass under band_visible, with K/V heads shared when k has fewer
    heads than q (as attention_fwd_gqa).  A row that sees no key has O = 0 and
    LSE = -inf."""
    h = np.shape(q)[-3] if np.ndim(q) >= 3 else None
    if h is not None and np.shape(k)[-3] != h:
        k, v = expand_kv_heads(k, h), expand_kv_heads(v, h)
    p, lse = _band_probs(q, k, scale, causal, q_offset, window)
    return np.matmul(p, _f64(v)), lse


def attention_bwd_band(q, k, v, do, scale: float, causal: bool = False, q_offset: int = 0,
                       window: int = -1):
    """Explicit backward pass of attention_fwd_band (the chain rule of
    attention_bwd on the banded P; a row that sees no key contributes
    nothing); dK, dV are summed over the query heads sharing a K/V head."""
    q, do = _f64(q), _f64(do)
    h = q.shape[-3] if q.ndim >= 3 else None
    h_kv = np.shape(k)[-3] if h is not None else None
    if h is not None and h_kv != h:
        k, v = expand_kv_heads(k, h), expand_kv_heads(v, h)
    k, v = _f64(k), _f64(v)
    p, _ = _band_probs(q, k, scale, causal, q_offset, window)
    o = np.matmul(p, v)
    dv = np.matmul(np.swapaxes(p, -1, -2), do)
    dp = np.matmul(do, np.swapaxes(v, -1, -2))
    ds = p * (dp - np.sum(do * o, axis=-1, keepdims=True))
    dq = float(scale) * np.matmul(ds, k)
    dk = float(scale) * np.matmul(np.swapaxes(ds, -1, -2), q)
    if h is not None and h_kv != h:
        g = h // h_kv

        def fold(x):
            return x.reshape(x.shape[:-3] + (h_kv, g) + x.shape[-2:]).sum(axis=-3)

        dk, dv = fold(dk), fold(dv)
    return dq, dk, dv


# ------------------------------------------------ merging key-split results


def lse_merge(o_parts, lse_parts):
    """Combine attention results over disjoint key sets into the result over
    their union.

    Part p holds O_p (softmax over its own keys, times their values) and
    LSE_p = ln sum_{j in part p} exp(S_ij).  Over the union the softmax
    denominator is sum_p exp(LSE_p), so

        LSE = ln sum_p exp(LSE_p),    O = sum_p exp(LSE_p - LSE) O_p.

    This is the online softmax's rescaling by exp(m_old - m_new) ("Attention
    Mechanism", section 13 "FlashAttention -- How It Works") applied to whole
    parts; it is what lets the key axis be split across workers (same page,
    section 16, "Ring Attention") or a long KV cache be split for decoding
    (same page, section 8, "Key-Value (KV) Cache").  A part with LSE = -inf
    (no visible key) contributes nothing; a row with no visible key in any
    part gets O = 0 and LSE = -inf.

    o_parts (P, ..., n, d), lse_parts (P, ..., n).
    """
    o = _f64(o_parts)
    lse = _f64(lse_parts)
    if o.shape[:-1] != lse.shape:
        raise ValueError(f"O parts {o.shape} do not match LSE parts {lse.shape}")
    m = np.max(lse, axis=0)
    empty = ~np.isfinite(m)
    ref = np.where(empty, 0.0, m)
    w = np.exp(lse - ref)                     # exp(-inf) = 0 for empty parts
    total = np.sum(w, axis=0)
    safe = np.where(empty, 1.0, total)
    out = np.sum(w[..., None] * o, axis=0) / safe[..., None]
    with np.errstate(divide="ignore"):
        out_lse = np.where(empty, -np.inf, ref + np.log(safe))
    return np.where(empty[..., None], 0.0, out), out_lse

