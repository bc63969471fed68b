"""Property tests of the oracle (CPU, hypothesis, derandomised): invariants that
hold for every input, checked on many random ones.

- The Quest bound is an upper bound: every token's q.k is at most its block's
  score (Pith review, "Assumptions & free parameters": the min/max premise).
  In float64 this holds exactly: each channel's term dominates the token's
  product, rounding is monotone, and both sums run in the same order.
- Selection is a valid top-n: the n_local newest blocks, then the highest
  scores with ties to the lower index, n in all, sorted ("What carries the
  argument").
- The count rule n = min(M, max(n_min, ceil(M r))) is bounded and monotone in M
  (referee report, major comment 1, Eq. 5).
- Pooling by the mean or by the sum ranks blocks the same (the bound is
  positively homogeneous in q; G a power of two keeps the scaling exact).
- Attention over a union of token sets equals the log-sum-exp merge of the
  attention over its parts (the identity a split decode relies on).
"""
import math

import numpy as np
from hypothesis import given, settings, strategies as st

from oracle import resa_oracle as O

SETTINGS = settings(max_examples=60, deadline=None, derandomize=True)


@SETTINGS
@given(seed=st.integers(0, 2**31 - 1), L=st.integers(1, 90), d=st.integers(1, 9),
       scale_q=st.sampled_from([1e-3, 1.0, 1e3]))
def test_bound_is_at_least_every_tokens_product(seed, L, d, scale_q):
    rng = np.random.default_rng(seed)
    K = rng.standard_normal((L, d)) * rng.choice([0.5, 1.0, 4.0], size=d)
    q = rng.standard_normal(d) * scale_q
    kmin, kmax = O.block_descriptors(K)
    s = O.block_upper_bounds(q, kmin, kmax)
    for t in range(L):
        assert float((q[None, :] * K[t][None, :]).sum(axis=1)[0]) <= s[t // O.BLOCK]


@SETTINGS
@given(seed=st.integers(0, 2**31 - 1), M=st.integers(1, 70), levels=st.integers(1, 6),
       n=st.integers(1, 80), n_local=st.integers(0, 3))
def test_selection_is_a_valid_top_n(seed, M, levels, n, n_local):
    rng = np.random.default_rng(seed)
    scores = rng.integers(0, levels, size=M).astype(np.float64)  # few levels: many exact ties
    sel = O.select_blocks(scores, n, n_local)
    n_eff = min(n, M)
    keep = min(n_local, n_eff)
    assert len(sel) == n_eff and len(set(sel.tolist())) == n_eff
    assert list(sel) == sorted(sel)
    chosen = set(sel.tolist())
    assert set(range(M - keep, M)) <= chosen
    cand_in = [j for j in chosen if j < M - keep]
    cand_out = [j for j in range(M - keep) if j not in chosen]
    for c in cand_in:
        for u in cand_out:
            assert scores[c] > scores[u] or (scores[c] == scores[u] and c < u)


@SETTINGS
@given(M=st.integers(1, 5000), n_min=st.integers(1, 64), r=st.floats(0.001, 1.0))
def test_count_rule_is_bounded_and_monotone(M, n_min, r):
    n = O.active_block_count(M, n_min, r)
    assert 1 <= n <= M
    assert n >= min(M, n_min) and n >= min(M, math.ceil(M * r))
    assert O.active_block_count(M + 1, n_min, r) >= n


@SETTINGS
@given(seed=st.integers(0, 2**31 - 1), G=st.sampled_from([1, 2, 4, 8]), L=st.integers(1, 200),
       d=st.integers(1, 8), n=st.integers(1, 16), n_local=st.integers(0, 2))
def test_mean_and_sum_pooling_select_the_same_blocks(seed, G, L, d, n, n_local):
    rng = np.random.default_rng(seed)
    qg = rng.standard_normal((G, d))
    kmin, kmax = O.block_descriptors(rng.standard_normal((L, d)))
    mean_sel = O.select_blocks(O.block_upper_bounds(O.pooled_query(qg), kmin, kmax), n, n_local)
    qsum = np.array(qg[0])
    for h in range(1, G):
        qsum = qsum + qg[h]
    sum_sel = O.select_blocks(O.block_upper_bounds(qsum, kmin, kmax), n, n_local)
    assert np.array_equal(mean_sel, sum_sel)


@SETTINGS
@given(seed=st.integers(0, 2**31 - 1), T=st.integers(2, 60), d=st.integers(1, 8), R=st.integers(1, 4),
       cut=st.floats(0.05, 0.95), spread=st.sampled_from([0.1, 1.0, 10.0]))
def test_attention_over_a_union_is_the_lse_merge_of_its_parts(seed, T, d, R, cut, spread):
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((R, d)) * spread
    k = rng.standard_normal((T, d))
    v = rng.standard_normal((T, d))
    scale = 1.0 / math.sqrt(d)
    perm = rng.permutation(T)
    a, b = np.sort(perm[:max(1, int(cut * T))]), np.sort(perm[max(1, int(cut * T)):])
    if len(b) == 0:
        return
    whole = O.attention(q, k, v, scale)
    parts = []
    for idx in (a, b):
        logits = (q @ k[idx].T) * scale
        m = logits.max(axis=1)
        l = np.exp(logits - m[:, None]).sum(axis=1)
        parts.append((m, l, O.attention(q, k[idx], v[idx], scale)))
    (m1, l1, o1), (m2, l2, o2) = parts
    m = np.maximum(m1, m2)
    w1, w2 = l1 * np.exp(m1 - m), l2 * np.exp(m2 - m)
    merged = (w1[:, None] * o1 + w2[:, None] * o2) / (w1 + w2)[:, None]
    assert np.allclose(merged, whole, rtol=1e-12, atol=1e-12)
