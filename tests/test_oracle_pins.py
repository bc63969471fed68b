"""Pins of the CPU oracle to things other than itself (CPU only).

Each test fixes one part of the oracle against brute force, a closed form, a
library routine in a special case, an invariant the pages state, or a value the
pages print. Each is chosen so that a plausible slip in the oracle (a dropped
term, a wrong sign, an off-by-one in a block or causal bound, a transposed
operand, a wrong scale) fails at least one of them.
"""
import json
import math
import os
from fractions import Fraction

import numpy as np
import pytest
import torch
import torch.nn.functional as F

from oracle import resa_oracle as O
from block_sparse_attention_quest_amd import workloads as W

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _golden(name):
    with open(os.path.join(GOLDEN, name)) as fh:
        return json.load(fh)


def _sdpa(q, k, v, mask=None):
    """torch SDPA in float64 on the CPU: q [H][R][d], k, v [H][T][d]."""
    q = torch.from_numpy(np.ascontiguousarray(q))
    k = torch.from_numpy(np.ascontiguousarray(k))
    v = torch.from_numpy(np.ascontiguousarray(v))
    m = None if mask is None else torch.from_numpy(np.ascontiguousarray(mask))
    return F.scaled_dot_product_attention(q, k, v, attn_mask=m).numpy()


def _random_cache(rng, B, Hkv, d, lens, extra_blocks=2, pad_value=None):
    maxb = max(O.num_blocks(L) for L in lens) + extra_blocks
    P = B * maxb
    k = rng.standard_normal((P, Hkv, 16, d))
    v = rng.standard_normal((P, Hkv, 16, d))
    if pad_value is not None:
        k[:] = pad_value
        v[:] = pad_value
    bt = rng.permutation(P).reshape(B, maxb)
    # fill valid tokens only
    for b, L in enumerate(lens):
        for t in range(L):
            page = bt[b, t // 16]
            k[page, :, t % 16] = rng.standard_normal((Hkv, d))
            v[page, :, t % 16] = rng.standard_normal((Hkv, d))
    desc = np.full((P, Hkv, 2, d), np.nan)
    cache = O.PagedCache(k, v, desc, bt, lens)
    cache.rebuild()
    return cache


# --- descriptors ------------------------------------------------------------

def test_descriptors_match_bruteforce_loops():
    rng = np.random.default_rng(0)
    k = rng.standard_normal((37, 5))          # 3 blocks, the last holds 5 tokens
    kmin, kmax = O.block_descriptors(k)
    assert kmin.shape == (3, 5)
    for j in range(3):
        for c in range(5):
            lo, hi = math.inf, -math.inf
            for t in range(j * 16, min(37, j * 16 + 16)):
                x = float(k[t, c])
                lo = x if x < lo else lo
                hi = x if x > hi else hi
            assert kmin[j, c] == lo and kmax[j, c] == hi


def test_partial_block_never_reads_padding():
    rng = np.random.default_rng(1)
    cache = _random_cache(rng, 2, 2, 8, [21, 50], pad_value=1e9)
    for b, L in enumerate([21, 50]):
        for j in range(O.num_blocks(L)):
            page = cache.block_table[b, j]
            assert np.all(cache.desc[page, :, 1] < 1e8)
            assert np.all(cache.desc[page, :, 0] > -1e8)


def test_bound_dominates_every_dot_product():
    """Quest premise ('Assumptions & free parameters': block min/max descriptors):
    the block score bounds q.k from above for every key of the block."""
    rng = np.random.default_rng(2)
    d = 16
    k = rng.standard_normal((16 * 9 + 7, d))
    kmin, kmax = O.block_descriptors(k)
    naive_fails = False
    for trial in range(50):
        q = rng.standard_normal(d)
        s = O.block_upper_bounds(q, kmin, kmax)
        for j in range(len(s)):
            tile = k[j * 16:(j + 1) * 16]
            best = max(float(np.dot(q, row)) for row in tile)
            assert s[j] >= best - 1e-12 * (1 + abs(best))
            # a bound built from kmax alone (a plausible slip) is not an upper bound
            if float(np.dot(q, kmax[j])) < best - 1e-9:
                naive_fails = True
    assert naive_fails


def test_single_token_block_bound_is_exact_dot():
    rng = np.random.default_rng(3)
    d = 32
    # dyadic values: every product and partial sum is exact in float64
    k = rng.integers(-64, 64, (16 * 2 + 1, d)) / 8.0
    q = rng.integers(-64, 64, d) / 16.0
    kmin, kmax = O.block_descriptors(k)
    s = O.block_upper_bounds(q, kmin, kmax)
    exact = sum(Fraction(float(a)) * Fraction(float(b)) for a, b in zip(q, k[-1]))
    assert s[-1] == float(exact)
    # a block of identical keys also gives the exact dot product
    kk = np.repeat(k[:1], 16, axis=0)
    mn, mx = O.block_descriptors(kk)
    assert O.block_upper_bounds(q, mn, mx)[0] == float(sum(Fraction(float(a)) * Fraction(float(b))
                                                           for a, b in zip(q, k[0])))


def test_append_updates_only_its_block():
    rng = np.random.default_rng(4)
    cache = _random_cache(rng, 1, 2, 8, [40])
    before = cache.desc.copy()
    kn = rng.standard_normal((1, 2, 8)) * 5
    vn = rng.standard_normal((1, 2, 8))
    O.append(cache, kn, vn)
    assert cache.seq_lens == [41]
    page = cache.block_table[0, 2]
    toks = np.stack([cache.k[page, :, t] for t in range(41 - 32)], axis=1)  # [Hkv][9][d]
    assert np.array_equal(cache.desc[page, :, 0], toks.min(axis=1))
    assert np.array_equal(cache.desc[page, :, 1], toks.max(axis=1))
    for j in (0, 1):
        p = cache.block_table[0, j]
        assert np.array_equal(cache.desc[p], before[p])


# --- count rule (Eq. 5) ------------------------------------------------------

def test_count_matches_worked_values():
    g = _golden("eq5_counts.json")
    for c in g["cases"]:
        assert O.active_block_count(c["M"], c["n_min"], c["r"]) == c["n"], c


@pytest.mark.parametrize("r_text", ["0.05", "0.1", "0.125", "0.3"])
def test_count_equals_exact_rational_ceiling(r_text):
    """IEEE ceil(M * r) agrees with the exact ceiling of M times the decimal r."""
    fr = Fraction(r_text)
    for n_min in (4, 16):
        for M in range(1, 20000):
            num = M * fr.numerator
            exact = -(-num // fr.denominator)
            assert O.active_block_count(M, n_min, float(r_text)) == min(M, max(n_min, exact))


def test_defaults_match_pages():
    g = _golden("defaults.json")
    for key in ("block_size", "f", "n_min", "n_local", "p"):
        assert O.DEFAULTS[key] == g[key]
    assert O.BLOCK == g["block_size"]


def test_memory_fraction_matches_printed_value():
    for c in _golden("eq6_memory_fraction.json")["cases"]:
        assert abs(O.memory_fraction(c["b"], c["active"], c["f"]) - c["value"]) <= c["abs_tol"]


# --- selection ----------------------------------------------------------------

def _rank_selection(scores, n, n_local):
    """Selection by its definition: the newest min(n_local, n) blocks, plus each
    other block whose count of strictly better other blocks (higher score, or
    equal score and lower index) is below the remaining quota."""
    M = len(scores)
    n = min(n, M)
    loc = set(range(M - min(n_local, n), M))
    quota = n - len(loc)
    sel = set(loc)
    for j in range(M):
        if j in loc:
            continue
        better = sum(1 for i in range(M) if i not in loc and
                     (scores[i] > scores[j] or (scores[i] == scores[j] and i < j)))
        if better < quota:
            sel.add(j)
    return sorted(sel)


def test_selection_matches_rank_definition_with_ties():
    rng = np.random.default_rng(5)
    for trial in range(200):
        M = int(rng.integers(1, 40))
        scores = rng.integers(0, 6, M).astype(np.float64)   # many exact ties
        n = int(rng.integers(1, M + 3))
        n_local = int(rng.integers(0, 3))
        got = O.select_blocks(scores, n, n_local).tolist()
        assert got == _rank_selection(scores, n, n_local), (scores, n, n_local)


def test_selection_threshold_invariant():
    rng = np.random.default_rng(6)
    for trial in range(100):
        M = int(rng.integers(2, 300))
        s = rng.standard_normal(M)
        n = int(rng.integers(1, M + 1))
        sel = set(O.select_blocks(s, n, 1).tolist())
        assert len(sel) == n and (M - 1) in sel
        others = [j for j in sel if j != M - 1]
        if others:
            lo = min(s[j] for j in others)
            assert all(s[j] <= lo for j in range(M - 1) if j not in sel)


def test_newest_block_kept_even_when_it_scores_lowest():
    s = np.array([5.0, 4.0, 3.0, 2.0, -100.0])
    assert O.select_blocks(s, 2, 1).tolist() == [0, 4]
    assert O.select_blocks(s, 2, 0).tolist() == [0, 1]
    assert O.select_blocks(s, 9, 1).tolist() == [0, 1, 2, 3, 4]


def test_pooling_is_the_group_mean():
    q = np.array([[1.0, -2.0], [3.0, 0.5], [-1.0, 4.0], [5.0, 1.5]])
    assert np.array_equal(O.pooled_query(q), np.array([2.0, 1.0]))


def test_planted_blocks_are_selected_at_the_first_step():
    """Keys planted along the group's pooled query direction outrank random
    blocks; this fixes the sign of the bound and the pooling."""
    w = W.tiny_fp32()
    cache = _workload_cache(w)
    q, k, v = (x.double().numpy() for x in (W.query(w, 0),) + W.append_kv(w, 0))
    O.append(cache, k, v)
    idx, counts, _ = O.select(cache, q, w.n_min, w.r, w.n_local)
    assert counts == [9]
    assert set(W.planted_blocks(w, 0)) <= set(idx[0][0].tolist())


def _workload_cache(w):
    bt = W.block_table(w).numpy()
    P, Hkv, d = w.num_pages, w.num_kv_heads, w.head_dim
    kp = np.zeros((P, Hkv, 16, d))
    vp = np.zeros((P, Hkv, 16, d))
    for b in range(w.batch):
        for h in range(Hkv):
            kk, vv = W.prefill_kv(w, b, h)
            L = w.prefill_lens[b]
            for t in range(L):
                kp[bt[b, t // 16], h, t % 16] = kk[t].double().numpy()
                vp[bt[b, t // 16], h, t % 16] = vv[t].double().numpy()
    cache = O.PagedCache(kp, vp, np.zeros((P, Hkv, 2, d)), bt, list(w.prefill_lens))
    cache.rebuild()
    return cache


# --- attention ----------------------------------------------------------------

def test_all_blocks_selected_equals_dense_sdpa():
    """n = M turns GBSA into dense attention (GQA heads sharing KV)."""
    rng = np.random.default_rng(7)
    B, Hq, Hkv, d = 2, 8, 2, 16
    cache = _random_cache(rng, B, Hkv, d, [50, 77])
    q = rng.standard_normal((B, Hq, d))
    idx, counts, _ = O.select(cache, q, n_min=100, r=0.1, n_local=1)
    out = O.decode(cache, q, idx, 1 / math.sqrt(d))
    G = Hq // Hkv
    for b in range(B):
        k = np.stack([cache.seq(b, h // G, "k") for h in range(Hq)])
        v = np.stack([cache.seq(b, h // G, "v") for h in range(Hq)])
        ref = _sdpa(q[b][:, None, :], k, v)[:, 0]
        np.testing.assert_allclose(out[b], ref, rtol=1e-12, atol=1e-12)


def test_block_mask_equals_masked_sdpa():
    """Eq. 2: key k is attended iff its block floor(k/16) is selected."""
    rng = np.random.default_rng(8)
    d, L = 16, 16 * 6 + 3
    k = rng.standard_normal((L, d))
    v = rng.standard_normal((L, d))
    q = rng.standard_normal((4, d))
    blocks = [0, 2, 6]
    out = O.sparse_decode_group(q, k, v, blocks, 1 / math.sqrt(d))
    mask = np.array([(t // 16) in blocks for t in range(L)])[None, None, :].repeat(4, 0)
    ref = _sdpa(q[:, None, :], np.repeat(k[None], 4, 0), np.repeat(v[None], 4, 0), mask)[:, 0]
    np.testing.assert_allclose(out, ref, rtol=1e-12, atol=1e-12)


def test_sparse_decode_matches_python_loops():
    rng = np.random.default_rng(9)
    d, L = 4, 40
    k = rng.standard_normal((L, d))
    v = rng.standard_normal((L, d))
    q = rng.standard_normal((2, d)) * 3
    blocks = [1, 2]
    out = O.sparse_decode_group(q, k, v, blocks, 0.5)
    for h in range(2):
        toks = [t for t in range(L) if t // 16 in blocks]
        logits = [0.5 * sum(q[h, c] * k[t, c] for c in range(d)) for t in toks]
        mx = max(logits)
        ws = [math.exp(x - mx) for x in logits]
        for c in range(d):
            ref = sum(wt * v[t, c] for wt, t in zip(ws, toks)) / sum(ws)
            assert abs(out[h, c] - ref) < 1e-12


def test_large_logits_stay_finite():
    rng = np.random.default_rng(10)
    k = rng.standard_normal((33, 8))
    v = rng.standard_normal((33, 8))
    q = rng.standard_normal((4, 8)) * 1e3
    out = O.sparse_decode_group(q, k, v, [0, 1, 2], 1.0)
    assert np.all(np.isfinite(out))
    ref = _sdpa(q[:, None, :] * math.sqrt(8), np.repeat(k[None], 4, 0), np.repeat(v[None], 4, 0))[:, 0]
    np.testing.assert_allclose(out, ref, rtol=1e-9, atol=1e-9)


# --- rectification -----------------------------------------------------------

def test_rectify_equals_causal_sdpa_and_rebuilds_cache():
    rng = np.random.default_rng(11)
    B, Hq, Hkv, d, f = 2, 4, 2, 8, 5
    lens = [45, 64]
    cache = _random_cache(rng, B, Hkv, d, lens)
    q = rng.standard_normal((B, f, Hq, d))
    kn = rng.standard_normal((B, f, Hkv, d))
    vn = rng.standard_normal((B, f, Hkv, d))
    out = O.rectify(cache, q, kn, vn, 1 / math.sqrt(d))
    G = Hq // Hkv
    for b, L in enumerate(lens):
        # cache rows [L-f, L) are exactly the inputs
        for i in range(f):
            pos = L - f + i
            page = cache.block_table[b, pos // 16]
            assert np.array_equal(cache.k[page, :, pos % 16], kn[b, i])
            assert np.array_equal(cache.v[page, :, pos % 16], vn[b, i])
        # descriptors equal a from-scratch build
        for h in range(Hkv):
            mn, mx = O.block_descriptors(cache.seq(b, h, "k"))
            for j in range(O.num_blocks(L)):
                page = cache.block_table[b, j]
                assert np.array_equal(cache.desc[page, h, 0], mn[j])
                assert np.array_equal(cache.desc[page, h, 1], mx[j])
        # outputs are causal dense attention over the updated cache
        mask = np.array([[t <= L - f + i for t in range(L)] for i in range(f)])
        for h in range(Hq):
            ref = _sdpa(q[b, :, h][None], cache.seq(b, h // G, "k")[None], cache.seq(b, h // G, "v")[None],
                        mask[None])[0]
            np.testing.assert_allclose(out[b, :, h], ref, rtol=1e-12, atol=1e-12)


def test_rectified_row_equals_dense_decode_at_its_position():
    rng = np.random.default_rng(12)
    d, L, f = 8, 70, 6
    cache = _random_cache(rng, 1, 1, d, [L])
    q = rng.standard_normal((1, f, 4, d))
    kn = rng.standard_normal((1, f, 1, d))
    vn = rng.standard_normal((1, f, 1, d))
    out = O.rectify(cache, q, kn, vn, 0.3)
    for i in range(f):
        P = L - f + i
        k = cache.seq(0, 0, "k")[:P + 1]
        v = cache.seq(0, 0, "v")[:P + 1]
        dense = O.sparse_decode_group(q[0, i], k, v, range(O.num_blocks(P + 1)), 0.3)
        np.testing.assert_allclose(out[0, i], dense, rtol=1e-12, atol=1e-12)


# --- the schedule ---------------------------------------------------------------

def test_loop_with_every_block_is_dense_decoding():
    rng = np.random.default_rng(13)
    B, Hq, Hkv, d, steps, f = 1, 4, 1, 8, 12, 4
    cache = _random_cache(rng, B, Hkv, d, [30], extra_blocks=3)
    qs = rng.standard_normal((steps, B, Hq, d))
    ks = rng.standard_normal((steps, B, Hkv, d))
    vs = rng.standard_normal((steps, B, Hkv, d))
    rect = {t: (rng.standard_normal((B, f, Hq, d)), rng.standard_normal((B, f, Hkv, d)),
                rng.standard_normal((B, f, Hkv, d))) for t in range(steps)}
    seen = []

    def check(t, c, o, idx):
        ref = _sdpa(qs[t][0][:, None, :], np.repeat(c.seq(0, 0, "k")[None], Hq, 0),
                    np.repeat(c.seq(0, 0, "v")[None], Hq, 0))[:, 0]
        np.testing.assert_allclose(o[0], ref, rtol=1e-12, atol=1e-12)
        seen.append(t)

    res = O.resa_loop(cache, steps, f, n_min=1000, r=0.1, n_local=1, scale=1 / math.sqrt(d),
                      step_inputs=lambda t: (qs[t], ks[t], vs[t]), rectify_inputs=lambda t: rect[t],
                      on_step=check)
    assert seen == list(range(steps))
    assert len(res["rectify_out"]) == steps // f
    assert cache.seq_lens == [30 + steps]


def test_loop_without_rectification_keeps_sparse_phase_kv():
    """f <= 0 is plain sparse decoding: the appended rows stay as written."""
    rng = np.random.default_rng(14)
    cache = _random_cache(rng, 1, 1, 8, [40], extra_blocks=2)
    ks = rng.standard_normal((8, 1, 1, 8))
    vs = rng.standard_normal((8, 1, 1, 8))
    qs = rng.standard_normal((8, 1, 4, 8))
    res = O.resa_loop(cache, 8, 0, 4, 0.1, 1, 0.35, step_inputs=lambda t: (qs[t], ks[t], vs[t]))
    assert res["rectify_out"] == []
    for t in range(8):
        pos = 40 + t
        assert np.array_equal(cache.k[cache.block_table[0, pos // 16], 0, pos % 16], ks[t, 0, 0])


# --- per-group wiring of the batched calls ------------------------------------

def _brute_desc(K):
    """Per-block channel min/max of K [L][d] by explicit loops."""
    L, d = K.shape
    out = []
    for j in range(-(-L // 16)):
        lo, hi = [math.inf] * d, [-math.inf] * d
        for t in range(j * 16, min(L, j * 16 + 16)):
            for c in range(d):
                x = float(K[t, c])
                lo[c] = min(lo[c], x)
                hi[c] = max(hi[c], x)
        out.append((lo, hi))
    return out


def test_batched_select_pools_each_group_over_its_own_heads_and_kv_head():
    """'What carries the argument': each GQA group pools its own G query heads
    and scores its own KV head's descriptors. Every (sequence, group) gets its
    own planted blocks, along that group's pooled query, so a slice of the
    wrong heads or the wrong KV head's descriptors picks other blocks."""
    rng = np.random.default_rng(21)
    B, Hkv, G, d = 2, 3, 2, 8
    Hq = Hkv * G
    lens = [150, 237]
    cache = _random_cache(rng, B, Hkv, d, lens)
    q = rng.standard_normal((B, Hq, d))
    n_min, r, n_local = 3, 0.1, 1
    planted = {}
    for b, L in enumerate(lens):
        M = O.num_blocks(L)
        perm = rng.permutation(M - 1)  # disjoint planted blocks per group
        for g in range(Hkv):
            qbar = q[b, g * G:(g + 1) * G].mean(axis=0)
            u = qbar / np.linalg.norm(qbar)
            blocks = sorted(perm[2 * g:2 * g + 2].tolist())
            planted[b, g] = blocks
            for j in blocks:
                cache.k[cache.block_table[b, j], g, :] += 12.0 * u
    cache.rebuild()
    idx, counts, scores = O.select(cache, q, n_min, r, n_local)
    distinct = set()
    for b, L in enumerate(lens):
        M = O.num_blocks(L)
        n = O.active_block_count(M, n_min, r)
        assert counts[b] == n == 3
        for g in range(Hkv):
            # brute force: the group's own heads, its own KV head's raw keys
            qbar = [sum(float(q[b, h, c]) for h in range(g * G, (g + 1) * G)) / G for c in range(d)]
            desc = _brute_desc(cache.seq(b, g, "k"))
            s = [sum(max(qbar[c] * lo[c], qbar[c] * hi[c]) for c in range(d)) for lo, hi in desc]
            np.testing.assert_allclose(scores[b][g], s, rtol=1e-13, atol=1e-13)
            ref = _rank_selection(np.array(s), n, n_local)
            assert idx[b][g].tolist() == ref, (b, g)
            # the planted blocks of this group, plus its newest block
            assert ref == sorted(planted[b, g] + [M - 1]), (b, g, ref, planted[b, g])
            distinct.add(tuple(ref))
    assert len(distinct) == B * Hkv  # every group's set is its own


def test_dense_decode_equals_sdpa_with_gqa_head_map():
    """The dense-decoding baseline the sparse path is compared with (Fig. 6
    caption): query head h attends to every cached token of KV head h // G."""
    rng = np.random.default_rng(22)
    B, Hkv, G, d = 2, 2, 3, 8
    Hq = Hkv * G
    lens = [41, 70]
    cache = _random_cache(rng, B, Hkv, d, lens)
    q = rng.standard_normal((B, Hq, d))
    scale = 0.37
    out = O.dense_decode(cache, q, scale)
    for b in range(B):
        k = torch.from_numpy(np.stack([cache.seq(b, g, "k") for g in range(Hkv)]))
        v = torch.from_numpy(np.stack([cache.seq(b, g, "v") for g in range(Hkv)]))
        k = k.repeat_interleave(G, dim=0).numpy()   # head h reads KV head h // G
        v = v.repeat_interleave(G, dim=0).numpy()
        ref = _sdpa(q[b][:, None, :] * (scale * math.sqrt(d)), k, v)[:, 0]
        np.testing.assert_allclose(out[b], ref, rtol=1e-12, atol=1e-12)
        # and it is the sparse decode with every block selected
        M = O.num_blocks(lens[b])
        for g in range(Hkv):
            sp = O.sparse_decode_group(q[b, g * G:(g + 1) * G], cache.seq(b, g, "k"), cache.seq(b, g, "v"),
                                       range(M), scale)
            np.testing.assert_allclose(out[b, g * G:(g + 1) * G], sp, rtol=1e-12, atol=1e-12)


def test_loop_rectifies_after_every_f_th_step_exactly():
    """'Every f decoding steps' ('What carries the argument', Fig. 2): the
    rectification follows decode steps f-1, 2f-1, ... (0-based), after that
    step's decode, and covers the f tokens those steps appended."""
    rng = np.random.default_rng(23)
    B, Hq, Hkv, d, steps, f = 1, 4, 1, 8, 14, 4
    L0 = 37
    cache = _random_cache(rng, B, Hkv, d, [L0], extra_blocks=3)
    qs = rng.standard_normal((steps, B, Hq, d))
    ks = rng.standard_normal((steps, B, Hkv, d))
    vs = rng.standard_normal((steps, B, Hkv, d))
    log = []

    def rect_inputs(t):
        log.append(("rectify", t, cache.seq_lens[0]))
        return (rng.standard_normal((B, f, Hq, d)), np.full((B, f, Hkv, d), 100.0 + t),
                np.full((B, f, Hkv, d), -100.0 - t))

    def on_step(t, c, o, idx):
        log.append(("step", t, c.seq_lens[0]))

    O.resa_loop(cache, steps, f, n_min=2, r=0.25, n_local=1, scale=0.35,
                step_inputs=lambda t: (qs[t], ks[t], vs[t]), rectify_inputs=rect_inputs, on_step=on_step)
    expect = []
    for t in range(steps):
        expect.append(("step", t, L0 + t + 1))
        if t % f == f - 1:
            expect.append(("rectify", t, L0 + t + 1))
    assert log == expect
    # the rectified rows overwrote exactly the f tokens appended since the last one
    for t in (f - 1, 2 * f - 1, 3 * f - 1):
        for pos in range(L0 + t + 1 - f, L0 + t + 1):
            assert np.all(cache.k[cache.block_table[0, pos // 16], 0, pos % 16] == 100.0 + t)
    for t in range(3 * f, steps):  # appended after the last rectification: untouched
        pos = L0 + t
        assert np.array_equal(cache.k[cache.block_table[0, pos // 16], 0, pos % 16], ks[t, 0, 0])
