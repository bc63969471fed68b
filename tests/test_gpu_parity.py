"""GPU parity: the HIP path through the C ABI against the CPU oracle, element by
element, on seeded inputs small enough for the oracle and spanning several
tiles and ragged tails.

Bars: descriptors bit-exact; selected block sets bit-exact except near-ties
(oracle score within 1e-6 relative of the threshold); attention outputs within
1e-4 absolute (fp32) and 2e-2 absolute (bf16); cache rows written by an append
or a rectification bit-exact.
"""
import math

import numpy as np
import pytest
import torch

from oracle import resa_oracle as O
from block_sparse_attention_quest_amd import workloads as W

import parity as P

pytestmark = pytest.mark.gpu


def _runner(w, steps=None, fused_append=True):
    from block_sparse_attention_quest_amd.schedule import ResaRunner
    print(f"[case] {w.name} seed={w.seed} B={w.batch} Hq={w.num_q_heads} Hkv={w.num_kv_heads} d={w.head_dim} "
          f"prefill={w.prefill_lens[:4]} steps={w.steps if steps is None else steps} f={w.f} "
          f"fused_append={fused_append}", flush=True)
    r = ResaRunner(w, steps=steps, fused_append=fused_append)
    r.fill_prefill()
    r.build_descriptors()
    return r


def _run_loop_parity(w, steps=None, check_all_desc_every=0, fused_append=True):
    steps = w.steps if steps is None else steps
    r = _runner(w, steps, fused_append)
    oc = P.oracle_cache(w)
    torch.cuda.synchronize()
    P.assert_desc_equal(r.cache.desc, oc)
    atol = P.ATOL[w.dtype]
    worst, ties = 0.0, 0
    for t in range(steps):
        q, k, v = W.query(w, t), *W.append_kv(w, t)
        O.append(oc, P.f64(k), P.f64(v))
        out = r.decode_step(t)
        torch.cuda.synchronize()
        # the appended rows and their blocks' descriptors
        for b in range(w.batch):
            pos = oc.seq_lens[b] - 1
            page = int(oc.block_table[b, pos // 16])
            assert torch.equal(r.cache.k_pages[page, :, pos % 16].cpu(), k[b]), (t, b)
            assert torch.equal(r.cache.v_pages[page, :, :, pos % 16].cpu(), v[b]), (t, b)
            P.assert_desc_equal(r.cache.desc, oc, [page])
        err, nt = P.check_select_and_decode(oc, P.f64(q), w, r.idx, r.count, out, atol)
        worst, ties = max(worst, err), ties + nt
        if w.f > 0 and (t + 1) % w.f == 0:
            rq, rk, rv = W.rectify_inputs(w, t)
            ref = O.rectify(oc, P.f64(rq), P.f64(rk), P.f64(rv), 1.0 / math.sqrt(w.head_dim))
            got = r.rectify(t, rq.cuda(), rk.cuda(), rv.cuda())
            torch.cuda.synchronize()
            rerr = P.out_error(P.f64(got), ref, w.dtype)
            assert rerr <= atol, f"rectify error {rerr} at step {t}"
            worst = max(worst, rerr)
            # rectified rows are in the cache exactly, descriptors refreshed exactly
            for b in range(w.batch):
                L = oc.seq_lens[b]
                for i in range(w.f):
                    pos = L - w.f + i
                    page = int(oc.block_table[b, pos // 16])
                    assert torch.equal(r.cache.k_pages[page, :, pos % 16].cpu(), rk[b, i])
                    assert torch.equal(r.cache.v_pages[page, :, :, pos % 16].cpu(), rv[b, i])
            P.assert_desc_equal(r.cache.desc, oc)
        if check_all_desc_every and (t + 1) % check_all_desc_every == 0:
            P.assert_desc_equal(r.cache.desc, oc)
    print(f"[result] {w.name}: max abs error {worst:.3g}, near-tie swaps {ties}", flush=True)
    return worst


def test_tiny_fp32_full_schedule():
    """1024-token fp32 case, one group of 4 heads, d 64: 64 steps, rectify at 32 and 64."""
    _run_loop_parity(W.tiny_fp32(), check_all_desc_every=16)


SMALL = [
    # name, dtype, B, Hq, Hkv, d, prefill, steps, f, n_min, r, n_local
    ("bf16_g4_d128", "bf16", 3, 8, 2, 128, (37, 300, 1000), 10, 4, 4, 0.1, 1),
    ("bf16_g4_d64", "bf16", 2, 8, 2, 64, (129, 777), 9, 3, 4, 0.2, 1),
    ("bf16_g1_d128", "bf16", 2, 2, 2, 128, (64, 500), 6, 3, 2, 0.1, 1),
    ("bf16_g2_d128", "bf16", 2, 4, 2, 128, (250, 99), 6, 6, 3, 0.15, 2),
    ("bf16_g8_d128", "bf16", 1, 16, 2, 128, (2000,), 8, 4, 16, 0.1, 1),
    ("fp32_g4_d128", "fp32", 2, 8, 2, 128, (333, 64), 8, 4, 4, 0.1, 1),
    ("bf16_dense_r1", "bf16", 2, 8, 2, 128, (100, 31), 5, 5, 1, 1.0, 1),
    ("bf16_no_local", "bf16", 2, 8, 2, 128, (600, 17), 6, 3, 4, 0.05, 0),
    ("bf16_nmin_over_M", "bf16", 2, 8, 2, 128, (40, 200), 4, 2, 64, 0.1, 1),
    ("bf16_g8_d64", "bf16", 2, 16, 2, 64, (700, 45), 6, 20, 8, 0.1, 1),   # 160 rectified rows: 256-row tiles
    ("bf16_g1_d64", "bf16", 2, 2, 2, 64, (300, 1200), 5, 5, 4, 0.1, 1),
    ("fp32_g8_d64", "fp32", 1, 16, 2, 64, (900,), 5, 5, 8, 0.1, 1),
    ("fp32_g2_d128", "fp32", 2, 4, 2, 128, (150, 420), 6, 3, 4, 0.2, 2),
    ("fp32_g1_d64", "fp32", 2, 2, 2, 64, (64, 257), 4, 4, 2, 0.25, 0),
    # the remaining (dtype, group, head_dim) instantiations of the decode
    ("bf16_g2_d64", "bf16", 2, 4, 2, 64, (410, 95), 5, 5, 4, 0.1, 1),
    ("fp32_g1_d128", "fp32", 2, 2, 2, 128, (180, 333), 4, 4, 4, 0.1, 1),
    ("fp32_g2_d64", "fp32", 2, 4, 2, 64, (600, 77), 4, 4, 4, 0.1, 1),
    ("fp32_g4_d64", "fp32", 2, 8, 2, 64, (260, 1030), 5, 5, 4, 0.1, 1),
    ("fp32_g8_d128", "fp32", 1, 16, 2, 128, (700,), 4, 4, 8, 0.1, 1),
    # the most KV heads the library takes: num_kv_heads * head_dim = 4096
    ("bf16_kv32_g2_d128", "bf16", 2, 64, 32, 128, (300, 77), 4, 2, 4, 0.1, 1),
    ("fp32_kv64_g1_d64", "fp32", 1, 64, 64, 64, (200,), 3, 3, 2, 0.1, 1),
    ("bf16_kv64_g4_d64", "bf16", 1, 256, 64, 64, (150,), 3, 3, 2, 0.2, 1),
    # a large ragged batch: 300 sequences of 1 to 400 tokens
    ("bf16_b300_ragged", "bf16", 300, 8, 2, 128,
     tuple(int(x) for x in np.random.default_rng(300).integers(1, 401, size=300)), 3, 2, 2, 0.1, 1),
]


@pytest.mark.parametrize("case", SMALL, ids=[c[0] for c in SMALL])
def test_small_schedules(case):
    name, dt, B, Hq, Hkv, d, pre, steps, f, n_min, r, n_local = case
    w = W.Workload(name, dt, B, Hq, Hkv, d, pre, steps, f, n_min, r, n_local,
                   tuple(max(0, min(3, (L // 16) - 1)) for L in pre), dt == "bf16", 100 + len(name))
    _run_loop_parity(w)


def _random_case(i):
    """A seeded random schedule: dtype, group size, KV heads, head_dim, ragged
    prefill lengths (one to a few hundred blocks), steps, f (0: never), n_min, r
    and n_local drawn independently."""
    g = np.random.default_rng(7000 + i)
    dt = "bf16" if g.random() < 0.7 else "fp32"
    G = int(g.choice([1, 2, 4, 8]))
    Hkv = int(g.integers(1, 4))
    d = int(g.choice([64, 128]))
    B = int(g.integers(1, 5))
    pre = tuple(int(x) for x in g.integers(1, 2600, size=B))
    steps = int(g.integers(2, 9))
    f = int(g.choice([0, 1, 2, 3, 4, 5, 8]))
    n_min = int(g.integers(1, 20))
    r = float(np.round(g.uniform(0.02, 0.6), 3))
    n_local = int(g.integers(0, 3))
    name = f"rand{i}_{dt}_b{B}_g{G}_kv{Hkv}_d{d}_f{f}"
    return (name, dt, B, G * Hkv, Hkv, d, pre, steps, f, n_min, r, n_local)


RANDOM = [_random_case(i) for i in range(16)]


@pytest.mark.parametrize("case", RANDOM, ids=[c[0] for c in RANDOM])
def test_random_schedules(case):
    """Seeded random shapes and parameters through the whole step loop: every
    step's append, descriptors, selection and decode, and every rectification,
    against the oracle."""
    name, dt, B, Hq, Hkv, d, pre, steps, f, n_min, r, n_local = case
    w = W.Workload(name, dt, B, Hq, Hkv, d, pre, steps, f, n_min, r, n_local,
                   tuple(max(0, min(3, (L // 16) - 1)) for L in pre), dt == "bf16", 7000 + len(name))
    _run_loop_parity(w)


@pytest.mark.parametrize("case", [SMALL[0], SMALL[7]], ids=["bf16_g4_d128", "bf16_no_local"])
def test_small_schedules_unfused_append(case):
    """The same schedules with the append as its own call (resa_update_descriptors)
    before resa_select_blocks."""
    name, dt, B, Hq, Hkv, d, pre, steps, f, n_min, r, n_local = case
    w = W.Workload(name, dt, B, Hq, Hkv, d, pre, steps, f, n_min, r, n_local,
                   tuple(max(0, min(3, (L // 16) - 1)) for L in pre), dt == "bf16", 100 + len(name))
    _run_loop_parity(w, fused_append=False)


def test_append_select_with_the_token_already_in_the_cache():
    """resa_append_select with k_new = v_new = NULL: the caller has written the
    step's token itself; only its block's descriptor is refreshed before the
    selection (the same result as passing the token)."""
    from block_sparse_attention_quest_amd import resa as R
    w = W.Workload("append_null", "bf16", 3, 8, 2, 128, (31, 300, 1000), 6, 0, 4, 0.1, 1, (0, 1, 2), True, 19)
    a, b = _runner(w), _runner(w)
    for t in range(w.steps):
        a.decode_step(t)
        b.set_step_lens(t + 1)
        q, k, v = (b.step_inputs[x][t] for x in ("q", "k", "v"))
        for s in range(w.batch):  # write the token where the append would
            pos = w.prefill_lens[s] + t
            page = int(b.block_table_cpu[s, pos // 16])
            b.cache.k_pages[page, :, pos % 16] = k[s, 0]
            b.cache.v_pages[page, :, :, pos % 16] = v[s, 0]
        R.resa_append_select(b.cache, None, None, q, b.params, b.idx, b.count, b.n_cap, b.ws)
        R.resa_sparse_decode(b.cache, q, b.idx, b.count, b.n_cap, b.out, b.ws, b.scale)
        torch.cuda.synchronize()
        assert torch.equal(a.count, b.count), t
        for s in range(w.batch):
            n = int(a.count[s])
            assert torch.equal(a.idx[s, :, :n], b.idx[s, :, :n]), (t, s)
        assert torch.equal(a.out, b.out), t
    assert torch.equal(a.cache.desc, b.cache.desc)


def test_fused_and_unfused_append_agree():
    """resa_append_select leaves the cache, descriptors, selection and output
    exactly as resa_update_descriptors + resa_select_blocks do."""
    w = W.Workload("fused_vs_unfused", "bf16", 3, 16, 4, 128, (15, 513, 3000), 20, 0, 8, 0.1, 2,
                   (0, 2, 3), True, 31)
    a, b = _runner(w, fused_append=True), _runner(w, fused_append=False)
    for t in range(w.steps):
        oa, ob = a.decode_step(t), b.decode_step(t)
        torch.cuda.synchronize()
        assert torch.equal(a.count, b.count), t
        for s in range(w.batch):
            n = int(a.count[s])
            assert torch.equal(a.idx[s, :, :n], b.idx[s, :, :n]), (t, s)
        assert torch.equal(oa, ob), t
    assert torch.equal(a.cache.desc, b.cache.desc)
    assert torch.equal(a.cache.k_pages, b.cache.k_pages)
    assert torch.equal(a.cache.v_pages, b.cache.v_pages)


def test_single_token_sequences():
    """A sequence whose only token is the one just appended (M = 1, n = 1)."""
    w = W.Workload("one_token", "bf16", 3, 8, 2, 128, (0, 15, 16), 3, 0, 4, 0.1, 1, (0, 0, 0), True, 7)
    _run_loop_parity(w)


def test_rectify_whole_sequence_and_ragged_batch():
    """f equal to the whole length of the shortest sequence; lengths across tiles."""
    # f = 32 sizes the workspace; four decode steps never reach a scheduled rectification
    w = W.Workload("rect_all", "bf16", 3, 8, 2, 128, (28, 70, 513), 4, 32, 2, 0.1, 1, (0, 1, 2), True, 8)
    r = _runner(w)
    oc = P.oracle_cache(w)
    for t in range(4):
        q, k, v = W.query(w, t), *W.append_kv(w, t)
        O.append(oc, P.f64(k), P.f64(v))
        r.decode_step(t)
    for f in (32, 1, 17):   # 32 = the whole first sequence
        rq, rk, rv = (x[:, :f] for x in _rect_inputs(w, f, seed=f))
        ref = O.rectify(oc, P.f64(rq), P.f64(rk), P.f64(rv), 1.0 / math.sqrt(w.head_dim))
        got = r.rectify(3, rq.cuda(), rk.cuda(), rv.cuda(), f=f)
        torch.cuda.synchronize()
        err = P.out_error(P.f64(got), ref, "bf16")
        assert err <= P.ATOL["bf16"], (f, err)
        P.assert_desc_equal(r.cache.desc, oc)


def _rect_inputs(w, f, seed):
    g = torch.Generator().manual_seed(1000 + seed)
    q = torch.randn(w.batch, f, w.num_q_heads, w.head_dim, generator=g).to(w.torch_dtype)
    k = torch.randn(w.batch, f, w.num_kv_heads, w.head_dim, generator=g).to(w.torch_dtype)
    v = torch.randn(w.batch, f, w.num_kv_heads, w.head_dim, generator=g).to(w.torch_dtype)
    return q, k, v


@pytest.mark.parametrize("f", [64, 100], ids=["f64_one_row_tile", "f100_two_row_tiles"])
def test_rectify_mixed_lengths_small(f):
    """Mixed-length batch, G * f = 256 query rows per KV head (one row tile of
    8 waves) or 400 (a full tile of 256 rows and a partial one of 144)."""
    w = W.rectify_mixed(batch=4, len_range=(150, 3000), seed=21, f=f)
    print(f"[case] mixed rectify f={f} lens={w.prefill_lens}", flush=True)
    r = _runner(w)
    oc = P.oracle_cache(w)
    got = r.rectify_only()
    q, k, v = r.rect_inputs[-1]
    for b in range(w.batch):
        oc.seq_lens[b] += w.f
    ref = O.rectify(oc, P.f64(q), P.f64(k), P.f64(v), 1.0 / math.sqrt(w.head_dim))
    torch.cuda.synchronize()
    err = P.out_error(P.f64(got), ref, "bf16")
    print(f"[result] mixed rectify error beyond output rounding {err:.3g}")
    assert err <= P.ATOL["bf16"]
    P.assert_desc_equal(r.cache.desc, oc)


def test_rectify_batch_beyond_the_plan_lds():
    """1100 short sequences (more than the 1024 whose lengths and tile prefixes
    the work plan keeps in LDS): the plan reads them back from global memory."""
    w = W.rectify_mixed(batch=1100, len_range=(17, 90), seed=23, f=4).replace(num_q_heads=8, num_kv_heads=2)
    print(f"[case] rectify of {w.batch} sequences f={w.f} lens {min(w.prefill_lens)}..{max(w.prefill_lens)}",
          flush=True)
    r = _runner(w)
    oc = P.oracle_cache(w)
    got = r.rectify_only()
    q, k, v = r.rect_inputs[-1]
    for b in range(w.batch):
        oc.seq_lens[b] += w.f
    ref = O.rectify(oc, P.f64(q), P.f64(k), P.f64(v), 1.0 / math.sqrt(w.head_dim))
    torch.cuda.synchronize()
    err = P.out_error(P.f64(got), ref, "bf16")
    print(f"[result] rectify of {w.batch} sequences: error beyond output rounding {err:.3g}")
    assert err <= P.ATOL["bf16"]
    P.assert_desc_equal(r.cache.desc, oc)


def test_rectify_of_some_sequences_then_decode():
    """Continuous batching: sequences 1 .. 2 of 3 are rectified through a
    sub-batch view of the cache while sequence 0 is not; decoding of all three
    then continues on the updated cache."""
    w = W.Workload("sub_batch", "bf16", 3, 8, 2, 128, (200, 517, 64), 6, 4, 4, 0.2, 1, (0, 1, 0), True, 12)
    r = _runner(w)
    oc = P.oracle_cache(w)
    atol = P.ATOL[w.dtype]
    for t in range(6):
        q, k, v = W.query(w, t), *W.append_kv(w, t)
        O.append(oc, P.f64(k), P.f64(v))
        out = r.decode_step(t)
        torch.cuda.synchronize()
        P.check_select_and_decode(oc, P.f64(q), w, r.idx, r.count, out, atol)
        if t == 3:
            rq, rk, rv = (x[1:3, :w.f].contiguous() for x in _rect_inputs(w, w.f, seed=5))
            got = r.rectify_subset(t, 1, 3, rq.cuda(), rk.cuda(), rv.cuda())
            sub = O.PagedCache(oc.k, oc.v, oc.desc, oc.block_table[1:3], oc.seq_lens[1:3])
            ref = O.rectify(sub, P.f64(rq), P.f64(rk), P.f64(rv), 1.0 / math.sqrt(w.head_dim))
            oc.k, oc.v, oc.desc = sub.k, sub.v, sub.desc
            torch.cuda.synchronize()
            err = P.out_error(P.f64(got), ref, "bf16")
            assert err <= atol, err
            P.assert_desc_equal(r.cache.desc, oc)


def test_decode_is_deterministic():
    w = W.Workload("det", "bf16", 2, 8, 2, 128, (3000, 1234), 3, 0, 16, 0.1, 1, (5, 5), True, 9)
    outs = []
    for _ in range(2):
        r = _runner(w)
        res = []
        for t in range(3):
            res.append(r.decode_step(t).clone())
            res.append(r.idx.clone())
        torch.cuda.synchronize()
        outs.append(res)
    for a, b in zip(*outs):
        assert torch.equal(a, b)


def test_rectify_is_deterministic():
    """Two runs of one schedule with rectifications give bit-identical decode
    and rectification outputs, cache rows and descriptors (no reduction in the
    path uses atomics or a data-dependent order)."""
    w = W.Workload("det_rect", "bf16", 3, 8, 2, 128, (900, 3000, 77), 6, 3, 16, 0.1, 1, (3, 3, 2), True, 11)
    runs = []
    for _ in range(2):
        r = _runner(w)
        res = []
        for t in range(w.steps):
            res.append(r.decode_step(t).clone())
            if (t + 1) % w.f == 0:
                rq, rk, rv = W.rectify_inputs(w, t)
                res.append(r.rectify(t, rq.cuda(), rk.cuda(), rv.cuda()).clone())
        torch.cuda.synchronize()
        res += [r.cache.k_pages.clone(), r.cache.v_pages.clone(), r.cache.desc.clone()]
        runs.append(res)
    for a, b in zip(*runs):
        assert torch.equal(a, b)


def test_rebuilt_descriptors_equal_the_incremental_ones():
    """Resume: after decode steps (one appended token each) and rectifications,
    rebuilding every descriptor from the cached keys (resa_update_descriptors
    with n_new = 0, what a restart from saved K/V pages does) gives exactly the
    set the steps maintained."""
    from block_sparse_attention_quest_amd import resa as R
    w = W.Workload("resume", "bf16", 3, 8, 2, 128, (40, 1500, 333), 7, 3, 16, 0.1, 1, (1, 3, 3), True, 13)
    r = _runner(w)
    for t in range(w.steps):
        r.decode_step(t)
        if (t + 1) % w.f == 0:
            rq, rk, rv = W.rectify_inputs(w, t)
            r.rectify(t, rq.cuda(), rk.cuda(), rv.cuda())
    torch.cuda.synchronize()
    held = []
    for b in range(w.batch):
        M = -(-(w.prefill_lens[b] + w.steps) // 16)
        held += r.block_table_cpu[b, :M].tolist()
    held = torch.tensor(held, dtype=torch.long, device="cuda")
    incremental = r.cache.desc[held].clone()
    r.cache.desc[held] = float("nan")
    r.set_step_lens(w.steps)
    R.resa_update_descriptors(r.cache, None, None, 0)
    torch.cuda.synchronize()
    assert torch.equal(r.cache.desc[held], incremental)


def test_calls_from_two_host_threads_on_two_streams():
    """The library keeps no mutable state but the thread-local error text: two
    host threads, each with its own stream, workspace and outputs, select and
    decode over one shared cache concurrently; both results equal a
    single-threaded call's bit for bit, and an error raised on one thread does
    not show in the other's message."""
    import threading
    from block_sparse_attention_quest_amd import resa as R
    w = W.Workload("threads", "bf16", 3, 8, 2, 128, (5000, 1234, 777), 2, 0, 16, 0.1, 1, (5, 5, 5), True, 21)
    r = _runner(w)
    q = W.query(w, 0).cuda()
    r.set_step_lens(0)
    ws_size = max(R.resa_select_workspace_size(r.cache), R.resa_decode_workspace_size(r.cache, r.n_cap))

    def call(stream):
        ws = R.workspace(ws_size)
        idx = torch.full_like(r.idx, -1)
        count = torch.zeros_like(r.count)
        out = torch.empty_like(r.out)
        stream.wait_stream(torch.cuda.current_stream())  # the fills above run on this thread's current stream
        with torch.cuda.stream(stream):
            R.resa_select_blocks(r.cache, q, r.params, idx, count, r.n_cap, ws, stream)
            R.resa_sparse_decode(r.cache, q, idx, count, r.n_cap, out, ws, r.scale, stream)
        stream.synchronize()
        return idx, count, out

    ref = call(torch.cuda.current_stream())
    results, errors = {}, {}

    def worker(i):
        try:
            s = torch.cuda.Stream()
            results[i] = [call(s) for _ in range(4)]
            if i == 1:  # a rejected call on this thread only
                try:
                    R.resa_sparse_decode(r.cache, q, r.idx, r.count, 0, r.out, r.ws)
                except R.ResaError:
                    errors[i] = R.load().resa_last_error().decode()
            else:
                errors[i] = R.load().resa_last_error().decode()
        except Exception as e:  # reported by the main thread
            errors[i] = repr(e)

    threads = [threading.Thread(target=worker, args=(i,)) for i in range(2)]
    for t in threads:
        t.start()
    for t in threads:
        t.join()
    assert "n_cap" in errors[1], errors
    assert errors[0] == "", errors
    for i in range(2):
        for idx, count, out in results[i]:
            assert torch.equal(idx, ref[0]) and torch.equal(count, ref[1]) and torch.equal(out, ref[2])
