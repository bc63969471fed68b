"""Full-size parity on sampled outputs, in the launch configuration the benchmark
times (same workloads, same runner, same plans).

For sampled (sequence, KV head) groups the oracle recomputes, one group at a
time from the seeded generators: every descriptor of the group (bit-exact), the
group's selection (bit-exact up to near-ties), the decode outputs of its G heads
(with the GPU's validated selection), and sampled rectified rows.
"""
import math

import numpy as np
import pytest
import torch

from oracle import resa_oracle as O
from block_sparse_attention_quest_amd import workloads as W

import parity as P

pytestmark = [pytest.mark.gpu, pytest.mark.slow]


def _group_kv(w, b, g, steps_done, rect=None):
    """K, V [L][d] float64 of group (b, g) after `steps_done` decode steps, with
    the rows of a rectification (k, v [B][f][Hkv][d]) applied at the tail."""
    k0, v0 = W.prefill_kv(w, b, g)
    ks, vs = [P.f64(k0)], [P.f64(v0)]
    for t in range(steps_done):
        k, v = W.append_kv(w, t)
        ks.append(P.f64(k[b, g])[None])
        vs.append(P.f64(v[b, g])[None])
    K, V = np.concatenate(ks), np.concatenate(vs)
    if rect is not None:
        rk, rv = rect
        f = rk.shape[1]
        K[-f:] = P.f64(rk[b, :, g])
        V[-f:] = P.f64(rv[b, :, g])
    return K, V


def _check_group_step(w, r_bt, desc_g, idx, count, out, q, b, g, K, V):
    G = w.group
    M = O.num_blocks(len(K))
    kmin, kmax = O.block_descriptors(K)
    assert np.array_equal(desc_g[:, 0], kmin) and np.array_equal(desc_g[:, 1], kmax), "descriptors differ"
    n = O.active_block_count(M, w.n_min, w.r)
    assert count[b] == n
    qg = P.f64(q[b, g * G:(g + 1) * G])
    qbar = O.pooled_query(qg)
    s = O.block_upper_bounds(qbar, kmin, kmax)
    sel = idx[b, g, :n]
    ties = P.assert_selection_valid(sel, M, n, w.n_local, s, qbar, kmin, kmax)
    ref = O.sparse_decode_group(qg, K, V, sel.tolist(), 1.0 / math.sqrt(w.head_dim))
    err = P.out_error(P.f64(out[b, g * G:(g + 1) * G]), ref, w.dtype)
    assert err <= P.ATOL[w.dtype], err
    return err, ties


def _desc_of_group(r, w, b, g, L):
    M = O.num_blocks(L)
    pages = r.block_table_cpu[b, :M].to(torch.long).cuda()
    return P.f64(r.cache.desc[pages, g])


def _samples(w, k=3):
    rng = np.random.default_rng(w.seed)
    picks = {(0, 0), (w.batch - 1, w.num_kv_heads - 1)}
    while len(picks) < min(k, w.batch * w.num_kv_heads):
        picks.add((int(rng.integers(w.batch)), int(rng.integers(w.num_kv_heads))))
    return sorted(picks)


@pytest.mark.parametrize("make", [W.gqa_128k, W.llama8b_32k, W.long_256k, lambda: W.long_256k(r=0.05, f=64),
                                  W.longest],
                         ids=["128k_b4", "32k_b8", "256k_b1", "256k_b1_r05_f64", "512k_b1_longest"])
def test_decode_and_rectify_sampled(make):
    from block_sparse_attention_quest_amd.schedule import ResaRunner
    w0 = make()
    steps = w0.f
    w = w0.replace(steps=steps)
    print(f"[case] {w.name} full size, {steps} steps with a rectification after the last", flush=True)
    r = ResaRunner(w)
    r.fill_prefill()
    r.build_descriptors()
    samples = _samples(w)
    # step 0
    out = r.decode_step(0)
    torch.cuda.synchronize()
    idx, count, o0 = r.idx.cpu().numpy(), r.count.cpu().tolist(), out.cpu()
    q0 = W.query(w, 0)
    for (b, g) in samples:
        K, V = _group_kv(w, b, g, 1)
        err, ties = _check_group_step(w, None, _desc_of_group(r, w, b, g, len(K)), idx, count, o0, q0, b, g, K, V)
        print(f"[result] step 0 group {(b, g)}: max abs error {err:.3g}, near-tie swaps {ties}", flush=True)
        if b == 0 and g == 0 and w.planted[0]:
            planted = set(W.planted_blocks(w, 0))
            got = set(idx[0, 0, :count[0]].tolist())
            print(f"[result] planted blocks recalled: {len(planted & got)}/{len(planted)}", flush=True)
    # remaining steps, then the scheduled rectification
    for t in range(1, steps):
        r.decode_step(t)
    t = steps - 1
    torch.cuda.synchronize()
    idx, count, ol = r.idx.cpu().numpy(), r.count.cpu().tolist(), r.out.cpu()
    ql = W.query(w, t)
    for (b, g) in samples[:1]:
        K, V = _group_kv(w, b, g, steps)
        err, ties = _check_group_step(w, None, _desc_of_group(r, w, b, g, len(K)), idx, count, ol, ql, b, g, K, V)
        print(f"[result] step {t} group {(b, g)}: max abs error {err:.3g}", flush=True)
    rq, rk, rv = W.rectify_inputs(w, t)
    got = r.rectify(t, rq.cuda(), rk.cuda(), rv.cuda())
    torch.cuda.synchronize()
    got = got.cpu()
    scale = 1.0 / math.sqrt(w.head_dim)
    for (b, g) in samples:
        K, V = _group_kv(w, b, g, steps, rect=(rk, rv))
        L = len(K)
        assert np.array_equal(_desc_of_group(r, w, b, g, L)[-3:, 0], O.block_descriptors(K)[0][-3:])
        for i in (0, w.f // 2, w.f - 1):
            for h in range(g * w.group, (g + 1) * w.group):
                ref = O.causal_rows(P.f64(rq[b, i:i + 1, h]), K, V, L - w.f + i, scale)[0]
                err = P.out_error(P.f64(got[b, i, h]), ref, w.dtype)
                assert err <= P.ATOL[w.dtype], (b, i, h, err)
        print(f"[result] rectify rows of group {(b, g)} ok", flush=True)


def test_rectify_mixed_sampled():
    from block_sparse_attention_quest_amd.schedule import ResaRunner
    w = W.rectify_mixed()
    print(f"[case] {w.name}: lengths {[L + w.f for L in w.prefill_lens]}", flush=True)
    r = ResaRunner(w)
    r.fill_prefill()
    r.build_descriptors()
    got = r.rectify_only()
    torch.cuda.synchronize()
    got = got.cpu()
    q, k, v = (x.cpu() for x in r.rect_inputs[-1])
    scale = 1.0 / math.sqrt(w.head_dim)
    for (b, g) in _samples(w, 4):
        k0, v0 = W.prefill_kv(w, b, g)
        K = np.concatenate([P.f64(k0), P.f64(k[b, :, g])])
        V = np.concatenate([P.f64(v0), P.f64(v[b, :, g])])
        L = len(K)
        assert np.array_equal(_desc_of_group(r, w, b, g, L)[:, 0], O.block_descriptors(K)[0])
        for i in (0, 31, 63):
            for h in (g * w.group, (g + 1) * w.group - 1):
                ref = O.causal_rows(P.f64(q[b, i:i + 1, h]), K, V, L - w.f + i, scale)[0]
                err = P.out_error(P.f64(got[b, i, h]), ref, "bf16")
                assert err <= P.ATOL["bf16"], (b, i, h, err)
        print(f"[result] group {(b, g)} (L={L}) ok", flush=True)


def test_skewed_batch_longest_next_to_tiny_sequences():
    """One sequence at the longest context beside a 5-token and a 300-token one:
    the decode's splits and the rectification's plan are sized by the longest,
    most of the short sequences' splits are empty. The whole step loop, every
    descriptor and every rectification against the oracle."""
    from test_gpu_parity import _run_loop_parity
    L = 524288 - 3
    w = W.Workload("skewed_512k_5_300", "bf16", 3, 4, 1, 64, (L, 5, 300), 3, 2, 16, 0.1, 1, (3, 0, 3), True, 23)
    _run_loop_parity(w)
