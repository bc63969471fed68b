"""Helpers of the GPU parity tests: build the oracle's state from the same seeded
inputs the GPU runner consumes, and compare the two to the stated bars."""
from __future__ import annotations

import numpy as np
import torch

from oracle import resa_oracle as O
from block_sparse_attention_quest_amd import workloads as W

# Output tolerances (absolute): fp32 accumulate in both paths. The bar is taken
# on top of the output's own rounding to its storage type: half a unit in the
# last place at the value's magnitude (a bf16 output of magnitude 8 .. 16 alone
# carries up to 2^-5 of it, above the 2e-2 bar, whatever computed it).
ATOL = {"fp32": 1e-4, "bf16": 2e-2}
TIE_REL = 1e-6
_SIGNIFICAND_BITS = {"fp32": 24, "bf16": 8}


def half_ulp(x: np.ndarray, dtype: str) -> np.ndarray:
    """Half a unit in the last place of `dtype` at |x| (normal range)."""
    a = np.maximum(np.abs(x), np.finfo(np.float64).tiny)
    e = np.floor(np.log2(a)).astype(np.int64)
    return np.ldexp(0.5, e - (_SIGNIFICAND_BITS[dtype] - 1))


def out_error(got: np.ndarray, ref: np.ndarray, dtype: str) -> float:
    """Largest deviation of a stored output from the oracle beyond the output's
    own rounding: max(|got - ref| - half_ulp(max(|got|, |ref|)))."""
    got, ref = np.asarray(got, dtype=np.float64), np.asarray(ref, dtype=np.float64)
    lim = half_ulp(np.maximum(np.abs(got), np.abs(ref)), dtype)
    return float(np.max(np.abs(got - ref) - lim))


def f64(t: torch.Tensor) -> np.ndarray:
    return t.detach().cpu().double().numpy()


def oracle_cache(w: W.Workload) -> O.PagedCache:
    """The oracle's paged cache after the prefill, same pages as the GPU."""
    bt = W.block_table(w).numpy()
    P, Hkv, d = w.num_pages, w.num_kv_heads, w.head_dim
    kp = np.zeros((P, Hkv, 16, d))
    vp = np.zeros((P, Hkv, 16, d))
    for b in range(w.batch):
        L = w.prefill_lens[b]
        for h in range(Hkv):
            k, v = W.prefill_kv(w, b, h)
            k, v = f64(k), f64(v)
            for t0 in range(0, L, 16):
                n = min(16, L - t0)
                kp[bt[b, t0 // 16], h, :n] = k[t0:t0 + n]
                vp[bt[b, t0 // 16], h, :n] = v[t0:t0 + n]
    cache = O.PagedCache(kp, vp, np.zeros((P, Hkv, 2, d)), bt, list(w.prefill_lens))
    cache.rebuild()
    return cache


def used_pages(cache: O.PagedCache):
    pages = []
    for b, L in enumerate(cache.seq_lens):
        pages.extend(cache.block_table[b, :O.num_blocks(L)].tolist())
    return np.array(sorted(pages), dtype=np.int64)


def assert_desc_equal(gpu_desc: torch.Tensor, oc: O.PagedCache, pages=None):
    """Descriptors bit-exact on the pages the sequences hold."""
    pages = used_pages(oc) if pages is None else np.asarray(pages, dtype=np.int64)
    g = f64(gpu_desc[torch.as_tensor(pages, device=gpu_desc.device)])
    o = oc.desc[pages]
    bad = np.argwhere(g != o)
    assert bad.size == 0, f"{len(bad)} descriptor values differ, first at {bad[0]}: gpu {g[tuple(bad[0])]} oracle {o[tuple(bad[0])]}"


def assert_selection_valid(sel, M, n, n_local, scores, qbar, kmin, kmax):
    """The GPU's set equals the oracle's, except for members whose oracle score
    is within TIE_REL of the threshold score (a near-tie decided by the
    order of the float64 sum)."""
    sel = [int(x) for x in sel]
    assert len(sel) == n, (len(sel), n)
    assert all(sel[i] < sel[i + 1] for i in range(len(sel) - 1)), "not strictly ascending"
    assert all(0 <= j < M for j in sel)
    keep = min(n_local, n)
    assert set(range(M - keep, M)) <= set(sel), "local blocks missing"
    ref = O.select_blocks(scores, n, n_local).tolist()
    if sel == ref:
        return 0
    others = sorted(range(M - keep), key=lambda j: (-scores[j], j))
    thr = scores[others[n - keep - 1]]
    mag = np.sum(np.abs(qbar)[None, :] * np.maximum(np.abs(kmin), np.abs(kmax)), axis=1)
    diff = set(sel) ^ set(ref)
    for j in diff:
        tol = TIE_REL * max(abs(thr), mag[j])
        assert abs(scores[j] - thr) <= tol, f"block {j}: score {scores[j]} vs threshold {thr}"
    return len(diff)


def check_select_and_decode(oc: O.PagedCache, q64: np.ndarray, w: W.Workload, gpu_idx: torch.Tensor,
                            gpu_count: torch.Tensor, gpu_out: torch.Tensor, atol: float):
    """Compare one decode step: counts, per-group selections, outputs (the
    oracle decodes with the GPU's validated selection)."""
    idx_o, cnt_o, scores_o = O.select(oc, q64, w.n_min, w.r, w.n_local)
    cnt = gpu_count.cpu().tolist()
    assert cnt == cnt_o, (cnt, cnt_o)
    gidx = gpu_idx.cpu().numpy()
    G = w.group
    sets = []
    ties = 0
    for b in range(w.batch):
        M = O.num_blocks(oc.seq_lens[b])
        row = []
        pages = oc.block_table[b, :M]
        for g in range(w.num_kv_heads):
            sel = gidx[b, g, :cnt[b]]
            ties += assert_selection_valid(sel, M, cnt[b], w.n_local, scores_o[b][g],
                                           O.pooled_query(q64[b, g * G:(g + 1) * G]),
                                           oc.desc[pages, g, 0], oc.desc[pages, g, 1])
            row.append(sel)
        sets.append(row)
    ref = O.decode(oc, q64, sets, 1.0 / np.sqrt(w.head_dim))
    err = out_error(f64(gpu_out), ref, w.dtype)
    assert err <= atol, f"decode error beyond output rounding {err} > {atol}"
    return err, ties
