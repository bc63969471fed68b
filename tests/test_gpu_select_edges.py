"""GPU parity of the block selection on crafted scores, through the C ABI.

The keys of every block are constant over its tokens in channels 0 and 1, the
queries are zero outside those two channels, so every Quest bound is
s_j = q0 * k0_j + q1 * k1_j, computed exactly in float64 on both sides (two
exact products, the other channels add signed zeros). With exact scores there
are no near-ties to excuse: the GPU's set must equal the oracle's exactly,
including which of several exactly tied blocks are taken (the lower indices).

The cases drive each branch of the selection: all scores equal, many exact
ties, keys that differ only in their low 32 bits, a threshold group of up to
64 blocks ranked one by one (and one of 70, which needs another radix pass),
a top group that fills the quota exactly, signed zeros and negative scores,
with n_local 0, 1 and 4 and rows of 1 to 5 register keys per thread, and
rows of 18 and 32 keys per thread (288K and 512K tokens, the longest rows).
"""

import numpy as np
import pytest
import torch

from oracle import resa_oracle as O
from block_sparse_attention_quest_amd import resa as R

import parity as P

pytestmark = pytest.mark.gpu

TINY = 2.0 ** -40  # q1: k1 * TINY changes only the low bits of a score near 1 .. 100


def _fill(kind, rng, M, quota, group=60):
    """(k0, k1) per block of one (sequence, KV head) row; every value is exact in bf16."""
    k0 = np.zeros(M)
    k1 = np.zeros(M)
    if kind == "all_equal":
        k0[:] = 3.25
    elif kind == "integer_ties":
        k0[:] = rng.integers(0, 20, M)
    elif kind == "low_word":
        k0[:] = 1.0
        k1[:] = rng.integers(0, 200, M)
    elif kind == "ranked_group":
        perm = rng.permutation(M)
        top = max(0, quota - group // 2)
        k0[:] = 10.0
        k1[:] = rng.integers(0, 100, M)
        k0[perm[:top]] = 100.0
        grp = perm[top:top + group]
        k0[grp] = 50.0
        k1[grp] = np.arange(len(grp)) % 45  # some exact ties inside the group
    elif kind == "exact_quota":
        k0[:] = 1.0
        k0[rng.permutation(M)[:quota]] = 2.0
    elif kind == "signed_zeros":
        k0[:] = rng.choice([-0.0, 0.0, 1.0, -1.0], M)
    elif kind == "negative":
        k0[:] = np.round(rng.standard_normal(M) * 32) / 32
    else:
        raise ValueError(kind)
    return k0, k1


def _run(kind, lens, params, q0=1.0, q1=0.0, group=60, Hkv=2, G=4, d=64, seed=0):
    n_min, r, n_local = params
    rng = np.random.default_rng(seed)
    B = len(lens)
    Ms = [O.num_blocks(L) for L in lens]
    maxb = min(max(Ms) + 2, 32768)  # the library's limit on blocks per sequence
    pages_needed = sum(Ms)
    Pn = pages_needed + 3
    perm = rng.permutation(Pn)
    bt = np.zeros((B, maxb), dtype=np.int64)
    off = 0
    for b, M in enumerate(Ms):
        bt[b, :M] = perm[off:off + M]
        off += M
    kp = rng.standard_normal((Pn, Hkv, 16, d))  # rounded to bf16 below
    for b, M in enumerate(Ms):
        n = O.active_block_count(M, n_min, r)
        quota = n - min(n_local, n)
        for g in range(Hkv):
            k0, k1 = _fill(kind, rng, M, quota, group)
            kp[bt[b, :M], g, :, 0] = k0[:, None]
            kp[bt[b, :M], g, :, 1] = k1[:, None]
    kb = torch.from_numpy(kp).to(torch.bfloat16)
    used = np.concatenate([bt[b, :M] for b, M in enumerate(Ms)])
    assert np.array_equal(P.f64(kb)[used, :, :, :2], kp[used, :, :, :2]), "crafted channels must be exact in bf16"
    kp = P.f64(kb)
    print(f"[case] {kind} lens={lens} params={params} q=({q0}, {q1}) group={group}", flush=True)

    cache = R.PagedKVCache(B, Hkv * G, Hkv, d, Pn, maxb, max(lens))
    cache.k_pages.copy_(kb)
    cache.block_table.copy_(torch.from_numpy(bt).to(torch.int32))
    cache.seq_lens.copy_(torch.tensor(lens, dtype=torch.int32))
    R.resa_update_descriptors(cache, None, None, 0)
    q = torch.zeros(B, Hkv * G, d, dtype=torch.bfloat16)
    q[:, :, 0] = q0
    q[:, :, 1] = q1
    prm = R.make_params(n_min, r, n_local)
    n_cap = R.resa_n_cap(cache, prm)
    idx = torch.full((B, Hkv, n_cap), -1, dtype=torch.int32, device="cuda")
    count = torch.zeros(B, dtype=torch.int32, device="cuda")
    ws = R.workspace(R.resa_select_workspace_size(cache))
    R.resa_select_blocks(cache, q.cuda(), prm, idx, count, n_cap, ws)
    torch.cuda.synchronize()

    oc = O.PagedCache(kp, np.zeros_like(kp), np.zeros((Pn, Hkv, 2, d)), bt, lens)
    oc.rebuild()
    P.assert_desc_equal(cache.desc, oc)
    idx_o, cnt_o, _ = O.select(oc, P.f64(q), n_min, r, n_local)
    assert count.cpu().tolist() == cnt_o
    gidx = idx.cpu().numpy()
    for b in range(B):
        for g in range(Hkv):
            got = gidx[b, g, :cnt_o[b]].tolist()
            ref = idx_o[b][g].tolist()
            assert got == ref, (kind, b, g, sorted(set(got) ^ set(ref))[:8])


LENS_A = [1026 * 16 + 3, 33, 4100 * 16, 16 * 700 + 1]   # up to 5 keys per thread
LENS_B = [1500 * 16, 17, 1]                              # 2 keys per thread, tiny rows


@pytest.mark.parametrize("params", [(16, 0.1, 1), (4, 0.3, 0), (8, 0.05, 4)], ids=["nl1", "nl0", "nl4"])
@pytest.mark.parametrize("kind", ["all_equal", "integer_ties", "low_word", "ranked_group", "exact_quota",
                                  "signed_zeros", "negative"])
def test_select_crafted_scores(kind, params):
    q0, q1 = {"low_word": (1.0, TINY), "ranked_group": (1.0, TINY), "signed_zeros": (-1.0, 0.0),
              "negative": (-0.5, 0.0)}.get(kind, (1.0, 0.0))
    _run(kind, LENS_A, params, q0, q1, seed=sum(map(ord, kind)))


@pytest.mark.parametrize("group", [64, 70])
def test_select_threshold_group_size(group):
    _run("ranked_group", LENS_A, (16, 0.1, 1), 1.0, TINY, group=group, seed=group)


@pytest.mark.parametrize("kind", ["integer_ties", "ranked_group", "low_word"])
def test_select_short_rows(kind):
    q1 = TINY if kind != "integer_ties" else 0.0
    _run(kind, LENS_B, (16, 0.1, 1), 1.0, q1, seed=7)


@pytest.mark.parametrize("kind", ["integer_ties", "ranked_group", "low_word"])
@pytest.mark.parametrize("lens", [[18000 * 16 + 5, 7000], [32768 * 16, 16 * 20000 + 3]], ids=["18_keys", "32_keys"])
def test_select_long_rows(kind, lens):
    q1 = 0.0 if kind == "integer_ties" else TINY
    _run(kind, lens, (16, 0.1, 1), 1.0, q1, Hkv=1, seed=11)


@pytest.mark.parametrize("keys_per_thread", [8, 10, 12, 14, 16, 20, 24])
def test_select_every_register_count(keys_per_thread):
    """Rows of 8 to 24 keys per thread (about 128K to 384K tokens): each of the
    selection's register-count builds, on a ranked threshold group."""
    M = keys_per_thread * 1000  # ceil(M / 1024) == keys_per_thread
    assert -(-M // 1024) == keys_per_thread
    _run("ranked_group", [M * 16 - 9, 7000], (16, 0.1, 1), 1.0, TINY, Hkv=1, seed=keys_per_thread)
