"""GPU parity of resa_update_descriptors through the C ABI when one call appends
several tokens to every sequence: the new rows land in their pages bit-exact
(K token-major, V channel-major) and every block's descriptor equals the
oracle's channel-wise min and max over its valid tokens.

Cases: an unaligned run of 37 tokens that spans four blocks, a sequence
shorter than the run (its positions below 0 are skipped), a run that ends on a
block boundary, and a refresh without new rows (k_new and v_new NULL) after
the cache rows were changed behind the descriptors' back; bf16 at d 128 and
fp32 at d 64.
"""
import numpy as np
import pytest
import torch

from oracle import resa_oracle as O
from block_sparse_attention_quest_amd import resa as R

import parity as P

pytestmark = pytest.mark.gpu

# lengths after the append: the first run starts in the last slot of a block
# and spans four blocks, the second sequence is shorter than the run, the third
# run ends on a block boundary
LENS = [16 * 5 + 15 + 37, 20, 16 * 12]
N_NEW = 37


def _setup(dtype, d, seed):
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float32
    rng = np.random.default_rng(seed)
    B, Hkv, G = len(LENS), 2, 4
    Ms = [O.num_blocks(L) for L in LENS]
    maxb = max(Ms) + 1
    Pn = sum(Ms) + 3
    perm = rng.permutation(Pn)
    bt = np.zeros((B, maxb), dtype=np.int64)
    off = 0
    for b, M in enumerate(Ms):
        bt[b, :M] = perm[off:off + M]
        off += M
    # the cache before the call: every slot holds an older value
    k_old = torch.from_numpy(rng.standard_normal((Pn, Hkv, 16, d))).to(tdt)
    v_old = torch.from_numpy(rng.standard_normal((Pn, Hkv, 16, d))).to(tdt)
    k_new = torch.from_numpy(rng.standard_normal((B, N_NEW, Hkv, d))).to(tdt)
    v_new = torch.from_numpy(rng.standard_normal((B, N_NEW, Hkv, d))).to(tdt)
    cache = R.PagedKVCache(B, Hkv * G, Hkv, d, Pn, maxb, max(LENS), dtype=tdt)
    cache.k_pages.copy_(k_old)
    cache.v_pages.copy_(v_old.transpose(2, 3))
    cache.block_table.copy_(torch.from_numpy(bt).to(torch.int32))
    cache.seq_lens.copy_(torch.tensor(LENS, dtype=torch.int32))
    oc = O.PagedCache(P.f64(k_old), P.f64(v_old), np.zeros((Pn, Hkv, 2, d)), bt, LENS)
    return cache, oc, k_new, v_new


def _check(cache, oc):
    torch.cuda.synchronize()
    pages = P.used_pages(oc)
    assert np.array_equal(P.f64(cache.k_pages)[pages], oc.k[pages])
    assert np.array_equal(P.f64(cache.v_pages.transpose(2, 3))[pages], oc.v[pages])
    P.assert_desc_equal(cache.desc, oc)


@pytest.mark.parametrize("dtype, d", [("bf16", 128), ("fp32", 64)])
def test_append_of_several_tokens(dtype, d):
    cache, oc, k_new, v_new = _setup(dtype, d, seed=31 if dtype == "bf16" else 32)
    print(f"[case] update_descriptors {dtype} d={d} lens={LENS} n_new={N_NEW}", flush=True)
    R.resa_update_descriptors(cache, None, None, 0)  # descriptors of the older rows
    R.resa_update_descriptors(cache, k_new.cuda(), v_new.cuda(), N_NEW)
    kn, vn = P.f64(k_new), P.f64(v_new)
    for b, L in enumerate(LENS):
        for i in range(N_NEW):
            pos = L - N_NEW + i
            if pos >= 0:
                oc.write(b, pos, kn[b, i], vn[b, i])
    oc.rebuild()
    _check(cache, oc)


@pytest.mark.parametrize("dtype, d", [("bf16", 128), ("fp32", 64)])
def test_refresh_without_new_rows(dtype, d):
    cache, oc, _, _ = _setup(dtype, d, seed=33)
    print(f"[case] refresh-only {dtype} d={d} lens={LENS} n_new=20", flush=True)
    R.resa_update_descriptors(cache, None, None, 0)
    # rows of the last 20 positions change behind the descriptors' back (the
    # cache already holds them), then only those blocks are refreshed
    rng = np.random.default_rng(34)
    for b, L in enumerate(LENS):
        for pos in range(max(0, L - 20), L):
            page, slot = int(oc.block_table[b, pos // 16]), pos % 16
            row = torch.from_numpy(rng.standard_normal((oc.num_kv_heads, d))).to(cache.dtype)
            cache.k_pages[page, :, slot] = row.cuda()
            oc.k[page, :, slot] = P.f64(row)
    R.resa_update_descriptors(cache, None, None, 20)
    oc.rebuild()
    _check(cache, oc)
