"""GPU parity of rectification work plans that the benchmark workloads do not
reach, on sampled rows against the oracle:

 * a plan of several rounds of workgroups (more key tiles than one round's
   ranges can hold: 8192 query rows per KV head in 32 row tiles over about
   270K keys), with 8-wave tiles at head_dim 64 and streaming (non-temporal)
   tile loads, since the K/V the call may read exceed the last-level cache;
 * the 4-wave tile at head_dim 64 with streaming loads.

Descriptors of the rewritten blocks are compared bit for bit, the rewritten
cache rows bit for bit, sampled output rows within the bf16 bar.
"""
import math

import numpy as np
import pytest
import torch

from oracle import resa_oracle as O
from block_sparse_attention_quest_amd import workloads as W

import parity as P

pytestmark = [pytest.mark.gpu, pytest.mark.slow]

LLC_BYTES = 256 << 20


def _check(w, rows, tiles_lower_bound=None):
    from block_sparse_attention_quest_amd.schedule import ResaRunner
    G = w.group
    lens = [L + w.f for L in w.prefill_lens]
    kv_capacity = w.batch * w.num_kv_heads * w.max_seq_len * 2 * w.head_dim * 2
    print(f"[case] {w.name}: B={w.batch} Hq={w.num_q_heads} Hkv={w.num_kv_heads} d={w.head_dim} f={w.f} "
          f"lens={lens} K/V capacity {kv_capacity >> 20} MiB", flush=True)
    assert kv_capacity > LLC_BYTES  # the tile loads stream past the caches
    r = ResaRunner(w)
    r.fill_prefill()
    r.build_descriptors()
    got = r.rectify_only()
    torch.cuda.synchronize()
    got = got.cpu()
    q, k, v = (x.cpu() for x in r.rect_inputs[-1])
    scale = 1.0 / math.sqrt(w.head_dim)
    bt = r.block_table_cpu
    for b in range(w.batch):
        for g in range(w.num_kv_heads):
            k0, v0 = W.prefill_kv(w, b, g)
            K = np.concatenate([P.f64(k0), P.f64(k[b, :, g])])
            V = np.concatenate([P.f64(v0), P.f64(v[b, :, g])])
            L = len(K)
            # rewritten rows and the descriptors of their blocks
            first = (L - w.f) // 16
            pages = bt[b, first:O.num_blocks(L)].to(torch.long)
            kp = P.f64(r.cache.k_pages[pages.cuda(), g]).reshape(-1, w.head_dim)
            assert np.array_equal(kp[(L - w.f) - first * 16:L - first * 16], K[L - w.f:])
            mn, mx = O.block_descriptors(K)
            dg = P.f64(r.cache.desc[pages.cuda(), g])
            assert np.array_equal(dg[:, 0], mn[first:]) and np.array_equal(dg[:, 1], mx[first:])
            for i in rows:
                for h in (g * G, g * G + G - 1):
                    ref = O.causal_rows(P.f64(q[b, i:i + 1, h]), K, V, L - w.f + i, scale)[0]
                    err = P.out_error(P.f64(got[b, i, h]), ref, "bf16")
                    assert err <= P.ATOL["bf16"], (b, g, i, h, err)
            print(f"[result] group {(b, g)} (L={L}) ok", flush=True)


def test_rectify_plan_of_several_rounds_d64_streaming():
    # 2 sequences x 2 KV heads x 32 row tiles, each tile's keys up to ~270K:
    # about 1.1M key tiles, more than the 256 x 1024 one round of 8-wave
    # workgroups can take, so the plan adds rounds
    w = W.rectify_mixed(batch=2, len_range=(270000, 272000), seed=61, f=1024).replace(
        name="rect_rounds_d64_g8_f1024", num_q_heads=16, num_kv_heads=2, head_dim=64)
    key_tiles = sum(w.num_kv_heads * 32 * ((L - 1024) // 32) for L in w.prefill_lens)
    assert key_tiles > 256 * 1024
    _check(w, rows=(0, 1, 511, 1023))


def test_rectify_four_wave_tiles_d64_streaming():
    w = W.rectify_mixed(batch=4, len_range=(135000, 140000), seed=62, f=32).replace(
        name="rect_4wave_d64_g4_f32", num_q_heads=8, num_kv_heads=2, head_dim=64)
    _check(w, rows=(0, 17, 31))
