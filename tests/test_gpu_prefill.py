"""GPU parity of the chunked prefill (dense causal prefill through the
rectification call, a chunk of positions per call) against the oracle's dense
causal attention, with the cache rows and every block descriptor compared
exactly."""
import math

import numpy as np
import pytest
import torch

from oracle import resa_oracle as O
from block_sparse_attention_quest_amd import workloads as W

import parity as P

pytestmark = pytest.mark.gpu

CASES = [
    # name, dtype, B, Hq, Hkv, d, T, chunk
    ("bf16_g4_d128_T300_c64", "bf16", 2, 8, 2, 128, 300, 64),
    ("bf16_g1_d64_T97_c32", "bf16", 1, 2, 2, 64, 97, 32),
    ("bf16_g8_d64_T150_c32", "bf16", 2, 16, 2, 64, 150, 32),      # 256 rows per KV head, head_dim 64
    ("bf16_g4_d128_T210_c48", "bf16", 1, 8, 2, 128, 210, 48),     # 192 rows: two waves without rows
    ("bf16_g8_d128_T200_c64", "bf16", 1, 16, 2, 128, 200, 64),    # 512 rows: two row tiles
    ("bf16_g4_d128_T700_c256", "bf16", 2, 8, 2, 128, 700, 256),   # 1024 rows: four row tiles
    ("bf16_g8_d64_T300_c100", "bf16", 1, 16, 2, 64, 300, 100),    # 800 rows: a partial fourth tile
    ("bf16_g8_d128_T130_c16", "bf16", 1, 16, 2, 128, 130, 16),
    ("fp32_g4_d64_T70_c16", "fp32", 1, 4, 1, 64, 70, 16),
]



def _random_case(i):
    """A seeded random prefill: dtype, group size, KV heads, head_dim, batch,
    prompt length and chunk size drawn independently."""
    g = np.random.default_rng(9000 + i)
    dt = "bf16" if g.random() < 0.75 else "fp32"
    G = int(g.choice([1, 2, 4, 8]))
    Hkv = int(g.integers(1, 4))
    d = int(g.choice([64, 128]))
    B = int(g.integers(1, 4))
    T = int(g.integers(20, 900))
    chunk = int(g.choice([1, 7, 16, 33, 64, 100, 256]))
    return (f"rand{i}_{dt}_b{B}_g{G}_kv{Hkv}_d{d}_T{T}_c{chunk}", dt, B, G * Hkv, Hkv, d, T, chunk)


CASES += [_random_case(i) for i in range(8)]

@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_chunked_prefill_matches_dense_causal(case):
    from block_sparse_attention_quest_amd.schedule import ChunkedPrefill
    name, dt, B, Hq, Hkv, d, T, chunk = case
    w = W.Workload(name, dt, B, Hq, Hkv, d, (T,) * B, 0, chunk, 16, 0.1, 1, (0,) * B, dt == "bf16", 31)
    print(f"[case] prefill {name}", flush=True)
    q, k, v = W.prompt_inputs(w)
    pf = ChunkedPrefill(w)
    pf.stage(q, k, v)
    pf.run()
    got = pf.output()
    torch.cuda.synchronize()
    G, scale = Hq // Hkv, 1.0 / math.sqrt(d)
    bt = pf.cache.block_table.cpu()
    worst = -1.0
    for b in range(B):
        M = -(-T // 16)
        pages = bt[b, :M].long()
        for g in range(Hkv):
            ks, vs = P.f64(k[b, :, g]), P.f64(v[b, :, g])
            # cache rows exactly as given
            assert torch.equal(pf.cache.k_pages[pages, g].cpu().reshape(M * 16, d)[:T], k[b, :, g])
            assert torch.equal(pf.cache.v_pages[pages, g].cpu().transpose(1, 2).reshape(M * 16, d)[:T], v[b, :, g])
            # every block descriptor built exactly
            kmin, kmax = O.block_descriptors(ks)
            dsc = P.f64(pf.cache.desc[pages, g].cpu())
            assert np.array_equal(dsc[:, 0], kmin) and np.array_equal(dsc[:, 1], kmax), (b, g)
            for h in range(g * G, (g + 1) * G):
                ref = O.causal_rows(P.f64(q[b, :, h]), ks, vs, 0, scale)
                err = P.out_error(P.f64(got[b, :, h]), ref, dt)
                worst = max(worst, err)
    print(f"[result] {name}: error beyond output rounding {worst:.3g}", flush=True)
    assert worst <= P.ATOL[dt]
