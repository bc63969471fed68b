"""GPU parity of the multi-stream schedule (schedule.Lanes) against the oracle.

The batch is cut into sequence ranges, each issuing its calls on a stream of
its own, a phase apart; every lane also has its own rectification phase
(continuous batching: sequences that are due rectify while the others keep
decoding; Pith review "If this is right" and the referee report's
"Significance" name compatibility with continuous batching). All steps are
queued without a host synchronisation in between; each step's selection,
count and outputs, and each rectification's rows, are copied out on the
lane's stream and checked against the oracle afterwards.
"""
import math

import numpy as np
import pytest
import torch

from oracle import resa_oracle as O
from block_sparse_attention_quest_amd import workloads as W

import parity as P

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("stagger", [True, False], ids=["staggered", "free"])
def test_lanes_with_their_own_rectification_phases(stagger):
    from block_sparse_attention_quest_amd.schedule import Lanes, ResaRunner
    w = W.Workload("lanes", "bf16", 4, 8, 2, 128, (700, 95, 2000, 333), 12, 4, 4, 0.1, 1, (2, 1, 3, 2), True, 33)
    ranges, phases = [(0, 1), (1, 3), (3, 4)], [0, 2, 1]
    print(f"[case] {w.name} lanes={ranges} phases={phases} stagger={stagger}", flush=True)
    r = ResaRunner(w)
    r.fill_prefill()
    r.build_descriptors()
    lanes = Lanes(r, ranges, stagger=stagger, phases=phases)
    rect_in = {t: tuple(x.cuda() for x in W.rectify_inputs(w, t)) for t in range(w.f - 1, w.steps)}
    outs = torch.empty(w.steps, *r.out.shape, dtype=r.out.dtype, device="cuda")
    idxs = torch.empty(w.steps, *r.idx.shape, dtype=r.idx.dtype, device="cuda")
    cnts = torch.empty(w.steps, *r.count.shape, dtype=r.count.dtype, device="cuda")
    routs = {}

    def keep(i, t, out, rout):
        b0, b1 = ranges[i]
        outs[t, b0:b1].copy_(out)
        idxs[t, b0:b1].copy_(r.idx[b0:b1])
        cnts[t, b0:b1].copy_(r.count[b0:b1])
        if rout is not None:
            routs[(i, t)] = rout[:, :w.f].clone()

    torch.cuda.synchronize()
    lanes.fork()
    for t in range(w.steps):
        lanes.step(t, rect_in, keep)
    lanes.join()
    torch.cuda.synchronize()

    oc = P.oracle_cache(w)
    scale = 1.0 / math.sqrt(w.head_dim)
    n_rect = 0
    for t in range(w.steps):
        q, k, v = W.query(w, t), *W.append_kv(w, t)
        O.append(oc, P.f64(k), P.f64(v))
        P.check_select_and_decode(oc, P.f64(q), w, idxs[t], cnts[t], outs[t], P.ATOL["bf16"])
        for i, (b0, b1) in enumerate(ranges):
            if not lanes.due(i, t):
                continue
            rq, rk, rv = (P.f64(x[b0:b1].cpu()) for x in rect_in[t])
            sub = O.PagedCache(oc.k, oc.v, oc.desc, oc.block_table[b0:b1], oc.seq_lens[b0:b1])
            ref = O.rectify(sub, rq, rk, rv, scale)
            oc.k, oc.v, oc.desc = sub.k, sub.v, sub.desc
            err = P.out_error(P.f64(routs[(i, t)]), ref, "bf16")
            assert err <= P.ATOL["bf16"], (i, t, err)
            n_rect += 1
    P.assert_desc_equal(r.cache.desc, oc)
    assert n_rect == len(routs) and n_rect >= 5
    print(f"[result] {w.name}: {w.steps} steps on {len(ranges)} lanes, {n_rect} lane rectifications, all match",
          flush=True)
