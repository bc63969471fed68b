#!/usr/bin/env python3
"""Benchmark of the ReSA hot path on one MI355X.

A step is one pass of the whole hot path over the batch: append + descriptor
update, GBSA selection, sparse decode, and, after every f-th step, the dense
rectification of the f newest tokens (so the step rate is amortised over the
rectification). Inputs are seeded synthetic tensors already resident in HBM.

Prints ONE JSON line. Default workload: batch 4, 32 query / 8 KV heads,
head_dim 128, bf16, 128K-token prefill, block 16, r = 0.1, n_min = 16, f = 32.

  python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]
                  [--no-cpu-baseline] [--cpu-seconds S]
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "GBSA decode steps/s + achieved HBM GB/s at 128K ctx (32q/8kv, d=128)"
HBM_PEAK_GBS = 8000.0
MFMA_BF16_PEAK_TFLOPS = 2500.0
MEASURE_STEPS = 64
COLD_REPS = 16
QUEUE_AHEAD_CYCLES = 100_000_000  # about 40 ms of spinning: covers queueing the measured steps


def _workloads():
    from block_sparse_attention_quest_amd import workloads as W
    return {"gqa_128k": W.gqa_128k, "llama8b_32k": W.llama8b_32k, "long_256k": W.long_256k,
            "long_256k_r05": lambda: W.long_256k(r=0.05), "long_256k_f64": lambda: W.long_256k(f=64),
            "long_256k_r05_f64": lambda: W.long_256k(r=0.05, f=64),
            # the longest context, less room for the bench's up to 512 steps
            "longest": lambda: W.longest(prefill_lens=(524288 - 512,)), "tiny_fp32": W.tiny_fp32, "rectify_mixed": W.rectify_mixed,
            "prompt_32k": W.prompt_32k,
            "prompt_32k_c256": lambda: W.prompt_32k(f=256), "prompt_32k_c1024": lambda: W.prompt_32k(f=1024)}


# ---------------------------------------------------------------------------
# Algorithmic bytes / flops (what the method must move; Eq. 6 accounting)
# ---------------------------------------------------------------------------

def step_bytes(w, L_list, n_list):
    """Algorithmic HBM bytes of one decode step at sequence lengths L_list (new
    token included) with n_list selected blocks per sequence."""
    e = 2 if w.dtype == "bf16" else 4
    d, Hkv, Hq = w.head_dim, w.num_kv_heads, w.num_q_heads
    append = desc = sel = 0
    for L, n in zip(L_list, n_list):
        M = -(-L // 16)
        valid_last = L - 16 * (M - 1)
        # append: the new K/V row, the block's K rows read, its descriptor written
        append += Hkv * (2 * d * e + valid_last * d * e + 2 * d * e)
        desc += Hkv * M * 2 * d * e
        # selected tokens of every group (the newest block is always selected)
        tokens = 16 * n - (16 - valid_last)
        sel += Hkv * tokens * 2 * d * e
    qo = w.batch * Hq * d * e * 2  # q read by select and by decode; out written
    return {"append": append, "select": desc + w.batch * Hq * d * e,
            "decode": sel + qo, "selected_kv": sel, "descriptors": desc}


def rectify_work(w, L_list, f):
    e = 2 if w.dtype == "bf16" else 4
    d, Hkv, Hq = w.head_dim, w.num_kv_heads, w.num_q_heads
    kv = sum(Hkv * L * 2 * d * e for L in L_list)
    flops = sum(4 * d * Hq * (f * (L - f) + f * (f + 1) // 2) for L in L_list)
    return kv, flops


def decode_traffic(w):
    """HBM bytes per resa_sparse_decode launch from the rocprofv3 FETCH_SIZE /
    WRITE_SIZE runs recorded under profiles/ (scaled by the copy-kernel
    calibration recorded with them); None if they were taken on another
    workload or on a different version of the decode kernels."""
    import hashlib
    path = os.path.join(ROOT, "profiles", "traffic_decode_gqa128k_b4.json")
    csrc = os.path.join(ROOT, "block_sparse_attention_quest_amd", "csrc")
    try:
        rec = json.load(open(path))
        h = hashlib.sha256()
        for name in ("k_decode.hip", "resa_internal.h"):  # the decode kernels and their helpers
            h.update(open(os.path.join(csrc, name), "rb").read())
        digest = h.hexdigest()
    except (OSError, ValueError):
        return None
    if rec.get("source_sha256") != digest or rec.get("workload") != w.name:
        return None
    return int(rec["bytes_per_launch"])


def n_for(M, w):
    return min(M, max(w.n_min, math.ceil(float(M) * float(w.r))))


# ---------------------------------------------------------------------------
# CPU baseline: the oracle as it stands, on a bounded sample of the workload
# ---------------------------------------------------------------------------

def cpu_baseline(w, first_step, budget_s):
    import numpy as np
    import torch
    from block_sparse_attention_quest_amd import workloads as W
    from oracle import resa_oracle as O

    cores = len(os.sched_getaffinity(0))
    try:
        from threadpoolctl import threadpool_info
        blas_threads = max([p.get("num_threads", 1) for p in threadpool_info()] or [1])
    except Exception:  # pragma: no cover
        blas_threads = 1
    G, d = w.group, w.head_dim
    scale = 1.0 / math.sqrt(d)
    groups = [(b, g) for b in range(w.batch) for g in range(w.num_kv_heads)]
    rng = np.random.default_rng(0)
    rng.shuffle(groups)
    t_dec, t_row = [], []
    t0 = time.perf_counter()
    q_all = W.query(w, first_step).double().numpy()
    for (b, g) in groups:
        k0, v0 = W.prefill_kv(w, b, g)
        ks = [k0.double().numpy()]
        vs = [v0.double().numpy()]
        for t in range(first_step + 1):
            k, v = W.append_kv(w, t)
            ks.append(k[b, g][None].double().numpy())
            vs.append(v[b, g][None].double().numpy())
        K = np.concatenate(ks)
        V = np.concatenate(vs)
        kmin, kmax = O.block_descriptors(K[:-1]) if len(K) > 1 else (None, None)
        qg = q_all[b, g * G:(g + 1) * G]
        M = O.num_blocks(len(K))
        # one decode step of this group: append's block descriptor, scoring, selection, decode
        s0 = time.perf_counter()
        last = (M - 1) * 16
        lmin, lmax = O.block_descriptors(K[last:])
        if kmin is not None and len(kmin) == M:
            kmin[-1], kmax[-1] = lmin[0], lmax[0]
        else:
            kmin = np.concatenate([kmin, lmin]) if kmin is not None else lmin
            kmax = np.concatenate([kmax, lmax]) if kmax is not None else lmax
        s = O.block_upper_bounds(O.pooled_query(qg), kmin, kmax)
        sel = O.select_blocks(s, O.active_block_count(M, w.n_min, w.r), w.n_local)
        O.sparse_decode_group(qg, K, V, sel, scale)
        t_dec.append(time.perf_counter() - s0)
        # rectification rows of this group, each over the full cache
        if w.f > 0 and len(t_row) < 4:
            for i in range(2):
                s1 = time.perf_counter()
                O.causal_rows(qg[i:i + 1], K, V, len(K) - 1, scale)
                t_row.append(time.perf_counter() - s1)
        if time.perf_counter() - t0 > budget_s:
            break
    dec = float(np.mean(t_dec))
    row = float(np.mean(t_row)) if t_row else 0.0
    # per step: every group decodes once; every f steps B * f * Hq rows are rectified
    sec_per_step = w.batch * w.num_kv_heads * dec + (w.batch * w.num_q_heads * row if w.f > 0 else 0.0)
    return {"value": 1.0 / sec_per_step, "unit": "steps/s", "cores": int(cores), "kind": "oracle",
            "blas_threads": int(blas_threads),
            "sample": (f"{len(t_dec)} of {w.batch * w.num_kv_heads} (sequence, KV-head) groups of one decode step "
                       f"and {len(t_row)} rectified query rows over the full context, timed on the host in float64 "
                       f"NumPy and scaled to the whole batch ({dec * 1e3:.1f} ms per group step, "
                       f"{row * 1e3:.1f} ms per rectified row); cores = the host threads this process may run on, "
                       f"of which the matrix products use {blas_threads} BLAS threads and the element-wise "
                       f"NumPy steps one")}


def oracle_sweep(args):
    """The oracle as it stands, timed on the host for every workload: all 64
    steps of the tiny fp32 schedule (rectifications included), and for each
    large workload one decode step (append, descriptor, selection and sparse
    decode of every (sequence, KV head) group) and one rectification event
    (every query row over its causal prefix), each measured on a bounded
    sample (whole groups, whole rows) and scaled to the batch. Prints one JSON
    line per workload and a markdown table."""
    import numpy as np
    from block_sparse_attention_quest_amd import workloads as W
    from oracle import resa_oracle as O

    cores = len(os.sched_getaffinity(0))
    budget = args.cpu_seconds
    rows_out = []

    # the tiny schedule, whole
    w = W.tiny_fp32()
    bt = W.block_table(w).numpy()
    kp = np.zeros((w.num_pages, 1, 16, w.head_dim))
    vp = np.zeros_like(kp)
    k0, v0 = W.prefill_kv(w, 0, 0)
    for t in range(w.prefill_lens[0]):
        kp[bt[0, t // 16], 0, t % 16] = k0[t].double().numpy()
        vp[bt[0, t // 16], 0, t % 16] = v0[t].double().numpy()
    cache = O.PagedCache(kp, vp, np.zeros((w.num_pages, 1, 2, w.head_dim)), bt, list(w.prefill_lens))
    cache.rebuild()
    steps = [(W.query(w, t).double().numpy(),) + tuple(x.double().numpy() for x in W.append_kv(w, t))
             for t in range(w.steps)]
    rect = {t: tuple(x.double().numpy() for x in W.rectify_inputs(w, t)) for t in W.rectify_steps(w)}
    t0 = time.perf_counter()
    O.resa_loop(cache, w.steps, w.f, w.n_min, w.r, w.n_local, 1.0 / math.sqrt(w.head_dim),
                step_inputs=lambda t: steps[t], rectify_inputs=lambda t: rect[t])
    sec = time.perf_counter() - t0
    rows_out.append({"workload": w.name, "oracle_steps_per_s": round(w.steps / sec, 2),
                     "sample": f"all {w.steps} steps and {len(rect)} rectifications, {sec:.2f} s"})
    print(json.dumps(rows_out[-1]), flush=True)

    for make in (W.llama8b_32k, W.gqa_128k, W.long_256k, lambda: W.long_256k(f=64), W.rectify_mixed):
        w = make()
        G, d = w.group, w.head_dim
        scale = 1.0 / math.sqrt(d)
        groups = [(b, g) for b in range(w.batch) for g in range(w.num_kv_heads)]
        np.random.default_rng(w.seed).shuffle(groups)
        decode = w.steps > 0
        t_dec, t_row = [], []
        q_step = W.query(w, 0).double().numpy() if decode else None
        rq = (W.rectify_only_inputs(w)[0] if not decode else W.rectify_inputs(w, w.f - 1)[0]).double().numpy()
        t_start = time.perf_counter()
        for (b, g) in groups:
            k0, v0 = W.prefill_kv(w, b, g)
            K, V = k0.double().numpy(), v0.double().numpy()
            if decode:
                k, v = W.append_kv(w, 0)
                K = np.concatenate([K, k[b, g][None].double().numpy()])
                V = np.concatenate([V, v[b, g][None].double().numpy()])
                kmin, kmax = O.block_descriptors(K[:len(K) - (len(K) - 1) % 16 - 1])  # the blocks before the newest
                qg = q_step[b, g * G:(g + 1) * G]
                M = O.num_blocks(len(K))
                best = math.inf
                for _ in range(2):  # the faster of two: the input draws' thread pool may still be spinning
                    s0 = time.perf_counter()
                    lmin, lmax = O.block_descriptors(K[(M - 1) * 16:])
                    km = np.concatenate([kmin[:M - 1], lmin])
                    kx = np.concatenate([kmax[:M - 1], lmax])
                    s = O.block_upper_bounds(O.pooled_query(qg), km, kx)
                    sel = O.select_blocks(s, O.active_block_count(M, w.n_min, w.r), w.n_local)
                    O.sparse_decode_group(qg, K, V, sel, scale)
                    best = min(best, time.perf_counter() - s0)
                t_dec.append(best)
            # rectified rows of this group: the last row of the f (the longest prefix)
            L = len(K) + (w.f if not decode else 0)
            if not decode:
                k, v = W.rectify_only_inputs(w)[1:]
                K = np.concatenate([K, k[b, :, g].double().numpy()])
                V = np.concatenate([V, v[b, :, g].double().numpy()])
            best = math.inf
            for _ in range(2):
                s1 = time.perf_counter()
                O.causal_rows(rq[b, -1:, g * G], K, V, len(K) - 1, scale)
                best = min(best, time.perf_counter() - s1)
            t_row.append(best)
            if time.perf_counter() - t_start > budget:
                break
        # every one of a group's f * G rows sees about as many keys as its
        # last row (f is small against the context)
        rect_s = float(np.mean(t_row)) * w.f * G * len(groups)
        row = {"workload": f"{w.name} (f {w.f})", "oracle_rectify_s": round(rect_s, 2),
               "sample": (f"{len(t_row)} of {len(groups)} groups; rectification: the last row of each sampled "
                          f"group timed, scaled to all {w.batch * w.f * w.num_q_heads} rows")}
        if decode:
            dec_s = float(np.mean(t_dec)) * len(groups)
            row["oracle_decode_step_s"] = round(dec_s, 3)
            row["oracle_steps_per_s_amortised"] = round(1.0 / (dec_s + rect_s / w.f), 3)
            row["sample"] += f"; decode: {len(t_dec)} groups' steps timed, scaled to {len(groups)}"
        rows_out.append(row)
        print(json.dumps(row), flush=True)
    print(f"| workload | oracle decode step (s) | oracle rectification event (s) | oracle steps/s | sample |")
    print("|---|---|---|---|---|")
    for r in rows_out:
        print(f"| {r['workload']} | {r.get('oracle_decode_step_s', '-')} | {r.get('oracle_rectify_s', '-')} | "
              f"{r.get('oracle_steps_per_s', r.get('oracle_steps_per_s_amortised', '-'))} | {r['sample']} |")
    print(f"host threads available: {cores}")


# ---------------------------------------------------------------------------

def rectify_only(w, args):
    """Rectify-only workload (mixed lengths, f new tokens per sequence): one
    rectification event is the unit; the same event is repeated (it rewrites
    the same positions, so every repetition does identical work)."""
    import torch
    from block_sparse_attention_quest_amd.schedule import ResaRunner

    K, Wu = args.steps, args.warmup
    r = ResaRunner(w)
    r.fill_prefill()
    r.build_descriptors()
    from block_sparse_attention_quest_amd import workloads as W
    q, k, v = (x.cuda() for x in W.rectify_only_inputs(w))
    for _ in range(Wu):
        r.rectify(0, q, k, v)
    stream = torch.cuda.current_stream()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record(stream)
    for _ in range(K):
        r.rectify(0, q, k, v)
    e1.record(stream)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / K
    L_list = [L + w.f for L in w.prefill_lens]
    kv, flops = rectify_work(w, L_list, w.f)
    tflops = flops / (ms * 1e-3) / 1e12
    gbs = kv / (ms * 1e-3) / 1e9
    print(json.dumps({
        "metric": "dense rectification events/s (mixed-length batch, MFMA path)", "value": round(1e3 / ms, 2),
        "unit": "events/s", "n_gpus": 1, "steps": K, "warmup": Wu, "ms_per_step": round(ms, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": w.dtype, "data": "synthetic",
        "config": {"workload": w.name, "batch": w.batch, "f": w.f, "q_heads": w.num_q_heads,
                   "kv_heads": w.num_kv_heads, "head_dim": w.head_dim, "total_tokens": sum(L_list)},
        "roofline": {"bound": "mfma", "achieved": round(tflops, 1), "peak": MFMA_BF16_PEAK_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(tflops / MFMA_BF16_PEAK_TFLOPS, 4), "traffic": None,
                     "hbm_gbs": round(gbs, 1), "hbm_frac": round(gbs / HBM_PEAK_GBS, 4),
                     "flops_per_launch": flops, "kv_bytes_per_launch": kv},
        "cpu_baseline": None}))


def prefill_only(w, args):
    """Chunked prefill workload: the whole prompt is one unit (every chunk of f
    positions through the rectification call, in order); repeated runs rewrite
    the same rows, so each does identical work."""
    import torch
    from block_sparse_attention_quest_amd import workloads as W
    from block_sparse_attention_quest_amd.schedule import ChunkedPrefill

    K, Wu = args.steps, args.warmup
    pf = ChunkedPrefill(w)
    pf.stage(*W.prompt_inputs(w))
    for _ in range(Wu):
        pf.run()
    stream = torch.cuda.current_stream()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record(stream)
    for _ in range(K):
        pf.run()
    e1.record(stream)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / K
    B, T, d, Hq, Hkv = w.batch, pf.T, w.head_dim, w.num_q_heads, w.num_kv_heads
    e = 2 if w.dtype == "bf16" else 4
    flops = 4.0 * d * Hq * B * T * (T + 1) / 2
    # each chunk reads the cache up to its end once
    kv = sum(B * Hkv * (c0 + fc) * 2 * d * e for c0, fc in pf.chunks)
    tflops = flops / (ms * 1e-3) / 1e12
    gbs = kv / (ms * 1e-3) / 1e9
    print(json.dumps({
        "metric": "chunked prefill tokens/s (dense causal, one rectification call per chunk)",
        "value": round(B * T / (ms * 1e-3), 1), "unit": "tokens/s", "n_gpus": 1, "steps": K, "warmup": Wu,
        "ms_per_step": round(ms, 4), "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": w.dtype, "data": "synthetic",
        "config": {"workload": w.name, "batch": B, "prompt": T, "chunk": pf.chunk, "q_heads": Hq, "kv_heads": Hkv,
                   "head_dim": d, "calls": len(pf.chunks)},
        "roofline": {"bound": "mfma", "achieved": round(tflops, 1), "peak": MFMA_BF16_PEAK_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(tflops / MFMA_BF16_PEAK_TFLOPS, 4), "traffic": None,
                     "hbm_gbs": round(gbs, 1), "hbm_frac": round(gbs / HBM_PEAK_GBS, 4),
                     "flops_per_prefill": flops, "kv_bytes_per_prefill": kv},
        "cpu_baseline": None}))


def sweep(args):
    """Context-length sweep at batch 1 (32q/8kv, d 128, bf16), the kernel-level
    breakdown the pages plot ("Rectified Sparse Attention", Figure 6): dense
    decode (every block, the same decode kernel), sparse decoding (append +
    select + sparse decode, no rectification: f = infinity) at several active
    ratios r, one rectification event at several f, and ReSA per step (sparse
    step + rectification / f). Prints a markdown table and one JSON line per
    context length."""
    import torch
    from block_sparse_attention_quest_amd import resa as R
    from block_sparse_attention_quest_amd import workloads as W
    from block_sparse_attention_quest_amd.schedule import ResaRunner

    torch.cuda.set_device(0)
    K, Wu = args.steps, args.warmup
    ratios, fs = (0.05, 0.1, 0.2), (16, 32, 64, 128)
    stream = torch.cuda.current_stream()

    def timed(fn, n):
        """GPU time per call of n calls queued back to back behind a spin kernel
        (so the host's per-call cost does not enter at batch 1)."""
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        torch.cuda._sleep(QUEUE_AHEAD_CYCLES)
        held = torch.cuda.Event()
        held.record(stream)
        e0.record(stream)
        for i in range(n):
            fn(i)
        e1.record(stream)
        if held.query():
            print("[sweep] warning: the GPU caught up with the host while calls were queued", file=sys.stderr)
        torch.cuda.synchronize()
        return 1e3 * e0.elapsed_time(e1) / n

    rows = []
    for L in (32768, 65536, 131072, 262144):
        steps = len(ratios) * (Wu + K) + 2
        w = W.long_256k(prefill_lens=(L,), steps=steps, r=1.0, f=max(fs),
                        planted=(int(round(0.01 * (L // 16))),))
        print(f"[sweep] context {L}: setting up", file=sys.stderr, flush=True)
        r = ResaRunner(w)
        r.fill_prefill()
        r.build_descriptors()
        # dense decode: every block selected (r = 1), decode call only, at length L + 1
        r.decode_step(0)
        dense = timed(lambda i: R.resa_sparse_decode(r.cache, r.step_inputs["q"][0], r.idx, r.count, r.n_cap,
                                                     r.out, r.ws, r.scale), K)
        t = 1
        sparse = {}
        for rv in ratios:
            # the index buffer sized for this ratio: the decode call splits its
            # work by the capacity n_cap it is given
            r.params = R.make_params(w.n_min, rv, w.n_local)
            r.n_cap = R.resa_n_cap(r.cache, r.params)
            r.idx = torch.full((w.batch, w.num_kv_heads, r.n_cap), -1, dtype=torch.int32, device="cuda")
            for _ in range(Wu):
                r.decode_step(t)
                t += 1
            t0 = t
            sparse[rv] = timed(lambda i: r.decode_step(t0 + i), K)
            t += K
        # one rectification of the f newest tokens
        rect = {}
        for f in fs:
            g = torch.Generator().manual_seed(f)
            ins = tuple(torch.randn(1, f, hh, 128, generator=g).to(torch.bfloat16).cuda() for hh in (32, 8, 8))

            def event(_i, ins=ins, f=f):
                r.rectify(t - 1, *ins, f=f)
            event(0)
            rect[f] = timed(event, max(4, K // 8))
        row = {"context": L, "dense_decode_us": round(dense, 1),
               **{f"sparse_r{rv}_us": round(sparse[rv], 1) for rv in ratios},
               **{f"rectify_f{f}_us": round(rect[f], 1) for f in fs}}
        for f in fs:
            resa = sparse[0.1] + rect[f] / f
            row[f"resa_r0.1_f{f}_us"] = round(resa, 1)
            row[f"rectify_share_f{f}"] = round(rect[f] / f / resa, 3)
        row["speedup_dense_over_resa_f32"] = round(dense / (sparse[0.1] + rect[32] / 32), 2)
        rows.append(row)
        print(json.dumps(row), flush=True)
        del r
        torch.cuda.empty_cache()
    cols = ["context", "dense_decode_us"] + [f"sparse_r{rv}_us" for rv in ratios] + \
           [f"rectify_f{f}_us" for f in fs] + [f"resa_r0.1_f{f}_us" for f in (32, 64)] + \
           ["rectify_share_f32", "speedup_dense_over_resa_f32"]
    print("| " + " | ".join(cols) + " |")
    print("|" + "---|" * len(cols))
    for row in rows:
        print("| " + " | ".join(str(row[c]) for c in cols) + " |")


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=256)
    ap.add_argument("--warmup", type=int, default=16)
    ap.add_argument("--workload", default="gqa_128k")
    ap.add_argument("--sweep", action="store_true",
                    help="context-length sweep at batch 1: dense / sparse / rectify breakdown (not the bench line)")
    ap.add_argument("--graph", action="store_true",
                    help="replay the timed steps from one HIP graph (no per-launch host work)")
    ap.add_argument("--unfused-append", action="store_true",
                    help="append with resa_update_descriptors, then resa_select_blocks (two calls)")
    ap.add_argument("--lanes", type=int, default=1,
                    help="cut the batch into this many sequence ranges, each issuing its calls on its own stream")
    ap.add_argument("--no-stagger", action="store_true", help="with --lanes: do not start the lanes a phase apart")
    ap.add_argument("--oracle-sweep", action="store_true",
                    help="time the CPU oracle on every workload (bounded samples; no GPU work)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=15.0)
    ap.add_argument("--copy-probe-mb", type=int, default=0,
                    help="also run one plain device copy of this many MiB (calibrates HBM byte counters)")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: the hot path here is the per-GPU kernel; "
              "sharding across GPUs is a design note, not built. Run with --gpus 1.", file=sys.stderr)
        sys.exit(2)
    if args.oracle_sweep:
        return oracle_sweep(args)

    import torch
    from block_sparse_attention_quest_amd import resa as R
    from block_sparse_attention_quest_amd import workloads as W
    from block_sparse_attention_quest_amd.schedule import ResaRunner

    torch.cuda.set_device(0)
    if args.sweep:
        return sweep(args)
    K, Wu = args.steps, args.warmup
    base = _workloads()[args.workload]()
    if args.workload.startswith("prompt"):
        return prefill_only(base, args)
    if base.steps == 0:
        return rectify_only(base, args)
    # The timed window holds whole rectification periods: any f consecutive
    # steps contain exactly one rectification, so the rate is amortised over
    # it whatever K is asked for (K is rounded up to a multiple of f).
    K_req = K
    if base.f > 0:
        K = -(-K // base.f) * base.f
    w = base.replace(steps=Wu + K + MEASURE_STEPS)
    t_setup = time.perf_counter()
    print(f"[bench] setting up {w.name}: batch {w.batch}, prefill {w.prefill_lens[0]}, steps {w.steps}",
          file=sys.stderr, flush=True)
    r = ResaRunner(w, fused_append=not args.unfused_append)
    r.fill_prefill()
    r.build_descriptors()
    rect_steps = [t for t in range(w.steps) if w.f > 0 and (t + 1) % w.f == 0]
    rect_in = {t: tuple(x.cuda() for x in W.rectify_inputs(w, t)) for t in rect_steps}
    torch.cuda.synchronize()
    print(f"[bench] setup {time.perf_counter() - t_setup:.1f}s", file=sys.stderr, flush=True)

    stream = torch.cuda.current_stream()
    if args.copy_probe_mb > 0:
        # a plain copy of known size: its FETCH_SIZE / WRITE_SIZE counters give
        # the factor between counted and actual HBM bytes on this device
        n = args.copy_probe_mb << 20
        src = torch.empty(n, dtype=torch.uint8, device="cuda").fill_(1)
        dst = torch.empty(n, dtype=torch.uint8, device="cuda")
        junk = torch.empty(512 << 20, dtype=torch.uint8, device="cuda").fill_(0)  # evict src from the caches
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst, junk

    lanes = None
    if args.lanes > 1:
        from block_sparse_attention_quest_amd.schedule import Lanes
        if w.batch % args.lanes:
            sys.exit(f"--lanes {args.lanes} does not divide the batch of {w.batch}")
        per = w.batch // args.lanes
        lanes = Lanes(r, [(i * per, (i + 1) * per) for i in range(args.lanes)], stagger=not args.no_stagger)

    def step(t):
        r.decode_step(t)
        if t in rect_in:
            r.rectify(t, *rect_in[t])

    if lanes is not None:
        lanes.fork()
        for t in range(Wu):
            lanes.step(t, rect_in)
        lanes.join()
    else:
        for t in range(Wu):
            step(t)
    torch.cuda.synchronize()

    def step_calls(t, ev=None):
        """One whole step through the C ABI. With `ev` (8 events): a pair around
        each call, and an empty pair between the calls that measures what a
        pair of event records costs on its own in the same queue."""
        r.set_step_lens(t + 1)
        q = r.step_inputs["q"][t]
        k, v = r.step_inputs["k"][t], r.step_inputs["v"][t]
        if ev is not None:
            ev[0].record(stream)
        if r.fused_append:
            R.resa_append_select(r.cache, k, v, q, r.params, r.idx, r.count, r.n_cap, r.ws)
        else:
            R.resa_update_descriptors(r.cache, k, v, 1)
            R.resa_select_blocks(r.cache, q, r.params, r.idx, r.count, r.n_cap, r.ws)
        if ev is not None:
            ev[1].record(stream)
            ev[2].record(stream)
            ev[3].record(stream)
            ev[4].record(stream)
        R.resa_sparse_decode(r.cache, q, r.idx, r.count, r.n_cap, r.out, r.ws, r.scale)
        if ev is not None:
            ev[5].record(stream)
        if t in rect_in:
            if ev is not None:
                ev[6].record(stream)
            r.rectify(t, *rect_in[t])
            if ev is not None:
                ev[7].record(stream)

    # ---- timed region: K whole steps; events only at its two ends. With
    # --graph the K steps are recorded into one HIP graph first (recording runs
    # nothing) and the timed region is its replay ----
    graph = None
    if args.graph and lanes is not None:
        # every lane's stream joins the capture through fork() and leaves it
        # through join(); the graph holds their calls as parallel branches
        graph = torch.cuda.CUDAGraph()
        cs = torch.cuda.Stream()
        cs.wait_stream(torch.cuda.current_stream())
        with torch.cuda.graph(graph, stream=cs):
            lanes.fork()
            for i in range(K):
                lanes.step(Wu + i, rect_in)
            lanes.join()
        torch.cuda.current_stream().wait_stream(cs)
        torch.cuda.synchronize()
    elif args.graph:
        graph, _, _ = r.capture(Wu, Wu + K, {t: x for t, x in rect_in.items() if Wu <= t < Wu + K})
        torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record(stream)
    if graph is not None:
        graph.replay()
    elif lanes is not None:
        lanes.fork()
        for i in range(K):
            lanes.step(Wu + i, rect_in)
        lanes.join()
    else:
        for i in range(K):
            step_calls(Wu + i)
    e1.record(stream)
    torch.cuda.synchronize()
    total_ms = e0.elapsed_time(e1)
    ms_per_step = total_ms / K
    del graph

    # ---- per-call durations: MEASURE_STEPS more steps, HIP events around every
    # call on the launch stream, queued without per-step synchronisation ----
    # A spin kernel holds the GPU while the host queues every measured step, so
    # that no call waits on its own submission (at small batch the host's
    # per-step cost exceeds the GPU's); `ahead` records whether it held long
    # enough.
    torch.cuda._sleep(QUEUE_AHEAD_CYCLES)
    held = torch.cuda.Event()
    held.record(stream)
    evs = []
    for i in range(MEASURE_STEPS):
        t = Wu + K + i
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(8)]
        step_calls(t, ev)
        evs.append((t, ev))
    ahead = not held.query()
    torch.cuda.synchronize()
    times = {"append_select": [], "decode": [], "rectify": []}
    pairs = []
    for t, ev in evs:
        times["append_select"].append(ev[0].elapsed_time(ev[1]))
        pairs.append(ev[2].elapsed_time(ev[3]))
        times["decode"].append(ev[4].elapsed_time(ev[5]))
        if t in rect_in:
            times["rectify"].append(ev[6].elapsed_time(ev[7]))
    pair_us = 1e3 * sum(pairs) / len(pairs)
    # a call's launch duration: its event-pair time less an empty pair's
    stage_us = {k: (1e3 * sum(v) / len(v) - pair_us if v else None) for k, v in times.items()}
    dec_ms = stage_us["decode"] * 1e-3
    sel_ms = stage_us["append_select"] * 1e-3

    # ---- cold-cache durations: the last step's calls again (both idempotent),
    # each after a 1 GiB read that evicts L2 and the 256 MB last-level cache
    # with clean lines (a write would leave dirty lines whose write-back then
    # competes with the timed call), so none of the step's working set is
    # cached when the call starts ----
    flush = torch.ones((1 << 30) // 4, dtype=torch.float32, device="cuda")
    sink = torch.empty(1, dtype=torch.float32, device="cuda")
    t_last = Wu + K + MEASURE_STEPS - 1
    cold_ev = []
    q_last = r.step_inputs["q"][t_last]
    k_last, v_last = r.step_inputs["k"][t_last], r.step_inputs["v"][t_last]
    r.set_step_lens(t_last + 1)
    for i in range(COLD_REPS):
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(4)]
        torch.sum(flush, dim=0, keepdim=True, out=sink)
        ev[0].record(stream)
        if r.fused_append:
            R.resa_append_select(r.cache, k_last, v_last, q_last, r.params, r.idx, r.count, r.n_cap, r.ws)
        else:
            R.resa_update_descriptors(r.cache, k_last, v_last, 1)
            R.resa_select_blocks(r.cache, q_last, r.params, r.idx, r.count, r.n_cap, r.ws)
        ev[1].record(stream)
        torch.sum(flush, dim=0, keepdim=True, out=sink)
        ev[2].record(stream)
        R.resa_sparse_decode(r.cache, q_last, r.idx, r.count, r.n_cap, r.out, r.ws, r.scale)
        ev[3].record(stream)
        cold_ev.append(ev)
    torch.cuda.synchronize()
    cold_us = {"append_select": 1e3 * sum(e[0].elapsed_time(e[1]) for e in cold_ev) / COLD_REPS - pair_us,
               "decode": 1e3 * sum(e[2].elapsed_time(e[3]) for e in cold_ev) / COLD_REPS - pair_us}
    del flush, sink

    # ---- a plain device copy of 1 GiB (read + write), this GPU's own
    # streaming reference beside the published peak ----
    src = torch.ones(1 << 30, dtype=torch.uint8, device="cuda")
    dst = torch.empty_like(src)
    times_copy = []
    for _ in range(5):
        c0, c1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        c0.record(stream)
        dst.copy_(src)
        c1.record(stream)
        c1.synchronize()
        times_copy.append(c0.elapsed_time(c1))
    copy_gbs = 2 * src.numel() / (sorted(times_copy)[2] * 1e-3) / 1e9
    del src, dst

    # ---- algorithmic work at the middle of the timed region ----
    tm = Wu + K // 2
    L_list = [L + tm + 1 for L in w.prefill_lens]
    n_list = [n_for(-(-L // 16), w) for L in L_list]
    sb = step_bytes(w, L_list, n_list)
    rkv, rflops = rectify_work(w, L_list, w.f) if w.f > 0 else (0, 0)
    full_cache = sum(w.num_kv_heads * L * 2 * w.head_dim * (2 if w.dtype == "bf16" else 4) for L in L_list)
    step_alg = sb["append"] + sb["select"] + sb["decode"] + (rkv / w.f if w.f > 0 else 0)
    # the bytes the timed window actually moved: every timed step's sparse work
    # at its own lengths, plus the rectifications that ran inside the window
    win_bytes = 0
    n_rect_win = 0
    for t in range(Wu, Wu + K):
        Lt = [L + t + 1 for L in w.prefill_lens]
        sbt = step_bytes(w, Lt, [n_for(-(-L // 16), w) for L in Lt])
        win_bytes += sbt["append"] + sbt["select"] + sbt["decode"]
        if t in rect_in:
            n_rect_win += 1
            win_bytes += rectify_work(w, Lt, w.f)[0]
    dec_gbs = sb["decode"] / (dec_ms * 1e-3) / 1e9
    sel_gbs = (sb["append"] + sb["select"]) / (sel_ms * 1e-3) / 1e9
    rect_us = stage_us["rectify"]
    rect_tflops = (rflops / (rect_us * 1e-6) / 1e12) if rect_us else None
    rect_gbs = (rkv / (rect_us * 1e-6) / 1e9) if rect_us else None

    result = {
        "metric": METRIC,
        "value": round(1e3 / ms_per_step, 2),
        "unit": "steps/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": Wu,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.dtype,
        "data": "synthetic",
        "launch": ("one HIP graph of the timed steps" if args.graph else
                   f"{args.lanes} lanes of {w.batch // args.lanes} sequences, each on its own stream"
                   f"{'' if args.no_stagger else ', a phase apart'}" if lanes is not None else
                   "calls from the host, one by one"),
        "config": {"workload": w.name, "batch": w.batch, "prefill": w.prefill_lens[0], "q_heads": w.num_q_heads,
                   "kv_heads": w.num_kv_heads, "head_dim": w.head_dim, "block": 16, "r": w.r, "n_min": w.n_min,
                   "n_local": w.n_local, "f": w.f, "parallelism": "single GPU"},
        "roofline": {"bound": "hbm", "kernel": "resa_sparse_decode (k_decode_mfma + k_decode_combine)",
                     "achieved": round(dec_gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(dec_gbs / HBM_PEAK_GBS, 4), "traffic": decode_traffic(w),
                     "alg_bytes_per_launch": sb["decode"], "avg_launch_us": round(dec_ms * 1e3, 2)},
        "steps_requested": K_req,
        "value_basis": (f"{K} timed steps = {K // w.f} whole rectification period(s) of f = {w.f}, "
                        f"{n_rect_win} rectification(s) inside the window" if w.f > 0 else
                        f"{K} timed steps, no rectification (f = 0)"),
        "hbm_gbs_step": round(win_bytes / (total_ms * 1e-3) / 1e9, 1),
        "alg_bytes_window": int(win_bytes),
        "alg_bytes_per_step": int(step_alg),
        "eq6_fraction": round(step_alg / full_cache, 5),
        "selected_kv_bytes_per_group": sb["selected_kv"] / (w.batch * w.num_kv_heads),
        "full_kv_bytes_per_group": full_cache / (w.batch * w.num_kv_heads),
        "stages_us": {k: (round(v, 2) if v is not None else None) for k, v in stage_us.items()},
        "event_pair_us": round(pair_us, 2),
        "calls_queued_ahead": ahead,
        "cold_cache_us": {k: round(v, 2) for k, v in cold_us.items()},
        "cold_decode_gbs": round(sb["decode"] / (cold_us["decode"] * 1e-6) / 1e9, 1),
        "append_select_gbs": round(sel_gbs, 1),
        "copy_1gib_gbs": round(copy_gbs, 1),
        "decode_frac_of_copy": round(dec_gbs / copy_gbs, 3),
        "decode_gbs": round(dec_gbs, 1),
        "sparse_steps_per_s": round(1e6 / (stage_us["append_select"] + stage_us["decode"]), 1),
        "rectify": {"us": rect_us and round(rect_us, 1), "tflops": rect_tflops and round(rect_tflops, 1),
                    "mfma_frac": rect_tflops and round(rect_tflops / MFMA_BF16_PEAK_TFLOPS, 4),
                    "gbs": rect_gbs and round(rect_gbs, 1)},
        "cpu_baseline": None,
    }
    if not args.no_cpu_baseline:
        print("[bench] timing the CPU oracle on a bounded sample", file=sys.stderr, flush=True)
        result["cpu_baseline"] = cpu_baseline(w, tm, args.cpu_seconds)
    print(json.dumps(result))


if __name__ == "__main__":
    main()
