"""GPU: decode steps and rectifications recorded into one HIP graph replay
exactly what the same calls do eagerly, on every replay (the steps are
idempotent: a replay writes the same tokens at the same positions), with the
program's own eager work and synchronisations between replays."""
import pytest
import torch

from block_sparse_attention_quest_amd import workloads as W

pytestmark = pytest.mark.gpu


def _runner(w):
    from block_sparse_attention_quest_amd.schedule import ResaRunner
    r = ResaRunner(w)
    r.fill_prefill()
    r.build_descriptors()
    return r


def test_graph_replays_match_eager():
    w = W.Workload("graph", "bf16", 3, 8, 2, 128, (40, 513, 2000), 12, 4, 8, 0.1, 1, (0, 2, 3), True, 41)
    print(f"[case] {w.name} B={w.batch} prefill={w.prefill_lens} steps={w.steps} f={w.f}", flush=True)
    t0 = 4  # steps 0 .. 3 run eagerly first in both runners
    rect = [t for t in range(w.steps) if (t + 1) % w.f == 0]
    # eager reference
    a = _runner(w)
    ref_out, ref_rect = {}, {}
    for t in range(w.steps):
        ref_out[t] = a.decode_step(t).clone()
        if t in rect:
            ref_rect[t] = a.rectify(t, *a.rectify_inputs(t)).clone()
    torch.cuda.synchronize()
    # graph of steps t0 .. steps-1
    b = _runner(w)
    for t in range(t0):
        b.decode_step(t)
        if t in rect:
            b.rectify(t, *b.rectify_inputs(t))
    rect_in = {t: b.rectify_inputs(t) for t in rect if t >= t0}
    torch.cuda.synchronize()
    graph, outs, routs = b.capture(t0, w.steps, rect_in, keep_outputs=True)
    for rep in range(3):
        graph.replay()
        torch.cuda.synchronize()
        for t in range(t0, w.steps):
            assert torch.equal(outs[t - t0], ref_out[t]), (rep, t)
        for t, ro in routs.items():
            assert torch.equal(ro, ref_rect[t]), (rep, t)
        assert torch.equal(b.cache.desc, a.cache.desc), rep
        assert torch.equal(b.cache.k_pages, a.cache.k_pages), rep
        assert torch.equal(b.cache.v_pages, a.cache.v_pages), rep
        # the program's own eager work between replays
        junk = torch.randn(1 << 20, device="cuda")
        junk.mul_(2.0).add_(1.0)
        torch.cuda.synchronize()
    print("[result] 3 replays equal to the eager steps", flush=True)
