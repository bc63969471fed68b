"""The ReSA generation schedule on the GPU (host side).

"Rectified Sparse Attention" (abstract; Pith review, "What carries the argument"
and Figure 2): after prefill the cache descriptors are built once; every decode
step appends its token (and updates that block's descriptor), selects blocks
per GQA group and decodes sparsely; after every f-th step the f newest tokens
are rectified densely. This module only orders the library calls and owns the
device buffers; every step of the computation runs in libresa's kernels.

Per-step sequence lengths are laid out up front as one small device table, and
the cache descriptor handed to the library points at the row of the current
step, so a decode step launches nothing but the library's own kernels.
"""
from __future__ import annotations

import math
from typing import Dict, Optional

import torch

from . import resa as R
from . import workloads as W


class ResaRunner:
    def __init__(self, w: W.Workload, device="cuda", steps: Optional[int] = None, inputs_on_device: bool = True,
                 fused_append: bool = True):
        self.w = w
        # one call appends the step's token and selects (resa_append_select)
        # instead of resa_update_descriptors followed by resa_select_blocks
        self.fused_append = fused_append
        self.device = device
        self.steps = w.steps if steps is None else steps
        B, Hq, Hkv, d = w.batch, w.num_q_heads, w.num_kv_heads, w.head_dim
        self.cache = R.PagedKVCache(B, Hq, Hkv, d, w.num_pages, w.max_blocks_per_seq, w.max_seq_len,
                                    dtype=w.torch_dtype, device=device)
        self.block_table_cpu = W.block_table(w)
        self.cache.block_table.copy_(self.block_table_cpu)
        # seq_lens of the prefill (row 0) and after each decode step (row t + 1)
        if self.steps > 0:
            rows = [[L + t for L in w.prefill_lens] for t in range(self.steps + 1)]
        else:  # rectify-only workload: row 1 holds the lengths with the f rectified tokens
            rows = [list(w.prefill_lens), [L + max(w.f, 0) for L in w.prefill_lens]]
        lens = torch.tensor(rows, dtype=torch.int32)
        self.lens = lens.to(device)
        self.params = R.make_params(w.n_min, w.r, w.n_local)
        self.set_step_lens(0)
        self.n_cap = R.resa_n_cap(self.cache, self.params)
        ws = max(R.resa_select_workspace_size(self.cache),
                 R.resa_decode_workspace_size(self.cache, self.n_cap),
                 R.resa_rectify_workspace_size(self.cache, w.f) if w.f > 0 else 0)
        self.ws = R.workspace(ws, device)
        self.idx = torch.full((B, Hkv, self.n_cap), -1, dtype=torch.int32, device=device)
        self.count = torch.zeros(B, dtype=torch.int32, device=device)
        self.out = torch.empty(B, Hq, d, dtype=w.torch_dtype, device=device)
        self.rect_out = torch.empty(B, max(w.f, 1), Hq, d, dtype=w.torch_dtype, device=device)
        self.scale = 1.0 / math.sqrt(d)
        self.step_inputs: Dict[str, torch.Tensor] = {}
        if inputs_on_device and self.steps > 0:
            self.step_inputs = {
                "q": torch.stack([W.query(w, t) for t in range(self.steps)]).to(device),
                "k": torch.stack([W.append_kv(w, t)[0] for t in range(self.steps)]).unsqueeze(2).to(device),
                "v": torch.stack([W.append_kv(w, t)[1] for t in range(self.steps)]).unsqueeze(2).to(device),
            }
        self.rect_inputs: Dict[int, tuple] = {}

    # -- layout ------------------------------------------------------------
    def set_step_lens(self, row: int) -> None:
        """Point the cache descriptor at the sequence lengths after `row` steps."""
        self.cache.c.seq_lens = self.lens[row].data_ptr()
        self.cache.seq_lens = self.lens[row]

    def fill_prefill(self) -> None:
        """Write the seeded prefill K/V into their pages (plumbing, not timed)."""
        w, c = self.w, self.cache
        bt = self.block_table_cpu
        for b in range(w.batch):
            L = w.prefill_lens[b]
            M = -(-L // 16)
            pages = bt[b, :M].to(self.device, torch.long)
            for h in range(w.num_kv_heads):
                k, v = W.prefill_kv(w, b, h)
                pad = M * 16 - L
                if pad:
                    k = torch.cat([k, torch.zeros(pad, w.head_dim, dtype=k.dtype)])
                    v = torch.cat([v, torch.zeros(pad, w.head_dim, dtype=v.dtype)])
                c.k_pages[pages, h] = k.view(M, 16, w.head_dim).to(self.device)
                # V tiles are stored channel-major: [page][head][channel][slot]
                c.v_pages[pages, h] = v.view(M, 16, w.head_dim).transpose(1, 2).contiguous().to(self.device)

    # -- the hot path -------------------------------------------------------
    def build_descriptors(self) -> None:
        self.set_step_lens(0)
        R.resa_update_descriptors(self.cache, None, None, 0)

    def decode_step(self, t: int, q=None, k=None, v=None) -> torch.Tensor:
        """Decode step t (0-based): append + descriptor, select, sparse decode."""
        self.set_step_lens(t + 1)
        si = self.step_inputs
        q = si["q"][t] if q is None else q
        k = si["k"][t] if k is None else k
        v = si["v"][t] if v is None else v
        if self.fused_append:
            R.resa_append_select(self.cache, k, v, q, self.params, self.idx, self.count, self.n_cap, self.ws)
        else:
            R.resa_update_descriptors(self.cache, k, v, 1)
            R.resa_select_blocks(self.cache, q, self.params, self.idx, self.count, self.n_cap, self.ws)
        R.resa_sparse_decode(self.cache, q, self.idx, self.count, self.n_cap, self.out, self.ws, self.scale)
        return self.out

    def rectify(self, t: int, q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, f: Optional[int] = None) -> torch.Tensor:
        """Rectify the f newest tokens after decode step t (lengths of row t + 1)."""
        f = self.w.f if f is None else f
        self.set_step_lens(t + 1)
        out = self.rect_out[:, :f]
        if f != self.rect_out.shape[1]:
            out = torch.empty(self.w.batch, f, self.w.num_q_heads, self.w.head_dim, dtype=self.w.torch_dtype,
                              device=self.device)
        R.resa_rectify(self.cache, q, k, v, f, out, self.ws, self.scale)
        return out

    def rectify_subset(self, t: int, b0: int, b1: int, q: torch.Tensor, k: torch.Tensor, v: torch.Tensor,
                       f: Optional[int] = None) -> torch.Tensor:
        """Rectify only sequences [b0, b1) after decode step t (the others
        keep their sparse-phase rows); q [b1-b0][f][Hq][d], k, v [b1-b0][f][Hkv][d]."""
        f = self.w.f if f is None else f
        self.set_step_lens(t + 1)
        out = torch.empty(b1 - b0, f, self.w.num_q_heads, self.w.head_dim, dtype=self.w.torch_dtype,
                          device=self.device)
        R.resa_rectify(R.CacheSubset(self.cache, b0, b1), q, k, v, f, out, self.ws, self.scale)
        return out

    def rectify_only(self) -> torch.Tensor:
        """Rectify-only workload: the f newest tokens of every sequence (beyond the
        prefill) are written, their blocks refreshed, and their rows attended."""
        q, k, v = (x.to(self.device) for x in W.rectify_only_inputs(self.w))
        self.rect_inputs[-1] = (q, k, v)
        return self.rectify(0, q, k, v)

    def rectify_inputs(self, t: int):
        if t not in self.rect_inputs:
            self.rect_inputs[t] = tuple(x.to(self.device) for x in W.rectify_inputs(self.w, t))
        return self.rect_inputs[t]

    def capture(self, t0: int, t1: int, rect_in: Optional[Dict[int, tuple]] = None,
                keep_outputs: bool = False):
        """Record decode steps t0 .. t1-1 (and, from `rect_in`, the
        rectification after each step listed there) into one HIP graph, so a
        replay issues them with no per-launch host work. Every call in the
        steps launches kernels only (no allocation, no memset), so the graph
        replays them exactly. With keep_outputs each step's output (and each
        rectification's) is also copied into a buffer of its own inside the
        graph; returns (graph, step outputs, rectify outputs)."""
        rect_in = rect_in or {}
        outs = torch.empty(t1 - t0, *self.out.shape, dtype=self.out.dtype, device=self.device) if keep_outputs else None
        routs: Dict[int, torch.Tensor] = {}
        stream = torch.cuda.Stream()
        stream.wait_stream(torch.cuda.current_stream())
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph, stream=stream):
            for t in range(t0, t1):
                o = self.decode_step(t)
                if keep_outputs:
                    outs[t - t0].copy_(o)
                if t in rect_in:
                    ro = self.rectify(t, *rect_in[t])
                    if keep_outputs:
                        routs[t] = ro.clone()
        torch.cuda.current_stream().wait_stream(stream)
        return graph, outs, routs

    def run(self, steps: Optional[int] = None, on_step=None, on_rectify=None) -> None:
        """The full schedule: every step, then a rectification after each f-th."""
        steps = self.steps if steps is None else steps
        for t in range(steps):
            o = self.decode_step(t)
            if on_step is not None:
                on_step(t, o)
            if self.w.f > 0 and (t + 1) % self.w.f == 0:
                ro = self.rectify(t, *self.rectify_inputs(t))
                if on_rectify is not None:
                    on_rectify(t, ro)


class Lanes:
    """The batch of a ResaRunner cut into contiguous sequence ranges ("lanes"),
    each issuing its calls on a HIP stream of its own, with its own workspace
    and its slices of the runner's index, count and output buffers.

    Sequences are independent within one attention layer, so the lanes'
    kernels may run at the same time. What that buys is overlap of unlike
    work: the top-n selection and the merge of the decode splits are
    latency-bound (few workgroups, dependent steps), the scoring and the
    sparse decode stream HBM. With `stagger`, lane i's append + selection
    of a step starts after lane i - 1's has finished, so the lanes run a phase
    apart and one lane's latency-bound kernels run under another's streaming
    ones. `phases` gives each lane its own rectification phase (continuous
    batching: lane i rectifies after step t when (t + 1 + phases[i]) % f == 0
    and t >= f - 1), so one lane's rectification overlaps the other lanes'
    decode steps.

    Host work per call is kept small: the calls go straight to the C ABI
    with argument lists prepared at construction (pointers of every step's
    inputs), since at batch sizes where a step takes tens of microseconds the
    host issues several calls per step.
    """

    def __init__(self, runner: "ResaRunner", ranges, stagger: bool = True, phases=None):
        import ctypes
        self.r = runner
        self.ranges = [(int(a), int(b)) for a, b in ranges]
        bs = [x for rg in self.ranges for x in range(*rg)]
        if bs != list(range(runner.w.batch)):
            raise ValueError(f"lanes {self.ranges} must cut the batch 0 .. {runner.w.batch} into contiguous ranges")
        self.stagger = stagger
        self.phases = list(phases) if phases is not None else [0] * len(self.ranges)
        w, c = runner.w, runner.cache
        self.lib = R.load()
        self.streams = [torch.cuda.Stream(device=runner.device) for _ in self.ranges]
        self.events = [torch.cuda.Event() for _ in self.ranges]
        self.views = [R.CacheSubset(c, b0, b1) for b0, b1 in self.ranges]
        self.structs = [v.struct for v in self.views]
        self.ws = []
        for v in self.views:
            n = max(R.resa_select_workspace_size(v), R.resa_decode_workspace_size(v, runner.n_cap),
                    R.resa_rectify_workspace_size(v, w.f) if w.f > 0 else 0)
            self.ws.append(R.workspace(n, runner.device))
        self.scale = ctypes.c_float(runner.scale)
        self.params = ctypes.byref(runner.params)
        self.rect_outs = [torch.empty(b1 - b0, max(w.f, 1), w.num_q_heads, w.head_dim, dtype=w.torch_dtype,
                                      device=runner.device) for b0, b1 in self.ranges]
        si = runner.step_inputs
        self.args = []  # per lane: per step (k, v, q) pointers, then the fixed pointers
        for (b0, b1), ws in zip(self.ranges, self.ws):
            steps = [(si["k"][t][b0:b1].data_ptr(), si["v"][t][b0:b1].data_ptr(), si["q"][t][b0:b1].data_ptr())
                     for t in range(runner.steps)] if si else []
            self.args.append({"steps": steps, "idx": runner.idx[b0:b1].data_ptr(),
                              "count": runner.count[b0:b1].data_ptr(), "out": runner.out[b0:b1].data_ptr(),
                              "ws": ws.data_ptr(), "ws_bytes": ws.numel()})

    def _check(self, st):
        if st != R.RESA_OK:
            raise R.ResaError(st, self.lib.resa_last_error().decode())

    def fork(self) -> None:
        """Every lane stream waits for the work queued so far on the current stream."""
        cur = torch.cuda.current_stream()
        for s in self.streams:
            s.wait_stream(cur)

    def join(self) -> None:
        """The current stream waits for every lane."""
        cur = torch.cuda.current_stream()
        for s in self.streams:
            cur.wait_stream(s)

    def due(self, i: int, t: int) -> bool:
        f = self.r.w.f
        return f > 0 and t >= f - 1 and (t + 1 + self.phases[i]) % f == 0

    def step(self, t: int, rect_in: Optional[Dict[int, tuple]] = None, keep=None) -> None:
        """Decode step t on every lane (append + selection, then the sparse
        decode), then the rectification of the lanes that are due, using
        rect_in[t] = (q, k, v) of the whole batch (sliced per lane). With
        `keep`, a callable (lane, t, out, rect_out) is run on the lane's stream
        after its calls (e.g. copies of the outputs)."""
        import ctypes
        r, lib = self.r, self.lib
        lens = r.lens[t + 1].data_ptr()
        for i, ((b0, b1), st, a, s) in enumerate(zip(self.ranges, self.structs, self.args, self.streams)):
            st.seq_lens = lens + 4 * b0
            if self.stagger and i > 0:
                s.wait_event(self.events[i - 1])
            k, v, q = a["steps"][t]
            self._check(lib.resa_append_select(ctypes.byref(st), k, v, q, self.params, a["idx"], a["count"], r.n_cap,
                                               a["ws"], a["ws_bytes"], s.cuda_stream))
            if self.stagger:
                self.events[i].record(s)
        for i, ((b0, b1), st, a, s) in enumerate(zip(self.ranges, self.structs, self.args, self.streams)):
            q = a["steps"][t][2]
            self._check(lib.resa_sparse_decode(ctypes.byref(st), q, a["idx"], a["count"], r.n_cap, self.scale,
                                               a["out"], a["ws"], a["ws_bytes"], s.cuda_stream))
            rout = None
            if rect_in is not None and self.due(i, t):
                rq, rk, rv = (x[b0:b1] for x in rect_in[t])
                rout = self.rect_outs[i]
                self._check(lib.resa_rectify(ctypes.byref(st), rq.data_ptr(), rk.data_ptr(), rv.data_ptr(), r.w.f,
                                             self.scale, rout.data_ptr(), a["ws"], a["ws_bytes"], s.cuda_stream))
            if keep is not None:
                with torch.cuda.stream(s):
                    keep(i, t, r.out[b0:b1], rout)


class ChunkedPrefill:
    """Dense causal prefill through the rectification call ("Rectified Sparse
    Attention": rectification re-encodes recent tokens with the dense pass;
    prefill is that pass over the whole prompt). An equal-length batch of
    T-token prompts goes through resa_rectify in chunks of at most `chunk`
    (<= 1024) positions: each call writes its chunk's K/V into the pages,
    refreshes the touched blocks' descriptors (so the whole cache's descriptors
    are built when the last chunk lands) and returns the chunk's causal
    attention rows. Prompts of different lengths are prefilled per length.
    """

    def __init__(self, w: W.Workload, chunk: Optional[int] = None, device="cuda"):
        self.w = w
        self.device = device
        self.chunk = w.f if chunk is None else chunk
        B, Hq, Hkv, d = w.batch, w.num_q_heads, w.num_kv_heads, w.head_dim
        self.T = w.prefill_lens[0]
        if any(L != self.T for L in w.prefill_lens):
            raise ValueError("ChunkedPrefill takes prompts of one length")
        self.cache = R.PagedKVCache(B, Hq, Hkv, d, w.num_pages, w.max_blocks_per_seq, w.max_seq_len,
                                    dtype=w.torch_dtype, device=device)
        self.cache.block_table.copy_(W.block_table(w))
        self.chunks = [(c0, min(self.chunk, self.T - c0)) for c0 in range(0, self.T, self.chunk)]
        # sequence lengths once chunk i is in: one device row per chunk
        self.lens = torch.tensor([[c0 + fc] * B for c0, fc in self.chunks], dtype=torch.int32, device=device)
        self.cache.c.seq_lens = self.lens[0].data_ptr()
        self.ws = R.workspace(R.resa_rectify_workspace_size(self.cache, self.chunk), device)
        self.scale = 1.0 / math.sqrt(d)
        self.inputs = []
        self.outs = []

    def stage(self, q: torch.Tensor, k: torch.Tensor, v: torch.Tensor) -> None:
        """Chunk-major device copies of the prompt ([B][T][H][d] each): every
        chunk's rows contiguous as the call expects."""
        self.inputs = [tuple(x[:, c0:c0 + fc].contiguous().to(self.device) for x in (q, k, v))
                       for c0, fc in self.chunks]
        self.outs = [torch.empty(self.w.batch, fc, self.w.num_q_heads, self.w.head_dim, dtype=self.w.torch_dtype,
                                 device=self.device) for _, fc in self.chunks]

    def run(self, stream=None):
        """Every chunk in order; returns the per-chunk outputs [B][fc][Hq][d]."""
        for i, (c0, fc) in enumerate(self.chunks):
            self.cache.c.seq_lens = self.lens[i].data_ptr()
            qc, kc, vc = self.inputs[i]
            R.resa_rectify(self.cache, qc, kc, vc, fc, self.outs[i], self.ws, self.scale, stream=stream)
        return self.outs

    def output(self) -> torch.Tensor:
        """The prompt's attention outputs [B][T][Hq][d]."""
        return torch.cat(self.outs, dim=1)
