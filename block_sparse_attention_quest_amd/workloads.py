"""Seeded synthetic inputs for the ReSA decode / rectify hot path.

This module only draws random numbers and lays them out. It holds none of the
method's arithmetic (no descriptors, scores, selection or attention), so that the
CPU oracle and the HIP path can both consume its tensors without sharing code.

Every tensor is drawn on the CPU from ``torch.Generator`` seeded by a digest of
(workload seed, tag, indices). Any piece (one sequence's keys for one KV head,
one step's queries) can therefore be regenerated on its own, which lets the
full-size parity tests check sampled groups without materialising the whole
cache on the host.

Distributions (stated once here, restated in the design notes):
  * q ~ N(0, 1).
  * K, V ~ N(0, 1) * s_c, where s_c ~ LogNormal(0, 0.5) per (KV head, channel),
    drawn independently for K and V and shared over batch and tokens
    ("outlier channels"). The tiny fp32 case uses s_c = 1.
  * Planted blocks: every key of a planted block gets ``+ 2 * u`` with u the
    unit vector of the mean of the group's step-0 queries (added after the
    channel scaling). Indices are drawn from the seed among the non-final
    prefill blocks.
  * Decode-step K/V rows are drawn like prefill rows.
  * Rectified K/V (the dense re-encoding of the last f tokens, which a model's
    lower layers would produce) are the sparse-phase rows plus
    ``0.05 * N(0, 1) * s_c``; rectify queries are fresh N(0, 1) draws.
  * Block tables are a seeded permutation of the physical page pool, so the
    selected blocks of one sequence are scattered through HBM as in a paged
    serving cache.
  All draws are fp32 and then cast round-to-nearest-even to the workload dtype.
"""
from __future__ import annotations

import dataclasses
import hashlib
import math
from typing import List, Optional, Sequence, Tuple

import torch

BLOCK = 16


def _gen(seed: int, *tags) -> torch.Generator:
    h = hashlib.blake2b(repr((int(seed),) + tuple(tags)).encode(), digest_size=8)
    g = torch.Generator(device="cpu")
    g.manual_seed(int.from_bytes(h.digest(), "little") & ((1 << 63) - 1))
    return g


def _randn(shape, seed, *tags) -> torch.Tensor:
    return torch.randn(*shape, generator=_gen(seed, *tags), dtype=torch.float32)


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    dtype: str                      # "fp32" | "bf16"
    batch: int
    num_q_heads: int
    num_kv_heads: int
    head_dim: int
    prefill_lens: Tuple[int, ...]   # tokens in the cache before the first decode step
    steps: int                      # decode steps
    f: int                          # rectification period (0 = never)
    n_min: int
    r: float
    n_local: int
    planted: Tuple[int, ...]        # planted blocks per sequence (same for every group)
    channel_scale: bool
    seed: int

    @property
    def group(self) -> int:
        return self.num_q_heads // self.num_kv_heads

    @property
    def torch_dtype(self) -> torch.dtype:
        return torch.float32 if self.dtype == "fp32" else torch.bfloat16

    @property
    def max_seq_len(self) -> int:
        # a rectify-only workload (no decode steps) grows by its f rectified tokens
        return max(self.prefill_lens) + (self.steps if self.steps > 0 else max(self.f, 0))

    @property
    def max_blocks_per_seq(self) -> int:
        return -(-self.max_seq_len // BLOCK)

    @property
    def num_pages(self) -> int:
        return self.batch * self.max_blocks_per_seq

    def replace(self, **kw) -> "Workload":
        return dataclasses.replace(self, **kw)


def _planted_count(prefill_len: int, frac: float, fixed: Optional[int]) -> int:
    if fixed is not None:
        return fixed
    return int(round(frac * (-(-prefill_len // BLOCK))))


def tiny_fp32(**kw) -> Workload:
    """Batch 1, one GQA group of 4 query heads, d 64, 1024-token prefill, fp32."""
    w = Workload("tiny_fp32_b1_h4kv1_d64_1k", "fp32", 1, 4, 1, 64, (1024,), 64, 32,
                 4, 0.125, 1, (3,), False, 0)
    return w.replace(**kw) if kw else w


def llama8b_32k(**kw) -> Workload:
    """Batch 8, 32 query heads over 8 KV heads, d 128, 32K prefill, bf16."""
    L = 32768
    w = Workload("gqa32x8_d128_bf16_b8_32k", "bf16", 8, 32, 8, 128, (L,) * 8, 256, 32,
                 16, 0.1, 1, (_planted_count(L, 0.01, None),) * 8, True, 1)
    return w.replace(**kw) if kw else w


def gqa_128k(**kw) -> Workload:
    """Batch 4, 32q/8kv, d 128, 128K prefill, bf16: the headline decode workload."""
    L = 131072
    w = Workload("gqa32x8_d128_bf16_b4_128k", "bf16", 4, 32, 8, 128, (L,) * 4, 256, 32,
                 16, 0.1, 1, (_planted_count(L, 0.01, None),) * 4, True, 2)
    return w.replace(**kw) if kw else w


def long_256k(**kw) -> Workload:
    """Batch 1, 32q/8kv, d 128, 256K prefill, bf16, 512 decode steps."""
    L = 262144
    w = Workload("gqa32x8_d128_bf16_b1_256k", "bf16", 1, 32, 8, 128, (L,), 512, 32,
                 16, 0.1, 1, (_planted_count(L, 0.01, None),), True, 3)
    return w.replace(**kw) if kw else w


def longest(**kw) -> Workload:
    """Batch 1, 32q/8kv, d 128, bf16, at the longest context the library takes:
    a 524,256-token prefill and 32 decode steps end at 524,288 tokens, 32,768
    blocks (f 32: the rectification after the last step covers the final 32)."""
    L = 524288 - 32
    w = Workload("gqa32x8_d128_bf16_b1_512k", "bf16", 1, 32, 8, 128, (L,), 32, 32,
                 16, 0.1, 1, (_planted_count(L, 0.01, None),), True, 5)
    return w.replace(**kw) if kw else w


def rectify_mixed(**kw) -> Workload:
    """16 sequences, total lengths U{4096..65536} (including the f=64 rectified
    tokens), 32q/8kv, d 128, bf16; one rectification of 64 tokens each."""
    seed = kw.get("seed", 4)
    n = kw.get("batch", 16)
    f = kw.get("f", 64)
    lo, hi = kw.pop("len_range", (4096, 65536))
    g = _gen(seed, "lengths")
    lens = torch.randint(lo, hi + 1, (n,), generator=g).tolist()
    w = Workload("gqa32x8_d128_bf16_b16_mixed4k-64k_f64", "bf16", n, 32, 8, 128,
                 tuple(int(x) - f for x in lens), 0, f, 16, 0.1, 1, (0,) * n, True, seed)
    kw.pop("batch", None)
    kw.pop("f", None)
    return w.replace(**kw) if kw else w


# ----------------------------------------------------------------------------
# Draws
# ----------------------------------------------------------------------------

def channel_scales(w: Workload) -> Tuple[torch.Tensor, torch.Tensor]:
    """(s_k, s_v), each fp32 [Hkv][d]."""
    shape = (w.num_kv_heads, w.head_dim)
    if not w.channel_scale:
        return torch.ones(shape), torch.ones(shape)
    sk = torch.exp(0.5 * _randn(shape, w.seed, "scale", "k"))
    sv = torch.exp(0.5 * _randn(shape, w.seed, "scale", "v"))
    return sk, sv


def query(w: Workload, step: int) -> torch.Tensor:
    """Decode query of step ``step`` (0-based): [B][Hq][d] in the workload dtype."""
    return _randn((w.batch, w.num_q_heads, w.head_dim), w.seed, "q", step).to(w.torch_dtype)


def planted_blocks(w: Workload, b: int) -> List[int]:
    """Sorted planted block indices of sequence b (shared by its KV heads)."""
    n = w.planted[b]
    m0 = -(-w.prefill_lens[b] // BLOCK)
    if n <= 0 or m0 < 2:
        return []
    perm = torch.randperm(m0 - 1, generator=_gen(w.seed, "plant", b))
    return sorted(perm[:n].tolist())


def _plant_direction(w: Workload, b: int, hkv: int) -> torch.Tensor:
    q0 = query(w, 0)[b, hkv * w.group:(hkv + 1) * w.group].float()
    u = q0.mean(dim=0)
    return u / u.norm()


def prefill_kv(w: Workload, b: int, hkv: int) -> Tuple[torch.Tensor, torch.Tensor]:
    """Prefill keys and values of sequence b, KV head hkv: each [L0][d]."""
    L0, d = w.prefill_lens[b], w.head_dim
    sk, sv = channel_scales(w)
    k = _randn((L0, d), w.seed, "prefill_k", b, hkv) * sk[hkv]
    v = _randn((L0, d), w.seed, "prefill_v", b, hkv) * sv[hkv]
    blocks = planted_blocks(w, b)
    if blocks:
        u = _plant_direction(w, b, hkv)
        for j in blocks:
            k[j * BLOCK:(j + 1) * BLOCK] += 2.0 * u
    return k.to(w.torch_dtype), v.to(w.torch_dtype)


def _append_f32(w: Workload, step: int) -> Tuple[torch.Tensor, torch.Tensor]:
    shape = (w.batch, w.num_kv_heads, w.head_dim)
    sk, sv = channel_scales(w)
    return _randn(shape, w.seed, "new_k", step) * sk, _randn(shape, w.seed, "new_v", step) * sv


def append_kv(w: Workload, step: int) -> Tuple[torch.Tensor, torch.Tensor]:
    """K/V rows appended at decode step ``step``: each [B][Hkv][d]."""
    k, v = _append_f32(w, step)
    return k.to(w.torch_dtype), v.to(w.torch_dtype)


def rectify_inputs(w: Workload, end_step: int) -> Tuple[torch.Tensor, torch.Tensor, torch.Tensor]:
    """Inputs of the rectification that follows decode step ``end_step`` (0-based,
    (end_step + 1) % f == 0): queries [B][f][Hq][d] and corrected K/V
    [B][f][Hkv][d] for the f most recent tokens of every sequence."""
    f = w.f
    sk, sv = channel_scales(w)
    ks, vs = [], []
    for i in range(f):
        step = end_step - f + 1 + i
        if step < 0:
            raise ValueError("a rectification needs f decode steps before it")
        k, v = append_kv(w, step)
        ks.append(k.float())
        vs.append(v.float())
    k = torch.stack(ks, dim=1)
    v = torch.stack(vs, dim=1)
    shape = (w.batch, f, w.num_kv_heads, w.head_dim)
    k = k + 0.05 * _randn(shape, w.seed, "drift_k", end_step) * sk
    v = v + 0.05 * _randn(shape, w.seed, "drift_v", end_step) * sv
    q = _randn((w.batch, f, w.num_q_heads, w.head_dim), w.seed, "rq", end_step)
    return q.to(w.torch_dtype), k.to(w.torch_dtype), v.to(w.torch_dtype)


def rectify_only_inputs(w: Workload) -> Tuple[torch.Tensor, torch.Tensor, torch.Tensor]:
    """For a rectify-only workload (``steps == 0``): queries [B][f][Hq][d] and
    the K/V of the f newest tokens [B][f][Hkv][d] (fresh draws with drift)."""
    f = w.f
    sk, sv = channel_scales(w)
    shape = (w.batch, f, w.num_kv_heads, w.head_dim)
    k = (_randn(shape, w.seed, "tail_k") + 0.05 * _randn(shape, w.seed, "drift_k", -1)) * sk
    v = (_randn(shape, w.seed, "tail_v") + 0.05 * _randn(shape, w.seed, "drift_v", -1)) * sv
    q = _randn((w.batch, f, w.num_q_heads, w.head_dim), w.seed, "rq", -1)
    return q.to(w.torch_dtype), k.to(w.torch_dtype), v.to(w.torch_dtype)


def prompt_inputs(w: Workload) -> Tuple[torch.Tensor, torch.Tensor, torch.Tensor]:
    """Prompt of a prefill workload (every sequence prefill_lens[0] tokens):
    queries [B][T][Hq][d] ~ N(0, 1) and the prompt K/V [B][T][Hkv][d], the same
    draws as prefill_kv, so a chunked prefill leaves the cache that fill-in
    would have written."""
    T = w.prefill_lens[0]
    if any(L != T for L in w.prefill_lens):
        raise ValueError("a prefill workload holds equal-length prompts")
    q = _randn((w.batch, T, w.num_q_heads, w.head_dim), w.seed, "prompt_q")
    ks, vs = [], []
    for b in range(w.batch):
        kv = [prefill_kv(w, b, h) for h in range(w.num_kv_heads)]
        ks.append(torch.stack([k for k, _ in kv], dim=1))
        vs.append(torch.stack([v for _, v in kv], dim=1))
    return q.to(w.torch_dtype), torch.stack(ks), torch.stack(vs)


def prompt_32k(**kw) -> Workload:
    """Chunked prefill of one 32768-token prompt, 32q/8kv, d 128, bf16, in
    chunks of f positions (64 unless given)."""
    f = kw.pop("f", 64)
    w = Workload(f"gqa32x8_d128_bf16_b1_prompt32k_chunk{f}", "bf16", 1, 32, 8, 128, (32768,), 0, f, 16, 0.1, 1,
                 (0,), True, 7)
    return w.replace(**kw) if kw else w


def block_table(w: Workload) -> torch.Tensor:
    """[B][max_blocks_per_seq] int32: a seeded permutation of the page pool."""
    perm = torch.randperm(w.num_pages, generator=_gen(w.seed, "block_table"))
    return perm.to(torch.int32).view(w.batch, w.max_blocks_per_seq).contiguous()


def rectify_steps(w: Workload) -> List[int]:
    """0-based decode steps after which a rectification runs."""
    if w.f <= 0:
        return []
    return [t for t in range(w.steps) if (t + 1) % w.f == 0]
