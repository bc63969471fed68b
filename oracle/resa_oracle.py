"""Plain CPU oracle of the ReSA hot path: TEST INFRASTRUCTURE, NOT THE PRODUCT.

Only the test suite, the package smoke check and the benchmark's CPU-baseline leg
may import this module. The HIP library never calls it and shares no code with
it; the two meet only on the seeded input tensors.

Everything is NumPy float64. Inputs given in bf16 or fp32 are widened exactly to
float64 by the caller. There is no tiling, no online softmax and no split of the
key axis: each function is the plain definition of what the method computes, or,
where the method is a heuristic (block selection), its steps in the order the
pages give them.

Sources (titles and sections of the pages this follows):
  [ABS]  "Rectified Sparse Attention" (arXiv 2506.04108), abstract on the
         Hugging Face papers page: block-sparse decoding plus a dense refresh of
         the KV cache at a fixed interval.
  [PITH] Pith review of "Rectified Sparse Attention":
         - "What carries the argument": group block-sparse attention (GBSA), in
           which each GQA group pools its queries and picks one set of blocks
           with Quest-style per-block key min/max descriptors, shared by all
           heads of the group; dense rectification re-encodes the last f
           decoded tokens every f steps, replaces their KV entries and updates
           the block statistics; n = max(n_min, ceil(M p)) blocks are attended.
         - Referee report, major comment 1 (quoting the paper's Eq. 5 and
           Eq. 6): the count rule, and the per-step memory-access fraction
           1/b + p + 1/f with the ambiguity of p (active vs. sparsity ratio).
         - Referee report, minor comment 3 (quoting the paper's Eq. 2): the
           mask is block-granular, a key k is attended iff its block floor(k/b)
           is selected.
         - "Assumptions & free parameters": f = 32, b = 16, n_min = 16,
           n_local = 1 (recent blocks always kept), p = 0.9 (ambiguous).
         - "The reading": rectification rebuilds the cache exactly.
  The upper-bound score is the Quest form sum_c max(q_c kmin_c, q_c kmax_c); the
  pages name it only as "Quest-style" (reference [23] of the Pith reference list).

Readings where the pages are silent (each is listed in the design notes):
  * p is taken as an explicit active-block ratio r: n = min(M, max(n_min, ceil(M r))),
    computed in IEEE double.
  * Pooling is the arithmetic mean of the group's query vectors, summed in head
    order in float64, then divided by the group size.
  * The n_local newest blocks (the partial current block included) are always
    selected and count toward n; ties in score go to the lower block index.
  * A partial last block's descriptor covers its valid tokens only.
  * The newest token is in the cache before selection, so it attends to itself.
  * Attention scale 1/sqrt(d), max-subtracted softmax, no sink or bias.
  * Rectification: the caller supplies the corrected K/V of the f newest
    positions; they overwrite the cache, the touched blocks' descriptors are
    recomputed, and row i (position L - f + i) attends causally to positions
    0 .. L - f + i of the updated cache.
"""
from __future__ import annotations

import math
from typing import Dict, List, Optional, Sequence, Tuple

import numpy as np

BLOCK = 16

# Defaults the Pith review lists under "Assumptions & free parameters".
DEFAULTS = {"block_size": 16, "f": 32, "n_min": 16, "n_local": 1, "p": 0.9}


# ---------------------------------------------------------------------------
# Per-(sequence, KV head) definitions
# ---------------------------------------------------------------------------

def num_blocks(seq_len: int) -> int:
    """M = ceil(L / b)."""
    return -(-int(seq_len) // BLOCK)


def block_descriptors(k_seq: np.ndarray) -> Tuple[np.ndarray, np.ndarray]:
    """Quest-style block statistics [PITH "What carries the argument"].

    k_seq: [L][d] keys of one sequence and KV head. Returns (kmin, kmax), each
    [M][d]: the channel-wise minimum and maximum over the valid tokens of each
    block of 16 (the last block may be partial).
    """
    L, d = k_seq.shape
    M = num_blocks(L)
    kmin = np.empty((M, d))
    kmax = np.empty((M, d))
    for j in range(M):
        tile = k_seq[j * BLOCK:min(L, (j + 1) * BLOCK)]
        kmin[j] = tile.min(axis=0)
        kmax[j] = tile.max(axis=0)
    return kmin, kmax


def active_block_count(M: int, n_min: int, r: float) -> int:
    """Eq. 5 [PITH referee major 1] with p read as the active ratio r,
    n = max(n_min, ceil(M r)), never more than the M blocks that exist."""
    return min(int(M), max(int(n_min), math.ceil(float(M) * float(r))))


def pooled_query(q_group: np.ndarray) -> np.ndarray:
    """GBSA query pooling [PITH "What carries the argument"]: the mean of the
    group's G query vectors, summed in head order, then divided by G."""
    acc = np.array(q_group[0], dtype=np.float64)
    for h in range(1, q_group.shape[0]):
        acc = acc + q_group[h]
    return acc / q_group.shape[0]


def block_upper_bounds(q_bar: np.ndarray, kmin: np.ndarray, kmax: np.ndarray) -> np.ndarray:
    """Quest upper bound of q.k over each block: s_j = sum_c max(q_c kmin_jc, q_c kmax_jc)."""
    return np.maximum(q_bar[None, :] * kmin, q_bar[None, :] * kmax).sum(axis=1)


def select_blocks(scores: np.ndarray, n: int, n_local: int) -> np.ndarray:
    """GBSA selection [PITH "What carries the argument", "Assumptions"]:
    keep the n_local newest blocks, fill the remaining n - n_local places with
    the highest-scoring other blocks (ties: lower index first), and return the
    set sorted ascending."""
    M = len(scores)
    n = min(n, M)
    keep_local = min(n_local, n)
    local = list(range(M - keep_local, M))
    others = [j for j in range(M - keep_local)]
    others.sort(key=lambda j: (-scores[j], j))
    chosen = local + others[:n - keep_local]
    return np.array(sorted(chosen), dtype=np.int64)


def block_tokens(blocks: Sequence[int], seq_len: int) -> np.ndarray:
    """Eq. 2 [PITH referee minor 3]: the positions attended when `blocks` are
    selected, i.e. every valid token k with floor(k / b) in the set."""
    toks = [np.arange(j * BLOCK, min(seq_len, (j + 1) * BLOCK)) for j in blocks]
    return np.concatenate(toks) if toks else np.zeros(0, dtype=np.int64)


def attention(q: np.ndarray, k: np.ndarray, v: np.ndarray, scale: float) -> np.ndarray:
    """softmax(q k^T * scale) v for q [R][d], k, v [T][d]; max-subtracted."""
    logits = (q @ k.T) * scale
    logits = logits - logits.max(axis=1, keepdims=True)
    w = np.exp(logits)
    return (w @ v) / w.sum(axis=1, keepdims=True)


def sparse_decode_group(q_group: np.ndarray, k_seq: np.ndarray, v_seq: np.ndarray,
                        blocks: Sequence[int], scale: float) -> np.ndarray:
    """One decode token of every head in a GQA group attending to the group's
    selected blocks only: [G][d]."""
    toks = block_tokens(blocks, k_seq.shape[0])
    return attention(q_group, k_seq[toks], v_seq[toks], scale)


def causal_rows(q_rows: np.ndarray, k_seq: np.ndarray, v_seq: np.ndarray,
                first_pos: int, scale: float) -> np.ndarray:
    """Dense causal attention of rows at positions first_pos + i over the cache:
    row i sees positions 0 .. first_pos + i. q_rows [f][d] -> [f][d]."""
    out = np.empty_like(q_rows, dtype=np.float64)
    for i in range(q_rows.shape[0]):
        P = first_pos + i
        out[i] = attention(q_rows[i:i + 1], k_seq[:P + 1], v_seq[:P + 1], scale)[0]
    return out


def memory_fraction(b: int, active: float, f: float) -> float:
    """Eq. 6 [PITH "Core claim", referee major 1]: per-step share of the cache
    read, 1/b (descriptors) + active share (selected KV) + 1/f (amortized
    rectification)."""
    return 1.0 / b + active + (0.0 if not f else 1.0 / f)


# ---------------------------------------------------------------------------
# A paged cache and the batched steps
# ---------------------------------------------------------------------------

class PagedCache:
    """The oracle's own paged KV cache in float64.

    k_pages, v_pages: [P][Hkv][16][d]; desc: [P][Hkv][2][d] (0 = min, 1 = max);
    block_table: [B][max_blocks] page ids; seq_lens: [B] tokens held.
    """

    def __init__(self, k_pages, v_pages, desc, block_table, seq_lens):
        self.k = np.array(k_pages, dtype=np.float64)
        self.v = np.array(v_pages, dtype=np.float64)
        self.desc = np.array(desc, dtype=np.float64)
        self.block_table = np.array(block_table, dtype=np.int64)
        self.seq_lens = [int(x) for x in seq_lens]

    @property
    def num_kv_heads(self) -> int:
        return self.k.shape[1]

    def _pages(self, b: int, L: int) -> np.ndarray:
        return self.block_table[b, :num_blocks(L)]

    def seq(self, b: int, hkv: int, which: str = "k") -> np.ndarray:
        """Tokens 0..L-1 of sequence b, KV head hkv, gathered through the block table."""
        L = self.seq_lens[b]
        pool = self.k if which == "k" else self.v
        return pool[self._pages(b, L), hkv].reshape(-1, pool.shape[-1])[:L]

    def write(self, b: int, pos: int, k_row: np.ndarray, v_row: np.ndarray) -> None:
        """Store the K/V of token `pos` (all KV heads, [Hkv][d])."""
        page = self.block_table[b, pos // BLOCK]
        self.k[page, :, pos % BLOCK] = k_row
        self.v[page, :, pos % BLOCK] = v_row

    def refresh(self, b: int, first_pos: int, last_pos: int) -> None:
        """Recompute the descriptors of every block holding a position in
        [first_pos, last_pos) of sequence b."""
        L = self.seq_lens[b]
        for j in range(max(0, first_pos) // BLOCK, num_blocks(min(L, last_pos))):
            page = self.block_table[b, j]
            valid = min(L, (j + 1) * BLOCK) - j * BLOCK
            for hkv in range(self.num_kv_heads):
                kmin, kmax = block_descriptors(self.k[page, hkv, :valid])
                self.desc[page, hkv, 0] = kmin[0]
                self.desc[page, hkv, 1] = kmax[0]

    def rebuild(self) -> None:
        for b in range(len(self.seq_lens)):
            self.refresh(b, 0, self.seq_lens[b])


def append(cache: PagedCache, k_new: np.ndarray, v_new: np.ndarray) -> None:
    """Decode-step append: token L_b of every sequence gets k_new[b], v_new[b]
    ([B][Hkv][d]), L_b grows by one and the descriptor of its block is updated."""
    for b in range(len(cache.seq_lens)):
        pos = cache.seq_lens[b]
        cache.seq_lens[b] = pos + 1
        cache.write(b, pos, k_new[b], v_new[b])
        cache.refresh(b, pos, pos + 1)


def select(cache: PagedCache, q: np.ndarray, n_min: int, r: float, n_local: int
           ) -> Tuple[List[List[np.ndarray]], List[int], List[List[np.ndarray]]]:
    """GBSA selection for every (sequence, group). q: [B][Hq][d].
    Returns (idx[b][g] sorted arrays, n[b], scores[b][g])."""
    B, Hq, _ = q.shape
    Hkv = cache.num_kv_heads
    G = Hq // Hkv
    idx, counts, scores = [], [], []
    for b in range(B):
        L = cache.seq_lens[b]
        M = num_blocks(L)
        n = active_block_count(M, n_min, r)
        counts.append(n)
        row_i, row_s = [], []
        for g in range(Hkv):
            pages = cache.block_table[b, :M]
            kmin = cache.desc[pages, g, 0]
            kmax = cache.desc[pages, g, 1]
            s = block_upper_bounds(pooled_query(q[b, g * G:(g + 1) * G]), kmin, kmax)
            row_s.append(s)
            row_i.append(select_blocks(s, n, n_local))
        idx.append(row_i)
        scores.append(row_s)
    return idx, counts, scores


def decode(cache: PagedCache, q: np.ndarray, idx: List[List[Sequence[int]]], scale: float) -> np.ndarray:
    """Sparse decode of one token per head. q [B][Hq][d] -> out [B][Hq][d]."""
    B, Hq, d = q.shape
    Hkv = cache.num_kv_heads
    G = Hq // Hkv
    out = np.empty((B, Hq, d))
    for b in range(B):
        for g in range(Hkv):
            out[b, g * G:(g + 1) * G] = sparse_decode_group(
                q[b, g * G:(g + 1) * G], cache.seq(b, g, "k"), cache.seq(b, g, "v"), idx[b][g], scale)
    return out


def rectify(cache: PagedCache, q: np.ndarray, k_new: np.ndarray, v_new: np.ndarray,
            scale: float) -> np.ndarray:
    """Dense rectification [PITH "What carries the argument", "The reading"].

    q [B][f][Hq][d]; k_new, v_new [B][f][Hkv][d] are the re-encoded K/V of the f
    newest positions [L_b - f, L_b). They overwrite the cache, the touched
    blocks' descriptors are recomputed, then row i of every head attends
    causally over the updated cache. Returns [B][f][Hq][d].
    """
    B, f, Hq, d = q.shape
    Hkv = cache.num_kv_heads
    G = Hq // Hkv
    out = np.empty((B, f, Hq, d))
    for b in range(B):
        L = cache.seq_lens[b]
        for i in range(f):
            cache.write(b, L - f + i, k_new[b, i], v_new[b, i])
        cache.refresh(b, L - f, L)
        for h in range(Hq):
            g = h // G
            out[b, :, h] = causal_rows(q[b, :, h], cache.seq(b, g, "k"), cache.seq(b, g, "v"), L - f, scale)
    return out


def dense_decode(cache: PagedCache, q: np.ndarray, scale: float) -> np.ndarray:
    """Dense decoding baseline: every head attends to every cached token."""
    B, Hq, d = q.shape
    G = Hq // cache.num_kv_heads
    out = np.empty((B, Hq, d))
    for b in range(B):
        for h in range(Hq):
            out[b, h] = attention(q[b, h:h + 1], cache.seq(b, h // G, "k"), cache.seq(b, h // G, "v"), scale)[0]
    return out


def resa_loop(cache: PagedCache, steps: int, f: int, n_min: int, r: float, n_local: int, scale: float,
              step_inputs, rectify_inputs=None, on_step=None) -> Dict[str, list]:
    """The ReSA generation schedule [ABS; PITH "What carries the argument"]:
    every decode step appends its token, updates that block's descriptor,
    selects blocks and decodes sparsely; after every f-th step the f newest
    tokens are rectified. f <= 0 means never (plain sparse decoding).

    step_inputs(t) -> (q [B][Hq][d], k [B][Hkv][d], v [B][Hkv][d]);
    rectify_inputs(t) -> (q [B][f][Hq][d], k, v [B][f][Hkv][d]).
    """
    outs, rect_outs, idxs = [], [], []
    for t in range(steps):
        q, k, v = step_inputs(t)
        append(cache, k, v)
        idx, _, _ = select(cache, q, n_min, r, n_local)
        o = decode(cache, q, idx, scale)
        outs.append(o)
        idxs.append(idx)
        if on_step is not None:
            on_step(t, cache, o, idx)
        if f > 0 and (t + 1) % f == 0:
            rq, rk, rv = rectify_inputs(t)
            rect_outs.append(rectify(cache, rq, rk, rv, scale))
    return {"out": outs, "idx": idxs, "rectify_out": rect_outs}
