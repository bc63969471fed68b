"""Thin ctypes binding over libresa.so (include/resa.h).

Argument marshalling only: every step of the hot path runs in the library's HIP
kernels. torch supplies device memory and the current stream. There is no CPU
fallback: if the library is missing, loading it raises.
"""
from __future__ import annotations

import ctypes
import math
import os
from typing import Optional

import torch

_LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libresa.so")
_lib = None

RESA_OK, RESA_ERR_INVALID, RESA_ERR_UNSUPPORTED, RESA_ERR_WORKSPACE, RESA_ERR_HIP = range(5)
RESA_FP32, RESA_BF16 = 0, 1
_STATUS = {0: "RESA_OK", 1: "RESA_ERR_INVALID", 2: "RESA_ERR_UNSUPPORTED",
           3: "RESA_ERR_WORKSPACE", 4: "RESA_ERR_HIP"}
EXPORTED = ("resa_n_cap", "resa_select_workspace_size", "resa_decode_workspace_size",
            "resa_rectify_workspace_size", "resa_update_descriptors", "resa_select_blocks",
            "resa_append_select", "resa_sparse_decode", "resa_sparse_decode_noalloc", "resa_rectify",
            "resa_last_error")


class ResaError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(f"{_STATUS.get(status, status)}: {msg}")
        self.status = status


class ResaCache(ctypes.Structure):
    _fields_ = [("dtype", ctypes.c_int32), ("batch", ctypes.c_int32),
                ("num_q_heads", ctypes.c_int32), ("num_kv_heads", ctypes.c_int32),
                ("head_dim", ctypes.c_int32), ("block_size", ctypes.c_int32),
                ("num_pages", ctypes.c_int32), ("max_blocks_per_seq", ctypes.c_int32),
                ("max_seq_len", ctypes.c_int32),
                ("k_pages", ctypes.c_void_p), ("v_pages", ctypes.c_void_p), ("desc", ctypes.c_void_p),
                ("block_table", ctypes.c_void_p), ("seq_lens", ctypes.c_void_p)]


class ResaSelectParams(ctypes.Structure):
    _fields_ = [("n_min", ctypes.c_int32), ("n_local", ctypes.c_int32), ("r", ctypes.c_double)]


def lib_path() -> str:
    return _LIB_PATH


def load(path: Optional[str] = None) -> ctypes.CDLL:
    """Load libresa.so (once; the RESA_LIB environment variable may name
    another build of it, e.g. the checked build). Raises if it has not been
    built."""
    global _lib
    if _lib is not None:
        return _lib
    p = path or os.environ.get("RESA_LIB") or _LIB_PATH
    if not os.path.exists(p):
        raise RuntimeError(f"{p} is missing: build it with `python -m block_sparse_attention_quest_amd.build`")
    lib = ctypes.CDLL(p)
    vp, i32, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_size_t
    cp, pp = ctypes.POINTER(ResaCache), ctypes.POINTER(ResaSelectParams)
    lib.resa_n_cap.argtypes, lib.resa_n_cap.restype = [cp, pp], i32
    lib.resa_select_workspace_size.argtypes, lib.resa_select_workspace_size.restype = [cp], sz
    lib.resa_decode_workspace_size.argtypes, lib.resa_decode_workspace_size.restype = [cp, i32], sz
    lib.resa_rectify_workspace_size.argtypes, lib.resa_rectify_workspace_size.restype = [cp, i32], sz
    lib.resa_update_descriptors.argtypes, lib.resa_update_descriptors.restype = [cp, vp, vp, i32, vp], i32
    lib.resa_select_blocks.argtypes = [cp, vp, pp, vp, vp, i32, vp, sz, vp]
    lib.resa_select_blocks.restype = i32
    lib.resa_append_select.argtypes = [cp, vp, vp, vp, pp, vp, vp, i32, vp, sz, vp]
    lib.resa_append_select.restype = i32
    lib.resa_sparse_decode.argtypes = [cp, vp, vp, vp, i32, ctypes.c_float, vp, vp, sz, vp]
    lib.resa_sparse_decode.restype = i32
    lib.resa_sparse_decode_noalloc.argtypes = [cp, vp, vp, vp, i32, ctypes.c_float, vp, vp]
    lib.resa_sparse_decode_noalloc.restype = i32
    lib.resa_rectify.argtypes = [cp, vp, vp, vp, i32, ctypes.c_float, vp, vp, sz, vp]
    lib.resa_rectify.restype = i32
    lib.resa_last_error.argtypes, lib.resa_last_error.restype = [], ctypes.c_char_p
    _lib = lib
    return lib


def _check(status: int) -> None:
    if status != RESA_OK:
        raise ResaError(status, load().resa_last_error().decode())


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream) -> ctypes.c_void_p:
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


class PagedKVCache:
    """Device buffers of the paged cache plus the resa_cache descriptor that
    points at them (all allocated with torch on the current device)."""

    def __init__(self, batch: int, num_q_heads: int, num_kv_heads: int, head_dim: int, num_pages: int,
                 max_blocks_per_seq: int, max_seq_len: int, dtype: torch.dtype = torch.bfloat16,
                 device="cuda"):
        self.dtype = dtype
        self.k_pages = torch.zeros(num_pages, num_kv_heads, 16, head_dim, dtype=dtype, device=device)
        # V pages are channel-major inside a page: [page][head][channel][slot]
        self.v_pages = torch.zeros(num_pages, num_kv_heads, head_dim, 16, dtype=dtype, device=device)
        self.desc = torch.zeros(num_pages, num_kv_heads, 2, head_dim, dtype=dtype, device=device)
        self.block_table = torch.zeros(batch, max_blocks_per_seq, dtype=torch.int32, device=device)
        self.seq_lens = torch.zeros(batch, dtype=torch.int32, device=device)
        self.batch, self.num_q_heads, self.num_kv_heads, self.head_dim = batch, num_q_heads, num_kv_heads, head_dim
        self.num_pages, self.max_blocks_per_seq, self.max_seq_len = num_pages, max_blocks_per_seq, max_seq_len
        self.refresh_struct()

    def refresh_struct(self) -> None:
        self.c = ResaCache(RESA_BF16 if self.dtype == torch.bfloat16 else RESA_FP32, self.batch, self.num_q_heads,
                           self.num_kv_heads, self.head_dim, 16, self.num_pages, self.max_blocks_per_seq,
                           self.max_seq_len, self.k_pages.data_ptr(), self.v_pages.data_ptr(),
                           self.desc.data_ptr(), self.block_table.data_ptr(), self.seq_lens.data_ptr())

    @property
    def struct(self) -> ResaCache:
        return self.c


class CacheSubset:
    """The cache descriptor of the contiguous sequences [b0, b1) of a
    PagedKVCache: the same pages, that range's block-table rows and lengths
    (pointer offsets into the parent's arrays, taken from the parent's current
    descriptor at every use). Any call can run on it, e.g. a rectification of
    the sequences that are due while the others keep decoding."""

    def __init__(self, cache: PagedKVCache, b0: int, b1: int):
        if not 0 <= b0 < b1 <= cache.batch:
            raise ValueError(f"sequence range [{b0}, {b1}) outside the batch of {cache.batch}")
        self.parent, self.b0, self.b1 = cache, b0, b1
        self.batch = b1 - b0
        self.head_dim = cache.head_dim

    @property
    def struct(self) -> ResaCache:
        c = self.parent.c
        return ResaCache(c.dtype, self.batch, c.num_q_heads, c.num_kv_heads, c.head_dim, c.block_size, c.num_pages,
                         c.max_blocks_per_seq, c.max_seq_len, c.k_pages, c.v_pages, c.desc,
                         c.block_table + self.b0 * c.max_blocks_per_seq * 4, c.seq_lens + self.b0 * 4)


def make_params(n_min: int, r: float, n_local: int) -> ResaSelectParams:
    return ResaSelectParams(int(n_min), int(n_local), float(r))


# ----------------------------------------------------------------------------
# The four calls (same names as the C ABI) and the size queries
# ----------------------------------------------------------------------------

def resa_n_cap(cache: PagedKVCache, params: ResaSelectParams) -> int:
    n = load().resa_n_cap(ctypes.byref(cache.struct), ctypes.byref(params))
    if n < 0:
        raise ResaError(RESA_ERR_INVALID, load().resa_last_error().decode())
    return int(n)


def resa_select_workspace_size(cache: PagedKVCache) -> int:
    return int(load().resa_select_workspace_size(ctypes.byref(cache.struct)))


def resa_decode_workspace_size(cache: PagedKVCache, n_cap: int) -> int:
    return int(load().resa_decode_workspace_size(ctypes.byref(cache.struct), int(n_cap)))


def resa_rectify_workspace_size(cache: PagedKVCache, f: int) -> int:
    return int(load().resa_rectify_workspace_size(ctypes.byref(cache.struct), int(f)))


def resa_update_descriptors(cache: PagedKVCache, k_new: Optional[torch.Tensor], v_new: Optional[torch.Tensor],
                            n_new: int, stream=None) -> None:
    _check(load().resa_update_descriptors(ctypes.byref(cache.struct), _ptr(k_new), _ptr(v_new), int(n_new),
                                          _stream(stream)))


def resa_select_blocks(cache: PagedKVCache, q: torch.Tensor, params: ResaSelectParams, idx: torch.Tensor,
                       count: torch.Tensor, n_cap: int, ws: torch.Tensor, stream=None) -> None:
    _check(load().resa_select_blocks(ctypes.byref(cache.struct), _ptr(q), ctypes.byref(params), _ptr(idx),
                                     _ptr(count), int(n_cap), _ptr(ws), ws.numel() * ws.element_size(),
                                     _stream(stream)))


def resa_append_select(cache: PagedKVCache, k_new: Optional[torch.Tensor], v_new: Optional[torch.Tensor],
                       q: torch.Tensor, params: ResaSelectParams, idx: torch.Tensor, count: torch.Tensor, n_cap: int,
                       ws: torch.Tensor, stream=None) -> None:
    _check(load().resa_append_select(ctypes.byref(cache.struct), _ptr(k_new), _ptr(v_new), _ptr(q),
                                     ctypes.byref(params), _ptr(idx), _ptr(count), int(n_cap), _ptr(ws),
                                     ws.numel() * ws.element_size(), _stream(stream)))


def resa_sparse_decode(cache: PagedKVCache, q: torch.Tensor, idx: torch.Tensor, count: torch.Tensor, n_cap: int,
                       out: torch.Tensor, ws: torch.Tensor, scale: Optional[float] = None, stream=None) -> None:
    scale = 1.0 / math.sqrt(cache.head_dim) if scale is None else scale
    _check(load().resa_sparse_decode(ctypes.byref(cache.struct), _ptr(q), _ptr(idx), _ptr(count), int(n_cap),
                                     ctypes.c_float(scale), _ptr(out), _ptr(ws), ws.numel() * ws.element_size(),
                                     _stream(stream)))


def resa_sparse_decode_noalloc(cache: PagedKVCache, q: torch.Tensor, idx: torch.Tensor, count: torch.Tensor,
                               n_cap: int, out: torch.Tensor, scale: Optional[float] = None, stream=None) -> None:
    scale = 1.0 / math.sqrt(cache.head_dim) if scale is None else scale
    _check(load().resa_sparse_decode_noalloc(ctypes.byref(cache.struct), _ptr(q), _ptr(idx), _ptr(count), int(n_cap),
                                             ctypes.c_float(scale), _ptr(out), _stream(stream)))


def resa_rectify(cache: PagedKVCache, q: torch.Tensor, k_new: torch.Tensor, v_new: torch.Tensor, f: int,
                 out: torch.Tensor, ws: torch.Tensor, scale: Optional[float] = None, stream=None) -> None:
    scale = 1.0 / math.sqrt(cache.head_dim) if scale is None else scale
    _check(load().resa_rectify(ctypes.byref(cache.struct), _ptr(q), _ptr(k_new), _ptr(v_new), int(f),
                               ctypes.c_float(scale), _ptr(out), _ptr(ws), ws.numel() * ws.element_size(),
                               _stream(stream)))


def workspace(nbytes: int, device="cuda") -> torch.Tensor:
    """A workspace for the calls (contents on entry do not matter)."""
    return torch.empty(max(int(nbytes), 256), dtype=torch.uint8, device=device)
