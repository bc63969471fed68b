"""The C ABI on the CPU: libresa.so loads, exports every entry point that
include/resa.h declares, and rejects bad arguments on the host before any
launch (no call here reaches the GPU)."""
import ctypes
import os
import re

import pytest

from block_sparse_attention_quest_amd import resa as R

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "resa.h")


def _declared():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(resa_[a-z_]+)\s*\(", text)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(R.lib_path()):
        pytest.skip("libresa.so not built")
    return R.load()


def _cache(**kw):
    base = dict(dtype=R.RESA_BF16, batch=2, num_q_heads=8, num_kv_heads=2, head_dim=128, block_size=16,
                num_pages=64, max_blocks_per_seq=32, max_seq_len=500,
                k_pages=0x1000, v_pages=0x2000, desc=0x3000, block_table=0x4000, seq_lens=0x5000)
    base.update(kw)
    c = R.ResaCache()
    for k, v in base.items():
        setattr(c, k, v)
    return c


def test_header_declares_the_four_calls():
    names = _declared()
    for n in ("resa_update_descriptors", "resa_select_blocks", "resa_sparse_decode", "resa_rectify"):
        assert n in names
    assert set(names) == set(R.EXPORTED)


def test_library_exports_every_declared_symbol(lib):
    for name in _declared():
        assert hasattr(lib, name), name


def test_n_cap_and_sizes(lib):
    c = _cache()
    p = R.ResaSelectParams(16, 1, 0.1)
    # M = ceil(500/16) = 32 blocks, n = max(16, ceil(3.2)) = 16
    assert lib.resa_n_cap(ctypes.byref(c), ctypes.byref(p)) == 16
    assert lib.resa_select_workspace_size(ctypes.byref(c)) >= 2 * 2 * 32 * 8  # scores + control block
    assert lib.resa_decode_workspace_size(ctypes.byref(c), 16) > 0
    assert lib.resa_rectify_workspace_size(ctypes.byref(c), 32) > 0
    assert lib.resa_rectify_workspace_size(ctypes.byref(c), 1025) == 0
    # more rows than one row tile (G 4 x f 500): several tiles, more workspace
    assert lib.resa_rectify_workspace_size(ctypes.byref(c), 500) > lib.resa_rectify_workspace_size(ctypes.byref(c), 32)


@pytest.mark.parametrize("bad, status", [
    (dict(block_size=8), R.RESA_ERR_INVALID),
    (dict(num_q_heads=6, num_kv_heads=4), R.RESA_ERR_INVALID),
    (dict(num_q_heads=24, num_kv_heads=2), R.RESA_ERR_UNSUPPORTED),   # group of 12
    (dict(head_dim=96), R.RESA_ERR_UNSUPPORTED),
    (dict(dtype=7), R.RESA_ERR_INVALID),
    (dict(max_seq_len=513), R.RESA_ERR_INVALID),                        # > 32 blocks * 16
    (dict(k_pages=0), R.RESA_ERR_INVALID),
    (dict(batch=0), R.RESA_ERR_INVALID),
    (dict(max_blocks_per_seq=40000, max_seq_len=500), R.RESA_ERR_UNSUPPORTED),
])
def test_bad_cache_is_rejected_before_launch(lib, bad, status):
    c = _cache(**bad)
    st = lib.resa_update_descriptors(ctypes.byref(c), None, None, 0, None)
    assert st == status
    assert lib.resa_last_error()


def test_null_cache_and_bad_params(lib):
    assert lib.resa_update_descriptors(None, None, None, 0, None) == R.RESA_ERR_INVALID
    c = _cache()
    idx = ctypes.c_void_p(0x6000)
    for p in (R.ResaSelectParams(0, 1, 0.1), R.ResaSelectParams(16, -1, 0.1), R.ResaSelectParams(16, 1, 0.0),
              R.ResaSelectParams(16, 1, 1.5)):
        st = lib.resa_select_blocks(ctypes.byref(c), ctypes.c_void_p(0x7000), ctypes.byref(p), idx, idx, 16,
                                    ctypes.c_void_p(0x8000), 1 << 20, None)
        assert st == R.RESA_ERR_INVALID
    assert lib.resa_n_cap(ctypes.byref(c), None) == -1


def test_small_n_cap_and_workspace_are_rejected(lib):
    c = _cache()
    p = R.ResaSelectParams(16, 1, 0.1)
    buf = ctypes.c_void_p(0x9000)
    assert lib.resa_select_blocks(ctypes.byref(c), buf, ctypes.byref(p), buf, buf, 15, buf, 1 << 20,
                                  None) == R.RESA_ERR_INVALID
    assert lib.resa_select_blocks(ctypes.byref(c), buf, ctypes.byref(p), buf, buf, 16, buf, 100,
                                  None) == R.RESA_ERR_WORKSPACE
    need = lib.resa_decode_workspace_size(ctypes.byref(c), 16)
    assert lib.resa_sparse_decode(ctypes.byref(c), buf, buf, buf, 16, ctypes.c_float(0.1), buf, buf, need - 1,
                                  None) == R.RESA_ERR_WORKSPACE
    assert lib.resa_sparse_decode(ctypes.byref(c), buf, buf, buf, 16, ctypes.c_float(-1.0), buf, buf, need,
                                  None) == R.RESA_ERR_INVALID


def test_append_select_argument_checks(lib):
    c = _cache()
    p = R.ResaSelectParams(16, 1, 0.1)
    buf = ctypes.c_void_p(0xB000)
    need = lib.resa_select_workspace_size(ctypes.byref(c))

    def call(k=buf, v=buf, q=buf, params=p, n_cap=16, ws_bytes=need, cache=c):
        return lib.resa_append_select(ctypes.byref(cache) if cache is not None else None, k, v, q,
                                      ctypes.byref(params), buf, buf, n_cap, buf, ws_bytes, None)

    assert call(cache=None) == R.RESA_ERR_INVALID
    assert call(cache=_cache(block_size=8)) == R.RESA_ERR_INVALID
    assert call(v=None) == R.RESA_ERR_INVALID          # k_new without v_new
    assert call(k=None) == R.RESA_ERR_INVALID
    assert call(q=None) == R.RESA_ERR_INVALID
    assert call(params=R.ResaSelectParams(16, -1, 0.1)) == R.RESA_ERR_INVALID
    assert call(params=R.ResaSelectParams(16, 1, 0.0)) == R.RESA_ERR_INVALID
    assert call(n_cap=15) == R.RESA_ERR_INVALID
    assert call(ws_bytes=need - 1) == R.RESA_ERR_WORKSPACE
    assert lib.resa_last_error()


def test_rectify_argument_checks(lib):
    c = _cache()
    buf = ctypes.c_void_p(0xA000)
    need = lib.resa_rectify_workspace_size(ctypes.byref(c), 32)
    assert lib.resa_rectify(ctypes.byref(c), buf, buf, buf, 0, ctypes.c_float(0.1), buf, buf, need,
                            None) == R.RESA_ERR_UNSUPPORTED
    assert lib.resa_rectify(ctypes.byref(c), buf, None, buf, 32, ctypes.c_float(0.1), buf, buf, need,
                            None) == R.RESA_ERR_INVALID
    assert lib.resa_rectify(ctypes.byref(c), buf, buf, buf, 32, ctypes.c_float(0.1), buf, buf, need - 1,
                            None) == R.RESA_ERR_WORKSPACE
    assert lib.resa_rectify(ctypes.byref(c), buf, buf, buf, 1025, ctypes.c_float(0.1), buf, buf, 1 << 40,
                            None) == R.RESA_ERR_UNSUPPORTED


def test_update_descriptor_argument_checks(lib):
    c = _cache()
    buf = ctypes.c_void_p(0xB000)
    assert lib.resa_update_descriptors(ctypes.byref(c), buf, None, 1, None) == R.RESA_ERR_INVALID
    assert lib.resa_update_descriptors(ctypes.byref(c), buf, buf, 0, None) == R.RESA_ERR_INVALID
    assert lib.resa_update_descriptors(ctypes.byref(c), None, None, -1, None) == R.RESA_ERR_INVALID


def test_misaligned_pointers_are_rejected(lib):
    """Element arrays must be 16-byte aligned, integer arrays 4-byte aligned;
    the check runs on the host, so the fake addresses are never touched."""
    for bad in (dict(k_pages=0x1002), dict(v_pages=0x2008), dict(desc=0x3004), dict(block_table=0x4002),
                dict(seq_lens=0x5001)):
        assert lib.resa_update_descriptors(ctypes.byref(_cache(**bad)), None, None, 0, None) == R.RESA_ERR_INVALID
    c = _cache()
    ok, odd = ctypes.c_void_p(0xC000), ctypes.c_void_p(0xC008)
    assert lib.resa_update_descriptors(ctypes.byref(c), odd, ok, 1, None) == R.RESA_ERR_INVALID
    assert lib.resa_update_descriptors(ctypes.byref(c), ok, odd, 1, None) == R.RESA_ERR_INVALID
    p = R.ResaSelectParams(16, 1, 0.1)
    need = lib.resa_select_workspace_size(ctypes.byref(c))
    assert lib.resa_select_blocks(ctypes.byref(c), odd, ctypes.byref(p), ok, ok, 16, ok, need,
                                  None) == R.RESA_ERR_INVALID
    assert lib.resa_select_blocks(ctypes.byref(c), ok, ctypes.byref(p), ctypes.c_void_p(0xC002), ok, 16, ok, need,
                                  None) == R.RESA_ERR_INVALID
    assert lib.resa_append_select(ctypes.byref(c), odd, odd, ok, ctypes.byref(p), ok, ok, 16, ok, need,
                                  None) == R.RESA_ERR_INVALID
    need = lib.resa_decode_workspace_size(ctypes.byref(c), 16)
    assert lib.resa_sparse_decode(ctypes.byref(c), ok, ok, ok, 16, ctypes.c_float(0.1), odd, ok, need,
                                  None) == R.RESA_ERR_INVALID
    need = lib.resa_rectify_workspace_size(ctypes.byref(c), 32)
    assert lib.resa_rectify(ctypes.byref(c), ok, ok, ok, 32, ctypes.c_float(0.1), ok, odd, need,
                            None) == R.RESA_ERR_INVALID
    assert "aligned" in lib.resa_last_error().decode()


def test_cache_subset_offsets_pointers():
    """A sub-batch view keeps the pages and offsets the block-table and length
    pointers to its first sequence (no device memory is touched)."""
    class _Parent:
        batch, head_dim = 4, 128
        c = _cache(batch=4)
    sub = R.CacheSubset(_Parent, 1, 3)
    s = sub.struct
    assert (s.batch, s.k_pages, s.v_pages, s.desc) == (2, 0x1000, 0x2000, 0x3000)
    assert s.block_table == 0x4000 + 1 * 32 * 4 and s.seq_lens == 0x5000 + 4
    with pytest.raises(ValueError):
        R.CacheSubset(_Parent, 3, 5)


def test_noalloc_decode_rejects_a_configuration_beyond_its_scratch(lib):
    """The no-allocation decode refuses, on the host and before touching any
    device, a configuration whose split partials exceed its 16 MiB scratch."""
    c = _cache(batch=2048, num_q_heads=32, num_kv_heads=8)
    assert lib.resa_decode_workspace_size(ctypes.byref(c), 16) > 16 << 20
    st = lib.resa_sparse_decode_noalloc(ctypes.byref(c), ctypes.c_void_p(0x6000), ctypes.c_void_p(0x7000),
                                        ctypes.c_void_p(0x8000), 16, ctypes.c_float(0.1), ctypes.c_void_p(0x9000),
                                        None)
    assert st == R.RESA_ERR_UNSUPPORTED
    assert b"scratch" in lib.resa_last_error()
    st = lib.resa_sparse_decode_noalloc(ctypes.byref(c), None, ctypes.c_void_p(0x7000), ctypes.c_void_p(0x8000), 16,
                                        ctypes.c_float(0.1), ctypes.c_void_p(0x9000), None)
    assert st == R.RESA_ERR_INVALID


def test_size_limits_are_exact(lib):
    """The build's limits, on both sides: 32768 blocks per sequence and
    num_kv_heads * head_dim = 4096 are taken (the host-only size queries
    answer), one more block or twice the heads is not."""
    ok = _cache(max_blocks_per_seq=32768, max_seq_len=524288, num_pages=32768 * 2)
    assert lib.resa_select_workspace_size(ctypes.byref(ok)) > 0
    assert lib.resa_n_cap(ctypes.byref(ok), ctypes.byref(R.ResaSelectParams(16, 1, 0.1))) == 3277
    over = _cache(max_blocks_per_seq=32769, max_seq_len=524288, num_pages=32769 * 2)
    assert lib.resa_select_workspace_size(ctypes.byref(over)) == 0
    heads_ok = _cache(num_q_heads=32, num_kv_heads=32, head_dim=128)
    assert lib.resa_select_workspace_size(ctypes.byref(heads_ok)) > 0
    heads_over = _cache(num_q_heads=64, num_kv_heads=64, head_dim=128)
    assert lib.resa_select_workspace_size(ctypes.byref(heads_over)) == 0
    assert "4096" in lib.resa_last_error().decode()
