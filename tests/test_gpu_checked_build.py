"""The checked build (libresa_debug.so, RESA_DEBUG_CHECKS) on the GPU.

On valid inputs it computes what the library computes, bit for bit. Broken
caller preconditions that the decode meets (a selected block outside the
sequence, a count above n_cap, a block-table entry outside the page pool) come
back as RESA_ERR_INVALID naming the check; these are inputs whose indices the
decode kernels clamp into their arrays in every build, so no access leaves its
buffer. (The whole GPU suite also runs against the checked build with
RESA_LIB pointing at it, on valid inputs only.)
"""
import ctypes
import os

import pytest
import torch

from block_sparse_attention_quest_amd import build as Bld
from block_sparse_attention_quest_amd import resa as R
from block_sparse_attention_quest_amd import workloads as W

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dbg():
    path = Bld.lib_path("debug_checks")
    if not os.path.exists(path):
        pytest.skip("libresa_debug.so not built")
    lib = ctypes.CDLL(path)
    vp, i32, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_size_t
    cp, pp = ctypes.POINTER(R.ResaCache), ctypes.POINTER(R.ResaSelectParams)
    lib.resa_append_select.argtypes = [cp, vp, vp, vp, pp, vp, vp, i32, vp, sz, vp]
    lib.resa_sparse_decode.argtypes = [cp, vp, vp, vp, i32, ctypes.c_float, vp, vp, sz, vp]
    lib.resa_last_error.restype = ctypes.c_char_p
    return lib


def _runner():
    from block_sparse_attention_quest_amd.schedule import ResaRunner
    w = W.Workload("checked", "bf16", 3, 8, 2, 128, (700, 2000, 333), 2, 0, 16, 0.1, 1, (2, 2, 2), True, 51)
    print(f"[case] {w.name} prefill={w.prefill_lens}", flush=True)
    r = ResaRunner(w)
    r.fill_prefill()
    r.build_descriptors()
    return w, r


def _call_decode(lib, r, cache_struct, idx, count, out):
    st = lib.resa_sparse_decode(ctypes.byref(cache_struct), r.step_inputs["q"][0].data_ptr(), idx.data_ptr(),
                                count.data_ptr(), r.n_cap, ctypes.c_float(r.scale), out.data_ptr(), r.ws.data_ptr(),
                                r.ws.numel(), torch.cuda.current_stream().cuda_stream)
    return st, lib.resa_last_error().decode()


def test_checked_build_matches_the_library(dbg):
    w, r = _runner()
    r.set_step_lens(1)
    si = r.step_inputs
    ref = r.decode_step(0).clone()  # the library: append + selection + decode
    ref_idx = r.idx.clone()
    torch.cuda.synchronize()
    # the checked build redoes the step on the same cache (the append rewrites the same token)
    idx = torch.full_like(r.idx, -1)
    count = torch.zeros_like(r.count)
    out = torch.empty_like(r.out)
    st = dbg.resa_append_select(ctypes.byref(r.cache.c), si["k"][0].data_ptr(), si["v"][0].data_ptr(),
                                si["q"][0].data_ptr(), ctypes.byref(r.params), idx.data_ptr(), count.data_ptr(),
                                r.n_cap, r.ws.data_ptr(), r.ws.numel(), torch.cuda.current_stream().cuda_stream)
    assert st == R.RESA_OK, dbg.resa_last_error()
    st, msg = _call_decode(dbg, r, r.cache.c, idx, count, out)
    assert st == R.RESA_OK, msg
    torch.cuda.synchronize()
    assert torch.equal(idx, ref_idx) and torch.equal(out, ref)


@pytest.mark.parametrize("case", ["block_outside_sequence", "count_above_n_cap", "page_outside_pool"])
def test_checked_build_reports_broken_decode_inputs(dbg, case):
    w, r = _runner()
    r.decode_step(0)
    torch.cuda.synchronize()
    idx, count = r.idx.clone(), r.count.clone()
    out = torch.empty_like(r.out)
    cache = r.cache.c
    expect = {"block_outside_sequence": "selected block", "count_above_n_cap": "count above n_cap",
              "page_outside_pool": "block_table entry"}[case]
    bt_saved = None
    if case == "block_outside_sequence":
        idx[1, 0, 3] = w.max_blocks_per_seq + 5   # past the sequence's blocks
    elif case == "count_above_n_cap":
        count[0] = r.n_cap + 7
    else:
        bt_saved = r.cache.block_table.clone()
        first = int(idx[2, 1, 0])
        r.cache.block_table[2, first] = w.num_pages + 100
    print(f"[case] checked build, {case}", flush=True)
    st, msg = _call_decode(dbg, r, cache, idx, count, out)
    if bt_saved is not None:
        r.cache.block_table.copy_(bt_saved)
    assert st == R.RESA_ERR_INVALID, (st, msg)
    assert expect in msg, msg
    # the check word was cleared: a valid call right after succeeds
    st, msg = _call_decode(dbg, r, cache, r.idx, r.count, out)
    assert st == R.RESA_OK, msg
