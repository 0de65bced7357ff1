"""Host-side checks of the C ABI that need no GPU: the library loads and exports every entry
point the header declares, the byte model agrees with the oracle's and the paper's figures,
and invalid arguments are rejected with the documented status before anything is launched."""
import ctypes
import os
import re

import numpy as np
import pytest

import oracle as O
from quantized_kv_decode_amd import loopkv as L

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def declared_symbols():
    text = open(os.path.join(ROOT, "include", "loopkv.h")).read()
    return sorted(set(re.findall(r"\b(loopkv_[a-z_]+)\s*\(", text)))


def test_library_exports_every_declared_symbol():
    names = declared_symbols()
    assert len(names) >= 8
    lib = L.lib()
    for n in names:
        assert hasattr(lib, n), n
    assert set(names) == set(L.SYMBOLS)


def shape(**kw):
    base = dict(num_layers=24, num_loops=4, page_tokens=32, v_group=128, max_batch=4,
                max_pages_per_seq=8, num_pages=32)
    base.update(kw)
    return L.make_shape(**base)


@pytest.mark.parametrize("v_group", [32, 64, 128])
@pytest.mark.parametrize("seed", [0, 1, 2])
def test_cache_bytes_matches_oracle_byte_model(v_group, seed):
    from quantized_kv_decode_amd import synth
    plan = synth.plan(24, 4, seed, 0.4)
    b = L.loopkv_cache_bytes(shape(v_group=v_group), plan)
    r = O.cache_bytes_ref(plan, 16, 128, v_group)
    assert b.stored_bytes_per_token == r["stored"]
    assert b.read_bytes_per_token_all_hot == r["read_all_hot"]
    assert b.read_bytes_per_token_hi_only == r["read_hi_only"]


def test_cache_bytes_paper_figures_with_32_channel_groups():
    s = shape(v_group=32)
    kivi4 = np.full((4, 24), L.INT4, np.uint8)
    b = L.loopkv_cache_bytes(s, kivi4)
    assert (b.stored_bytes_per_token / 1024, b.read_bytes_per_token_all_hot / 1024) == (240, 240)
    share = kivi4.copy()
    share[2] = L.REUSE
    b = L.loopkv_cache_bytes(s, share)
    assert (b.stored_bytes_per_token / 1024, b.read_bytes_per_token_all_hot / 1024) == (180, 240)
    int2 = kivi4.copy()
    int2[:3] = L.INT2
    assert L.loopkv_cache_bytes(s, int2).stored_bytes_per_token / 1024 == 168
    # skipping a token's lo plane saves half a KiB per INT4 cell
    b = L.loopkv_cache_bytes(s, kivi4)
    assert (b.read_bytes_per_token_all_hot - b.read_bytes_per_token_hi_only) / 1024 == 96 * 0.5


def test_arena_accounting():
    plan = np.array([[4, 2], [0, 4], [4, 2]], np.uint8)
    s = shape(num_layers=2, num_loops=3, num_pages=10, page_tokens=16, max_batch=3)
    b = L.loopkv_cache_bytes(s, plan)
    hb4 = O.head_block_layout(4, 16)["total"][1]
    hb2 = O.head_block_layout(2, 16)["total"][1]
    pools = [10 * 16 * hb for hb in (hb4, hb2, hb4, hb4, hb2)]
    assert b.pool_bytes == sum((p + 255) // 256 * 256 for p in pools)
    assert b.tail_bytes == 6 * 2 * ((3 * 64 * 16 * 128 * 2 + 255) // 256 * 256)
    assert b.arena_bytes == b.meta_bytes + b.workspace_bytes + b.tail_bytes + b.pool_bytes
    assert b.sink_bytes == 0
    # a 32-token sink per (cell, request), kept by reusing cells too; a window widens the ring
    s = shape(num_layers=2, num_loops=3, num_pages=10, page_tokens=16, max_batch=3,
              sink_tokens=32, window_tokens=256, tail_tokens=320)
    b2 = L.loopkv_cache_bytes(s, plan)
    assert b2.sink_bytes == 6 * 2 * ((3 * 32 * 16 * 128 * 2 + 255) // 256 * 256)
    assert b2.tail_bytes == 6 * 2 * ((3 * 320 * 16 * 128 * 2 + 255) // 256 * 256)
    assert b2.arena_bytes == b2.meta_bytes + b2.workspace_bytes + b2.tail_bytes + b2.sink_bytes + b2.pool_bytes
    assert b2.pool_bytes == b.pool_bytes


@pytest.mark.parametrize("bad,status", [
    (dict(head_dim=64), L.ENOTSUP), (dict(page_tokens=8), L.ENOTSUP), (dict(v_group=16), L.ENOTSUP),
    (dict(tail_tokens=48), L.EINVAL), (dict(tail_tokens=0), L.EINVAL), (dict(max_batch=0), L.EINVAL),
    (dict(num_pages=0), L.EINVAL), (dict(max_splits=0), L.EINVAL), (dict(num_layers=0), L.EINVAL),
    (dict(sink_tokens=16), L.EINVAL), (dict(sink_tokens=64), L.EINVAL), (dict(window_tokens=100), L.EINVAL),
    (dict(window_tokens=-32), L.EINVAL), (dict(window_tokens=256, tail_tokens=288), L.EINVAL),
])
def test_bad_shapes(bad, status):
    s = shape(**bad)
    with pytest.raises(L.LoopKVError) as e:
        L.loopkv_cache_bytes(s, np.full((s.num_loops, max(s.num_layers, 1)), 4, np.uint8))
    assert e.value.status == status


def test_gqa_not_supported():
    s = shape()
    s.num_q_heads = 8
    with pytest.raises(L.LoopKVError) as e:
        L.loopkv_cache_bytes(s, np.full((4, 24), 4, np.uint8))
    assert e.value.status == L.ENOTSUP


def test_bad_plans():
    s = shape()
    p = np.full((4, 24), 4, np.uint8)
    p[3, 5] = L.REUSE                      # REUSE in the final loop has no source
    with pytest.raises(L.LoopKVError) as e:
        L.loopkv_cache_bytes(s, p)
    assert e.value.status == L.EPLAN
    p = np.full((4, 24), 4, np.uint8)
    p[1, 1] = 3                            # unknown code
    with pytest.raises(L.LoopKVError) as e:
        L.loopkv_cache_bytes(s, p)
    assert e.value.status == L.EPLAN


def test_plan_load_validates_before_touching_the_device():
    lib = L.lib()
    s = shape()
    plan = np.full((4, 24), 4, np.uint8)
    need = L.loopkv_cache_bytes(s, plan).arena_bytes
    h = ctypes.c_void_p()
    # a fake, aligned arena address: the size check fails first, nothing is enqueued
    st = lib.loopkv_plan_load(ctypes.byref(s), plan.ctypes.data, 1 << 20, need - 1, None, ctypes.byref(h))
    assert st == L.ECAPACITY and h.value is None
    st = lib.loopkv_plan_load(ctypes.byref(s), plan.ctypes.data, (1 << 20) + 4, need, None, ctypes.byref(h))
    assert st == L.EINVAL
    st = lib.loopkv_plan_load(ctypes.byref(s), plan.ctypes.data, None, need, None, ctypes.byref(h))
    assert st == L.EINVAL
    st = lib.loopkv_plan_load(ctypes.byref(s), None, 1 << 20, need, None, ctypes.byref(h))
    assert st == L.EINVAL


def test_calls_on_null_handle_are_rejected():
    lib = L.lib()
    opts = L.DecodeOpts()
    assert lib.loopkv_decode_attention(None, 0, 0, 1, 1, 1, 1, 1, ctypes.byref(opts), 1, None) == L.EINVAL
    assert lib.loopkv_quantize_append(None, 0, 0, 1, 1, 1, 1, None, 1, 1, 1, None) == L.EINVAL
    info = L.CellInfo()
    assert lib.loopkv_get_cell_info(None, 0, 0, ctypes.byref(info)) == L.EINVAL
    v = ctypes.c_uint32()
    assert lib.loopkv_device_errors(None, None, ctypes.byref(v)) == L.EINVAL
    assert lib.loopkv_plan_free(None) == L.OK
    assert L.loopkv_status_string(L.ECAPACITY) == "insufficient capacity"
