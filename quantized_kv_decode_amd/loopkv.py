"""ctypes binding of libloopkv (include/loopkv.h): the same entry points, argument marshalling
only. Every step of the path runs in the library's HIP kernels; PyTorch supplies device
memory and streams. Importing this module does not load the library; the first call does,
and raises if libloopkv.so has not been built (there is no fallback)."""
from __future__ import annotations

import ctypes
import os

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
# The in-tree build; LOOPKV_LIBRARY names another build of the same library (e.g. one compiled
# with different launch parameters) to load instead.
LIB_PATH = os.environ.get("LOOPKV_LIBRARY") or os.path.join(HERE, "libloopkv.so")

REUSE, INT2, INT4 = 0, 2, 4
SPLIT_AUTO = -1
OK, EINVAL, EPLAN, ENOTSUP, ECAPACITY, EHIP, EINFEASIBLE = range(7)
ERR_LENGTH, ERR_PAGE, ERR_TAIL = 1, 2, 4


class Shape(ctypes.Structure):
    _fields_ = [("num_layers", ctypes.c_int32), ("num_loops", ctypes.c_int32),
                ("num_kv_heads", ctypes.c_int32), ("num_q_heads", ctypes.c_int32),
                ("head_dim", ctypes.c_int32), ("page_tokens", ctypes.c_int32),
                ("v_group", ctypes.c_int32), ("max_batch", ctypes.c_int32),
                ("max_pages_per_seq", ctypes.c_int32), ("tail_tokens", ctypes.c_int32),
                ("max_splits", ctypes.c_int32), ("sink_tokens", ctypes.c_int32),
                ("window_tokens", ctypes.c_int32), ("reserved", ctypes.c_int32),
                ("num_pages", ctypes.c_int64)]


class Bytes(ctypes.Structure):
    _fields_ = [("arena_bytes", ctypes.c_uint64), ("pool_bytes", ctypes.c_uint64),
                ("tail_bytes", ctypes.c_uint64), ("meta_bytes", ctypes.c_uint64),
                ("workspace_bytes", ctypes.c_uint64),
                ("stored_bytes_per_token", ctypes.c_double),
                ("read_bytes_per_token_hi_only", ctypes.c_double),
                ("read_bytes_per_token_all_hot", ctypes.c_double),
                ("sink_bytes", ctypes.c_uint64)]


class DecodeOpts(ctypes.Structure):
    _fields_ = [("tau", ctypes.c_float), ("sm_scale", ctypes.c_float),
                ("split_tokens", ctypes.c_int32), ("mask_stride", ctypes.c_int32),
                ("seed_dev", ctypes.c_void_p), ("fetch_mask_dev", ctypes.c_void_p),
                ("stats_dev", ctypes.c_void_p), ("no_sink_seed", ctypes.c_int32)]


class CellInfo(ctypes.Structure):
    _fields_ = [("code", ctypes.c_int32), ("read_bits", ctypes.c_int32),
                ("gated", ctypes.c_int32), ("head_block_bytes", ctypes.c_int32),
                ("page_bytes", ctypes.c_int64), ("read_pool_dev", ctypes.c_void_p),
                ("own_pool_dev", ctypes.c_void_p), ("tail_k_dev", ctypes.c_void_p),
                ("tail_v_dev", ctypes.c_void_p), ("qgroups_dev", ctypes.c_void_p),
                ("sink_k_dev", ctypes.c_void_p), ("sink_v_dev", ctypes.c_void_p)]


class PlanBudget(ctypes.Structure):
    _fields_ = [("max_damage", ctypes.c_double), ("max_stored_bytes", ctypes.c_double),
                ("hot_fraction", ctypes.c_double)]


class PlanCost(ctypes.Structure):
    _fields_ = [("damage", ctypes.c_double), ("stored_bytes_per_token", ctypes.c_double),
                ("read_bytes_per_token", ctypes.c_double)]


SYMBOLS = ["loopkv_cache_bytes", "loopkv_plan_load", "loopkv_plan_free",
           "loopkv_quantize_append", "loopkv_decode_attention", "loopkv_get_cell_info",
           "loopkv_device_errors", "loopkv_plan_solve", "loopkv_auto_split",
           "loopkv_decode_attention_static",
           "loopkv_status_string"]

_lib = None


def lib() -> ctypes.CDLL:
    """Loads libloopkv.so once; raises if it is missing."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is not built; run quantized_kv_decode_amd.build.build()")
        L = ctypes.CDLL(LIB_PATH)
        vp, i32, u64 = ctypes.c_void_p, ctypes.c_int32, ctypes.c_uint64
        L.loopkv_cache_bytes.argtypes = [ctypes.POINTER(Shape), vp, ctypes.POINTER(Bytes)]
        L.loopkv_plan_load.argtypes = [ctypes.POINTER(Shape), vp, vp, u64, vp, ctypes.POINTER(vp)]
        L.loopkv_plan_free.argtypes = [vp]
        L.loopkv_quantize_append.argtypes = [vp, i32, i32, vp, vp, i32, i32, vp, vp, vp, i32, vp]
        L.loopkv_decode_attention.argtypes = [vp, i32, i32, vp, i32, vp, vp, i32,
                                              ctypes.POINTER(DecodeOpts), vp, vp]
        L.loopkv_get_cell_info.argtypes = [vp, i32, i32, ctypes.POINTER(CellInfo)]
        L.loopkv_device_errors.argtypes = [vp, vp, ctypes.POINTER(ctypes.c_uint32)]
        L.loopkv_plan_solve.argtypes = [ctypes.POINTER(Shape), vp, ctypes.POINTER(PlanBudget), vp,
                                        ctypes.POINTER(PlanCost)]
        L.loopkv_auto_split.argtypes = [vp, i32, i32, ctypes.POINTER(ctypes.c_int32)]
        L.loopkv_decode_attention_static.argtypes = L.loopkv_decode_attention.argtypes
        L.loopkv_status_string.argtypes = [ctypes.c_int]
        L.loopkv_status_string.restype = ctypes.c_char_p
        for name in SYMBOLS:
            if name != "loopkv_status_string":
                getattr(L, name).restype = ctypes.c_int
        _lib = L
    return _lib


class LoopKVError(RuntimeError):
    def __init__(self, status: int, what: str):
        self.status = status
        super().__init__(f"{what}: {loopkv_status_string(status)} ({status})")


def _check(status: int, what: str) -> None:
    if status != OK:
        raise LoopKVError(status, what)


def _u8(plan) -> np.ndarray:
    return np.ascontiguousarray(np.asarray(plan, dtype=np.uint8).reshape(-1))


def loopkv_status_string(status: int) -> str:
    return lib().loopkv_status_string(int(status)).decode()


def loopkv_cache_bytes(shape: Shape, plan) -> Bytes:
    p = _u8(plan)
    out = Bytes()
    _check(lib().loopkv_cache_bytes(ctypes.byref(shape), p.ctypes.data, ctypes.byref(out)),
           "loopkv_cache_bytes")
    return out


def loopkv_plan_load(shape: Shape, plan, arena_dev: int, arena_bytes: int, stream: int) -> int:
    p = _u8(plan)
    h = ctypes.c_void_p()
    _check(lib().loopkv_plan_load(ctypes.byref(shape), p.ctypes.data, arena_dev, arena_bytes,
                                  stream, ctypes.byref(h)), "loopkv_plan_load")
    return h.value


def loopkv_plan_free(handle: int) -> None:
    _check(lib().loopkv_plan_free(handle), "loopkv_plan_free")


def loopkv_quantize_append(handle, layer, loop, k_new_dev, v_new_dev, batch, n_new, n_new_dev,
                           seq_lens_dev, page_table_dev, page_table_stride, stream) -> None:
    _check(lib().loopkv_quantize_append(handle, layer, loop, k_new_dev, v_new_dev, batch, n_new,
                                        n_new_dev, seq_lens_dev, page_table_dev, page_table_stride,
                                        stream), "loopkv_quantize_append")


def loopkv_decode_attention(handle, layer, loop, q_dev, batch, seq_lens_dev, page_table_dev,
                            page_table_stride, opts: DecodeOpts | None, out_dev, stream) -> None:
    _check(lib().loopkv_decode_attention(handle, layer, loop, q_dev, batch, seq_lens_dev,
                                         page_table_dev, page_table_stride,
                                         ctypes.byref(opts) if opts is not None else None,
                                         out_dev, stream), "loopkv_decode_attention")


def loopkv_decode_attention_static(handle, layer, loop, q_dev, batch, seq_lens_dev, page_table_dev,
                                   page_table_stride, opts: DecodeOpts | None, out_dev, stream) -> None:
    _check(lib().loopkv_decode_attention_static(handle, layer, loop, q_dev, batch, seq_lens_dev,
                                                page_table_dev, page_table_stride,
                                                ctypes.byref(opts) if opts is not None else None,
                                                out_dev, stream), "loopkv_decode_attention_static")


def loopkv_auto_split(handle, batch, page_table_stride) -> int:
    v = ctypes.c_int32()
    _check(lib().loopkv_auto_split(handle, batch, page_table_stride, ctypes.byref(v)), "loopkv_auto_split")
    return v.value


def loopkv_get_cell_info(handle, layer, loop) -> CellInfo:
    out = CellInfo()
    _check(lib().loopkv_get_cell_info(handle, layer, loop, ctypes.byref(out)), "loopkv_get_cell_info")
    return out


def loopkv_device_errors(handle, stream) -> int:
    v = ctypes.c_uint32()
    _check(lib().loopkv_device_errors(handle, stream, ctypes.byref(v)), "loopkv_device_errors")
    return v.value


def loopkv_plan_solve(shape: Shape, damage, max_damage: float = -1.0, max_stored_bytes: float = 0.0,
                      hot_fraction: float = 1.0):
    """damage: float64 [num_loops, num_layers, 3] (INT4, INT2, REUSE). Returns (plan uint8
    [num_loops, num_layers], PlanCost)."""
    d = np.ascontiguousarray(np.asarray(damage, dtype=np.float64))
    assert d.shape == (shape.num_loops, shape.num_layers, 3)
    plan = np.zeros((shape.num_loops, shape.num_layers), np.uint8)
    cost = PlanCost()
    b = PlanBudget(float(max_damage), float(max_stored_bytes), float(hot_fraction))
    _check(lib().loopkv_plan_solve(ctypes.byref(shape), d.ctypes.data, ctypes.byref(b), plan.ctypes.data,
                                   ctypes.byref(cost)), "loopkv_plan_solve")
    return plan, cost


def make_shape(*, num_layers, num_loops, num_kv_heads=16, head_dim=128, page_tokens=32,
               v_group=128, max_batch, max_pages_per_seq, tail_tokens=64, max_splits=64,
               num_pages, sink_tokens=0, window_tokens=0) -> Shape:
    return Shape(num_layers, num_loops, num_kv_heads, num_kv_heads, head_dim, page_tokens,
                 v_group, max_batch, max_pages_per_seq, tail_tokens, max_splits, sink_tokens,
                 window_tokens, 0, num_pages)
