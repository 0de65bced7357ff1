"""LoopKV fused decode attention for AMD Instinct MI355X (gfx950).

The work runs in libloopkv.so (include/loopkv.h): a C ABI over hand-written HIP kernels.
`loopkv` is its ctypes binding and `cache.LoopKVCache` a tensor-level wrapper; `synth` draws
the seeded synthetic inputs used by the tests and the benchmark.
"""
from . import loopkv  # noqa: F401
from .loopkv import INT2, INT4, REUSE, LoopKVError, make_shape  # noqa: F401

__all__ = ["loopkv", "INT2", "INT4", "REUSE", "LoopKVError", "make_shape"]
