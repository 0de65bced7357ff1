"""fp64 CPU oracle for the LoopKV decode path -- test infrastructure only.

Only tests/, the package smoke check and bench.py's CPU-baseline leg import this package.
"""
from .loopkv_oracle import *  # noqa: F401,F403
