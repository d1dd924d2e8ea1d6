"""CPU oracle for split-KV attention forward (float64, numpy).

TEST INFRASTRUCTURE ONLY: imported by tests/, by the smoke check and by the
benchmark's CPU-baseline leg, never by the library or its binding.  It shares
no code with the HIP path.  See oracle/splitkv.py for the functions and the
passages of the pages each one follows.
"""
from .splitkv import *  # noqa: F401,F403
from .splitkv import __all__  # noqa: F401
