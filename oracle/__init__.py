"""fp64 CPU oracle for Kascade anchor/reuse Top-k sparse attention.

TEST INFRASTRUCTURE ONLY: imported by tests/, __graft_entry__.smoke() and the
cpu_baseline leg of bench.py, never by the HIP library or its binding.
"""
from .kascade_oracle import *  # noqa: F401,F403
from .kascade_oracle import __all__  # noqa: F401
