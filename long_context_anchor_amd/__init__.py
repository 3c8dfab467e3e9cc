"""Kascade cross-layer Top-k sparse attention for MI355X (gfx950).

The compute path is the C-ABI library ``libkascade.so`` built from ``csrc/``
(hand-written HIP kernels); ``kascade`` is its thin ctypes binding.  Importing
this package does not load the library: the binding loads it on first use and
raises if it is missing.
"""
__all__ = ["configs", "synth", "kascade"]
