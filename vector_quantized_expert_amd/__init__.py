"""Routed RVQ-MoE decode layer for MI355X (gfx950): HIP kernels behind a C ABI.

The Python side is a thin ctypes binding (``rvq_moe``); all computation runs in
``librvq_moe.so`` built from ``csrc/``.
"""
from .rvq_moe import RvqMoe, RvqMoeError, lib  # noqa: F401

__all__ = ["RvqMoe", "RvqMoeError", "lib"]
