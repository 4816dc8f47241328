"""Measured machine ceilings for the benchmark report (ceilings.hip).

Not part of the layer: a read-only HBM streaming kernel, the table path's LDS
gather pattern, and a chain of empty persistent-shaped launches.  Built in-tree
by __graft_entry__.build() with the layer library's flags.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libvqe_ceilings.so")
SRC_PATH = os.path.join(_HERE, "ceilings.hip")


def build() -> str:
    from vector_quantized_expert_amd import build_lib
    hipcc = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
    subprocess.run([hipcc, *build_lib.HIPCC_FLAGS, SRC_PATH, "-o", LIB_PATH + ".tmp"], check=True,
                   stderr=subprocess.DEVNULL)
    os.replace(LIB_PATH + ".tmp", LIB_PATH)
    return LIB_PATH


_lib = None


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with __graft_entry__.build()")
        L = ctypes.CDLL(LIB_PATH)
        vp, f32p = ctypes.c_void_p, ctypes.POINTER(ctypes.c_float)
        i32 = ctypes.c_int
        L.vqe_ceiling_read.argtypes = [vp, ctypes.c_uint64, i32, i32, i32, vp, f32p]
        L.vqe_ceiling_lds.argtypes = [i32, i32, vp, f32p, ctypes.POINTER(ctypes.c_int)]
        L.vqe_ceiling_launch_gap.argtypes = [i32, vp, f32p]
        for n in ("vqe_ceiling_read", "vqe_ceiling_lds", "vqe_ceiling_launch_gap"):
            getattr(L, n).restype = ctypes.c_int
        _lib = L
    return _lib


def _ok(rc, what):
    if rc != 0:
        raise RuntimeError(f"{what} failed (hipError {rc})")


def hbm_read_GBps(buf, reps: int, stream) -> dict:
    """Read rate of the whole device buffer `buf` (a torch uint8 tensor), GB/s,
    for each kernel shape tried; `best` is the ceiling."""
    out = {}
    for name, variant, per_cu in (("256x8_4inflight", 0, 0), ("1024x1_8inflight", 1, 1), ("1024x2_8inflight", 1, 2)):
        ms = ctypes.c_float()
        _ok(lib().vqe_ceiling_read(buf.data_ptr(), buf.numel(), reps, variant, per_cu, stream.cuda_stream,
                                   ctypes.byref(ms)), "read")
        out[name] = buf.numel() * reps / (ms.value * 1e-3) / 1e9
    out["best"] = max(out.values())
    return out


def lds_rates(stream) -> dict:
    """LDS read rates over every CU: the table path's 4-byte lookups (per second;
    one lookup per code byte) and 16-byte streaming reads (bytes per CU per clock
    at 2.4 GHz as well as GB/s in all)."""
    out = {}
    ms, blocks = ctypes.c_float(), ctypes.c_int()
    iters = 4000
    _ok(lib().vqe_ceiling_lds(0, iters, stream.cuda_stream, ctypes.byref(ms), ctypes.byref(blocks)), "lds b32")
    lookups = blocks.value * 1024 * 48 * iters
    out["table_lookups_per_s"] = lookups / (ms.value * 1e-3)
    out["table_lookup_bytes_per_clk_per_cu"] = 4 * lookups / (ms.value * 1e-3) / blocks.value / 2.4e9
    _ok(lib().vqe_ceiling_lds(1, iters, stream.cuda_stream, ctypes.byref(ms), ctypes.byref(blocks)), "lds b128")
    byts = blocks.value * 1024 * 8 * 16 * iters
    out["b128_GBps"] = byts / (ms.value * 1e-3) / 1e9
    out["b128_bytes_per_clk_per_cu"] = byts / (ms.value * 1e-3) / blocks.value / 2.4e9
    return out


def launch_gap_us(launches: int, stream) -> float:
    """Time per launch of an empty persistent-shaped grid, launched back to back."""
    ms = ctypes.c_float()
    _ok(lib().vqe_ceiling_launch_gap(launches, stream.cuda_stream, ctypes.byref(ms)), "launch gap")
    return ms.value * 1e3 / launches
