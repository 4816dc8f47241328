"""ctypes wrapper of the C oracle (rvq_oracle.c).

TEST INFRASTRUCTURE ONLY: imported by the tests, by the benchmark's
CPU-baseline leg and by the smoke check, never by the product package.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from dataclasses import dataclass

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "librvq_oracle.so")
SRC_PATH = os.path.join(_HERE, "rvq_oracle.c")

_f64p = ctypes.POINTER(ctypes.c_double)
_f32p = ctypes.POINTER(ctypes.c_float)
_i32p = ctypes.POINTER(ctypes.c_int32)
_u8p = ctypes.POINTER(ctypes.c_uint8)


def build(openmp: bool = True) -> str:
    """Compile the oracle with gcc (no fast-math, no FP contraction)."""
    cmd = ["gcc", "-std=c11", "-O2", "-ffp-contract=off", "-fno-fast-math", "-fPIC", "-shared",
           SRC_PATH, "-o", LIB_PATH + ".tmp", "-lm"]
    if openmp:
        cmd.insert(1, "-fopenmp")
    subprocess.run(cmd, check=True)
    os.replace(LIB_PATH + ".tmp", LIB_PATH)
    return LIB_PATH


_lib = None


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH) or os.path.getmtime(LIB_PATH) < os.path.getmtime(SRC_PATH):
            build()
        L = ctypes.CDLL(LIB_PATH)
        L.rvq_oracle_threads.argtypes = []
        L.rvq_oracle_threads.restype = ctypes.c_int
        L.rvq_oracle_set_threads.argtypes = [ctypes.c_int]
        L.rvq_oracle_set_threads.restype = None
        L.rvq_oracle_half_to_double.argtypes = [ctypes.c_uint16]
        L.rvq_oracle_half_to_double.restype = ctypes.c_double
        L.rvq_oracle_rmsnorm.argtypes = [ctypes.c_int, _f32p, ctypes.c_double, _f64p]
        L.rvq_oracle_router.argtypes = [ctypes.c_int, ctypes.c_int, _f64p, _f32p, _f64p]
        L.rvq_oracle_topk.argtypes = [ctypes.c_int, ctypes.c_int, _f64p, _i32p, _f64p, _f64p, _f64p]
        L.rvq_oracle_matvec.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_void_p, ctypes.c_int,
                                        _u8p, _f64p, _f64p]
        L.rvq_oracle_expert.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_void_p, ctypes.c_int,
                                        _u8p, _f64p, _f64p, _f64p, _f64p, _f64p]
        L.rvq_oracle_moe.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int, _f64p,
                                     ctypes.POINTER(ctypes.c_void_p), ctypes.c_int,
                                     ctypes.POINTER(ctypes.c_void_p), _f64p, _f32p, _f64p]
        L.rvq_oracle_crc32.argtypes = [_u8p, ctypes.c_int64]
        L.rvq_oracle_crc32.restype = ctypes.c_uint32
        for name in ("rvq_oracle_rmsnorm", "rvq_oracle_router", "rvq_oracle_topk", "rvq_oracle_matvec",
                     "rvq_oracle_expert", "rvq_oracle_moe"):
            getattr(L, name).restype = ctypes.c_int
        _lib = L
    return _lib


def _p(a: np.ndarray, t):
    return a.ctypes.data_as(t)


def _cb_dtype_code(cb: np.ndarray) -> int:
    if cb.dtype == np.float32:
        return 0
    if cb.dtype == np.float16:
        return 1
    raise TypeError(f"codebook dtype {cb.dtype} not supported")


def _check(rc: int, what: str):
    if rc != 0:
        raise ValueError(f"oracle {what} rejected its arguments (rc={rc})")


def threads() -> int:
    return lib().rvq_oracle_threads()


def set_threads(n: int) -> None:
    """OpenMP threads of later oracle calls (results are bitwise independent of it)."""
    lib().rvq_oracle_set_threads(int(n))


def half_to_double(bits: int) -> float:
    return lib().rvq_oracle_half_to_double(bits)


def rmsnorm(h: np.ndarray, eps: float) -> np.ndarray:
    h = np.ascontiguousarray(h, dtype=np.float32)
    out = np.empty(h.shape[0], np.float64)
    _check(lib().rvq_oracle_rmsnorm(h.shape[0], _p(h, _f32p), eps, _p(out, _f64p)), "rmsnorm")
    return out


def router(x: np.ndarray, w_r: np.ndarray) -> np.ndarray:
    x = np.ascontiguousarray(x, dtype=np.float64)
    w_r = np.ascontiguousarray(w_r, dtype=np.float32)
    d, E = w_r.shape
    assert x.shape == (d,)
    out = np.empty(E, np.float64)
    _check(lib().rvq_oracle_router(d, E, _p(x, _f64p), _p(w_r, _f32p), _p(out, _f64p)), "router")
    return out


@dataclass
class Route:
    ids: np.ndarray      # [k] int32, descending logit
    gates: np.ndarray    # [k] float64
    logits: np.ndarray   # [E] float64
    margin: float        # l_(k) - l_(k+1)
    min_gap: float       # smallest gap inside the top-k


def topk(logits: np.ndarray, k: int) -> Route:
    logits = np.ascontiguousarray(logits, dtype=np.float64)
    E = logits.shape[0]
    ids = np.empty(k, np.int32)
    gates = np.empty(k, np.float64)
    margin = ctypes.c_double()
    gap = ctypes.c_double()
    _check(lib().rvq_oracle_topk(E, k, _p(logits, _f64p), _p(ids, _i32p), _p(gates, _f64p),
                                 ctypes.byref(margin), ctypes.byref(gap)), "topk")
    return Route(ids, gates, logits, margin.value, gap.value)


def route(x_in: np.ndarray, w_r: np.ndarray, k: int, pre_rmsnorm: bool = False, eps: float = 1e-6) -> Route:
    x = rmsnorm(x_in, eps) if pre_rmsnorm else np.asarray(x_in, dtype=np.float32).astype(np.float64)
    return topk(router(x, w_r), k)


def matvec(codebook: np.ndarray, codes: np.ndarray, v: np.ndarray) -> np.ndarray:
    """One RVQ matrix: codebook [3][256][8], codes [rows][cols/8][3], v [cols]."""
    codebook = np.ascontiguousarray(codebook)
    codes = np.ascontiguousarray(codes, dtype=np.uint8)
    v = np.ascontiguousarray(v, dtype=np.float64)
    rows, ns, _ = codes.shape
    out = np.empty(rows, np.float64)
    _check(lib().rvq_oracle_matvec(rows, ns * 8, codebook.ctypes.data, _cb_dtype_code(codebook),
                                   _p(codes, _u8p), _p(v, _f64p), _p(out, _f64p)), "matvec")
    return out


@dataclass
class ExpertOut:
    pre_gate: np.ndarray
    pre_up: np.ndarray
    h: np.ndarray
    y: np.ndarray


def expert(d: int, ffn: int, codebook: np.ndarray, record: np.ndarray, x: np.ndarray) -> ExpertOut:
    codebook = np.ascontiguousarray(codebook)
    record = np.ascontiguousarray(record, dtype=np.uint8)
    x = np.ascontiguousarray(x, dtype=np.float64)
    a = np.empty(ffn, np.float64)
    b = np.empty(ffn, np.float64)
    h = np.empty(ffn, np.float64)
    y = np.empty(d, np.float64)
    _check(lib().rvq_oracle_expert(d, ffn, codebook.ctypes.data, _cb_dtype_code(codebook),
                                   _p(record, _u8p), _p(x, _f64p), _p(a, _f64p), _p(b, _f64p),
                                   _p(h, _f64p), _p(y, _f64p)), "expert")
    return ExpertOut(a, b, h, y)


def moe(d: int, ffn: int, gates: np.ndarray, codebooks: list, records: list, x: np.ndarray,
        resid: np.ndarray | None = None) -> np.ndarray:
    """Gate-weighted combine of already-selected experts (codebooks[j], records[j])."""
    k = len(gates)
    gates = np.ascontiguousarray(gates, dtype=np.float64)
    cbs = [np.ascontiguousarray(c) for c in codebooks]
    recs = [np.ascontiguousarray(r, dtype=np.uint8) for r in records]
    dt = _cb_dtype_code(cbs[0])
    assert all(_cb_dtype_code(c) == dt for c in cbs)
    cb_arr = (ctypes.c_void_p * k)(*[c.ctypes.data for c in cbs])
    rec_arr = (ctypes.c_void_p * k)(*[r.ctypes.data for r in recs])
    x = np.ascontiguousarray(x, dtype=np.float64)
    out = np.empty(d, np.float64)
    rp = None
    if resid is not None:
        resid = np.ascontiguousarray(resid, dtype=np.float32)
        rp = _p(resid, _f32p)
    _check(lib().rvq_oracle_moe(d, ffn, k, _p(gates, _f64p), cb_arr, dt, rec_arr, _p(x, _f64p), rp,
                                _p(out, _f64p)), "moe")
    return out


@dataclass
class LayerOut:
    route: Route
    x_hat: np.ndarray    # normalised input (float64)
    delta: np.ndarray    # MoE output before any residual add (float64)
    out: np.ndarray      # delta + input when residual (float64)


def layer(x_in: np.ndarray, w_r: np.ndarray, k: int, get_codebook, get_record, d: int, ffn: int,
          pre_rmsnorm: bool = False, eps: float = 1e-6, residual: bool = False) -> LayerOut:
    """Full layer for one token; get_codebook(e) / get_record(e) supply expert e's data."""
    x_in = np.asarray(x_in, dtype=np.float32)
    x = rmsnorm(x_in, eps) if pre_rmsnorm else x_in.astype(np.float64)
    r = topk(router(x, w_r), k)
    cbs = [get_codebook(int(e)) for e in r.ids]
    recs = [get_record(int(e)) for e in r.ids]
    delta = moe(d, ffn, r.gates, cbs, recs, x)
    out = delta + x_in.astype(np.float64) if residual else delta
    return LayerOut(r, x, delta, out)


# --------------------------------------------------------------------------- expert-record integrity
# [FR] "Architecture de streaming depuis le disque": every record read from
# an expert bank is checked for its magic, its expert id and its offset range
# (a truncated or wrongly assembled bank must not hand out another expert's
# weights); the crc32 of the payload is checked on request only.  The record
# layout checked here is the library's documented bank format, restated:
# record e spans [e * stride, (e + 1) * stride); the payload comes first, the
# trailer starts at the first 4096-byte boundary at or after its end, as
# little-endian fields magic u32, version u32, expert u32, n_experts u32,
# offset u64, payload_bytes u64, d i32, ffn i32, crc32 u32, reserved u32.

RECORD_MAGIC = int.from_bytes(b"RVQR", "little")
RECORD_VERSION = 1
BAD_MAGIC, BAD_ID, BAD_RANGE, BAD_CRC = 1, 2, 4, 8
_TRAILER = "<IIIIQQiiII"


def crc32(buf) -> int:
    """CRC-32 of a byte buffer (bitwise C loop; see rvq_oracle_crc32)."""
    a = np.ascontiguousarray(np.frombuffer(bytes(buf), np.uint8) if not isinstance(buf, np.ndarray) else buf,
                             dtype=np.uint8)
    if a.size == 0:
        return lib().rvq_oracle_crc32(None, 0)
    return int(lib().rvq_oracle_crc32(_p(a, _u8p), a.size))


def trailer_offset(payload: int) -> int:
    return (payload + 4095) // 4096 * 4096


def record_check_flags(record: np.ndarray, e: int, n_experts: int, stride: int, payload: int, d: int, ffn: int,
                       verify: bool) -> int:
    """Flags of the checks one record (its `stride` bytes) fails, 0 if none."""
    import struct
    t0 = trailer_offset(payload)
    magic, version, expert, n_exp, offset, pay, td, tffn, crc, _ = struct.unpack_from(
        _TRAILER, bytes(record[t0:t0 + struct.calcsize(_TRAILER)]))
    flags = 0
    if magic != RECORD_MAGIC or version != RECORD_VERSION:
        flags |= BAD_MAGIC
    if expert != e or n_exp != n_experts:
        flags |= BAD_ID
    if offset != e * stride or pay != payload or td != d or tffn != ffn:
        flags |= BAD_RANGE
    if verify and crc32(record[:payload]) != crc:
        flags |= BAD_CRC
    return flags
