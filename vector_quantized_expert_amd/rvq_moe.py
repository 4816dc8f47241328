"""ctypes binding of librvq_moe.so (include/rvq_moe.h).

Argument marshalling only: every step of the layer runs in the HIP library.
Device buffers are torch tensors (passed as ``data_ptr()``) and streams are
torch streams (passed as ``cuda_stream``); torch is used for memory and
streams, nothing else.  There is no fallback: if the library is missing or
fails to load, every entry point raises.
"""
from __future__ import annotations

import ctypes
import os
import re

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
LIB_PATH = os.path.join(PKG, "librvq_moe.so")
HEADER = os.path.join(ROOT, "include", "rvq_moe.h")

OK, EINVAL, ENOTSUP, EBUDGET, ENOMEM, EHIP, EDEVICE, ECORRUPT = 0, -1, -2, -3, -4, -5, -6, -7
STATUS_NAMES = {0: "OK", -1: "EINVAL", -2: "ENOTSUP", -3: "EBUDGET", -4: "ENOMEM", -5: "EHIP", -6: "EDEVICE",
                -7: "ECORRUPT"}
CB_F32, CB_F16 = 0, 1
CODES_DEVICE, CODES_PINNED_HOST, CODES_PINNED_BANK = 0, 1, 2
RECORD_MAGIC, RECORD_VERSION = 0x52515652, 1
RECORD_BAD_MAGIC, RECORD_BAD_ID, RECORD_BAD_RANGE, RECORD_BAD_CRC = 1, 2, 4, 8
KERNEL_KINDS = 4


class RvqMoeError(RuntimeError):
    def __init__(self, status: int, what: str, reason: str):
        super().__init__(f"{what}: {STATUS_NAMES.get(status, status)} ({reason})")
        self.status = status


class Desc(ctypes.Structure):
    _fields_ = [
        ("struct_size", ctypes.c_uint32),
        ("d", ctypes.c_int32),
        ("ffn", ctypes.c_int32),
        ("n_experts", ctypes.c_int32),
        ("top_k", ctypes.c_int32),
        ("n_stages", ctypes.c_int32),
        ("n_codes", ctypes.c_int32),
        ("vec_dim", ctypes.c_int32),
        ("codebook_dtype", ctypes.c_int32),
        ("codes_location", ctypes.c_int32),
        ("cache_slots", ctypes.c_int32),
        ("pre_rmsnorm", ctypes.c_int32),
        ("residual", ctypes.c_int32),
        ("max_tokens", ctypes.c_int32),
        ("chunk_min_tokens", ctypes.c_int32),
        ("lut_expert_tokens", ctypes.c_int32),
        ("verify_records", ctypes.c_int32),
        ("deterministic", ctypes.c_int32),
        ("eps", ctypes.c_double),
        ("router_w", ctypes.c_void_p),
        ("codebooks", ctypes.c_void_p),
        ("codes", ctypes.c_void_p),
        ("stream", ctypes.c_void_p),
    ]


class Stats(ctypes.Structure):
    _fields_ = [(n, ctypes.c_uint64) for n in (
        "route_calls", "forward_calls", "tokens_routed", "tokens_forwarded", "expert_evals",
        "code_bytes_resident", "record_bytes", "codebook_bytes", "h2d_bytes", "slot_hits", "slot_misses",
        "host_syncs", "prefetch_fills", "prefetch_hits", "records_checked", "records_verified")]


class RecordTrailer(ctypes.Structure):
    """rvq_moe_record_trailer: the start of each record's 4 KiB trailer page."""
    _fields_ = [
        ("magic", ctypes.c_uint32),
        ("version", ctypes.c_uint32),
        ("expert", ctypes.c_uint32),
        ("n_experts", ctypes.c_uint32),
        ("offset", ctypes.c_uint64),
        ("payload_bytes", ctypes.c_uint64),
        ("d", ctypes.c_int32),
        ("ffn", ctypes.c_int32),
        ("crc32", ctypes.c_uint32),
        ("reserved", ctypes.c_uint32),
    ]


_lib = None


def lib():
    """Load librvq_moe.so (built by __graft_entry__.build()); raise if absent."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with __graft_entry__.build()")
        L = ctypes.CDLL(LIB_PATH)
        vp, i32 = ctypes.c_void_p, ctypes.c_int32
        L.rvq_moe_open.argtypes = [ctypes.POINTER(Desc), ctypes.POINTER(vp)]
        L.rvq_moe_route_topk.argtypes = [vp, vp, i32, vp, vp, vp]
        L.rvq_moe_layer_forward.argtypes = [vp, vp, i32, vp, vp, vp, vp]
        L.rvq_moe_route_forward.argtypes = [vp, vp, i32, vp, vp, vp, vp]
        L.rvq_moe_layer_forward_noalloc.argtypes = [vp, vp, i32, vp, vp, vp, vp]
        L.rvq_moe_prefetch.argtypes = [vp, vp, i32, i32, vp]
        L.rvq_moe_bank_layout.argtypes = [ctypes.POINTER(Desc), ctypes.POINTER(ctypes.c_int64),
                                          ctypes.POINTER(ctypes.c_int64)]
        L.rvq_moe_write_bank.argtypes = [ctypes.POINTER(Desc), vp]
        L.rvq_moe_sync.argtypes = [vp, vp]
        L.rvq_moe_close.argtypes = [vp]
        L.rvq_moe_last_error.argtypes = []
        L.rvq_moe_last_error.restype = ctypes.c_char_p
        L.rvq_moe_abi_version.argtypes = []
        L.rvq_moe_get_stats.argtypes = [vp, ctypes.POINTER(Stats)]
        L.rvq_moe_set_profiling.argtypes = [vp, ctypes.c_int]
        L.rvq_moe_kernel_times.argtypes = [vp, ctypes.POINTER(ctypes.c_char_p), ctypes.POINTER(ctypes.c_uint64),
                                           ctypes.POINTER(ctypes.c_double), ctypes.c_int]
        for n in ("rvq_moe_open", "rvq_moe_route_topk", "rvq_moe_layer_forward", "rvq_moe_route_forward",
                  "rvq_moe_layer_forward_noalloc",
                  "rvq_moe_prefetch", "rvq_moe_sync", "rvq_moe_bank_layout", "rvq_moe_write_bank",
                  "rvq_moe_close", "rvq_moe_abi_version", "rvq_moe_get_stats", "rvq_moe_set_profiling",
                  "rvq_moe_kernel_times"):
            getattr(L, n).restype = ctypes.c_int
        _lib = L
    return _lib


def header_functions() -> list[str]:
    """Names of the functions include/rvq_moe.h declares."""
    text = open(HEADER, encoding="utf-8").read()
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\s*\*?\s*(rvq_moe_\w+)\s*\(", text, re.M)))


def last_error() -> str:
    return lib().rvq_moe_last_error().decode()


def _check(rc: int, what: str) -> int:
    if rc < 0:
        raise RvqMoeError(rc, what, last_error())
    return rc


def _ptr(t) -> int:
    if t is None:
        return 0
    if isinstance(t, int):
        return t
    return t.data_ptr()


def _stream(stream) -> int:
    if stream is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def make_desc(*, d, ffn, n_experts, top_k, codebook_dtype, router_w, codebooks, codes,
              codes_location=CODES_DEVICE, cache_slots=0, pre_rmsnorm=False, eps=1e-6, residual=False,
              max_tokens=1, chunk_min_tokens=0, lut_expert_tokens=0, verify_records=False, stream=None,
              n_stages=3, n_codes=256, vec_dim=8, deterministic=0) -> Desc:
    return Desc(ctypes.sizeof(Desc), d, ffn, n_experts, top_k, n_stages, n_codes, vec_dim, codebook_dtype,
                codes_location, cache_slots, int(bool(pre_rmsnorm)), int(bool(residual)), max_tokens,
                chunk_min_tokens, lut_expert_tokens, int(bool(verify_records)), int(deterministic), eps,
                _ptr(router_w),
                _ptr(codebooks), _ptr(codes), _stream(stream) if stream != 0 else 0)


def bank_layout(**kw) -> tuple[int, int]:
    """rvq_moe_bank_layout: (record stride, payload bytes) of the layer's record bank."""
    kw.setdefault("router_w", None)
    kw.setdefault("codebooks", None)
    kw.setdefault("codes", None)
    kw.setdefault("stream", 0)
    desc = make_desc(**kw)
    stride, payload = ctypes.c_int64(), ctypes.c_int64()
    _check(lib().rvq_moe_bank_layout(ctypes.byref(desc), ctypes.byref(stride), ctypes.byref(payload)),
           "rvq_moe_bank_layout")
    return stride.value, payload.value


def write_bank(bank, **kw) -> None:
    """rvq_moe_write_bank into `bank` (a pinned host tensor of n_experts * stride bytes)."""
    kw.setdefault("router_w", None)
    kw.setdefault("codebooks", None)
    desc = make_desc(**kw)
    _check(lib().rvq_moe_write_bank(ctypes.byref(desc), _ptr(bank)), "rvq_moe_write_bank")


def read_trailer(bank_bytes, expert: int, stride: int, payload: int) -> RecordTrailer:
    """The trailer of record `expert` from a host byte buffer (numpy uint8 / bytes) of the bank."""
    off = expert * stride + (payload + 4095) // 4096 * 4096
    raw = bytes(bank_bytes[off:off + ctypes.sizeof(RecordTrailer)])
    return RecordTrailer.from_buffer_copy(raw)


def open_raw(desc: Desc) -> tuple[int, int]:
    """rvq_moe_open; returns (status, handle) without raising."""
    h = ctypes.c_void_p()
    rc = lib().rvq_moe_open(ctypes.byref(desc), ctypes.byref(h))
    return rc, (h.value or 0)


class RvqMoe:
    """One routed RVQ-MoE layer handle (rvq_moe_open .. rvq_moe_close)."""

    def __init__(self, **kw):
        desc = make_desc(**kw)
        rc, h = open_raw(desc)
        _check(rc, "rvq_moe_open")
        self.h = h
        self.d, self.ffn, self.n_experts, self.top_k = kw["d"], kw["ffn"], kw["n_experts"], kw["top_k"]
        self.max_tokens = kw.get("max_tokens", 1)

    def route_topk(self, x, n_tokens, ids, gates, stream=None):
        return _check(lib().rvq_moe_route_topk(self.h, _ptr(x), n_tokens, _ptr(ids), _ptr(gates),
                                               _stream(stream)), "rvq_moe_route_topk")

    def layer_forward(self, x, n_tokens, ids, gates, y, stream=None):
        return _check(lib().rvq_moe_layer_forward(self.h, _ptr(x), n_tokens, _ptr(ids), _ptr(gates), _ptr(y),
                                                  _stream(stream)), "rvq_moe_layer_forward")

    def layer_forward_noalloc(self, x, n_tokens, ids, gates, y, stream=None):
        return _check(lib().rvq_moe_layer_forward_noalloc(self.h, _ptr(x), n_tokens, _ptr(ids), _ptr(gates),
                                                          _ptr(y), _stream(stream)), "rvq_moe_layer_forward_noalloc")

    def route_forward(self, x, n_tokens, ids, gates, y, stream=None):
        return _check(lib().rvq_moe_route_forward(self.h, _ptr(x), n_tokens, _ptr(ids), _ptr(gates), _ptr(y),
                                                  _stream(stream)), "rvq_moe_route_forward")

    def prefetch(self, ids, n_tokens, per_token, stream=None):
        return _check(lib().rvq_moe_prefetch(self.h, _ptr(ids), n_tokens, per_token, _stream(stream)),
                      "rvq_moe_prefetch")

    def sync(self, stream=None):
        return _check(lib().rvq_moe_sync(self.h, _stream(stream)), "rvq_moe_sync")

    def stats(self) -> dict:
        s = Stats()
        _check(lib().rvq_moe_get_stats(self.h, ctypes.byref(s)), "rvq_moe_get_stats")
        return {n: getattr(s, n) for n, _ in Stats._fields_}

    def set_profiling(self, every: int):
        _check(lib().rvq_moe_set_profiling(self.h, every), "rvq_moe_set_profiling")

    def kernel_times(self) -> dict:
        names = (ctypes.c_char_p * KERNEL_KINDS)()
        launches = (ctypes.c_uint64 * KERNEL_KINDS)()
        ms = (ctypes.c_double * KERNEL_KINDS)()
        n = _check(lib().rvq_moe_kernel_times(self.h, names, launches, ms, KERNEL_KINDS), "rvq_moe_kernel_times")
        return {names[i].decode(): (launches[i], ms[i]) for i in range(n)}

    def close(self):
        if self.h:
            h, self.h = self.h, 0
            return _check(lib().rvq_moe_close(h), "rvq_moe_close")
        return OK

    def __del__(self):
        try:
            if self.h:
                lib().rvq_moe_close(self.h)
                self.h = 0
        except Exception:
            pass
