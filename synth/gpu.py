"""Stage the seeded synthetic inputs in device memory (tests and benchmark).

Input generation only: codebooks, router weights and tokens come from
synth.py on the host and are copied to the device; the (large) canonical code
bank is generated on the device by synth_codes.hip, bit-identical to
synth.expert_record().
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

from . import synth as S

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libvqe_synth.so")
SRC_PATH = os.path.join(_HERE, "synth_codes.hip")


def build() -> str:
    hipcc = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
    subprocess.run([hipcc, "--offload-arch=gfx950", "-O3", "-fPIC", "-shared", "-Xclang", "-target-feature",
                    "-Xclang", "-packed-fp32-ops", SRC_PATH, "-o", LIB_PATH + ".tmp"], check=True,
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
        L.vqe_synth_codes.argtypes = [ctypes.c_void_p, ctypes.c_uint64, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                      ctypes.c_uint64, ctypes.c_void_p]
        L.vqe_synth_codes.restype = ctypes.c_int
        _lib = L
    return _lib


def codes_on_device(seed: int, layer: int, n_experts: int, rec_bytes: int, device="cuda", expert0: int = 0):
    """[n_experts][rec_bytes] uint8 torch tensor of canonical codes, generated on the device."""
    import torch
    out = torch.empty((n_experts, rec_bytes), dtype=torch.uint8, device=device)
    stream = torch.cuda.current_stream().cuda_stream
    rc = lib().vqe_synth_codes(out.data_ptr(), seed, layer, expert0, n_experts, rec_bytes, stream)
    if rc != 0:
        raise RuntimeError("vqe_synth_codes failed")
    return out


def to_device(a: np.ndarray, device="cuda"):
    import torch
    return torch.from_numpy(np.ascontiguousarray(a)).to(device)


class LayerInputs:
    """Host and device copies of one layer's seeded inputs."""

    def __init__(self, shape: S.Shape, seed: int, layer: int, device="cuda", host_codes: bool = False):
        self.shape, self.seed, self.layer = shape, seed, layer
        self.cb = S.codebooks(seed, layer, shape.n_experts, shape.np_cb_dtype)
        self.w_r = S.router_weights(seed, layer, shape.d, shape.n_experts)
        self.cb_dev = to_device(self.cb, device)
        self.w_r_dev = to_device(self.w_r, device)
        if host_codes:
            self.codes_host = S.codes_bank(seed, layer, shape.n_experts, shape.record_bytes)
            self.codes_dev = to_device(self.codes_host, device)
        else:
            self.codes_host = None
            self.codes_dev = codes_on_device(seed, layer, shape.n_experts, shape.record_bytes, device)

    def record(self, e: int) -> np.ndarray:
        if self.codes_host is not None:
            return self.codes_host[e]
        return S.expert_record(self.seed, self.layer, e, self.shape.record_bytes)

    def codebook(self, e: int) -> np.ndarray:
        return self.cb[e]

    def free_codes(self):
        self.codes_dev = None
