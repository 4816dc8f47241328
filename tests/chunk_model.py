"""Precision model of the chunk path's rounding points (test helper).

[FR] "Quantification et exactitude" fixes the format: a weight is c1 + c2 + c3,
the sum of one entry of each stage codebook over an 8-wide vector.  The chunk
path evaluates it at reduced precision at fixed points only (the reading the
layer documents): each weight is the fp32 sum (c1 + c2) + c3 rounded to bf16
(round to nearest even), the normalised tokens and the SwiGLU output h are
rounded to bf16, and every product is accumulated exactly enough (fp32) that
those roundings dominate.  This module applies exactly those roundings around
plain float64 dense products, so that a chunk-path output can be checked
element by element: what remains between the two is fp32 accumulation order
and, rarely, a one-ulp difference in a rounded h entry.

Dense weights are materialised with numpy gathers from the canonical record;
routing (ids, gates) is taken as given.  Nothing here is shared with the HIP
path.  Pinned against the fp64 oracle in tests/test_chunk_model.py.
"""
from __future__ import annotations

import numpy as np


def bf16(a) -> np.ndarray:
    """Round fp32 values to bf16 (nearest, ties to even); returned as float64."""
    u = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32).astype(np.uint64)
    u = (u + 0x7FFF + ((u >> 16) & 1)) & 0xFFFF0000
    return u.astype(np.uint32).view(np.float32).astype(np.float64)


def matrices(record: np.ndarray, d: int, ffn: int):
    """Canonical record -> codes of gate [ffn][d/8][3], up [ffn][d/8][3], down [d][ffn/8][3]."""
    n_gu = ffn * (d // 8) * 3
    g = record[:n_gu].reshape(ffn, d // 8, 3)
    u = record[n_gu:2 * n_gu].reshape(ffn, d // 8, 3)
    dn = record[2 * n_gu:].reshape(d, ffn // 8, 3)
    return g, u, dn


def dense_weights(cb: np.ndarray, codes: np.ndarray, rounded: bool = True) -> np.ndarray:
    """bf16((c1 + c2) + c3) with the two sums in fp32, as a [rows][cols] float64
    matrix (rounded=False: the exact sum, in float64)."""
    rows, ns, _ = codes.shape
    if not rounded:
        c = cb.astype(np.float64)
        return ((c[0][codes[:, :, 0]] + c[1][codes[:, :, 1]]) + c[2][codes[:, :, 2]]).reshape(rows, ns * 8)
    c = cb.astype(np.float32)
    w = (c[0][codes[:, :, 0]] + c[1][codes[:, :, 1]]) + c[2][codes[:, :, 2]]
    return bf16(w.reshape(rows, ns * 8))


def expert(cb: np.ndarray, record: np.ndarray, d: int, ffn: int, xb: np.ndarray, rounded: bool = True):
    """One expert on tokens xb: returns (y, Wd, H) with H = bf16(silu(a) b)
    (rounded=False: no rounding anywhere, for experts the table path evaluates)."""
    gc, uc, dc = matrices(record, d, ffn)
    a = dense_weights(cb[0], gc, rounded) @ xb
    b = dense_weights(cb[1], uc, rounded) @ xb
    h = a / (1.0 + np.exp(-a)) * b
    H = bf16(h.astype(np.float32)) if rounded else h
    Wd = dense_weights(cb[2], dc, rounded)
    return Wd @ H, Wd, H


def token_x(x: np.ndarray, pre_rmsnorm: bool, eps: float) -> np.ndarray:
    """The bf16 token the chunk path contracts: x, or x / sqrt(mean(x^2) + eps)
    divided in fp64 and rounded to fp32 first."""
    x = np.asarray(x, dtype=np.float32)
    if pre_rmsnorm:
        x64 = x.astype(np.float64)
        r = np.sqrt(np.dot(x64, x64) / x.shape[0] + eps)
        x = (x64 / r).astype(np.float32)
    return bf16(x)


def token_exact(x: np.ndarray, pre_rmsnorm: bool, eps: float) -> np.ndarray:
    """The unrounded token (float64) the table path takes."""
    x64 = np.asarray(x, dtype=np.float32).astype(np.float64)
    return x64 / np.sqrt(np.dot(x64, x64) / x64.shape[0] + eps) if pre_rmsnorm else x64


def layer(x, ids, gates, get_codebook, get_record, d: int, ffn: int, pre_rmsnorm=False, eps=1e-6,
          table_experts=()):
    """MoE output (before any residual add) of one token under the chunk path's
    rounding, plus per-element error scales: for each output element q,
    `peak` = sum_j g_j max_r |Wd_qr H_r| and `mass` = sum_j g_j sum_r |Wd_qr| |H_r|.
    Experts in table_experts (handed to the fp32 table path by adaptive
    dispatch) are taken without any rounding."""
    xb = token_x(x, pre_rmsnorm, eps)
    xe = token_exact(x, pre_rmsnorm, eps)
    y = np.zeros(d)
    peak = np.zeros(d)
    mass = np.zeros(d)
    for e, g in zip(ids, gates):
        exact = int(e) in table_experts
        ye, Wd, H = expert(get_codebook(int(e)), get_record(int(e)), d, ffn, xe if exact else xb,
                           rounded=not exact)
        prod = np.abs(Wd) * np.abs(H)[None, :]
        y += float(g) * ye
        peak += float(g) * prod.max(axis=1)
        mass += float(g) * prod.sum(axis=1)
    return y, peak, mass


def element_tolerance(peak: np.ndarray, mass: np.ndarray) -> np.ndarray:
    """Per-element bound between a chunk-path output and this model: up to two
    one-ulp flips of a rounded h entry (each at most 2^-7 |Wd_qr H_r|) plus
    fp32 accumulation over the ffn products (2^-12 of their absolute sum)."""
    return 2.0 ** -6 * peak + 2.0 ** -12 * mass
