"""Seeded synthetic inputs for the routed RVQ-MoE layer.

This module is input-generation infrastructure shared by the tests, the
benchmark and the oracle side.  It draws numbers and nothing else: it holds
none of the layer's arithmetic (no routing, no lookup tables, no FFN).

Recipe (every value is a pure function of ``seed`` and its indices):

* codebooks   -- for (layer, expert): a PCG64 stream keyed by
  ``SeedSequence([seed, layer, expert, TAG_CB])`` draws a float64 standard
  normal array of shape [3 matrices][3 stages][256 codes][8], scaled per stage
  by sigma = (0.02, 0.005, 0.00125) and rounded (RNE) to fp32 or fp16.
* router      -- for a layer: ``SeedSequence([seed, layer, TAG_ROUTER])`` draws
  W_r[d][E] ~ N(0, 0.02) in float64, rounded to fp32.
* tokens      -- token t: ``SeedSequence([seed, TAG_TOKEN, t])`` draws x ~ N(0, 1)
  of length d, rounded to fp32 (one seed per token).
* codes       -- the canonical expert record (gate [F][d/8][3], up [F][d/8][3],
  down [d][F/8][3], one uint8 per stage) is a stream of little-endian 64-bit
  words; word w of (layer, expert) is ``mix64(key + (w + 1) * GAMMA)`` with
  ``key = expert_key(seed, layer, expert)``.  mix64 is the SplitMix64 output
  function (Steele, Lea & Flood, "Fast splittable pseudorandom number
  generators", OOPSLA 2014, with Stafford's "Mix13" constants).  Being
  counter-based, the same bytes are produced on the GPU by ``synth_codes.hip``
  without a host round trip; the two are compared bit for bit in the GPU tests.
  Uniform bytes are the maximum-entropy stand-in for trained codes: nothing
  can be cached or compressed.

The pages measure on the real Kimi K3 / Kimi-Linear weights; those weights are
not available, so these seeded inputs stand in for them.
"""
from __future__ import annotations

from dataclasses import dataclass

import numpy as np

GAMMA = 0x9E3779B97F4A7C15
MIX_M1 = 0xBF58476D1CE4E5B9
MIX_M2 = 0x94D049BB133111EB
KEY_SALT = 0x5851F42D4C957F2D
_MASK = (1 << 64) - 1

TAG_CB = 0xC0DEB00C
TAG_ROUTER = 0x0707E4
TAG_TOKEN = 0x70CE17

SIGMA = (0.02, 0.005, 0.00125)

N_STAGES = 3
N_CODES = 256
VEC = 8
N_MATS = 3  # gate, up, down


@dataclass(frozen=True)
class Shape:
    """Layer shape: hidden d, expert FFN width F, experts E, top-k, codebook dtype."""

    d: int
    ffn: int
    n_experts: int
    top_k: int
    cb_dtype: str  # "f32" or "f16"

    @property
    def record_bytes(self) -> int:
        return record_bytes(self.d, self.ffn)

    @property
    def np_cb_dtype(self):
        return np.float32 if self.cb_dtype == "f32" else np.float16


# The tiny parity case and the K3-scale batch-1 decode layer.
TINY = Shape(256, 128, 16, 4, "f32")
K3 = Shape(7168, 2048, 384, 16, "f16")


def record_bytes(d: int, ffn: int) -> int:
    """Bytes of one canonical expert record: 3 matrices x rows x slices x 3 stages."""
    return 2 * ffn * (d // VEC) * N_STAGES + d * (ffn // VEC) * N_STAGES


def mix64_int(z: int) -> int:
    z &= _MASK
    z = ((z ^ (z >> 30)) * MIX_M1) & _MASK
    z = ((z ^ (z >> 27)) * MIX_M2) & _MASK
    return z ^ (z >> 31)


def mix64_array(z: np.ndarray) -> np.ndarray:
    z = z.astype(np.uint64, copy=True)
    with np.errstate(over="ignore"):
        z ^= z >> np.uint64(30)
        z *= np.uint64(MIX_M1)
        z ^= z >> np.uint64(27)
        z *= np.uint64(MIX_M2)
        z ^= z >> np.uint64(31)
    return z


def expert_key(seed: int, layer: int, expert: int) -> int:
    k = mix64_int(seed ^ KEY_SALT)
    k = mix64_int(k + (layer + 1) * GAMMA)
    return mix64_int(k + (expert + 1) * GAMMA)


def expert_record(seed: int, layer: int, expert: int, rec_bytes: int,
                  word_lo: int = 0, word_hi: int | None = None) -> np.ndarray:
    """Canonical code record bytes of one expert (or words [word_lo, word_hi) of it)."""
    assert rec_bytes % 8 == 0
    n_words = rec_bytes // 8
    word_hi = n_words if word_hi is None else word_hi
    key = np.uint64(expert_key(seed, layer, expert))
    w = np.arange(word_lo + 1, word_hi + 1, dtype=np.uint64)
    with np.errstate(over="ignore"):
        z = key + w * np.uint64(GAMMA)
    return mix64_array(z).view(np.uint8)


def codes_bank(seed: int, layer: int, n_experts: int, rec_bytes: int) -> np.ndarray:
    """[E][record] uint8 canonical code bank (for small shapes)."""
    return np.stack([expert_record(seed, layer, e, rec_bytes) for e in range(n_experts)])


def expert_codebooks(seed: int, layer: int, expert: int, dtype) -> np.ndarray:
    """[3 matrices][3 stages][256][8] codebook of one expert, rounded to ``dtype``."""
    rng = np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, layer, expert, TAG_CB])))
    z = rng.standard_normal((N_MATS, N_STAGES, N_CODES, VEC))
    z *= np.asarray(SIGMA, dtype=np.float64)[None, :, None, None]
    return z.astype(dtype)


def codebooks(seed: int, layer: int, n_experts: int, dtype) -> np.ndarray:
    """[E][3][3][256][8] codebooks."""
    return np.stack([expert_codebooks(seed, layer, e, dtype) for e in range(n_experts)])


def router_weights(seed: int, layer: int, d: int, n_experts: int) -> np.ndarray:
    """[d][E] fp32 router matrix, N(0, 0.02)."""
    rng = np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, layer, TAG_ROUTER])))
    return (rng.standard_normal((d, n_experts)) * 0.02).astype(np.float32)


def token(seed: int, t: int, d: int) -> np.ndarray:
    rng = np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, TAG_TOKEN, t])))
    return rng.standard_normal(d).astype(np.float32)


def tokens(seed: int, t0: int, n: int, d: int) -> np.ndarray:
    """[n][d] fp32 tokens t0 .. t0+n-1, one seed per token."""
    return np.stack([token(seed, t0 + i, d) for i in range(n)]) if n else np.zeros((0, d), np.float32)
