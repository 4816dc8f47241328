"""Pins of the CPU oracle against facts fixed by the pages and by mathematics.

Each test checks the oracle against something other than itself: exact closed
forms, textbook reductions, brute force on tiny inputs, invariants, library
routines for special cases, and the structural facts the pages print
(tests/golden/rvq_format.txt).  The pins are chosen so that a dropped stage, a
swapped stage/slice/lane index, a transposed operand, a sign error in SiLU or
the softmax, or a wrong top-k order fails at least one of them.
"""
import itertools
import math
import os
from fractions import Fraction

import numpy as np
import pytest
import scipy.special

from oracle import oracle as O
from synth import synth as S

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "rvq_format.txt")


def golden():
    out = {}
    for line in open(GOLDEN, encoding="utf-8"):
        line = line.strip()
        if not line or line.startswith("#"):
            continue
        kv, _src = line.split("|", 1)
        k, v = kv.split("=")
        out[k.strip()] = float(v)
    return out


def rand_cb(rng, dtype, mats=None):
    shape = (3, 256, 8) if mats is None else (mats, 3, 256, 8)
    sig = np.array(S.SIGMA)[:, None, None] if mats is None else np.array(S.SIGMA)[None, :, None, None]
    return (rng.standard_normal(shape) * sig).astype(dtype)


def dense_from_codes(cb, codes):
    """Materialise W [rows][cols] with an independent numpy gather."""
    cb = cb.astype(np.float64)
    rows, ns, _ = codes.shape
    w = np.zeros((rows, ns, 8))
    for s in range(3):
        w += cb[s][codes[:, :, s]]
    return w.reshape(rows, ns * 8)


# ---------------------------------------------------------------- format facts
def test_golden_format_facts():
    g = golden()
    assert g["stages"] == S.N_STAGES == 3
    assert g["codebook_entries"] == S.N_CODES == 256
    assert g["vector_dim"] == S.VEC == 8
    assert g["experts_per_token"] == S.K3.top_k
    assert g["matrices_per_expert"] == S.N_MATS
    # 3 bytes (one per stage, log2(256) = 8 bits each) per 8 weights = 3.00 bits/weight
    for d, f in [(256, 128), (7168, 2048), (64, 16)]:
        weights = 3 * d * f
        assert S.record_bytes(d, f) * 8 / weights == pytest.approx(g["bits_per_weight"], abs=0)
        assert math.log2(g["codebook_entries"]) * g["stages"] / g["vector_dim"] == g["bits_per_weight"]


def test_lut_identity_three_lookups_two_adds():
    """The table-of-partial-dot-products evaluation (3 lookups + 2 adds per row
    and slice) agrees with the oracle's explicit c1+c2+c3 reconstruction."""
    g = golden()
    rng = np.random.default_rng(11)
    rows, ns = 37, 11
    cb = rand_cb(rng, np.float32)
    codes = rng.integers(0, 256, (rows, ns, 3), dtype=np.uint8)
    v = rng.standard_normal(ns * 8)
    # lut[s][j][c] = <C_s[c], v[8j:8j+8]>
    lut = np.einsum("sci,ji->sjc", cb.astype(np.float64), v.reshape(ns, 8))
    out = np.zeros(rows)
    lookups = adds = 0
    for r in range(rows):
        for j in range(ns):
            t = lut[0, j, codes[r, j, 0]] + lut[1, j, codes[r, j, 1]] + lut[2, j, codes[r, j, 2]]
            lookups += 3
            adds += 2
            out[r] += t
    assert lookups / (rows * ns) == g["lookups_per_row_slice"]
    assert adds / (rows * ns) == g["adds_per_row_slice"]
    ref = O.matvec(cb, codes, v)
    np.testing.assert_allclose(ref, out, rtol=1e-12, atol=1e-13)


# ---------------------------------------------------------------- fp16 decode
def test_half_to_double_matches_numpy_for_every_pattern():
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    ref = bits.view(np.float16).astype(np.float64)
    got = np.array([O.half_to_double(int(b)) for b in bits])
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan], ref[~nan])
    assert np.array_equal(np.signbit(got[~nan]), np.signbit(ref[~nan]))


# ---------------------------------------------------------------- rmsnorm
def test_rmsnorm_closed_forms():
    d, eps = 16, 1e-6
    x = O.rmsnorm(np.full(d, 3.0, np.float32), eps)
    assert np.all(x == 3.0 / math.sqrt(9.0 + eps))
    assert np.all(O.rmsnorm(np.zeros(d, np.float32), eps) == 0.0)
    # one-hot of height a: x = a / sqrt(a^2/d + eps) at the hot index
    h = np.zeros(d, np.float32)
    h[5] = 2.0
    x = O.rmsnorm(h, 0.0)
    assert x[5] == pytest.approx(math.sqrt(d), rel=1e-15) and np.count_nonzero(x) == 1
    # scale invariance at eps = 0, and unit mean square
    rng = np.random.default_rng(1)
    h = rng.standard_normal(64).astype(np.float32)
    np.testing.assert_allclose(O.rmsnorm(h, 0.0), O.rmsnorm(2 * h, 0.0), rtol=1e-15)
    assert np.mean(O.rmsnorm(h, 0.0) ** 2) == pytest.approx(1.0, rel=1e-14)


# ---------------------------------------------------------------- router
def test_router_exact_on_dyadic_inputs():
    rng = np.random.default_rng(2)
    d, E = 48, 9
    x = rng.integers(-64, 64, d) / 8.0
    w = (rng.integers(-512, 512, (d, E)) / 1024.0).astype(np.float32)
    got = O.router(x, w)
    for e in range(E):
        exact = sum(Fraction(float(x[i])) * Fraction(float(w[i, e])) for i in range(d))
        assert got[e] == float(exact)


def test_topk_equals_best_subset_by_brute_force():
    rng = np.random.default_rng(3)
    for trial in range(50):
        E = int(rng.integers(2, 9))
        k = int(rng.integers(1, E + 1))
        logits = rng.standard_normal(E)
        r = O.topk(logits, k)
        best = max(itertools.combinations(range(E), k), key=lambda c: sum(logits[list(c)]))
        assert set(r.ids.tolist()) == set(best)
        assert np.all(np.diff(logits[r.ids]) <= 0)  # descending
        srt = np.sort(logits)[::-1]
        if k < E:
            assert r.margin == srt[k - 1] - srt[k]


def test_topk_min_gap_is_the_smallest_pairwise_distance_in_the_top_k():
    """min_gap decides how strictly ids are compared (ordered list vs set), so
    it is pinned on its own: brute force over every pair of the selected
    logits (the smallest |l_i - l_j| among the top k, no sorting involved),
    exact ties give 0, k = 1 gives +inf, and dyadic logits give exact gaps."""
    rng = np.random.default_rng(11)
    for trial in range(200):
        E = int(rng.integers(2, 40))
        k = int(rng.integers(2, E + 1))
        logits = rng.standard_normal(E) * (10.0 ** rng.integers(-3, 3))
        r = O.topk(logits, k)
        sel = logits[r.ids]
        brute = min(abs(sel[i] - sel[j]) for i in range(k) for j in range(k) if i != j)
        assert r.min_gap == brute, (trial, r.min_gap, brute)
        # the k selected logits are the k largest: every pairwise distance is
        # taken among them, never across the boundary
        assert r.min_gap >= 0.0
    assert O.topk(np.array([0.25, 3.0, -1.0, 3.0, 2.5]), 3).min_gap == 0.0      # exact tie inside the top k
    assert O.topk(np.array([0.25, 3.0, -1.0, 3.0, 2.5]), 2).min_gap == 0.0
    assert O.topk(np.array([4.0, 3.0, 3.0]), 2).min_gap == 1.0                   # the tie sits on the boundary
    assert O.topk(np.array([4.0, 3.0, 3.0]), 2).margin == 0.0
    assert math.isinf(O.topk(np.array([0.5, 2.0, 1.0]), 1).min_gap)              # no pair in a top 1
    assert O.topk(np.array([1.0, 0.125, 0.75, -2.0, 0.5]), 4).min_gap == 0.25   # 1, .75, .5, .125 -> min 0.25


def test_results_do_not_depend_on_the_thread_count():
    """Rows are summed sequentially, so one thread and all threads agree bitwise."""
    shape = S.Shape(264, 136, 5, 2, "f16")
    cb = S.codebooks(6, 0, shape.n_experts, shape.np_cb_dtype)
    bank = S.codes_bank(6, 0, shape.n_experts, shape.record_bytes)
    x = S.tokens(6, 0, 1, shape.d)[0].astype(np.float64)
    n = O.threads()
    try:
        O.set_threads(1)
        one = O.expert(shape.d, shape.ffn, cb[1], bank[1], x)
    finally:
        O.set_threads(n)
    many = O.expert(shape.d, shape.ffn, cb[1], bank[1], x)
    assert np.array_equal(one.y, many.y) and np.array_equal(one.h, many.h)


def test_topk_ties_go_to_lower_id():
    r = O.topk(np.array([1.0, 2.0, 2.0, 2.0, 0.0]), 2)
    assert r.ids.tolist() == [1, 2]
    r = O.topk(np.array([0.5, 0.5, 0.5]), 3)
    assert r.ids.tolist() == [0, 1, 2]
    assert np.all(r.gates == 1.0 / 3.0) or np.allclose(r.gates, 1.0 / 3.0, rtol=1e-15)


def test_gates_equal_full_softmax_renormalised_over_topk():
    rng = np.random.default_rng(4)
    for _ in range(20):
        E, k = 24, 5
        logits = rng.standard_normal(E) * 3
        r = O.topk(logits, k)
        p = scipy.special.softmax(logits)
        ref = p[r.ids] / p[r.ids].sum()
        np.testing.assert_allclose(r.gates, ref, rtol=1e-14)
        assert abs(r.gates.sum() - 1.0) < 1e-15
        assert np.all(np.diff(r.gates) <= 0)
        i, j = 0, k - 1
        assert r.gates[i] / r.gates[j] == pytest.approx(math.exp(logits[r.ids[i]] - logits[r.ids[j]]), rel=1e-14)


def test_topk_k1_gate_is_one():
    r = O.topk(np.array([0.1, -3.0, 7.0]), 1)
    assert r.ids.tolist() == [2] and r.gates[0] == 1.0


# ---------------------------------------------------------------- one RVQ matrix
@pytest.mark.parametrize("dtype", [np.float32, np.float16])
@pytest.mark.parametrize("rows,cols", [(1, 8), (5, 24), (16, 64), (33, 136)])
def test_matvec_matches_dense_bruteforce(dtype, rows, cols):
    rng = np.random.default_rng(rows * 1000 + cols)
    cb = rand_cb(rng, dtype)
    codes = rng.integers(0, 256, (rows, cols // 8, 3), dtype=np.uint8)
    v = rng.standard_normal(cols)
    ref = dense_from_codes(cb, codes) @ v
    got = O.matvec(cb, codes, v)
    np.testing.assert_allclose(got, ref, rtol=1e-12, atol=1e-14)


def test_matvec_decodes_each_code_byte_at_its_stage_and_lane():
    """C_s[c][i] = 2^(12 s) (c + 256 i): a one-hot v at position 8j+i reads out
    the three code bytes of (row, slice j) and the lane i exactly, as base-4096
    digits.  Any stage/slice/lane/row index mix-up changes the digits."""
    rng = np.random.default_rng(5)
    rows, ns = 7, 5
    cb = np.zeros((3, 256, 8), np.float32)
    c = np.arange(256)[:, None]
    i = np.arange(8)[None, :]
    for s in range(3):
        cb[s] = (2.0 ** (12 * s)) * (c + 256 * i)
    codes = rng.integers(0, 256, (rows, ns, 3), dtype=np.uint8)
    for j in range(ns):
        for lane in range(8):
            v = np.zeros(ns * 8)
            v[8 * j + lane] = 1.0
            out = O.matvec(cb, codes, v)
            for r in range(rows):
                val = int(out[r])
                assert out[r] == val
                digits = [(val >> (12 * s)) & 0xFFF for s in range(3)]
                assert digits == [int(codes[r, j, s]) + 256 * lane for s in range(3)]


def test_matvec_unit_codebook_is_an_index_sum():
    """C1[c] = e_(c mod 8), C2 = C3 = 0: (W v)_r = sum_j v[8j + (code_rj0 mod 8)]."""
    rng = np.random.default_rng(6)
    rows, ns = 9, 13
    cb = np.zeros((3, 256, 8), np.float32)
    for c in range(256):
        cb[0, c, c % 8] = 1.0
    codes = rng.integers(0, 256, (rows, ns, 3), dtype=np.uint8)
    v = rng.standard_normal(ns * 8)
    got = O.matvec(cb, codes, v)
    for r in range(rows):
        ref = 0.0
        for j in range(ns):
            ref += v[8 * j + codes[r, j, 0] % 8]
        assert got[r] == pytest.approx(ref, rel=1e-14, abs=1e-14)


def test_matvec_constant_codebooks_closed_form():
    """Each stage constant alpha_s: every weight is alpha_1+alpha_2+alpha_3
    whatever the codes, so (W v)_r = (sum alpha) * sum v, exactly (dyadic)."""
    rng = np.random.default_rng(7)
    alphas = (0.375, -0.0625, 0.0078125)
    cb = np.stack([np.full((256, 8), a, np.float32) for a in alphas])
    rows, ns = 11, 6
    codes = rng.integers(0, 256, (rows, ns, 3), dtype=np.uint8)
    v = rng.integers(-50, 50, ns * 8) / 4.0
    got = O.matvec(cb, codes, v)
    assert np.all(got == sum(alphas) * v.sum())


# ---------------------------------------------------------------- one expert
def test_expert_closed_form_constant_codebooks():
    d, f = 64, 32
    al = {0: (0.125, 0.03125, -0.0078125), 1: (-0.25, 0.0625, 0.015625), 2: (0.0625, -0.015625, 0.00390625)}
    cb = np.zeros((3, 3, 256, 8), np.float32)
    for m in range(3):
        for s in range(3):
            cb[m, s] = al[m][s]
    rng = np.random.default_rng(8)
    rec = rng.integers(0, 256, S.record_bytes(d, f), dtype=np.uint8)
    x = rng.integers(-20, 20, d) / 8.0
    out = O.expert(d, f, cb, rec, x)
    A = [sum(al[m]) for m in range(3)]
    a = A[0] * x.sum()
    b = A[1] * x.sum()
    h = a * scipy.special.expit(a) * b
    assert np.all(out.pre_gate == a) and np.all(out.pre_up == b)
    np.testing.assert_allclose(out.h, h, rtol=1e-15)
    np.testing.assert_allclose(out.y, A[2] * f * h, rtol=1e-14)


def test_expert_zero_codebooks_give_exact_zero():
    d, f = 32, 16
    rng = np.random.default_rng(9)
    rec = rng.integers(0, 256, S.record_bytes(d, f), dtype=np.uint8)
    out = O.expert(d, f, np.zeros((3, 3, 256, 8), np.float16), rec, rng.standard_normal(d))
    assert np.all(out.y == 0.0) and np.all(out.h == 0.0)


def test_expert_linearity_in_x_is_exact():
    d, f = 64, 24
    rng = np.random.default_rng(10)
    cb = rand_cb(rng, np.float16, mats=3)
    rec = rng.integers(0, 256, S.record_bytes(d, f), dtype=np.uint8)
    x = rng.standard_normal(d)
    o1 = O.expert(d, f, cb, rec, x)
    o2 = O.expert(d, f, cb, rec, 2.0 * x)
    assert np.array_equal(o2.pre_gate, 2.0 * o1.pre_gate)
    assert np.array_equal(o2.pre_up, 2.0 * o1.pre_up)


@pytest.mark.parametrize("d,f", [(8, 8), (16, 8), (64, 16), (256, 128), (264, 136)])
def test_expert_matches_dense_bruteforce(d, f):
    rng = np.random.default_rng(d + f)
    cb = rand_cb(rng, np.float32, mats=3)
    rec = rng.integers(0, 256, S.record_bytes(d, f), dtype=np.uint8)
    g_bytes = f * (d // 8) * 3
    Wg = dense_from_codes(cb[0], rec[:g_bytes].reshape(f, d // 8, 3))
    Wu = dense_from_codes(cb[1], rec[g_bytes:2 * g_bytes].reshape(f, d // 8, 3))
    Wd = dense_from_codes(cb[2], rec[2 * g_bytes:].reshape(d, f // 8, 3))
    x = rng.standard_normal(d)
    a, b = Wg @ x, Wu @ x
    h = a * scipy.special.expit(a) * b
    y = Wd @ h
    out = O.expert(d, f, cb, rec, x)
    np.testing.assert_allclose(out.pre_gate, a, rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(out.pre_up, b, rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(out.y, y, rtol=1e-11, atol=1e-13)


def test_silu_sign_and_limits():
    """silu(z) = z * sigmoid(z): checked through the expert with a 1-row gate."""
    d, f = 8, 8
    cb = np.zeros((3, 3, 256, 8), np.float32)
    cb[0, 0, :, 0] = 1.0   # a_r = x[0] for every gate row
    cb[1, 0, :, 0] = 1.0   # b_r = x[0]
    rec = np.zeros(S.record_bytes(d, f), np.uint8)
    for z in (-30.0, -2.0, 0.0, 0.5, 3.0, 40.0):
        x = np.zeros(d)
        x[0] = z
        out = O.expert(d, f, cb, rec, x)
        ref = z * scipy.special.expit(z) * z
        np.testing.assert_allclose(out.h, ref, rtol=1e-15, atol=1e-300)


# ---------------------------------------------------------------- whole layer
def _tiny_layer(seed=0, d=64, f=32, E=8, k=3):
    cbs = S.codebooks(seed, 0, E, np.float32)
    recs = S.codes_bank(seed, 0, E, S.record_bytes(d, f))
    w = S.router_weights(seed, 0, d, E)
    return cbs, recs, w


def test_layer_expert_relabelling_is_bitwise_invariant():
    d, f, E, k = 64, 32, 8, 3
    cbs, recs, w = _tiny_layer(d=d, f=f, E=E, k=k)
    x = S.token(0, 3, d)
    base = O.layer(x, w, k, lambda e: cbs[e], lambda e: recs[e], d, f)
    perm = np.random.default_rng(12).permutation(E)  # new id p holds old expert perm[p]
    inv = np.argsort(perm)
    w2 = w[:, perm]
    out = O.layer(x, w2, k, lambda e: cbs[perm[e]], lambda e: recs[perm[e]], d, f)
    assert np.array_equal(perm[out.route.ids], base.route.ids)
    assert np.array_equal(inv[base.route.ids], out.route.ids)
    assert np.array_equal(out.delta, base.delta)


def test_layer_identical_experts_reduce_to_one_expert():
    d, f, E, k = 64, 32, 8, 4
    cbs, recs, w = _tiny_layer(d=d, f=f, E=E, k=k)
    x = S.token(0, 5, d)
    out = O.layer(x, w, k, lambda e: cbs[0], lambda e: recs[0], d, f)
    single = O.expert(d, f, cbs[0], recs[0], x.astype(np.float64)).y
    np.testing.assert_allclose(out.delta, single, rtol=1e-14, atol=1e-15)


def test_layer_zero_codebooks_and_residual():
    d, f, E, k = 64, 32, 8, 3
    _, recs, w = _tiny_layer(d=d, f=f, E=E, k=k)
    zero = np.zeros((3, 3, 256, 8), np.float16)
    x = S.token(0, 1, d)
    out = O.layer(x, w, k, lambda e: zero, lambda e: recs[e], d, f, residual=True)
    assert np.all(out.delta == 0.0)
    assert np.array_equal(out.out, x.astype(np.float64))


def test_layer_combine_is_gate_weighted_sum():
    d, f, E, k = 64, 32, 8, 3
    cbs, recs, w = _tiny_layer(d=d, f=f, E=E, k=k)
    x = S.token(0, 9, d)
    out = O.layer(x, w, k, lambda e: cbs[e], lambda e: recs[e], d, f, pre_rmsnorm=True, eps=1e-6)
    ys = [O.expert(d, f, cbs[e], recs[e], out.x_hat).y for e in out.route.ids]
    ref = sum(g * y for g, y in zip(out.route.gates, ys))
    np.testing.assert_allclose(out.delta, ref, rtol=1e-14, atol=1e-15)
    # routing uses the normalised input
    np.testing.assert_allclose(out.x_hat, x / np.sqrt(np.mean(x.astype(np.float64) ** 2) + 1e-6), rtol=1e-14)


# --------------------------------------------------------------------------- record integrity (crc32, trailer)
def test_crc32_standard_check_value():
    # The CRC-32 of IEEE 802.3 / ITU-T V.42 (zlib's) has the published check
    # value 0xCBF43926 for the nine ASCII digits "123456789".
    assert O.crc32(b"123456789") == 0xCBF43926
    assert O.crc32(b"") == 0


@pytest.mark.parametrize("n", [1, 3, 15, 16, 17, 4095, 4096, 4097, 100003])
def test_crc32_equals_the_library_routine(n):
    import zlib
    buf = np.random.default_rng(n).integers(0, 256, n, dtype=np.uint8)
    assert O.crc32(buf) == zlib.crc32(buf.tobytes())


def test_crc32_residue_and_affinity():
    rng = np.random.default_rng(7)
    for n in (1, 8, 77, 4096):
        m = rng.integers(0, 256, n, dtype=np.uint8)
        c = O.crc32(m)
        # appending the checksum (least significant byte first) leaves the
        # generator's fixed residue, 0x2144DF1C after the final inversion
        assert O.crc32(np.concatenate([m, np.frombuffer(c.to_bytes(4, "little"), np.uint8)])) == 0x2144DF1C
        # the checksum is affine over GF(2): an odd number of equal-length
        # messages xor-ed together has the xor of their checksums
        a, b = rng.integers(0, 256, (2, n), dtype=np.uint8)
        assert O.crc32(m ^ a ^ b) == c ^ O.crc32(a) ^ O.crc32(b)
        # any single flipped bit changes it
        for bit in (0, 7, 8 * n - 1):
            f = m.copy()
            f[bit // 8] ^= np.uint8(1 << (bit % 8))
            assert O.crc32(f) != c


def _record(e, n_experts, payload_bytes, d, ffn, seed=0, **over):
    import struct
    stride = O.trailer_offset(payload_bytes) + 4096
    rec = np.zeros(stride, np.uint8)
    rec[:payload_bytes] = np.random.default_rng(seed).integers(0, 256, payload_bytes, dtype=np.uint8)
    f = dict(magic=int.from_bytes(b"RVQR", "little"), version=1, expert=e, n_exp=n_experts,
             offset=e * stride, payload=payload_bytes, t_d=d, t_ffn=ffn, crc=O.crc32(rec[:payload_bytes]))
    f.update(over)
    t = struct.pack("<IIIIQQiiII", f["magic"], f["version"], f["expert"], f["n_exp"], f["offset"],
                    f["payload"], f["t_d"], f["t_ffn"], f["crc"], 0)
    t0 = O.trailer_offset(payload_bytes)
    rec[t0:t0 + len(t)] = np.frombuffer(t, np.uint8)
    return rec, stride


@pytest.mark.parametrize("over,flags", [
    ({}, 0),
    (dict(magic=0), O.BAD_MAGIC),
    (dict(version=2), O.BAD_MAGIC),
    (dict(expert=4), O.BAD_ID),
    (dict(n_exp=9), O.BAD_ID),
    (dict(offset=0), O.BAD_RANGE),
    (dict(payload=3072), O.BAD_RANGE),
    (dict(t_d=72), O.BAD_RANGE),
    (dict(t_ffn=48), O.BAD_RANGE),
    (dict(crc=1), O.BAD_CRC),
])
def test_record_check_flags_each_field(over, flags):
    d, ffn, E, e, payload = 64, 40, 8, 3, 6144
    rec, stride = _record(e, E, payload, d, ffn, **over)
    assert O.record_check_flags(rec, e, E, stride, payload, d, ffn, verify=True) == flags
    # without verify only the crc goes unchecked
    assert O.record_check_flags(rec, e, E, stride, payload, d, ffn, verify=False) == flags & ~O.BAD_CRC


def test_record_check_catches_a_payload_flip_only_with_crc():
    d, ffn, E, e, payload = 64, 40, 8, 5, 6144
    rec, stride = _record(e, E, payload, d, ffn)
    rec[1234] ^= 0x10
    assert O.record_check_flags(rec, e, E, stride, payload, d, ffn, verify=False) == 0
    assert O.record_check_flags(rec, e, E, stride, payload, d, ffn, verify=True) == O.BAD_CRC
    # a record read for another expert (a mis-assembled bank)
    rec2, _ = _record(e, E, payload, d, ffn)
    assert O.record_check_flags(rec2, e + 1, E, stride, payload, d, ffn, verify=False) == O.BAD_ID | O.BAD_RANGE
