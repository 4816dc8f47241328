"""Expert-record integrity on the GPU, through the C ABI.

[FR] "Architecture de streaming depuis le disque": every record read from an
expert bank is checked for its magic, expert id and offset range, and its
payload's crc32 on request.  Checked here:
  - rvq_moe_write_bank's trailers and payload CRC-32 against the oracle's
    (bitwise crc32 and trailer rules), over shapes whose payload is ragged
    against 4 KiB and spans several rows per workgroup;
  - a clean bank streams exactly like resident codes, every fill checked;
  - damage the checks must see (a flipped payload byte: only with the CRC;
    two records swapped after open: always), reported as ECORRUPT with the
    flags and expert the oracle predicts, and kept until close;
  - open refusing a bank whose trailers are wrong.
Every corruption is in the codes' bytes or trailers only: any code byte is a
valid index, so the kernels reading a damaged slot stay in bounds.
"""
import re

import numpy as np
import pytest

from oracle import oracle as O
from synth import synth as S

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def torch_mod():
    import torch
    assert torch.cuda.is_available()
    return torch


def _kw(shape):
    return dict(d=shape.d, ffn=shape.ffn, n_experts=shape.n_experts, top_k=shape.top_k,
                codebook_dtype=0 if shape.cb_dtype == "f32" else 1)


def _bank(torch, inp, shape, from_host=False):
    from vector_quantized_expert_amd import rvq_moe as R
    stride, payload = R.bank_layout(**_kw(shape))
    bank = torch.empty(shape.n_experts * stride, dtype=torch.uint8, pin_memory=True)
    bank.fill_(0xA5)  # the writer must set every byte
    if from_host:
        canon = torch.empty(inp.codes_dev.shape, dtype=torch.uint8, pin_memory=True)
        canon.copy_(inp.codes_dev)
        R.write_bank(bank, codes=canon, codes_location=R.CODES_PINNED_HOST, **_kw(shape))
    else:
        R.write_bank(bank, codes=inp.codes_dev, codes_location=R.CODES_DEVICE, **_kw(shape))
    return bank, stride, payload


def _layer(inp, shape, codes, max_tokens=1, **kw):
    from vector_quantized_expert_amd import RvqMoe
    return RvqMoe(router_w=inp.w_r_dev, codebooks=inp.cb_dev, codes=codes, max_tokens=max_tokens,
                  **_kw(shape), **kw)


def _tokens(torch, layer, shape, x):
    """One route_topk + layer_forward call per token, then a sync (which may raise)."""
    from synth import gpu as G
    T = x.shape[0]
    xd = G.to_device(x)
    ids = torch.empty((T, shape.top_k), dtype=torch.int32, device="cuda")
    gates = torch.empty((T, shape.top_k), dtype=torch.float32, device="cuda")
    y = torch.empty((T, shape.d), dtype=torch.float32, device="cuda")
    for t in range(T):
        layer.route_topk(xd[t:t + 1], 1, ids[t:t + 1], gates[t:t + 1])
        layer.layer_forward(xd[t:t + 1], 1, ids[t:t + 1], gates[t:t + 1], y[t:t + 1])
    torch.cuda.synchronize()
    return ids.cpu().numpy(), y.cpu().numpy()


def _flags_of(msg):
    m = re.search(r"flags 0x([0-9a-f]+).*expert (-?\d+)", msg)
    assert m, msg
    return int(m.group(1), 16), int(m.group(2))


# --------------------------------------------------------------------------- the bank writer
@pytest.mark.parametrize("shape", [
    S.TINY,                              # payload 12 whole pages, one row per workgroup
    S.Shape(264, 136, 12, 3, "f16"),     # payload 21.75 pages: zero pad before the first row
    S.Shape(2064, 2056, 3, 2, "f16"),    # 1316.25 pages: 2 rows per workgroup, pad over a page
], ids=["tiny", "ragged", "multi-row"])
def test_write_bank_trailers_and_crc32_match_the_oracle(torch_mod, shape):
    from synth import gpu as G
    inp = G.LayerInputs(shape, seed=31, layer=0)
    bank, stride, payload = _bank(torch_mod, inp, shape)
    b = bank.numpy()
    t0 = O.trailer_offset(payload)
    assert stride == t0 + 4096
    for e in range(shape.n_experts):
        rec = b[e * stride:(e + 1) * stride]
        assert O.record_check_flags(rec, e, shape.n_experts, stride, payload, shape.d, shape.ffn, verify=True) == 0, e
        assert not rec[payload:t0].any() and not rec[t0 + 48:].any()
    if shape is S.TINY:
        host_bank, _, _ = _bank(torch_mod, inp, shape, from_host=True)
        assert np.array_equal(host_bank.numpy(), b)


# --------------------------------------------------------------------------- streaming from a clean bank
def test_clean_bank_streams_like_resident_codes_with_every_fill_checked(torch_mod):
    shape = S.TINY
    from synth import gpu as G
    inp = G.LayerInputs(shape, seed=0, layer=0)
    bank, stride, payload = _bank(torch_mod, inp, shape)
    st = _layer(inp, shape, bank, max_tokens=4, codes_location=2, cache_slots=5, verify_records=True)
    rs = _layer(inp, shape, inp.codes_dev)
    x = S.tokens(0, 700, 20, shape.d)
    a = _tokens(torch_mod, st, shape, x)
    b = _tokens(torch_mod, rs, shape, x)
    st.sync()
    assert np.array_equal(a[0], b[0])
    err = np.linalg.norm(a[1] - b[1], axis=1) / np.linalg.norm(b[1], axis=1)
    assert err.max() <= 1e-6, err.max()
    # prefetched records are checked too (16 experts asked, 5 slots: some are copied)
    ids = torch_mod.arange(16, dtype=torch_mod.int32, device="cuda").reshape(4, 4)
    st.prefetch(ids, 4, shape.top_k)
    st.sync()
    s = st.stats()
    assert s["prefetch_fills"] > 0
    fills = s["slot_misses"] + s["prefetch_fills"]
    assert s["records_checked"] == s["records_verified"] == fills
    assert s["h2d_bytes"] == fills * stride
    assert st.close() == 0
    # the handle's own bank (pinned canonical codes) is checked the same way
    canon = torch_mod.empty(inp.codes_dev.shape, dtype=torch_mod.uint8, pin_memory=True)
    canon.copy_(inp.codes_dev)
    own = _layer(inp, shape, canon, codes_location=1, cache_slots=4, verify_records=True)
    c = _tokens(torch_mod, own, shape, x[:6])
    own.sync()
    assert np.array_equal(c[0], b[0][:6])
    assert own.stats()["records_verified"] == own.stats()["slot_misses"] > 0
    own.close()
    rs.close()


# --------------------------------------------------------------------------- damage
def test_flipped_payload_byte_is_reported_only_with_crc(torch_mod):
    from vector_quantized_expert_amd import RvqMoeError
    from vector_quantized_expert_amd import rvq_moe as R
    shape = S.TINY
    from synth import gpu as G
    inp = G.LayerInputs(shape, seed=0, layer=0)
    bank, stride, payload = _bank(torch_mod, inp, shape)
    x = S.tokens(0, 900, 1, shape.d)
    rs = _layer(inp, shape, inp.codes_dev)
    ids = _tokens(torch_mod, rs, shape, x)[0][0]
    rs.close()
    e = int(ids[1])
    b = bank.numpy()
    b[e * stride + 777] ^= 0x5A
    rec = b[e * stride:(e + 1) * stride]
    kw = dict(n_experts=shape.n_experts, stride=stride, payload=payload, d=shape.d, ffn=shape.ffn)
    assert O.record_check_flags(rec, e, verify=False, **kw) == 0
    assert O.record_check_flags(rec, e, verify=True, **kw) == O.BAD_CRC
    plain = _layer(inp, shape, bank, codes_location=2, cache_slots=4)
    _tokens(torch_mod, plain, shape, x)
    plain.sync()  # the trailer checks pass: the damage is in the payload
    assert plain.close() == 0
    ver = _layer(inp, shape, bank, codes_location=2, cache_slots=4, verify_records=True)
    _tokens(torch_mod, ver, shape, x)
    for _ in range(2):  # kept: every later sync reports it
        with pytest.raises(RvqMoeError) as ei:
            ver.sync()
        assert ei.value.status == R.ECORRUPT
        assert _flags_of(str(ei.value)) == (O.BAD_CRC, e)
    with pytest.raises(RvqMoeError) as ei:
        ver.close()
    assert ei.value.status == R.ECORRUPT


def test_swapped_records_are_reported_without_crc(torch_mod):
    from vector_quantized_expert_amd import RvqMoeError
    from vector_quantized_expert_amd import rvq_moe as R
    shape = S.TINY
    from synth import gpu as G
    inp = G.LayerInputs(shape, seed=0, layer=0)
    bank, stride, payload = _bank(torch_mod, inp, shape)
    x = S.tokens(0, 910, 1, shape.d)
    rs = _layer(inp, shape, inp.codes_dev)
    ids = _tokens(torch_mod, rs, shape, x)[0][0]
    rs.close()
    st = _layer(inp, shape, bank, codes_location=2, cache_slots=4)  # open's host checks see a clean bank
    e1 = int(ids[0])
    e2 = (e1 + 5) % shape.n_experts
    b = bank.numpy()
    r1 = b[e1 * stride:(e1 + 1) * stride].copy()
    b[e1 * stride:(e1 + 1) * stride] = b[e2 * stride:(e2 + 1) * stride]
    b[e2 * stride:(e2 + 1) * stride] = r1
    kw = dict(n_experts=shape.n_experts, stride=stride, payload=payload, d=shape.d, ffn=shape.ffn, verify=False)
    want, worst = 0, -1
    for e in ids.tolist():
        f = O.record_check_flags(b[e * stride:(e + 1) * stride], e, **kw)
        want |= f
        if f:
            worst = max(worst, e)
    assert want == O.BAD_ID | O.BAD_RANGE
    _tokens(torch_mod, st, shape, x)
    with pytest.raises(RvqMoeError) as ei:
        st.sync()
    assert ei.value.status == R.ECORRUPT
    assert _flags_of(str(ei.value)) == (want, worst)
    with pytest.raises(RvqMoeError):
        st.close()


def test_open_refuses_banks_with_wrong_trailers(torch_mod):
    from vector_quantized_expert_amd import RvqMoeError
    from vector_quantized_expert_amd import rvq_moe as R
    shape = S.TINY
    from synth import gpu as G
    inp = G.LayerInputs(shape, seed=0, layer=0)
    bank, stride, payload = _bank(torch_mod, inp, shape)
    b = bank.numpy()
    t0 = O.trailer_offset(payload)
    last = (shape.n_experts - 1) * stride + t0
    saved = b[last:last + 48].copy()
    b[last:last + 48] = 0  # a bank cut short: the last trailer is missing
    with pytest.raises(RvqMoeError) as ei:
        _layer(inp, shape, bank, codes_location=2, cache_slots=4)
    assert ei.value.status == R.ECORRUPT and f"record {shape.n_experts - 1}" in str(ei.value)
    b[last:last + 48] = saved
    b[3 * stride + t0 + 8] ^= 1  # record 3 claims another expert
    with pytest.raises(RvqMoeError) as ei:
        _layer(inp, shape, bank, codes_location=2, cache_slots=4)
    assert ei.value.status == R.ECORRUPT and "record 3" in str(ei.value)
    b[3 * stride + t0 + 8] ^= 1
    # a bank written for another shape
    other = S.Shape(264, 136, 12, 3, "f32")
    oinp = G.LayerInputs(other, seed=1, layer=0)
    obank, _, _ = _bank(torch_mod, oinp, other)
    assert obank.numel() >= shape.n_experts * stride
    with pytest.raises(RvqMoeError) as ei:
        _layer(inp, shape, obank, codes_location=2, cache_slots=4)
    assert ei.value.status == R.ECORRUPT
    # the repaired bank opens
    ok = _layer(inp, shape, bank, codes_location=2, cache_slots=4)
    assert ok.close() == 0
