"""rvq_moe_layer_forward_noalloc (scratch in a static device array) against
rvq_moe_layer_forward (scratch in the handle's workspace), through the C ABI.

Same inputs, ids and gates: outputs agree within 1e-6 relative L2 per token
(both accumulate the output with fp32 atomics, whose order varies) and both
follow the oracle at the 1e-4 bar; two calls in a row, the second smaller,
and a call of another handle in between (the static array is shared by every
handle on the GPU and keeps the last call's contents).
"""
import numpy as np
import pytest

from oracle import oracle as O
from synth import synth as S

pytestmark = pytest.mark.gpu


def _layer(inp, shape, max_tokens, **kw):
    from vector_quantized_expert_amd import RvqMoe
    return RvqMoe(d=shape.d, ffn=shape.ffn, n_experts=shape.n_experts, top_k=shape.top_k,
                  codebook_dtype=0 if shape.cb_dtype == "f32" else 1, router_w=inp.w_r_dev,
                  codebooks=inp.cb_dev, codes=inp.codes_dev, max_tokens=max_tokens, **kw)


def _both(torch, layer, shape, x):
    from synth import gpu as G
    T = x.shape[0]
    xd = G.to_device(x)
    ids = torch.empty((T, shape.top_k), dtype=torch.int32, device="cuda")
    gates = torch.empty((T, shape.top_k), device="cuda")
    y_ws = torch.empty((T, shape.d), device="cuda")
    y_st = torch.full((T, shape.d), float("nan"), device="cuda")
    layer.route_topk(xd, T, ids, gates)
    layer.layer_forward(xd, T, ids, gates, y_ws)
    layer.layer_forward_noalloc(xd, T, ids, gates, y_st)
    layer.sync()
    return ids.cpu().numpy(), gates.cpu().numpy(), y_ws.cpu().numpy(), y_st.cpu().numpy()


def _compare(inp, shape, x, ids, gates, y_ws, y_st, tokens=None):
    assert np.all(np.isfinite(y_st))
    err = np.linalg.norm(y_st - y_ws, axis=1) / np.linalg.norm(y_ws, axis=1)
    assert err.max() <= 1e-6, err.max()
    for t in (range(x.shape[0]) if tokens is None else tokens):
        ref = O.layer(x[t], inp.w_r, shape.top_k, inp.codebook, inp.record, shape.d, shape.ffn)
        assert np.array_equal(ids[t], ref.route.ids)
        assert np.linalg.norm(y_st[t] - ref.delta) / np.linalg.norm(ref.delta) <= 1e-4


def test_noalloc_matches_layer_forward_two_calls_second_smaller():
    import torch
    from synth import gpu as G
    shape = S.TINY
    inp = G.LayerInputs(shape, seed=0, layer=3, host_codes=True)
    other = G.LayerInputs(S.Shape(264, 136, 5, 2, "f16"), seed=1, layer=0, host_codes=True)
    a = _layer(inp, shape, 8)
    b = _layer(other, other.shape, 4)
    for T, t0 in ((6, 0), (2, 50)):   # the second call is smaller
        x = S.tokens(3, t0, T, shape.d)
        ids, gates, y_ws, y_st = _both(torch, a, shape, x)
        _compare(inp, shape, x, ids, gates, y_ws, y_st)
        # another handle's call on the same GPU in between: it leaves its own
        # contents in the shared array
        xb = S.tokens(1, t0, 3, other.shape.d)
        ids, gates, y_ws, y_st = _both(torch, b, other.shape, xb)
        _compare(other, other.shape, xb, ids, gates, y_ws, y_st)
    a.close()
    b.close()


def test_noalloc_k3_batch1_and_scratch_limit():
    import torch
    from synth import gpu as G
    from vector_quantized_expert_amd import RvqMoeError
    from vector_quantized_expert_amd import rvq_moe as R
    shape = S.K3
    inp = G.LayerInputs(shape, seed=0, layer=11)
    layer = _layer(inp, shape, 8)
    inp.free_codes()
    torch.cuda.empty_cache()
    for T, t0 in ((2, 0), (1, 10)):   # the second call is smaller
        x = S.tokens(0, 11000 + t0, T, shape.d)
        ids, gates, y_ws, y_st = _both(torch, layer, shape, x)
        _compare(inp, shape, x, ids, gates, y_ws, y_st, tokens=[0])
    # five K3 tokens need 36.7 MB of scratch, above the static 32 MiB: refused
    # before anything is enqueued
    x = torch.zeros((5, shape.d), device="cuda")
    ids = torch.zeros((5, shape.top_k), dtype=torch.int32, device="cuda")
    g = torch.zeros((5, shape.top_k), device="cuda")
    y = torch.zeros((5, shape.d), device="cuda")
    with pytest.raises(RvqMoeError) as ei:
        layer.layer_forward_noalloc(x, 5, ids, g, y)
    assert ei.value.status == R.EINVAL
    assert torch.count_nonzero(y).item() == 0
    layer.close()


def test_noalloc_deterministic_is_bitwise_layer_forward():
    """With deterministic=1 the allocation-free call (output rows in the static
    array too) gives the same bits as rvq_moe_layer_forward, twice in a row
    (the second call smaller)."""
    import torch
    from synth import gpu as G
    shape = S.Shape(264, 136, 5, 2, "f16")
    inp = G.LayerInputs(shape, seed=2, layer=1, host_codes=True)
    layer = _layer(inp, shape, 8, deterministic=1)
    for T, t0 in ((7, 0), (3, 20)):
        x = S.tokens(2, t0, T, shape.d)
        ids, gates, y_ws, y_st = _both(torch, layer, shape, x)
        assert np.array_equal(y_ws, y_st)
        _compare(inp, shape, x, ids, gates, y_ws, y_st, tokens=[0])
    layer.close()
