"""GPU parity of the HIP path against the CPU oracle, through the C ABI.

Bars: expert ids bit-exact (compared as ordered lists); gates within 1e-6
relative of the oracle's fp64 gates; layer outputs within 1e-4 relative L2
per token (taken on the MoE output before any residual add).  Inputs are the
seeded synthetic ones of synth/synth.py.
"""
import numpy as np
import pytest

from oracle import oracle as O
from synth import synth as S

pytestmark = pytest.mark.gpu

TOL_Y = 1e-4
TOL_G = 1e-6


@pytest.fixture(scope="module")
def torch_mod():
    import torch
    assert torch.cuda.is_available()
    return torch


def _layer(torch, inp, shape, max_tokens, **kw):
    from vector_quantized_expert_amd import RvqMoe
    return RvqMoe(d=shape.d, ffn=shape.ffn, n_experts=shape.n_experts, top_k=shape.top_k,
                  codebook_dtype=0 if shape.cb_dtype == "f32" else 1, router_w=inp.w_r_dev,
                  codebooks=inp.cb_dev, codes=kw.pop("codes", inp.codes_dev), max_tokens=max_tokens, **kw)


def _run(torch, layer, shape, x, per_token=False):
    from synth import gpu as G
    T = x.shape[0]
    xd = G.to_device(x)
    ids = torch.empty((T, shape.top_k), dtype=torch.int32, device="cuda")
    gates = torch.empty((T, shape.top_k), dtype=torch.float32, device="cuda")
    y = torch.empty((T, shape.d), dtype=torch.float32, device="cuda")
    if per_token:
        for t in range(T):
            layer.route_topk(xd[t:t + 1], 1, ids[t:t + 1], gates[t:t + 1])
            layer.layer_forward(xd[t:t + 1], 1, ids[t:t + 1], gates[t:t + 1], y[t:t + 1])
    else:
        layer.route_topk(xd, T, ids, gates)
        layer.layer_forward(xd, T, ids, gates, y)
    layer.sync()
    return ids.cpu().numpy(), gates.cpu().numpy(), y.cpu().numpy()


def _forward(torch, layer, shape, x, ids, gates, per_token=False):
    """layer_forward on given ids and gates (host arrays): one call, or one token per call."""
    from synth import gpu as G
    T = x.shape[0]
    xd, idd, gd = G.to_device(x), G.to_device(ids), G.to_device(gates)
    y = torch.empty((T, shape.d), dtype=torch.float32, device="cuda")
    if per_token:
        for t in range(T):
            layer.layer_forward(xd[t:t + 1], 1, idd[t:t + 1], gd[t:t + 1], y[t:t + 1])
    else:
        layer.layer_forward(xd, T, idd, gd, y)
    layer.sync()
    return y.cpu().numpy()


def _check(inp, shape, x, ids, gates, y, pre_rmsnorm=False, residual=False, tokens=None):
    worst = 0.0
    for t in (range(x.shape[0]) if tokens is None else tokens):
        ref = O.layer(x[t], inp.w_r, shape.top_k, inp.codebook, inp.record, shape.d, shape.ffn,
                      pre_rmsnorm=pre_rmsnorm, eps=1e-6)
        if ref.route.margin > 1e-9 and ref.route.min_gap > 1e-9:
            assert np.array_equal(ids[t], ref.route.ids), (t, ids[t], ref.route.ids)
        else:  # a logit tie within 1e-9: only the selected set is unique
            assert set(ids[t].tolist()) == set(ref.route.ids.tolist())
        np.testing.assert_allclose(gates[t], ref.route.gates, rtol=TOL_G, atol=0)
        delta = y[t].astype(np.float64) - (x[t].astype(np.float64) if residual else 0.0)
        nrm = np.linalg.norm(ref.delta)
        err = np.linalg.norm(delta - ref.delta) / nrm if nrm > 0 else np.abs(delta).max()
        assert err <= TOL_Y, (t, err)
        worst = max(worst, err)
    return worst


# --------------------------------------------------------------------------- generator
def test_device_code_generator_matches_host(torch_mod):
    from synth import gpu as G
    rb = S.record_bytes(256, 128)
    dev = G.codes_on_device(3, 1, 4, rb).cpu().numpy()
    host = S.codes_bank(3, 1, 4, rb)
    assert np.array_equal(dev, host)
    rb = S.K3.record_bytes
    dev = G.codes_on_device(0, 0, 1, rb, expert0=383).cpu().numpy()[0]
    assert np.array_equal(dev[:1 << 20], S.expert_record(0, 0, 383, rb, 0, 1 << 17))
    assert np.array_equal(dev[-4096:], S.expert_record(0, 0, 383, rb, rb // 8 - 512, rb // 8))


# --------------------------------------------------------------------------- tiny layer
@pytest.fixture(scope="module")
def tiny(torch_mod):
    from synth import gpu as G
    return G.LayerInputs(S.TINY, seed=0, layer=0, host_codes=True)


def test_tiny_layer_64_tokens(torch_mod, tiny):
    shape = S.TINY
    layer = _layer(torch_mod, tiny, shape, 64, chunk_min_tokens=65)  # the table path
    x = S.tokens(0, 0, 64, shape.d)
    ids, gates, y = _run(torch_mod, layer, shape, x)
    worst = _check(tiny, shape, x, ids, gates, y)
    print(f"tiny layer worst rel L2 {worst:.3e}")
    layer.close()


def test_tiny_per_token_calls_match_batched_call(torch_mod, tiny):
    """Ids and gates are bitwise identical whether tokens come one per call or
    all in one call, and across repeated calls.  Outputs are accumulated with
    fp32 atomics (summation order varies), so they agree to 1e-6 relative."""
    shape = S.TINY
    layer = _layer(torch_mod, tiny, shape, 16)
    x = S.tokens(0, 100, 16, shape.d)
    a = _run(torch_mod, layer, shape, x)
    b = _run(torch_mod, layer, shape, x, per_token=True)
    c = _run(torch_mod, layer, shape, x)
    for other in (b, c):
        assert np.array_equal(a[0], other[0]) and np.array_equal(a[1], other[1])
        err = np.linalg.norm(a[2] - other[2], axis=1) / np.linalg.norm(a[2], axis=1)
        assert err.max() <= 1e-6, err.max()
    layer.close()


@pytest.mark.parametrize("d,ffn,E,k,cb", [
    (8, 8, 1, 1, "f32"),          # smallest: one slice, one row chunk (ragged)
    (264, 136, 5, 2, "f16"),      # ragged slice tile (33 slices) and ragged row chunk (136 rows)
    (520, 72, 7, 7, "f32"),       # k == E, 65 slices -> 3 tiles, down over 9 slices
    (1024, 520, 9, 3, "f16"),     # several tiles in both directions
])
def test_ragged_shapes(torch_mod, d, ffn, E, k, cb):
    from synth import gpu as G
    shape = S.Shape(d, ffn, E, k, cb)
    inp = G.LayerInputs(shape, seed=5, layer=2, host_codes=True)
    layer = _layer(torch_mod, inp, shape, 3)
    x = S.tokens(5, 0, 3, d)
    ids, gates, y = _run(torch_mod, layer, shape, x)
    _check(inp, shape, x, ids, gates, y)
    layer.close()


@pytest.mark.parametrize("d,ffn,E,k,cb", [
    (16392, 16, 3, 2, "f32"),     # 2049 slices: 65 input tiles, just past one 64-bit slot mask
    (40968, 24, 2, 1, "f16"),     # 5121 slices: 161 input tiles (three mask words)
])
def test_wide_hidden_size_past_64_input_tiles(torch_mod, d, ffn, E, k, cb):
    """Hidden sizes whose gate/up matrices have more than 64 input tiles: the
    SwiGLU finish must sum the partial slots of every tile, in the batch-1
    pair order (merged slots), the grouped order, and the routed launch."""
    from synth import gpu as G
    shape = S.Shape(d, ffn, E, k, cb)
    inp = G.LayerInputs(shape, seed=41, layer=0, host_codes=True)
    layer = _layer(torch_mod, inp, shape, 3)
    x = S.tokens(41, 0, 3, d)
    ids, gates, y = _run(torch_mod, layer, shape, x, per_token=True)
    _check(inp, shape, x, ids, gates, y)
    ids, gates, y = _run(torch_mod, layer, shape, x)
    _check(inp, shape, x, ids, gates, y)
    xd = G.to_device(x[:1])
    ids_d = torch_mod.empty((1, k), dtype=torch_mod.int32, device="cuda")
    g_d = torch_mod.empty((1, k), device="cuda")
    y_d = torch_mod.empty((1, d), device="cuda")
    layer.route_forward(xd, 1, ids_d, g_d, y_d)
    layer.sync()
    _check(inp, shape, x[:1], ids_d.cpu().numpy(), g_d.cpu().numpy(), y_d.cpu().numpy())
    layer.close()


@pytest.mark.parametrize("scale_exp", [-24, -8, 0, 12, 20])
def test_fp32_codebooks_at_any_scale(torch_mod, scale_exp):
    """fp32 codebooks scaled by 2^s (s = -24 .. 20: entries from ~1e-10 to
    beyond the fp16 range) follow the oracle at the 1e-4 bar on the table
    path, and scaling the up and down codebooks by powers of two scales the
    output exactly (bitwise; one expert per token and one down tile, so every
    output element is a single addition onto zero)."""
    from synth import gpu as G
    shape = S.Shape(264, 136, 5, 1, "f32")
    base = G.LayerInputs(shape, seed=43, layer=0, host_codes=True)
    cb0 = base.cb.copy()
    base.cb = np.ldexp(cb0, scale_exp).astype(np.float32)
    base.cb_dev.copy_(G.to_device(base.cb))
    layer = _layer(torch_mod, base, shape, 4)
    x = S.tokens(43, 0, 4, shape.d)
    ids, gates, y = _run(torch_mod, layer, shape, x)
    _check(base, shape, x, ids, gates, y)
    layer.close()
    # up scaled by 2^3, down by 2^-5 (gate unchanged): y scales by 2^-2 exactly
    scaled = np.array(base.cb)
    scaled[:, 1] = np.ldexp(scaled[:, 1], 3)
    scaled[:, 2] = np.ldexp(scaled[:, 2], -5)
    base.cb_dev.copy_(G.to_device(scaled))
    layer = _layer(torch_mod, base, shape, 4)
    ids2, gates2, y2 = _run(torch_mod, layer, shape, x)
    assert np.array_equal(ids, ids2)
    assert np.array_equal(y2, np.ldexp(y, -2).astype(np.float32))
    layer.close()


def test_zero_codebooks_give_exact_zero(torch_mod, tiny):
    from synth import gpu as G
    shape = S.TINY
    tiny_zero = G.LayerInputs(shape, seed=0, layer=0, host_codes=True)
    tiny_zero.cb_dev.zero_()
    layer = _layer(torch_mod, tiny_zero, shape, 4)
    x = S.tokens(0, 7, 4, shape.d)
    _, _, y = _run(torch_mod, layer, shape, x)
    assert np.all(y == 0.0)
    layer.close()


def test_constant_codebooks_closed_form(torch_mod):
    """Stage constants alpha_{m,s}: every weight of matrix m is A_m whatever the
    codes, so a = A_g sum(x), b = A_u sum(x), y = A_d * ffn * silu(a) * b."""
    from synth import gpu as G
    shape = S.Shape(512, 256, 8, 3, "f16")
    inp = G.LayerInputs(shape, seed=1, layer=0, host_codes=True)
    al = np.array([[0.0625, 0.015625, -0.00390625], [-0.03125, 0.0078125, 0.001953125],
                   [0.015625, -0.00390625, 0.0009765625]])
    cb = np.broadcast_to(al[None, :, :, None, None], inp.cb.shape).astype(np.float16)
    inp.cb = np.ascontiguousarray(cb)
    inp.cb_dev.copy_(G.to_device(inp.cb))
    layer = _layer(torch_mod, inp, shape, 2)
    x = S.tokens(1, 0, 2, shape.d)
    _, _, y = _run(torch_mod, layer, shape, x)
    A = al.sum(axis=1)
    for t in range(2):
        s = x[t].astype(np.float64).sum()
        a, b = A[0] * s, A[1] * s
        ref = A[2] * shape.ffn * (a / (1 + np.exp(-a))) * b
        np.testing.assert_allclose(y[t], ref, rtol=1e-4)
    layer.close()


def test_rmsnorm_residual_chain_teacher_forced(torch_mod):
    """Three layers with RMS normalisation before routing and a residual add:
    each GPU layer is checked against the oracle fed the GPU's own input."""
    from synth import gpu as G
    shape = S.Shape(512, 256, 32, 8, "f16")
    T = 4
    h = S.tokens(9, 0, T, shape.d)
    for L in range(3):
        inp = G.LayerInputs(shape, seed=9, layer=L, host_codes=True)
        layer = _layer(torch_mod, inp, shape, T, pre_rmsnorm=True, residual=True, eps=1e-6)
        ids, gates, y = _run(torch_mod, layer, shape, h)
        _check(inp, shape, h, ids, gates, y, pre_rmsnorm=True, residual=True)
        layer.close()
        h = y


def test_invalid_ids_are_reported_and_poison_only_their_token(torch_mod, tiny):
    from synth import gpu as G
    from vector_quantized_expert_amd import RvqMoeError
    from vector_quantized_expert_amd import rvq_moe as R
    shape = S.TINY
    layer = _layer(torch_mod, tiny, shape, 2)
    x = G.to_device(S.tokens(0, 0, 2, shape.d))
    ids = torch_mod.tensor([[0, 1, 2, 3], [0, 1, shape.n_experts + 5, 3]], dtype=torch_mod.int32, device="cuda")
    gates = torch_mod.full((2, 4), 0.25, device="cuda")
    y = torch_mod.zeros((2, shape.d), device="cuda")
    layer.layer_forward(x, 2, ids, gates, y)
    with pytest.raises(RvqMoeError) as ei:
        layer.sync()
    assert ei.value.status == R.EDEVICE
    yh = y.cpu().numpy()
    assert np.all(np.isfinite(yh[0])) and np.all(np.isnan(yh[1]))
    layer.sync()  # the error was cleared
    layer.close()


def test_call_validation(torch_mod, tiny):
    from vector_quantized_expert_amd import RvqMoeError
    shape = S.TINY
    layer = _layer(torch_mod, tiny, shape, 2)
    x = torch_mod.zeros((4, shape.d), device="cuda")
    ids = torch_mod.zeros((4, 4), dtype=torch_mod.int32, device="cuda")
    g = torch_mod.zeros((4, 4), device="cuda")
    with pytest.raises(RvqMoeError):
        layer.route_topk(x, 3, ids, g)        # above max_tokens
    with pytest.raises(RvqMoeError):
        layer.layer_forward(x, 0, ids, g, x)  # empty
    with pytest.raises(RvqMoeError):
        layer.layer_forward(x, 1, ids, g, x)  # y aliases x
    layer.close()


# --------------------------------------------------------------------------- K3-scale layer
def test_k3_layer_batch1_sampled_tokens(torch_mod):
    """d=7168, ffn=2048, E=384, top-16, fp16 codebooks, T=1 per call (the
    benchmark's launch configuration); tokens checked one by one."""
    from synth import gpu as G
    shape = S.K3
    inp = G.LayerInputs(shape, seed=0, layer=0)
    layer = _layer(torch_mod, inp, shape, 1)
    inp.free_codes()
    torch_mod.cuda.empty_cache()
    x = S.tokens(0, 0, 3, shape.d)
    ids, gates, y = _run(torch_mod, layer, shape, x, per_token=True)
    worst = _check(inp, shape, x, ids, gates, y)
    print(f"K3 layer worst rel L2 {worst:.3e}")
    layer.close()


def test_k3_every_expert_record_against_the_oracle(torch_mod):
    """Explicit ids 0..383 in 24 tokens of 16: every expert record of the
    K3-scale layer (offsets up to 6.3 GB) is read and checked against the
    oracle, through one grouped 24-token call and through 24 one-token calls
    (the batch-1 launch configuration)."""
    from synth import gpu as G
    shape = S.K3
    T = shape.n_experts // shape.top_k
    inp = G.LayerInputs(shape, seed=0, layer=7)
    layer = _layer(torch_mod, inp, shape, T)
    inp.free_codes()
    torch_mod.cuda.empty_cache()
    x = S.tokens(0, 7000, T, shape.d)
    ids = np.arange(shape.n_experts, dtype=np.int32).reshape(T, shape.top_k)
    rng = np.random.default_rng(7)
    gates = rng.random((T, shape.top_k)).astype(np.float32) + 0.5
    gates /= gates.sum(axis=1, keepdims=True)
    xd, ids_d, g_d = G.to_device(x), G.to_device(ids), G.to_device(gates)
    y_grp = torch_mod.empty((T, shape.d), device="cuda")
    y_one = torch_mod.empty((T, shape.d), device="cuda")
    layer.layer_forward(xd, T, ids_d, g_d, y_grp)
    for t in range(T):
        layer.layer_forward(xd[t:t + 1], 1, ids_d[t:t + 1], g_d[t:t + 1], y_one[t:t + 1])
    layer.sync()
    yg, yo = y_grp.cpu().numpy(), y_one.cpu().numpy()
    worst = 0.0
    for t in range(T):
        recs = [inp.record(int(e)) for e in ids[t]]
        ref = O.moe(shape.d, shape.ffn, gates[t].astype(np.float64), [inp.codebook(int(e)) for e in ids[t]], recs,
                    x[t].astype(np.float64))
        for yy in (yg, yo):
            err = np.linalg.norm(yy[t] - ref) / np.linalg.norm(ref)
            assert err <= TOL_Y, (t, err)
            worst = max(worst, err)
    print(f"K3 all 384 experts: worst rel L2 {worst:.3e}")
    layer.close()


def test_k3_depth_chain_teacher_forced(torch_mod):
    """Four K3-scale layers (d=7168, ffn=2048, E=384, top-16) with RMS
    normalisation before routing and a residual add, each call one token
    through rvq_moe_route_forward (the batch-1 launch configuration): every
    layer against the oracle fed the GPU's own input of that layer."""
    from synth import gpu as G
    shape = S.K3
    L, T = 4, 2
    h = S.tokens(0, 9000, T, shape.d)
    for li in range(L):
        inp = G.LayerInputs(shape, seed=0, layer=20 + li)
        layer = _layer(torch_mod, inp, shape, 1, pre_rmsnorm=True, residual=True, eps=1e-6)
        inp.free_codes()
        torch_mod.cuda.empty_cache()
        hd = G.to_device(h)
        ids = torch_mod.empty((T, shape.top_k), dtype=torch_mod.int32, device="cuda")
        gates = torch_mod.empty((T, shape.top_k), device="cuda")
        y = torch_mod.empty((T, shape.d), device="cuda")
        for t in range(T):
            layer.route_forward(hd[t:t + 1], 1, ids[t:t + 1], gates[t:t + 1], y[t:t + 1])
        layer.sync()
        yh = y.cpu().numpy()
        worst = _check(inp, shape, h, ids.cpu().numpy(), gates.cpu().numpy(), yh, pre_rmsnorm=True, residual=True)
        print(f"K3 chain layer {li}: worst rel L2 {worst:.3e}")
        layer.close()
        del inp
        torch_mod.cuda.empty_cache()
        h = yh


def test_router_ties_go_to_the_lower_id_and_k_equals_e(torch_mod):
    """Experts 3 and 9 (and 5, 11) get identical router columns, so their logits
    tie exactly on both sides; the lower id must come first, as in the oracle."""
    from synth import gpu as G
    shape = S.Shape(256, 64, 12, 12, "f32")
    inp = G.LayerInputs(shape, seed=4, layer=0, host_codes=True)
    inp.w_r[:, 9] = inp.w_r[:, 3]
    inp.w_r[:, 11] = inp.w_r[:, 5]
    inp.w_r_dev.copy_(G.to_device(inp.w_r))
    layer = _layer(torch_mod, inp, shape, 4)
    x = S.tokens(4, 0, 4, shape.d)
    ids, gates, y = _run(torch_mod, layer, shape, x)
    for t in range(4):
        ref = O.layer(x[t], inp.w_r, shape.top_k, inp.codebook, inp.record, shape.d, shape.ffn)
        assert np.array_equal(ids[t], ref.route.ids)
        pos = {int(e): j for j, e in enumerate(ids[t])}
        assert pos[3] + 1 == pos[9] and pos[5] + 1 == pos[11]
        np.testing.assert_allclose(gates[t], ref.route.gates, rtol=TOL_G)
    layer.close()


@pytest.mark.parametrize("shape_args,T,pre", [
    ((256, 128, 16, 4, "f32"), 8, False),
    ((264, 136, 5, 2, "f16"), 3, False),
    ((512, 256, 32, 8, "f16"), 4, True),
])
def test_route_forward_one_launch_matches_two_calls_and_oracle(torch_mod, shape_args, T, pre):
    from synth import gpu as G
    shape = S.Shape(*shape_args)
    inp = G.LayerInputs(shape, seed=13, layer=1, host_codes=True)
    layer = _layer(torch_mod, inp, shape, T, pre_rmsnorm=pre, residual=pre, eps=1e-6)
    x = S.tokens(13, 0, T, shape.d)
    xd = G.to_device(x)
    ids = torch_mod.empty((T, shape.top_k), dtype=torch_mod.int32, device="cuda")
    gates = torch_mod.empty((T, shape.top_k), dtype=torch_mod.float32, device="cuda")
    y = torch_mod.empty((T, shape.d), dtype=torch_mod.float32, device="cuda")
    for _ in range(2):  # second call checks that the in-launch counters were reset
        layer.route_forward(xd, T, ids, gates, y)
        layer.sync()
    fused = (ids.cpu().numpy(), gates.cpu().numpy(), y.cpu().numpy())
    two = _run(torch_mod, layer, shape, x)
    _check(inp, shape, x, *fused, pre_rmsnorm=pre, residual=pre)
    assert np.array_equal(fused[0], two[0])
    np.testing.assert_allclose(fused[1], two[1], rtol=1e-6)
    err = np.linalg.norm(fused[2] - two[2], axis=1) / np.linalg.norm(two[2], axis=1)
    assert err.max() <= 1e-6
    layer.close()


@pytest.mark.parametrize("case", ["tied_groups", "many_zero_logits"])
def test_route_forward_exact_selection_with_ties(torch_mod, case):
    """The one-launch routing selects each token's top k from candidates at or
    above the k-th largest maximum of the 16-expert groups.  tied_groups: every
    group holds the same 16 router columns, so all group maxima tie and the top
    k are equal logits from different groups (lower ids first).  many_zero_logits:
    all but 6 router columns are zero, so the k-th place is usually among 122
    exact zeros (more than 64 candidates).  Ids must equal the oracle's."""
    from synth import gpu as G
    shape = S.Shape(256, 64, 128, 4, "f32")
    inp = G.LayerInputs(shape, seed=21, layer=0, host_codes=True)
    if case == "tied_groups":
        for e in range(16, shape.n_experts):
            inp.w_r[:, e] = inp.w_r[:, e % 16]
    else:
        keep = [7, 19, 40, 77, 100, 127]
        for e in range(shape.n_experts):
            if e not in keep:
                inp.w_r[:, e] = 0.0
    inp.w_r_dev.copy_(G.to_device(inp.w_r))
    T = 6
    layer = _layer(torch_mod, inp, shape, T)
    x = S.tokens(21, 0, T, shape.d)
    ids = torch_mod.empty((T, shape.top_k), dtype=torch_mod.int32, device="cuda")
    gates = torch_mod.empty((T, shape.top_k), dtype=torch_mod.float32, device="cuda")
    y = torch_mod.empty((T, shape.d), dtype=torch_mod.float32, device="cuda")
    layer.route_forward(G.to_device(x), T, ids, gates, y)
    layer.sync()
    ih, gh = ids.cpu().numpy(), gates.cpu().numpy()
    n_zero_in_top = 0
    for t in range(T):
        ref = O.route(x[t], inp.w_r, shape.top_k)
        assert np.array_equal(ih[t], ref.ids), (t, ih[t], ref.ids)
        np.testing.assert_allclose(gh[t], ref.gates, rtol=TOL_G, atol=0)
        n_zero_in_top += int(np.sum(ref.logits[ih[t]] == 0.0))
    if case == "many_zero_logits":
        assert n_zero_in_top > 0  # the boundary did fall among the zeros
    layer.close()


def test_k3_route_forward_batch1(torch_mod):
    from synth import gpu as G
    shape = S.K3
    inp = G.LayerInputs(shape, seed=0, layer=0)
    layer = _layer(torch_mod, inp, shape, 1)
    inp.free_codes()
    torch_mod.cuda.empty_cache()
    x = S.tokens(0, 500, 2, shape.d)
    xd = G.to_device(x)
    ids = torch_mod.empty((2, shape.top_k), dtype=torch_mod.int32, device="cuda")
    gates = torch_mod.empty((2, shape.top_k), dtype=torch_mod.float32, device="cuda")
    y = torch_mod.empty((2, shape.d), dtype=torch_mod.float32, device="cuda")
    for t in range(2):
        layer.route_forward(xd[t], 1, ids[t], gates[t], y[t])
    layer.sync()
    _check(inp, shape, x, ids.cpu().numpy(), gates.cpu().numpy(), y.cpu().numpy())
    layer.close()


# --------------------------------------------------------------------------- batched decode (pair order)
def test_explicit_ids_with_repeats_follow_the_oracle(torch_mod, tiny):
    """Caller-supplied ids may repeat within a token and across tokens; the
    expert-grouped pair order must still give every pair its own gate-weighted
    contribution."""
    from synth import gpu as G
    shape = S.TINY
    T = 6
    ids_h = np.array([[2, 2, 2, 2], [2, 5, 7, 2], [0, 15, 8, 1], [15, 15, 3, 3], [5, 6, 7, 8], [9, 9, 9, 0]],
                     dtype=np.int32)
    rng = np.random.default_rng(21)
    gates_h = rng.uniform(-1.0, 1.0, size=(T, 4)).astype(np.float32)
    layer = _layer(torch_mod, tiny, shape, T)
    x = S.tokens(0, 300, T, shape.d)
    ids = torch_mod.tensor(ids_h, device="cuda")
    gates = torch_mod.tensor(gates_h, device="cuda")
    y = torch_mod.empty((T, shape.d), device="cuda")
    layer.layer_forward(G.to_device(x), T, ids, gates, y)
    layer.sync()
    yh = y.cpu().numpy()
    for t in range(T):
        ref = O.moe(shape.d, shape.ffn, gates_h[t].astype(np.float64), [tiny.codebook(int(e)) for e in ids_h[t]],
                    [tiny.record(int(e)) for e in ids_h[t]], x[t])
        err = np.linalg.norm(yh[t] - ref) / np.linalg.norm(ref)
        assert err <= TOL_Y, (t, err)
    layer.close()


def test_batch_beyond_the_order_table_uses_pair_order(torch_mod, tiny):
    """160 tokens x top-4 = 640 pairs: above the grouped-order table, so the
    pairs run in plain pair order; every token still matches the oracle."""
    shape = S.TINY
    layer = _layer(torch_mod, tiny, shape, 160, chunk_min_tokens=161)  # the table path
    x = S.tokens(0, 1000, 160, shape.d)
    ids, gates, y = _run(torch_mod, layer, shape, x)
    _check(tiny, shape, x, ids, gates, y)
    layer.close()


def test_k3_batch32_grouped_matches_per_token_and_oracle(torch_mod):
    """d=7168, ffn=2048, E=384, top-16, 32 tokens in one call (512 pairs, the
    expert-grouped order): the whole batch agrees with 32 one-token calls, and
    sampled tokens with the oracle.  The one-launch routed call is checked too."""
    from synth import gpu as G
    shape = S.K3
    T = 32
    inp = G.LayerInputs(shape, seed=0, layer=3)
    layer = _layer(torch_mod, inp, shape, T)
    inp.free_codes()
    torch_mod.cuda.empty_cache()
    x = S.tokens(0, 2000, T, shape.d)
    batched = _run(torch_mod, layer, shape, x)
    single = _run(torch_mod, layer, shape, x, per_token=True)
    assert np.array_equal(batched[0], single[0]) and np.array_equal(batched[1], single[1])
    err = np.linalg.norm(batched[2] - single[2], axis=1) / np.linalg.norm(single[2], axis=1)
    assert err.max() <= 1e-6, err.max()
    xd = G.to_device(x)
    ids = torch_mod.empty((T, shape.top_k), dtype=torch_mod.int32, device="cuda")
    gates = torch_mod.empty((T, shape.top_k), dtype=torch_mod.float32, device="cuda")
    y = torch_mod.empty((T, shape.d), dtype=torch_mod.float32, device="cuda")
    layer.route_forward(xd, T, ids, gates, y)
    layer.sync()
    assert np.array_equal(ids.cpu().numpy(), batched[0])
    err = np.linalg.norm(y.cpu().numpy() - batched[2], axis=1) / np.linalg.norm(batched[2], axis=1)
    assert err.max() <= 1e-6, err.max()
    worst = _check(inp, shape, x, *batched, tokens=[0, 17, 31])
    print(f"K3 batch-32 worst rel L2 {worst:.3e}")
    layer.close()


def test_grouped_blocks_dealt_within_each_xcd_match_per_token_calls(torch_mod):
    """512 pairs at d=1024, ffn=512 (64 tokens, 32 experts, top-8) on the table
    path: the grouped order deals whole (pair, tile) blocks round-robin to each XCD's workgroups
    in both phases (at least 4 blocks per workgroup).  With the deterministic
    combine the grouped call equals 64 one-token calls (pair order, contiguous
    ranges) bit for bit; the atomic combine agrees within 1e-6; sampled tokens
    follow the oracle."""
    from synth import gpu as G
    shape = S.Shape(1024, 512, 32, 8, "f16")
    T = 64
    inp = G.LayerInputs(shape, seed=71, layer=0, host_codes=True)
    # (the chunk threshold above the call: the table path at 64 tokens)
    det = _layer(torch_mod, inp, shape, T, deterministic=1, chunk_min_tokens=T + 1)
    fast = _layer(torch_mod, inp, shape, T, chunk_min_tokens=T + 1)
    x = S.tokens(71, 0, T, shape.d)
    a = _run(torch_mod, det, shape, x)
    assert np.array_equal(a[2], _forward(torch_mod, det, shape, x, a[0], a[1], per_token=True))
    f = _run(torch_mod, fast, shape, x)
    assert np.array_equal(a[0], f[0]) and np.array_equal(a[1], f[1])
    _same_outputs(a[2], f[2], False)
    _check(inp, shape, x, *f, tokens=[0, 31, 63])
    for h in (det, fast):
        h.close()


# --------------------------------------------------------------------------- chunk path (bf16 matrix cores)
TOL_Y_BF16 = 2e-2  # bf16 operands (weights, tokens, h) with fp32 accumulation


def _check_chunk(inp, shape, x, ids, gates, y, pre_rmsnorm=False, residual=False, tokens=None, table_experts=()):
    """Per token: ids bit-exact against the oracle, the MoE output within 2e-2
    relative L2 of the fp64 oracle, and every output element within
    chunk_model.element_tolerance of the chunk path's precision model (the
    documented bf16 roundings around exact products), so that one wrong
    element or row fails even where the L2 norm would hide it.  table_experts:
    experts adaptive dispatch hands to the fp32 table path (no rounding)."""
    import chunk_model as M
    worst = 0.0
    for t in (range(x.shape[0]) if tokens is None else tokens):
        ref = O.layer(x[t], inp.w_r, shape.top_k, inp.codebook, inp.record, shape.d, shape.ffn,
                      pre_rmsnorm=pre_rmsnorm, eps=1e-6)
        assert np.array_equal(ids[t], ref.route.ids), t
        delta = y[t].astype(np.float64) - (x[t].astype(np.float64) if residual else 0.0)
        err = np.linalg.norm(delta - ref.delta) / np.linalg.norm(ref.delta)
        assert err <= TOL_Y_BF16, (t, err)
        worst = max(worst, err)
        ym, peak, mass = M.layer(x[t], ids[t], gates[t], inp.codebook, inp.record, shape.d, shape.ffn,
                                 pre_rmsnorm=pre_rmsnorm, eps=1e-6, table_experts=table_experts)
        # the residual add is one more fp32 rounding of x + delta
        tol = M.element_tolerance(peak, mass) + (np.abs(y[t]) * 2.0 ** -23 if residual else 0.0)
        bad = np.nonzero(np.abs(delta - ym) > tol)[0]
        assert bad.size == 0, (t, bad[:8], delta[bad[:8]], ym[bad[:8]], tol[bad[:8]])
    return worst


@pytest.mark.parametrize("d,ffn,E,k,cb,T", [
    (256, 128, 16, 4, "f32", 64),     # the small layer; 64 tokens, 16 pairs per expert on average
    (264, 136, 5, 2, "f16", 200),     # ragged tiles and chunks; 80 tokens per expert: two 64-token passes
    (520, 72, 7, 7, "f32", 9),        # k == E: every expert gets every token
    (1024, 520, 9, 3, "f16", 33),     # several tiles both ways, ragged row chunks
    (8, 8, 1, 1, "f32", 1),           # smallest
])
def test_chunk_path_follows_the_oracle(torch_mod, d, ffn, E, k, cb, T):
    from synth import gpu as G
    shape = S.Shape(d, ffn, E, k, cb)
    inp = G.LayerInputs(shape, seed=17, layer=1, host_codes=True)
    layer = _layer(torch_mod, inp, shape, T, chunk_min_tokens=1)
    x = S.tokens(17, 0, T, d)
    ids, gates, y = _run(torch_mod, layer, shape, x)
    worst = _check_chunk(inp, shape, x, ids, gates, y)
    print(f"chunk path {shape} T={T}: worst rel L2 {worst:.3e}")
    layer.close()


def test_chunk_group_sizes_at_the_kernel_boundaries(torch_mod):
    """Explicit ids put exactly 32 tokens on one expert (the largest group one
    32-token tile holds), one token on another and 33 on a third (the kernels
    for larger groups), on a shape with ragged input tiles both ways and row
    chunks that leave most waves of the last workgroup past the matrix.  Every
    token is within the bf16 bar of the fp64 oracle on the same experts and,
    element by element, within the precision model's tolerance."""
    import chunk_model as M
    from synth import gpu as G
    shape = S.Shape(520, 264, 4, 2, "f16")
    T = 33
    inp = G.LayerInputs(shape, seed=29, layer=0, host_codes=True)
    layer = _layer(torch_mod, inp, shape, T, chunk_min_tokens=1, lut_expert_tokens=1)
    x = S.tokens(29, 0, T, shape.d)
    ids = np.zeros((T, 2), np.int32)
    ids[:, 0] = 2          # expert 2: all 33 tokens
    ids[:32, 1] = 0        # expert 0: exactly 32
    ids[32, 1] = 1         # expert 1: one token (expert 3: none)
    g = np.random.default_rng(29).uniform(0.2, 0.8, (T, 1))
    gates = np.concatenate([g, 1.0 - g], axis=1).astype(np.float32)
    y = _forward(torch_mod, layer, shape, x, ids, gates)
    for t in range(T):
        ref = O.moe(shape.d, shape.ffn, gates[t], [inp.codebook(int(e)) for e in ids[t]],
                    [inp.record(int(e)) for e in ids[t]], x[t])
        err = np.linalg.norm(y[t] - ref) / np.linalg.norm(ref)
        assert err <= TOL_Y_BF16, (t, err)
        ym, peak, mass = M.layer(x[t], ids[t], gates[t], inp.codebook, inp.record, shape.d, shape.ffn)
        bad = np.nonzero(np.abs(y[t] - ym) > M.element_tolerance(peak, mass))[0]
        assert bad.size == 0, (t, bad[:8], y[t][bad[:8]], ym[bad[:8]])
    layer.close()


def test_chunk_kernel_families_agree_bitwise(torch_mod):
    """The chunk path's two kernel families compute the same sums in the same
    order: 24 tokens in one call (96 pairs, 6 per expert: the replicated-
    codebook kernels) and the same tokens one per call (4 pairs: the one-copy
    kernels) give bitwise equal outputs with the deterministic combine, on
    ragged tiles both ways; and the oracle at the bf16 bar."""
    from synth import gpu as G
    shape = S.Shape(1032, 264, 16, 4, "f16")
    T = 24
    inp = G.LayerInputs(shape, seed=37, layer=0, host_codes=True)
    layer = _layer(torch_mod, inp, shape, T, chunk_min_tokens=1, lut_expert_tokens=1, deterministic=True)
    x = S.tokens(37, 0, T, shape.d)
    grp = _run(torch_mod, layer, shape, x)
    one = _run(torch_mod, layer, shape, x, per_token=True)
    assert np.array_equal(grp[0], one[0])
    assert np.array_equal(grp[2], one[2]), np.abs(grp[2] - one[2]).max()
    _check_chunk(inp, shape, x, *grp, tokens=[0, 11, 23])
    layer.close()


@pytest.mark.parametrize("cb", ["f32", "f16"])
def test_chunk_path_closed_form_element_by_element(torch_mod, cb):
    """Stage codebooks that are one-hot vectors scaled by 1, 2, 4 (signs per
    matrix): weight (r, 8j + i) is sum_s sign_s 2^s [code_s(r, j) % 8 == i], an
    integer in [-7, 7].  With small-integer tokens every weight, token and the
    pre-activations a, b are exact in bf16 and fp32, so a and b are exact index
    sums computed here by plain indexing; h is rounded to bf16 as the chunk path
    does, and the down projection is again an index sum of those h values.
    Every output element must match (a wrong code byte, stage, slice or lane
    picks a different h)."""
    import chunk_model as M
    from synth import gpu as G
    d, ffn, E, k, T = 264, 136, 5, 2, 24
    shape = S.Shape(d, ffn, E, k, cb)
    inp = G.LayerInputs(shape, seed=23, layer=0, host_codes=True)
    signs = [(1, 2, 4), (1, -2, 4), (-1, 2, 4)]
    cbv = np.zeros((E, 3, 3, 256, 8), np.float32)
    for m in range(3):
        for s_ in range(3):
            cbv[:, m, s_, np.arange(256), np.arange(256) % 8] = signs[m][s_]
    inp.cb = cbv.astype(shape.np_cb_dtype)
    inp.cb_dev.copy_(G.to_device(inp.cb))
    layer = _layer(torch_mod, inp, shape, T, chunk_min_tokens=1)
    rng = np.random.default_rng(5)
    x = rng.integers(-16, 17, (T, d)).astype(np.float32)
    ids, gates, y = _run(torch_mod, layer, shape, x)

    def index_sum(codes, v, sg):  # sum_j sum_s sg_s 2^s v[8j + code_s(r, j) % 8]
        rows, ns, _ = codes.shape
        base = (np.arange(ns) * 8)[None, :]
        return sum(sg[s_] * v[base + codes[:, :, s_] % 8].sum(axis=1) for s_ in range(3))

    for t in range(T):
        ref = np.zeros(d)
        peak = np.zeros(d)
        for j in range(k):
            e, g = int(ids[t, j]), float(gates[t, j])
            gc, uc, dc = M.matrices(inp.record(e), d, ffn)
            a = index_sum(gc, x[t].astype(np.float64), signs[0])
            b = index_sum(uc, x[t].astype(np.float64), signs[1])
            with np.errstate(over="ignore"):  # silu of a large negative a: exp overflows, h -> -0
                H = M.bf16((a / (1 + np.exp(-a)) * b).astype(np.float32))
            ref += g * index_sum(dc, H, signs[2])
            peak += g * 7 * np.abs(H).max()
        # two one-ulp flips of a rounded h, plus fp32 accumulation and atomics
        tol = 2.0 ** -6 * peak + 2.0 ** -20 * np.abs(ref).max()
        bad = np.nonzero(np.abs(y[t] - ref) > tol)[0]
        assert bad.size == 0, (t, bad[:8], y[t][bad[:8]], ref[bad[:8]])
    layer.close()


def test_chunk_path_rmsnorm_residual_and_threshold(torch_mod):
    """RMS normalisation and the residual on the chunk path; a call below the
    threshold of the same handle takes the table path (1e-4 bar)."""
    from synth import gpu as G
    shape = S.Shape(512, 256, 32, 8, "f16")
    inp = G.LayerInputs(shape, seed=9, layer=4, host_codes=True)
    layer = _layer(torch_mod, inp, shape, 40, pre_rmsnorm=True, residual=True, eps=1e-6, chunk_min_tokens=16)
    x = S.tokens(9, 50, 40, shape.d)
    ids, gates, y = _run(torch_mod, layer, shape, x)            # 40 >= 16: chunk path
    _check_chunk(inp, shape, x, ids, gates, y, pre_rmsnorm=True, residual=True)
    ids2, gates2, y2 = _run(torch_mod, layer, shape, x[:15])   # 15 < 16: table path
    _check(inp, shape, x[:15], ids2, gates2, y2, pre_rmsnorm=True, residual=True)
    layer.close()


def _listed_experts(ids, E, lut_tokens, cap=512):
    """Experts a chunk-path call hands to the table path: those with fewer than
    lut_tokens tokens (and at least one), in id order while their pairs fit
    the order table."""
    cnt = np.bincount(ids.ravel(), minlength=E)
    listed, total = set(), 0
    for e in range(E):
        if 0 < cnt[e] < lut_tokens:
            total += cnt[e]
            if total > cap:
                break
            listed.add(e)
    return listed


def test_adaptive_dispatch_by_tokens_per_expert(torch_mod):
    """A chunk-path call with lut_expert_tokens = 12: experts routed fewer than
    12 of the 48 tokens go to the table path (fp32), the others to the matrix
    cores.  Tokens whose experts are all on one side match that side's path
    alone (table-only and matrix-core-only handles on the same weights); every
    token follows the oracle at the bf16 bar; with a threshold above every
    count all pairs take the table path and match it at 1e-6."""
    from synth import gpu as G
    shape = S.Shape(264, 136, 12, 3, "f16")
    T, tau = 48, 12
    inp = G.LayerInputs(shape, seed=23, layer=2, host_codes=True)
    mix = _layer(torch_mod, inp, shape, T, chunk_min_tokens=8, lut_expert_tokens=tau)
    mma = _layer(torch_mod, inp, shape, T, chunk_min_tokens=8, lut_expert_tokens=1)
    tab = _layer(torch_mod, inp, shape, T, chunk_min_tokens=T + 1)
    alll = _layer(torch_mod, inp, shape, T, chunk_min_tokens=8, lut_expert_tokens=T + 1)
    x = S.tokens(23, 0, T, shape.d)
    a, b, c, d_ = (_run(torch_mod, h, shape, x) for h in (mix, mma, tab, alll))
    for r in (b, c, d_):
        assert np.array_equal(a[0], r[0])
    listed = _listed_experts(a[0], shape.n_experts, tau)
    side = [sum(e in listed for e in row) for row in a[0]]
    assert 0 < len(listed) < len(set(a[0].ravel().tolist()))
    n_tab = n_mma = 0
    for t in range(T):
        if side[t] == shape.top_k:
            ref, n_tab = c, n_tab + 1
        elif side[t] == 0:
            ref, n_mma = b, n_mma + 1
        else:
            continue
        err = np.linalg.norm(a[2][t] - ref[2][t]) / np.linalg.norm(ref[2][t])
        assert err <= 1e-6, (t, side[t], err)
    assert n_tab > 0 and n_mma > 0, (n_tab, n_mma)
    _check_chunk(inp, shape, x, *a, table_experts=set(listed))
    err = np.linalg.norm(d_[2] - c[2], axis=1) / np.linalg.norm(c[2], axis=1)
    assert err.max() <= 1e-6, err.max()
    _check(inp, shape, x, *d_, tokens=range(4))
    for h in (mix, mma, tab, alll):
        h.close()


def test_chunk_path_invalid_ids_poison_only_their_token(torch_mod, tiny):
    from synth import gpu as G
    from vector_quantized_expert_amd import RvqMoeError
    from vector_quantized_expert_amd import rvq_moe as R
    shape = S.TINY
    layer = _layer(torch_mod, tiny, shape, 3, chunk_min_tokens=1)
    x = G.to_device(S.tokens(0, 0, 3, shape.d))
    ids = torch_mod.tensor([[0, 1, 2, 3], [0, 1, -4, 3], [5, 6, 7, 8]], dtype=torch_mod.int32, device="cuda")
    gates = torch_mod.full((3, 4), 0.25, device="cuda")
    y = torch_mod.zeros((3, shape.d), device="cuda")
    layer.layer_forward(x, 3, ids, gates, y)
    with pytest.raises(RvqMoeError) as ei:
        layer.sync()
    assert ei.value.status == R.EDEVICE
    yh = y.cpu().numpy()
    assert np.all(np.isfinite(yh[0])) and np.all(np.isnan(yh[1])) and np.all(np.isfinite(yh[2]))
    layer.close()


def test_k3_chunk_512_tokens_against_table_path_and_oracle(torch_mod):
    """The prefill chunk: 512 tokens through the d=7168, ffn=2048, E=384, top-16
    layer in one call on the chunk path; every token against the table path of a
    second handle on the same weights, sampled tokens against the oracle."""
    from synth import gpu as G
    shape = S.K3
    T = 512
    inp = G.LayerInputs(shape, seed=0, layer=5)
    chunk = _layer(torch_mod, inp, shape, T, chunk_min_tokens=64)
    table = _layer(torch_mod, inp, shape, T, chunk_min_tokens=T + 1)
    inp.free_codes()
    torch_mod.cuda.empty_cache()
    x = S.tokens(0, 3000, T, shape.d)
    a = _run(torch_mod, chunk, shape, x)
    b = _run(torch_mod, table, shape, x)
    assert np.array_equal(a[0], b[0])
    err = np.linalg.norm(a[2] - b[2], axis=1) / np.linalg.norm(b[2], axis=1)
    print(f"K3 chunk vs table: max rel L2 {err.max():.3e}, mean {err.mean():.3e}")
    assert err.max() <= TOL_Y_BF16
    worst = _check_chunk(inp, shape, x, *a, tokens=[0, 255, 511])
    print(f"K3 chunk vs oracle: worst rel L2 {worst:.3e}")
    chunk.close()
    table.close()


# --------------------------------------------------------------------------- HBM slot cache (pinned host bank)
def _pinned_bank(torch, inp):
    """The canonical code bank copied into pinned host memory (hipHostMalloc)."""
    dev = inp.codes_dev
    bank = torch.empty(dev.shape, dtype=torch.uint8, pin_memory=True)
    bank.copy_(dev)
    return bank


def _lru_model(S, runs):
    """Hits and misses of the cache policy: per acquire, hits keep their slots;
    each miss takes the least recently used slot not used by this acquire
    (the lowest index among equals)."""
    slot_of, expert_in, last = {}, [-1] * S, [0] * S
    hits = misses = 0
    for clock, experts in enumerate(runs, start=1):
        for e in experts:
            if e in slot_of:
                last[slot_of[e]] = clock
                hits += 1
        for e in experts:
            if e in slot_of:
                continue
            v = min((sl for sl in range(S) if last[sl] != clock), key=lambda sl: (last[sl], sl))
            if expert_in[v] >= 0:
                del slot_of[expert_in[v]]
            expert_in[v], slot_of[e], last[v] = e, v, clock
            misses += 1
    return hits, misses


def _table_runs(ids, S):
    """Token runs of one table-path call whose distinct experts fit S slots."""
    runs, cur = [], []
    for row in ids:
        fresh = [e for e in dict.fromkeys(row.tolist()) if e not in cur]
        if len(cur) + len(fresh) > S:
            runs.append(cur)
            cur = []
            fresh = list(dict.fromkeys(row.tolist()))
        cur += fresh
    runs.append(cur)
    return runs


def _same_outputs(a, b, det):
    """Deterministic handles: bitwise equal outputs.  Otherwise outputs agree
    within the fp32 atomic summation order (1e-6 relative L2 per token)."""
    if det:
        assert np.array_equal(a, b), np.abs(a - b).max()
    else:
        err = np.linalg.norm(a - b, axis=1) / np.linalg.norm(b, axis=1)
        assert err.max() <= 1e-6, err.max()


@pytest.mark.parametrize("det", [False, True])
def test_streaming_table_path_matches_resident_and_counts_lru(torch_mod, tiny, det):
    """Codes in pinned host memory through 5 HBM slots (k = 4): one-token calls
    that evict, and a 12-token call whose experts exceed the slots (run
    splitting), against a resident handle; hits/misses/bytes against the
    policy's model.  With the deterministic combine, streaming and resident,
    and grouped and one-token calls, give bitwise identical outputs."""
    from synth import gpu as G
    shape = S.TINY
    bank = _pinned_bank(torch_mod, tiny)
    slots = 5
    st = _layer(torch_mod, tiny, shape, 12, codes=bank, codes_location=1, cache_slots=slots, deterministic=det)
    rs = _layer(torch_mod, tiny, shape, 12, deterministic=det)
    x = S.tokens(0, 700, 20, shape.d)
    a = _run(torch_mod, st, shape, x, per_token=True)
    b = _run(torch_mod, rs, shape, x, per_token=True)
    assert np.array_equal(a[0], b[0])
    _same_outputs(a[2], b[2], det)
    runs = [list(dict.fromkeys(row.tolist())) for row in a[0]]
    x2 = S.tokens(0, 800, 12, shape.d)
    a2 = _run(torch_mod, st, shape, x2)
    b2 = _run(torch_mod, rs, shape, x2)
    _same_outputs(a2[2], b2[2], det)
    if det:  # grouped (one 12-token call) and one token per call, on the same ids and gates
        assert np.array_equal(b2[2], _forward(torch_mod, rs, shape, x2, b2[0], b2[1], per_token=True))
    runs += _table_runs(a2[0], slots)
    hits, misses = _lru_model(slots, runs)
    stats = st.stats()
    assert (stats["slot_hits"], stats["slot_misses"]) == (hits, misses)
    assert stats["h2d_bytes"] == misses * (stats["code_bytes_resident"] // slots)
    assert stats["host_syncs"] == 21
    _check(tiny, shape, x, *a, tokens=range(4))
    st.close()
    rs.close()


def test_streaming_rounds_of_64_experts_on_the_replicated_kernels(torch_mod):
    """128 slots: experts in rounds of 64, enough for the replicated-codebook
    kernels to take a slot-cache round (they read each expert's record through
    the slot table).  Same outputs as with resident codes, bitwise with the
    deterministic combine, and the oracle at the bf16 bar."""
    from synth import gpu as G
    shape = S.Shape(256, 128, 128, 4, "f16")
    T = 96  # 384 pairs: 3 per expert on average
    inp = G.LayerInputs(shape, seed=31, layer=0, host_codes=True)
    bank = _pinned_bank(torch_mod, inp)
    st = _layer(torch_mod, inp, shape, T, codes=bank, codes_location=1, cache_slots=128, chunk_min_tokens=8,
                lut_expert_tokens=1, deterministic=True)
    rs = _layer(torch_mod, inp, shape, T, chunk_min_tokens=8, lut_expert_tokens=1, deterministic=True)
    x = S.tokens(31, 0, T, shape.d)
    a = _run(torch_mod, st, shape, x)
    b = _run(torch_mod, rs, shape, x)
    assert np.array_equal(a[0], b[0])
    assert np.array_equal(a[2], b[2])
    assert len(np.unique(a[0])) > 64  # at least two rounds
    _check_chunk(inp, shape, x, *a, tokens=[0, 50, 95])
    st.close()
    rs.close()


@pytest.mark.parametrize("det", [False, True])
def test_streaming_chunk_path_matches_resident(torch_mod, det):
    """The chunk path with 4 slots: experts in rounds of 2, copies overlapping
    the previous round's kernels; same outputs as with resident codes (bitwise
    with the deterministic combine)."""
    from synth import gpu as G
    shape = S.Shape(264, 136, 12, 3, "f16")
    inp = G.LayerInputs(shape, seed=23, layer=0, host_codes=True)
    bank = _pinned_bank(torch_mod, inp)
    st = _layer(torch_mod, inp, shape, 48, codes=bank, codes_location=1, cache_slots=4, chunk_min_tokens=8,
                deterministic=det)
    rs = _layer(torch_mod, inp, shape, 48, chunk_min_tokens=8, deterministic=det)
    x = S.tokens(23, 0, 48, shape.d)
    for _ in range(2):
        a = _run(torch_mod, st, shape, x)
        b = _run(torch_mod, rs, shape, x)
        assert np.array_equal(a[0], b[0])
        _same_outputs(a[2], b[2], det)
    _check_chunk(inp, shape, x, *a, tokens=[0, 47])
    n_exp = len(np.unique(a[0]))
    assert st.stats()["slot_misses"] + st.stats()["slot_hits"] == 2 * n_exp
    st.close()
    rs.close()


def test_streaming_validation(torch_mod, tiny):
    from vector_quantized_expert_amd import RvqMoeError
    from vector_quantized_expert_amd import rvq_moe as R
    shape = S.TINY
    bank = _pinned_bank(torch_mod, tiny)
    with pytest.raises(RvqMoeError) as ei:
        _layer(torch_mod, tiny, shape, 1, codes=bank, codes_location=1, cache_slots=3)   # < top_k
    assert ei.value.status == R.EBUDGET
    pageable = tiny.codes_dev.cpu()
    with pytest.raises(RvqMoeError) as ei:
        _layer(torch_mod, tiny, shape, 1, codes=pageable, codes_location=1, cache_slots=4)
    assert ei.value.status == R.EINVAL
    st = _layer(torch_mod, tiny, shape, 2, codes=bank, codes_location=1, cache_slots=4)
    x = torch_mod.zeros((2, shape.d), device="cuda")
    ids = torch_mod.zeros((2, 4), dtype=torch_mod.int32, device="cuda")
    g = torch_mod.zeros((2, 4), device="cuda")
    y = torch_mod.zeros((2, shape.d), device="cuda")
    with pytest.raises(RvqMoeError) as ei:
        st.route_forward(x, 1, ids, g, y)
    assert ei.value.status == R.ENOTSUP
    st.close()


def _lru_prefetch_model(S, events):
    """The cache policy with prefetches: events are ("acquire", experts) or
    ("prefetch", experts), each one clock tick.  A prefetch refreshes the
    resident experts, then fills least-recently-used slots not touched by it
    (the lowest index among equals) until none is left.  Returns (hits,
    misses, prefetch fills, prefetch hits)."""
    slot_of, expert_in, last, pref = {}, [-1] * S, [0] * S, [False] * S
    hits = misses = fills = phits = 0

    def take(e, clock):
        free = [sl for sl in range(S) if last[sl] != clock]
        if not free:
            return None
        v = min(free, key=lambda sl: (last[sl], sl))
        if expert_in[v] >= 0:
            del slot_of[expert_in[v]]
        expert_in[v], slot_of[e], last[v] = e, v, clock
        return v

    for clock, (kind, experts) in enumerate(events, start=1):
        for e in experts:
            if e in slot_of:
                sl = slot_of[e]
                last[sl] = clock
                if kind == "acquire":
                    hits += 1
                    if pref[sl]:
                        pref[sl] = False
                        phits += 1
        for e in experts:
            if e in slot_of:
                continue
            v = take(e, clock)
            if kind == "acquire":
                pref[v] = False
                misses += 1
            elif v is None:
                break
            else:
                pref[v] = True
                fills += 1
    return hits, misses, fills, phits


@pytest.mark.parametrize("det", [False, True])
def test_router_lookahead_prefetch_chain(torch_mod, det):
    """[FR] "Lecture anticipée et prédiction du routeur": a 3-layer streaming
    chain (RMS normalisation, residual), run with and without prefetching
    layer l+1's first 3 predicted experts (its router on layer l's input).
    Ids are identical, outputs equal within the fp32 atomic-order bound
    (bitwise with the deterministic combine: reading ahead leaves the output
    exactly as it was), and the slot counters match the cache policy's model,
    prefetches included."""
    from synth import gpu as G
    shape = S.Shape(512, 256, 32, 8, "f16")
    L, T, slots, ahead = 3, 6, 12, 3
    inps = [G.LayerInputs(shape, seed=31, layer=l, host_codes=True) for l in range(L)]
    banks = [_pinned_bank(torch_mod, inp) for inp in inps]
    kw = dict(codes_location=1, cache_slots=slots, pre_rmsnorm=True, residual=True, eps=1e-6, deterministic=det)
    runs = {}
    for mode in ("plain", "ahead"):
        layers = [_layer(torch_mod, inps[l], shape, 1, codes=banks[l], **kw) for l in range(L)]
        h = torch_mod.empty((L + 1, T, shape.d), device="cuda")
        h[0].copy_(G.to_device(S.tokens(31, 0, T, shape.d)))
        ids = torch_mod.empty((L, T, shape.top_k), dtype=torch_mod.int32, device="cuda")
        pred = torch_mod.full((L, T, shape.top_k), -1, dtype=torch_mod.int32, device="cuda")
        g = torch_mod.empty((L, T, shape.top_k), device="cuda")
        gp = torch_mod.empty((T, shape.top_k), device="cuda")
        for t in range(T):
            for l in range(L):
                layers[l].route_topk(h[l, t:t + 1], 1, ids[l, t:t + 1], g[l, t:t + 1])
                layers[l].layer_forward(h[l, t:t + 1], 1, ids[l, t:t + 1], g[l, t:t + 1], h[l + 1, t:t + 1])
                if mode == "ahead" and l + 1 < L:
                    layers[l + 1].route_topk(h[l, t:t + 1], 1, pred[l + 1, t:t + 1], gp[t:t + 1])
                    layers[l + 1].prefetch(pred[l + 1, t:t + 1], 1, ahead)
        for layer in layers:
            layer.sync()
        runs[mode] = (ids.cpu().numpy(), pred.cpu().numpy(), h.cpu().numpy(), [x.stats() for x in layers])
        for layer in layers:
            layer.close()
    (ia, _, ha, sa), (ib, pb, hb, sb) = runs["plain"], runs["ahead"]
    assert np.array_equal(ia, ib)
    for l in range(1, L + 1):
        _same_outputs(hb[l], ha[l], det)
    assert sum(st["prefetch_fills"] for st in sb) > 0
    assert all(st["prefetch_fills"] == 0 for st in sa)
    for l in range(L):
        events = []
        for t in range(T):
            if l > 0:  # layer l's prefetch was issued right after layer l-1's call of token t
                events.append(("prefetch", list(dict.fromkeys(pb[l, t, :ahead].tolist()))))
            events.append(("acquire", list(dict.fromkeys(ib[l, t].tolist()))))
        # the prefetch of token t comes after layer l-1's call of token t, which
        # precedes layer l's call of token t: the order above
        hits, misses, fills, phits = _lru_prefetch_model(slots, events)
        st = sb[l]
        assert (st["slot_hits"], st["slot_misses"], st["prefetch_fills"], st["prefetch_hits"]) == \
            (hits, misses, fills, phits), (l, st)
        assert st["h2d_bytes"] == (misses + fills) * (st["code_bytes_resident"] // slots)
    # the chain's outputs against the oracle, teacher-forced, on the first token
    for l in range(L):
        ref = O.layer(ha[l][0], inps[l].w_r, shape.top_k, inps[l].codebook, inps[l].record, shape.d, shape.ffn,
                      pre_rmsnorm=True, eps=1e-6)
        assert np.array_equal(ib[l][0], ref.route.ids)
        delta = hb[l + 1][0].astype(np.float64) - ha[l][0].astype(np.float64)
        assert np.linalg.norm(delta - ref.delta) / np.linalg.norm(ref.delta) <= TOL_Y


def test_prefetch_validation(torch_mod, tiny):
    from vector_quantized_expert_amd import RvqMoeError
    from vector_quantized_expert_amd import rvq_moe as R
    shape = S.TINY
    ids = torch_mod.zeros((2, 4), dtype=torch_mod.int32, device="cuda")
    rs = _layer(torch_mod, tiny, shape, 2)
    with pytest.raises(RvqMoeError) as ei:
        rs.prefetch(ids, 1, 2)
    assert ei.value.status == R.ENOTSUP
    rs.close()
    bank = _pinned_bank(torch_mod, tiny)
    st = _layer(torch_mod, tiny, shape, 2, codes=bank, codes_location=1, cache_slots=4)
    for n, per in ((0, 1), (3, 1), (1, 0), (1, 5)):
        with pytest.raises(RvqMoeError) as ei:
            st.prefetch(ids, n, per)
        assert ei.value.status == R.EINVAL
    bad = torch_mod.tensor([[-1, shape.n_experts, 2, 2], [2, 3, 1, 0]], dtype=torch_mod.int32, device="cuda")
    st.prefetch(bad, 2, 4)  # out-of-range ids skipped, duplicates once, at most 4 slots
    s = st.stats()
    assert s["prefetch_fills"] == 4 and s["h2d_bytes"] == 4 * (s["code_bytes_resident"] // 4)
    st.close()


@pytest.mark.parametrize("det", [False, True])
def test_k3_streaming_batch1_matches_resident(torch_mod, det):
    """d=7168, ffn=2048, E=384, top-16 from a pinned host bank through 32 slots
    (every record's CRC-32 checked), one token per call; against a resident
    handle (bitwise with the deterministic combine) and the oracle."""
    from synth import gpu as G
    shape = S.K3
    inp = G.LayerInputs(shape, seed=0, layer=6)
    bank = _pinned_bank(torch_mod, inp)
    st = _layer(torch_mod, inp, shape, 1, codes=bank, codes_location=1, cache_slots=32, verify_records=True,
                deterministic=det)
    rs = _layer(torch_mod, inp, shape, 1, deterministic=det)
    inp.free_codes()
    torch_mod.cuda.empty_cache()
    x = S.tokens(0, 4000, 4, shape.d)
    a = _run(torch_mod, st, shape, x, per_token=True)
    b = _run(torch_mod, rs, shape, x, per_token=True)
    assert np.array_equal(a[0], b[0])
    _same_outputs(a[2], b[2], det)
    _check(inp, shape, x, *a, tokens=[0])
    assert st.stats()["slot_misses"] >= 16
    # every record copied in had its trailer and its 16.5 MB payload's CRC-32 checked
    assert st.stats()["records_verified"] == st.stats()["slot_misses"]
    st.sync()
    st.close()
    rs.close()
    del bank


@pytest.mark.parametrize("shape_args", [(256, 128, 16, 4, "f32"), (1024, 520, 9, 3, "f16")])
def test_deterministic_combine_repeats_bitwise_and_follows_the_oracle(torch_mod, shape_args):
    """deterministic=1: repeated calls of every kind give the same bits
    (one-token and grouped table path, the routed one-launch call, the chunk
    path), the same bits as each other where the arithmetic is the same
    (grouped vs one token per call), the fast handle's outputs within the fp32
    atomic-order bound, and the oracle at the usual bars; an invalid id still
    poisons only its token."""
    from synth import gpu as G
    from vector_quantized_expert_amd import RvqMoeError
    shape = S.Shape(*shape_args)
    inp = G.LayerInputs(shape, seed=61, layer=0, host_codes=True)
    T = 6
    det = _layer(torch_mod, inp, shape, T, deterministic=1, residual=True)
    fast = _layer(torch_mod, inp, shape, T, residual=True)
    chk = _layer(torch_mod, inp, shape, T, deterministic=1, chunk_min_tokens=4)
    x = S.tokens(61, 0, T, shape.d)
    a = _run(torch_mod, det, shape, x)
    again = _run(torch_mod, det, shape, x)
    assert np.array_equal(a[0], again[0]) and np.array_equal(a[1], again[1]) and np.array_equal(a[2], again[2])
    assert np.array_equal(a[2], _forward(torch_mod, det, shape, x, a[0], a[1], per_token=True))
    f = _run(torch_mod, fast, shape, x)
    assert np.array_equal(a[0], f[0])
    _same_outputs(a[2], f[2], False)
    _check(inp, shape, x, *a, residual=True)
    # the routed one-launch call, twice
    xd = G.to_device(x[:1])
    outs = []
    for _ in range(2):
        ids_d = torch_mod.empty((1, shape.top_k), dtype=torch_mod.int32, device="cuda")
        g_d = torch_mod.empty((1, shape.top_k), device="cuda")
        y_d = torch_mod.empty((1, shape.d), device="cuda")
        det.route_forward(xd, 1, ids_d, g_d, y_d)
        det.sync()
        outs.append((ids_d.cpu().numpy(), g_d.cpu().numpy(), y_d.cpu().numpy()))
    assert all(np.array_equal(u, v) for u, v in zip(*outs))
    _check(inp, shape, x[:1], *outs[0], residual=True)
    # the chunk path, twice
    c1, c2 = _run(torch_mod, chk, shape, x), _run(torch_mod, chk, shape, x)
    assert np.array_equal(c1[2], c2[2])
    _check_chunk(inp, shape, x, *c1)
    # an invalid id: its token's output is NaN, the others are finite
    ids = torch_mod.tensor(a[0], device="cuda")
    ids[1, 0] = shape.n_experts + 3
    y = torch_mod.zeros((T, shape.d), device="cuda")
    det.layer_forward(G.to_device(x), T, ids, G.to_device(a[1]), y)
    with pytest.raises(RvqMoeError):
        det.sync()
    yh = y.cpu().numpy()
    assert np.all(np.isnan(yh[1])) and np.all(np.isfinite(np.delete(yh, 1, axis=0)))
    for h in (det, fast, chk):
        h.close()


def test_mixed_calls_on_one_handle_match_fresh_handles(torch_mod):
    """One handle through a long mix of calls, enqueued back to back with no
    host synchronisation between them: one-token table path, one-launch routed
    calls (one and several tokens), grouped batches, and chunk-path calls that
    hand few-token experts to the table path.  The layer kernel's completion
    counters alternate between two sets across its launches, each launch
    zeroing the other set as it ends; every call must give what the same call
    gives on a freshly opened handle (ids bit-exact, outputs within 1e-6
    relative L2: only the order of the fp32 output additions may differ)."""
    from synth import gpu as G
    torch = torch_mod
    shape = S.Shape(264, 136, 12, 3, "f16")
    T_max = 48
    inp = G.LayerInputs(shape, seed=31, layer=1, host_codes=True)
    kw = dict(chunk_min_tokens=8, lut_expert_tokens=12)
    x = G.to_device(S.tokens(31, 0, T_max, shape.d))
    plan = [("fused", 1), ("two", 1), ("two", 5), ("two", 48), ("fused", 3), ("two", 1), ("two", 9)] * 3

    def call(layer, kind, T, off):
        xs = x[off:off + T]
        ids = torch.empty((T, shape.top_k), dtype=torch.int32, device="cuda")
        gates = torch.empty((T, shape.top_k), dtype=torch.float32, device="cuda")
        y = torch.empty((T, shape.d), dtype=torch.float32, device="cuda")
        if kind == "fused":
            layer.route_forward(xs, T, ids, gates, y)
        else:
            layer.route_topk(xs, T, ids, gates)
            layer.layer_forward(xs, T, ids, gates, y)
        return ids, gates, y

    h = _layer(torch, inp, shape, T_max, **kw)
    outs = [call(h, kind, T, i % (T_max - T + 1)) for i, (kind, T) in enumerate(plan)]
    h.sync()
    for i, (kind, T) in enumerate(plan):
        fresh = _layer(torch, inp, shape, T_max, **kw)
        ref = call(fresh, kind, T, i % (T_max - T + 1))
        fresh.sync()
        a = [t.cpu().numpy() for t in outs[i]]
        r = [t.cpu().numpy() for t in ref]
        assert np.array_equal(a[0], r[0]), (i, kind, T)
        np.testing.assert_allclose(a[1], r[1], rtol=1e-6, atol=0)
        err = np.linalg.norm(a[2] - r[2], axis=1) / np.linalg.norm(r[2], axis=1)
        assert err.max() <= 1e-6, (i, kind, T, err.max())
        fresh.close()
    h.close()


def test_mixed_calls_on_one_streaming_handle_match_resident(torch_mod):
    """A streaming handle (codes in pinned host memory through 5 HBM slots,
    k = 3) through a mix of one-token calls, grouped batches, chunk-path calls
    (run in rounds of slots) and prefetches of a call's experts just ahead of it, enqueued without host synchronisation between them (beyond
    the slot cache's own read of each call's ids): every call matches the same
    sequence on a resident handle (ids bit-exact, outputs within 1e-6 relative
    L2), and every call and prefetch is counted once by the slot cache."""
    from synth import gpu as G
    torch = torch_mod
    shape = S.Shape(264, 136, 12, 3, "f16")
    T_max = 48
    inp = G.LayerInputs(shape, seed=37, layer=3, host_codes=True)
    bank = _pinned_bank(torch, inp)
    # a streaming handle puts every expert of a chunk-path call on the matrix
    # cores (lut_expert_tokens acts as 1), so the resident reference does too
    st = _layer(torch, inp, shape, T_max, codes=bank, codes_location=1, cache_slots=5, chunk_min_tokens=8,
                lut_expert_tokens=12)
    rs = _layer(torch, inp, shape, T_max, chunk_min_tokens=8, lut_expert_tokens=1)
    x = G.to_device(S.tokens(37, 0, T_max, shape.d))
    plan = [1, 5, 48, 1, 9, 1, 48, 2] * 2

    def run(layer, stream_pf):
        outs = []
        for i, T in enumerate(plan):
            off = (7 * i) % (T_max - T + 1)
            xs = x[off:off + T]
            ids = torch.empty((T, shape.top_k), dtype=torch.int32, device="cuda")
            gates = torch.empty((T, shape.top_k), dtype=torch.float32, device="cuda")
            y = torch.empty((T, shape.d), dtype=torch.float32, device="cuda")
            layer.route_topk(xs, T, ids, gates)
            if stream_pf and i % 3 == 0:
                layer.prefetch(ids, T, 2)  # this call's first two experts per token, just ahead of it
            layer.layer_forward(xs, T, ids, gates, y)
            outs.append((ids, gates, y))
        layer.sync()
        return [[t.cpu().numpy() for t in o] for o in outs]

    a = run(st, True)
    b = run(rs, False)
    for i, T in enumerate(plan):
        assert np.array_equal(a[i][0], b[i][0]), (i, T)
        np.testing.assert_allclose(a[i][1], b[i][1], rtol=1e-6, atol=0)
        err = np.linalg.norm(a[i][2] - b[i][2], axis=1) / np.linalg.norm(b[i][2], axis=1)
        assert err.max() <= 1e-6, (i, T, err.max())
    stats = st.stats()
    assert stats["forward_calls"] == len(plan)
    assert stats["slot_hits"] + stats["slot_misses"] > 0
    _check(inp, shape, S.tokens(37, 0, T_max, shape.d)[:1], a[0][0], a[0][1], a[0][2])
    st.close()
    rs.close()
