"""C-ABI checks that need no GPU: the library loads, exports every symbol the
header declares, and rejects bad arguments before touching the device."""
import ctypes

import pytest

from vector_quantized_expert_amd import rvq_moe as R


def test_library_exports_every_header_symbol():
    names = R.header_functions()
    for core in ("rvq_moe_open", "rvq_moe_route_topk", "rvq_moe_layer_forward", "rvq_moe_close"):
        assert core in names
    L = R.lib()
    for n in names:
        assert hasattr(L, n), n
    assert L.rvq_moe_abi_version() == 6


def _desc(**over):
    kw = dict(d=256, ffn=128, n_experts=16, top_k=4, codebook_dtype=R.CB_F32, router_w=0x1000,
              codebooks=0x2000, codes=0x3000, stream=0, max_tokens=4)
    kw.update(over)
    return R.make_desc(**kw)


@pytest.mark.parametrize("over,status", [
    (dict(d=0), R.EINVAL),
    (dict(d=260), R.EINVAL),          # not a multiple of 8
    (dict(ffn=12), R.EINVAL),
    (dict(top_k=17), R.EINVAL),       # k > E
    (dict(top_k=0), R.EINVAL),
    (dict(n_experts=2000), R.EINVAL),
    (dict(max_tokens=0), R.EINVAL),
    (dict(router_w=0), R.EINVAL),
    (dict(codes=0), R.EINVAL),
    (dict(codebook_dtype=7), R.EINVAL),
    (dict(n_stages=4), R.ENOTSUP),
    (dict(n_codes=16), R.ENOTSUP),
    (dict(vec_dim=4), R.ENOTSUP),
    (dict(cache_slots=3), R.EBUDGET),  # below one token's working set (k = 4)
    (dict(cache_slots=-1), R.EINVAL),
    (dict(cache_slots=8), R.EINVAL),   # slots stream pinned host codes only
    (dict(codes_location=1), R.EINVAL),  # pinned host codes need slots
    (dict(codes_location=5), R.EINVAL),
    (dict(codes_location=2), R.EINVAL),  # a bank needs slots too
    (dict(codes_location=2, cache_slots=4), R.EINVAL),  # not pinned host memory
    (dict(deterministic=2), R.EINVAL),
    (dict(chunk_min_tokens=-1), R.EINVAL),
    (dict(eps=-1.0), R.EINVAL),
])
def test_open_rejects_bad_descriptions_before_any_device_call(over, status):
    rc, h = R.open_raw(_desc(**over))
    assert rc == status, R.last_error()
    assert h == 0
    assert R.last_error()


def test_open_rejects_wrong_struct_size_and_nulls():
    d = _desc()
    d.struct_size = 8
    rc, h = R.open_raw(d)
    assert rc == R.EINVAL and h == 0
    L = R.lib()
    assert L.rvq_moe_open(None, ctypes.byref(ctypes.c_void_p())) == R.EINVAL
    assert L.rvq_moe_open(ctypes.byref(_desc()), None) == R.EINVAL


def test_calls_reject_null_handle():
    L = R.lib()
    assert L.rvq_moe_route_topk(None, 0x1000, 1, 0x2000, 0x3000, None) == R.EINVAL
    assert L.rvq_moe_layer_forward(None, 0x1000, 1, 0x2000, 0x3000, 0x4000, None) == R.EINVAL
    assert L.rvq_moe_sync(None, None) == R.EINVAL
    assert L.rvq_moe_prefetch(None, 0x1000, 1, 1, None) == R.EINVAL
    assert L.rvq_moe_close(None) == R.OK
    s = R.Stats()
    assert L.rvq_moe_get_stats(None, ctypes.byref(s)) == R.EINVAL


def test_bank_layout_k3_shape():
    # d=7168, ffn=2048: every matrix fills whole 32-slice x 32-row blocks, so
    # the payload is the canonical 9 d ffn / 8 bytes (4032 pages) and the
    # trailer takes one more page
    stride, payload = R.bank_layout(d=7168, ffn=2048, n_experts=384, top_k=16, codebook_dtype=R.CB_F16)
    assert payload == 16_515_072 == 9 * 7168 * 2048 // 8
    assert stride == payload + 4096


@pytest.mark.parametrize("d,ffn", [(256, 128), (264, 136), (64, 40), (8, 8)])
def test_bank_layout_pages(d, ffn):
    stride, payload = R.bank_layout(d=d, ffn=ffn, n_experts=4, top_k=2, codebook_dtype=R.CB_F32)
    assert payload >= 9 * d * ffn // 8 and payload % 16 == 0
    assert stride % 4096 == 0 and stride - 4096 >= payload > stride - 8192


def test_bank_calls_reject_bad_arguments_before_any_device_call():
    L = R.lib()
    s, p = ctypes.c_int64(), ctypes.c_int64()
    assert L.rvq_moe_bank_layout(None, ctypes.byref(s), ctypes.byref(p)) == R.EINVAL
    assert L.rvq_moe_bank_layout(ctypes.byref(_desc()), None, ctypes.byref(p)) == R.EINVAL
    assert L.rvq_moe_bank_layout(ctypes.byref(_desc(d=12)), ctypes.byref(s), ctypes.byref(p)) == R.EINVAL
    assert L.rvq_moe_bank_layout(ctypes.byref(_desc(n_stages=2)), ctypes.byref(s), ctypes.byref(p)) == R.ENOTSUP
    assert L.rvq_moe_write_bank(ctypes.byref(_desc()), None) == R.EINVAL
    assert L.rvq_moe_write_bank(ctypes.byref(_desc(codes=0)), 0x5000) == R.EINVAL
    assert L.rvq_moe_write_bank(ctypes.byref(_desc(codes_location=2)), 0x5000) == R.EINVAL
    assert L.rvq_moe_write_bank(ctypes.byref(_desc()), 0x5000) == R.EINVAL  # bank not pinned host memory
