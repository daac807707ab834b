"""Host-side checks of libmoe: every symbol include/moe.h declares is
exported, the size helpers agree with the record format, and argument checking
rejects bad calls before anything is enqueued (no GPU needed: every call here
fails validation or only computes sizes)."""
import ctypes as C

import pytest

from bit_dequant_expert_route_amd import synth

moe = pytest.importorskip("bit_dequant_expert_route_amd.moe")


def test_all_header_symbols_exported():
    names = moe.header_functions()
    assert len(names) >= 20
    missing = [n for n in names if not hasattr(moe.lib, n)]
    assert not missing, missing


def test_sizes():
    assert moe.expert_bytes(4096, 1024, 4) == 7077888
    assert moe.expert_bytes(4096, 1024, 2) == 3932160
    assert moe.expert_bytes(256, 128, 4) == 55296
    assert moe.expert_bytes(100, 128, 4) == 0
    assert moe.expert_bytes(4096, 1024, 3) == 0
    assert moe.lib.moe_expert_bytes(4096, 1024, 4, 32) == 0
    assert moe.qmatrix_bytes(1024, 4096, 4) == 1024 * 2048 + 1024 * 64 * 4
    for H, I, b in ((4096, 1024, 4), (256, 128, 4), (192, 320, 2)):
        lay = synth.record_layout(H, I, b)
        assert moe.expert_offsets(H, I, b) == [lay.gate_codes, lay.up_codes, lay.down_codes,
                                              lay.gate_sb, lay.up_sb, lay.down_sb]
    assert moe.lib.moe_abi_version() == 2
    for s in (0, -1, -2, -3, -4, -5):
        assert moe.lib.moe_strerror(s)


def _layer(**over):
    d = dict(hidden=4096, inter=1024, n_experts=512, top_k=4, group=64, bits_routed=4,
             bits_shared=4, renorm_topk=1, router_dtype=1, router=0x100000, gate_dtype=1,
             shared_gate=0x200000, experts=0x10000000, expert_stride=7077888,
             shared_expert=0x300000)
    d.update(over)
    s = moe.LayerStruct()
    for k, v in d.items():
        setattr(s, k, v)
    return s


def _decode(L, ws_bytes=1 << 20, ws=0x400000, x=0x500000, hres=0x600000, hout=0x700000,
            idx=0x800000, w=0x900000, T=1):
    return moe.lib.moe_layer_decode(C.byref(L), T, 1, x, hres, hout, idx, w, ws, ws_bytes, None)


def _err():
    return moe.lib.moe_last_error().decode()


@pytest.mark.parametrize("over,status", [
    (dict(group=32), moe.MOE_EUNSUPPORTED),
    (dict(bits_routed=3), moe.MOE_EUNSUPPORTED),
    (dict(bits_shared=8), moe.MOE_EUNSUPPORTED),
    (dict(router_dtype=7), moe.MOE_EUNSUPPORTED),
    (dict(hidden=100), moe.MOE_EINVAL),
    (dict(hidden=16384), moe.MOE_EINVAL),
    (dict(inter=0), moe.MOE_EINVAL),
    (dict(top_k=0), moe.MOE_EINVAL),
    (dict(top_k=9), moe.MOE_EINVAL),
    (dict(n_experts=3), moe.MOE_EINVAL),
    (dict(n_experts=2048), moe.MOE_EINVAL),
    (dict(renorm_topk=2), moe.MOE_EINVAL),
    (dict(router=0), moe.MOE_EINVAL),
    (dict(experts=0), moe.MOE_EINVAL),
    (dict(router=0x100004), moe.MOE_EALIGN),
    (dict(router_tiles=0x100008), moe.MOE_EALIGN),
    (dict(experts=0x10000010), moe.MOE_EALIGN),
    (dict(expert_stride=7077888 + 16), moe.MOE_EALIGN),
    (dict(expert_stride=7077888 - 256), moe.MOE_EINVAL),
])
def test_layer_validation(over, status):
    assert _decode(_layer(**over)) == status
    assert _err()


def test_call_validation():
    L = _layer()
    assert _decode(L, T=0) == moe.MOE_EINVAL
    assert _decode(L, T=65) == moe.MOE_EINVAL
    assert _decode(L, x=0) == moe.MOE_EINVAL
    assert _decode(L, x=0x500008) == moe.MOE_EALIGN
    assert _decode(L, hout=0x600000) == moe.MOE_EINVAL  # aliases h_res
    assert _decode(L, idx=0) == moe.MOE_EINVAL
    assert _decode(L, ws=0) == moe.MOE_EWORKSPACE
    assert _decode(L, ws=0x400010) == moe.MOE_EALIGN
    need = moe.lib.moe_layer_workspace_bytes(C.byref(L), 1)
    assert need > 0
    assert _decode(L, ws_bytes=need - 1) == moe.MOE_EWORKSPACE
    assert "needed" in _err()
    assert moe.lib.moe_layer_workspace_bytes(C.byref(L), 0) == 0
    assert moe.lib.moe_layer_workspace_bytes(C.byref(L), 16) > need


def test_other_entry_points_validate():
    L = _layer()
    ws = 0x400000
    assert moe.lib.moe_route(C.byref(L), 1, 1, 0, 0x1000, 0x2000, 0x3000, None, ws, 1 << 20, None) == moe.MOE_EINVAL
    assert moe.lib.moe_route(C.byref(L), 1, 5, 0x500000, 0x1000, 0x2000, 0x3000, None, ws, 1 << 20, None) == moe.MOE_EUNSUPPORTED
    # caller logits are read with 16-byte loads
    assert moe.lib.moe_route(C.byref(L), 1, 1, 0x500000, 0x1000, 0x2000, 0x3000, 0x4004, ws, 1 << 20, None) == moe.MOE_EALIGN
    assert "16-byte" in _err()
    # 2-bit entry point on a 4-bit layer
    assert moe.lib.moe_expert_forward_q2(C.byref(L), 1, 0x500000, 0x1000, 1, 0x2000, None, ws, 1 << 20, None) == moe.MOE_EUNSUPPORTED
    assert moe.lib.moe_expert_forward_q4(C.byref(L), 1, 0x500000, 0x1000, 0, 0x2000, None, ws, 1 << 20, None) == moe.MOE_EINVAL
    assert moe.lib.moe_expert_forward_q4(C.byref(L), 1, 0x500000, None, 1, 0x2000, None, ws, 1 << 20, None) == moe.MOE_EINVAL
    assert moe.lib.moe_combine(0, 4, 0x1000, 0x2000, 0x3000, 0x4000, 0x5000, 0x6000, None) == moe.MOE_EINVAL
    assert moe.lib.moe_combine(4096, 4, 0x1008, 0x2000, 0x3000, 0x4000, 0x5000, 0x6000, None) == moe.MOE_EALIGN
    arr = (moe.LayerStruct * 2)(L, _layer(inter=512))
    assert moe.lib.moe_stack_decode(arr, 2, None, 0x1000, 0x2000, 0x3000, ws, 1 << 24, None) == moe.MOE_EINVAL
    assert "differs" in _err()
    assert moe.lib.moe_stack_decode(arr, 0, None, 0x1000, 0x2000, 0x3000, ws, 1 << 24, None) == moe.MOE_EINVAL
    assert moe.lib.moe_graph_capture_begin(None) == moe.MOE_EINVAL
    assert moe.lib.moe_graph_launch(None, None) == moe.MOE_EINVAL
    assert moe.lib.moe_graph_destroy(None) == moe.MOE_EINVAL
    assert moe.lib.moe_fill_experts(None, 0, 1, 0, 0, 0, 4096, 1024, 4, 0.0, 1.0, 0.0, 1.0, None) == moe.MOE_EINVAL
    assert moe.lib.moe_fill_experts(0x1010, 0, 1, 0, 0, 0, 4096, 1024, 4, 0.0, 1.0, 0.0, 1.0, None) == moe.MOE_EALIGN
    assert moe.lib.moe_fill_experts(0x1000, 256, 2, 0, 0, 0, 4096, 1024, 4, 0.0, 1.0, 0.0, 1.0, None) == moe.MOE_EINVAL
    assert moe.lib.moe_zero(None, 16, None) == moe.MOE_EINVAL
    v = moe.WsView()
    assert moe.lib.moe_layer_ws_view(C.byref(L), 1, 0x400000, 16, C.byref(v)) == moe.MOE_EWORKSPACE


def test_gdn_step_validates():
    g = moe.lib.moe_gdn_step
    ok = (0x1000, 0x2000, 0x3000, 0x4000, 0x5000, 0x6000, 0x7000)
    assert g(0, 64, 128, 128, *ok, None) == moe.MOE_EINVAL
    assert g(1, 0, 128, 128, *ok, None) == moe.MOE_EINVAL
    assert g(1, 64, 96, 128, *ok, None) == moe.MOE_EUNSUPPORTED
    assert "d_k" in _err()
    assert g(1, 64, 128, 0, *ok, None) == moe.MOE_EINVAL
    assert g(1, 64, 128, 128, None, *ok[1:], None) == moe.MOE_EINVAL
    assert g(1, 64, 128, 128, 0x1004, *ok[1:], None) == moe.MOE_EALIGN
    assert g(1, 64, 128, 128, *ok[:5], 0x6008, 0x7000, None) == moe.MOE_EALIGN
    assert g(1, 64, 128, 128, *ok[:6], 0x7002, None) == moe.MOE_EALIGN


def test_noalloc_refuses_a_workspace_beyond_its_scratch():
    """The largest shapes need more workspace than the library's scratch array
    holds: refused with MOE_EWORKSPACE before anything is enqueued (no GPU
    call is made on this path)."""
    L = _layer(hidden=8192, inter=8192, top_k=8, n_experts=1024, expert_stride=moe.expert_bytes(8192, 8192, 4))
    need = moe.lib.moe_layer_workspace_bytes(C.byref(L), 64)
    assert need > (8 << 20)
    st = moe.lib.moe_layer_decode_noalloc(C.byref(L), 64, 1, 0x500000, 0x600000, 0x700000,
                                          0x800000, 0x900000, None)
    assert st == moe.MOE_EWORKSPACE
    assert "scratch" in _err()
    # and invalid layers are refused first
    st = moe.lib.moe_layer_decode_noalloc(C.byref(_layer(group=32)), 1, 1, 0x500000, 0x600000,
                                          0x700000, 0x800000, 0x900000, None)
    assert st == moe.MOE_EUNSUPPORTED


def test_router_tile_validates():
    f = moe.lib.moe_router_tile
    R, O = 0x1000000, 0x2000000
    assert f(0, 512, 4096, 1, O, None) == moe.MOE_EINVAL
    assert f(R, 512, 4096, 1, 0, None) == moe.MOE_EINVAL
    assert f(R + 8, 512, 4096, 1, O, None) == moe.MOE_EALIGN
    assert f(R, 512, 4096, 7, O, None) == moe.MOE_EUNSUPPORTED
    assert f(R, 0, 4096, 1, O, None) == moe.MOE_EINVAL
    assert f(R, 512, 100, 1, O, None) == moe.MOE_EINVAL
    assert f(R, 512, 4096, 1, R + 4096, None) == moe.MOE_EINVAL  # out overlaps router
    assert "overlaps" in _err()
