"""The C-ABI library loads and exports every entry point include/triroute.h declares; host-side
argument checks answer without a GPU (no compute call is made here)."""

import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "triroute.h")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(tr_[a-z0-9_]+)\s*\(", text)))


@pytest.fixture(scope="module")
def lib():
    import mixed_precision_kv_tr_amd as tr
    return tr.lib


def test_header_declares_the_boundary():
    names = declared_functions()
    for required in ("tr_kv_cache_alloc", "tr_kv_quantize_write", "tr_routed_attn_decode",
                     "tr_routed_attn_prefill"):
        assert required in names


def test_every_declared_symbol_is_exported(lib):
    for name in declared_functions():
        assert hasattr(lib, name), f"{name} declared in triroute.h but not exported"


def test_status_strings(lib):
    import mixed_precision_kv_tr_amd as tr
    for code in range(9):
        s = tr.tr_status_str(code)
        assert s and s != "unknown status"
    assert tr.tr_status_str(99) == "unknown status"


def test_host_side_validation_without_gpu():
    import mixed_precision_kv_tr_amd as tr
    from mixed_precision_kv_tr_amd._lib import _Desc, _alloc, _free, _length, _write, _decode, _prefill, _export

    h = ctypes.c_void_p()
    assert _alloc(None, ctypes.byref(h)) == 1
    bad_dim = _Desc(1, 1, 1, 96, 16, 0, 0)
    assert _alloc(ctypes.byref(bad_dim), ctypes.byref(h)) == 5 and h.value is None
    bad_page = _Desc(1, 1, 1, 64, 16, 3000, 0)
    assert _alloc(ctypes.byref(bad_page), ctypes.byref(h)) == 1
    too_long = _Desc(1, 1, 1, 128, (1 << 23), 0, 0)          # staging offsets need < 2^31 bytes
    assert _alloc(ctypes.byref(too_long), ctypes.byref(h)) == 5 and h.value is None
    zero_layers = _Desc(0, 1, 1, 64, 16, 0, 0)
    assert _alloc(ctypes.byref(zero_layers), ctypes.byref(h)) == 1
    assert _free(None) == 0
    from mixed_precision_kv_tr_amd._lib import _set_chunks
    assert _set_chunks(None, 3) == 1
    for bad_pf in (-2, 17):                                  # prefill capacity: -1, 0 or 1 .. max_tokens
        d = _Desc(1, 1, 1, 64, 16, 0, 0, 0, bad_pf)
        assert _alloc(ctypes.byref(d), ctypes.byref(h)) == 1 and h.value is None
    assert _length(None, 0) == -1
    assert _write(None, 0, None, None, None, 1, None) == 1
    assert _decode(None, 0, None, None, 0, None, None) == 1
    assert _prefill(None, 0, None, None, None, None, None, 4, 0, None, None) == 1
    assert _export(None, 0, 0, 1, None, None, None, None, None) == 1
    with pytest.raises(tr.TriRouteError):
        tr.tr_kv_cache_alloc(1, 1, 1, 96, 16)


def test_controller_host_validation_without_gpu():
    import mixed_precision_kv_tr_amd as tr
    from mixed_precision_kv_tr_amd._lib import _CtlWeights, _ctl_route

    fake = 0x1000                                    # never dereferenced: every call below fails
    w = _CtlWeights(256, 0, 128, 4, *([fake] * 11))  # or returns before any launch
    route = lambda w, n: _ctl_route(ctypes.byref(w), fake, None, n, fake, fake, None)
    assert route(w, 0) == 0                          # no tokens: nothing to do
    assert route(w, -1) == 1
    for field, bad in (("d_r", 64), ("d", 100), ("d", 32), ("d", 96), ("d_side", 33), ("heads", 0), ("heads", 65)):
        w2 = _CtlWeights.from_buffer_copy(w)
        setattr(w2, field, bad)
        assert route(w2, 5) == 1, field
    w3 = _CtlWeights.from_buffer_copy(w)
    w3.w_b = None
    assert route(w3, 5) == 1
    w4 = _CtlWeights.from_buffer_copy(w)
    w4.d_side = 4                                    # side features without a side pointer
    assert _ctl_route(ctypes.byref(w4), fake, None, 5, fake, fake, None) == 1
    assert _ctl_route(None, fake, None, 5, fake, fake, None) == 1


def test_controller_workspace_host_checks_without_gpu():
    from mixed_precision_kv_tr_amd._lib import _CtlWeights, _ctl_route, _ctl_ws_bytes

    # 4 bytes x 8 token blocks x ceil(d / 256) channel slices x 32 tokens x (128 units + 1)
    for d, slices in ((64, 1), (256, 1), (320, 2), (768, 3), (2048, 8), (16384, 64)):
        assert _ctl_ws_bytes(d) == 4 * 8 * slices * 32 * 129, d
    for d in (0, 32, 100, 16448):
        assert _ctl_ws_bytes(d) == -1
    fake = 0x1000                                    # never dereferenced: every call fails first
    need = _ctl_ws_bytes(2048)
    w = _CtlWeights(2048, 0, 128, 4, *([fake] * 11), fake, need - 4)
    route = lambda w, n: _ctl_route(ctypes.byref(w), fake, None, n, fake, fake, None)
    assert route(w, 5) == 1                          # one float short
    assert route(w, 1000) == 1                       # checked for large calls too
    w.workspace_bytes, w.workspace = need, fake + 4  # not 16-byte aligned
    assert route(w, 5) == 1


def test_controller_pack_host_validation_without_gpu():
    from mixed_precision_kv_tr_amd._lib import _ctl_pack
    a, b = 0x1000, 0x2000                            # never dereferenced: every call fails first
    assert _ctl_pack(None, b, 128, None) == 1
    assert _ctl_pack(a, None, 128, None) == 1
    assert _ctl_pack(a, a, 128, None) == 1
    for d in (0, 32, 100, 16448):
        assert _ctl_pack(a, b, d, None) == 1


def test_moe_host_validation_without_gpu():
    from mixed_precision_kv_tr_amd._lib import _MoeDesc, _moe_alloc, _moe_ffn, _moe_set, _moe_free, _moe_status
    h = ctypes.c_void_p()
    for bad in ((100, 128, 4, 2, 16), (128, 100, 4, 2, 16), (128, 128, 0, 2, 16), (128, 128, 65, 2, 16),
                (128, 128, 4, 3, 16), (128, 128, 4, 0, 16), (128, 128, 4, 2, 0), (64, 128, 4, 2, 16)):
        assert _moe_alloc(ctypes.byref(_MoeDesc(*bad)), ctypes.byref(h)) == 1, bad
    assert _moe_alloc(None, ctypes.byref(h)) == 1
    assert _moe_ffn(None, 0x1000, 0x1000, 4, 0x1000, None) == 1
    assert _moe_set(None, 0x1000, 0x1000, 0x1000, None) == 1
    assert _moe_status(None, None) == 1
    assert _moe_free(None) == 0
