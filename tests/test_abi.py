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
    for code in range(7):
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
    zero_layers = _Desc(0, 1, 1, 64, 16, 0, 0)
    assert _alloc(ctypes.byref(zero_layers), ctypes.byref(h)) == 1
    assert _free(None) == 0
    assert _length(None, 0) == -1
    assert _write(None, 0, None, None, None, 1, None) == 1
    assert _decode(None, 0, None, None, 0, None, None) == 1
    assert _prefill(None, 0, None, None, None, None, None, 4, 0, None, None) == 1
    assert _export(None, 0, 0, 1, None, None, None, None, None) == 1
    with pytest.raises(tr.TriRouteError):
        tr.tr_kv_cache_alloc(1, 1, 1, 96, 16)
