"""ctypes binding of libtriroute.so with the C ABI's names (include/triroute.h).

Argument marshalling only: tensors are passed as device pointers (``data_ptr()``), the stream
as the raw hipStream_t of ``torch.cuda.current_stream()`` unless one is given.  Every wrapper
checks the returned status and raises TriRouteError on failure.
"""

from __future__ import annotations

import ctypes
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
lib_path = os.path.join(_HERE, "libtriroute.so")

if not os.path.exists(lib_path):
    raise ImportError(
        f"{lib_path} is missing: build it with `python -m mixed_precision_kv_tr_amd.build` "
        "(or __graft_entry__.build()); there is no CPU fallback")

lib = ctypes.CDLL(lib_path)

TR_MODE_SKIP, TR_MODE_LOCAL, TR_MODE_FULL = 0, 1, 2
_vp, _i32, _i64 = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64


class _Desc(ctypes.Structure):
    _fields_ = [("num_layers", _i32), ("batch", _i32), ("num_heads", _i32), ("head_dim", _i32),
                ("max_tokens", _i32), ("page_code_bytes", _i32), ("pool_pages", _i64),
                ("num_query_heads", _i32), ("prefill_tokens", _i32)]


class _CtlWeights(ctypes.Structure):
    _fields_ = [("d", _i32), ("d_side", _i32), ("d_r", _i32), ("heads", _i32)] + [
        (n, _vp) for n in ("w1", "w1_side", "b1", "w2", "b2", "mu_a", "sigma_a", "mu_b", "sigma_b", "w_a", "w_b")] + [
        ("workspace", _vp), ("workspace_bytes", _i64)]


class _MoeDesc(ctypes.Structure):
    _fields_ = [("d", _i32), ("d_expert", _i32), ("experts", _i32), ("top_k", _i32), ("max_tokens", _i32)]


def _sig(name, res, *args):
    fn = getattr(lib, name)
    fn.restype = res
    fn.argtypes = list(args)
    return fn


_alloc = _sig("tr_kv_cache_alloc", ctypes.c_int, ctypes.POINTER(_Desc), ctypes.POINTER(_vp))
_free = _sig("tr_kv_cache_free", ctypes.c_int, _vp)
_reset = _sig("tr_kv_cache_reset", ctypes.c_int, _vp, _vp)
_length = _sig("tr_kv_cache_length", _i32, _vp, _i32)
_write = _sig("tr_kv_quantize_write", ctypes.c_int, _vp, _i32, _vp, _vp, _vp, _i32, _vp)
_decode = _sig("tr_routed_attn_decode", ctypes.c_int, _vp, _i32, _vp, _vp, _i32, _vp, _vp)
_decode_noalloc = _sig("tr_routed_attn_decode_noalloc", ctypes.c_int, _vp, _i32, _vp, _vp, _i32, _vp, _vp)
_prefill = _sig("tr_routed_attn_prefill", ctypes.c_int, _vp, _i32, _vp, _vp, _vp, _vp, _vp, _i32, _i32, _vp, _vp)
_export = _sig("tr_kv_cache_export", ctypes.c_int, _vp, _i32, _i32, _i32, _vp, _vp, _vp, _vp, _vp)
_status = _sig("tr_kv_cache_status", ctypes.c_int, _vp, _vp)
_pages = _sig("tr_kv_cache_pages_used", _i64, _vp, _vp)
_status_str = _sig("tr_status_str", ctypes.c_char_p, ctypes.c_int)
_truncate = _sig("tr_kv_cache_truncate", ctypes.c_int, _vp, _i32, _i32)
_ctl_pack = _sig("tr_controller_pack_w1", ctypes.c_int, _vp, _vp, _i32, _vp)
_ctl_ws_bytes = _sig("tr_controller_workspace_bytes", _i64, _i32)
_ctl_route = _sig("tr_controller_route", ctypes.c_int, ctypes.POINTER(_CtlWeights), _vp, _vp, _i64, _vp, _vp, _vp)
_moe_alloc = _sig("tr_moe_alloc", ctypes.c_int, ctypes.POINTER(_MoeDesc), ctypes.POINTER(_vp))
_moe_free = _sig("tr_moe_free", ctypes.c_int, _vp)
_moe_set = _sig("tr_moe_set_weights", ctypes.c_int, _vp, _vp, _vp, _vp, _vp)
_moe_ffn = _sig("tr_moe_ffn", ctypes.c_int, _vp, _vp, _vp, _i32, _vp, _vp)
_moe_status = _sig("tr_moe_status", ctypes.c_int, _vp, _vp)
_set_chunks = _sig("tr_kv_cache_set_decode_chunks", ctypes.c_int, _vp, _i32)
_prof_enable = _sig("tr_profile_enable", ctypes.c_int, _vp, _i32)
_prof_read = _sig("tr_profile_read", ctypes.c_int, _vp, ctypes.POINTER(_i64), ctypes.POINTER(ctypes.c_double))
PROFILE_FAMILIES = ("write", "decode_split", "decode_combine", "prefill_prep", "prefill_attn", "prefill_merge")

STATUS_NAMES = {0: "TR_OK", 1: "TR_ERR_INVALID_ARG", 2: "TR_ERR_CAPACITY", 3: "TR_ERR_OUT_OF_PAGES",
                4: "TR_ERR_HIP", 5: "TR_ERR_UNSUPPORTED", 6: "TR_ERR_BAD_VALUE", 7: "TR_ERR_RANGE",
                8: "TR_ERR_SCRATCH"}


class TriRouteError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: {STATUS_NAMES.get(status, status)} ({tr_status_str(status)})")


def tr_status_str(status: int) -> str:
    return _status_str(int(status)).decode()


def _check(status: int, where: str):
    if status != 0:
        raise TriRouteError(status, where)


def _ptr(t):
    if t is None:
        return None
    if isinstance(t, int):
        return t
    if not t.is_cuda:
        raise ValueError("tensor arguments must live in GPU memory")
    if not t.is_contiguous():
        raise ValueError("tensor arguments must be contiguous")
    return t.data_ptr()


def _stream(stream):
    if stream is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


class KVCache:
    """Owning handle of a tr_kv_cache (freed on close / garbage collection)."""

    def __init__(self, handle: int, desc: dict):
        self.handle = handle
        self.desc = desc

    def close(self):
        if self.handle:
            _free(self.handle)
            self.handle = None

    def __del__(self):  # pragma: no cover
        try:
            self.close()
        except Exception:
            pass


def tr_kv_cache_alloc(num_layers: int, batch: int, num_heads: int, head_dim: int, max_tokens: int,
                      page_code_bytes: int = 0, pool_pages: int = 0, num_query_heads: int = 0,
                      prefill_tokens: int = 0) -> KVCache:
    """num_heads: KV heads; num_query_heads: query heads (0 = num_heads; a multiple for GQA);
    prefill_tokens: positions a prefill may reach (0 = max_tokens, -1 = no prefill scratch)."""
    d = _Desc(num_layers, batch, num_heads, head_dim, max_tokens, page_code_bytes, pool_pages, num_query_heads,
              prefill_tokens)
    h = _vp()
    _check(_alloc(ctypes.byref(d), ctypes.byref(h)), "tr_kv_cache_alloc")
    return KVCache(h.value, dict(num_layers=num_layers, batch=batch, num_heads=num_heads, head_dim=head_dim,
                                 max_tokens=max_tokens, page_code_bytes=page_code_bytes, pool_pages=pool_pages,
                                 num_query_heads=num_query_heads or num_heads, prefill_tokens=prefill_tokens))


def tr_kv_cache_free(cache: KVCache):
    cache.close()


def tr_kv_cache_reset(cache: KVCache, stream=None):
    _check(_reset(cache.handle, _stream(stream)), "tr_kv_cache_reset")


def tr_kv_cache_length(cache: KVCache, layer: int) -> int:
    return int(_length(cache.handle, layer))


def tr_kv_quantize_write(cache: KVCache, layer: int, k, v, bits, n_new: int | None = None, stream=None):
    n = int(bits.shape[1]) if n_new is None else int(n_new)
    _check(_write(cache.handle, layer, _ptr(k), _ptr(v), _ptr(bits), n, _stream(stream)), "tr_kv_quantize_write")


def tr_routed_attn_decode(cache: KVCache, layer: int, q, mode, window: int, out, stream=None):
    _check(_decode(cache.handle, layer, _ptr(q), _ptr(mode), int(window), _ptr(out), _stream(stream)),
           "tr_routed_attn_decode")


def tr_routed_attn_decode_noalloc(cache: KVCache, layer: int, q, mode, window: int, out, stream=None):
    """tr_routed_attn_decode with the split-K partials in the library's fixed device array."""
    _check(_decode_noalloc(cache.handle, layer, _ptr(q), _ptr(mode), int(window), _ptr(out), _stream(stream)),
           "tr_routed_attn_decode_noalloc")


def tr_routed_attn_prefill(cache: KVCache, layer: int, q, k, v, bits, mode, T: int, window: int, out,
                           stream=None):
    _check(_prefill(cache.handle, layer, _ptr(q), _ptr(k), _ptr(v), _ptr(bits), _ptr(mode), int(T), int(window),
                    _ptr(out), _stream(stream)), "tr_routed_attn_prefill")


def tr_kv_cache_export(cache: KVCache, layer: int, tok0: int, n: int, codes, scale, zero, bits, stream=None):
    _check(_export(cache.handle, layer, tok0, n, _ptr(codes), _ptr(scale), _ptr(zero), _ptr(bits),
                   _stream(stream)), "tr_kv_cache_export")


def tr_kv_cache_status(cache: KVCache, stream=None) -> int:
    """Synchronizes and returns the sticky status code (0 = ok); does not raise."""
    return int(_status(cache.handle, _stream(stream)))


def tr_kv_cache_pages_used(cache: KVCache, stream=None) -> int:
    return int(_pages(cache.handle, _stream(stream)))


def tr_kv_cache_set_decode_chunks(cache: KVCache, n: int):
    """Force n position chunks per full decode window (0 = the library's automatic choice)."""
    _check(_set_chunks(cache.handle, n), "tr_kv_cache_set_decode_chunks")


def tr_kv_cache_truncate(cache: KVCache, layer: int, new_len: int):
    _check(_truncate(cache.handle, layer, new_len), "tr_kv_cache_truncate")


class ControllerWeights:
    """The C struct tr_controller_weights built once from a dict of device tensors (and holding
    them alive, with w1 packed by tr_controller_pack_w1), so that a call passes one pointer.
    With workspace=True (the default) it also owns the optional workspace that lets calls of up
    to 256 tokens spread over many workgroups."""

    NAMES = ("w1", "w1_side", "b1", "w2", "b2", "mu_a", "sigma_a", "mu_b", "sigma_b", "w_a", "w_b")

    def __init__(self, weights: dict, stream=None, workspace: bool = True):
        import torch
        d_r, d = weights["w1"].shape
        side = weights.get("w1_side")
        self.d_side = int(side.shape[1]) if side is not None else 0
        self.heads = weights["w_a"].shape[1] // 3
        self.tensors = dict(weights)
        # the first layer in the matrix-core operand order (packed once, on the device)
        self.tensors["w1"] = torch.empty_like(weights["w1"])
        _check(_ctl_pack(_ptr(weights["w1"]), _ptr(self.tensors["w1"]), int(d), _stream(stream)),
               "tr_controller_pack_w1")
        ws, ws_bytes = None, 0
        if workspace:
            ws_bytes = int(_ctl_ws_bytes(int(d)))
            if ws_bytes < 0:
                raise ValueError(f"tr_controller_workspace_bytes: unsupported d = {d}")
            self.workspace = torch.empty((ws_bytes,), dtype=torch.uint8, device=weights["w1"].device)
            ws = _ptr(self.workspace)
        self.struct = _CtlWeights(d, self.d_side, d_r, self.heads,
                                  *[_ptr(self.tensors[n]) if (n != "w1_side" or self.d_side) else None
                                    for n in self.NAMES], ws, ws_bytes)


def tr_controller_route(weights, x, side, n_tokens: int, mode, bits, stream=None):
    """weights: a ControllerWeights, or a dict of device tensors w1 (bf16 [128][d], unpacked), w1_side
    ([128][d_side]), b1, w2 ([128][128], in x out), b2, mu_a, sigma_a, mu_b, sigma_b, w_a
    ([128][3 heads], in x out), w_b ([128][4]); x bf16 [n, d]; side float32 [n, d_side] or None;
    mode uint8 [n, heads] and bits uint8 [n] receive the decisions."""
    if not isinstance(weights, ControllerWeights):
        weights = ControllerWeights(weights)
    _check(_ctl_route(ctypes.byref(weights.struct), _ptr(x), _ptr(side) if weights.d_side else None,
                      int(n_tokens), _ptr(mode), _ptr(bits), _stream(stream)), "tr_controller_route")


class MoE:
    """Owning handle of a tr_moe (freed on close / garbage collection)."""

    def __init__(self, handle: int, desc: dict):
        self.handle = handle
        self.desc = desc

    def close(self):
        if self.handle:
            _moe_free(self.handle)
            self.handle = None

    def __del__(self):  # pragma: no cover
        try:
            self.close()
        except Exception:
            pass


def tr_moe_alloc(d: int, d_expert: int, experts: int, top_k: int, max_tokens: int) -> MoE:
    desc = _MoeDesc(d, d_expert, experts, top_k, max_tokens)
    h = _vp()
    _check(_moe_alloc(ctypes.byref(desc), ctypes.byref(h)), "tr_moe_alloc")
    return MoE(h.value, dict(d=d, d_expert=d_expert, experts=experts, top_k=top_k, max_tokens=max_tokens))


def tr_moe_set_weights(moe: MoE, w_gate, w_up, w_down, stream=None):
    _check(_moe_set(moe.handle, _ptr(w_gate), _ptr(w_up), _ptr(w_down), _stream(stream)), "tr_moe_set_weights")


def tr_moe_ffn(moe: MoE, x, gate_logits, n_tokens: int, y, stream=None):
    _check(_moe_ffn(moe.handle, _ptr(x), _ptr(gate_logits), int(n_tokens), _ptr(y), _stream(stream)), "tr_moe_ffn")


def tr_moe_status(moe: MoE, stream=None) -> int:
    """Synchronizes and returns the handle's sticky status code (0 = ok); does not raise."""
    return int(_moe_status(moe.handle, _stream(stream)))


def tr_profile_enable(cache: KVCache, enable: bool = True):
    _check(_prof_enable(cache.handle, 1 if enable else 0), "tr_profile_enable")


def tr_profile_read(cache: KVCache) -> dict:
    """{family: (launches, total_ms)} since the last read (synchronizes)."""
    n = (_i64 * len(PROFILE_FAMILIES))()
    ms = (ctypes.c_double * len(PROFILE_FAMILIES))()
    _check(_prof_read(cache.handle, n, ms), "tr_profile_read")
    return {name: (int(n[i]), float(ms[i])) for i, name in enumerate(PROFILE_FAMILIES)}
