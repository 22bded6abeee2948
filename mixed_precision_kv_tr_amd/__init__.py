"""Python binding of libtriroute (TriRoute routed attention over a mixed-precision KV cache,
hand-written HIP kernels for MI355X / gfx950).

The binding only marshals arguments: every step runs in the C-ABI library declared in
include/triroute.h.  There is no CPU fallback: the first use of any binding name loads
libtriroute.so and raises ImportError if it is missing.  (The ``build`` submodule imports
without the library, so it can build it.)
"""

_EXPORTS = (
    "TR_MODE_SKIP", "TR_MODE_LOCAL", "TR_MODE_FULL", "TriRouteError", "KVCache", "lib", "lib_path",
    "tr_kv_cache_alloc", "tr_kv_cache_free", "tr_kv_cache_reset", "tr_kv_cache_length",
    "tr_kv_quantize_write", "tr_routed_attn_decode", "tr_routed_attn_prefill", "tr_kv_cache_export",
    "tr_kv_cache_status", "tr_kv_cache_pages_used", "tr_status_str", "tr_kv_cache_truncate",
    "tr_kv_cache_set_decode_chunks", "tr_routed_attn_decode_noalloc",
    "tr_profile_enable", "tr_profile_read", "PROFILE_FAMILIES", "tr_controller_route",
    "ControllerWeights", "MoE", "tr_moe_alloc", "tr_moe_set_weights", "tr_moe_ffn", "tr_moe_status",
)

__all__ = list(_EXPORTS)


def __getattr__(name):
    if name in _EXPORTS:
        from . import _lib
        return getattr(_lib, name)
    raise AttributeError(name)
