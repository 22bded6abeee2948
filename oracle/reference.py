"""The inference step of the TriRoute review page (xllm-io.github.io, the paragraph that
follows Algorithm 1): each token's K/V is stored in the cache at the width b the controller
chose for it (Eq. 4), and every query attends, in its per-head mode (Eq. 2), to what was
stored -- including its own K/V, since the cache is written before it is read.

TEST INFRASTRUCTURE ONLY (see the package docstring).
"""

from __future__ import annotations

import numpy as np

from .attention import routed_attention
from .quantize import bf16_bits_to_f32, dequantize, quantize


def attend_cached(q_bits, k_bits, v_bits, bits, mode, q_pos, window: int):
    """Quantize-write every token of one sequence, then run routed attention over the cache.

    q_bits: uint16 bf16 [Tq, Hq, D]     queries (Hq a multiple of H: grouped-query attention)
    k_bits, v_bits: uint16 bf16 [T, H, D]  K/V of positions 0 .. T-1 (the cache contents)
    bits:   int [T]                      width b of each position, shared by K, V and heads
    mode:   int [Tq, Hq]                 0 skip, 1 local, 2 full
    q_pos:  int [Tq]                     position of each query (< T)

    Returns a dict with the attention output (float64 [Tq, Hq, D]), the cache contents
    (codes uint16 [T, 2, H, D]; scale, zero float32 [T, 2, H]; index 0 = K, 1 = V) and the
    dequantized K/V (float64 [T, H, D]).
    """
    k_bits = np.asarray(k_bits, dtype=np.uint16)
    v_bits = np.asarray(v_bits, dtype=np.uint16)
    T, H, D = k_bits.shape
    b = np.broadcast_to(np.asarray(bits, dtype=np.int64)[:, None], (T, H))
    kc, ks, kz = quantize(k_bits, b)
    vc, vs, vz = quantize(v_bits, b)
    k_hat = dequantize(kc, ks, kz, b)
    v_hat = dequantize(vc, vs, vz, b)
    q = bf16_bits_to_f32(np.asarray(q_bits, dtype=np.uint16)).astype(np.float64)
    out = routed_attention(q, k_hat, v_hat, mode, q_pos, window)
    return {
        "out": out,
        "codes": np.stack([kc, vc], axis=1),
        "scale": np.stack([ks, vs], axis=1),
        "zero": np.stack([kz, vz], axis=1),
        "k_hat": k_hat,
        "v_hat": v_hat,
    }
