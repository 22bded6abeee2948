"""Eq. (2) of the TriRoute review page (xllm-io.github.io, "core formulas", item (A) attention
resolution): routed attention with one mode per (query token, head).

TEST INFRASTRUCTURE ONLY (see the package docstring).

    Attn_t = sum_m 1[a_t = m] Attn_t^(m)
    Attn_t^skip  = 0
    Attn_t^local = Attn(q_t, K[t-w .. t], V[t-w .. t])
    Attn_t^full  = Attn(q_t, K[<= t],     V[<= t])

Attn(q, K, V) is softmax attention with scores q . k_j / sqrt(D).  The same page routes
attention per head by default, so the mode is indexed by (query, head).  With grouped-query
attention (the page's experimental setup, section 5, uses H_kv = H/4) query head h reads KV
head h // (H / H_kv); H_kv = H is plain multi-head attention.  Positions are
0-based; the local window is the inclusive range [max(0, t - w), t] (w + 1 keys once t >= w).
Everything is float64; K and V are whatever the caller passes (for TriRoute: the cached,
dequantized values, see ``reference.attend_cached``).
"""

from __future__ import annotations

import numpy as np

MODE_SKIP = 0
MODE_LOCAL = 1
MODE_FULL = 2


def key_range(t: int, mode: int, window: int) -> tuple[int, int]:
    """Inclusive key-position range [lo, t] that a query at position t reads in `mode`."""
    if mode == MODE_FULL:
        return 0, t
    if mode == MODE_LOCAL:
        return max(0, t - window), t
    raise ValueError("skip mode reads no keys")


def routed_attention(q, k, v, mode, q_pos, window: int):
    """Routed attention, Eq. (2).

    q:     float [Tq, H, D]   queries
    k, v:  float [Tk, Hkv, D] keys / values by absolute position 0 .. Tk-1; Hkv divides H
    mode:  int   [Tq, H]      0 = skip, 1 = local-w, 2 = full
    q_pos: int   [Tq]         absolute position t of each query (t < Tk)
    window: w >= 0

    Returns float64 [Tq, H, D].  One query at a time, exactly as the definition reads.
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    mode = np.asarray(mode)
    q_pos = np.asarray(q_pos, dtype=np.int64)
    Tq, H, D = q.shape
    if k.ndim != 3 or k.shape[2] != D or v.shape != k.shape:
        raise ValueError("k/v must be [Tk, Hkv, D] matching q's D")
    Hkv = k.shape[1]
    if Hkv < 1 or H % Hkv:
        raise ValueError("the KV head count must divide the query head count")
    group = H // Hkv
    if window < 0:
        raise ValueError("window must be >= 0")
    if Tq and (q_pos.min() < 0 or q_pos.max() >= k.shape[0]):
        raise ValueError("query position outside the key range")
    inv_sqrt_d = 1.0 / np.sqrt(np.float64(D))
    out = np.zeros((Tq, H, D), dtype=np.float64)
    for i in range(Tq):
        t = int(q_pos[i])
        for h in range(H):
            m = int(mode[i, h])
            if m == MODE_SKIP:
                continue                                  # Attn^skip = 0
            if m not in (MODE_LOCAL, MODE_FULL):
                raise ValueError("mode must be 0, 1 or 2")
            lo, hi = key_range(t, m, window)
            kk = k[lo:hi + 1, h // group, :]
            vv = v[lo:hi + 1, h // group, :]
            scores = (kk @ q[i, h, :]) * inv_sqrt_d
            p = np.exp(scores - scores.max())
            out[i, h, :] = (p @ vv) / p.sum()
    return out
