"""The FFN axis of the TriRoute review page (xllm-io.github.io, "core formulas" item 3, Eq. (3)):
E experts plus a null expert f_0 = 0, a softmax gate over the E + 1 options, the top-k set S_t,
and the selected experts' outputs weighted by their gate probabilities renormalized over S_t.

TEST INFRASTRUCTURE ONLY (see the package docstring).

    p_t       = softmax(z_t^e)                                   E + 1 logits, index 0 = null
    S_t       = the k largest p_t (ties: the lower index)
    FFN_t     = sum_{j in S_t} p_tj / sum_{j' in S_t} p_tj' * f_j(Norm(x_t)),   f_0 = 0

Readings where the page is silent (each listed in the design notes):
* Norm is RMSNorm with unit gain and eps 1e-6.
* Each expert is a SwiGLU FFN, f_j(u) = W2_j (silu(W1_j u) * (W3_j u)), no biases: the model
  table's FFN widths are 8/3 of the model width, the SwiGLU convention; with top-2 routing the
  page keeps the active FFN FLOPs of the dense model, so an expert's hidden width is half of it.
* Every step after the bf16 inputs (x, the weights) is float64: Eq. (3) fixes no intermediate
  precision, so none is imposed here.
* The gate logits z^e come from the controller's expert head (Eq. (5)); here they are an input.

Weight layouts (the arrays the GPU path packs):
    w_gate, w_up  bf16 bits uint16 [E][d_e][d]     W1_j, W3_j (out x in)
    w_down        bf16 bits uint16 [E][d][d_e]     W2_j (out x in)
"""

from __future__ import annotations

import numpy as np

from .quantize import bf16_bits_to_f32

EPS_NORM = 1e-6


def gate(z, k: int):
    """Top-k of softmax(z) with renormalized weights.  z: [M, E + 1].
    Returns (sel int64 [M, k] in selection order, weights float64 [M, k])."""
    z = np.asarray(z, dtype=np.float64)
    p = np.exp(z - z.max(axis=1, keepdims=True))
    p /= p.sum(axis=1, keepdims=True)
    sel = np.zeros((z.shape[0], k), dtype=np.int64)
    avail = np.ones_like(p, dtype=bool)
    for j in range(k):
        masked = np.where(avail, p, -np.inf)
        sel[:, j] = np.argmax(masked, axis=1)                       # first maximum on ties
        avail[np.arange(z.shape[0]), sel[:, j]] = False
    ps = np.take_along_axis(p, sel, axis=1)
    return sel, ps / ps.sum(axis=1, keepdims=True)


def expert_out(u, w_gate_e, w_up_e, w_down_e):
    """f_j(u) = W2 (silu(W1 u) * (W3 u)) for rows u [n, d] of one expert, float64."""
    g = u @ w_gate_e.T
    h = g / (1.0 + np.exp(-g)) * (u @ w_up_e.T)
    return h @ w_down_e.T


def moe_ffn(x_bits, z, w_gate, w_up, w_down, k: int, sel=None):
    """Eq. (3) for M tokens.  x_bits: uint16 bf16 [M, d]; z: [M, E + 1] gate logits.
    sel: optional int [M, k] selected gate indices to use instead of the top-k of the gate (for
    checking a result against another valid choice where gate probabilities tie); the weights
    are then p renormalized over that set.
    Returns (y float64 [M, d], sel, weights)."""
    x = bf16_bits_to_f32(np.asarray(x_bits, dtype=np.uint16)).astype(np.float64)
    u = x / np.sqrt(np.mean(x * x, axis=1, keepdims=True) + EPS_NORM)          # Norm(x_t)
    w1 = bf16_bits_to_f32(np.asarray(w_gate, dtype=np.uint16)).astype(np.float64)
    w3 = bf16_bits_to_f32(np.asarray(w_up, dtype=np.uint16)).astype(np.float64)
    w2 = bf16_bits_to_f32(np.asarray(w_down, dtype=np.uint16)).astype(np.float64)
    if sel is None:
        sel, wt = gate(z, k)
    else:
        sel = np.asarray(sel, dtype=np.int64)
        zz = np.asarray(z, dtype=np.float64)
        p = np.exp(zz - zz.max(axis=1, keepdims=True))
        p /= p.sum(axis=1, keepdims=True)
        ps = np.take_along_axis(p, sel, axis=1)
        wt = ps / ps.sum(axis=1, keepdims=True)
    y = np.zeros_like(x)
    for e in range(1, w1.shape[0] + 1):                            # expert e is gate index e
        rows, slots = np.nonzero(sel == e)
        if rows.size == 0:
            continue
        y[rows] += wt[rows, slots][:, None] * expert_out(u[rows], w1[e - 1], w3[e - 1], w2[e - 1])
    return y, sel, wt
