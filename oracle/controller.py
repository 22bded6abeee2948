"""The inference-time routing decisions of the TriRoute review page (xllm-io.github.io, "core
formulas" item 5, the shared controller, Eq. (5); item 10, per-axis whitening, Eq. (11); and
the inference paragraph after Algorithm 1: the routers take the hard argmax).

TEST INFRASTRUCTURE ONLY (see the package docstring).

For every token t of a layer:

    h_t      = trunk([Norm(x_t); psi_t])            two-layer MLP to d_r = 128 units   (Eq. 5)
    hhat_t   = RMSNorm(h_t)                                                            (Eq. 5)
    hhat^ax  = (hhat_t - mu_ax) / (sigma_ax + eps_w)   per axis, frozen statistics      (Eq. 11)
    z^a      = W_a hhat^a   (3 logits per attention head: skip, local, full)            (Eq. 5)
    z^b      = W_b hhat^b   (4 logits: b = 2, 4, 8, 16)                                 (Eq. 5)
    mode[t, h] = argmax z^a[h],  bits[t] = (2, 4, 8, 16)[argmax z^b]          (inference: hard)

Readings where the page is silent (each listed in the design notes):
* Norm is RMSNorm with unit gain and eps 1e-6 (a learned gain folds into the trunk's first
  layer); RMSNorm of h likewise.
* The trunk is Linear(d + d_side -> d_r) with bias, SiLU, Linear(d_r -> d_r) with bias.
* The side features psi_t are given by the caller (the page lists relative position, distance
  to the last whitespace/BOS, a running entropy estimate and the previous layer's decisions).
* Eq. (11)'s statistics are the frozen running values at inference; eps_w = 1e-5.
* The heads have no bias.  Head h's logits sit in columns 3h, 3h + 1, 3h + 2 of z^a.
* Ties go to the lowest index (skip before local before full; the narrower width first).
* The experts head (z^e) belongs to the FFN experts and is not computed here.

Weight layouts (the same arrays the GPU path receives):
    w1      bf16 bits uint16 [d_r][d]      layer 1, residual part (out x in)
    w1_side float32 [d_r][d_side]          layer 1, side-feature part (out x in)
    b1, b2  float32 [d_r]
    w2      float32 [d_r][d_r]             layer 2, stored in x out
    mu_a, sigma_a, mu_b, sigma_b  float32 [d_r]
    w_a     float32 [d_r][3 H]             attention head, stored in x out
    w_b     float32 [d_r][4]               bit head, stored in x out
Everything is computed in float64 from these values.
"""

from __future__ import annotations

import numpy as np

from .quantize import bf16_bits_to_f32

BIT_CHOICES = (2, 4, 8, 16)
EPS_NORM = 1e-6
EPS_WHITEN = 1e-5


def _rms_norm(v: np.ndarray, eps: float) -> np.ndarray:
    """v / sqrt(mean(v^2) + eps) over the last axis (unit gain)."""
    return v / np.sqrt(np.mean(v * v, axis=-1, keepdims=True) + eps)


def _silu(v: np.ndarray) -> np.ndarray:
    return v / (1.0 + np.exp(-v))


def controller_logits(x_bits, side, w: dict):
    """Eq. (5) and (11) for M tokens.

    x_bits: uint16 bf16 [M, d] residual states; side: float32 [M, d_side] (d_side may be 0).
    Returns (z_a float64 [M, H, 3], z_b float64 [M, 4])."""
    x = bf16_bits_to_f32(np.asarray(x_bits, dtype=np.uint16)).astype(np.float64)
    side = np.asarray(side, dtype=np.float64).reshape(x.shape[0], -1)
    w1 = bf16_bits_to_f32(np.asarray(w["w1"], dtype=np.uint16)).astype(np.float64)
    w1s = np.asarray(w["w1_side"], dtype=np.float64).reshape(w1.shape[0], -1)
    f = lambda k: np.asarray(w[k], dtype=np.float64)
    u = _rms_norm(x, EPS_NORM)                                  # Norm(x_t)
    h1 = _silu(u @ w1.T + side @ w1s.T + f("b1"))               # trunk layer 1 on [Norm(x); psi]
    h = h1 @ f("w2") + f("b2")                                  # trunk layer 2
    hh = _rms_norm(h, EPS_NORM)                                 # RMSNorm(h_t)
    ha = (hh - f("mu_a")) / (f("sigma_a") + EPS_WHITEN)         # Eq. (11), attention axis
    hb = (hh - f("mu_b")) / (f("sigma_b") + EPS_WHITEN)         # Eq. (11), bit axis
    za = ha @ f("w_a")
    zb = hb @ f("w_b")
    return za.reshape(x.shape[0], -1, 3), zb


def controller_route(x_bits, side, w: dict):
    """Hard decisions: (mode uint8 [M, H] with 0 skip / 1 local / 2 full, bits uint8 [M] in
    {2, 4, 8, 16}, z_a, z_b)."""
    za, zb = controller_logits(x_bits, side, w)
    mode = np.argmax(za, axis=2).astype(np.uint8)               # first maximum on ties
    bits = np.asarray(BIT_CHOICES, dtype=np.uint8)[np.argmax(zb, axis=1)]
    return mode, bits, za, zb
