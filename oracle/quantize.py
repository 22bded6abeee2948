"""Eq. (4) of the TriRoute review page (xllm-io.github.io, "core formulas", item (C) KV-cache
bit width): asymmetric per-token grouped quantization at width b.

TEST INFRASTRUCTURE ONLY (see the package docstring).

Definition followed, per group x (one head's K or V vector of one token):

    s = (max(x) - min(x)) / (2^b - 1),   z = min(x),   code = round((x - z) / s),
    Q_b(x) = code * s + z,               b = 16  ->  native storage (no quantization).

Every floating-point step of the code computation is a single IEEE binary32 operation with
round-to-nearest-even, done with numpy float32 arrays, in this order:

    mx, mn = max(x), min(x)          (exact)
    z      = mn + 0.0                (turns -0 into +0; otherwise exact)
    R      = fl32(mx - mn)
    s      = fl32(R / n) + 0.0   n = 2^b - 1 (the + 0.0 turns a -0 range into +0)
    d      = fl32(x - z)
    r      = fl32(d / s)
    code   = rint(r)                 (round half to even; exact on a float32)

A group with s == 0 (all elements equal) gets code 0 everywhere, so Q_b(x) = z = x.
For b = 16 the "code" is the raw bf16 bit pattern and (s, z) = (1, 0) by convention.
"""

from __future__ import annotations

import numpy as np

BITS_ALLOWED = (2, 4, 8, 16)


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    """Widen bf16 bit patterns (uint16) to float32 exactly: the bf16 bits are the top half."""
    bits = np.asarray(bits, dtype=np.uint16)
    return (bits.astype(np.uint32) << np.uint32(16)).view(np.float32)


def quantize(x_bits: np.ndarray, b, group_size: int | None = None):
    """Quantize bf16 groups at width b (Eq. 4).

    x_bits: uint16 bf16 bit patterns, shape [..., G]; the last axis holds one or more groups.
    b: width per group row, an int or an integer array broadcastable to x_bits.shape[:-1];
       every value must be in {2, 4, 8, 16}.
    group_size: elements per quantization group (default: the whole last axis).  Must divide
       the last axis.  The HIP library supports only the default (one head vector per group).

    Returns (codes uint16 [..., G], s float32, z float32); s and z have shape [...] for the
    default group, else [..., G // group_size].  For b = 16 rows, codes are the input bits and
    s = 1, z = 0.
    """
    x_bits = np.asarray(x_bits, dtype=np.uint16)
    lead, G = x_bits.shape[:-1], x_bits.shape[-1]
    g = G if group_size is None else int(group_size)
    if g <= 0 or G % g:
        raise ValueError("group_size must divide the last axis")
    ng = G // g
    b_arr = np.broadcast_to(np.asarray(b, dtype=np.int64), lead)
    if not np.isin(b_arr, BITS_ALLOWED).all():
        raise ValueError("b must be one of 2, 4, 8, 16")

    xb = x_bits.reshape(lead + (ng, g))
    x = bf16_bits_to_f32(xb)                                   # [..., ng, g] float32
    bg = np.broadcast_to(b_arr[..., None], lead + (ng,))       # width per group

    mx = x.max(axis=-1)
    mn = x.min(axis=-1)
    z = mn + np.float32(0.0)
    R = mx - mn
    n = (np.left_shift(np.int64(1), bg) - 1).astype(np.float32)
    s = R / n + np.float32(0.0)

    native = bg == 16
    degenerate = (s == np.float32(0.0)) & ~native
    safe_s = np.where(degenerate | native, np.float32(1.0), s)
    d = x - z[..., None]
    r = d / safe_s[..., None]
    c = np.rint(r)
    c = np.where((degenerate | native)[..., None], np.float32(0.0), c)   # native rows keep bits
    quant = ~native
    if quant.any():
        cq = c[quant]
        nq = n[quant][..., None]
        if not np.all((cq >= 0) & (cq <= nq)):
            # Cannot happen for finite input: r lies in [0, n(1 + 2^-23)] and rint of the
            # upper end is n.  An out-of-range code means non-finite input.
            raise FloatingPointError("quantizer produced an out-of-range code (non-finite input?)")
    codes = np.where(native[..., None], xb, c.astype(np.uint16))
    s_out = np.where(native, np.float32(1.0), s).astype(np.float32)
    z_out = np.where(native, np.float32(0.0), z).astype(np.float32)
    if group_size is None:                      # one group per row: drop the group axis
        s_out, z_out = s_out[..., 0], z_out[..., 0]
    return codes.reshape(lead + (G,)).astype(np.uint16), s_out, z_out


def dequantize(codes: np.ndarray, s: np.ndarray, z: np.ndarray, b, group_size: int | None = None):
    """Reconstruct Q_b(x) = code * s + z in float64 (Eq. 4); b = 16 rows widen the bf16 bits.

    code * s is exact in float64 (at most 8 + 24 significant bits), so the only rounding is
    the final addition of z.
    """
    codes = np.asarray(codes, dtype=np.uint16)
    lead, G = codes.shape[:-1], codes.shape[-1]
    g = G if group_size is None else int(group_size)
    ng = G // g
    b_arr = np.broadcast_to(np.asarray(b, dtype=np.int64), lead)
    cg = codes.reshape(lead + (ng, g))
    sg = np.asarray(s, dtype=np.float32).reshape(lead + (ng,)).astype(np.float64)
    zg = np.asarray(z, dtype=np.float32).reshape(lead + (ng,)).astype(np.float64)
    quant = cg.astype(np.float64) * sg[..., None] + zg[..., None]
    native = bf16_bits_to_f32(cg).astype(np.float64)
    out = np.where((b_arr == 16)[..., None, None], native, quant)
    return out.reshape(lead + (G,))
