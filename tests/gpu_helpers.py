"""Helpers shared by the GPU parity tests: run the HIP path through the C ABI, hand the very
same inputs (copied to the host) to the oracle, and compare."""

from __future__ import annotations

import sys

import numpy as np
import torch

import oracle

ATOL, RTOL = 2e-3, 1e-2        # |gpu - oracle| <= ATOL + RTOL * |oracle|, element-wise


def say(*args):
    print(*args, flush=True)
    sys.stdout.flush()


def u16(t: torch.Tensor) -> np.ndarray:
    """bf16 / uint16 tensor -> numpy uint16 bit patterns (host copy)."""
    if t.dtype == torch.bfloat16:
        t = t.view(torch.int16)
    return t.detach().cpu().numpy().view(np.uint16)


def bf16_to_f64(t: torch.Tensor) -> np.ndarray:
    return oracle.bf16_bits_to_f32(u16(t)).astype(np.float64)


def export_layer(tr, cache, layer: int, tok0: int, n: int, B: int, H: int, D: int):
    dev = torch.device("cuda")
    codes = torch.empty((B, n, 2, H, D), dtype=torch.int16, device=dev)
    scale = torch.empty((B, n, 2, H), dtype=torch.float32, device=dev)
    zero = torch.empty((B, n, 2, H), dtype=torch.float32, device=dev)
    bits = torch.empty((B, n), dtype=torch.uint8, device=dev)
    tr.tr_kv_cache_export(cache, layer, tok0, n, codes, scale, zero, bits)
    torch.cuda.synchronize()
    return (codes.cpu().numpy().view(np.uint16), scale.cpu().numpy(), zero.cpu().numpy(), bits.cpu().numpy())


def check_codes(exp, k, v, bits, seqs=None, where=""):
    """Bit-exact comparison of exported cache contents with the oracle's quantizer.

    exp: export_layer(...) result for positions 0..n-1; k, v: bf16 tensors [B, n, H, D];
    bits: uint8 tensor [B, n]."""
    codes, scale, zero, ebits = exp
    kb, vb, bb = u16(k), u16(v), bits.cpu().numpy().astype(np.int64)
    B = kb.shape[0]
    for s in (range(B) if seqs is None else seqs):
        b = np.broadcast_to(bb[s][:, None], kb.shape[1:3])
        kc, ks, kz = oracle.quantize(kb[s], b)
        vc, vs, vz = oracle.quantize(vb[s], b)
        assert np.array_equal(ebits[s], bb[s].astype(np.uint8)), f"{where} seq {s}: widths differ"
        for name, got, want in (("K codes", codes[s, :, 0], kc), ("V codes", codes[s, :, 1], vc)):
            bad = np.argwhere(got != want)
            assert bad.size == 0, f"{where} seq {s}: {name} differ at {bad[:5].tolist()}"
        for name, got, want in (("K scale", scale[s, :, 0], ks), ("V scale", scale[s, :, 1], vs),
                                ("K zero", zero[s, :, 0], kz), ("V zero", zero[s, :, 1], vz)):
            g, w = got.view(np.uint32), np.asarray(want, dtype=np.float32).view(np.uint32)
            bad = np.argwhere(g != w)
            assert bad.size == 0, f"{where} seq {s}: {name} bits differ at {bad[:5].tolist()}"


def compare_out(got: np.ndarray, ref: np.ndarray, where: str):
    err = np.abs(got - ref)
    tol = ATOL + RTOL * np.abs(ref)
    bad = np.argwhere(err > tol)
    rel = err / np.maximum(np.abs(ref), 1e-30)
    say(f"  {where}: max abs err {err.max():.3e}, max err/tol {(err / tol).max():.3f}, "
        f"elements {ref.size}")
    assert bad.size == 0, (f"{where}: {len(bad)} elements out of tolerance, first {bad[:5].tolist()}, "
                           f"max abs {err.max():.3e}, max rel {rel.max():.3e}")
