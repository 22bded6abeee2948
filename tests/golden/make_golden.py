"""Writes tests/golden/tiny_cached_attention.json from the oracle alone.

The TriRoute pages print no numeric worked example for Eq. (2) or Eq. (4), so the stored
fixture is the oracle's own output on small, fixed inputs.  It guards the oracle against
silent drift (tests/test_golden.py re-derives it) and gives the GPU tests a tiny case whose
expected values do not depend on a live oracle call.  Inputs are drawn from numpy's PCG64
with a fixed seed; every expected value comes from ``oracle.attend_cached``.

Run from the repository root:  python tests/golden/make_golden.py
"""

import json
import os
import sys

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
sys.path.insert(0, ROOT)

import oracle  # noqa: E402

CASES = [
    # (name, T, H, D, window, seed)
    ("T7_H2_D64_w2", 7, 2, 64, 2, 11),
    ("T9_H3_D128_w4", 9, 3, 128, 4, 12),
]


def bf16_bits(x):
    return (np.asarray(x, dtype=np.float32).view(np.uint32) >> 16).astype(np.uint16)


def make_case(name, T, H, D, w, seed):
    rng = np.random.Generator(np.random.PCG64(seed))
    q = bf16_bits(rng.normal(size=(T, H, D)))
    k = bf16_bits(rng.normal(size=(T, H, D)) * np.exp(0.5 * rng.normal(size=(1, H, D))))
    v = bf16_bits(rng.normal(size=(T, H, D)))
    bits = np.array([2, 4, 8, 16] * T, dtype=np.int64)[:T]
    rng.shuffle(bits)
    mode = rng.integers(0, 3, size=(T, H))
    res = oracle.attend_cached(q, k, v, bits, mode, np.arange(T), w)
    return {
        "name": name, "T": T, "H": H, "D": D, "window": w,
        "q": q.tolist(), "k": k.tolist(), "v": v.tolist(),
        "bits": bits.tolist(), "mode": mode.tolist(),
        "codes": res["codes"].tolist(),
        "scale_f32_bits": res["scale"].view(np.uint32).tolist(),
        "zero_f32_bits": res["zero"].view(np.uint32).tolist(),
        "out_f64_hex": [[[float(x).hex() for x in row] for row in head] for head in res["out"]],
    }


def main():
    data = {
        "about": "oracle output on fixed inputs; written by tests/golden/make_golden.py",
        "cases": [make_case(*c) for c in CASES],
    }
    path = os.path.join(os.path.dirname(os.path.abspath(__file__)), "tiny_cached_attention.json")
    with open(path, "w") as f:
        json.dump(data, f, separators=(",", ":"))
    print("wrote", path)


if __name__ == "__main__":
    main()
