"""Host check of the argument behind the quantizer's fast path (the GPU kernels round each
quotient d / s of Eq. (4) from q = fl(d * r), r an approximate reciprocal of s with at most 1 ulp
error, and fall back to the correctly rounded divide when q lies within (2^b - 1) * 2^-20 of a
half-integer).

The claim: whenever q passes that test, rint(q) equals rint(fl(d / s)).  It is checked here in
float32 with the reciprocal pushed a full ulp either way, on Eq. (4)'s own inputs (bf16 groups,
b in {2, 4, 8}) and on quotients steered next to half-integers, where the claim is tightest."""

import numpy as np


def margin(b: int) -> np.float32:
    return np.float32(0.5) - np.float32(2 ** b - 1) * np.float32(2.0 ** -20)


def bf16_round(x: np.ndarray) -> np.ndarray:
    u = x.astype(np.float32).view(np.uint32).astype(np.uint64)
    u = (u + 0x7FFF + ((u >> 16) & 1)) >> 16 << 16
    return u.astype(np.uint32).view(np.float32)


def check(d: np.ndarray, s: np.ndarray, b: int):
    d = d.astype(np.float32)
    s = s.astype(np.float32)
    exact = np.rint(d / s)
    r0 = np.float32(1.0) / s
    fast_taken = 0
    for r in (r0, np.nextafter(r0, np.float32(np.inf)), np.nextafter(r0, np.float32(0))):
        q = d * r
        cf = np.rint(q)
        ok = np.abs(q - cf) < margin(b)
        assert np.array_equal(cf[ok], exact[ok]), "fast path disagrees with the exact divide"
        fast_taken += int(ok.sum())
    return fast_taken


def test_eq4_groups():
    rng = np.random.default_rng(3)
    for b in (2, 4, 8):
        nlev = np.float32(2 ** b - 1)
        for scale in (1e-3, 1.0, 7.0, 300.0):
            x = bf16_round(rng.standard_normal((20000, 64)).astype(np.float32) * np.float32(scale))
            mn, mx = x.min(1), x.max(1)
            z = mn + np.float32(0)
            s = (mx - mn) / nlev + np.float32(0)
            d = x - z[:, None]
            taken = check(d, np.broadcast_to(s[:, None], d.shape), b)
            assert taken > 0.99 * 3 * d.size


def test_near_half_integers():
    rng = np.random.default_rng(5)
    for b in (2, 4, 8):
        nlev = 2 ** b - 1
        s = (rng.uniform(0.5, 2.0, 200000) * 2.0 ** rng.integers(-20, 20, 200000)).astype(np.float32)
        k = rng.integers(0, nlev, 200000).astype(np.float32) + np.float32(0.5)
        d = (k * s).astype(np.float32)
        # walk d a few ulps around k * s so that d / s straddles the half-integer
        for steps in (-3, -1, 0, 1, 3):
            dd = d.copy()
            direction = np.float32(np.inf) if steps > 0 else np.float32(0)
            for _ in range(abs(steps)):
                dd = np.nextafter(dd, direction)
            check(dd, s, b)
