"""Pins for the oracle's quantizer (Eq. 4 of the TriRoute review page, item (C)).

None of these re-derive the oracle's own code path: they check it against hand-worked
closed forms, an exact-rational model of IEEE binary32 arithmetic, invariants the equation
implies (code range, extremes, reconstruction error, nearest quantization level) and the
special cases the page states (b = 16 is native storage).
"""

from fractions import Fraction

import numpy as np
import pytest

import oracle
from tests.exact_f32 import bf16_to_fraction, f32_bits, quantize_group_exact, round_f32


def bf16(values):
    """bf16 bit patterns of values that are exactly representable in bf16."""
    a = np.asarray(values, dtype=np.float32)
    bits = a.view(np.uint32)
    assert np.all(bits & 0xFFFF == 0), "test value not exact in bf16"
    return (bits >> 16).astype(np.uint16)


def random_groups(rng, n_groups, D, spread):
    """bf16 groups: N(0,1) values times a per-group scale, rounded to bf16 by truncation of
    a float32 (any bf16 pattern is a valid input; the rounding method does not matter here)."""
    scale = np.exp(rng.normal(0.0, spread, size=(n_groups, 1))).astype(np.float32)
    x = (rng.normal(size=(n_groups, D)).astype(np.float32) * scale).astype(np.float32)
    return (x.view(np.uint32) >> 16).astype(np.uint16)


# --- hand-worked closed forms (round half to even on exact ties) -------------------------

def test_ties_b2():
    # x = [0, .5, 1.5, 3], b = 2: z = 0, s = 3/3 = 1, (x - z)/s = [0, .5, 1.5, 3] -> [0, 0, 2, 3]
    codes, s, z = oracle.quantize(bf16([0.0, 0.5, 1.5, 3.0]), 2)
    assert codes.tolist() == [0, 0, 2, 3]
    assert float(s) == 1.0 and float(z) == 0.0


def test_ties_b4():
    # z = -1, s = 15/15 = 1; (x - z) = [0, 15, .5, 1.5, 2.5, 3.5] -> [0, 15, 0, 2, 2, 4]
    codes, s, z = oracle.quantize(bf16([-1.0, 14.0, -0.5, 0.5, 1.5, 2.5]), 4)
    assert codes.tolist() == [0, 15, 0, 2, 2, 4]
    assert float(s) == 1.0 and float(z) == -1.0


def test_ties_b8():
    # z = 0, s = 255/255 = 1; 127.5 -> 128 (even), 126.5 -> 126 (even)
    codes, s, z = oracle.quantize(bf16([0.0, 255.0, 127.5, 126.5]), 8)
    assert codes.tolist() == [0, 255, 128, 126]
    assert float(s) == 1.0


def test_non_unit_scale_b2():
    # x = [2, 8, 4, 6, 5], b = 2: z = 2, s = 6/3 = 2, (x - z)/s = [0, 3, 1, 2, 1.5] -> 1.5 -> 2
    codes, s, z = oracle.quantize(bf16([2.0, 8.0, 4.0, 6.0, 5.0]), 2)
    assert codes.tolist() == [0, 3, 1, 2, 2]
    assert float(s) == 2.0 and float(z) == 2.0
    xh = oracle.dequantize(codes, s, z, 2)
    assert xh.tolist() == [2.0, 8.0, 4.0, 6.0, 6.0]


# --- special cases stated by the page or forced by the definition ------------------------

def test_b16_is_native_storage():
    rng = np.random.default_rng(1)
    x = random_groups(rng, 7, 64, 2.0)
    codes, s, z = oracle.quantize(x, 16)
    assert np.array_equal(codes, x)
    assert np.all(s == 1.0) and np.all(z == 0.0)
    xh = oracle.dequantize(codes, s, z, 16)
    assert np.array_equal(xh, oracle.bf16_bits_to_f32(x).astype(np.float64))


@pytest.mark.parametrize("b", [2, 4, 8])
def test_constant_group(b):
    x = bf16([-3.25] * 16)
    codes, s, z = oracle.quantize(x, b)
    assert np.all(codes == 0) and float(s) == 0.0 and float(z) == -3.25
    assert np.all(oracle.dequantize(codes, s, z, b) == -3.25)


def test_negative_zero_becomes_positive_zero():
    neg0 = np.uint16(0x8000)
    codes, s, z = oracle.quantize(np.array([neg0, neg0, neg0], dtype=np.uint16), 4)
    assert f32_bits(Fraction(0)) == 0 and np.float32(z).view(np.uint32) == 0
    assert np.all(codes == 0)
    codes, s, z = oracle.quantize(np.array([neg0, bf16([3.0])[0], 0], dtype=np.uint16), 2)
    assert np.float32(z).view(np.uint32) == 0
    assert codes.tolist() == [0, 3, 0] and float(s) == 1.0


def test_signed_zero_range_gives_positive_zero_scale():
    # a group of +0 and -0 has max - min = +-0 depending on which zero is taken as the max;
    # the scale is canonicalised to +0 either way, so its bits are well defined
    for pattern in ([0x0000, 0x8000], [0x8000, 0x0000], [0x8000, 0x8000, 0x0000]):
        codes, s, z = oracle.quantize(np.array(pattern, dtype=np.uint16), 8)
        assert np.float32(s).view(np.uint32) == 0 and np.float32(z).view(np.uint32) == 0
        assert np.all(codes == 0)


def test_rejects_other_widths():
    with pytest.raises(ValueError):
        oracle.quantize(bf16([1.0, 2.0]), 3)


# --- exact IEEE binary32 semantics ------------------------------------------------------

@pytest.mark.parametrize("b", [2, 4, 8])
@pytest.mark.parametrize("D,spread", [(8, 0.5), (64, 0.5), (128, 3.0)])
def test_matches_exact_rational_model(b, D, spread):
    rng = np.random.default_rng(100 + b * 7 + D)
    x = random_groups(rng, 40, D, spread)
    codes, s, z = oracle.quantize(x, b)
    for g in range(x.shape[0]):
        ec, es, ez = quantize_group_exact(x[g].tolist(), b)
        assert codes[g].tolist() == ec
        assert np.float32(s[g]).view(np.uint32) == f32_bits(es)
        assert np.float32(z[g]).view(np.uint32) == f32_bits(ez)


def test_tiny_and_huge_magnitudes_match_exact_model():
    # bf16 subnormals, values near the fp32 normal boundary and large (but finite-range)
    # magnitudes: the quantizer must not flush or lose them.
    groups = [
        np.array([0x0001, 0x0003, 0x007F, 0x0000, 0x8002], dtype=np.uint16),  # subnormal bf16
        np.array([0x0080, 0x0081, 0x00FF, 0x8080], dtype=np.uint16),          # around 2^-126
        np.array([0x7149, 0xF149, 0x6FF2, 0x0000], dtype=np.uint16),         # about +-1e30
        np.array([0x3F80, 0x3F81, 0x3F82, 0x3F83], dtype=np.uint16),          # 1 .. 1+3 ulp
    ]
    for x in groups:
        for b in (2, 4, 8):
            codes, s, z = oracle.quantize(x, b)
            ec, es, ez = quantize_group_exact(x.tolist(), b)
            assert codes.tolist() == ec, (x, b)
            assert np.float32(s).view(np.uint32) == f32_bits(es)
            assert np.float32(z).view(np.uint32) == f32_bits(ez)


def test_divide_is_a_true_divide_not_a_reciprocal_multiply():
    """Find bf16 inputs where x / s and x * (1/s) round to different codes, and check the
    oracle follows the correctly rounded divide.  (A search over all bf16 values in [0, M].)"""
    found = 0
    for M in (3.0, 5.0, 7.0, 11.0, 13.0, 100.0, 1000.0):
        top = bf16([M])[0]
        xs = np.arange(0, int(top) + 1, dtype=np.uint32).astype(np.uint16)
        xf = oracle.bf16_bits_to_f32(xs)
        for b in (2, 4, 8):
            n = np.float32(2 ** b - 1)
            s = np.float32(M) / n
            recip = np.rint(xf * (np.float32(1.0) / s))
            true = np.rint(xf / s)
            idx = np.nonzero((recip != true) & (xf <= np.float32(M)))[0]
            for i in idx[:4]:
                group = np.array([0, top, xs[i]], dtype=np.uint16)
                codes, _, _ = oracle.quantize(group, b)
                ec, _, _ = quantize_group_exact(group.tolist(), b)
                assert codes.tolist() == ec
                assert codes[2] == true[i] != recip[i]
                found += 1
    assert found > 0, "search found no discriminating input; widen it"


# --- invariants of Eq. (4) ---------------------------------------------------------------

@pytest.mark.parametrize("b", [2, 4, 8])
def test_invariants(b):
    rng = np.random.default_rng(7 + b)
    x = random_groups(rng, 300, 64, 1.5)
    codes, s, z = oracle.quantize(x, b)
    n = 2 ** b - 1
    xf = oracle.bf16_bits_to_f32(x).astype(np.float64)
    assert codes.max() <= n
    rows = np.arange(x.shape[0])
    live = s > 0
    # the minimum maps to code 0 and the maximum to code n
    assert np.all(codes[rows, xf.argmin(1)] == 0)
    assert np.all(codes[rows[live], xf[live].argmax(1)] == n)
    # reconstruction error: half a step plus the fp32 rounding of d, s and r
    xh = oracle.dequantize(codes, s, z, b)
    bound = s.astype(np.float64) * (0.5 + (n + 1) * 2.0 ** -22)
    assert np.all(np.abs(xh - xf) <= bound[:, None])
    # nearest level: away from exact half-way points, the code is the integer nearest to
    # (x - z)/s computed exactly
    for g in range(0, x.shape[0], 17):
        sg, zg = Fraction(float(s[g])), Fraction(float(z[g]))
        for i in range(x.shape[1]):
            t = (bf16_to_fraction(x[g, i]) - zg) / sg
            k = int(t + Fraction(1, 2))                  # t >= 0
            if abs(t - int(t) - Fraction(1, 2)) > Fraction(1, 2 ** 16):
                assert codes[g, i] == min(k, n)


def test_group_size_splits_the_vector():
    rng = np.random.default_rng(3)
    x = random_groups(rng, 5, 64, 1.0)
    c_all, s_all, z_all = oracle.quantize(x, 4, group_size=16)
    for j in range(4):
        c, s, z = oracle.quantize(x[:, 16 * j:16 * (j + 1)], 4)
        assert np.array_equal(c_all[:, 16 * j:16 * (j + 1)], c)
        assert np.array_equal(s_all[:, j], s) and np.array_equal(z_all[:, j], z)


def test_exact_model_self_check():
    # the exact model's rounding itself: 1 + 2^-24 is a tie between 1 and 1 + 2^-23 -> 1;
    # 1 + 3*2^-24 is a tie between 1 + 2^-23 and 1 + 2^-22 -> 1 + 2^-22 (even significand)
    assert round_f32(1 + Fraction(1, 2 ** 24)) == 1
    assert round_f32(1 + Fraction(3, 2 ** 24)) == 1 + Fraction(1, 2 ** 22)
    assert round_f32(Fraction(1, 3)) == Fraction(float(np.float32(1.0) / np.float32(3.0)))
