"""Pins for the oracle's routed attention (Eq. 2 of the TriRoute review page, item (A)) and
for the cached inference step that feeds it quantized K/V (Eq. 4 + the inference paragraph).

Checked against: torch's scaled-dot-product attention in float64 on the CPU (a library
routine, with is_causal or an explicit boolean mask), closed forms (skip = 0, one key gives
its value, a zero query averages the window, equal values give that value), and a
pure-Python brute force over every mode assignment of tiny inputs.
"""

import itertools
import math

import numpy as np
import pytest
import torch

import oracle
from oracle import MODE_FULL, MODE_LOCAL, MODE_SKIP


def sdpa(q, k, v, mask=None, causal=False):
    """torch SDPA in float64; q [Tq,H,D], k/v [Tk,H,D] -> [Tq,H,D]."""
    qt = torch.from_numpy(np.ascontiguousarray(q.transpose(1, 0, 2)))
    kt = torch.from_numpy(np.ascontiguousarray(k.transpose(1, 0, 2)))
    vt = torch.from_numpy(np.ascontiguousarray(v.transpose(1, 0, 2)))
    m = None if mask is None else torch.from_numpy(mask)
    out = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, attn_mask=m, is_causal=causal)
    return out.numpy().transpose(1, 0, 2)


def rand(rng, *shape):
    return rng.normal(size=shape)


# --- closed forms -----------------------------------------------------------------------

def test_skip_outputs_zero():
    rng = np.random.default_rng(0)
    q, k, v = rand(rng, 5, 2, 8), rand(rng, 5, 2, 8), rand(rng, 5, 2, 8)
    mode = np.zeros((5, 2), dtype=np.int64)
    out = oracle.routed_attention(q, k, v, mode, np.arange(5), 3)
    assert np.all(out == 0.0)


@pytest.mark.parametrize("m", [MODE_LOCAL, MODE_FULL])
def test_first_position_returns_its_value(m):
    rng = np.random.default_rng(1)
    q, k, v = rand(rng, 1, 3, 8), rand(rng, 1, 3, 8), rand(rng, 1, 3, 8)
    out = oracle.routed_attention(q, k, v, np.full((1, 3), m), np.array([0]), 4)
    np.testing.assert_allclose(out, v, rtol=0, atol=1e-15)


def test_local_window_zero_is_own_value():
    rng = np.random.default_rng(2)
    q, k, v = rand(rng, 6, 2, 4), rand(rng, 6, 2, 4), rand(rng, 6, 2, 4)
    out = oracle.routed_attention(q, k, v, np.full((6, 2), MODE_LOCAL), np.arange(6), 0)
    np.testing.assert_allclose(out, v, rtol=0, atol=1e-15)


@pytest.mark.parametrize("w", [0, 1, 3, 7, 20])
def test_zero_query_averages_exactly_the_window(w):
    # One-hot values (v_j = e_j) with a zero query: the output is 1/|J| on the keys of the
    # window J and 0 elsewhere, which reads the key set off directly.
    T = 12
    v = np.zeros((T, 1, T))
    v[np.arange(T), 0, np.arange(T)] = 1.0
    k = np.random.default_rng(3).normal(size=(T, 1, T))
    q = np.zeros((T, 1, T))
    for m in (MODE_LOCAL, MODE_FULL):
        out = oracle.routed_attention(q, k, v, np.full((T, 1), m), np.arange(T), w)
        for t in range(T):
            lo = 0 if m == MODE_FULL else max(0, t - w)
            expect = np.zeros(T)
            expect[lo:t + 1] = 1.0 / (t + 1 - lo)          # keys t-w .. t inclusive
            np.testing.assert_allclose(out[t, 0], expect, rtol=0, atol=1e-15)


def test_equal_values_give_that_value():
    rng = np.random.default_rng(4)
    row = rng.normal(size=8)
    v = np.broadcast_to(row, (9, 2, 8)).copy()
    q, k = rand(rng, 9, 2, 8), rand(rng, 9, 2, 8)
    mode = rng.integers(1, 3, size=(9, 2))
    out = oracle.routed_attention(q, k, v, mode, np.arange(9), 2)
    np.testing.assert_allclose(out, np.broadcast_to(row, out.shape), rtol=1e-14, atol=1e-14)


# --- library routine: torch SDPA in float64 ---------------------------------------------------

def test_all_full_equals_causal_sdpa():
    rng = np.random.default_rng(5)
    T, H, D = 33, 3, 16
    q, k, v = rand(rng, T, H, D), rand(rng, T, H, D) * 2.0, rand(rng, T, H, D)
    out = oracle.routed_attention(q, k, v, np.full((T, H), MODE_FULL), np.arange(T), 0)
    np.testing.assert_allclose(out, sdpa(q, k, v, causal=True), rtol=1e-12, atol=1e-12)


def test_mixed_modes_equal_masked_sdpa():
    rng = np.random.default_rng(6)
    T, H, D, w = 40, 4, 8, 5
    q, k, v = rand(rng, T, H, D), rand(rng, T, H, D), rand(rng, T, H, D)
    mode = rng.integers(0, 3, size=(T, H))
    out = oracle.routed_attention(q, k, v, mode, np.arange(T), w)
    pos = np.arange(T)
    for h in range(H):
        mask = np.zeros((1, T, T), dtype=bool)
        for t in range(T):
            if mode[t, h] == MODE_FULL:
                mask[0, t] = pos <= t
            elif mode[t, h] == MODE_LOCAL:
                mask[0, t] = (pos <= t) & (pos >= t - w)
            else:
                mask[0, t, 0] = True                       # placeholder row, checked below
        ref = sdpa(q[:, h:h + 1], k[:, h:h + 1], v[:, h:h + 1], mask=mask)[:, 0]
        live = mode[:, h] != MODE_SKIP
        np.testing.assert_allclose(out[live, h], ref[live], rtol=1e-12, atol=1e-12)
        assert np.all(out[~live, h] == 0.0)


def test_wide_local_window_equals_full():
    rng = np.random.default_rng(7)
    T, H, D = 20, 2, 8
    q, k, v = rand(rng, T, H, D), rand(rng, T, H, D), rand(rng, T, H, D)
    full = oracle.routed_attention(q, k, v, np.full((T, H), MODE_FULL), np.arange(T), 0)
    for w in (T - 1, T, 5 * T):
        local = oracle.routed_attention(q, k, v, np.full((T, H), MODE_LOCAL), np.arange(T), w)
        np.testing.assert_array_equal(local, full)


# --- brute force on tiny inputs ------------------------------------------------------------

def brute(q, k, v, mode, w):
    """Scalar loops with math.exp: Eq. (2) one (query, head, key, channel) at a time."""
    T, H, D = len(q), len(q[0]), len(q[0][0])
    out = [[[0.0] * D for _ in range(H)] for _ in range(T)]
    for t in range(T):
        for h in range(H):
            if mode[t][h] == MODE_SKIP:
                continue
            keys = range(0, t + 1) if mode[t][h] == MODE_FULL else range(max(0, t - w), t + 1)
            sc = {j: sum(q[t][h][c] * k[j][h][c] for c in range(D)) / math.sqrt(D) for j in keys}
            mx = max(sc.values())
            wts = {j: math.exp(sc[j] - mx) for j in keys}
            tot = sum(wts.values())
            for c in range(D):
                out[t][h][c] = sum(wts[j] * v[j][h][c] for j in keys) / tot
    return np.array(out)


def test_bruteforce_every_mode_assignment():
    rng = np.random.default_rng(8)
    T, H, D = 4, 2, 3
    q, k, v = rand(rng, T, H, D), rand(rng, T, H, D), rand(rng, T, H, D)
    for w in (0, 1, 2):
        for flat in itertools.product((0, 1, 2), repeat=T * H):
            mode = np.array(flat).reshape(T, H)
            out = oracle.routed_attention(q, k, v, mode, np.arange(T), w)
            ref = brute(q.tolist(), k.tolist(), v.tolist(), mode.tolist(), w)
            np.testing.assert_allclose(out, ref, rtol=1e-13, atol=1e-13)


def test_query_subset_positions():
    # Queries at arbitrary positions (decode: one query at the last position) equal the
    # corresponding rows of the all-positions result.
    rng = np.random.default_rng(9)
    T, H, D = 15, 2, 8
    q, k, v = rand(rng, T, H, D), rand(rng, T, H, D), rand(rng, T, H, D)
    mode = rng.integers(0, 3, size=(T, H))
    every = oracle.routed_attention(q, k, v, mode, np.arange(T), 3)
    sel = np.array([14, 3, 0, 9])
    some = oracle.routed_attention(q[sel], k, v, mode[sel], sel, 3)
    np.testing.assert_array_equal(some, every[sel])


# --- the cached inference step ----------------------------------------------------------------

def bf16_bits(x):
    return (np.asarray(x, dtype=np.float32).view(np.uint32) >> 16).astype(np.uint16)


def test_cached_b16_full_is_dense_causal_attention():
    rng = np.random.default_rng(10)
    T, H, D = 24, 2, 16
    qb, kb, vb = (bf16_bits(rand(rng, T, H, D)) for _ in range(3))
    res = oracle.attend_cached(qb, kb, vb, np.full(T, 16), np.full((T, H), MODE_FULL), np.arange(T), 0)
    f = lambda b: oracle.bf16_bits_to_f32(b).astype(np.float64)
    np.testing.assert_allclose(res["out"], sdpa(f(qb), f(kb), f(vb), causal=True), rtol=1e-12, atol=1e-12)


@pytest.mark.parametrize("b", [2, 4, 8])
def test_cached_lossless_when_values_sit_on_the_grid(b):
    # K/V rows whose values are z + c*s with s a power of two and integer c spanning 0..n
    # quantize without loss, so attention over the cache equals attention over the raw rows.
    rng = np.random.default_rng(11 + b)
    T, H, D = 10, 2, 8
    n = 2 ** b - 1

    def grid_rows():
        c = rng.integers(0, n + 1, size=(T, H, D))
        c[..., 0], c[..., 1] = 0, n                           # pin min and max
        s = 2.0 ** rng.integers(-3, 2, size=(T, H, 1))
        z = s * rng.integers(-n, 1, size=(T, H, 1))          # z/s + c stays within bf16's
        return z + c * s                                        # 8 significant bits

    kx, vx = grid_rows(), grid_rows()
    qx = rand(rng, T, H, D)
    qb, kb, vb = bf16_bits(qx), bf16_bits(kx), bf16_bits(vx)
    mode = rng.integers(0, 3, size=(T, H))
    res = oracle.attend_cached(qb, kb, vb, np.full(T, b), mode, np.arange(T), 3)
    np.testing.assert_array_equal(res["k_hat"], kx)
    np.testing.assert_array_equal(res["v_hat"], vx)
    f = lambda x: oracle.bf16_bits_to_f32(x).astype(np.float64)
    ref = brute(f(qb).tolist(), kx.tolist(), vx.tolist(), mode.tolist(), 3)
    np.testing.assert_allclose(res["out"], ref, rtol=1e-12, atol=1e-12)


def test_cached_attends_to_the_quantized_values():
    # With b = 2 a generic row is not reproduced exactly; the output must follow the
    # quantized row, which differs from attention over the raw row.
    rng = np.random.default_rng(12)
    T, H, D = 6, 1, 8
    qb, kb, vb = (bf16_bits(rand(rng, T, H, D)) for _ in range(3))
    mode = np.full((T, H), MODE_FULL)
    res2 = oracle.attend_cached(qb, kb, vb, np.full(T, 2), mode, np.arange(T), 0)
    res16 = oracle.attend_cached(qb, kb, vb, np.full(T, 16), mode, np.arange(T), 0)
    assert np.max(np.abs(res2["out"] - res16["out"])) > 1e-3
    # the first query has a single key: its output is exactly the dequantized value row
    np.testing.assert_array_equal(res2["out"][0], res2["v_hat"][0])


# --- grouped-query attention (query head h reads KV head h // (H / H_kv)) -------------------

def test_gqa_all_full_equals_sdpa_with_grouped_kv():
    rng = np.random.default_rng(21)
    T, Hq, Hkv, D = 29, 8, 2, 16
    q, k, v = rand(rng, T, Hq, D), rand(rng, T, Hkv, D), rand(rng, T, Hkv, D)
    out = oracle.routed_attention(q, k, v, np.full((T, Hq), MODE_FULL), np.arange(T), 0)
    qt = torch.from_numpy(np.ascontiguousarray(q.transpose(1, 0, 2)))
    kt = torch.from_numpy(np.ascontiguousarray(k.transpose(1, 0, 2)))
    vt = torch.from_numpy(np.ascontiguousarray(v.transpose(1, 0, 2)))
    ref = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, is_causal=True, enable_gqa=True)
    np.testing.assert_allclose(out, ref.numpy().transpose(1, 0, 2), rtol=1e-12, atol=1e-12)


def test_gqa_mixed_modes_equal_mha_on_repeated_kv():
    rng = np.random.default_rng(22)
    T, Hq, Hkv, D, w = 37, 6, 3, 8, 4
    q, k, v = rand(rng, T, Hq, D), rand(rng, T, Hkv, D), rand(rng, T, Hkv, D)
    mode = rng.integers(0, 3, size=(T, Hq))
    out = oracle.routed_attention(q, k, v, mode, np.arange(T), w)
    rep = Hq // Hkv                                      # KV head j serves query heads j*rep .. j*rep+rep-1
    ref = oracle.routed_attention(q, np.repeat(k, rep, axis=1), np.repeat(v, rep, axis=1), mode, np.arange(T), w)
    np.testing.assert_allclose(out, ref, rtol=0, atol=0)
    # a KV head mapping h % Hkv (instead of h // rep) would differ
    bad = oracle.routed_attention(q, np.tile(k, (1, rep, 1)), np.tile(v, (1, rep, 1)), mode, np.arange(T), w)
    assert not np.allclose(out, bad)


def test_gqa_rejects_a_kv_head_count_that_does_not_divide():
    rng = np.random.default_rng(23)
    q, k = rand(rng, 4, 6, 8), rand(rng, 4, 4, 8)
    with pytest.raises(ValueError):
        oracle.routed_attention(q, k, k, np.full((4, 6), MODE_FULL), np.arange(4), 0)
