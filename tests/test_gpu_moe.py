"""GPU parity of the expert FFN (Eq. (3)) against the oracle: |gpu - oracle| <= 2e-3 + 1e-2 |oracle|
element-wise on fp32 outputs.  The oracle computes Eq. (3) in float64 throughout; the GPU feeds the
matrix cores bf16 operands (the normalized input and the hidden activation rounded to bf16) and
accumulates in fp32, which the tolerance covers.

Expert selection is a top-k of softmax probabilities, fp32 on the GPU and fp64 in the oracle.
Where the k-th and (k+1)-th largest gate logits of a token differ by more than
TAU = 1e-4 * (1 + max |z|) the selected set is unique and the oracle's must be used; inside that
margin any set that takes every logit above the tie and k of the tied ones is a correct top-k, and
the GPU's output must match the oracle evaluated on one of them.  (The GPU's probabilities carry
fp32 rounding of ~1e-6 relative, two orders of magnitude below TAU.)"""

import itertools

import numpy as np
import pytest
import torch

import oracle
from tests.gpu_helpers import ATOL, RTOL, compare_out, say, u16
from workloads import moe_case

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def tr():
    import mixed_precision_kv_tr_amd as tr
    return tr


def run(tr, c, k, n=None):
    M, d = c["x"].shape
    E, de = c["w_gate"].shape[0], c["w_gate"].shape[1]
    n = M if n is None else n
    moe = tr.tr_moe_alloc(d, de, E, k, M)
    tr.tr_moe_set_weights(moe, c["w_gate"], c["w_up"], c["w_down"])
    y = torch.full((M, d), float("nan"), dtype=torch.float32, device="cuda")
    tr.tr_moe_ffn(moe, c["x"], c["z"], n, y)
    torch.cuda.synchronize()
    assert tr.tr_moe_status(moe) == 0, "fp16 range flag set on ordinary inputs"
    moe.close()
    return y.cpu().numpy()


def reference(c, k, rows):
    return oracle.moe_ffn(u16(c["x"])[rows], c["z"].cpu().numpy()[rows], u16(c["w_gate"]), u16(c["w_up"]),
                          u16(c["w_down"]), k)


def tied_sets(z, k):
    """Every correct top-k set of one token's logits z [E + 1] under the TAU margin."""
    tau = 1e-4 * (1 + np.abs(z).max())
    zk = np.sort(z)[::-1][k - 1]
    sure = [j for j in range(z.size) if z[j] > zk + tau]
    cand = [j for j in range(z.size) if abs(z[j] - zk) <= tau]
    return [sure + list(extra) for extra in itertools.combinations(cand, k - len(sure))]


def compare_with_ties(c, k, rows, y, where):
    """compare_out on tokens whose top-k set is unique; each tied token must match the oracle on one
    of its correct sets."""
    z = c["z"].cpu().numpy()[rows].astype(np.float64)
    sets = [tied_sets(z[i], k) for i in range(len(rows))]
    unique = np.array([len(s) == 1 for s in sets])
    ref, _, _ = reference(c, k, rows)
    compare_out(y[unique], ref[unique], where)
    args = (u16(c["w_gate"]), u16(c["w_up"]), u16(c["w_down"]), k)
    for i in np.nonzero(~unique)[0]:
        r = rows[i]
        ok = False
        for S in sets[i]:
            alt, _, _ = oracle.moe_ffn(u16(c["x"])[[r]], c["z"].cpu().numpy()[[r]], *args, sel=np.array([S]))
            err = np.abs(y[i] - alt[0])
            ok = ok or bool(np.all(err <= ATOL + RTOL * np.abs(alt[0])))
        assert ok, f"{where}: token {r} (tied gate logits) matches none of its correct top-{k} sets"
    say(f"  {where}: {int((~unique).sum())} tokens with tied top-{k} sets")


# calls above 512 tokens take the tiled products (the down product only when d is a multiple of
# 256: (600, 640, ...) takes the other one)
@pytest.mark.parametrize("M,d,de,E,k", [(100, 128, 128, 4, 2), (1000, 768, 1024, 8, 2), (33, 256, 384, 3, 1),
                                        (1, 128, 128, 1, 2), (77, 384, 256, 16, 1), (700, 512, 256, 5, 2),
                                        (600, 640, 256, 4, 2), (513, 256, 384, 3, 1)])
def test_moe_matches_oracle(tr, M, d, de, E, k):
    say(f"moe M={M} d={d} d_e={de} E={E} k={k}")
    c = moe_case(M, d, de, E, seed=M + E, device="cuda")
    y = run(tr, c, k)
    compare_with_ties(c, k, np.arange(M), y, f"M={M} d={d} E={E} k={k}")
    _, sel, _ = reference(c, k, np.arange(min(M, 64)))
    say(f"  null-expert share of the choices: {np.mean(sel == 0):.3f}")


def test_moe_null_expert_heavy(tr):
    """Most tokens pick the null expert first: their outputs are exactly zero (k = 1) or the other
    expert's weighted output (k = 2)."""
    for M, k in ((300, 1), (300, 2), (800, 1), (800, 2)):
        c = moe_case(M, 256, 256, 4, seed=9, device="cuda", null_bias=2.0)
        y = run(tr, c, k)
        _, sel, _ = reference(c, k, np.arange(M))
        if k == 1:
            z = c["z"].cpu().numpy()
            alone = [i for i in range(M) if sel[i, 0] == 0 and len(tied_sets(z[i].astype(np.float64), 1)) == 1]
            assert np.all(y[alone] == 0.0)
        compare_with_ties(c, k, np.arange(M), y, f"null-heavy M={M} k={k}")


def test_moe_partial_call_and_full_size_sample(tr):
    """A 1.3B-shaped layer (2048 tokens, d = 2048, d_e = 2688, 8 experts, top-2) checked on sampled
    tokens, and a call on the first n < max_tokens tokens leaves the rest untouched."""
    c = moe_case(2048, 2048, 2688, 8, seed=3, device="cuda", cid=5)
    y = run(tr, c, 2)
    rows = np.random.default_rng(0).choice(2048, 48, replace=False)
    compare_with_ties(c, 2, rows, y[rows], "1.3B-shaped, sampled tokens")
    y2 = run(tr, c, 2, n=1000)
    assert np.array_equal(y2[:1000], y[:1000]) and np.all(np.isnan(y2[1000:]))


def test_moe_fp16_range_is_flagged(tr):
    """The down product runs on fp16 operands: a W2 weight or a hidden value beyond fp16's range
    (|v| > 65504) sets the handle's sticky TR_ERR_RANGE flag instead of passing silently."""
    M, d, de, E = 64, 256, 256, 4
    c = moe_case(M, d, de, E, seed=21, device="cuda")
    y = torch.empty((M, d), dtype=torch.float32, device="cuda")
    # a W2 weight of 2^17
    w_down = c["w_down"].clone()
    w_down[1, 5, 7] = 131072.0
    moe = tr.tr_moe_alloc(d, de, E, 2, M)
    tr.tr_moe_set_weights(moe, c["w_gate"], c["w_up"], w_down)
    assert tr.tr_moe_status(moe) == 7                                   # TR_ERR_RANGE
    moe.close()
    # hidden values beyond fp16's range: gate and up weights 400x larger, so silu(g) * u ~ 1e5
    moe = tr.tr_moe_alloc(d, de, E, 2, M)
    tr.tr_moe_set_weights(moe, (c["w_gate"].float() * 400).to(torch.bfloat16),
                          (c["w_up"].float() * 400).to(torch.bfloat16), c["w_down"])
    assert tr.tr_moe_status(moe) == 0
    tr.tr_moe_ffn(moe, c["x"], c["z"], M, y)
    assert tr.tr_moe_status(moe) == 7
    moe.close()


@pytest.mark.parametrize("M,k", [(32, 2), (300, 2), (33, 1), (1000, 2)])
def test_moe_is_deterministic(tr, M, k):
    """Two calls on the same inputs give bit-identical outputs (no atomics; small top-2 calls sum
    their per-slot partial rows in a fixed order, large calls store slot 0 and add slot 1)."""
    c = moe_case(M, 256, 384, 4, seed=5 + M, device="cuda")
    y1 = run(tr, c, k)
    y2 = run(tr, c, k)
    assert np.array_equal(y1, y2)
    assert np.all(np.isfinite(y1))
