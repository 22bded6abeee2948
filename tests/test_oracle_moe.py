"""Pins of the expert-FFN oracle (Eq. (3): softmax gate over E experts and the null expert, top-k,
renormalized weights, SwiGLU experts) against library routines, closed forms and invariants."""

import numpy as np
import torch
import torch.nn.functional as F

import oracle
from workloads import moe_case


def _np(c):
    u16 = lambda t: t.view(torch.int16).numpy().view(np.uint16)
    return u16(c["x"]), c["z"].numpy(), u16(c["w_gate"]), u16(c["w_up"]), u16(c["w_down"])


def _torch_ffn(c, k):
    """Eq. (3) with torch's rms_norm / softmax / topk / silu / linear, all in float64."""
    x = c["x"].double()
    u = F.rms_norm(x, (x.shape[1],), eps=1e-6)
    p = F.softmax(c["z"].double(), dim=1)
    top, idx = torch.topk(p, k, dim=1)
    w = top / top.sum(dim=1, keepdim=True)
    y = torch.zeros_like(x)
    for t in range(x.shape[0]):
        for j in range(k):
            e = int(idx[t, j])
            if e == 0:
                continue
            h = F.silu(F.linear(u[t], c["w_gate"][e - 1].double())) * F.linear(u[t], c["w_up"][e - 1].double())
            y[t] += w[t, j] * F.linear(h, c["w_down"][e - 1].double())
    return y.numpy(), idx.numpy()


def test_matches_torch_library_routines():
    for k in (1, 2):
        c = moe_case(24, 128, 64, 4, seed=k)
        y, sel, _ = oracle.moe_ffn(*_np(c), k)
        yt, idx = _torch_ffn(c, k)
        assert np.array_equal(sel, idx)
        np.testing.assert_allclose(y, yt, rtol=1e-9, atol=1e-12)


def test_null_expert_alone_gives_zero():
    c = moe_case(16, 128, 64, 3, seed=4, null_bias=50.0)
    y, sel, wt = oracle.moe_ffn(*_np(c), 1)
    assert np.all(sel[:, 0] == 0) and np.all(wt == 1.0)
    assert np.all(y == 0.0)


def test_equal_logits_take_the_lowest_indices_with_equal_weights():
    """All E + 1 logits equal: S = {null, expert 1} with weights 1/2, so FFN = f_1 / 2."""
    c = moe_case(8, 128, 64, 3, seed=5)
    c["z"][:] = 0.25
    x, z, wg, wu, wd = _np(c)
    y, sel, wt = oracle.moe_ffn(x, z, wg, wu, wd, 2)
    assert np.all(sel == [0, 1]) and np.allclose(wt, 0.5)
    c1 = dict(c)
    c1["z"] = c["z"].clone()
    c1["z"][:, 1] = 10.0                              # expert 1 alone (k = 1): weight 1
    y1, sel1, _ = oracle.moe_ffn(x, c1["z"].numpy(), wg, wu, wd, 1)
    assert np.all(sel1[:, 0] == 1)
    np.testing.assert_allclose(y, 0.5 * y1, rtol=1e-13, atol=0)


def test_expert_order_does_not_matter():
    c = moe_case(40, 128, 64, 5, seed=6)
    x, z, wg, wu, wd = _np(c)
    y, _, _ = oracle.moe_ffn(x, z, wg, wu, wd, 2)
    perm = np.array([3, 0, 4, 2, 1])                  # new expert i is old expert perm[i]
    z2 = np.concatenate([z[:, :1], z[:, 1:][:, perm]], axis=1)
    y2, _, _ = oracle.moe_ffn(x, z2, wg[perm], wu[perm], wd[perm], 2)
    np.testing.assert_allclose(y2, y, rtol=1e-12, atol=1e-14)


def test_given_selection_reweights_over_that_set():
    """sel = the gate's own choice reproduces the default result; a single forced expert (k = 1)
    gets weight 1, so the output is that expert's f_j(Norm(x)) alone, and a forced pair is the
    p-weighted mean of the two single-expert outputs."""
    c = moe_case(20, 128, 64, 4, seed=8)
    x, z, wg, wu, wd = _np(c)
    y, sel, wt = oracle.moe_ffn(x, z, wg, wu, wd, 2)
    y_same, _, wt_same = oracle.moe_ffn(x, z, wg, wu, wd, 2, sel=sel)
    assert np.array_equal(y_same, y) and np.array_equal(wt_same, wt)
    ys = {e: oracle.moe_ffn(x, z, wg, wu, wd, 1, sel=np.full((20, 1), e))[0] for e in (2, 4)}
    yt, _ = _torch_ffn(dict(c, z=torch.full_like(c["z"], -30.0).index_fill_(1, torch.tensor([2]), 0.0)), 1)
    np.testing.assert_allclose(ys[2], yt, rtol=1e-9, atol=1e-12)
    pair, _, wpair = oracle.moe_ffn(x, z, wg, wu, wd, 2, sel=np.tile([2, 4], (20, 1)))
    z64 = z.astype(np.float64)
    p = np.exp(z64 - z64.max(axis=1, keepdims=True))
    w2 = p[:, 2] / (p[:, 2] + p[:, 4])
    np.testing.assert_allclose(wpair[:, 0], w2, rtol=1e-12)
    np.testing.assert_allclose(pair, w2[:, None] * ys[2] + (1 - w2)[:, None] * ys[4], rtol=1e-10, atol=1e-13)
