"""Pins of the routing-controller oracle (Eq. (5), Eq. (11), hard argmax at inference) against
library routines, closed forms and invariants."""

import numpy as np
import pytest
import torch
import torch.nn.functional as F

import oracle
from workloads import controller_case


def _np_case(c):
    u16 = lambda t: t.view(torch.int16).numpy().view(np.uint16)
    w = {k: (u16(v) if v.dtype == torch.bfloat16 else v.numpy()) for k, v in c["w"].items()}
    return u16(c["x"]), c["side"].numpy(), w


def test_logits_match_torch_functional_layers():
    """Eq. (5) written with torch's own rms_norm / linear / silu on the concatenated input
    [Norm(x); psi] (float64), against the oracle's separate numpy products."""
    c = controller_case(40, 192, 5, d_side=6, seed=3)
    x, side, w = _np_case(c)
    xd = c["x"].double()
    inp = torch.cat([F.rms_norm(xd, (xd.shape[1],), eps=1e-6), c["side"].double()], dim=1)
    w1 = torch.cat([c["w"]["w1"].double(), c["w"]["w1_side"].double()], dim=1)
    h = F.linear(F.silu(F.linear(inp, w1, c["w"]["b1"].double())), c["w"]["w2"].double().T,
                 c["w"]["b2"].double())
    hh = F.rms_norm(h, (h.shape[1],), eps=1e-6)
    za = F.linear((hh - c["w"]["mu_a"].double()) / (c["w"]["sigma_a"].double() + 1e-5), c["w"]["w_a"].double().T)
    zb = F.linear((hh - c["w"]["mu_b"].double()) / (c["w"]["sigma_b"].double() + 1e-5), c["w"]["w_b"].double().T)
    oza, ozb = oracle.controller_logits(x, side, w)
    np.testing.assert_allclose(oza.reshape(40, -1), za.numpy(), rtol=1e-10, atol=1e-10)
    np.testing.assert_allclose(ozb, zb.numpy(), rtol=1e-10, atol=1e-10)


def _constructed(M=6, d=64, H=5, d_r=128):
    """Weights whose decisions are known in closed form: the trunk ignores x (w1 = 0) and maps
    every token to the same vector hh; head h's column for its target mode is +hh and the other
    two are -hh, so z = +-sum(hh^2) and the target wins by 2 * d_r."""
    rng = np.random.default_rng(0)
    x = rng.standard_normal((M, d)).astype(np.float32)
    xb = (x.view(np.uint32) >> 16).astype(np.uint16)
    b1 = rng.uniform(8.0, 12.0, d_r)
    w = {"w1": np.zeros((d_r, d), np.uint16), "w1_side": np.zeros((d_r, 0), np.float32), "b1": b1,
         "w2": np.eye(d_r), "b2": np.zeros(d_r), "mu_a": np.zeros(d_r), "sigma_a": np.ones(d_r),
         "mu_b": np.zeros(d_r), "sigma_b": np.ones(d_r)}
    h = b1 / (1 + np.exp(-b1))
    hh = h / np.sqrt(np.mean(h * h) + 1e-6)
    target = np.array([(2 * h + 1) % 3 for h in range(H)])
    wa = np.zeros((d_r, 3 * H))
    for h in range(H):
        for j in range(3):
            wa[:, 3 * h + j] = hh if j == target[h] else -hh
    wb = np.stack([-hh, -hh, hh, -hh], axis=1)               # width 8
    w["w_a"], w["w_b"] = wa, wb
    return xb, np.zeros((M, 0), np.float32), w, target


def test_constructed_decisions_head_layout_and_width_table():
    xb, side, w, target = _constructed()
    mode, bits, za, zb = oracle.controller_route(xb, side, w)
    assert np.array_equal(mode, np.broadcast_to(target, mode.shape))
    assert np.all(bits == 8)
    # the winning margin in closed form: z = +-sum(hh^2) / (1 + eps_w), with
    # sum(hh^2) = d_r * m / (m + eps), m = mean(silu(b1)^2)
    h = w["b1"] / (1 + np.exp(-w["b1"]))
    m = np.mean(h * h)
    margin = 2 * 128 * m / (m + 1e-6) / (1 + 1e-5)
    top2 = np.sort(za, axis=2)
    assert np.allclose(top2[..., 2] - top2[..., 1], margin, rtol=1e-12)


def test_ties_go_to_the_lowest_index():
    xb, side, w, _ = _constructed()
    w["w_a"] = np.zeros_like(w["w_a"])
    w["w_b"] = np.zeros_like(w["w_b"])
    mode, bits, _, _ = oracle.controller_route(xb, side, w)
    assert np.all(mode == oracle.MODE_SKIP) and np.all(bits == 2)


def test_rms_norm_makes_decisions_scale_free():
    """Norm(x) removes the scale of the residual state: x and 4x (exact in bf16) give the same
    logits up to the eps term."""
    c = controller_case(50, 256, 4, seed=5)
    x, side, w = _np_case(c)
    x4 = ((c["x"].float() * 4).to(torch.bfloat16)).view(torch.int16).numpy().view(np.uint16)
    za, zb = oracle.controller_logits(x, side, w)
    za4, zb4 = oracle.controller_logits(x4, side, w)
    np.testing.assert_allclose(za4, za, rtol=1e-5, atol=1e-5)
    np.testing.assert_allclose(zb4, zb, rtol=1e-5, atol=1e-5)


@pytest.mark.parametrize("axis", ["a", "b"])
def test_whitening_statistics_are_per_axis(axis):
    """Eq. (11): moving one axis's mean changes only that axis's logits."""
    c = controller_case(30, 128, 3, seed=9)
    x, side, w = _np_case(c)
    za, zb = oracle.controller_logits(x, side, w)
    w2 = dict(w)
    w2["mu_" + axis] = w["mu_" + axis] + 0.5
    za2, zb2 = oracle.controller_logits(x, side, w2)
    untouched, moved = ((zb, zb2), (za, za2)) if axis == "a" else ((za, za2), (zb, zb2))
    assert np.array_equal(untouched[0], untouched[1])
    assert not np.allclose(moved[0], moved[1])
