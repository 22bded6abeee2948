"""GPU parity of the routing controller (Eq. (5), Eq. (11), hard argmax) against the oracle.

The decisions are argmaxes of fp32 logits on the GPU and fp64 logits in the oracle.  Where the
oracle's best logit beats the runner-up by more than TAU = 1e-3 * (1 + max |z|) the decision is
unique and must match exactly; inside that margin either near-maximal choice is correct, and
the GPU's choice must be one of them.  (The GPU's logits differ from the exact ones by fp32
accumulation -- first layer: 2^-24 per add over d products, then normalized layers of width
128 -- i.e. by ~1e-5 relative, two orders of magnitude below TAU.)"""

import numpy as np
import pytest
import torch

import oracle
from tests.gpu_helpers import say, u16
from workloads import controller_case

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def tr():
    import mixed_precision_kv_tr_amd as tr
    return tr


def run(tr, c, workspace=True):
    M, H = c["x"].shape[0], c["w"]["w_a"].shape[1] // 3
    mode = torch.full((M, H), 255, dtype=torch.uint8, device="cuda")
    bits = torch.full((M,), 255, dtype=torch.uint8, device="cuda")
    cw = tr.ControllerWeights(c["w"], workspace=workspace)
    tr.tr_controller_route(cw, c["x"], c["side"] if c["side"].shape[1] else None, M, mode, bits)
    torch.cuda.synchronize()
    return mode.cpu().numpy(), bits.cpu().numpy()


def oracle_of(c):
    w = {k: (u16(v) if v.dtype == torch.bfloat16 else v.cpu().numpy()) for k, v in c["w"].items()}
    return oracle.controller_route(u16(c["x"]), c["side"].cpu().numpy(), w)


def check(gmode, gbits, omode, obits, za, zb, where):
    def one(g, o, z, name):
        zmax = z.max(axis=-1)
        tau = 1e-3 * (1 + np.abs(z).max(axis=-1))
        top2 = np.sort(z, axis=-1)
        unique = top2[..., -1] - top2[..., -2] > tau
        assert np.array_equal(g[unique], o[unique]), f"{where}: {name} differs where the argmax is unique"
        zg = np.take_along_axis(z, g[..., None].astype(np.int64), axis=-1)[..., 0]
        assert np.all(zg >= zmax - tau), f"{where}: {name} picked a clearly smaller logit"
        return int((~unique).sum())
    ties_a = one(gmode, omode, za, "mode")
    gidx = np.log2(gbits.astype(np.float64)).astype(np.int64) - 1
    oidx = np.log2(obits.astype(np.float64)).astype(np.int64) - 1
    assert set(np.unique(gbits)) <= {2, 4, 8, 16}
    ties_b = one(gidx, oidx, zb, "bits")
    say(f"  {where}: {gmode.size} modes, {gbits.size} widths, near-ties {ties_a} / {ties_b}, "
        f"exact matches {np.mean(gmode == omode):.5f} / {np.mean(gbits == obits):.5f}")


@pytest.mark.parametrize("M,d,H,d_side", [(1000, 768, 12, 8), (32, 2048, 16, 0), (77, 64, 1, 3),
                                          (333, 4096, 64, 32), (1, 64, 2, 1), (40, 192, 3, 2)])
def test_controller_matches_oracle(tr, M, d, H, d_side):
    say(f"controller M={M} d={d} H={H} d_side={d_side}")
    c = controller_case(M, d, H, d_side=d_side, seed=M + d, device="cuda")
    gmode, gbits = run(tr, c)
    omode, obits, za, zb = oracle_of(c)
    check(gmode, gbits, omode, obits, za, zb, f"M={M} d={d} H={H}")


@pytest.mark.parametrize("M,d,H,d_side", [(1, 2048, 16, 8), (31, 768, 12, 8), (33, 320, 5, 1), (256, 4096, 64, 32),
                                          (257, 2048, 16, 8), (200, 16384, 7, 0)])
def test_controller_split_and_single_workgroup_forms(tr, M, d, H, d_side):
    """Up to 256 tokens the call spreads the first layer over channel slices (the workspace
    form); with no workspace, or beyond 256 tokens, one workgroup takes 32 tokens.  Both forms
    against the oracle, on the same inputs: ragged token blocks, a channel slice of fewer than
    4 groups (d = 320), the most heads and side features, the widest model."""
    say(f"controller forms M={M} d={d} H={H} d_side={d_side}")
    c = controller_case(M, d, H, d_side=d_side, seed=3 * M + d, device="cuda")
    omode, obits, za, zb = oracle_of(c)
    for ws in (True, False):
        gmode, gbits = run(tr, c, workspace=ws)
        check(gmode, gbits, omode, obits, za, zb, f"M={M} d={d} H={H} workspace={ws}")


def test_controller_workspace_reuse_across_calls(tr):
    """One workspace serves calls of different sizes in a row (nothing carried over).  The cases
    share the seed, so their weights are the same and one ControllerWeights serves all three."""
    cw = None
    for M in (256, 3, 100):
        c = controller_case(M, 2048, 16, d_side=8, seed=11, device="cuda")
        if cw is None:
            cw = tr.ControllerWeights(c["w"])
        assert torch.equal(cw.tensors["w2"], c["w"]["w2"]) and torch.equal(cw.tensors["w_a"], c["w"]["w_a"])
        H = 16
        mode = torch.full((M, H), 255, dtype=torch.uint8, device="cuda")
        bits = torch.full((M,), 255, dtype=torch.uint8, device="cuda")
        tr.tr_controller_route(cw, c["x"], c["side"], M, mode, bits)
        torch.cuda.synchronize()
        omode, obits, za, zb = oracle_of(c)
        check(mode.cpu().numpy(), bits.cpu().numpy(), omode, obits, za, zb, f"reuse M={M}")


def test_controller_graph_replays_match_eager(tr):
    """The decode-step call (split form, 32 tokens) and a 300-token call (one-workgroup form)
    captured in a HIP graph: every replay, with eager work and synchronizations in between,
    writes exactly the eager decisions."""
    for M in (32, 300):
        c = controller_case(M, 2048, 16, d_side=8, seed=5, device="cuda")
        cw = tr.ControllerWeights(c["w"])
        mode = torch.full((M, 16), 255, dtype=torch.uint8, device="cuda")
        bits = torch.full((M,), 255, dtype=torch.uint8, device="cuda")
        tr.tr_controller_route(cw, c["x"], c["side"], M, mode, bits)
        torch.cuda.synchronize()
        emode, ebits = mode.clone(), bits.clone()
        s = torch.cuda.Stream()
        with torch.cuda.stream(s):
            tr.tr_controller_route(cw, c["x"], c["side"], M, mode, bits, s.cuda_stream)
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            tr.tr_controller_route(cw, c["x"], c["side"], M, mode, bits, torch.cuda.current_stream().cuda_stream)
        for rep in range(4):
            mode.fill_(255)
            bits.fill_(255)
            torch.cuda.synchronize()
            g.replay()
            torch.cuda.synchronize()
            assert torch.equal(mode, emode) and torch.equal(bits, ebits), f"M={M} replay {rep}"
            tr.tr_controller_route(cw, c["x"], c["side"], M, mode, bits)   # eager work in between
            torch.cuda.synchronize()


def test_controller_full_size_prefill_layer(tr):
    """One 160M-shaped prefill layer's tokens (4 x 2048, d = 768, 12 heads) and one 1.3B decode
    step (32 tokens, d = 2048, 16 heads)."""
    for M, d, H in ((8192, 768, 12), (32, 2048, 16)):
        say(f"controller full size M={M} d={d} H={H}")
        c = controller_case(M, d, H, d_side=8, seed=7, device="cuda", cid=2)
        gmode, gbits = run(tr, c)
        omode, obits, za, zb = oracle_of(c)
        check(gmode, gbits, omode, obits, za, zb, f"M={M} d={d} H={H}")


def test_controller_closed_form_decisions(tr):
    """The trunk ignores x (w1 = 0), every token maps to the same vector, and head h's target
    mode wins by 2 * d_r: the decisions are known exactly."""
    d_r, H, M, d = 128, 5, 70, 64
    b1 = torch.linspace(8.0, 12.0, d_r, dtype=torch.float64)
    h = b1 / (1 + torch.exp(-b1))
    hh = h / torch.sqrt((h * h).mean() + 1e-6)
    target = [(2 * i + 1) % 3 for i in range(H)]
    wa = torch.stack([hh if j == target[i] else -hh for i in range(H) for j in range(3)], dim=1)
    wb = torch.stack([-hh, -hh, hh, -hh], dim=1)
    f = lambda t: t.to(torch.float32).cuda().contiguous()
    w = {"w1": torch.zeros((d_r, d), dtype=torch.bfloat16, device="cuda"), "w1_side": torch.zeros((d_r, 0), device="cuda"),
         "b1": f(b1), "w2": f(torch.eye(d_r)), "b2": f(torch.zeros(d_r)), "mu_a": f(torch.zeros(d_r)),
         "sigma_a": f(torch.ones(d_r)), "mu_b": f(torch.zeros(d_r)), "sigma_b": f(torch.ones(d_r)),
         "w_a": f(wa), "w_b": f(wb)}
    x = torch.randn((M, d), device="cuda").to(torch.bfloat16)
    gmode, gbits = run(tr, {"x": x, "side": torch.zeros((M, 0), device="cuda"), "w": w})
    assert np.array_equal(gmode, np.broadcast_to(np.array(target, np.uint8), (M, H)))
    assert np.all(gbits == 8)
