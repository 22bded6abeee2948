"""Deterministic, seeded generation of the synthetic inputs (torch, on any device).

Each tensor comes from its own torch.Generator seeded from (seed, workload, layer, stream),
so a tensor can be regenerated alone.  Values for a given seed depend on the device type
(CPU and GPU generators differ); consumers that compare the GPU path with the oracle hand
the oracle the very tensors the GPU received (copied to the host).
"""

from __future__ import annotations

import torch

from .configs import WorkloadConfig

MODE_CODES = {"skip": 0, "local": 1, "full": 2}
_STREAMS = {"q": 0, "k": 1, "v": 2, "kscale": 3, "bits": 4, "mode": 5, "runs": 6,
            "ctl_x": 7, "ctl_side": 8, "ctl_w": 9, "moe_x": 10, "moe_z": 11, "moe_w": 12}


def _gen(device, seed: int, cid: int, layer: int, stream: str) -> torch.Generator:
    g = torch.Generator(device=device)
    mixed = (int(seed) * 1_000_003 + int(cid) * 10_007 + int(layer) * 101 + _STREAMS[stream]) % (2**63 - 1)
    g.manual_seed(mixed)
    return g


def _categorical(weights: dict, shape, gen, device, values=None) -> torch.Tensor:
    keys = list(weights.keys())
    probs = torch.tensor([float(weights[k]) for k in keys], dtype=torch.float64)
    cdf = torch.cumsum(probs / probs.sum(), 0).to(torch.float32)
    cdf[-1] = 2.0                                     # u < 1 always lands in the last bucket
    vals = torch.tensor(values if values is not None else keys, dtype=torch.uint8)
    u = torch.rand(shape, generator=gen, device=device, dtype=torch.float32)
    idx = torch.searchsorted(cdf.to(device), u.reshape(-1), right=True).reshape(shape)
    return vals.to(device)[idx]


def _bits(batch: int, positions: int, weights: dict, clustered: bool, gen, gen_runs, device):
    if not clustered:
        return _categorical(weights, (batch, positions), gen, device)
    # Runs of geometric(p = 1/16) length on {1, 2, ...} (mean 16); each run's b drawn iid.
    p = 1.0 / 16.0
    rows = []
    for _ in range(batch):
        total, lens = 0, []
        while total < positions:
            n = max(64, (positions - total) // 8)
            u = torch.rand(n, generator=gen_runs, device=device, dtype=torch.float64)
            ln = torch.floor(torch.log1p(-u) / torch.log1p(torch.tensor(-p, dtype=torch.float64))) + 1
            ln = ln.clamp(min=1).to(torch.int64)
            lens.append(ln)
            total += int(ln.sum())
        ln = torch.cat(lens)
        vals = _categorical(weights, (ln.numel(),), gen, device)
        rows.append(torch.repeat_interleave(vals, ln)[:positions])
    return torch.stack(rows)


def _normal_bf16(shape, gen, device, scale=None) -> torch.Tensor:
    x = torch.randn(shape, generator=gen, device=device, dtype=torch.float32)
    if scale is not None:
        x.mul_(scale)
    return x.to(torch.bfloat16)


def random_case(batch: int, tokens: int, heads: int, head_dim: int, *, window: int,
                bit_weights: dict, mode_weights: dict, seed: int = 0, device="cpu",
                clustered_bits: bool = False, n_queries: int | None = None,
                layer: int = 0, cid: int = 99, kv_heads: int | None = None) -> dict:
    """One layer of inputs for `batch` sequences of `tokens` positions.

    Returns bf16 q [B, Tq, H, D] (Tq = tokens, or n_queries trailing positions), bf16 k, v
    [B, tokens, Hkv, D] (Hkv = kv_heads, default H; grouped-query attention when smaller),
    uint8 bits [B, tokens] (values 2/4/8/16) and uint8 mode [B, Tq, H] (0 skip, 1 local, 2 full).
    """
    dev = torch.device(device)
    Tq = tokens if n_queries is None else int(n_queries)
    hkv = heads if kv_heads is None else int(kv_heads)
    g_scale = _gen(dev, seed, cid, layer, "kscale")
    kscale = torch.exp(0.5 * torch.randn((hkv, head_dim), generator=g_scale, device=dev,
                                         dtype=torch.float32))
    k = _normal_bf16((batch, tokens, hkv, head_dim), _gen(dev, seed, cid, layer, "k"), dev, kscale)
    v = _normal_bf16((batch, tokens, hkv, head_dim), _gen(dev, seed, cid, layer, "v"), dev)
    q = _normal_bf16((batch, Tq, heads, head_dim), _gen(dev, seed, cid, layer, "q"), dev)
    bits = _bits(batch, tokens, bit_weights, clustered_bits, _gen(dev, seed, cid, layer, "bits"),
                 _gen(dev, seed, cid, layer, "runs"), dev)
    mode = _categorical(mode_weights, (batch, Tq, heads), _gen(dev, seed, cid, layer, "mode"), dev,
                        values=[MODE_CODES[m] for m in mode_weights])
    return {"q": q, "k": k, "v": v, "bits": bits, "mode": mode}


def layer_inputs(cfg: WorkloadConfig, layer: int, seed: int = 1234, device="cpu") -> dict:
    """Inputs of one layer of a workload.

    prefill: q [B, T, H, D]; k, v [B, T, Hkv, D]; bits [B, T]; mode [B, T, H]; queries at
             positions 0..T-1.
    decode:  k, v [B, C+1, Hkv, D] (positions 0..C; the new token is position C); bits [B, C+1];
             q [B, H, D] and mode [B, H] for the one query at position C.
    (H = cfg.heads query heads, Hkv = cfg.num_kv_heads.)
    """
    if cfg.kind == "prefill":
        return random_case(cfg.batch, cfg.tokens, cfg.heads, cfg.head_dim, window=cfg.window,
                           bit_weights=cfg.bit_weights, mode_weights=cfg.mode_weights, seed=seed,
                           device=device, clustered_bits=cfg.clustered_bits, layer=layer, cid=cfg.cid,
                           kv_heads=cfg.num_kv_heads)
    case = random_case(cfg.batch, cfg.tokens + 1, cfg.heads, cfg.head_dim, window=cfg.window,
                       bit_weights=cfg.bit_weights, mode_weights=cfg.mode_weights, seed=seed,
                       device=device, clustered_bits=cfg.clustered_bits, n_queries=1,
                       layer=layer, cid=cfg.cid, kv_heads=cfg.num_kv_heads)
    case["q"] = case["q"][:, 0]
    case["mode"] = case["mode"][:, 0]
    return case


def controller_case(tokens: int, d: int, heads: int, *, d_side: int = 8, d_r: int = 128, seed: int = 0,
                    device="cpu", layer: int = 0, cid: int = 99) -> dict:
    """Inputs of the routing controller for one layer: residual states x (bf16 [tokens, d], N(0, 1)
    with a few channels scaled up 8x, as residual streams carry outlier channels), side features
    (float32 [tokens, d_side], N(0, 1)) and random weights at the usual 1/sqrt(fan_in) scale:

        w1 bf16 [d_r][d], w1_side [d_r][d_side], b1, w2 [d_r][d_r] (in x out), b2,
        mu_a, sigma_a, mu_b, sigma_b [d_r], w_a [d_r][3 heads] (in x out), w_b [d_r][4].

    The head weights get a 3x gain so that the decisions are not near-uniform ties.  No trained
    weights exist for the pages' controller; these only give the kernel realistic shapes."""
    dev = torch.device(device)
    gx = _gen(dev, seed, cid, layer, "ctl_x")
    x = torch.randn((tokens, d), generator=gx, device=dev, dtype=torch.float32)
    x[:, : max(1, d // 64)] *= 8.0
    side = torch.randn((tokens, d_side), generator=_gen(dev, seed, cid, layer, "ctl_side"), device=dev,
                       dtype=torch.float32)
    gw = _gen(dev, seed, cid, layer, "ctl_w")
    rn = lambda *shape: torch.randn(shape, generator=gw, device=dev, dtype=torch.float32)
    w = {
        "w1": (rn(d_r, d) / d ** 0.5).to(torch.bfloat16),
        "w1_side": rn(d_r, d_side) / max(1, d_side) ** 0.5,
        "b1": 0.1 * rn(d_r),
        "w2": rn(d_r, d_r) / d_r ** 0.5,
        "b2": 0.1 * rn(d_r),
        "mu_a": 0.1 * rn(d_r),
        "sigma_a": 0.5 + torch.rand((d_r,), generator=gw, device=dev, dtype=torch.float32),
        "mu_b": 0.1 * rn(d_r),
        "sigma_b": 0.5 + torch.rand((d_r,), generator=gw, device=dev, dtype=torch.float32),
        "w_a": 3.0 * rn(d_r, 3 * heads) / d_r ** 0.5,
        "w_b": 3.0 * rn(d_r, 4) / d_r ** 0.5,
    }
    return {"x": x.to(torch.bfloat16), "side": side, "w": w}


def moe_case(tokens: int, d: int, d_e: int, experts: int, *, seed: int = 0, device="cpu", layer: int = 0,
             cid: int = 99, null_bias: float = 0.0) -> dict:
    """Inputs of the expert FFN for one layer: x (bf16 [tokens, d], N(0, 1) with a few 8x channels),
    gate logits z (float32 [tokens, experts + 1], N(0, 1); index 0 is the null expert, shifted by
    null_bias), and random bf16 weights w_gate, w_up [E][d_e][d] at 1/sqrt(d) and w_down [E][d][d_e]
    at 1/sqrt(d_e).  No trained weights exist; these only give the kernels realistic shapes."""
    dev = torch.device(device)
    x = torch.randn((tokens, d), generator=_gen(dev, seed, cid, layer, "moe_x"), device=dev, dtype=torch.float32)
    x[:, : max(1, d // 64)] *= 8.0
    z = torch.randn((tokens, experts + 1), generator=_gen(dev, seed, cid, layer, "moe_z"), device=dev,
                    dtype=torch.float32)
    z[:, 0] += null_bias
    gw = _gen(dev, seed, cid, layer, "moe_w")
    rn = lambda *shape: torch.randn(shape, generator=gw, device=dev, dtype=torch.float32)
    return {"x": x.to(torch.bfloat16), "z": z,
            "w_gate": (rn(experts, d_e, d) / d ** 0.5).to(torch.bfloat16),
            "w_up": (rn(experts, d_e, d) / d ** 0.5).to(torch.bfloat16),
            "w_down": (rn(experts, d, d_e) / d_e ** 0.5).to(torch.bfloat16)}
