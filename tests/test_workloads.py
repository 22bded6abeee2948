"""The seeded input generator: shapes, determinism and the stated distributions."""

import numpy as np
import torch

from workloads import CONFIGS, layer_inputs, random_case


def test_prefill_config_shapes_and_determinism():
    cfg = CONFIGS[0]
    a = layer_inputs(cfg, 0, seed=5)
    b = layer_inputs(cfg, 0, seed=5)
    c = layer_inputs(cfg, 0, seed=6)
    assert a["q"].shape == (1, 256, 4, 64) and a["q"].dtype == torch.bfloat16
    assert a["k"].shape == a["v"].shape == (1, 256, 4, 64)
    assert a["bits"].shape == (1, 256) and a["bits"].dtype == torch.uint8
    assert a["mode"].shape == (1, 256, 4) and a["mode"].dtype == torch.uint8
    for key in a:
        assert torch.equal(a[key], b[key])
    assert not torch.equal(a["k"], c["k"])


def test_decode_config_shapes():
    cfg = CONFIGS[1]
    d = layer_inputs(cfg, 0)
    assert d["k"].shape == (8, 2049, 12, 64)
    assert d["bits"].shape == (8, 2049)
    assert d["q"].shape == (8, 12, 64) and d["mode"].shape == (8, 12)


def test_category_frequencies():
    case = random_case(4, 20000, 2, 8, window=4, bit_weights={2: 0.3, 4: 0.4, 8: 0.2, 16: 0.1},
                       mode_weights={"skip": 0.2, "local": 0.4, "full": 0.4}, seed=1)
    bits = case["bits"].numpy().ravel()
    for b, p in {2: 0.3, 4: 0.4, 8: 0.2, 16: 0.1}.items():
        assert abs((bits == b).mean() - p) < 0.01
    mode = case["mode"].numpy().ravel()
    for m, p in {0: 0.2, 1: 0.4, 2: 0.4}.items():
        assert abs((mode == m).mean() - p) < 0.01


def test_clustered_runs_have_mean_16():
    case = random_case(2, 65537, 1, 8, window=4, bit_weights={2: 0.6, 4: 0.3, 8: 0.08, 16: 0.02},
                       mode_weights={"local": 0.3, "full": 0.7}, seed=2, clustered_bits=True)
    bits = case["bits"].numpy()
    assert set(np.unique(bits)) <= {2, 4, 8, 16}
    # a run boundary is a change of b or a new run with the same b; changes alone give a
    # lower bound on the number of runs: mean run length between changes must exceed 16
    changes = (bits[:, 1:] != bits[:, :-1]).sum()
    mean_between_changes = bits.size / (changes + bits.shape[0])
    assert 16.0 < mean_between_changes < 40.0
    assert not np.any(case["mode"].numpy() == 0)


def test_key_channel_scales_are_shared_across_tokens():
    case = random_case(2, 4000, 3, 16, window=4, bit_weights={16: 1.0}, mode_weights={"full": 1.0}, seed=3)
    k = case["k"].float().numpy()
    std = k.reshape(-1, 3, 16).std(axis=0)               # per (head, channel)
    assert std.max() / std.min() > 2.0                   # lognormal(0, 0.5) spread
    v = case["v"].float().numpy()
    vstd = v.reshape(-1, 3, 16).std(axis=0)
    assert np.all(np.abs(vstd - 1.0) < 0.05)
