"""GPU parity of the Eq. (4) write path: codes, scales and zeros exported from the paged cache
must equal the oracle's bit for bit (fp32 divide, round half to even, fixed op order)."""

import numpy as np
import pytest
import torch

from tests.gpu_helpers import check_codes, export_layer, say
from workloads import CONFIGS, layer_inputs, random_case

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def tr():
    import mixed_precision_kv_tr_amd as tr
    return tr


def write_case(tr, case, page_code_bytes=0, pieces=None):
    k, v, bits = case["k"], case["v"], case["bits"]
    B, T, H, D = k.shape
    cache = tr.tr_kv_cache_alloc(1, B, H, D, T, page_code_bytes=page_code_bytes)
    cuts = [0] + (pieces or []) + [T]
    for a, b in zip(cuts[:-1], cuts[1:]):
        tr.tr_kv_quantize_write(cache, 0, k[:, a:b].contiguous(), v[:, a:b].contiguous(),
                                bits[:, a:b].contiguous())
    assert tr.tr_kv_cache_status(cache) == 0
    return cache


@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("pieces", [None, [1, 100, 101, 300]])
def test_random_widths_bit_exact(tr, D, pieces):
    say(f"quantize bit-exact D={D} pieces={pieces}")
    case = random_case(3, 333, 5, D, window=8, bit_weights={2: 0.3, 4: 0.3, 8: 0.2, 16: 0.2},
                       mode_weights={"full": 1.0}, seed=D + (0 if pieces is None else 1), device="cuda")
    cache = write_case(tr, case, pieces=pieces)
    exp = export_layer(tr, cache, 0, 0, 333, 3, 5, D)
    check_codes(exp, case["k"], case["v"], case["bits"], where=f"D={D}")
    cache.close()


@pytest.mark.parametrize("cid", [0, 1])
def test_small_configs_bit_exact(tr, cid):
    cfg = CONFIGS[cid]
    say(f"quantize bit-exact config {cid} ({cfg.name})")
    case = layer_inputs(cfg, 0, device="cuda")
    cache = write_case(tr, case)
    B, T, H, D = case["k"].shape
    exp = export_layer(tr, cache, 0, 0, T, B, H, D)
    check_codes(exp, case["k"], case["v"], case["bits"], where=cfg.name)
    cache.close()


def test_config2_layer_bit_exact(tr):
    cfg = CONFIGS[2]
    say("quantize bit-exact config 2, one layer, all 4 sequences")
    case = layer_inputs(cfg, 3, device="cuda")
    cache = write_case(tr, case)
    B, T, H, D = case["k"].shape
    exp = export_layer(tr, cache, 0, 0, T, B, H, D)
    check_codes(exp, case["k"], case["v"], case["bits"], where=cfg.name)
    cache.close()


def test_config3_full_size_sampled(tr):
    cfg = CONFIGS[3]
    say("quantize bit-exact config 3 full size (B=32, C+1=8193, H=16, D=128), sampled sequences")
    case = layer_inputs(cfg, 0, device="cuda")
    cache = write_case(tr, case)
    B, T, H, D = case["k"].shape
    exp = export_layer(tr, cache, 0, 0, T, B, H, D)
    check_codes(exp, case["k"], case["v"], case["bits"], seqs=[0, 17, 31], where=cfg.name)
    cache.close()


def test_config4_clustered_full_size(tr):
    cfg = CONFIGS[4]
    say("quantize bit-exact config 4 full size (C+1=65537, clustered widths)")
    case = layer_inputs(cfg, 0, device="cuda")
    cache = write_case(tr, case)
    B, T, H, D = case["k"].shape
    # export a window straddling many width runs and the tail
    for tok0, n in ((0, 4096), (T - 3000, 3000)):
        exp = export_layer(tr, cache, 0, tok0, n, B, H, D)
        sub = {x: case[x][:, tok0:tok0 + n] for x in ("k", "v", "bits")}
        check_codes(exp, sub["k"], sub["v"], sub["bits"], where=f"{cfg.name} [{tok0},{tok0 + n})")
    cache.close()


def adversarial_groups(D):
    """bf16 patterns of groups that stress the quantizer's edge cases."""
    f = lambda vals: (np.asarray(vals, dtype=np.float32).view(np.uint32) >> 16).astype(np.uint16)
    rng = np.random.default_rng(5)
    rows = []
    rows.append(f([1.25] * D))                                         # constant -> s = 0
    rows.append(np.array([0x0000, 0x8000] * (D // 2), dtype=np.uint16))  # +0 / -0 mix
    rows.append(np.array([0x8000] * D, dtype=np.uint16))               # all -0
    ties = [0.0, 0.5, 1.5, 3.0] * (D // 4)                             # b = 2 ties
    rows.append(f(ties))
    ties8 = ([0.0, 255.0, 127.5, 126.5] * (D // 4))
    rows.append(f(ties8))
    rows.append(np.array(([0x0001, 0x0003, 0x007F, 0x8002] * D)[:D], dtype=np.uint16))  # subnormal bf16
    rows.append(np.array(([0x7149, 0xF149, 0x6FF2, 0x0000] * D)[:D], dtype=np.uint16))  # ~1e30
    wide = rng.normal(size=D).astype(np.float32) * np.float32(10.0) ** rng.integers(-20, 20, size=D).astype(np.float32)
    rows.append((wide.view(np.uint32) >> 16).astype(np.uint16))        # wide exponent spread
    one_ulp = np.array(([0x3F80, 0x3F81] * D)[:D], dtype=np.uint16)
    rows.append(one_ulp)
    return np.stack(rows)


@pytest.mark.parametrize("D", [64, 128])
def test_adversarial_groups_every_width(tr, D):
    say(f"quantize adversarial groups D={D}")
    groups = adversarial_groups(D)                                     # [G, D]
    G = groups.shape[0]
    widths = [2, 4, 8, 16]
    # tokens = G * 4 (each group at every width); one head; K and V get the same group
    kk = np.repeat(groups, len(widths), axis=0)[:, None, :]            # [T, 1, D]
    bits = np.tile(np.array(widths, dtype=np.uint8), G)
    T = kk.shape[0]
    k = torch.from_numpy(kk.view(np.int16).copy()).view(torch.bfloat16)[None].cuda()
    v = torch.from_numpy(kk[::-1].view(np.int16).copy()).view(torch.bfloat16)[None].cuda()
    b = torch.from_numpy(bits)[None].cuda()
    cache = write_case(tr, {"k": k, "v": v, "bits": b})
    exp = export_layer(tr, cache, 0, 0, T, 1, 1, D)
    check_codes(exp, k, v, b, where=f"adversarial D={D}")
    cache.close()


def test_page_size_does_not_change_contents(tr):
    say("quantize page-size invariance")
    case = random_case(2, 700, 3, 64, window=8, bit_weights={2: 0.25, 4: 0.25, 8: 0.25, 16: 0.25},
                       mode_weights={"full": 1.0}, seed=9, device="cuda")
    outs = []
    for pcb in (1024, 4096, 16384):
        cache = write_case(tr, case, page_code_bytes=pcb)
        outs.append(export_layer(tr, cache, 0, 0, 700, 2, 3, 64))
        cache.close()
    for o in outs[1:]:
        for a, b in zip(outs[0], o):
            assert np.array_equal(a, b)


def test_bad_width_sets_sticky_flag(tr):
    say("quantize bad width value -> TR_ERR_BAD_VALUE")
    case = random_case(1, 16, 2, 64, window=4, bit_weights={4: 1.0}, mode_weights={"full": 1.0}, device="cuda")
    case["bits"][0, 5] = 3
    cache = tr.tr_kv_cache_alloc(1, 1, 2, 64, 16)
    tr.tr_kv_quantize_write(cache, 0, case["k"], case["v"], case["bits"])
    assert tr.tr_kv_cache_status(cache) == 6
    cache.close()


def test_pool_exhaustion_is_reported(tr):
    say("quantize tiny pool -> TR_ERR_OUT_OF_PAGES")
    case = random_case(2, 600, 2, 64, window=4, bit_weights={16: 1.0}, mode_weights={"full": 1.0}, device="cuda")
    cache = tr.tr_kv_cache_alloc(1, 2, 2, 64, 600, page_code_bytes=1024, pool_pages=3)
    tr.tr_kv_quantize_write(cache, 0, case["k"], case["v"], case["bits"])
    assert tr.tr_kv_cache_status(cache) == 3
    cache.close()


def test_capacity_is_checked_on_the_host(tr):
    case = random_case(1, 10, 1, 64, window=4, bit_weights={8: 1.0}, mode_weights={"full": 1.0}, device="cuda")
    cache = tr.tr_kv_cache_alloc(1, 1, 1, 64, 8)
    with pytest.raises(tr.TriRouteError) as err:
        tr.tr_kv_quantize_write(cache, 0, case["k"], case["v"], case["bits"])
    assert err.value.status == 2
    assert tr.tr_kv_cache_length(cache, 0) == 0
    cache.close()


@pytest.mark.parametrize("D", [64, 128])
def test_prefill_write_bit_exact(tr, D):
    """The prefill call quantizes its own K/V (fused with staging them for its attention): the
    stored codes, scales and zeros must be the write path's, also for chunks that start inside a
    32-position tile."""
    say(f"prefill quantize-on-write bit-exact D={D}")
    B, T, H = 2, 333, 3
    case = random_case(B, T, H, D, window=8, bit_weights={2: 0.3, 4: 0.3, 8: 0.2, 16: 0.2},
                       mode_weights={"full": 0.5, "local": 0.3, "skip": 0.2}, seed=40 + D, device="cuda")
    cache = tr.tr_kv_cache_alloc(1, B, H, D, T)
    cuts = [0, 70, 97, 200, T]
    for a, b in zip(cuts[:-1], cuts[1:]):
        sl = lambda x: case[x][:, a:b].contiguous()
        out = torch.empty((B, b - a, H, D), dtype=torch.bfloat16, device="cuda")
        tr.tr_routed_attn_prefill(cache, 0, sl("q"), sl("k"), sl("v"), sl("bits"), sl("mode"), b - a, 8, out)
    assert tr.tr_kv_cache_status(cache) == 0
    exp = export_layer(tr, cache, 0, 0, T, B, H, D)
    check_codes(exp, case["k"], case["v"], case["bits"], where=f"prefill D={D}")
    cache.close()
