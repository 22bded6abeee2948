"""GPU parity of prefill routed attention (Eq. 2 for every prompt query over the cache that
Eq. 4 just wrote): |gpu - oracle| <= 2e-3 + 1e-2 |oracle| element-wise; cache contents
bit-exact."""

import numpy as np
import pytest
import torch

import oracle
from tests.gpu_helpers import bf16_to_f64, check_codes, compare_out, export_layer, say, u16
from workloads import CONFIGS, layer_inputs, random_case

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def tr():
    import mixed_precision_kv_tr_amd as tr
    return tr


def run_prefill(tr, case, window, cuts=None, page_code_bytes=0, layers=1, layer=0):
    """Prefill positions 0..T-1 in one call, or in pieces split at `cuts` (chunked prefill)."""
    q, k, v, bits, mode = (case[x] for x in ("q", "k", "v", "bits", "mode"))
    B, T, H, D = k.shape
    HQ = q.shape[2]
    cache = tr.tr_kv_cache_alloc(layers, B, H, D, T, page_code_bytes=page_code_bytes, num_query_heads=HQ)
    out = torch.full((B, T, HQ, D), float("nan"), dtype=torch.bfloat16, device="cuda")
    edges = [0] + (cuts or []) + [T]
    for a, b in zip(edges[:-1], edges[1:]):
        piece = torch.empty((B, b - a, HQ, D), dtype=torch.bfloat16, device="cuda")
        tr.tr_routed_attn_prefill(cache, layer, q[:, a:b].contiguous(), k[:, a:b].contiguous(),
                                  v[:, a:b].contiguous(), bits[:, a:b].contiguous(), mode[:, a:b].contiguous(),
                                  b - a, window, piece)
        out[:, a:b] = piece
    status = tr.tr_kv_cache_status(cache)
    return cache, out, status


def oracle_prefill(case, window, seqs):
    kb, vb, qb = u16(case["k"]), u16(case["v"]), u16(case["q"])
    bb, mb = case["bits"].cpu().numpy(), case["mode"].cpu().numpy()
    T = kb.shape[1]
    return {s: oracle.attend_cached(qb[s], kb[s], vb[s], bb[s], mb[s], np.arange(T), window)["out"] for s in seqs}


def check(case, out, window, seqs, where):
    got = bf16_to_f64(out)
    refs = oracle_prefill(case, window, seqs)
    for s in seqs:
        compare_out(got[s], refs[s], f"{where} seq {s}")


def test_prefill_config0(tr):
    cfg = CONFIGS[0]
    say(f"prefill {cfg.name}")
    case = layer_inputs(cfg, 0, device="cuda")
    cache, out, status = run_prefill(tr, case, cfg.window)
    assert status == 0
    B, T, H, D = case["k"].shape
    check_codes(export_layer(tr, cache, 0, 0, T, B, H, D), case["k"], case["v"], case["bits"], where=cfg.name)
    cache.close()
    check(case, out, cfg.window, [0], cfg.name)


@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("T", [1, 5, 31, 32, 33, 127, 128, 129, 300])
def test_prefill_ragged(tr, D, T):
    say(f"prefill ragged D={D} T={T}")
    case = random_case(2, T, 3, D, window=11, bit_weights={2: 0.3, 4: 0.3, 8: 0.2, 16: 0.2},
                       mode_weights={"skip": 0.2, "local": 0.4, "full": 0.4}, seed=T * 7 + D, device="cuda")
    cache, out, status = run_prefill(tr, case, 11)
    cache.close()
    assert status == 0
    check(case, out, 11, range(2), f"D={D} T={T}")


@pytest.mark.parametrize("bw", [2, 4, 8, 16])
@pytest.mark.parametrize("window", [0, 3, 1000])
def test_prefill_single_width_windows(tr, bw, window):
    say(f"prefill b={bw} w={window}")
    case = random_case(1, 200, 2, 64, window=window, bit_weights={bw: 1.0},
                       mode_weights={"local": 0.5, "full": 0.5}, seed=bw * 31 + window, device="cuda")
    cache, out, status = run_prefill(tr, case, window)
    cache.close()
    assert status == 0
    check(case, out, window, [0], f"b={bw} w={window}")


def test_prefill_all_skip_zero_and_own_value(tr):
    case = random_case(1, 70, 2, 64, window=0, bit_weights={4: 1.0}, mode_weights={"skip": 1.0},
                       seed=3, device="cuda")
    cache, out, status = run_prefill(tr, case, 0)
    cache.close()
    assert status == 0 and torch.count_nonzero(out.float()) == 0
    case["mode"].fill_(1)                                        # local with w = 0: own v_hat
    cache, out, status = run_prefill(tr, case, 0)
    cache.close()
    check(case, out, 0, [0], "local w=0")


def test_prefill_chunked_matches_oracle(tr):
    say("prefill in three chunks (later queries read earlier chunks)")
    case = random_case(2, 400, 3, 64, window=50, bit_weights={2: 0.3, 4: 0.3, 8: 0.2, 16: 0.2},
                       mode_weights={"skip": 0.1, "local": 0.4, "full": 0.5}, seed=12, device="cuda")
    cache, out, status = run_prefill(tr, case, 50, cuts=[97, 256])
    cache.close()
    assert status == 0
    check(case, out, 50, range(2), "chunked")


def test_prefill_then_decode_agree(tr):
    say("decode after prefill equals the last prefill row")
    B, T, H, D, w = 2, 257, 4, 128, 40
    case = random_case(B, T, H, D, window=w, bit_weights={2: 0.3, 4: 0.4, 8: 0.2, 16: 0.1},
                       mode_weights={"local": 0.5, "full": 0.5}, seed=21, device="cuda")
    _, out_full, _ = run_prefill(tr, case, w)
    cache = tr.tr_kv_cache_alloc(1, B, H, D, T)
    part = torch.empty((B, T - 1, H, D), dtype=torch.bfloat16, device="cuda")
    sl = lambda x, a, b: case[x][:, a:b].contiguous()
    tr.tr_routed_attn_prefill(cache, 0, sl("q", 0, T - 1), sl("k", 0, T - 1), sl("v", 0, T - 1),
                              sl("bits", 0, T - 1), sl("mode", 0, T - 1), T - 1, w, part)
    tr.tr_kv_quantize_write(cache, 0, sl("k", T - 1, T), sl("v", T - 1, T), sl("bits", T - 1, T))
    dec = torch.empty((B, H, D), dtype=torch.bfloat16, device="cuda")
    tr.tr_routed_attn_decode(cache, 0, case["q"][:, T - 1].contiguous(), case["mode"][:, T - 1].contiguous(), w, dec)
    assert tr.tr_kv_cache_status(cache) == 0
    cache.close()
    a, b = bf16_to_f64(out_full[:, T - 1]), bf16_to_f64(dec)
    refs = oracle_prefill(case, w, range(B))
    for s in range(B):
        compare_out(a[s], refs[s][T - 1], f"prefill last row seq {s}")
        compare_out(b[s], refs[s][T - 1], f"decode seq {s}")


def test_prefill_page_size_invariance(tr):
    case = random_case(1, 300, 2, 64, window=30, bit_weights={2: 0.3, 4: 0.3, 8: 0.2, 16: 0.2},
                       mode_weights={"skip": 0.2, "local": 0.4, "full": 0.4}, seed=5, device="cuda")
    outs = []
    for pcb in (1024, 4096, 32768):
        cache, out, _ = run_prefill(tr, case, 30, page_code_bytes=pcb)
        cache.close()
        outs.append(out)
    assert torch.equal(outs[0], outs[1]) and torch.equal(outs[0], outs[2])


def test_prefill_config2_layer_full_size(tr):
    cfg = CONFIGS[2]
    say(f"prefill {cfg.name}, layer 5 of a 12-layer workload, all sequences")
    case = layer_inputs(cfg, 5, device="cuda")
    cache, out, status = run_prefill(tr, case, cfg.window, layers=2, layer=1)
    cache.close()
    assert status == 0
    check(case, out, cfg.window, range(cfg.batch), cfg.name)


def test_prefill_bad_mode_is_flagged(tr):
    case = random_case(1, 40, 2, 64, window=3, bit_weights={4: 1.0}, mode_weights={"full": 1.0},
                       seed=2, device="cuda")
    case["mode"][0, 7, 1] = 5
    cache, out, status = run_prefill(tr, case, 3)
    cache.close()
    assert status == 6
    assert torch.count_nonzero(out[0, 7, 1].float()) == 0


@pytest.mark.parametrize("G", [2, 4])
@pytest.mark.parametrize("D", [64, 128])
def test_prefill_grouped_query_heads(tr, G, D):
    """Grouped-query attention: 8 query heads over 8 / G KV heads (query head h reads KV head
    h // G), in one call and in two chunks; cache contents bit-exact per KV head."""
    say(f"prefill GQA G={G} D={D}")
    case = random_case(2, 333, 8, D, window=25, bit_weights={2: 0.3, 4: 0.3, 8: 0.2, 16: 0.2},
                       mode_weights={"skip": 0.2, "local": 0.4, "full": 0.4}, seed=G * 17 + D,
                       device="cuda", kv_heads=8 // G)
    cache, out, status = run_prefill(tr, case, 25)
    assert status == 0
    B, T, H, _ = case["k"].shape
    check_codes(export_layer(tr, cache, 0, 0, T, B, H, D), case["k"], case["v"], case["bits"], where="GQA")
    cache.close()
    check(case, out, 25, range(2), f"G={G} D={D}")
    cache, out2, status = run_prefill(tr, case, 25, cuts=[130])
    cache.close()
    assert status == 0
    check(case, out2, 25, range(2), f"G={G} D={D} chunked")


def test_prefill_config6_gqa_layer_full_size(tr):
    cfg = CONFIGS[6]
    say(f"prefill {cfg.name}, one layer, all sequences")
    case = layer_inputs(cfg, 3, device="cuda")
    cache, out, status = run_prefill(tr, case, cfg.window)
    cache.close()
    assert status == 0
    check(case, out, cfg.window, range(cfg.batch), cfg.name)


@pytest.mark.parametrize("variant", ["dense_bf16", "uniform_b4", "uniform_b2", "routing_only_bf16"])
def test_prefill_baseline_variants(tr, variant):
    """The comparison configurations the benchmark runs, against the oracle."""
    bw, mw = {"dense_bf16": ({16: 1.0}, {"full": 1.0}), "uniform_b4": ({4: 1.0}, {"full": 1.0}),
              "uniform_b2": ({2: 1.0}, {"full": 1.0}),
              "routing_only_bf16": ({16: 1.0}, {"skip": 0.15, "local": 0.45, "full": 0.4})}[variant]
    say(f"prefill baseline variant {variant}")
    case = random_case(2, 450, 4, 64, window=60, bit_weights=bw, mode_weights=mw, seed=len(variant) + 1,
                       device="cuda")
    cache, out, status = run_prefill(tr, case, 60)
    cache.close()
    assert status == 0
    check(case, out, 60, range(2), variant)


def test_prefill_long_prompt_sampled(tr):
    """An 80000-token prompt: more row tiles than the compaction keeps in LDS (512), so the unit
    list reads the tile bounds back from the row list, and full rows attend up to 80000 keys.
    Checked on sampled query rows (the oracle attends only those) and every skip row."""
    T, W = 80000, 512
    say(f"prefill long prompt T={T}")
    case = random_case(1, T, 1, 64, window=W, bit_weights={2: 0.3, 4: 0.3, 8: 0.2, 16: 0.2},
                       mode_weights={"skip": 0.1, "local": 0.45, "full": 0.45}, seed=80, device="cuda")
    cache, out, status = run_prefill(tr, case, W)
    cache.close()
    assert status == 0
    mode = case["mode"].cpu().numpy()[0, :, 0]
    rng = np.random.default_rng(5)
    pos = np.unique(np.concatenate([[0, 1, 127, 128, T - 2, T - 1], rng.integers(0, T, 40)]))
    ref = oracle.attend_cached(u16(case["q"])[0, pos], u16(case["k"])[0], u16(case["v"])[0],
                               case["bits"].cpu().numpy()[0], mode[pos][:, None], pos, W)["out"]
    got = bf16_to_f64(out)[0]
    compare_out(got[pos], ref, f"T={T} sampled rows")
    skip = np.nonzero(mode == 0)[0]
    assert np.all(got[skip] == 0.0)


def test_prefill_d128_split_tiles(tr):
    """head_dim 128 with key-split row tiles: 1536 mostly-full rows.  A full row tile near the end
    spans ~48 key tiles of 32 keys; the unit list cuts such tiles into chunks (32 key tiles each
    here: chunks of 16 would need more than the 16 partial slots of a head), so split units write
    partial results and the head_dim-128 merge combines them."""
    T, w = 1536, 300
    say(f"prefill D=128 T={T}, split tiles")
    case = random_case(2, T, 2, 128, window=w, bit_weights={2: 0.3, 4: 0.3, 8: 0.2, 16: 0.2},
                       mode_weights={"skip": 0.05, "local": 0.15, "full": 0.8}, seed=1536, device="cuda")
    cache, out, status = run_prefill(tr, case, w)
    cache.close()
    assert status == 0
    full = (case["mode"].cpu().numpy() == 2).sum(axis=1)           # [B, H] full rows per head
    assert full.min() > 1024                                       # so the last full tile spans > 32 key tiles
    check(case, out, w, range(2), f"D=128 T={T}")


def test_prefill_value_range_is_flagged_and_decode_is_not_limited(tr):
    """A V value beyond fp16's range (the prefill attention's V operand) sets TR_ERR_RANGE in
    prefill, while the cache stores it bit-exactly and decode over the same positions matches the
    oracle; values up to 65280 (the largest bf16 below 65504) pass prefill unflagged and match."""
    B, T, H, D, w = 1, 200, 2, 128, 50
    case = random_case(B, T, H, D, window=w, bit_weights={2: 0.3, 4: 0.3, 8: 0.2, 16: 0.2},
                       mode_weights={"local": 0.5, "full": 0.5}, seed=65504, device="cuda")
    v = case["v"].float()
    g = torch.Generator(device="cuda").manual_seed(3)
    big = 7.0e4 + 10.0 * torch.randn((D,), generator=g, device="cuda")
    v[0, 30, 0] = big                                             # a native (b = 16) row beyond fp16
    v[0, 90, 1] = big.flip(0)                                     # an 8-bit group beyond fp16
    case["bits"][0, 30], case["bits"][0, 90] = 16, 8
    case["v"] = v.to(torch.bfloat16)
    cache, out, status = run_prefill(tr, case, w)
    assert status == 7                                            # TR_ERR_RANGE
    check_codes(export_layer(tr, cache, 0, 0, T, B, H, D), case["k"], case["v"], case["bits"], where="range")
    cache.close()
    # decode at t = T - 1 over the same positions (written by tr_kv_quantize_write): no limit
    dcase = {x: case[x] for x in ("k", "v", "bits")}
    dcase["q"], dcase["mode"] = case["q"][:, T - 1].contiguous(), case["mode"][:, T - 1].contiguous()
    dcase["mode"].fill_(2)
    cache = tr.tr_kv_cache_alloc(1, B, H, D, T, prefill_tokens=-1)
    tr.tr_kv_quantize_write(cache, 0, case["k"][:, :T - 1].contiguous(), case["v"][:, :T - 1].contiguous(),
                            case["bits"][:, :T - 1].contiguous())
    tr.tr_kv_quantize_write(cache, 0, case["k"][:, T - 1:].contiguous(), case["v"][:, T - 1:].contiguous(),
                            case["bits"][:, T - 1:].contiguous())
    dec = torch.empty((B, H, D), dtype=torch.bfloat16, device="cuda")
    tr.tr_routed_attn_decode(cache, 0, dcase["q"], dcase["mode"], w, dec)
    assert tr.tr_kv_cache_status(cache) == 0
    cache.close()
    ref = oracle.attend_cached(u16(dcase["q"])[0][None], u16(case["k"])[0], u16(case["v"])[0],
                               case["bits"].cpu().numpy()[0], dcase["mode"].cpu().numpy()[0][None],
                               np.array([T - 1]), w)["out"][0]
    compare_out(bf16_to_f64(dec)[0], ref, "decode over values beyond fp16")
    # the largest bf16 below fp16's limit: no flag, and prefill matches the oracle
    v[0, 30, 0] = 65280.0
    v[0, 90, 1] = -65280.0
    case["v"] = v.to(torch.bfloat16)
    cache, out, status = run_prefill(tr, case, w)
    cache.close()
    assert status == 0
    check(case, out, w, [0], "prefill with |v| = 65280")


def test_prefill_capacity_of_the_scratch(tr):
    """prefill_tokens bounds the positions a prefill may reach; -1 makes a decode-only cache that
    refuses prefill (host-side, nothing launched) but still writes and decodes."""
    case = random_case(1, 64, 2, 64, window=8, bit_weights={4: 1.0}, mode_weights={"full": 1.0}, seed=6,
                       device="cuda")
    out = torch.empty((1, 64, 2, 64), dtype=torch.bfloat16, device="cuda")
    args = (case["q"], case["k"], case["v"], case["bits"], case["mode"], 64, 8, out)
    cache = tr.tr_kv_cache_alloc(1, 1, 2, 64, 200, prefill_tokens=-1)
    with pytest.raises(tr.TriRouteError, match="UNSUPPORTED"):
        tr.tr_routed_attn_prefill(cache, 0, *args)
    assert tr.tr_kv_cache_length(cache, 0) == 0
    cache.close()
    cache = tr.tr_kv_cache_alloc(1, 1, 2, 64, 200, prefill_tokens=100)
    tr.tr_routed_attn_prefill(cache, 0, *args)                     # positions 0 .. 63
    with pytest.raises(tr.TriRouteError, match="UNSUPPORTED"):
        tr.tr_routed_attn_prefill(cache, 0, *args)                 # would reach 128 > 100
    assert tr.tr_kv_cache_length(cache, 0) == 64 and tr.tr_kv_cache_status(cache) == 0
    cache.close()
    check(case, out, 8, [0], "prefill within a 100-position scratch")
