"""GPU parity of decode routed attention (Eq. 2 over the Eq. 4 cache) against the oracle:
|gpu - oracle| <= 2e-3 + 1e-2 |oracle| element-wise, on the same dequantized K/V."""

import numpy as np
import pytest
import torch

import oracle
from tests.gpu_helpers import bf16_to_f64, compare_out, say, u16
from workloads import CONFIGS, layer_inputs, random_case

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def tr():
    import mixed_precision_kv_tr_amd as tr
    return tr


def run_decode(tr, case, window, page_code_bytes=0, layers=1, layer=0, split_at=None, chunks=0):
    """Write positions 0..C-1, then the new token C (a second write), then decode at t = C
    (split into `chunks` position chunks if > 0)."""
    k, v, bits, q, mode = case["k"], case["v"], case["bits"], case["q"], case["mode"]
    B, T, H, D = k.shape
    HQ = q.shape[1]
    cache = tr.tr_kv_cache_alloc(layers, B, H, D, T, page_code_bytes=page_code_bytes, num_query_heads=HQ)
    C = T - 1
    cut = C if split_at is None else split_at
    if cut > 0:
        tr.tr_kv_quantize_write(cache, layer, k[:, :cut].contiguous(), v[:, :cut].contiguous(),
                                bits[:, :cut].contiguous())
    tr.tr_kv_quantize_write(cache, layer, k[:, cut:].contiguous(), v[:, cut:].contiguous(),
                            bits[:, cut:].contiguous())
    out = torch.empty((B, HQ, D), dtype=torch.bfloat16, device="cuda")
    tr.tr_kv_cache_set_decode_chunks(cache, chunks)
    try:
        tr.tr_routed_attn_decode(cache, layer, q, mode, window, out)
        status = tr.tr_kv_cache_status(cache)
    finally:
        cache.close()
    return out, status


def oracle_decode(case, window, seqs):
    kb, vb, qb = u16(case["k"]), u16(case["v"]), u16(case["q"])
    bb, mb = case["bits"].cpu().numpy(), case["mode"].cpu().numpy()
    T = kb.shape[1]
    refs = {}
    for s in seqs:
        res = oracle.attend_cached(qb[s][None], kb[s], vb[s], bb[s], mb[s][None], np.array([T - 1]), window)
        refs[s] = res["out"][0]
    return refs


def check(case, out, window, seqs, where):
    got = bf16_to_f64(out)
    refs = oracle_decode(case, window, seqs)
    for s in seqs:
        compare_out(got[s], refs[s], f"{where} seq {s}")


@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("C", [0, 1, 63, 64, 300, 1500])
def test_decode_random(tr, D, C):
    say(f"decode random D={D} C={C}")
    case = random_case(3, C + 1, 5, D, window=17, bit_weights={2: 0.3, 4: 0.3, 8: 0.2, 16: 0.2},
                       mode_weights={"skip": 0.2, "local": 0.4, "full": 0.4}, seed=C * 3 + D,
                       device="cuda", n_queries=1)
    case["q"], case["mode"] = case["q"][:, 0].contiguous(), case["mode"][:, 0].contiguous()
    out, status = run_decode(tr, case, 17)
    assert status == 0
    check(case, out, 17, range(3), f"D={D} C={C}")


@pytest.mark.parametrize("window", [0, 1, 5, 4000])
def test_decode_windows_single_width(tr, window):
    for bw in (2, 4, 8, 16):
        say(f"decode window={window} b={bw}")
        case = random_case(2, 901, 3, 128, window=window, bit_weights={bw: 1.0},
                           mode_weights={"local": 0.5, "full": 0.5}, seed=window + bw, device="cuda", n_queries=1)
        case["q"], case["mode"] = case["q"][:, 0].contiguous(), case["mode"][:, 0].contiguous()
        out, status = run_decode(tr, case, window)
        assert status == 0
        check(case, out, window, range(2), f"w={window} b={bw}")


def test_decode_all_skip_is_zero(tr):
    case = random_case(2, 50, 4, 64, window=3, bit_weights={4: 1.0}, mode_weights={"skip": 1.0},
                       seed=1, device="cuda", n_queries=1)
    case["q"], case["mode"] = case["q"][:, 0].contiguous(), case["mode"][:, 0].contiguous()
    out, status = run_decode(tr, case, 3)
    assert status == 0 and torch.count_nonzero(out.float()) == 0


def test_decode_config1(tr):
    cfg = CONFIGS[1]
    say(f"decode {cfg.name}")
    case = layer_inputs(cfg, 0, device="cuda")
    out, status = run_decode(tr, case, cfg.window)
    assert status == 0
    check(case, out, cfg.window, range(cfg.batch), cfg.name)


def test_decode_config3_full_size_sampled(tr):
    cfg = CONFIGS[3]
    say(f"decode {cfg.name} full size, layer 1 of a 2-layer cache, sampled sequences")
    case = layer_inputs(cfg, 1, device="cuda")
    out, status = run_decode(tr, case, cfg.window, layers=2, layer=1)
    assert status == 0
    check(case, out, cfg.window, [0, 9, 31], cfg.name)


def test_decode_config4_full_size(tr):
    cfg = CONFIGS[4]
    say(f"decode {cfg.name} full size")
    case = layer_inputs(cfg, 0, device="cuda")
    out, status = run_decode(tr, case, cfg.window)
    assert status == 0
    check(case, out, cfg.window, [0], cfg.name)


def test_decode_chunking_and_paging_invariance(tr):
    """With the chunk count fixed, page sizes leave the output bit-identical; every forced split-K
    chunk count matches the oracle: 5 and 8 chunks (one combine batch), 40 and 64 chunks (merges of more than 32 chunks,
    i.e. two combine batches), a single chunk over a whole window of the largest item (544
    positions), and a single chunk over a longer window is refused."""
    say("decode: split-K chunk counts and page sizes agree")
    case = random_case(2, 2500, 4, 128, window=700, bit_weights={2: 0.3, 4: 0.3, 8: 0.2, 16: 0.2},
                       mode_weights={"local": 0.5, "full": 0.5}, seed=77, device="cuda", n_queries=1)
    case["q"], case["mode"] = case["q"][:, 0].contiguous(), case["mode"][:, 0].contiguous()
    # pages of 1024 code bytes hold 4 bf16 tokens at head_dim 128, which caps a chunk at 136
    # positions; with the chunk count fixed (20 chunks of 125) the page size must not matter
    base, _ = run_decode(tr, case, 700, chunks=20)
    for pcb in (1024, 16384):
        other, _ = run_decode(tr, case, 700, page_code_bytes=pcb, chunks=20)
        assert torch.equal(base, other), f"page_code_bytes={pcb} changed the output"
    refs = oracle_decode(case, 700, range(2))
    got = bf16_to_f64(base)
    for s in range(2):
        compare_out(got[s], refs[s], f"nch=20 seq {s}")
    for nch in (5, 8, 40, 64):
        out, status = run_decode(tr, case, 700, chunks=nch)
        assert status == 0
        got = bf16_to_f64(out)
        for s in range(2):
            compare_out(got[s], refs[s], f"nch={nch} seq {s}")
    with pytest.raises(tr.TriRouteError):
        run_decode(tr, case, 700, chunks=1)               # 2500 positions in one item: refused
    short = random_case(2, 544, 4, 128, window=100, bit_weights={2: 0.3, 4: 0.3, 8: 0.2, 16: 0.2},
                        mode_weights={"local": 0.5, "full": 0.5}, seed=78, device="cuda", n_queries=1)
    short["q"], short["mode"] = short["q"][:, 0].contiguous(), short["mode"][:, 0].contiguous()
    out, status = run_decode(tr, short, 100, chunks=1)
    assert status == 0
    check(short, out, 100, range(2), "nch=1, 544-position window")

def test_decode_repeated_calls_on_one_cache(tr):
    """Calls in a row on one cache, with multi-chunk windows (merged by the wave that finishes a
    window's last chunk, through per-window counters that each call must leave at zero) between
    one-chunk ones: every call matches the oracle and repeating a call repeats its output bit for
    bit, for both head sizes and a chunk count above one merge batch (32 chunks)."""
    for D in (64, 128):
        say(f"decode: repeated calls on one cache, D={D}")
        case = random_case(3, 1800, 4, D, window=300, bit_weights={2: 0.3, 4: 0.3, 8: 0.2, 16: 0.2},
                           mode_weights={"skip": 0.1, "local": 0.45, "full": 0.45}, seed=90 + D, device="cuda",
                           n_queries=1)
        q, mode = case["q"][:, 0].contiguous(), case["mode"][:, 0].contiguous()
        B, T, H, _ = case["k"].shape
        cache = tr.tr_kv_cache_alloc(1, B, H, D, T)
        try:
            tr.tr_kv_quantize_write(cache, 0, case["k"], case["v"], case["bits"])
            refs = oracle_decode({**case, "q": q, "mode": mode}, 300, range(B))
            first = {}
            for chunks in (0, 7, 1, 40, 7, 0, 40):
                if chunks == 1:
                    continue                                 # 1800 positions exceed one item
                out = torch.empty((B, H, D), dtype=torch.bfloat16, device="cuda")
                tr.tr_kv_cache_set_decode_chunks(cache, chunks)
                tr.tr_routed_attn_decode(cache, 0, q, mode, 300, out)
                torch.cuda.synchronize()
                assert tr.tr_kv_cache_status(cache) == 0
                if chunks in first:
                    assert torch.equal(first[chunks], out), f"D={D}: a repeated call with {chunks} chunks differs"
                else:
                    first[chunks] = out
                    got = bf16_to_f64(out)
                    for s in range(B):
                        compare_out(got[s], refs[s], f"D={D} chunks={chunks} seq {s}")
        finally:
            cache.close()


def test_decode_bad_mode_is_flagged(tr):
    case = random_case(1, 20, 2, 64, window=3, bit_weights={4: 1.0}, mode_weights={"full": 1.0},
                       seed=2, device="cuda", n_queries=1)
    case["q"], case["mode"] = case["q"][:, 0].contiguous(), case["mode"][:, 0].contiguous()
    case["mode"][0, 1] = 9
    out, status = run_decode(tr, case, 3)
    assert status == 6
    assert torch.count_nonzero(out[0, 1].float()) == 0


@pytest.mark.parametrize("G", [2, 4, 8])
@pytest.mark.parametrize("D", [64, 128])
def test_decode_grouped_query_heads(tr, G, D):
    """Grouped-query attention: 8 query heads over 8 / G KV heads, query head h reading KV
    head h // G (the oracle's mapping, pinned against SDPA's grouped-query mode)."""
    say(f"decode GQA G={G} D={D}")
    case = random_case(3, 700, 8, D, window=40, bit_weights={2: 0.3, 4: 0.3, 8: 0.2, 16: 0.2},
                       mode_weights={"skip": 0.2, "local": 0.4, "full": 0.4}, seed=G * 13 + D,
                       device="cuda", n_queries=1, kv_heads=8 // G)
    case["q"], case["mode"] = case["q"][:, 0].contiguous(), case["mode"][:, 0].contiguous()
    out, status = run_decode(tr, case, 40)
    assert status == 0
    check(case, out, 40, range(3), f"G={G} D={D}")


def test_decode_grouped_mode_mixes(tr):
    """Groups of 4 query heads with every kind of mode mix: a local head inside a group that
    also has a full head only sees its window; an all-skip group writes zeros."""
    B, C, H, Hkv, D, w = 1, 1500, 16, 4, 128, 100
    case = random_case(B, C + 1, H, D, window=w, bit_weights={2: 0.3, 4: 0.3, 8: 0.2, 16: 0.2},
                       mode_weights={"local": 1.0}, seed=41, device="cuda", n_queries=1, kv_heads=Hkv)
    case["q"] = case["q"][:, 0].contiguous()
    case["mode"] = torch.tensor([[2, 1, 0, 1, 1, 1, 1, 1, 0, 0, 0, 0, 2, 2, 0, 2]], dtype=torch.uint8,
                                device="cuda")
    out, status = run_decode(tr, case, w)
    assert status == 0
    assert torch.count_nonzero(out[0, 8:12].float()) == 0
    check(case, out, w, [0], "GQA mode mixes")


def test_decode_config5_gqa_full_size_sampled(tr):
    cfg = CONFIGS[5]
    say(f"decode {cfg.name} full size, sampled sequences")
    case = layer_inputs(cfg, 0, device="cuda")
    out, status = run_decode(tr, case, cfg.window)
    assert status == 0
    check(case, out, cfg.window, [0, 17, 31], cfg.name)


def test_decode_grouped_query_heads_share_kv(tr):
    """Query heads of one group given the same query and mode return the same row."""
    case = random_case(2, 300, 8, 128, window=20, bit_weights={2: 0.4, 4: 0.3, 8: 0.2, 16: 0.1},
                       mode_weights={"local": 0.5, "full": 0.5}, seed=77, device="cuda", n_queries=1, kv_heads=2)
    q = case["q"][:, 0].contiguous()
    mode = case["mode"][:, 0].contiguous()
    q[:, 1:4] = q[:, 0:1]
    mode[:, 1:4] = mode[:, 0:1]
    case["q"], case["mode"] = q, mode
    out, status = run_decode(tr, case, 20)
    assert status == 0
    for h in (1, 2, 3):
        assert torch.equal(out[:, h], out[:, 0])
    check(case, out, 20, range(2), "GQA shared rows")


def test_alloc_rejects_bad_query_head_count(tr):
    with pytest.raises(tr.TriRouteError):
        tr.tr_kv_cache_alloc(1, 1, 3, 64, 16, num_query_heads=4)
    with pytest.raises(tr.TriRouteError):
        tr.tr_kv_cache_alloc(1, 1, 4, 64, 16, num_query_heads=2)


@pytest.mark.parametrize("variant", ["dense_bf16", "uniform_b4", "uniform_b2", "routing_only_bf16"])
def test_decode_baseline_variants(tr, variant):
    """The comparison configurations the benchmark runs (dense bf16 cache with every head full,
    one width for every token, bf16 with routed modes) against the oracle."""
    bw, mw = {"dense_bf16": ({16: 1.0}, {"full": 1.0}), "uniform_b4": ({4: 1.0}, {"full": 1.0}),
              "uniform_b2": ({2: 1.0}, {"full": 1.0}),
              "routing_only_bf16": ({16: 1.0}, {"skip": 0.2, "local": 0.4, "full": 0.4})}[variant]
    say(f"decode baseline variant {variant}")
    case = random_case(4, 1201, 8, 128, window=100, bit_weights=bw, mode_weights=mw, seed=len(variant),
                       device="cuda", n_queries=1)
    case["q"], case["mode"] = case["q"][:, 0].contiguous(), case["mode"][:, 0].contiguous()
    out, status = run_decode(tr, case, 100)
    assert status == 0
    check(case, out, 100, range(4), variant)


def test_profile_families_count_the_launches(tr):
    """tr_profile_read: one entry per kernel family, launches counted while enabled, nothing
    recorded while disabled."""
    case = random_case(2, 300, 4, 64, window=40, bit_weights={2: 0.3, 4: 0.3, 8: 0.2, 16: 0.2},
                       mode_weights={"skip": 0.2, "local": 0.4, "full": 0.4}, seed=11, device="cuda")
    cache = tr.tr_kv_cache_alloc(1, 2, 4, 64, 301)
    out = torch.empty((2, 300, 4, 64), dtype=torch.bfloat16, device="cuda")
    tr.tr_profile_enable(cache, True)
    tr.tr_routed_attn_prefill(cache, 0, case["q"], case["k"], case["v"], case["bits"], case["mode"], 300, 40, out)
    tr.tr_kv_quantize_write(cache, 0, case["k"][:, :1].contiguous(), case["v"][:, :1].contiguous(),
                            case["bits"][:, :1].contiguous(), 1)
    dout = torch.empty((2, 4, 64), dtype=torch.bfloat16, device="cuda")
    tr.tr_routed_attn_decode(cache, 0, case["q"][:, 0].contiguous(), case["mode"][:, 0].contiguous(), 40, dout)
    prof = tr.tr_profile_read(cache)
    assert set(prof) == {"write", "decode_split", "decode_combine", "prefill_prep", "prefill_attn", "prefill_merge"}
    for fam in ("write", "decode_split", "prefill_prep", "prefill_attn", "prefill_merge"):
        n, ms = prof[fam]
        assert n >= 1 and ms > 0.0, (fam, n, ms)
    assert all(v == (0, 0.0) for v in tr.tr_profile_read(cache).values())   # the read clears
    tr.tr_profile_enable(cache, False)
    tr.tr_routed_attn_decode(cache, 0, case["q"][:, 0].contiguous(), case["mode"][:, 0].contiguous(), 40, dout)
    assert all(v == (0, 0.0) for v in tr.tr_profile_read(cache).values())
    cache.close()
