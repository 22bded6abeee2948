"""The no-allocation decode entry point (tr_routed_attn_decode_noalloc) against the plain one:
the same kernels with the split-K partials in the library's fixed device array.  Two calls in a
row on different caches, the second smaller, each matching tr_routed_attn_decode bit for bit
(the same chunk count) and the oracle within the attention tolerance; a call whose partials do not
fit the fixed array is refused with TR_ERR_SCRATCH and launches nothing."""

import numpy as np
import pytest
import torch

import oracle
from tests.gpu_helpers import bf16_to_f64, compare_out, say, u16
from workloads import random_case

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def tr():
    import mixed_precision_kv_tr_amd as tr
    return tr


def filled_cache(tr, case):
    k, v, bits = case["k"], case["v"], case["bits"]
    B, T, H, D = k.shape
    cache = tr.tr_kv_cache_alloc(1, B, H, D, T, num_query_heads=case["q"].shape[1], prefill_tokens=-1)
    tr.tr_kv_quantize_write(cache, 0, k[:, :T - 1].contiguous(), v[:, :T - 1].contiguous(), bits[:, :T - 1].contiguous())
    tr.tr_kv_quantize_write(cache, 0, k[:, T - 1:].contiguous(), v[:, T - 1:].contiguous(), bits[:, T - 1:].contiguous())
    return cache


def decode_case(B, T, H, D, w, seed, kv_heads=None):
    case = random_case(B, T, H, D, window=w, bit_weights={2: 0.3, 4: 0.4, 8: 0.2, 16: 0.1},
                       mode_weights={"skip": 0.2, "local": 0.4, "full": 0.4}, seed=seed, device="cuda",
                       n_queries=1, kv_heads=kv_heads)
    case["q"], case["mode"] = case["q"][:, 0].contiguous(), case["mode"][:, 0].contiguous()
    return case


def test_noalloc_decode_matches_the_plain_entry_point(tr):
    for (B, T, H, D, w, kv) in ((4, 3001, 8, 128, 300, 4), (2, 501, 4, 64, 40, None)):
        say(f"no-allocation decode B={B} T={T} H={H} D={D} kv={kv}")
        case = decode_case(B, T, H, D, w, seed=T + D, kv_heads=kv)
        cache = filled_cache(tr, case)
        ref = torch.empty((B, H, D), dtype=torch.bfloat16, device="cuda")
        got = torch.full((B, H, D), float("nan"), dtype=torch.bfloat16, device="cuda")
        tr.tr_routed_attn_decode(cache, 0, case["q"], case["mode"], w, ref)
        tr.tr_routed_attn_decode_noalloc(cache, 0, case["q"], case["mode"], w, got)
        assert tr.tr_kv_cache_status(cache) == 0
        cache.close()
        assert torch.equal(got, ref), "no-allocation decode differs from tr_routed_attn_decode"
        g = bf16_to_f64(got)
        bb, mb = case["bits"].cpu().numpy(), case["mode"].cpu().numpy()
        for s in range(B):
            want = oracle.attend_cached(u16(case["q"])[s][None], u16(case["k"])[s], u16(case["v"])[s], bb[s],
                                        mb[s][None], np.array([T - 1]), w)["out"][0]
            compare_out(g[s], want, f"no-allocation decode seq {s}")


def test_noalloc_decode_refuses_what_does_not_fit(tr):
    """32 x 16 (seq, head) pairs forced to 64 chunks of 520-byte partials need 17 MB > 8 MiB."""
    case = decode_case(32, 2048, 16, 128, 100, seed=5)
    cache = filled_cache(tr, case)
    tr.tr_kv_cache_set_decode_chunks(cache, 64)
    out = torch.zeros((32, 16, 128), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(tr.TriRouteError, match="TR_ERR_SCRATCH"):
        tr.tr_routed_attn_decode_noalloc(cache, 0, case["q"], case["mode"], 100, out)
    torch.cuda.synchronize()
    assert torch.count_nonzero(out.float()) == 0                     # nothing was launched
    tr.tr_routed_attn_decode(cache, 0, case["q"], case["mode"], 100, out)   # the plain call has room
    assert tr.tr_kv_cache_status(cache) == 0
    cache.close()
