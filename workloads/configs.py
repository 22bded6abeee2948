"""The five synthetic workloads, shaped after the model table of the TriRoute review page
(xllm-io.github.io, experimental setup: 160M has d = 768 and 12 heads -> head_dim 64; 1.3B
has d = 2048 and 16 heads -> head_dim 128; training sequence length 2048).

Every workload is synthetic: q, k, v ~ N(0, 1) rounded to bf16, keys multiplied by one
lognormal(0, 0.5) scale per (layer, head, channel) before rounding; widths b drawn iid per
(sequence, token) from ``bit_weights`` (or in geometric runs of mean 16 when ``clustered``);
modes drawn iid per (sequence, query token, head) from ``mode_weights``.
"""

from __future__ import annotations

from dataclasses import dataclass, field


@dataclass(frozen=True)
class WorkloadConfig:
    cid: int
    name: str
    kind: str                  # "prefill" or "decode"
    layers: int
    batch: int
    heads: int
    head_dim: int
    tokens: int                # prefill: T;  decode: cached context C (the new token is at C)
    window: int
    bit_weights: dict = field(default_factory=dict)    # {2: p, 4: p, 8: p, 16: p}
    mode_weights: dict = field(default_factory=dict)   # {"skip": p, "local": p, "full": p}
    clustered_bits: bool = False                       # b in runs of geometric(mean 16) length
    kv_heads: int = 0                                  # KV heads (0 = heads; fewer: grouped-query)

    @property
    def num_kv_heads(self) -> int:
        return self.kv_heads or self.heads

    @property
    def positions(self) -> int:
        """Cache positions per sequence after the workload's write (decode: C + 1)."""
        return self.tokens + 1 if self.kind == "decode" else self.tokens


CONFIGS = {
    0: WorkloadConfig(0, "tiny-prefill-T256-H4-D64", "prefill", 1, 1, 4, 64, 256, 32,
                      {2: 0.3, 4: 0.4, 8: 0.2, 16: 0.1},
                      {"skip": 0.2, "local": 0.4, "full": 0.4}),
    1: WorkloadConfig(1, "160m-decode-B8-C2048-H12-D64", "decode", 1, 8, 12, 64, 2048, 256,
                      {2: 0.3, 4: 0.4, 8: 0.2, 16: 0.1},
                      {"skip": 0.2, "local": 0.4, "full": 0.4}),
    2: WorkloadConfig(2, "160m-prefill-L12-B4-T2048-H12-D64", "prefill", 12, 4, 12, 64, 2048, 256,
                      {2: 0.25, 4: 0.35, 8: 0.25, 16: 0.15},
                      {"skip": 0.15, "local": 0.45, "full": 0.4}),
    3: WorkloadConfig(3, "1.3b-decode-L24-B32-C8192-H16-D128", "decode", 24, 32, 16, 128, 8192, 512,
                      {2: 0.3, 4: 0.4, 8: 0.2, 16: 0.1},
                      {"skip": 0.2, "local": 0.4, "full": 0.4}),
    4: WorkloadConfig(4, "1.3b-longctx-decode-B1-C65536-H16-D128", "decode", 1, 1, 16, 128, 65536, 1024,
                      {2: 0.6, 4: 0.3, 8: 0.08, 16: 0.02},
                      {"skip": 0.0, "local": 0.3, "full": 0.7},
                      clustered_bits=True),
    # Grouped-query variants with the model table's KV-head counts (160M: 3 KV heads for 12
    # query heads; 1.3B: 4 for 16), otherwise the shapes and mixes of workloads 2 and 3.
    5: WorkloadConfig(5, "1.3b-gqa-decode-L24-B32-C8192-H16-KV4-D128", "decode", 24, 32, 16, 128, 8192, 512,
                      {2: 0.3, 4: 0.4, 8: 0.2, 16: 0.1},
                      {"skip": 0.2, "local": 0.4, "full": 0.4}, kv_heads=4),
    6: WorkloadConfig(6, "160m-gqa-prefill-L12-B4-T2048-H12-KV3-D64", "prefill", 12, 4, 12, 64, 2048, 256,
                      {2: 0.25, 4: 0.35, 8: 0.25, 16: 0.15},
                      {"skip": 0.15, "local": 0.45, "full": 0.4}, kv_heads=3),
}


def get_config(cid: int) -> WorkloadConfig:
    return CONFIGS[int(cid)]
