"""Plain CPU oracle for TriRoute's routed attention over a per-token mixed-precision KV cache.

TEST INFRASTRUCTURE ONLY.  This package is the slow, obviously correct reference that the
HIP library is checked against.  Only the test suite, the smoke check in
``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of ``bench.py`` may import it.  It
shares no code with the HIP path (``mixed_precision_kv_tr_amd``) and imports nothing from it.

What it computes, and where the definitions come from (TriRoute: Unified Learned Routing for
Joint Adaptive Attention, Experts, and KV-Cache Allocation; the paper-review page on
xllm-io.github.io, section "core formulas"):

* ``quantize`` / ``dequantize`` -- Eq. (4): asymmetric per-token quantization of one head's
  K or V vector at width b in {2, 4, 8, 16}; s = (max - min) / (2^b - 1), z = min,
  Q_b(x) = round((x - z) / s) * s + z; b = 16 keeps the native (bf16) value.
* ``routed_attention`` -- Eq. (2): per (query, head) one of skip (output 0),
  local-w (keys t-w .. t) or full causal (keys <= t), softmax attention over the cached,
  dequantized K/V.
* ``attend_cached`` -- the inference step that combines them (the paragraph after
  Algorithm 1 on the same page: each token's K/V is stored at its chosen width, and later
  queries attend to what was stored).
* ``controller_route`` -- Eq. (5) with Eq. (11)'s whitening and the hard argmax of inference:
  the routing decisions (a mode per head, a width per token) from a token's residual state.
* ``moe_ffn`` -- Eq. (3): E SwiGLU experts plus the null expert, top-k of a softmax gate with
  the weights renormalized over the selected set.

Readings where the pages leave a step open (all in fp32 for the quantizer, fp64 for attention):
the quantization group is one head's D-vector of one token, separately for K and V; "round"
is round-half-to-even on the fp32 quotient; s and the quotient are correctly rounded fp32
divides taken in the fixed order R = fl(max - min), s = fl(R / n), d = fl(x - z),
r = fl(d / s); z = min + 0.0 so that -0 becomes +0; a constant group (s = 0) gets codes 0;
the local window holds w + 1 keys clipped at position 0; scores are scaled by 1/sqrt(D).

Pins: every function here is checked in ``tests/test_oracle_*.py`` against closed forms,
invariants, special cases that reduce to library routines (torch's scaled-dot-product
attention in fp64) and brute force on tiny inputs.  The pages print no numeric worked example
for either equation, so no function is pinned to a value the pages print.
"""

from .quantize import BITS_ALLOWED, bf16_bits_to_f32, dequantize, quantize
from .attention import MODE_FULL, MODE_LOCAL, MODE_SKIP, routed_attention
from .reference import attend_cached
from .controller import BIT_CHOICES, controller_logits, controller_route
from . import moe
from .moe import gate as moe_gate, moe_ffn

__all__ = [
    "BITS_ALLOWED",
    "MODE_SKIP",
    "MODE_LOCAL",
    "MODE_FULL",
    "bf16_bits_to_f32",
    "quantize",
    "dequantize",
    "routed_attention",
    "BIT_CHOICES",
    "controller_logits",
    "controller_route",
    "moe_gate",
    "moe_ffn",
    "attend_cached",
]
