"""Float64 CPU oracle for the MXFP4 expert-weight MoE decode layer.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import or call anything in this
package.  The product path (the C-ABI library and its Python binding) never
imports it, and this package imports nothing from the product path: the two
share no code.  Inputs come from the seeded generator module
``mxfp4_expert_weight_amd.synth``, which holds none of the layer's arithmetic.

Every function is pinned by ``-m "not gpu"`` tests against values that do not
come from the oracle itself (exhaustive bit-field decoding, hand-worked bytes
and routing examples in ``tests/golden/``, brute force on tiny inputs,
closed forms, exact power-of-two metamorphics).  No function here is
"parity unpinned".
"""
from .prefetch_oracle import expert_heat, prefetch_checksums, prefetch_priority, select_experts  # noqa: F401
from .lmhead_oracle import E4M3_MAX, e4m3_decode, e4m3_round, lmhead_logits, lmhead_quantize  # noqa: F401
from .w4a8_oracle import (  # noqa: F401
    bf16_round,
    expert_hidden,
    expert_mlp_w4a8,
    moe_layer_w4a8,
    moe_layer_w4a8_tokens,
    mxfp8_dequantize,
    mxfp8_fake_quant,
    mxfp8_quantize,
    mxfp8_scale_exponent,
)
from .moe_oracle import (  # noqa: F401
    E2M1_MAGNITUDE,
    bf16_bits_to_f64,
    dequant_mxfp4,
    e2m1_decode,
    e8m0_decode,
    expert_mlp,
    moe_layer,
    moe_layer_tokens,
    router_logits,
    silu,
    sort_by_expert,
    topk_softmax,
)
