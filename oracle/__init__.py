"""The CPU oracle for the MoE layer forward: test infrastructure only.

A plain, slow, fp64 numpy statement of what the layer computes. Only the test
suite, the package's smoke check and the benchmark's CPU-baseline leg may import
it; the GPU library never calls into it and shares no code with it.

Every function cites the passage of the Colibri pages it follows. Pages are
named by address: [0539edu] www.0539edu.com/news/4774449, [mhpq]
www.mhpq.cn/news/563172, [hotelren] www.hotelren.com/news/4731937, [trdm]
www.trdm.cn/news/555962, [pptc] www.pptc.cn/news/100465.

Pinned (see tests/test_oracle.py): router logits, top-k selection and tie rule,
top-k weights (softmax over the chosen logits, or the chosen raw logits),
shared-expert gate, scatter (counts, offsets, permutation), SwiGLU expert,
combine, int8 and int4 group-wise dequantisation, the layer with a caller-given
routing. No function is parity-unpinned.
"""
from .moe_oracle import (
    router_logits,
    select_topk,
    topk_weights,
    topk_raw_weights,
    shared_gate,
    scatter_stable_sort,
    scatter_counting,
    dequantize,
    dequantize_groupwise,
    swiglu_expert,
    valid_selections,
    moe_forward,
    moe_forward_routed,
    OracleLayer,
)

__all__ = [
    "router_logits", "select_topk", "topk_weights", "topk_raw_weights", "shared_gate",
    "scatter_stable_sort", "scatter_counting", "dequantize", "dequantize_groupwise", "swiglu_expert",
    "valid_selections", "moe_forward", "moe_forward_routed", "OracleLayer",
]
