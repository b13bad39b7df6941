"""Float64 CPU oracle (test infrastructure only; never on the product path).

Only the tests, the smoke check and the benchmark's CPU-baseline leg import
this package.  It shares no code with the HIP library.
"""
from .ref import (  # noqa: F401
    unpack_int4,
    half_bits_to_f64,
    dequant,
    sigmoid,
    silu,
    router_logits,
    topk_ids,
    softmax_renormalised,
    kth_gap,
    route,
    experts,
    shared_expert,
    forward,
    forward_dense,
    routed_expert_weights,
    swiglu_ffn,
    f64_to_half_bits,
    rmsnorm,
    block_forward,
)
