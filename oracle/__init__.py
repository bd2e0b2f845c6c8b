"""fp64 CPU oracle of one batch-1 decode step -- test infrastructure only.

Only tests/, the bench's cpu_baseline leg and the package's smoke check use it. The HIP
path never imports, links or calls anything here; the two share no code. Functions are
pinned by tests/test_oracle_pins.py against closed forms, invariants, brute force and
independent library routines.
"""
from .decode_oracle import (  # noqa: F401
    widen_bf16, decode_e4m3, round_to_bf16, rmsnorm, rope, linear, linear_bits, softmax, attend,
    attend_partial, merge_partials, attend_split, silu, swiglu, route, gqa_layer,
    mla_attention, mla_attention_absorbed, moe_ffn, mla_layer, layer, head, forward,
    dict_weights, kv_group, gqa_verify_layer, verify_forward, decode_e2m1, decode_e8m0, dequant_mxfp4,
    MX_BLOCK, index_scores, select_positions,
)
