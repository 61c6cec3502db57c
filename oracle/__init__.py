"""Float64 CPU oracle (test infrastructure; see mxfp4_oracle's header)."""
from .mxfp4_oracle import (  # noqa: F401
    E2M1_VALUES, E2M1_TABLE, SCALE_BIAS, split_nibbles, group_codes, scale_factor,
    decode_rows, decode_expert, bucket_pairs, expert_linear, expert_linear_rows,
    expert_linear_scalar, silu, swiglu_hidden, expert_swiglu, expert_swiglu_rows, expert_swiglu_scalar,
    route_softmax, route_sigmoid, route_sigmoid_grouped, route_scalar, route_grouped_scalar, route_keys, route_weights, SOFTMAX_MASS_FLOOR, SIGMOID_EPS,
    E4M3_MAX, E4M3_TABLE, e4m3_value, mxfp8_block_exponent, quantize_e4m3, quantize_mxfp8, dequantize_mxfp8,
    expert_linear_mxfp8, expert_linear_mxfp8_rows,
    E2M1_MAX, mxfp4_block_exponent, quantize_e2m1, quantize_mxfp4, pack_codes, dequantize_mxfp4,
    expert_linear_mxfp4act, expert_linear_mxfp4act_rows,
)
