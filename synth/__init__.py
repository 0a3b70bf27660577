"""Seeded synthetic inputs for the quantized routed-expert MoE layer.

This package only draws random numbers and encodes them into the layer's input formats
(packed int2/int3/int4/int6/int8 codes with fp16 scales, bf16 activations, fp32 router).  It holds
none of the layer's arithmetic (routing, selection, expert FFN, combine), and both the
GPU library's tests and the CPU oracle's tests take their inputs from here.
"""
from .workloads import WORKLOADS, Workload  # noqa: F401
from .inputs import (  # noqa: F401
    FMT_FP32, FMT_INT8_ROW, FMT_INT4_G32, FMT_INT6_G32, FMT_INT3_G32, FMT_INT2_G32,
    Layer, Norm, make_layer, make_layer_all_codes, make_norm, make_tokens, quantize_int4_g32,
    quantize_int6_g32, quantize_int3_g32, quantize_int2_g32, quantize_int8_row, pack_int4,
    pack_int6, pack_int3, pack_int2, zipf_bias, bits16,
)
