"""Seeded synthetic inputs for the quantized expert-FFN MoE layer.

This package only draws random numbers into arrays of the right shapes and
dtypes.  It holds none of the layer's arithmetic: no routing, no
dequantisation, no normalisation.  Both the float64 oracle (through the
tests) and the GPU path (through the tests and the benchmark) are fed from
here, so they always see the same bits.
"""
from .workloads import (  # noqa: F401
    HIDDEN, N_EXPERTS, TOP_K, INTER, SHARED_INTER, NORM_EPS,
    QFmt, Workload, WORKLOADS, workload, make_layer, make_tokens,
    make_tiny_layer, bf16_bits_to_f32, f32_to_bf16_bits,
    VOCAB, DENSE_INTER, make_lm_head, make_dense_ffn, make_hidden,
    HEADS, HEAD_DIM, RSWA_WINDOW, make_rswa, make_attn_weights,
)
