"""Seeded synthetic inputs for the fused attention forward pass.

This package only draws random numbers and encodes them into the storage
formats the attention path consumes (bf16 bit patterns, OCP E4M3FN codes with
per-block fp32 scales, int32 document ids).  It holds none of the attention
arithmetic; both the CPU oracle and the GPU path read what it produces.
"""

from .gen import (  # noqa: F401
    ATTN_ALIBI,
    ATTN_CAUSAL,
    ATTN_DOCUMENT,
    ATTN_SOFTCAP,
    ATTN_WINDOW,
    CONFIGS,
    Problem,
    bf16_bits_from_f32,
    config_problem,
    doc_ids_from_lengths,
    draw_doc_lengths,
    e4m3_codes_from_f64,
    make_problem,
    make_varlen_problem,
    make_dout,
    quantize_e4m3_blocks,
    rotation_matrix,
    sylvester_hadamard,
)
