"""CPU oracle for the streaming code2wav decoder.

TEST INFRASTRUCTURE ONLY.  Only tests/, __graft_entry__.smoke() and bench.py's
cpu_baseline leg may import this package.  The product path (the HIP library
and its Python binding) never calls it and shares no code with it.

Every function is a plain, slow, layer-by-layer numpy evaluation of what the
decoder computes, written from the pages' description; see decoder.py for the
citations and for which functions are pinned by which tests.
"""
from .decoder import (  # noqa: F401
    OracleState,
    causal_conv1d,
    conv_transpose1d_causal,
    decode_chunk,
    decode_whole,
    dequantize_rows_int8,
    int8_eligible,
    quantize_rows_int8,
    quantize_weights_int8,
    gelu,
    layer_norm,
    new_state,
    rope_rotate,
    round_operand,
    cast_operand_weights,
    rvq_embed_sum,
    snake,
    transformer_layer,
    window_attention,
)
