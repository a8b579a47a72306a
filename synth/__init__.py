"""Seeded synthetic inputs shared by the oracle side and the GPU side.

This package holds configurations, random streams and dtype rounding only.  It
contains none of the method's arithmetic (no pair scoring, no SVD, no RoPE, no
attention, no quantisation); both `oracle/` and the GPU tests import it, and it
imports neither of them.
"""

from .inputs import (  # noqa: F401
    Config,
    CONFIGS,
    FAMILIES,
    GQA_FAMILIES,
    bf16_bits,
    bits_to_f64,
    context_x,
    eval_x,
    gqa_layer_weights,
    layer_weights,
    query_rows,
    round_to_device,
    scaled,
    seq_lens,
    structured_layer_weights,
)
