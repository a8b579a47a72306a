"""MHA2MLA latent-cache attention for MI355X (gfx950): a C-ABI HIP library plus this thin binding.

    from mla_latent_kv_cache_amd import LayerShape, pack_weights, LatentCache, append, decode, prefill
"""

from .api import (  # noqa: F401
    BoundDecode,
    LatentCache,
    LayerShape,
    LayerWeights,
    MlaError,
    append,
    append_workspace_bytes,
    append_ws,
    decode,
    decode_multi,
    decode_phase,
    decode_step,
    decode_step_static,
    decode_step_workspace_bytes,
    decode_workspace_bytes,
    pack_weights,
    prefill,
    prefill_workspace_bytes,
    quantize_int2,
    quantize_int4,
    rope_tables,
    STATIC_SCRATCH_BYTES,
)
from .convert import convert_layer  # noqa: F401
