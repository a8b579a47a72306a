"""Plain fp64 CPU oracle for the MHA2MLA latent-cache attention path.

TEST INFRASTRUCTURE ONLY.  Nothing in the library imports, calls or links this
package.  Only the test suite, the smoke check in __graft_entry__ and the
cpu_baseline leg of bench.py use it, to check and to time against.

It is written from the method as the pages state it (Paper-Notes ACL2025 page
"MHA2MLA: Towards Economical Inference ...", section 方法详解 / 关键设计
"method / key designs"), as plainly as possible:

* convert.py   -- 2-norm pair scores, head-wise top-r selection, joint SVD of
                  [W_k,nope ; W_v]; the ablation variants (fixed S_high / S_low /
                  S_uniform subspaces, SVD_split at the same latent width)
* attention.py -- latent-cache append (down-projection + partial RoPE) and the
                  UNABSORBED attention in which K_nope and V are rebuilt per head;
                  the absorbed form is kept separately only to pin the algebra
* int4.py      -- group-32 absmax int4 codec of the latent (4-bit cache)
* int2.py      -- group-32 affine 2-bit codec and the window of recent bf16 rows
                  (2-bit cache)
* paged.py     -- page-table gather of a paged cache and multi-query (causal) decode
* cache_bytes.py -- KV-cache bytes per token and the reduction percentages

All floating point is fp64 except the int4 codec, which emulates IEEE fp32 /
fp16 arithmetic with numpy scalar types because its integer codes are decided
in that precision.
"""

from .convert import (  # noqa: F401
    calibration_qk,
    convert_gqa_layer,
    convert_layer,
    gqa_pair_scores,
    group_of,
    joint_svd,
    pair_scores,
    select_pairs,
    select_pairs_by,
    split_dims,
    split_svd,
    split_svd_layer,
)
from .attention import (  # noqa: F401
    absorbed_decode_ref,
    append_ref,
    attend_ref,
    decode_ref,
    prefill_ref,
    reconstruct_head,
    rope_rotate,
)
from .int4 import (  # noqa: F401
    dequant_int4,
    int4_codes,
    int4_scale,
    pack_nibbles,
    quantize_int4_g32,
    unpack_nibbles,
    windowed_latent_int4,
)
from . import int2  # noqa: F401
from .paged import gather_pages, multi_query_decode_ref  # noqa: F401
from .cache_bytes import cache_bytes_per_token, mha_bytes_per_token, reduction_pct  # noqa: F401
