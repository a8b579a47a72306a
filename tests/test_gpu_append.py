"""GPU parity of mla_cache_append for whole prompts against the oracle, through the C ABI.

Prompts long enough for the large-tile path (256 tokens x 192 output columns, at least 192 tiles), a
ragged last tile, and a sequence appended at a non-zero start position; latent rows in bf16 and int4,
RoPE rows compared element by element, rows outside the appended ranges left untouched."""

import numpy as np
import pytest
import torch

import oracle
import synth
from synth import CONFIGS, scaled

from parity_lib import check_int4_cache, check_rows, converted_layer, log, shape_of, torch_dtype

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("fmt", ["dense", "int4"])
def test_append_long_prompt(fmt):
    from mla_latent_kv_cache_amd import LatentCache, append, pack_weights

    cfg = scaled(CONFIGS[1] if fmt == "dense" else CONFIGS[4], family="mid", batch=3)
    S, starts = 4200, [0, 37, 0]
    t_max = S + 40
    log(f"[append] {fmt} B=3 S={S} starts={starts}")
    layer = converted_layer(cfg.family, cfg.r_pairs, cfg.d_kv, cfg.dtype)
    shape = shape_of(cfg)
    w = pack_weights(shape, layer, rope_len=t_max, theta=cfg.theta)
    cache = LatentCache.allocate(shape, 3, t_max, fill=float("nan"))
    xs = [synth.context_x(cfg, b, S) for b in range(3)]
    x = torch.from_numpy(np.stack(xs).astype(np.float32)).cuda().to(torch_dtype(cfg))
    start = torch.tensor(starts, dtype=torch.int32, device="cuda")
    append(w, cache, x, start, max(starts))
    torch.cuda.synchronize()
    for b in range(3):
        p0 = starts[b]
        c, kr = oracle.append_ref(xs[b], layer["w_dkv"], layer["w_krope"], layer["pair_idx"], p0 + np.arange(S),
                                  cfg.d_head, cfg.theta)
        got_kr = cache.krope[b, p0:p0 + S].float().cpu().numpy().astype(np.float64).reshape(S, cfg.n_heads, -1)
        check_rows(cfg, got_kr, kr, f"k_rope b={b}")
        if fmt == "int4":
            check_int4_cache(c, oracle.unpack_nibbles(cache.ckv[b, p0:p0 + S].cpu().numpy()),
                             cache.ckv_scale[b, p0:p0 + S].cpu().numpy(), f"int4 b={b}")
        else:
            got = cache.ckv[b, p0:p0 + S].float().cpu().numpy().astype(np.float64)
            check_rows(cfg, got, c, f"c_kv b={b}")
            assert torch.isnan(cache.ckv[b, :p0].float()).all() and torch.isnan(cache.ckv[b, p0 + S:].float()).all()
        assert torch.isnan(cache.krope[b, :p0].float()).all() and torch.isnan(cache.krope[b, p0 + S:].float()).all()
        log(f"  b={b} ok")
