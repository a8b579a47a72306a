"""mla_decode_step_static (the decode step whose workspace is the library's static per-GPU buffer) against
mla_decode_step with a caller workspace, through the C ABI: outputs and cache contents bit for bit, on two
calls in a row, the second with a smaller batch and shorter contexts (the buffer keeps the first call's
contents, which the second must not read)."""

import numpy as np
import pytest
import torch

from mla_latent_kv_cache_amd import (STATIC_SCRATCH_BYTES, LatentCache, LayerShape, MlaError, append, decode_step,
                                     decode_step_static, decode_step_workspace_bytes, pack_weights)

pytestmark = pytest.mark.gpu


def _random_layer(shape, seed):
    """Seeded random weights of the layer's shapes (both entry points get the same ones; only their results are
    compared with each other)."""
    rng = np.random.default_rng(seed)
    d, n_h, d_h, r, D = shape.d_model, shape.n_heads, shape.d_head, shape.r_pairs, shape.d_kv
    return {"w_dkv": rng.standard_normal((d, D)) / np.sqrt(d), "w_krope": rng.standard_normal((d, n_h * 2 * r)) * 0.02,
            "w_uk": rng.standard_normal((n_h, D, d_h - 2 * r)) * 0.05, "w_uv": rng.standard_normal((n_h, D, d_h)) * 0.05,
            "pair_idx": np.sort(np.stack([rng.choice(d_h // 2, r, replace=False) for _ in range(n_h)]), axis=1)}


def _same_bits(u, v):
    return torch.equal(u.contiguous().view(torch.uint8), v.contiguous().view(torch.uint8))


def _one_call(shape, lens, seed):
    B, t_max = len(lens), max(lens)
    print(f"[static-step] {shape.cache_fmt} d_kv={shape.d_kv} B={B} lens={lens[:4]}...", flush=True)
    need = decode_step_workspace_bytes(shape, B, 1, t_max)
    assert need <= STATIC_SCRATCH_BYTES
    w = pack_weights(shape, _random_layer(shape, seed), rope_len=t_max)
    g = torch.Generator(device="cuda")
    g.manual_seed(seed)
    caches = [LatentCache.allocate(shape, B, t_max, fill=float("nan")) for _ in range(2)]
    zero = torch.zeros(1, dtype=torch.int32, device="cuda")
    for b, L in enumerate(lens):
        x = torch.randn((1, L - 1, shape.d_model), generator=g, device="cuda").to(torch.bfloat16)
        for cache in caches:
            append(w, cache.view(b, b + 1), x, zero, 0)
    x_new = torch.randn((B, 1, shape.d_model), generator=g, device="cuda").to(torch.bfloat16)
    q = torch.randn((B, shape.n_heads, shape.d_head), generator=g, device="cuda").to(torch.bfloat16)
    start = torch.tensor([L - 1 for L in lens], dtype=torch.int32, device="cuda")
    lens_t = torch.tensor(lens, dtype=torch.int32, device="cuda")
    out_ref = torch.empty_like(q)
    out_st = torch.full_like(q, float("nan"))
    decode_step(w, caches[0], x_new, start, t_max - 1, q, lens_t, t_max, out=out_ref)
    decode_step_static(w, caches[1], x_new, start, t_max - 1, q, lens_t, t_max, out_st)
    torch.cuda.synchronize()
    assert torch.isfinite(out_ref.float()).all()
    assert torch.equal(out_st, out_ref), "mla_decode_step_static differs from mla_decode_step"
    for name in ("ckv", "ckv_scale", "krope"):
        if getattr(caches[0], name) is not None:
            assert _same_bits(getattr(caches[0], name), getattr(caches[1], name)), name
    print(f"  identical: out {tuple(out_st.shape)}, workspace {need / 2**20:.1f} MiB of the static "
          f"{STATIC_SCRATCH_BYTES >> 20} MiB", flush=True)


def test_static_step_matches_workspace_step_twice():
    """First a Llama-2-7B-shaped layer at 32 sequences x 4096 positions (22.7 MiB of workspace), then a smaller
    int4 layer at 3 ragged sequences, on the same static buffer."""
    _one_call(LayerShape(4096, 32, 128, 4, 512, "bf16", "dense"), [4096] * 32, 1)
    _one_call(LayerShape(1024, 32, 128, 4, 512, "bf16", "int4_g32"), [300, 2, 97], 2)


def test_static_step_rejects_oversized_request():
    """A request beyond the static buffer fails with MLA_ERR_WORKSPACE and writes nothing."""
    shape = LayerShape(4096, 32, 128, 4, 512, "bf16", "dense")
    B, t_max = 256, 4096
    assert decode_step_workspace_bytes(shape, B, 1, t_max) > STATIC_SCRATCH_BYTES
    w = pack_weights(shape, _random_layer(shape, 3), rope_len=t_max)
    cache = LatentCache.allocate(shape, B, t_max)  # full size (1.5 GB), so that nothing could read past it
    x = torch.zeros((B, 1, shape.d_model), dtype=torch.bfloat16, device="cuda")
    q = torch.zeros((B, shape.n_heads, shape.d_head), dtype=torch.bfloat16, device="cuda")
    out = torch.full_like(q, 7.0)
    lens = torch.full((B,), t_max, dtype=torch.int32, device="cuda")
    with pytest.raises(MlaError) as e:
        decode_step_static(w, cache, x, lens - 1, t_max - 1, q, lens, t_max, out)
    assert e.value.status == -4
    torch.cuda.synchronize()
    assert (out == 7.0).all()
