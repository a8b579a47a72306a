"""GPU parity of caches that store each RoPE key once per key head (LayerShape.rope_heads < n_heads), the layout of
a layer converted from a grouped-query source: every query head of a group keeps the same RoPE subspaces of the
same KV head, so its RoPE keys are one key.  The oracle runs the per-query-head form of the same conversion
(oracle.convert_gqa_layer, expanded); the GPU's compact cache rows must be its keys of the group's first head,
and every output must match it to the usual tolerance.  Cases cover each attention kernel that reads the
compact rows: the dense ring kernel at latent width 512 with 4 pairs (8 key heads), the int4 register-staged
kernel (any divisor), the generic kernel (the other shapes), the fused decode step, a paged pool, multi-query
decode and the prefill."""

import numpy as np
import pytest
import torch

import oracle
import synth
from synth import CONFIGS, scaled

from parity_lib import (assert_close, check_rows, decode_query, gqa_converted_layer, log, oracle_cache, rope_key_rows,
                        shape_of, torch_dtype)
from test_gpu_decode import run_decode_case
from test_gpu_paged import _fill, _np, _table, run_paged_case
from test_gpu_prefill import run_prefill_case

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize(
    "fmt,d_kv,r,rope_heads",
    [
        ("dense", 512, 4, 8),      # ring kernel, compact instance
        ("dense", 512, 2, 8),      # generic kernel
        ("dense", 256, 4, 8),      # generic kernel (the per-wave kernel takes per-head keys only)
        ("int4_g32", 512, 4, 8),   # register-staged kernel
        ("int4_g32", 512, 2, 16),  # register-staged kernel, pairs of query heads per key head
        ("int4_g32", 256, 4, 8),   # generic kernel
    ],
)
def test_compact_rope_decode(fmt, d_kv, r, rope_heads):
    cfg = scaled(CONFIGS[4] if fmt == "int4_g32" else CONFIGS[1], family="mid", batch=5, context=0, d_kv=d_kv,
                 r_pairs=r, cache_fmt=fmt)
    layer = gqa_converted_layer("gqa_mid", cfg.r_pairs, cfg.d_kv, cfg.dtype)
    run_decode_case(cfg, [700, 1, 0, 333, 64], 704, layer=layer, rope_heads=rope_heads)


def test_compact_rope_decode_per_head_layout_equal():
    """The same layer and sequences through per-query-head and compact RoPE caches: the attention reads the same
    key values either way, so the outputs are equal bit for bit (ring kernel, dense latent)."""
    from mla_latent_kv_cache_amd import LatentCache, decode, pack_weights

    cfg = scaled(CONFIGS[1], family="mid", batch=3, context=0)
    layer = gqa_converted_layer("gqa_mid", cfg.r_pairs, cfg.d_kv, cfg.dtype)
    lens, t_max = [515, 40, 129], 576
    outs = []
    for nrh in (0, 8):
        shape = shape_of(cfg, nrh)
        w = pack_weights(shape, layer, rope_len=t_max, theta=cfg.theta)
        cache = LatentCache.allocate(shape, len(lens), t_max, fill=float("nan"))
        xs = [synth.context_x(cfg, b, L) for b, L in enumerate(lens)]
        _fill(cfg, layer, w, cache, lens, 0, xs)
        q = np.stack([decode_query(cfg, layer, x[-1]) for x in xs])
        qt = torch.from_numpy(q.astype(np.float32)).cuda().to(torch_dtype(cfg))
        outs.append(decode(w, cache, qt, torch.tensor(lens, dtype=torch.int32, device="cuda"), max(lens)))
        torch.cuda.synchronize()
    assert torch.equal(outs[0], outs[1]), "compact RoPE keys change the decode output"


@pytest.mark.parametrize("fmt", ["dense", "int4_g32"])
def test_compact_rope_decode_step(fmt):
    """mla_decode_step on a compact cache (the new rows' RoPE keys are formed inside the attention launch) equals
    mla_cache_append_ws + mla_decode bit for bit, writes the same cache rows, and matches the oracle."""
    from mla_latent_kv_cache_amd import LatentCache, append, append_ws, decode, decode_step, pack_weights

    cfg = scaled(CONFIGS[4] if fmt == "int4_g32" else CONFIGS[1], family="mid", batch=4, context=0)
    lens, t_max = [97, 2, 64, 200], 256
    log(f"[compact-rope decode-step] {fmt} lens={lens}")
    layer = gqa_converted_layer("gqa_mid", cfg.r_pairs, cfg.d_kv, cfg.dtype)
    shape = shape_of(cfg, 8)
    w = pack_weights(shape, layer, rope_len=t_max, theta=cfg.theta)
    caches = [LatentCache.allocate(shape, len(lens), t_max, fill=float("nan")) for _ in range(2)]
    xs = [synth.context_x(cfg, b, L) for b, L in enumerate(lens)]
    zero = torch.zeros(1, dtype=torch.int32, device="cuda")
    for cache in caches:
        for b, L in enumerate(lens):
            xt = torch.from_numpy(xs[b][: L - 1].astype(np.float32)).cuda().to(torch_dtype(cfg)).reshape(1, L - 1, -1)
            append(w, cache.view(b, b + 1), xt, zero, 0)
    x_new = torch.from_numpy(np.stack([x[-1] for x in xs])[:, None, :].astype(np.float32)).cuda().to(torch_dtype(cfg))
    start = torch.tensor([L - 1 for L in lens], dtype=torch.int32, device="cuda")
    lens_t = torch.tensor(lens, dtype=torch.int32, device="cuda")
    q = np.stack([decode_query(cfg, layer, x[-1]) for x in xs])
    qt = torch.from_numpy(q.astype(np.float32)).cuda().to(torch_dtype(cfg))
    out_step = decode_step(w, caches[0], x_new.contiguous(), start, max(lens) - 1, qt, lens_t, max(lens))
    append_ws(w, caches[1], x_new.contiguous(), start, max(lens) - 1)
    out_sep = decode(w, caches[1], qt, lens_t, max(lens))
    torch.cuda.synchronize()
    assert torch.equal(out_step, out_sep), "decode_step differs from append_ws + decode"
    same = lambda u, v: torch.equal(u.contiguous().view(torch.uint8), v.contiguous().view(torch.uint8))  # noqa: E731
    assert same(caches[0].ckv, caches[1].ckv) and same(caches[0].krope, caches[1].krope)
    got = _np(out_step)
    for b, L in enumerate(lens):
        c, kr = oracle_cache(cfg, layer, xs[b])
        check_rows(cfg, caches[0].krope[b, :L], rope_key_rows(kr, cfg.n_heads, 8), f"k_rope b={b}")
        if fmt == "int4_g32":
            c = oracle.dequant_int4(*oracle.quantize_int4_g32(c.astype(np.float32)))
        ref = oracle.decode_ref(q[b], c, kr, layer["w_uk"], layer["w_uv"], layer["pair_idx"], cfg.d_head, cfg.theta)
        rr, a = assert_close(got[b], ref, cfg.dtype, f"decode_step b={b}")
        log(f"  b={b} rel-L2={rr:.2e} max-abs={a:.2e}")


@pytest.mark.parametrize("fmt", ["dense", "int4_g32"])
def test_compact_rope_paged(fmt):
    """A paged pool of compact rows (the ring kernel's paged instance for the dense latent)."""
    base = CONFIGS[4] if fmt == "int4_g32" else CONFIGS[1]
    cfg = scaled(base, family="mid")
    layer = gqa_converted_layer("gqa_mid", cfg.r_pairs, cfg.d_kv, cfg.dtype)
    run_paged_case(base, "mid", 512, 4, [700, 1, 129, 0, 64], seed=21, name=f"compact-{fmt}", layer=layer,
                   rope_heads=8)


def test_compact_rope_multi_query():
    """Three queries per sequence decoded causally at once over a paged compact cache."""
    from mla_latent_kv_cache_amd import LatentCache, decode_multi, pack_weights

    prompts, steps, P, q_len = [500, 2, 70, 0], 3, 64, 3
    cfg = scaled(CONFIGS[1], family="mid", batch=len(prompts), context=0)
    lens = [p + steps for p in prompts]
    pps = (max(lens) + P - 1) // P
    log(f"[compact-rope multi-query] lens={lens}")
    layer = gqa_converted_layer("gqa_mid", cfg.r_pairs, cfg.d_kv, cfg.dtype)
    shape = shape_of(cfg, 8)
    w = pack_weights(shape, layer, rope_len=pps * P, theta=cfg.theta)
    table, n_pages = _table(len(prompts), pps, 5, seed=9)
    cache = LatentCache.allocate_paged(shape, table, P, n_pages, fill=float("nan"))
    xs = [synth.context_x(cfg, b, L) for b, L in enumerate(lens)]
    _fill(cfg, layer, w, cache, prompts, steps, xs)
    q = np.zeros((len(prompts), q_len, cfg.n_heads, cfg.d_head))
    for b, L in enumerate(lens):
        for i in range(q_len):
            if L - q_len + i >= 0:
                q[b, i] = decode_query(cfg, layer, xs[b][L - q_len + i])
    qt = torch.from_numpy(q.astype(np.float32)).cuda().to(torch_dtype(cfg)).contiguous()
    out = decode_multi(w, cache, qt, torch.tensor(lens, dtype=torch.int32, device="cuda"), max(lens))
    torch.cuda.synchronize()
    got = _np(out)
    for b, L in enumerate(lens):
        c, kr = oracle_cache(cfg, layer, xs[b])
        ref = oracle.multi_query_decode_ref(q[b], c, kr, layer["w_uk"], layer["w_uv"], layer["pair_idx"], cfg.d_head,
                                            cfg.theta)
        for i in range(q_len):
            if L - q_len + i < 0:
                assert np.all(got[b, i] == 0)
                continue
            assert_close(got[b, i], ref[i], cfg.dtype, f"multi-query b={b} i={i}")


@pytest.mark.parametrize("rope_heads", [8, 16])
def test_compact_rope_prefill(rope_heads):
    cfg = scaled(CONFIGS[2], family="mid")
    layer = gqa_converted_layer("gqa_mid", cfg.r_pairs, cfg.d_kv, cfg.dtype)
    run_prefill_case(cfg, S=300, B=2, layer=layer, rope_heads=rope_heads)
