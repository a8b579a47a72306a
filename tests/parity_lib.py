"""Shared setup for the GPU parity tests: seeded inputs (synth), the oracle's conversion and reference
results (oracle), and the library calls (mla_latent_kv_cache_amd) on identical rounded values."""

from __future__ import annotations

import functools
import sys

import numpy as np

import oracle
import synth
from synth import FAMILIES


def log(msg: str) -> None:
    print(msg, flush=True)
    sys.stdout.flush()


def rel_l2(got, ref) -> float:
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    den = np.linalg.norm(ref)
    return float(np.linalg.norm(got - ref) / (den if den > 0 else 1.0))


def max_abs(got, ref) -> float:
    return float(np.max(np.abs(np.asarray(got, dtype=np.float64) - np.asarray(ref, dtype=np.float64)))) if np.size(ref) else 0.0


# Tolerances fixed by the benchmark spec for this path.
BF16_REL, BF16_ABS = 5e-3, 2e-2
F32_REL = 1e-5


def assert_close(got, ref, dtype, what=""):
    r, a = rel_l2(got, ref), max_abs(got, ref)
    if dtype == "f32":
        assert r <= F32_REL, f"{what}: rel-L2 {r:.3e} > {F32_REL}"
    else:
        assert r <= BF16_REL and a <= BF16_ABS, f"{what}: rel-L2 {r:.3e} (<= {BF16_REL}), max-abs {a:.3e} (<= {BF16_ABS})"
    return r, a


@functools.lru_cache(maxsize=4)
def converted_layer(family: str, r: int, d_kv: int, dtype: str, strategy: str = "2-norm", svd: str = "joint"):
    """The oracle's conversion of the family's seeded layer, with every weight rounded to the device dtype
    (the GPU gets exactly these values; the oracle consumes them upcast to fp64).  strategy / svd select
    the pages' ablation variants (partial-RoPE strategy, joint or split SVD)."""
    d, n_h, d_h, _ = FAMILIES[family]
    wq, wk, wv, xc = synth.layer_weights(family)
    conv = oracle.convert_layer(wq, wk, wv, xc, n_h, d_h, r, d_kv, strategy=strategy, svd=svd)
    out = {k: synth.round_to_device(conv[k], dtype) for k in ("w_dkv", "w_krope", "w_uk", "w_uv")}
    out["pair_idx"] = conv["pair_idx"]
    out["w_q"] = wq
    out["sigma"] = conv.get("sigma")
    return out


@functools.lru_cache(maxsize=2)
def gqa_converted_layer(family: str, r: int, d_kv: int, dtype: str):
    """The oracle's conversion of a seeded grouped-query layer (synth.GQA_FAMILIES), expanded per query head
    and rounded to the device dtype like converted_layer."""
    d, n_h, n_kv, d_h, _ = synth.GQA_FAMILIES[family]
    wq, wk, wv, xc = synth.gqa_layer_weights(family)
    conv = oracle.convert_gqa_layer(wq, wk, wv, xc, n_h, n_kv, d_h, r, d_kv)
    out = {k: synth.round_to_device(conv[k], dtype) for k in ("w_dkv", "w_krope", "w_uk", "w_uv")}
    out["pair_idx"] = conv["pair_idx"]
    out["w_q"] = wq
    out["sigma"] = conv["sigma"]
    return out


def shape_of(cfg):
    from mla_latent_kv_cache_amd import LayerShape

    return LayerShape(cfg.d_model, cfg.n_heads, cfg.d_head, cfg.r_pairs, cfg.d_kv, cfg.dtype, cfg.cache_fmt)


def torch_dtype(cfg):
    import torch

    return torch.bfloat16 if cfg.dtype == "bf16" else torch.float32


def fill_cache_per_sequence(cfg, layer, w, cache, lens, keep_x=()):
    """Append every sequence's seeded activations (positions 0..L_b-1) one sequence at a time through
    mla_cache_append on a one-sequence view of the cache.  Returns ({b: x_b} for b in keep_x,
    {b: last activation row} for every non-empty sequence)."""
    import torch

    from mla_latent_kv_cache_amd import LatentCache, append

    kept, last = {}, {}
    zero = torch.zeros(1, dtype=torch.int32, device="cuda")
    for b, L in enumerate(lens):
        L = int(L)
        if L == 0:
            continue
        x = synth.context_x(cfg, b, L)
        last[b] = x[-1].copy()
        if b in keep_x:
            kept[b] = x
        xt = torch.from_numpy(x.astype(np.float32)).to("cuda").to(torch_dtype(cfg)).reshape(1, L, cfg.d_model)
        view = cache.view(b, b + 1)
        append(w, view, xt, zero, 0)
        del xt
        if b % 8 == 7:
            log(f"    filled {b + 1}/{len(lens)} sequences")
    torch.cuda.synchronize()
    return kept, last


def oracle_cache(cfg, layer, x):
    """Oracle cache rows (c_kv fp64, k_rope fp64) of one sequence's activations at positions 0..L-1."""
    return oracle.append_ref(x, layer["w_dkv"], layer["w_krope"], layer["pair_idx"], np.arange(x.shape[0]),
                             cfg.d_head, cfg.theta)


def decode_query(cfg, layer, x_last):
    """Raw query of the decode token (the sequence's last token), rounded to the device dtype."""
    return synth.query_rows(x_last[None, :], layer["w_q"], cfg.dtype).reshape(cfg.n_heads, cfg.d_head)


def check_int4_cache(c, codes, scales):
    """GPU int4 codes against the oracle's codec applied to the oracle's fp32 latent.  The GPU quantises its
    own fp32 accumulator, which differs from the oracle's latent by accumulation order, so a code may differ
    only where the oracle's quotient lies within 1e-3 of a rounding boundary (or the absmax itself sits at an
    fp16 rounding boundary of the scale); every dequantised value stays within half a step of the latent."""
    c32 = c.astype(np.float32)
    oc, osc = oracle.quantize_int4_g32(c32)
    s_gpu = scales.astype(np.float32)
    assert np.all(np.isfinite(s_gpu))
    same_scale = s_gpu == osc.astype(np.float32)
    assert same_scale.mean() > 0.999, f"scales differ in {1 - same_scale.mean():.2e} of groups"
    g_codes = codes.reshape(codes.shape[0], -1, 32)
    o_codes = oc.reshape(oc.shape[0], -1, 32)
    quot = (c32.reshape(c.shape[0], -1, 32) / osc.astype(np.float32)[..., None])
    near = np.abs(np.abs(quot - np.floor(quot)) - 0.5) < 1e-3
    diff = (g_codes != o_codes) & same_scale[..., None]
    assert not np.any(diff & ~near), f"{np.count_nonzero(diff & ~near)} int4 codes differ away from a tie"
    deq = g_codes.astype(np.float64) * s_gpu[..., None]
    err = np.abs(deq - c.reshape(deq.shape))
    bound = s_gpu[..., None] * 0.5 + 1e-6 * np.abs(c.reshape(deq.shape)) + 1e-6
    assert np.all(err <= bound + s_gpu[..., None] * 1e-3)
    log(f"  int4: {np.count_nonzero(diff)} tie-adjacent code differences of {diff.size}")
