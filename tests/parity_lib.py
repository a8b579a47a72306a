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


def shape_of(cfg, rope_heads=0):
    from mla_latent_kv_cache_amd import LayerShape

    return LayerShape(cfg.d_model, cfg.n_heads, cfg.d_head, cfg.r_pairs, cfg.d_kv, cfg.dtype, cfg.cache_fmt,
                      rope_heads=rope_heads)


def rope_key_rows(kr, n_heads, rope_heads=0):
    """The oracle's RoPE keys [L, n_heads * 2r] (one key per query head) in the cache layout of `rope_heads` key
    heads: key head g is query head g * (n_heads / rope_heads), whose group all hold the same key."""
    kr = np.asarray(kr)
    if not rope_heads or rope_heads == n_heads:
        return kr
    L = kr.shape[0]
    k3 = kr.reshape(L, n_heads, -1)
    hpg = n_heads // rope_heads
    for g in range(rope_heads):  # the shared key is one key: every head of the group computes the same one
        assert np.array_equal(k3[:, g * hpg:(g + 1) * hpg], np.repeat(k3[:, g * hpg:g * hpg + 1], hpg, axis=1))
    return k3[:, ::hpg].reshape(L, -1)


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


# ---------------------------------------------------------------- exact checks of rounded and coded values
#
# The GPU forms every latent and pre-RoPE key as an fp32 sum of products of bf16 activations and bf16 weights:
# the products are exact in fp32, the sums are rounded in an order that depends on the kernel.  The oracle forms
# the same value c in fp64.  Each integer-valued decision taken on that value -- its bf16 rounding, an int4 scale
# and code, a 2-bit offset, scale and code -- is checked per element: the GPU's result must be what the decision
# gives for SOME value within acc_eps(c) = ACC_EPS * (1 + |c|) of the oracle's c.  Every decision here is
# monotone in its input (IEEE division and round-to-nearest-even are), so the possible results are exactly the
# range between the decisions at c - acc_eps(c) and c + acc_eps(c); no count or fraction of differing values is
# tolerated outside that range.  ACC_EPS = 2^-15 (3.1e-5): the latents and keys are about N(0, 1) per component,
# so the running sums stay within a few units and the fp32 accumulation error over the at most 4096 / 16 MFMA
# steps of a dot product is of order 2^-24 * 16 ~ 1e-6; the bound leaves a factor of about 30.
ACC_EPS = 2.0 ** -15


def acc_eps(c):
    return ACC_EPS * (1.0 + np.abs(np.asarray(c, dtype=np.float64)))


def _first(mask):
    return np.argwhere(mask)[:3].tolist()


def check_bf16_values(got, ref, what=""):
    """GPU bf16 values `got` (exact, any float array) against the oracle's fp64 values `ref` of the same shape:
    each must be the bf16 rounding (fp32 then bf16, nearest even) of a value within acc_eps of the oracle's.
    Returns the number of values rounded to the other neighbour at a rounding boundary."""
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert got.shape == ref.shape, f"{what}: shape {got.shape} != {ref.shape}"
    assert np.all(np.isfinite(got)), f"{what}: non-finite values at {_first(~np.isfinite(got))}"
    e = acc_eps(ref)
    b_lo = synth.round_to_device(ref - e, "bf16")
    b_hi = synth.round_to_device(ref + e, "bf16")
    bad = (got < b_lo) | (got > b_hi)
    assert not bad.any(), (f"{what}: {np.count_nonzero(bad)} bf16 values are no rounding of a value within the "
                           f"accumulation bound of the oracle's, first at {_first(bad)}: got {got[bad][:3]}, "
                           f"oracle {ref[bad][:3]}")
    n = int(np.count_nonzero(got != synth.round_to_device(ref, "bf16")))
    log(f"  {what}: bf16 values exact up to {n} of {got.size} rounded to the other neighbour at a boundary")
    return n


def check_int4_cache(c, codes, scales, what="int4", via_bf16=False):
    """GPU int4 codes [L, d_kv] (int8, unpacked) and fp16 scales [L, d_kv/32] against the oracle's fp64 latent c
    [L, d_kv].  The GPU quantises its own fp32 latent, which lies within acc_eps of c -- or, with via_bf16 (the
    windowed int4 format, which codes rows from their bf16 values), the bf16 rounding of that latent, which
    lies between bf16(c - acc_eps) and bf16(c + acc_eps).  So per group of 32: the GPU scale must lie between
    the codec's scales of the smallest and the largest absmax those inputs can have, and each code, under the
    GPU's scale, between the codec's codes at the lowest and the highest input.  Every dequantised value stays
    within half a step of some allowed input."""
    c = np.asarray(c, dtype=np.float64)
    L, D = c.shape
    g = c.reshape(L, D // 32, 32)
    e = acc_eps(g)
    lo, hi = g - e, g + e
    if via_bf16:
        lo, hi = synth.round_to_device(lo, "bf16"), synth.round_to_device(hi, "bf16")
    s_gpu = np.asarray(scales, dtype=np.float16).reshape(L, D // 32)
    k_gpu = np.asarray(codes, dtype=np.int8).reshape(L, D // 32, 32)
    assert np.all(np.isfinite(s_gpu.astype(np.float32))), f"{what}: non-finite scales"
    min_abs = np.where(lo > 0, lo, np.where(hi < 0, -hi, 0.0))
    max_abs = np.maximum(np.abs(lo), np.abs(hi))
    s_lo = oracle.int4_scale(np.max(min_abs, axis=-1).astype(np.float32))
    s_hi = oracle.int4_scale(np.max(max_abs, axis=-1).astype(np.float32))
    sg = s_gpu.astype(np.float32)
    bad_s = (sg < s_lo.astype(np.float32)) | (sg > s_hi.astype(np.float32))
    assert not bad_s.any(), (f"{what}: {np.count_nonzero(bad_s)} group scales are no scale of a latent within the "
                             f"accumulation bound, first at {_first(bad_s)}: got {sg[bad_s][:3]}, "
                             f"range [{s_lo[bad_s][:3]}, {s_hi[bad_s][:3]}]")
    k_lo = oracle.int4_codes(lo.astype(np.float32), s_gpu)
    k_hi = oracle.int4_codes(hi.astype(np.float32), s_gpu)
    bad_k = (k_gpu < k_lo) | (k_gpu > k_hi)
    assert not bad_k.any(), (f"{what}: {np.count_nonzero(bad_k)} codes are no code of a latent within the "
                             f"accumulation bound under the group's scale, first at {_first(bad_k)}")
    deq = k_gpu.astype(np.float64) * sg.astype(np.float64)[..., None]
    bound = 0.5 * sg.astype(np.float64)[..., None] + np.maximum(g - lo, hi - g)
    assert np.all(np.abs(deq - g) <= bound), f"{what}: a dequantised value is more than half a step from the latent"
    ref_in = synth.round_to_device(c, "bf16") if via_bf16 else c
    oc, osc = oracle.quantize_int4_g32(ref_in.astype(np.float32))
    n_s = int(np.count_nonzero(s_gpu.view(np.uint16) != osc.reshape(L, D // 32).view(np.uint16)))
    n_k = int(np.count_nonzero(k_gpu != oc.reshape(k_gpu.shape)))
    log(f"  {what}: scales exact up to {n_s} of {s_gpu.size} groups and codes up to {n_k} of {k_gpu.size} at "
        f"rounding boundaries within the accumulation bound")
    return n_s, n_k


def check_int2_codes(c, codes, meta, what="int2"):
    """GPU 2-bit codes [n, d_kv] (unpacked) and fp16 (s, z) [n, d_kv/32, 2] against the oracle's fp64 latent c
    [n, d_kv].  The GPU codes the bf16 rounding of its own fp32 latent; that bf16 value lies between
    b_lo = bf16(c - acc_eps) and b_hi = bf16(c + acc_eps).  Per group: z must lie between the codec's offsets
    of the smallest and largest group minimum those values allow, s (given the GPU's z) between the codec's
    scales of the smallest and largest maximum, and each code (given the GPU's s and z) between the codec's
    codes at b_lo and b_hi.  Dequantised values stay within half a step of those bf16 values, or within the
    offset's fp16 rounding of the group minimum."""
    c = np.asarray(c, dtype=np.float64)
    n, D = c.shape
    g = c.reshape(n, D // 32, 32)
    e = acc_eps(g)
    b_lo = synth.round_to_device(g - e, "bf16").astype(np.float32)
    b_hi = synth.round_to_device(g + e, "bf16").astype(np.float32)
    m = np.asarray(meta, dtype=np.float16).reshape(n, D // 32, 2)
    s_gpu, z_gpu = m[..., 0], m[..., 1]
    k_gpu = np.asarray(codes, dtype=np.uint8).reshape(n, D // 32, 32)
    zg, sg = z_gpu.astype(np.float32), s_gpu.astype(np.float32)
    assert np.all(np.isfinite(zg)) and np.all(np.isfinite(sg)), f"{what}: non-finite (s, z)"
    z_lo = oracle.int2.int2_offset(b_lo.min(axis=-1)).astype(np.float32)
    z_hi = oracle.int2.int2_offset(b_hi.min(axis=-1)).astype(np.float32)
    bad_z = (zg < z_lo) | (zg > z_hi)
    assert not bad_z.any(), f"{what}: {np.count_nonzero(bad_z)} offsets out of range, first at {_first(bad_z)}"
    s_lo = oracle.int2.int2_scale(b_lo.max(axis=-1), z_gpu).astype(np.float32)
    s_hi = oracle.int2.int2_scale(b_hi.max(axis=-1), z_gpu).astype(np.float32)
    bad_s = (sg < s_lo) | (sg > s_hi)
    assert not bad_s.any(), f"{what}: {np.count_nonzero(bad_s)} scales out of range, first at {_first(bad_s)}"
    k_lo = oracle.int2.int2_codes(b_lo, s_gpu, z_gpu)
    k_hi = oracle.int2.int2_codes(b_hi, s_gpu, z_gpu)
    bad_k = (k_gpu < k_lo) | (k_gpu > k_hi)
    assert not bad_k.any(), f"{what}: {np.count_nonzero(bad_k)} codes out of range, first at {_first(bad_k)}"
    deq = oracle.int2.dequant_int2(k_gpu, m).reshape(g.shape)
    step = np.maximum(0.5 * sg, 2.0 ** -11 * np.abs(zg)).astype(np.float64)[..., None] * (1 + 2.0 ** -10)
    far = np.maximum(np.maximum(b_lo - deq, deq - b_hi), 0.0)
    assert np.all(far <= step + 2.0 ** -23 * np.abs(deq)), f"{what}: a dequantised value is more than half a step away"
    c_bf = synth.round_to_device(c, "bf16").astype(np.float32)
    oc, om = oracle.int2.quantize_int2_g32(c_bf)
    n_m = int(np.count_nonzero(np.any(m.view(np.uint16) != om.reshape(m.shape).view(np.uint16), axis=-1)))
    n_k = int(np.count_nonzero(k_gpu != oc.reshape(k_gpu.shape)))
    log(f"  {what}: (s, z) exact up to {n_m} of {s_gpu.size} groups and codes up to {n_k} of {k_gpu.size} at bf16 "
        f"rounding boundaries within the accumulation bound")
    return n_m, n_k


def check_rows(cfg, got, ref, what=""):
    """Dense cache rows (c_kv or k_rope) from the GPU against the oracle's fp64 rows of the same shape (got may be
    a torch tensor): bf16 values exact up to accumulation-order roundings (check_bf16_values) and within the bf16
    contract; fp32 values within the fp32 contract."""
    g = got.float().cpu().numpy().astype(np.float64) if hasattr(got, "cpu") else np.asarray(got, dtype=np.float64)
    g = g.reshape(np.shape(ref))
    if cfg.dtype == "f32":
        assert np.all(np.isfinite(g)), f"{what}: non-finite values"
        return assert_close(g, ref, "f32", what)
    check_bf16_values(g, ref, what)
    return assert_close(g, ref, "bf16", what)


def assert_finite(t, what=""):
    """Every element of a GPU output tensor (torch or numpy) is finite."""
    a = t.float().cpu().numpy() if hasattr(t, "cpu") else np.asarray(t)
    assert np.all(np.isfinite(a)), f"{what}: {np.count_nonzero(~np.isfinite(a))} non-finite values"
