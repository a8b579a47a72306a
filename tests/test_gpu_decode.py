"""GPU parity of mla_cache_append + mla_decode against the oracle, through the C ABI.

Small cases (seconds of oracle work) span several 32-token tiles, several splits, ragged tails, a
one-token and an empty sequence, and NaN-filled cache rows past every sequence's length (a kernel that
read them would return NaN).  Full-size cases check sampled sequences at the task's shapes."""

import numpy as np
import pytest
import torch

import oracle
import synth
from synth import CONFIGS, scaled

from parity_lib import (assert_close, assert_finite, check_int4_cache, check_rows, converted_layer, decode_query,
                        fill_cache_per_sequence, log, max_abs, oracle_cache, rel_l2, rope_key_rows, shape_of,
                        torch_dtype)

pytestmark = pytest.mark.gpu


def _to_np(t):
    return t.float().cpu().numpy().astype(np.float64)


def run_decode_case(cfg, lens, t_max, sample=None, check_cache=True, repeat_bitwise=True, variant=("2-norm", "joint"),
                    layer=None, rope_heads=0):
    from mla_latent_kv_cache_amd import LatentCache, decode, pack_weights

    log(f"[decode] {cfg.name} family={cfg.family} d_kv={cfg.d_kv} r={cfg.r_pairs} fmt={cfg.cache_fmt} "
        f"B={len(lens)} lens={list(lens)[:8]} t_max={t_max} conversion={variant if layer is None else 'given'} "
        f"rope_heads={rope_heads or cfg.n_heads}")
    B = len(lens)
    if layer is None:
        layer = converted_layer(cfg.family, cfg.r_pairs, cfg.d_kv, cfg.dtype, *variant)
    shape = shape_of(cfg, rope_heads)
    w = pack_weights(shape, layer, rope_len=t_max, theta=cfg.theta)
    cache = LatentCache.allocate(shape, B, t_max, fill=float("nan"))
    if cache.ckv_scale is not None:
        cache.ckv_scale.fill_(float("nan"))
    sample = list(range(B)) if sample is None else list(sample)
    # activations are regenerated from their seeds when checked unless the batch is small (full-size batches
    # would hold gigabytes of them)
    keep = sample if sum(int(lens[b]) for b in sample) * cfg.d_model <= (1 << 28) else ()
    xs, last = fill_cache_per_sequence(cfg, layer, w, cache, lens, keep_x=keep)

    rng = np.random.default_rng(7)
    q = np.zeros((B, cfg.n_heads, cfg.d_head))
    for b in range(B):
        if b in last:
            q[b] = decode_query(cfg, layer, last[b])
        else:
            q[b] = synth.round_to_device(rng.standard_normal((cfg.n_heads, cfg.d_head)), cfg.dtype)
    qt = torch.from_numpy(q.astype(np.float32)).to("cuda").to(torch_dtype(cfg))
    lens_t = torch.tensor(np.asarray(lens, dtype=np.int32), device="cuda")
    max_len = int(max(lens)) if len(lens) else 0
    out = decode(w, cache, qt, lens_t, max_len)
    torch.cuda.synchronize()
    assert_finite(out, "decode out")
    got = _to_np(out)
    if repeat_bitwise:
        out2 = decode(w, cache, qt, lens_t, max_len)
        torch.cuda.synchronize()
        assert torch.equal(out, out2), "decode is not bitwise deterministic"

    results = []
    err2 = ref2 = 0.0
    for b in sample:
        L = int(lens[b])
        if L == 0:
            assert np.all(got[b] == 0.0), "empty sequence must give a zero output row"
            continue
        x = xs[b] if b in xs else synth.context_x(cfg, b, L)
        c, kr = oracle_cache(cfg, layer, x)
        del x
        if cfg.cache_fmt == "int4_g32":
            codes = oracle.unpack_nibbles(cache.ckv[b, :L].cpu().numpy())
            scales = cache.ckv_scale[b, :L].cpu().numpy()
            check_int4_cache(c, codes, scales, f"int4 b={b}")
            oc, osc = oracle.quantize_int4_g32(c.astype(np.float32))
            c_used = oracle.dequant_int4(oc, osc)  # attention over the oracle's own dequantised cache
        else:
            c_used = c
            if check_cache:
                check_rows(cfg, cache.ckv[b, :L], c, f"c_kv b={b}")
        if check_cache and cfg.r_pairs > 0:
            check_rows(cfg, cache.krope[b, :L], rope_key_rows(kr, cfg.n_heads, rope_heads), f"k_rope b={b}")
        ref = oracle.decode_ref(q[b], c_used, kr, layer["w_uk"], layer["w_uv"], layer["pair_idx"], cfg.d_head, cfg.theta)
        r, a = assert_close(got[b], ref, cfg.dtype, f"decode out b={b} L={L}")
        err2 += float(np.sum((got[b] - ref) ** 2))
        ref2 += float(np.sum(ref ** 2))
        results.append((b, L, r, a))
        log(f"  b={b} L={L} rel-L2={r:.2e} max-abs={a:.2e}")
    if len(sample) == B and results:
        # the contract over the whole output tensor (empty sequences' zero rows included above)
        r_all = float(np.sqrt(err2 / ref2)) if ref2 > 0 else 0.0
        a_all = max(a for _, _, _, a in results)
        assert r_all <= (1e-5 if cfg.dtype == "f32" else 5e-3), f"whole-tensor rel-L2 {r_all:.3e}"
        log(f"  whole output [{B}, {cfg.n_heads}, {cfg.d_head}]: rel-L2 {r_all:.2e}, max-abs {a_all:.2e}")
    return results


# ------------------------------------------------------------------ small cases

def test_tiny_f32_config_exact_shape():
    """The tiny fp32 configuration as specified: batch 1, context 256."""
    run_decode_case(CONFIGS[0], [256], 256)


def test_tiny_f32_ragged():
    run_decode_case(CONFIGS[0], [256, 1, 100, 0, 65], 300)


def test_tiny_bf16_generic_path():
    cfg = scaled(CONFIGS[0], dtype="bf16")
    run_decode_case(cfg, [200, 57, 1], 256)


@pytest.mark.parametrize("d_kv,r", [(512, 4), (256, 2)])
def test_odd_heads_bf16_generic_attention_combine(d_kv, r):
    """Five heads: the generic attention kernel writes fp32 split results, which the one-launch merge and
    W_uv projection reads (the MFMA kernels write the fp16 form); ragged lengths across several splits."""
    cfg = scaled(CONFIGS[1], family="odd", batch=4, d_kv=d_kv, r_pairs=r)
    run_decode_case(cfg, [700, 1, 129, 0], 768)


def test_head_dim_80_single_part_combine():
    """d_head 80: five 16-wide output blocks, so the combine projects each head in one part; one long
    sequence on the generic kernel gives 63 fp32 split results, which the combine's 8 waves merge in
    groups of 4 (two groups per wave, the waves' states met in LDS)."""
    cfg = scaled(CONFIGS[1], family="head80", batch=1, d_kv=256, r_pairs=2)
    run_decode_case(cfg, [4000], 4096)


def test_mid_bf16_dkv512_r4():
    cfg = scaled(CONFIGS[1], family="mid", batch=5)
    run_decode_case(cfg, [1000, 1, 0, 333, 64], 1024)


def test_mid_bf16_dkv256_r2():
    cfg = scaled(CONFIGS[3], family="mid", batch=4, ctx_range=None)
    run_decode_case(cfg, [2000, 777, 31, 1500], 2048)


def test_mid_bf16_dkv512_r2():
    cfg = scaled(CONFIGS[1], family="mid", batch=3, r_pairs=2)
    run_decode_case(cfg, [700, 33, 96], 768)


def test_mid_bf16_dkv256_r4():
    cfg = scaled(CONFIGS[3], family="mid", batch=3, r_pairs=4, ctx_range=None)
    run_decode_case(cfg, [129, 1200, 64], 1280)


def test_mid_bf16_many_sequences():
    """More sequences than one wave scans at once (the work split walks the batch 64 lengths at a time),
    lengths from 0 to 300, so that work items of one sequence straddle those groups."""
    cfg = scaled(CONFIGS[1], family="mid", batch=70)
    lens = np.random.default_rng(11).integers(0, 301, size=70)
    lens[[3, 64]] = 0
    lens[[5, 65]] = 1
    sample = sorted({0, 1, 5, 63, 64, 65, 69, int(np.argmax(lens))})
    run_decode_case(cfg, [int(v) for v in lens], 320, sample=sample)


@pytest.mark.parametrize("d_kv,r", [(512, 2), (256, 4), (256, 2)])
def test_mid_int4_shapes(d_kv, r):
    """The other int4 latent shapes of the per-wave kernel (latent width 256 / 512, 2 or 4 pairs)."""
    cfg = scaled(CONFIGS[4], family="mid", batch=3, d_kv=d_kv, r_pairs=r)
    run_decode_case(cfg, [700, 17, 130], 768)


def test_mid_short_ragged_lengths():
    """Lengths around the 16-token tile and the per-wave quarters of a work item (latent width 256)."""
    cfg = scaled(CONFIGS[3], family="mid", batch=13, ctx_range=None)
    lens = [1, 2, 15, 16, 17, 31, 33, 63, 64, 65, 127, 200, 513]
    run_decode_case(cfg, lens, 520, sample=[0, 2, 3, 4, 6, 9, 11, 12])


@pytest.mark.parametrize("strategy,svd,fmt", [("high", "split", "dense"), ("low", "joint", "dense"),
                                              ("uniform", "split", "int4_g32")])
def test_ablation_variant_layers(strategy, svd, fmt):
    """Layers converted with the pages' ablation variants (fixed partial-RoPE subspaces, SVD_split at the same
    latent width) run through the same append and decode kernels; SVD_split leaves half of each
    up-projection zero."""
    cfg = scaled(CONFIGS[1], family="mid", batch=3, context=0, cache_fmt=fmt)
    run_decode_case(cfg, [700, 33, 260], 704, variant=(strategy, svd))


@pytest.mark.parametrize("fmt", ["dense", "int4_g32"])
def test_gqa_source_layer(fmt):
    """A layer converted from a grouped-query source (32 query heads, 8 KV heads, Llama head shapes) runs
    through the same append and decode kernels: every head of a group shares its subspaces and maps."""
    from parity_lib import gqa_converted_layer

    cfg = scaled(CONFIGS[1], family="mid", batch=3, context=0, cache_fmt=fmt)
    layer = gqa_converted_layer("gqa_mid", cfg.r_pairs, cfg.d_kv, cfg.dtype)
    run_decode_case(cfg, [640, 1, 333], 640, layer=layer)


def test_mid_int4():
    cfg = scaled(CONFIGS[4], family="mid", batch=4)
    run_decode_case(cfg, [1000, 65, 512, 3], 1024)


def test_quantize_int4_bit_exact():
    from mla_latent_kv_cache_amd import quantize_int4

    rng = np.random.default_rng(11)
    x = (rng.standard_normal((4096, 32)) * rng.uniform(1e-4, 50, (4096, 1))).astype(np.float32)
    # exact ties x/s = k + 1/2 with s = 0.25, absmax elements, zero groups, fp16-subnormal scales
    x[0] = 0
    x[1, :] = np.float32(0.125) * np.arange(-16, 16, dtype=np.float32) / 2
    x[1, 0] = np.float32(1.75)
    x[2] = rng.standard_normal(32).astype(np.float32) * np.float32(1e-6)
    x[3] = -x[3]
    x[4] = np.float32(7 * 2.0 ** -20)
    x[5] = np.float32(1e-9)
    codes_g, scales_g = quantize_int4(torch.from_numpy(x).cuda())
    torch.cuda.synchronize()
    codes_o, scales_o = oracle.quantize_int4_g32(x)
    np.testing.assert_array_equal(scales_g.cpu().numpy().view(np.uint16).reshape(-1),
                                  scales_o.view(np.uint16).reshape(-1))
    np.testing.assert_array_equal(codes_g.cpu().numpy(), oracle.pack_nibbles(codes_o))


# ------------------------------------------------------------------ full-size cases (every sequence)

@pytest.mark.slow
@pytest.mark.timeout(900)
def test_full_llama_bf16_decode_b32_l4096():
    cfg = CONFIGS[1]
    run_decode_case(cfg, synth.seq_lens(cfg), cfg.context)


@pytest.mark.slow
@pytest.mark.timeout(900)
def test_full_llama_longctx_decode():
    cfg = CONFIGS[3]
    lens = synth.seq_lens(cfg)
    run_decode_case(cfg, lens, int(lens.max()))


@pytest.mark.slow
@pytest.mark.timeout(1200)
def test_full_llama_int4_decode_b64_l8192():
    cfg = CONFIGS[4]
    run_decode_case(cfg, synth.seq_lens(cfg), cfg.context, repeat_bitwise=False)


@pytest.mark.parametrize("variant,use_ws", [("bf16", False), ("bf16", True), ("int4", False), ("int4", True),
                                             ("f32", False)])
def test_step_append_batched_positions(variant, use_ws):
    """A decode step's append: one new token per sequence, each at its own position, in one call (with and
    without the workspace that splits the down-projection over the model width)."""
    from mla_latent_kv_cache_amd import LatentCache, append, append_ws, pack_weights

    if variant == "f32":
        cfg = scaled(CONFIGS[0], batch=4)
    elif variant == "int4":
        cfg = scaled(CONFIGS[4], family="mid", batch=4)
    else:
        cfg = scaled(CONFIGS[1], family="mid", batch=4)
    lens = [97, 2, 64, 200]
    t_max = 256
    log(f"[step-append] {variant} ws={use_ws} lens={lens}")
    layer = converted_layer(cfg.family, cfg.r_pairs, cfg.d_kv, cfg.dtype)
    shape = shape_of(cfg)
    w = pack_weights(shape, layer, rope_len=t_max, theta=cfg.theta)
    cache = LatentCache.allocate(shape, len(lens), t_max, fill=float("nan"))
    xs = [synth.context_x(cfg, b, L) for b, L in enumerate(lens)]
    zero = torch.zeros(1, dtype=torch.int32, device="cuda")
    for b, L in enumerate(lens):
        xt = torch.from_numpy(xs[b][: L - 1].astype(np.float32)).cuda().to(torch_dtype(cfg)).reshape(1, L - 1, -1)
        view = cache.view(b, b + 1)
        append(w, view, xt, zero, 0)
    x_new = np.stack([x[-1] for x in xs])[:, None, :]
    start = torch.tensor([L - 1 for L in lens], dtype=torch.int32, device="cuda")
    xn = torch.from_numpy(x_new.astype(np.float32)).cuda().to(torch_dtype(cfg)).contiguous()
    if use_ws:
        append_ws(w, cache, xn, start, max(lens) - 1)
    else:
        append(w, cache, xn, start, max(lens) - 1)
    torch.cuda.synchronize()
    for b, L in enumerate(lens):
        c, kr = oracle_cache(cfg, layer, xs[b])
        check_rows(cfg, cache.krope[b, :L], kr, f"k_rope b={b}")
        if variant == "int4":
            check_int4_cache(c, oracle.unpack_nibbles(cache.ckv[b, :L].cpu().numpy()), cache.ckv_scale[b, :L].cpu().numpy(),
                             f"int4 b={b}")
        else:
            check_rows(cfg, cache.ckv[b, :L], c, f"c_kv b={b}")
        # rows past the sequence were never written
        if L < t_max and variant != "int4":
            assert torch.isnan(cache.ckv[b, L:].float()).all()


@pytest.mark.parametrize("variant", ["bf16", "int4", "f32"])
def test_decode_step_matches_separate_calls(variant):
    """mla_decode_step (append + decode with the fused prologue) equals mla_cache_append_ws followed by
    mla_decode bit for bit, and the oracle within tolerance (f32 takes the unfused path)."""
    from mla_latent_kv_cache_amd import LatentCache, append, append_ws, decode, decode_step, pack_weights

    if variant == "f32":
        cfg = scaled(CONFIGS[0], batch=4)
    elif variant == "int4":
        cfg = scaled(CONFIGS[4], family="mid", batch=4)
    else:
        cfg = scaled(CONFIGS[1], family="mid", batch=4)
    lens = [97, 2, 64, 200]
    t_max = 256
    log(f"[decode-step] {variant} lens={lens}")
    layer = converted_layer(cfg.family, cfg.r_pairs, cfg.d_kv, cfg.dtype)
    shape = shape_of(cfg)
    w = pack_weights(shape, layer, rope_len=t_max, theta=cfg.theta)
    caches = [LatentCache.allocate(shape, len(lens), t_max, fill=float("nan")) for _ in range(2)]
    xs = [synth.context_x(cfg, b, L) for b, L in enumerate(lens)]
    zero = torch.zeros(1, dtype=torch.int32, device="cuda")
    for cache in caches:
        for b, L in enumerate(lens):
            xt = torch.from_numpy(xs[b][: L - 1].astype(np.float32)).cuda().to(torch_dtype(cfg)).reshape(1, L - 1, -1)
            view = cache.view(b, b + 1)
            append(w, view, xt, zero, 0)
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
    def same_bits(u, v):  # the unwritten rows hold NaN, which == never matches
        return torch.equal(u.contiguous().view(torch.uint8), v.contiguous().view(torch.uint8))

    assert same_bits(caches[0].ckv, caches[1].ckv) and same_bits(caches[0].krope, caches[1].krope)
    got = _to_np(out_step)
    for b, L in enumerate(lens):
        c, kr = oracle_cache(cfg, layer, xs[b])
        if cfg.cache_fmt == "int4_g32":
            oc, osc = oracle.quantize_int4_g32(c.astype(np.float32))
            c = oracle.dequant_int4(oc, osc)
        ref = oracle.decode_ref(q[b], c, kr, layer["w_uk"], layer["w_uv"], layer["pair_idx"], cfg.d_head, cfg.theta)
        r, a = assert_close(got[b], ref, cfg.dtype, f"decode_step b={b}")
        log(f"  b={b} rel-L2={r:.2e} max-abs={a:.2e}")


@pytest.mark.parametrize("fmt", ["dense", "int4_g32"])
def test_running_max_raised_mid_item(fmt):
    """The first 32 rows of every 64-row block get a latent whose score is -20 for every head at once
    (minimum-norm solution of the 32 heads' absorbed queries, RoPE keys zero).  The work items here are 64
    rows long, so each item's first tile sets a very low running max and its second tile raises it by far
    more than the 2^8 headroom, mid-item: the owner waves' rescale factors and flags must reach every
    wave's accumulators, or the low tile's rows would weigh about e^20 too much."""
    from mla_latent_kv_cache_amd import LatentCache, decode, pack_weights, quantize_int4

    cfg = scaled(CONFIGS[4] if fmt == "int4_g32" else CONFIGS[1], family="mid", batch=3)
    lens, t_max = [600, 257, 130], 640
    log(f"[raise] fmt={fmt} lens={lens}")
    layer = converted_layer(cfg.family, cfg.r_pairs, cfg.d_kv, cfg.dtype)
    shape = shape_of(cfg)
    w = pack_weights(shape, layer, rope_len=t_max, theta=cfg.theta)
    cache = LatentCache.allocate(shape, len(lens), t_max, fill=0.0)
    _, last = fill_cache_per_sequence(cfg, layer, w, cache, lens)
    q = np.stack([decode_query(cfg, layer, last[b]) for b in range(len(lens))])
    d_h = cfg.d_head
    qas = {}
    for b, L in enumerate(lens):
        qa = qas[b] = np.zeros((cfg.n_heads, cfg.d_kv))  # absorbed queries W_uk,h q_nope(h)
        for h in range(cfg.n_heads):
            kept = {2 * int(p_) + c for p_ in layer["pair_idx"][h] for c in (0, 1)}
            nope = [i for i in range(d_h) if i not in kept]
            qa[h] = layer["w_uk"][h] @ q[b, h, nope]
        c_low = qa.T @ np.linalg.solve(qa @ qa.T, -20.0 * np.sqrt(d_h) * np.ones(cfg.n_heads))
        rows = torch.tensor([t for t in range(L) if t % 64 < 32], device="cuda")
        cl = torch.from_numpy(c_low.astype(np.float32)).cuda()
        if fmt == "int4_g32":
            codes, scales = quantize_int4(cl[None].contiguous())
            cache.ckv[b, rows] = codes[0]
            cache.ckv_scale[b, rows] = scales[0]
        else:
            cache.ckv[b, rows] = cl.to(torch.bfloat16)
        cache.krope[b, rows] = 0
    lens_t = torch.tensor(lens, dtype=torch.int32, device="cuda")
    qt = torch.from_numpy(q.astype(np.float32)).cuda().to(torch_dtype(cfg))
    got = _to_np(decode(w, cache, qt, lens_t, max(lens)))
    torch.cuda.synchronize()
    for b, L in enumerate(lens):
        if fmt == "int4_g32":
            c = oracle.dequant_int4(oracle.unpack_nibbles(cache.ckv[b, :L].cpu().numpy()), cache.ckv_scale[b, :L].cpu().numpy())
        else:
            c = _to_np(cache.ckv[b, :L])
        kr = _to_np(cache.krope[b, :L]).reshape(L, cfg.n_heads, -1)
        ref = oracle.decode_ref(q[b], c, kr, layer["w_uk"], layer["w_uv"], layer["pair_idx"], d_h, cfg.theta)
        r, a = assert_close(got[b], ref, cfg.dtype, f"raise b={b}")
        log(f"  b={b} rel-L2={r:.2e} max-abs={a:.2e}")
        # the stored low rows score far below the others for every head (NoPE part; their RoPE keys are 0)
        low = [t for t in range(L) if t % 64 < 32]
        assert (c[low] @ qas[b].T / np.sqrt(d_h) < -12.0).all()


@pytest.mark.parametrize("variant", ["bf16", "int4"])
def test_decode_step_new_row_inside_context(variant):
    """A step whose new token goes inside the decoded range (start = L - 3 for two sequences: the row is
    overwritten and two later rows stay in the context): the fused step's guess that the new rows end the
    sequence fails there and its general path runs; the result equals mla_cache_append_ws followed by
    mla_decode bit for bit, for the cache and the outputs."""
    from mla_latent_kv_cache_amd import LatentCache, append, append_ws, decode, decode_step, pack_weights

    cfg = scaled(CONFIGS[4], family="mid", batch=4) if variant == "int4" else scaled(CONFIGS[1], family="mid", batch=4)
    lens = [97, 40, 64, 200]
    starts = [94, 39, 61, 199]  # sequences 0 and 2 rewrite a row inside their context
    t_max = 256
    log(f"[decode-step-inside] {variant} lens={lens} starts={starts}")
    layer = converted_layer(cfg.family, cfg.r_pairs, cfg.d_kv, cfg.dtype)
    shape = shape_of(cfg)
    w = pack_weights(shape, layer, rope_len=t_max, theta=cfg.theta)
    caches = [LatentCache.allocate(shape, len(lens), t_max, fill=float("nan")) for _ in range(2)]
    xs = [synth.context_x(cfg, b, L) for b, L in enumerate(lens)]
    zero = torch.zeros(1, dtype=torch.int32, device="cuda")
    for cache in caches:
        for b, L in enumerate(lens):
            xt = torch.from_numpy(xs[b].astype(np.float32)).cuda().to(torch_dtype(cfg)).reshape(1, L, -1)
            append(w, cache.view(b, b + 1), xt, zero, 0)
    rng = np.random.default_rng(11)
    x_new = torch.from_numpy(rng.standard_normal((len(lens), 1, cfg.d_model)).astype(np.float32)).cuda().to(torch_dtype(cfg))
    start = torch.tensor(starts, dtype=torch.int32, device="cuda")
    lens_t = torch.tensor(lens, dtype=torch.int32, device="cuda")
    q = np.stack([decode_query(cfg, layer, x[-1]) for x in xs])
    qt = torch.from_numpy(q.astype(np.float32)).cuda().to(torch_dtype(cfg))
    before = [caches[0].krope[b, starts[b]].clone() for b in range(len(lens))]
    out_step = decode_step(w, caches[0], x_new.contiguous(), start, max(starts), qt, lens_t, max(lens))
    append_ws(w, caches[1], x_new.contiguous(), start, max(starts))
    out_sep = decode(w, caches[1], qt, lens_t, max(lens))
    torch.cuda.synchronize()
    assert torch.equal(out_step, out_sep), "decode_step differs from append_ws + decode"
    assert torch.equal(caches[0].ckv.contiguous().view(torch.uint8), caches[1].ckv.contiguous().view(torch.uint8))
    assert torch.equal(caches[0].krope.contiguous().view(torch.uint8), caches[1].krope.contiguous().view(torch.uint8))
    # every sequence's row at its start position was rewritten with the new token's keys
    for b in range(len(lens)):
        assert not torch.equal(caches[0].krope[b, starts[b]], before[b]), f"row {starts[b]} of sequence {b} unchanged"


@pytest.mark.parametrize("variant", ["wave_bf16", "wave_int4", "multi_bf16", "multi_int4"])
def test_decode_step_fused_rows(variant):
    """Decode steps whose append reduction runs inside the attention launch: the latent-256 per-wave kernel
    (bf16 and int4), and several new tokens per sequence with new rows in a first tile, straddling two work
    items, at the end of a range, and past a sequence's decode length (written by the extra workgroups).
    Output and cache rows equal mla_cache_append_ws followed by mla_decode bit for bit."""
    from mla_latent_kv_cache_amd import LatentCache, append, append_ws, decode, decode_step, pack_weights

    fmt = "int4_g32" if variant.endswith("int4") else "dense"
    if variant.startswith("wave"):
        cfg = scaled(CONFIGS[3], family="mid", batch=4, cache_fmt=fmt, ctx_range=None)
        t_new, ctx = 1, [300, 1, 77, 129]          # tokens already cached per sequence
        extra = [0, 0, 0, 0]                         # new rows past the decode length
    else:
        cfg = scaled(CONFIGS[1], family="mid", batch=5, cache_fmt=fmt)
        t_new, ctx = 3, [0, 61, 126, 250, 40]
        extra = [0, 0, 0, 0, 2]
    B = len(ctx)
    t_max = 320
    start = [c for c in ctx]
    lens = [c + t_new - e for c, e in zip(ctx, extra)]
    log(f"[decode-step-fused] {variant} ctx={ctx} t_new={t_new} lens={lens}")
    layer = converted_layer(cfg.family, cfg.r_pairs, cfg.d_kv, cfg.dtype)
    shape = shape_of(cfg)
    w = pack_weights(shape, layer, rope_len=t_max, theta=cfg.theta)
    caches = [LatentCache.allocate(shape, B, t_max, fill=float("nan")) for _ in range(2)]
    xs = [synth.context_x(cfg, b, c + t_new) for b, c in enumerate(ctx)]
    zero = torch.zeros(1, dtype=torch.int32, device="cuda")
    for cache in caches:
        if cache.ckv_scale is not None:
            cache.ckv_scale.fill_(float("nan"))
        for b, c in enumerate(ctx):
            if c == 0:
                continue
            xt = torch.from_numpy(xs[b][:c].astype(np.float32)).cuda().to(torch_dtype(cfg)).reshape(1, c, -1)
            view = cache.view(b, b + 1)
            append(w, view, xt, zero, 0)
    x_new = torch.from_numpy(np.stack([x[c:c + t_new] for x, c in zip(xs, ctx)]).astype(np.float32))
    x_new = x_new.cuda().to(torch_dtype(cfg)).contiguous()
    start_t = torch.tensor(start, dtype=torch.int32, device="cuda")
    lens_t = torch.tensor(lens, dtype=torch.int32, device="cuda")
    q = np.stack([decode_query(cfg, layer, x[c + t_new - 1]) for x, c in zip(xs, ctx)])
    qt = torch.from_numpy(q.astype(np.float32)).cuda().to(torch_dtype(cfg))
    out_step = decode_step(w, caches[0], x_new, start_t, max(start), qt, lens_t, max(lens))
    append_ws(w, caches[1], x_new, start_t, max(start))
    out_sep = decode(w, caches[1], qt, lens_t, max(lens))
    torch.cuda.synchronize()

    def same_bits(u, v):  # rows never written hold NaN, which == never matches
        return torch.equal(u.contiguous().view(torch.uint8), v.contiguous().view(torch.uint8))

    assert torch.equal(out_step, out_sep), "decode_step differs from append_ws + decode"
    assert same_bits(caches[0].ckv, caches[1].ckv) and same_bits(caches[0].krope, caches[1].krope)
    if caches[0].ckv_scale is not None:
        assert same_bits(caches[0].ckv_scale, caches[1].ckv_scale)
    # the new rows were written (not NaN) for every sequence, including rows past the decode length
    for b, c in enumerate(ctx):
        assert not torch.isnan(caches[0].krope[b, c:c + t_new].float()).any(), f"new RoPE rows of b={b} missing"


@pytest.mark.parametrize("variant", ["bf16", "int4", "f32"])
def test_decode_step_phases_match_the_step(variant):
    """mla_decode_step_phase 1, 2, 3 in order equals mla_decode_step bit for bit (outputs and cache rows), for
    the fused step (bf16, int4) and the unfused one (f32)."""
    from mla_latent_kv_cache_amd import BoundDecode, LatentCache, append, pack_weights

    if variant == "f32":
        cfg = scaled(CONFIGS[0], batch=3)
    elif variant == "int4":
        cfg = scaled(CONFIGS[4], family="mid", batch=3)
    else:
        cfg = scaled(CONFIGS[1], family="mid", batch=3)
    lens, t_max = [150, 3, 64], 160
    log(f"[decode-step-phases] {variant} lens={lens}")
    layer = converted_layer(cfg.family, cfg.r_pairs, cfg.d_kv, cfg.dtype)
    w = pack_weights(shape_of(cfg), layer, rope_len=t_max, theta=cfg.theta)
    caches = [LatentCache.allocate(shape_of(cfg), len(lens), t_max, fill=float("nan")) for _ in range(2)]
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
    outs = [torch.full_like(qt, float("nan")) for _ in range(2)]
    bd = [BoundDecode(w, caches[i], x_new.contiguous(), start, max(lens) - 1, qt, lens_t, max(lens), outs[i])
          for i in range(2)]
    bd[0].step()
    for p in (1, 2, 3):
        bd[1].step_phase(p)
    torch.cuda.synchronize()
    assert torch.equal(outs[0], outs[1]), "the step's phases differ from the step"
    for name in ("ckv", "krope"):
        a, b_ = getattr(caches[0], name), getattr(caches[1], name)
        assert torch.equal(a.contiguous().view(torch.uint8), b_.contiguous().view(torch.uint8)), name
    if cfg.cache_fmt == "dense":
        c, kr = oracle_cache(cfg, layer, xs[0])
        ref = oracle.decode_ref(q[0], c, kr, layer["w_uk"], layer["w_uv"], layer["pair_idx"], cfg.d_head, cfg.theta)
        assert_close(_to_np(outs[1])[0], ref, cfg.dtype, "phases b=0")
