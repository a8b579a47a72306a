"""GPU parity of paged latent caches (a page table over a shared pool) and multi-query decode against the
oracle (oracle/paged.py), through the C ABI.

Every test fills a NaN-initialised pool through a random page table with spare pages, so that a read or a
write through a wrong page shows up.  Paged results must equal the same work on a contiguous cache bit for
bit (the kernels' arithmetic does not depend on where rows live) and the oracle within tolerance."""

import numpy as np
import pytest
import torch

import oracle
import synth
from synth import CONFIGS, scaled

from parity_lib import (assert_close, check_int4_cache, check_rows, converted_layer, decode_query, log, oracle_cache,
                        rope_key_rows, shape_of, torch_dtype)

pytestmark = pytest.mark.gpu


def _np(t):
    return t.float().cpu().numpy().astype(np.float64)


def _table(B, pps, spare, seed):
    """A page table [B, pps] drawing distinct pages from a pool of B * pps + spare pages, in random order."""
    n_pages = B * pps + spare
    perm = np.random.default_rng(seed).permutation(n_pages)[: B * pps].reshape(B, pps)
    return torch.from_numpy(perm.astype(np.int32)).cuda(), n_pages


def _fill(cfg, layer, w, cache, prompts, steps, xs):
    """Prompts one sequence at a time (views), then `steps` batched single-token appends (split-K path)."""
    from mla_latent_kv_cache_amd import append, append_ws

    zero = torch.zeros(1, dtype=torch.int32, device="cuda")
    B = len(prompts)
    for b, P in enumerate(prompts):
        if P:
            xt = torch.from_numpy(xs[b][:P].astype(np.float32)).cuda().to(torch_dtype(cfg)).reshape(1, P, -1)
            append(w, cache.view(b, b + 1), xt, zero, 0)
    for i in range(steps):
        xn = torch.from_numpy(np.stack([xs[b][prompts[b] + i] for b in range(B)])[:, None, :].astype(np.float32))
        xn = xn.cuda().to(torch_dtype(cfg)).contiguous()
        start = torch.tensor([prompts[b] + i for b in range(B)], dtype=torch.int32, device="cuda")
        append_ws(w, cache, xn, start, max(prompts) + i)


def _pool_rows(cache, b, L):
    """Rows 0..L-1 of sequence b gathered from a paged cache's pools (oracle.gather_pages on the GPU's data)."""
    tab = cache.block_table[b].cpu().numpy()
    P = cache.page_size
    flat = lambda t: t.reshape(-1, t.shape[-1]).cpu()  # noqa: E731
    ckv = oracle.gather_pages(flat(cache.ckv).float().numpy() if cache.ckv.dtype != torch.uint8 else flat(cache.ckv).numpy(),
                              tab, L, P)
    sc = None if cache.ckv_scale is None else oracle.gather_pages(flat(cache.ckv_scale).numpy(), tab, L, P)
    kr = oracle.gather_pages(flat(cache.krope).float().numpy(), tab, L, P)
    return ckv, sc, kr


CASES = {
    # name: (config, family, d_kv, r, prompts) -- the kernel each takes
    "dense512_dma": (CONFIGS[1], "mid", 512, 4, [700, 1, 129, 0, 64]),
    "int4_512_mfma": (CONFIGS[4], "mid", 512, 4, [700, 1, 129, 0, 64]),
    "dense256_wave": (CONFIGS[3], "mid", 256, 2, [700, 1, 129, 0, 64]),
    "int4_256_wave": (CONFIGS[4], "mid", 256, 2, [700, 1, 129, 0, 64]),
    "odd_generic": (CONFIGS[1], "odd", 512, 4, [300, 5, 0]),
}


@pytest.mark.parametrize("case", list(CASES))
def test_paged_append_and_decode(case):
    """Pool rows through the page table against the oracle's cache; decode equal to a contiguous cache bit for bit
    and to the oracle within tolerance."""
    run_paged_case(*CASES[case], seed=list(CASES).index(case) + 1, name=case)


def run_paged_case(base, family, d_kv, r, prompts, seed, name="", layer=None, rope_heads=0):
    from mla_latent_kv_cache_amd import LatentCache, decode, pack_weights

    cfg = scaled(base, family=family, d_kv=d_kv, r_pairs=r, batch=len(prompts), context=0, ctx_range=None)
    steps, P = 2, 64
    lens = [p + steps for p in prompts]
    pps = (max(lens) + P - 1) // P
    t_max = pps * P
    log(f"[paged] {name} prompts={prompts} page={P} pages/seq={pps} rope_heads={rope_heads or cfg.n_heads}")
    if layer is None:
        layer = converted_layer(cfg.family, cfg.r_pairs, cfg.d_kv, cfg.dtype)
    shape = shape_of(cfg, rope_heads)
    w = pack_weights(shape, layer, rope_len=t_max, theta=cfg.theta)
    table, n_pages = _table(len(prompts), pps, 7, seed=seed)
    paged = LatentCache.allocate_paged(shape, table, P, n_pages, fill=float("nan"))
    contig = LatentCache.allocate(shape, len(prompts), t_max, fill=float("nan"))
    xs = [synth.context_x(cfg, b, L) for b, L in enumerate(lens)]
    for cache in (paged, contig):
        _fill(cfg, layer, w, cache, prompts, steps, xs)
    q = np.stack([decode_query(cfg, layer, x[-1]) for x in xs])
    qt = torch.from_numpy(q.astype(np.float32)).cuda().to(torch_dtype(cfg))
    lens_t = torch.tensor(lens, dtype=torch.int32, device="cuda")
    out_p = decode(w, paged, qt, lens_t, max(lens))
    out_c = decode(w, contig, qt, lens_t, max(lens))
    torch.cuda.synchronize()
    assert torch.equal(out_p, out_c), "paged decode differs from the contiguous one"
    got = _np(out_p)
    for b, L in enumerate(lens):
        c, kr = oracle_cache(cfg, layer, xs[b])
        ckv, sc, krg = _pool_rows(paged, b, L)
        check_rows(cfg, krg.reshape(L, shape.n_rope_heads, -1), rope_key_rows(kr, cfg.n_heads, rope_heads).reshape(
            L, shape.n_rope_heads, -1), f"pool k_rope b={b}")
        if cfg.cache_fmt == "int4_g32":
            check_int4_cache(c, oracle.unpack_nibbles(ckv), sc, f"pool int4 b={b}")
            oc, osc = oracle.quantize_int4_g32(c.astype(np.float32))
            c = oracle.dequant_int4(oc, osc)
        else:
            check_rows(cfg, ckv, c, f"pool c_kv b={b}")
        ref = oracle.decode_ref(q[b], c, kr, layer["w_uk"], layer["w_uv"], layer["pair_idx"], cfg.d_head, cfg.theta)
        rr, a = assert_close(got[b], ref, cfg.dtype, f"decode b={b} L={L}")
        log(f"  b={b} L={L} rel-L2={rr:.2e} max-abs={a:.2e}")


@pytest.mark.parametrize("fmt", ["dense", "int4_g32", "int4_g32_win", "int2_g32_win"])
def test_paged_prefill(fmt):
    """Prefill over a paged cache (quantised latents dequantised through the page table first; the windowed
    formats take their last 128 rows from the per-sequence ring)."""
    from mla_latent_kv_cache_amd import LatentCache, append, pack_weights, prefill
    from oracle import int2

    cfg = scaled(CONFIGS[2], family="mid", cache_fmt=fmt)
    B, S, P = 2, 300, 64
    pps = (S + P - 1) // P
    log(f"[paged-prefill] {fmt} B={B} S={S} page={P}")
    layer = converted_layer(cfg.family, cfg.r_pairs, cfg.d_kv, cfg.dtype)
    shape = shape_of(cfg)
    w = pack_weights(shape, layer, rope_len=pps * P, theta=cfg.theta)
    table, n_pages = _table(B, pps, 3, seed=11)
    cache = LatentCache.allocate_paged(shape, table, P, n_pages, fill=float("nan"))
    xs = [synth.context_x(cfg, b, S) for b in range(B)]
    x = torch.from_numpy(np.stack(xs).astype(np.float32)).cuda().to(torch_dtype(cfg))
    append(w, cache, x, torch.zeros(B, dtype=torch.int32, device="cuda"), 0)
    qs = [synth.query_rows(xb, layer["w_q"], cfg.dtype).reshape(S, cfg.n_heads, cfg.d_head) for xb in xs]
    q = torch.from_numpy(np.stack(qs).astype(np.float32)).cuda().to(torch_dtype(cfg))
    out = prefill(w, cache, q)
    torch.cuda.synchronize()
    got = _np(out)
    for b in range(B):
        c, kr = oracle.append_ref(xs[b], layer["w_dkv"], layer["w_krope"], layer["pair_idx"], np.arange(S), cfg.d_head,
                                  cfg.theta)
        if fmt == "int4_g32":
            c = oracle.dequant_int4(*oracle.quantize_int4_g32(c.astype(np.float32)))
        elif fmt == "int4_g32_win":
            c = oracle.windowed_latent_int4(synth.round_to_device(c, "bf16"), 128)[0]
        elif fmt == "int2_g32_win":
            c = int2.windowed_latent(synth.round_to_device(c, "bf16"), 128)[0]
        ref = oracle.prefill_ref(qs[b], c, kr, layer["w_uk"], layer["w_uv"], layer["pair_idx"], cfg.d_head, cfg.theta)
        rr, a = assert_close(got[b], ref, cfg.dtype, f"paged prefill b={b}")
        log(f"  b={b} rel-L2={rr:.2e} max-abs={a:.2e}")


@pytest.mark.parametrize("fmt,paged,q_len,W,fam", [("dense", False, 4, 0, "mid"), ("dense", True, 3, 0, "mid"),
                                                  ("int4_g32", True, 2, 0, "mid"), ("dense", False, 1, 0, "mid"),
                                                  ("int4_g32_win", False, 4, 128, "mid"),
                                                  ("int2_g32_win", True, 3, 64, "mid"),
                                                  ("int4_g32_win", True, 2, 64, "mid"),
                                                  ("int2_g32_win", False, 3, 64, "odd")])
def test_multi_query_decode(fmt, paged, q_len, W, fam):
    """q_len new tokens of each sequence decoded at once, each causally (sequence lengths below, at and above
    q_len); equal to the oracle's multi-query decode, and for q_len = 1 to mla_decode bit for bit.  With a
    window of W bf16 rows (windowed formats) the ring holds the last W appended positions of every sequence, so
    the queries see the same coded rows and ring rows up to their own positions."""
    from mla_latent_kv_cache_amd import LatentCache, decode, decode_multi, pack_weights
    from oracle import int2

    base = CONFIGS[4] if fmt != "dense" else CONFIGS[1]
    prompts = [500, 2, 70, 0]
    cfg = scaled(base, family=fam, batch=len(prompts), context=0, cache_fmt=fmt)
    steps, P = 3, 64
    lens = [p + steps for p in prompts]
    pps = (max(lens) + P - 1) // P
    log(f"[multi-query] fmt={fmt} paged={paged} q_len={q_len} W={W} family={fam} lens={lens}")
    layer = converted_layer(cfg.family, cfg.r_pairs, cfg.d_kv, cfg.dtype)
    shape = shape_of(cfg)
    w = pack_weights(shape, layer, rope_len=pps * P, theta=cfg.theta)
    if paged:
        table, n_pages = _table(len(prompts), pps, 5, seed=q_len)
        cache = LatentCache.allocate_paged(shape, table, P, n_pages, fill=float("nan"), window=W)
    else:
        cache = LatentCache.allocate(shape, len(prompts), pps * P, fill=float("nan"), window=W)
    xs = [synth.context_x(cfg, b, L) for b, L in enumerate(lens)]
    _fill(cfg, layer, w, cache, prompts, steps, xs)
    # query i of sequence b: the token at position L_b - q_len + i (zeros where that position is negative)
    q = np.zeros((len(prompts), q_len, cfg.n_heads, cfg.d_head))
    for b, L in enumerate(lens):
        for i in range(q_len):
            pos = L - q_len + i
            if pos >= 0:
                q[b, i] = decode_query(cfg, layer, xs[b][pos])
    qt = torch.from_numpy(q.astype(np.float32)).cuda().to(torch_dtype(cfg)).contiguous()
    lens_t = torch.tensor(lens, dtype=torch.int32, device="cuda")
    out = decode_multi(w, cache, qt, lens_t, max(lens))
    if q_len == 1:
        one = decode(w, cache, qt[:, 0].contiguous(), lens_t, max(lens))
    torch.cuda.synchronize()
    if q_len == 1:
        assert torch.equal(out[:, 0], one), "multi-query decode with one query differs from mla_decode"
    got = _np(out)
    for b, L in enumerate(lens):
        c, kr = oracle_cache(cfg, layer, xs[b])
        if fmt == "int4_g32":
            oc, osc = oracle.quantize_int4_g32(c.astype(np.float32))
            c = oracle.dequant_int4(oc, osc)
        elif fmt == "int4_g32_win":
            c = oracle.windowed_latent_int4(synth.round_to_device(c, "bf16"), W)[0]
        elif fmt == "int2_g32_win":
            c = int2.windowed_latent(synth.round_to_device(c, "bf16"), W)[0]
        ref = oracle.multi_query_decode_ref(q[b], c, kr, layer["w_uk"], layer["w_uv"], layer["pair_idx"], cfg.d_head,
                                            cfg.theta)
        for i in range(q_len):
            if L - q_len + i < 0:
                assert np.all(got[b, i] == 0), "a query before the sequence start gives a zero row"
                continue
            rr, a = assert_close(got[b, i], ref[i], cfg.dtype, f"multi-query b={b} i={i}")
        log(f"  b={b} L={L} ok")


def test_paged_decode_step_matches_separate_calls():
    """mla_decode_step on a paged cache (its append is not fused into the attention) equals
    mla_cache_append_ws + mla_decode on the same paged cache bit for bit."""
    from mla_latent_kv_cache_amd import LatentCache, append_ws, decode, decode_step, pack_weights

    cfg = scaled(CONFIGS[1], family="mid", batch=3, context=0)
    prompts, P = [130, 1, 64], 64
    lens = [p + 1 for p in prompts]
    pps = (max(lens) + P - 1) // P
    layer = converted_layer(cfg.family, cfg.r_pairs, cfg.d_kv, cfg.dtype)
    shape = shape_of(cfg)
    w = pack_weights(shape, layer, rope_len=pps * P, theta=cfg.theta)
    table, n_pages = _table(3, pps, 2, seed=5)
    caches = [LatentCache.allocate_paged(shape, table, P, n_pages, fill=float("nan")) for _ in range(2)]
    xs = [synth.context_x(cfg, b, L) for b, L in enumerate(lens)]
    for cache in caches:
        _fill(cfg, layer, w, cache, prompts, 0, xs)
    x_new = torch.from_numpy(np.stack([x[-1] for x in xs])[:, None, :].astype(np.float32)).cuda().to(torch_dtype(cfg))
    start = torch.tensor(prompts, dtype=torch.int32, device="cuda")
    lens_t = torch.tensor(lens, dtype=torch.int32, device="cuda")
    q = np.stack([decode_query(cfg, layer, x[-1]) for x in xs])
    qt = torch.from_numpy(q.astype(np.float32)).cuda().to(torch_dtype(cfg))
    out_step = decode_step(w, caches[0], x_new.contiguous(), start, max(prompts), qt, lens_t, max(lens))
    append_ws(w, caches[1], x_new.contiguous(), start, max(prompts))
    out_sep = decode(w, caches[1], qt, lens_t, max(lens))
    torch.cuda.synchronize()
    assert torch.equal(out_step, out_sep)
    got = _np(out_step)
    for b, L in enumerate(lens):
        c, kr = oracle_cache(cfg, layer, xs[b])
        ref = oracle.decode_ref(q[b], c, kr, layer["w_uk"], layer["w_uv"], layer["pair_idx"], cfg.d_head, cfg.theta)
        assert_close(got[b], ref, cfg.dtype, f"paged decode_step b={b}")


def _pool_gather(pool, table_row, L, P):
    """Rows 0..L-1 of one sequence from a pool tensor [n_pages, P, ...] through its page-table row."""
    pos = np.arange(L)
    rows = torch.from_numpy(table_row[pos // P] * P + pos % P).to(pool.device)
    return pool.reshape(-1, *pool.shape[2:])[rows]


@pytest.mark.parametrize("fmt,W", [("int2_g32_win", 128), ("int4_g32_win", 128), ("int4_g32_win", 64)])
def test_paged_windowed_append_and_decode(fmt, W):
    """The windowed formats on a paged cache (codes, scales and RoPE keys in the pool, the bf16 ring per sequence):
    pool rows equal to a contiguous cache filled the same way, decode equal to it bit for bit (window rows start at
    L - W, so their tiles cross page boundaries) and to the oracle over its windowed latent within tolerance."""
    from mla_latent_kv_cache_amd import LatentCache, decode, pack_weights
    from oracle import int2

    prompts = [700, 1, 129, 0, 200]
    cfg = scaled(CONFIGS[4], family="mid", cache_fmt=fmt, batch=len(prompts), context=0, ctx_range=None)
    steps, P = 3, 64
    lens = [p + steps for p in prompts]
    pps = (max(lens) + P - 1) // P
    t_max = pps * P
    log(f"[paged-win] {fmt} W={W} prompts={prompts} page={P} pages/seq={pps}")
    layer = converted_layer(cfg.family, cfg.r_pairs, cfg.d_kv, cfg.dtype)
    shape = shape_of(cfg)
    w = pack_weights(shape, layer, rope_len=t_max, theta=cfg.theta)
    table, n_pages = _table(len(prompts), pps, 5, seed=31 + W)
    paged = LatentCache.allocate_paged(shape, table, P, n_pages, fill=float("nan"), window=W)
    contig = LatentCache.allocate(shape, len(prompts), t_max, fill=float("nan"), window=W)
    xs = [synth.context_x(cfg, b, L) for b, L in enumerate(lens)]
    for cache in (paged, contig):
        _fill(cfg, layer, w, cache, prompts, steps, xs)
    q = np.stack([decode_query(cfg, layer, x[-1]) for x in xs])
    qt = torch.from_numpy(q.astype(np.float32)).cuda().to(torch_dtype(cfg))
    lens_t = torch.tensor(lens, dtype=torch.int32, device="cuda")
    out_p = decode(w, paged, qt, lens_t, max(lens))
    out_c = decode(w, contig, qt, lens_t, max(lens))
    torch.cuda.synchronize()
    assert torch.equal(out_p, out_c), "paged decode differs from the contiguous one"
    # bit patterns (slots no append reached still hold the NaN fill in both)
    assert torch.equal(paged.ckv_window.view(torch.int16), contig.ckv_window.view(torch.int16)), "rings differ"
    tab = table.cpu().numpy()
    got = _np(out_p)
    for b, L in enumerate(lens):
        nq = L - min(L, W)
        for name, pool, flat in (("codes", paged.ckv, contig.ckv), ("scales", paged.ckv_scale, contig.ckv_scale)):
            assert torch.equal(_pool_gather(pool, tab[b], L, P)[:nq], flat[b, :nq]), f"pool {name} b={b}"
        kr_p = _pool_gather(paged.krope, tab[b], L, P)
        assert torch.equal(kr_p, contig.krope[b, :L]), f"pool k_rope b={b}"
        c, kr = oracle_cache(cfg, layer, xs[b])
        c_bf = synth.round_to_device(c, "bf16")
        eff = (int2.windowed_latent(c_bf, W) if fmt == "int2_g32_win" else oracle.windowed_latent_int4(c_bf, W))[0]
        ref = oracle.decode_ref(q[b], eff, kr, layer["w_uk"], layer["w_uv"], layer["pair_idx"], cfg.d_head, cfg.theta)
        rr, a = assert_close(got[b], ref, cfg.dtype, f"decode b={b} L={L}")
        log(f"  b={b} L={L} rel-L2={rr:.2e} max-abs={a:.2e}")
