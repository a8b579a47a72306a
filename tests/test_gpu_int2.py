"""GPU parity of the 2-bit latent cache with a window of recent bf16 rows (MLA_CACHE_INT2_G32_WIN) against the
oracle (oracle/int2.py), through the C ABI.

The codec alone is checked bit for bit (mla_quantize_int2 on identical fp32 inputs).  Cache contents after
sequences of appends (a long prompt, then single tokens that push rows out of the window) are checked row by
row: the ring against the oracle's bf16 rows, the codes against the oracle's codec on those rows (the GPU
rounds its own fp32 projection, so a bf16 rounding tie may move a code).  Decode outputs are checked against
the oracle's unabsorbed attention over its own windowed latent."""

import numpy as np
import pytest
import torch

import oracle
import synth
from oracle import int2
from synth import CONFIGS, scaled

from parity_lib import (assert_close, assert_finite, check_bf16_values, check_int2_codes, check_rows, converted_layer,
                        decode_query, log, oracle_cache, shape_of, torch_dtype)

pytestmark = pytest.mark.gpu


def _np(t):
    return t.float().cpu().numpy().astype(np.float64)


def test_quantize_int2_bit_exact():
    """mla_quantize_int2 equals the oracle's codec bit for bit: codes and the fp16 (s, z) pairs, on Gaussian groups
    of several scales, bf16-grid values, constant groups, exact ties and values beyond the fp16 range."""
    from mla_latent_kv_cache_amd import quantize_int2

    rng = np.random.default_rng(31)
    parts = [
        rng.standard_normal((512, 32)) * rng.lognormal(0, 3, size=(512, 1)) + rng.standard_normal((512, 1)),
        synth.round_to_device(rng.standard_normal((256, 32)) * 4, "bf16"),
        np.full((8, 32), 2.5),
        np.tile(np.array([0.0, 0.5, 1.5, 2.5, 3.0] + [0.0] * 27), (8, 1)),
        rng.standard_normal((8, 32)) * 1e6,
        rng.standard_normal((8, 32)) * 1e-7,
    ]
    x = np.concatenate(parts).astype(np.float32)
    log(f"[int2-codec] {x.shape[0]} groups")
    codes, meta = quantize_int2(torch.from_numpy(x).cuda())
    torch.cuda.synchronize()
    oc, om = int2.quantize_int2_g32(x)
    np.testing.assert_array_equal(codes.cpu().numpy(), int2.pack_crumbs(oc))
    np.testing.assert_array_equal(meta.cpu().numpy().view(np.uint16), om.view(np.uint16))


def _check_int2_sequence(cache, b, c, W):
    """Ring rows and code rows of sequence b (L = len(c) tokens) against the oracle's fp64 latent rows c: ring
    values are the bf16 rounding of the latent, codes and (s, z) the codec of it, each exact up to roundings
    that the fp32 accumulation bound of the projection can move (parity_lib.check_bf16_values,
    check_int2_codes).  Returns the number of codes that differ from the oracle codec of the oracle's rows."""
    L, D = c.shape
    lw = int2.window_len(L, W)
    nq = L - lw
    if lw:
        ring = _np(cache.ckv_window[b])
        got = np.stack([ring[p % W] for p in range(nq, L)])
        check_bf16_values(got, c[nq:], f"ring b={b}")
    if nq == 0:
        return 0
    codes = int2.unpack_crumbs(cache.ckv[b, :nq].cpu().numpy())
    meta = cache.ckv_scale[b, :nq].cpu().numpy()
    _, n_k = check_int2_codes(c[:nq], codes, meta, f"int2 b={b}")
    return n_k


def _oracle_effective(c, W):
    c_bf = synth.round_to_device(c, "bf16")
    eff, _, _ = int2.windowed_latent(c_bf, W)
    return c_bf, eff


@pytest.mark.parametrize("W,steps_ws,steps_plain", [(128, 5, 2), (64, 3, 0), (0, 2, 1)])
def test_int2_batched_prompt_then_steps(W, steps_ws, steps_plain):
    """Four sequences: one batched prompt append of 3100 tokens each (the long-prompt GEMM path), then single
    tokens through the split-K append (workspace) and the few-token path, each pushing the oldest window row
    into the codes.  Cache rows and the decode outputs against the oracle."""
    from mla_latent_kv_cache_amd import LatentCache, append, append_ws, decode, pack_weights

    cfg = scaled(CONFIGS[4], family="mid", batch=4, cache_fmt="int2_g32_win")
    B, P = 4, 3100
    n_steps = steps_ws + steps_plain
    L = P + n_steps
    t_max = L + 4
    log(f"[int2] batched prompt B={B} P={P} then {steps_ws}+{steps_plain} steps, W={W}")
    layer = converted_layer(cfg.family, cfg.r_pairs, cfg.d_kv, cfg.dtype)
    shape = shape_of(cfg)
    w = pack_weights(shape, layer, rope_len=t_max, theta=cfg.theta)
    cache = LatentCache.allocate(shape, B, t_max, fill=float("nan"), window=W)
    xs = [synth.context_x(cfg, b, L) for b in range(B)]
    xp = torch.from_numpy(np.stack([x[:P] for x in xs]).astype(np.float32)).cuda().to(torch_dtype(cfg))
    append(w, cache, xp, torch.zeros(B, dtype=torch.int32, device="cuda"), 0)
    del xp
    for i in range(n_steps):
        pos = P + i
        xn = torch.from_numpy(np.stack([x[pos:pos + 1] for x in xs]).astype(np.float32)).cuda().to(torch_dtype(cfg))
        start = torch.full((B,), pos, dtype=torch.int32, device="cuda")
        if i < steps_ws:
            append_ws(w, cache, xn.contiguous(), start, pos)
        else:
            append(w, cache, xn.contiguous(), start, pos)
    q = np.stack([decode_query(cfg, layer, x[-1]) for x in xs])
    qt = torch.from_numpy(q.astype(np.float32)).cuda().to(torch_dtype(cfg))
    lens = torch.full((B,), L, dtype=torch.int32, device="cuda")
    out = decode(w, cache, qt, lens, L)
    out2 = decode(w, cache, qt, lens, L)
    torch.cuda.synchronize()
    assert torch.equal(out, out2), "decode is not bitwise deterministic"
    got = _np(out)
    for b in range(B):
        c, kr = oracle_cache(cfg, layer, xs[b])
        c_bf, eff = _oracle_effective(c, W)
        nd = _check_int2_sequence(cache, b, c, W)
        check_rows(cfg, cache.krope[b, :L], kr, f"k_rope b={b}")
        ref = oracle.decode_ref(q[b], eff, kr, layer["w_uk"], layer["w_uv"], layer["pair_idx"], cfg.d_head, cfg.theta)
        r, a = assert_close(got[b], ref, cfg.dtype, f"decode b={b}")
        log(f"  b={b} code differences {nd}, rel-L2={r:.2e} max-abs={a:.2e}")


@pytest.mark.parametrize("family", ["mid", "odd"])
def test_int2_ragged_per_sequence(family):
    """Ragged sequences filled one at a time (the 128x128 MFMA append, the few-token append), lengths below,
    at and above the window, an empty one; then three single-token steps for every non-empty sequence at its
    own position.  "odd" (5 heads) decodes through the generic kernel."""
    from mla_latent_kv_cache_amd import LatentCache, append, append_ws, decode, pack_weights

    cfg = scaled(CONFIGS[4], family=family, batch=6, cache_fmt="int2_g32_win")
    W = 128
    prompts = [700, 33, 129, 128, 1, 0]
    B = len(prompts)
    steps = 3
    lens = [p + steps if p else 0 for p in prompts]
    t_max = max(lens) + 2
    log(f"[int2] ragged {family} prompts={prompts} W={W}")
    layer = converted_layer(cfg.family, cfg.r_pairs, cfg.d_kv, cfg.dtype)
    shape = shape_of(cfg)
    w = pack_weights(shape, layer, rope_len=t_max, theta=cfg.theta)
    cache = LatentCache.allocate(shape, B, t_max, fill=float("nan"), window=W)
    xs = [synth.context_x(cfg, b, max(L, 1)) for b, L in enumerate(lens)]
    zero = torch.zeros(1, dtype=torch.int32, device="cuda")
    for b, P in enumerate(prompts):
        if P:
            xt = torch.from_numpy(xs[b][:P].astype(np.float32)).cuda().to(torch_dtype(cfg)).reshape(1, P, -1)
            append(w, cache.view(b, b + 1), xt, zero, 0)
    live = [b for b in range(B) if prompts[b]]
    for i in range(steps):
        xn = torch.from_numpy(np.stack([xs[b][prompts[b] + i] if prompts[b] else np.zeros(cfg.d_model)
                                        for b in range(B)])[:, None, :].astype(np.float32)).cuda().to(torch_dtype(cfg))
        # empty sequences stay empty: they take part in no step (their start would be 0 and write a row)
        sub = cache.view(0, 4)
        start = torch.tensor([prompts[b] + i for b in range(4)], dtype=torch.int32, device="cuda")
        append_ws(w, sub, xn[:4].contiguous(), start, max(prompts) + i)
        append(w, cache.view(4, 5), xn[4:5].contiguous(), torch.tensor([prompts[4] + i], dtype=torch.int32,
                                                                       device="cuda"), prompts[4] + i)
    q = np.stack([decode_query(cfg, layer, xs[b][lens[b] - 1]) if lens[b] else np.zeros((cfg.n_heads, cfg.d_head))
                  for b in range(B)])
    qt = torch.from_numpy(q.astype(np.float32)).cuda().to(torch_dtype(cfg))
    lens_t = torch.tensor(lens, dtype=torch.int32, device="cuda")
    out = decode(w, cache, qt, lens_t, max(lens))
    torch.cuda.synchronize()
    got = _np(out)
    assert np.all(got[5] == 0.0), "an empty sequence gives a zero output row"
    for b in live:
        L = lens[b]
        c, kr = oracle_cache(cfg, layer, xs[b][:L])
        c_bf, eff = _oracle_effective(c, W)
        _check_int2_sequence(cache, b, c, W)
        ref = oracle.decode_ref(q[b], eff, kr, layer["w_uk"], layer["w_uv"], layer["pair_idx"], cfg.d_head, cfg.theta)
        r, a = assert_close(got[b], ref, cfg.dtype, f"decode b={b} L={L}")
        log(f"  b={b} L={L} rel-L2={r:.2e} max-abs={a:.2e}")


def test_int2_gqa_source_layer():
    """A grouped-query-source layer (8 KV heads) on the 2-bit cache with a window: cache rows and decode."""
    from mla_latent_kv_cache_amd import LatentCache, append, decode, pack_weights
    from parity_lib import gqa_converted_layer

    cfg = scaled(CONFIGS[4], family="mid", batch=2, cache_fmt="int2_g32_win")
    W, lens = 128, [500, 90]
    t_max = max(lens)
    log(f"[int2-gqa] lens={lens} W={W}")
    layer = gqa_converted_layer("gqa_mid", cfg.r_pairs, cfg.d_kv, cfg.dtype)
    shape = shape_of(cfg)
    w = pack_weights(shape, layer, rope_len=t_max, theta=cfg.theta)
    cache = LatentCache.allocate(shape, len(lens), t_max, fill=float("nan"), window=W)
    xs = [synth.context_x(cfg, b, L) for b, L in enumerate(lens)]
    zero = torch.zeros(1, dtype=torch.int32, device="cuda")
    for b, L in enumerate(lens):
        xt = torch.from_numpy(xs[b].astype(np.float32)).cuda().to(torch_dtype(cfg)).reshape(1, L, -1)
        append(w, cache.view(b, b + 1), xt, zero, 0)
    q = np.stack([decode_query(cfg, layer, x[-1]) for x in xs])
    qt = torch.from_numpy(q.astype(np.float32)).cuda().to(torch_dtype(cfg))
    out = decode(w, cache, qt, torch.tensor(lens, dtype=torch.int32, device="cuda"), t_max)
    torch.cuda.synchronize()
    got = _np(out)
    for b, L in enumerate(lens):
        c, kr = oracle_cache(cfg, layer, xs[b])
        c_bf, eff = _oracle_effective(c, W)
        _check_int2_sequence(cache, b, c, W)
        ref = oracle.decode_ref(q[b], eff, kr, layer["w_uk"], layer["w_uv"], layer["pair_idx"], cfg.d_head, cfg.theta)
        r, a = assert_close(got[b], ref, cfg.dtype, f"decode b={b}")
        log(f"  b={b} L={L} rel-L2={r:.2e} max-abs={a:.2e}")


def test_int2_decode_step_matches_separate_calls():
    """mla_decode_step on the 2-bit cache equals mla_cache_append_ws followed by mla_decode bit for bit (cache
    codes, (s, z), ring and output)."""
    from mla_latent_kv_cache_amd import LatentCache, append, append_ws, decode, decode_step, pack_weights

    cfg = scaled(CONFIGS[4], family="mid", batch=4, cache_fmt="int2_g32_win")
    W = 64
    lens = [300, 2, 65, 64]
    t_max = 320
    log(f"[int2-step] lens={lens} W={W}")
    layer = converted_layer(cfg.family, cfg.r_pairs, cfg.d_kv, cfg.dtype)
    shape = shape_of(cfg)
    w = pack_weights(shape, layer, rope_len=t_max, theta=cfg.theta)
    caches = [LatentCache.allocate(shape, len(lens), t_max, fill=float("nan"), window=W) for _ in range(2)]
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

    def same_bits(u, v):
        return torch.equal(u.contiguous().view(torch.uint8), v.contiguous().view(torch.uint8))

    for name in ("ckv", "ckv_scale", "ckv_window", "krope"):
        assert same_bits(getattr(caches[0], name), getattr(caches[1], name)), name
    got = _np(out_step)
    for b, L in enumerate(lens):
        c, kr = oracle_cache(cfg, layer, xs[b])
        c_bf, eff = _oracle_effective(c, W)
        _check_int2_sequence(caches[0], b, c, W)
        ref = oracle.decode_ref(q[b], eff, kr, layer["w_uk"], layer["w_uv"], layer["pair_idx"], cfg.d_head, cfg.theta)
        r, a = assert_close(got[b], ref, cfg.dtype, f"decode_step b={b}")
        log(f"  b={b} rel-L2={r:.2e} max-abs={a:.2e}")
