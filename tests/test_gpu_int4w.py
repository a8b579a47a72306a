"""GPU parity of the int4 latent cache with a window of recent bf16 rows (MLA_CACHE_INT4_G32_WIN) against the
oracle (oracle.windowed_latent_int4), through the C ABI.

The README page's quantised-cache evaluation keeps the most recent tokens unquantised beside a 4-bit cache;
here the last `window` positions of every sequence are bf16 rows in a ring and every older row is the int4
codec of its bf16 value.  Cache contents after appends that push rows out of the window are checked row by
row (ring rows: the bf16 rounding of the latent; code rows: the int4 codec of that bf16 row, exact up to
roundings the fp32 accumulation bound allows), and the decode outputs against the oracle's unabsorbed
attention over its own windowed latent."""

import numpy as np
import pytest
import torch

import oracle
import synth
from synth import CONFIGS, scaled

from parity_lib import (assert_close, assert_finite, check_bf16_values, check_int4_cache, check_rows, converted_layer,
                        decode_query, log, oracle_cache, shape_of, torch_dtype)

pytestmark = pytest.mark.gpu


def _np(t):
    return t.float().cpu().numpy().astype(np.float64)


def _check_sequence(cache, b, c, W):
    """Ring rows and int4 code rows of sequence b (L = len(c) tokens) against the oracle's fp64 latent c."""
    L, D = c.shape
    lw = min(L, W)
    nq = L - lw
    if lw:
        ring = _np(cache.ckv_window[b])
        check_bf16_values(np.stack([ring[p % W] for p in range(nq, L)]), c[nq:], f"ring b={b}")
    if nq:
        check_int4_cache(c[:nq], oracle.unpack_nibbles(cache.ckv[b, :nq].cpu().numpy()),
                         cache.ckv_scale[b, :nq].cpu().numpy(), f"int4 b={b}", via_bf16=True)


def _effective(c, W):
    eff, _, _ = oracle.windowed_latent_int4(synth.round_to_device(c, "bf16"), W)
    return eff


@pytest.mark.parametrize("W,steps_ws,steps_plain", [(128, 5, 2), (64, 3, 0), (0, 2, 1)])
def test_int4w_batched_prompt_then_steps(W, steps_ws, steps_plain):
    """Four sequences: one batched prompt append of 3100 tokens each (the long-prompt GEMM path), then single
    tokens through the split-K append (workspace) and the few-token path, each pushing the oldest window row into
    the codes.  Cache rows and decode outputs against the oracle."""
    from mla_latent_kv_cache_amd import LatentCache, append, append_ws, decode, pack_weights

    cfg = scaled(CONFIGS[4], family="mid", batch=4, cache_fmt="int4_g32_win")
    B, P = 4, 3100
    n_steps = steps_ws + steps_plain
    L = P + n_steps
    t_max = L + 4
    log(f"[int4w] batched prompt B={B} P={P} then {steps_ws}+{steps_plain} steps, W={W}")
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
        (append_ws if i < steps_ws else append)(w, cache, xn.contiguous(), start, pos)
    q = np.stack([decode_query(cfg, layer, x[-1]) for x in xs])
    qt = torch.from_numpy(q.astype(np.float32)).cuda().to(torch_dtype(cfg))
    lens = torch.full((B,), L, dtype=torch.int32, device="cuda")
    out = decode(w, cache, qt, lens, L)
    out2 = decode(w, cache, qt, lens, L)
    torch.cuda.synchronize()
    assert torch.equal(out, out2), "decode is not bitwise deterministic"
    assert_finite(out, "decode out")
    got = _np(out)
    for b in range(B):
        c, kr = oracle_cache(cfg, layer, xs[b])
        _check_sequence(cache, b, c, W)
        check_rows(cfg, cache.krope[b, :L], kr, f"k_rope b={b}")
        ref = oracle.decode_ref(q[b], _effective(c, W), kr, layer["w_uk"], layer["w_uv"], layer["pair_idx"],
                                cfg.d_head, cfg.theta)
        r, a = assert_close(got[b], ref, cfg.dtype, f"decode b={b}")
        log(f"  b={b} rel-L2={r:.2e} max-abs={a:.2e}")


@pytest.mark.parametrize("family", ["mid", "odd"])
def test_int4w_ragged_per_sequence(family):
    """Ragged sequences filled one at a time, lengths below, at and above the window, an empty one; then three
    single-token steps for every non-empty sequence.  "odd" (5 heads) decodes through the generic kernel."""
    from mla_latent_kv_cache_amd import LatentCache, append, append_ws, decode, pack_weights

    cfg = scaled(CONFIGS[4], family=family, batch=6, cache_fmt="int4_g32_win")
    W = 128
    prompts = [700, 33, 129, 128, 1, 0]
    B, steps = len(prompts), 3
    lens = [p + steps if p else 0 for p in prompts]
    t_max = max(lens) + 2
    log(f"[int4w] ragged {family} prompts={prompts} W={W}")
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
    for i in range(steps):
        xn = torch.from_numpy(np.stack([xs[b][prompts[b] + i] if prompts[b] else np.zeros(cfg.d_model)
                                        for b in range(B)])[:, None, :].astype(np.float32)).cuda().to(torch_dtype(cfg))
        start = torch.tensor([prompts[b] + i for b in range(5)], dtype=torch.int32, device="cuda")
        append_ws(w, cache.view(0, 5), xn[:5].contiguous(), start, max(prompts) + i)
    q = np.stack([decode_query(cfg, layer, xs[b][lens[b] - 1]) if lens[b] else np.zeros((cfg.n_heads, cfg.d_head))
                  for b in range(B)])
    qt = torch.from_numpy(q.astype(np.float32)).cuda().to(torch_dtype(cfg))
    out = decode(w, cache, qt, torch.tensor(lens, dtype=torch.int32, device="cuda"), max(lens))
    torch.cuda.synchronize()
    got = _np(out)
    assert np.all(got[5] == 0.0), "an empty sequence gives a zero output row"
    for b in range(5):
        L = lens[b]
        c, kr = oracle_cache(cfg, layer, xs[b][:L])
        _check_sequence(cache, b, c, W)
        ref = oracle.decode_ref(q[b], _effective(c, W), kr, layer["w_uk"], layer["w_uv"], layer["pair_idx"],
                                cfg.d_head, cfg.theta)
        r, a = assert_close(got[b], ref, cfg.dtype, f"decode b={b} L={L}")
        log(f"  b={b} L={L} rel-L2={r:.2e} max-abs={a:.2e}")


def test_int4w_decode_step_matches_separate_calls():
    """mla_decode_step on the windowed int4 cache equals mla_cache_append_ws followed by mla_decode bit for bit
    (codes, scales, ring and output), and the oracle within tolerance."""
    from mla_latent_kv_cache_amd import LatentCache, append, append_ws, decode, decode_step, pack_weights

    cfg = scaled(CONFIGS[4], family="mid", batch=4, cache_fmt="int4_g32_win")
    W, lens, t_max = 64, [300, 2, 65, 64], 320
    log(f"[int4w-step] lens={lens} W={W}")
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
    for name in ("ckv", "ckv_scale", "ckv_window", "krope"):
        u, v = getattr(caches[0], name), getattr(caches[1], name)
        assert torch.equal(u.contiguous().view(torch.uint8), v.contiguous().view(torch.uint8)), name
    got = _np(out_step)
    for b, L in enumerate(lens):
        c, kr = oracle_cache(cfg, layer, xs[b])
        _check_sequence(caches[0], b, c, W)
        ref = oracle.decode_ref(q[b], _effective(c, W), kr, layer["w_uk"], layer["w_uv"], layer["pair_idx"],
                                cfg.d_head, cfg.theta)
        r, a = assert_close(got[b], ref, cfg.dtype, f"decode_step b={b}")
        log(f"  b={b} rel-L2={r:.2e} max-abs={a:.2e}")
