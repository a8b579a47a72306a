"""GPU parity of mla_cache_append + mla_prefill (causal, unabsorbed) against the oracle, through the C ABI.

Small cases compare every query row; lengths that are not multiples of the 64-key / 256-query tiles
exercise the ragged tails, and a one-token prompt reduces to the first value row.  The full-size case
(4 sequences x 4096 tokens, Llama-2-7B shapes) compares every query row of the first and last sequences and
sampled rows (both ends of the causal range, tile boundaries) of the others.  The appended cache rows are
compared element by element in every case."""

import numpy as np
import pytest
import torch

import oracle
import synth
from synth import CONFIGS, scaled

from parity_lib import (assert_close, assert_finite, check_rows, converted_layer, log, rope_key_rows, shape_of,
                        torch_dtype)

pytestmark = pytest.mark.gpu


def run_prefill_case(cfg, S, B, rows=None, full_b=None, variant=("2-norm", "joint"), layer=None, rope_heads=0):
    """Append + prefill of B seeded prompts of S tokens.  Sequences in full_b (all when None) are compared on
    every query row; the others on `rows`.  The appended cache rows of every sequence are compared too."""
    from mla_latent_kv_cache_amd import LatentCache, append, pack_weights, prefill

    log(f"[prefill] family={cfg.family} r={cfg.r_pairs} d_kv={cfg.d_kv} B={B} S={S} "
        f"every row of {'all' if full_b is None else full_b}, else rows {rows} "
        f"conversion={variant if layer is None else 'given'} rope_heads={rope_heads or cfg.n_heads}")
    if layer is None:
        layer = converted_layer(cfg.family, cfg.r_pairs, cfg.d_kv, cfg.dtype, *variant)
    shape = shape_of(cfg, rope_heads)
    t_max = S + 3
    w = pack_weights(shape, layer, rope_len=t_max, theta=cfg.theta)
    cache = LatentCache.allocate(shape, B, t_max, fill=float("nan"))
    xs = [synth.context_x(cfg, b, S) for b in range(B)]
    x = torch.from_numpy(np.stack(xs).astype(np.float32)).cuda().to(torch_dtype(cfg))
    append(w, cache, x, torch.zeros(B, dtype=torch.int32, device="cuda"), 0)
    del x
    qs = [synth.query_rows(xb, layer["w_q"], cfg.dtype).reshape(S, cfg.n_heads, cfg.d_head) for xb in xs]
    q = torch.from_numpy(np.stack(qs).astype(np.float32)).cuda().to(torch_dtype(cfg))
    out = prefill(w, cache, q)
    torch.cuda.synchronize()
    out2 = prefill(w, cache, q)
    torch.cuda.synchronize()
    assert torch.equal(out, out2), "prefill is not bitwise deterministic"
    assert_finite(out, "prefill out")
    got = out.float().cpu().numpy().astype(np.float64)
    for b in range(B):
        c, kr = oracle.append_ref(xs[b], layer["w_dkv"], layer["w_krope"], layer["pair_idx"], np.arange(S),
                                  cfg.d_head, cfg.theta)
        check_rows(cfg, cache.ckv[b, :S], c, f"c_kv b={b}")
        check_rows(cfg, cache.krope[b, :S], rope_key_rows(kr, cfg.n_heads, rope_heads), f"k_rope b={b}")
        rr = np.arange(S) if (full_b is None or b in full_b or rows is None) else np.asarray(rows)
        ref = oracle.prefill_ref(qs[b], c, kr, layer["w_uk"], layer["w_uv"], layer["pair_idx"], cfg.d_head,
                                 cfg.theta, rows=rr)
        r, a = assert_close(got[b][rr], ref, cfg.dtype, f"prefill b={b}")
        log(f"  b={b} {len(rr)} rows: rel-L2={r:.2e} max-abs={a:.2e}")


def test_prefill_mid_ragged():
    run_prefill_case(scaled(CONFIGS[2], family="mid"), S=200, B=2)


def test_prefill_mid_tiles():
    run_prefill_case(scaled(CONFIGS[2], family="mid"), S=256, B=1)


def test_prefill_single_token_and_one_past_tile():
    cfg = scaled(CONFIGS[2], family="mid")
    run_prefill_case(cfg, S=1, B=1)
    run_prefill_case(cfg, S=65, B=1)


def test_prefill_mid_several_query_tiles():
    """Three 256-row query tiles, the last one ragged: every row against the oracle."""
    run_prefill_case(scaled(CONFIGS[2], family="mid"), S=600, B=1)


def test_prefill_two_pairs_per_head():
    """r = 2: four retained dims per head, the RoPE keys fill only part of a 16-byte chunk."""
    run_prefill_case(scaled(CONFIGS[2], family="mid", r_pairs=2), S=130, B=2)


def test_prefill_head_count_not_multiple_of_8():
    """5 heads x 3 sequences = 15 (sequence, head) pairs: the scheduler's non-XCD-grouped order."""
    run_prefill_case(scaled(CONFIGS[2], family="odd"), S=300, B=3)


@pytest.mark.parametrize("strategy,svd", [("high", "split"), ("uniform", "joint")])
def test_prefill_ablation_variant_layers(strategy, svd):
    """Layers converted with the pages' ablation variants run through the same append and prefill kernels."""
    run_prefill_case(scaled(CONFIGS[2], family="mid"), S=300, B=2, variant=(strategy, svd))


def test_prefill_gqa_source_layer():
    """A layer converted from a grouped-query source (8 KV heads for 32 query heads) through append + prefill."""
    from parity_lib import gqa_converted_layer

    cfg = scaled(CONFIGS[2], family="mid")
    run_prefill_case(cfg, S=300, B=2, layer=gqa_converted_layer("gqa_mid", cfg.r_pairs, cfg.d_kv, cfg.dtype))


@pytest.mark.slow
@pytest.mark.timeout(900)
def test_prefill_full_llama_b4_s4096():
    cfg = CONFIGS[2]
    rows = [0, 1, 2, 63, 64, 127, 128, 129, 1000, 2047, 2048, 4031, 4032, 4094, 4095]
    run_prefill_case(cfg, S=cfg.context, B=cfg.batch, rows=rows, full_b=[0, 3])


@pytest.mark.parametrize("fmt,window", [("int4_g32", 0), ("int2_g32_win", 128), ("int2_g32_win", 0),
                                        ("int2_g32_win", 512), ("int4_g32_win", 128)])
def test_prefill_quantised_latent(fmt, window):
    """Prefill over a quantised latent cache (the key-designs section's 4- and 2-bit compatibility): the latent
    rows are dequantised exactly as decode reads them, so the reference is the oracle's unabsorbed attention over
    its own dequantised latent (int4 codec of the fp32 latent; 2-bit codec of the bf16 rows outside the last
    `window` positions).  Window 512 exceeds the prompt (every row in the ring); window 0 codes every row."""
    from mla_latent_kv_cache_amd import LatentCache, append, pack_weights, prefill
    from oracle import int2

    cfg = scaled(CONFIGS[2], family="mid", cache_fmt=fmt)
    B, S = 2, 300
    log(f"[prefill-quantised] {fmt} window={window} B={B} S={S}")
    layer = converted_layer(cfg.family, cfg.r_pairs, cfg.d_kv, cfg.dtype)
    shape = shape_of(cfg)
    w = pack_weights(shape, layer, rope_len=S, theta=cfg.theta)
    cache = LatentCache.allocate(shape, B, S, fill=float("nan"), window=window)
    xs = [synth.context_x(cfg, b, S) for b in range(B)]
    x = torch.from_numpy(np.stack(xs).astype(np.float32)).cuda().to(torch_dtype(cfg))
    append(w, cache, x, torch.zeros(B, dtype=torch.int32, device="cuda"), 0)
    qs = [synth.query_rows(xb, layer["w_q"], cfg.dtype).reshape(S, cfg.n_heads, cfg.d_head) for xb in xs]
    q = torch.from_numpy(np.stack(qs).astype(np.float32)).cuda().to(torch_dtype(cfg))
    out = prefill(w, cache, q)
    out2 = prefill(w, cache, q)
    torch.cuda.synchronize()
    assert torch.equal(out, out2), "prefill is not bitwise deterministic"
    assert_finite(out, "prefill out")
    got = out.float().cpu().numpy().astype(np.float64)
    for b in range(B):
        c, kr = oracle.append_ref(xs[b], layer["w_dkv"], layer["w_krope"], layer["pair_idx"], np.arange(S),
                                  cfg.d_head, cfg.theta)
        if fmt == "int4_g32":
            oc, osc = oracle.quantize_int4_g32(c.astype(np.float32))
            c_used = oracle.dequant_int4(oc, osc)
        elif fmt == "int4_g32_win":
            c_used, _, _ = oracle.windowed_latent_int4(synth.round_to_device(c, "bf16"), window)
        else:
            c_used, _, _ = int2.windowed_latent(synth.round_to_device(c, "bf16"), window)
        ref = oracle.prefill_ref(qs[b], c_used, kr, layer["w_uk"], layer["w_uv"], layer["pair_idx"], cfg.d_head,
                                 cfg.theta)
        r, a = assert_close(got[b], ref, cfg.dtype, f"prefill b={b}")
        log(f"  b={b} rel-L2={r:.2e} max-abs={a:.2e}")
