"""Pins of the oracle's int4 latent codec (hand-worked golden groups and codec properties) and of its
cache-byte accounting (the reduction percentages printed on the pages)."""

import json
import os

import numpy as np
import pytest

import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def test_int4_worked_example():
    with open(os.path.join(GOLDEN, "int4_worked_example.json")) as f:
        g = json.load(f)
    for grp in g["groups"]:
        x = np.array(grp["x"], dtype=np.float32)
        codes, scales = oracle.quantize_int4_g32(x)
        assert codes.tolist() == grp["codes"]
        assert float(scales[0]) == grp["scale"]
        assert oracle.pack_nibbles(codes).tolist() == grp["bytes"]
        assert oracle.unpack_nibbles(np.array(grp["bytes"], dtype=np.uint8)).tolist() == grp["codes"]


def test_int4_properties():
    rng = np.random.default_rng(7)
    x = (rng.standard_normal((500, 64)) * rng.uniform(1e-3, 10, (500, 1))).astype(np.float32)
    codes, scales = oracle.quantize_int4_g32(x)
    assert codes.min() >= -7 and codes.max() <= 7
    deq = oracle.dequant_int4(codes, scales)
    g = x.reshape(-1, 32).astype(np.float64)
    s = scales.reshape(-1).astype(np.float64)
    c = codes.reshape(-1, 32)
    # the absmax element maps to +-7 (its quotient lies within fp16 rounding of 7)
    am = np.argmax(np.abs(g), axis=1)
    assert np.all(np.abs(c[np.arange(len(am)), am]) == 7)
    # reconstruction error at most half a step where no clamping happened
    inside = np.abs(g) <= 7 * s[:, None]
    err = np.abs(g - deq.reshape(-1, 32))
    assert np.all(err[inside] <= s[:, None].repeat(32, 1)[inside] / 2 * (1 + 1e-6))
    # values on the grid k*s come back as k
    s0 = np.float16(0.375)
    grid = (np.arange(-7, 8, dtype=np.float32) * np.float32(s0))
    vals = np.concatenate([grid, np.zeros(32 - 15, dtype=np.float32)])
    cg, sg = oracle.quantize_int4_g32(vals)
    assert float(sg[0]) == float(s0)
    assert cg[:15].tolist() == list(range(-7, 8))
    # dequantised values are exact fp32 products
    assert np.all(deq == (c.astype(np.float32) * s.astype(np.float32)[:, None]).reshape(deq.shape))


def test_int4_ties_round_half_even_and_tiny_scales():
    s = np.float32(0.25)  # absmax 1.75 -> s = 0.25 exactly
    x = np.zeros(32, dtype=np.float32)
    x[:6] = np.array([1.75, 0.125, 0.375, -0.125, -0.375, 0.625], dtype=np.float32)  # x/s: 7, .5, 1.5, -.5, -1.5, 2.5
    c, sc = oracle.quantize_int4_g32(x)
    assert float(sc[0]) == float(s)
    assert c[:6].tolist() == [7, 0, 2, 0, -2, 2]
    # fp16-subnormal scale
    y = np.zeros(32, dtype=np.float32)
    y[3] = np.float32(7 * 2.0 ** -20)
    c2, s2 = oracle.quantize_int4_g32(y)
    assert float(s2[0]) == 2.0 ** -20 and c2[3] == 7
    # scale underflows to zero -> all codes zero
    z = np.full(32, np.float32(1e-9))
    c3, s3 = oracle.quantize_int4_g32(z)
    assert float(s3[0]) == 0.0 and not c3.any()


def test_cache_reduction_matches_pages():
    with open(os.path.join(GOLDEN, "cache_reduction.json")) as f:
        g = json.load(f)
    mha = oracle.mha_bytes_per_token(g["n_heads"], g["d_head"], g["elem_bytes"])
    bf = oracle.cache_bytes_per_token(g["n_heads"], g["r_pairs"], g["d_kv"], latent_bits=16)
    i4 = oracle.cache_bytes_per_token(g["n_heads"], g["r_pairs"], g["d_kv"], latent_bits=4)
    tol = g["printed_precision"] + 1e-9
    assert abs(oracle.reduction_pct(bf, mha) - g["printed_pct"]["latent_bf16"]) <= tol
    assert abs(oracle.reduction_pct(i4, mha) - g["printed_pct"]["latent_int4"]) <= tol


def test_cache_bytes_of_configs():
    # bytes/token of the cache layouts used here: dense bf16 (d_kv 512, r 4), (d_kv 256, r 2), int4 g32 with fp16 scales
    assert oracle.cache_bytes_per_token(32, 4, 512) == 1536
    assert oracle.cache_bytes_per_token(32, 2, 256) == 768
    assert oracle.cache_bytes_per_token(32, 4, 512, latent_bits=4, scale_bytes=2) == 800
    assert oracle.cache_bytes_per_token(9, 4, 32, latent_bits=32, rope_bytes=4) == 416
