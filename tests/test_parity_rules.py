"""The per-element parity rules of tests/parity_lib.py, on the CPU.

A latent projected with float32 BLAS (another accumulation order than the oracle's fp64, as the GPU's is)
must pass every rule; the same values with one planted mistake -- a scale one fp16 step off, a code one off,
a bf16 value one step off, a 2-bit offset one step off -- must fail it."""

import numpy as np
import pytest

import oracle
import synth
from oracle import int2

from parity_lib import ACC_EPS, check_bf16_values, check_int2_codes, check_int4_cache


def _latents(seed=3, n=256, d=4096, d_kv=512):
    """fp64 oracle latents and an fp32 projection of the same bf16 inputs in another summation order."""
    rng = np.random.default_rng(seed)
    x = synth.round_to_device(rng.standard_normal((n, d)), "bf16")
    w = synth.round_to_device(np.linalg.qr(rng.standard_normal((d, d_kv)))[0], "bf16")
    c = x @ w
    c32 = (x.astype(np.float32) @ w.astype(np.float32)).astype(np.float64)
    return c, c32


def test_fp32_projection_within_accumulation_bound():
    c, c32 = _latents()
    assert np.max(np.abs(c32 - c) / (1 + np.abs(c))) < ACC_EPS / 8


def test_bf16_rule():
    c, c32 = _latents()
    got = synth.round_to_device(c32, "bf16")
    check_bf16_values(got, c, "fp32 BLAS")
    bad = got.copy()
    i = np.unravel_index(np.argmax(np.abs(c)), c.shape)
    bad[i] = synth.bits_to_f64(synth.bf16_bits(np.array([bad[i]])) + np.uint16(1))[0]
    with pytest.raises(AssertionError):
        check_bf16_values(bad, c, "planted")


def test_int4_rule():
    c, c32 = _latents()
    codes, scales = oracle.quantize_int4_g32(c32.astype(np.float32))
    check_int4_cache(c, codes, scales, "fp32 BLAS")
    # a scale one fp16 step off in a group whose absmax/7 is far from a rounding boundary
    s = scales.copy().reshape(-1)
    s.view(np.uint16)[5] += 1
    with pytest.raises(AssertionError):
        check_int4_cache(c, codes, s.reshape(scales.shape), "planted scale")
    # one code off by one where the quotient is not near a half-integer
    q = c.astype(np.float32).reshape(-1, 32) / scales.reshape(-1).astype(np.float32)[:, None]
    far = np.abs(np.abs(q - np.floor(q)) - 0.5) > 0.1
    k = codes.copy().reshape(-1, 32)
    g, j = np.argwhere(far & (np.abs(k) < 7))[0]
    k[g, j] += 1
    with pytest.raises(AssertionError):
        check_int4_cache(c, k.reshape(codes.shape), scales, "planted code")


def test_int4_rule_accepts_a_scale_tie():
    """A group whose absmax/7 sits on an fp16 rounding midpoint: both neighbouring scales are accepted, and
    under the other one the codes recomputed by the codec are accepted too."""
    c = np.zeros((1, 32))
    s_lo, s_hi = np.float16(0.25), np.nextafter(np.float16(0.25), np.float16(1))
    mid = (np.float64(s_lo) + np.float64(s_hi)) / 2
    c[0, 0] = 7 * mid
    c[0, 1:] = np.linspace(-1.5, 1.5, 31)
    for s in (s_lo, s_hi):
        codes = oracle.int4_codes(c.astype(np.float32), np.array([s]))
        check_int4_cache(c, codes, np.array([[s]]), "tie")
    with pytest.raises(AssertionError):
        s2 = np.nextafter(s_hi, np.float16(1))
        check_int4_cache(c, oracle.int4_codes(c.astype(np.float32), np.array([s2])), np.array([[s2]]), "two steps")


def test_int2_rule():
    c, c32 = _latents(d_kv=256)
    b = synth.round_to_device(c32, "bf16").astype(np.float32)
    codes, meta = int2.quantize_int2_g32(b)
    check_int2_codes(c, codes, meta, "fp32 BLAS")
    m = meta.copy().reshape(-1, 2)
    m.view(np.uint16)[7, 1] += 1  # offset one fp16 step off
    with pytest.raises(AssertionError):
        check_int2_codes(c, codes, m.reshape(meta.shape), "planted offset")
    m = meta.copy().reshape(-1, 2)
    m.view(np.uint16)[9, 0] += 1  # scale one fp16 step off
    with pytest.raises(AssertionError):
        check_int2_codes(c, codes, m.reshape(meta.shape), "planted scale")
    k = codes.copy().reshape(-1, 32)
    s = meta.reshape(-1, 2)[:, 0].astype(np.float32)
    z = meta.reshape(-1, 2)[:, 1].astype(np.float32)
    q = (b.reshape(-1, 32) - z[:, None]) / s[:, None]
    far = np.abs(np.abs(q - np.floor(q)) - 0.5) > 0.1
    g, j = np.argwhere(far & (k < 3))[0]
    k[g, j] += 1
    with pytest.raises(AssertionError):
        check_int2_codes(c, k.reshape(codes.shape), meta, "planted code")


def test_int2_rule_accepts_a_bf16_tie():
    """A group whose maximum sits on a bf16 rounding midpoint: the GPU may code either bf16 neighbour, and
    the (s, z) and codes the codec gives for the other one are accepted."""
    rng = np.random.default_rng(5)
    c = synth.round_to_device(rng.standard_normal((1, 32)), "bf16")
    j = int(np.argmax(c))
    lo = c[0, j]
    hi = synth.bits_to_f64(synth.bf16_bits(np.array([lo])) + np.uint16(1))[0]
    c[0, j] = (lo + hi) / 2
    for v in (lo, hi):
        b = c.copy()
        b[0, j] = v
        codes, meta = int2.quantize_int2_g32(b.astype(np.float32))
        check_int2_codes(c, codes, meta, "tie")


def test_int4_rule_through_bf16():
    """The windowed int4 format codes rows from their bf16 values: the rule then bounds the inputs by the bf16
    roundings of the accumulation window, and a code planted one off still fails."""
    c, c32 = _latents()
    b = synth.round_to_device(c32, "bf16").astype(np.float32)
    codes, scales = oracle.quantize_int4_g32(b)
    check_int4_cache(c, codes, scales, "bf16 rows", via_bf16=True)
    q = b.reshape(-1, 32) / scales.reshape(-1).astype(np.float32)[:, None]
    far = np.abs(np.abs(q - np.floor(q)) - 0.5) > 0.1
    k = codes.copy().reshape(-1, 32)
    g, j = np.argwhere(far & (np.abs(k) < 7))[0]
    k[g, j] -= 1
    with pytest.raises(AssertionError):
        check_int4_cache(c, k.reshape(codes.shape), scales, "planted", via_bf16=True)
