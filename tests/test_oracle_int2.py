"""Pins of the oracle's 2-bit latent codec and recent-token window (oracle/int2.py): hand-worked golden
groups, nearest-level and error-bound properties checked in fp64, a brute-force ring simulation, and the
cache-byte accounting of the format."""

import json
import os

import numpy as np
import pytest

import oracle
from oracle import int2

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def test_int2_worked_example():
    with open(os.path.join(GOLDEN, "int2_worked_example.json")) as f:
        groups = json.load(f)["groups"]
    for g in groups:
        x = np.array(g["x"], dtype=np.float32)
        codes, meta = int2.quantize_int2_g32(x)
        assert codes.tolist() == g["codes"]
        assert float(meta[0, 0]) == g["s"] and float(meta[0, 1]) == g["z"]
        assert int2.pack_crumbs(codes).tolist() == g["bytes"]
        assert int2.unpack_crumbs(np.array(g["bytes"], dtype=np.uint8)).tolist() == g["codes"]
        if "dequant_of_code_3" in g:
            deq = int2.dequant_int2(codes, meta)
            assert deq[0] == g["dequant_of_code_3"]
    # constant group: every element dequantises to z exactly
    c, m = int2.quantize_int2_g32(np.array(groups[2]["x"], dtype=np.float32))
    assert np.all(int2.dequant_int2(c, m) == 5.0)


def test_int2_nearest_level_and_error_bound():
    """Each code names the nearest of the four levels z + c s (fp64, with the stored fp16 s and z; ties only
    up to fp32 rounding of the quotient), and every value inside [z, z + 3s] is within s/2 of its level."""
    rng = np.random.default_rng(3)
    x = (rng.standard_normal((400, 64)) * rng.lognormal(size=(400, 1)) + rng.standard_normal((400, 1))).astype(np.float32)
    codes, meta = int2.quantize_int2_g32(x)
    s = meta[..., 0].astype(np.float64)
    z = meta[..., 1].astype(np.float64)
    xv = x.reshape(400, 2, 32).astype(np.float64)
    lev = z[..., None, None] + np.arange(4)[None, None, :, None] * s[..., None, None]  # [400, 2, 4, 1]
    dist = np.abs(xv[:, :, None, :] - lev)  # [400, 2, 4, 32]
    cg = codes.reshape(400, 2, 32).astype(np.int64)
    chosen = np.take_along_axis(dist, cg[:, :, None, :], axis=2)[:, :, 0, :]
    assert np.all(chosen <= dist.min(axis=2) + 1e-6 * s[..., None])
    inside = (xv >= z[..., None]) & (xv <= z[..., None] + 3 * s[..., None])
    deq = int2.dequant_int2(codes, meta).reshape(400, 2, 32)
    err = np.abs(deq - xv)
    assert np.all(err[inside] <= (0.5 * s[..., None] * (1 + 1e-6) + 1e-7 * np.abs(xv))[inside])
    # the group minimum maps to code 0, the maximum to code 3 (z and s are exact here: values are fp16-grid)
    g = np.round(x.reshape(-1, 32) * 64) / 64
    cg2, mg2 = int2.quantize_int2_g32(g.astype(np.float32))
    cg2 = cg2.reshape(-1, 32)
    rows = np.arange(g.shape[0])
    span = g.max(axis=1) - g.min(axis=1)
    ok = span > 0
    assert np.all(cg2[rows, np.argmin(g, axis=1)][ok] == 0)
    assert np.all(cg2[rows, np.argmax(g, axis=1)][ok] == 3)


def test_int2_ties_half_even_and_fp32_decisions():
    # s = 1, z = 0: quotients 0.5, 1.5, 2.5 are exact ties and go to the even code
    x = np.zeros(32, dtype=np.float32)
    x[:5] = [0.5, 1.5, 2.5, 3.0, 0.0]
    c, m = int2.quantize_int2_g32(x)
    assert c[:5].tolist() == [0, 2, 2, 3, 0]
    # the quotient is an fp32 division: a value just above the tie in fp32 rounds up
    y = x.copy()
    y[0] = np.nextafter(np.float32(0.5), np.float32(1.0))
    assert int2.quantize_int2_g32(y)[0][0] == 1


def test_crumb_bit_layout():
    assert int2.pack_crumbs(np.array([0, 1, 2, 3], dtype=np.uint8)).tolist() == [0b11100100]
    assert int2.pack_crumbs(np.array([3, 0, 0, 0, 0, 0, 0, 2], dtype=np.uint8)).tolist() == [3, 0b10000000]
    rng = np.random.default_rng(4)
    c = rng.integers(0, 4, size=(7, 64)).astype(np.uint8)
    assert np.array_equal(int2.unpack_crumbs(int2.pack_crumbs(c)), c)


def _ring_by_simulation(appends, W):
    """Push tokens one append at a time into a ring of W slots (overwriting the oldest), recording which
    tokens ever left it; returns (slot -> position, set of positions quantised)."""
    slots = [-1] * W
    quantised = set()
    L = 0
    for t_new in appends:
        for p in range(L, L + t_new):
            if W == 0:
                quantised.add(p)
                continue
            old = slots[p % W]
            if old >= 0:
                quantised.add(old)
            slots[p % W] = p
        L += t_new
    return np.array(slots), quantised, L


@pytest.mark.parametrize("appends,W", [([300], 128), ([100, 1, 1, 1], 128), ([50], 128), ([129, 200, 3], 64),
                                       ([5, 5, 5], 0), ([1] * 40, 16), ([128], 128), ([129], 128)])
def test_window_matches_ring_simulation(appends, W):
    """The window of the last min(L, W) positions is exactly what a ring of W slots holds after the appends,
    and the quantised positions are exactly those that left it, whatever the append sizes."""
    slots, quantised, L = _ring_by_simulation(appends, W)
    if W:
        np.testing.assert_array_equal(int2.ring_positions(L, W), slots)
    assert quantised == set(range(L - int2.window_len(L, W)))
    rng = np.random.default_rng(L + W)
    rows = np.round(rng.standard_normal((L, 64)) * 256) / 256
    eff, codes, meta = int2.windowed_latent(rows, W)
    nq = L - int2.window_len(L, W)
    assert codes.shape == (nq, 64) and meta.shape == (nq, 2, 2)
    np.testing.assert_array_equal(eff[nq:], rows[nq:])
    for p in range(nq):  # old rows: their own group codes, dequantised
        c1, m1 = int2.quantize_int2_g32(rows[p].astype(np.float32))
        np.testing.assert_array_equal(eff[p], int2.dequant_int2(c1, m1))


def test_int2_cache_bytes():
    # Llama-2-7B layer, d_kv 512, r 4: 512 latent values at 2 bits + (fp16 s, fp16 z) per group of 32 + 256 bf16 RoPE keys
    b = oracle.cache_bytes_per_token(32, 4, 512, latent_bits=2, scale_bytes=4)
    assert b == 128 + 64 + 512 == 704
    mha = oracle.mha_bytes_per_token(32, 128)
    assert oracle.reduction_pct(b, mha) == pytest.approx(100 * (1 - 704 / 16384))
    # the window adds W * d_kv * 2 bytes per sequence: 128 KiB at W = 128, d_kv = 512
    assert 128 * 512 * 2 == 131072


@pytest.mark.parametrize("appends,W", [([300], 128), ([129, 200, 3], 64), ([5, 5, 5], 0), ([50], 128)])
def test_int4_window_matches_ring_simulation(appends, W):
    """The int4 cache with a window: the rows a ring of W slots still holds after the appends stay bf16, every
    row that left it (or never entered it) is the int4 codec of its own bf16 values, row by row; W = 0 is the
    plain int4 codec of the bf16 rows."""
    slots, quantised, L = _ring_by_simulation(appends, W)
    rng = np.random.default_rng(L + W + 1)
    rows = np.round(rng.standard_normal((L, 64)) * 256) / 256
    eff, codes, scales = oracle.windowed_latent_int4(rows, W)
    nq = L - int2.window_len(L, W)
    assert set(range(nq)) == quantised
    assert codes.shape == (nq, 64) and scales.shape == (nq, 2)
    np.testing.assert_array_equal(eff[nq:], rows[nq:])
    for p in sorted(quantised):
        c1, s1 = oracle.quantize_int4_g32(rows[p].astype(np.float32))
        np.testing.assert_array_equal(eff[p], oracle.dequant_int4(c1, s1))
    if W == 0:
        c_all, s_all = oracle.quantize_int4_g32(rows.astype(np.float32))
        np.testing.assert_array_equal(eff, oracle.dequant_int4(c_all, s_all))
