"""Pins of the oracle's append and attention against textbook attention (a library routine), closed-form
special cases and exact algebraic identities."""

import numpy as np
import pytest
import torch

import oracle


def _layer(seed, d, n_h, d_h, t):
    rng = np.random.default_rng(seed)
    wq, wk, wv = (rng.standard_normal((d, n_h * d_h)) * 0.3 for _ in range(3))
    x = rng.standard_normal((t, d))
    xc = rng.standard_normal((32, d))
    return wq, wk, wv, x, xc


def _complex_rope(a, kept, positions, d_h, theta=1e4):
    """Rotate the kept pairs of a [T, n_h, d_h] by multiplying (a_2p + i a_2p+1) with exp(i pos theta_p)."""
    out = a.copy()
    pos = np.asarray(positions, dtype=np.float64)
    for h, pairs in enumerate(kept):
        for p in pairs:
            z = (a[:, h, 2 * p] + 1j * a[:, h, 2 * p + 1]) * np.exp(1j * pos * theta ** (-2.0 * p / d_h))
            out[:, h, 2 * p], out[:, h, 2 * p + 1] = z.real, z.imag
    return out


def _textbook_mha(x, wq, wk, wv, n_h, d_h, kept):
    """Causal multi-head attention with RoPE on the `kept` pairs, via torch's scaled_dot_product_attention."""
    t = x.shape[0]
    q = _complex_rope((x @ wq).reshape(t, n_h, d_h), kept, np.arange(t), d_h)
    k = _complex_rope((x @ wk).reshape(t, n_h, d_h), kept, np.arange(t), d_h)
    v = (x @ wv).reshape(t, n_h, d_h)
    tq, tk, tv = (torch.from_numpy(np.ascontiguousarray(a.transpose(1, 0, 2)))[None] for a in (q, k, v))
    o = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, is_causal=True)
    return o[0].numpy().transpose(1, 0, 2)


def _mla_prefill(x, wq, wk, wv, xc, n_h, d_h, r, d_kv):
    conv = oracle.convert_layer(wq, wk, wv, xc, n_h, d_h, r, d_kv)
    t = x.shape[0]
    c, kr = oracle.append_ref(x, conv["w_dkv"], conv["w_krope"], conv["pair_idx"], np.arange(t), d_h, 1e4)
    q = (x @ wq).reshape(t, n_h, d_h)
    out = oracle.prefill_ref(q, c, kr, conv["w_uk"], conv["w_uv"], conv["pair_idx"], d_h, 1e4)
    return out, conv


def test_full_rank_all_pairs_is_plain_mha():
    """Full rank and r = d_h/2 reproduces textbook MHA with full RoPE."""
    d, n_h, d_h, t = 24, 2, 8, 11
    wq, wk, wv, x, xc = _layer(10, d, n_h, d_h, t)
    out, _ = _mla_prefill(x, wq, wk, wv, xc, n_h, d_h, d_h // 2, n_h * d_h)
    ref = _textbook_mha(x, wq, wk, wv, n_h, d_h, [range(d_h // 2)] * n_h)
    np.testing.assert_allclose(out, ref, rtol=0, atol=1e-11 * np.abs(ref).max())


def test_full_rank_partial_rope_is_partial_rope_mha():
    """Full rank with r < d_h/2 reproduces MHA whose RoPE acts only on each head's selected pairs."""
    d, n_h, d_h, r, t = 48, 2, 8, 2, 13
    wq, wk, wv, x, xc = _layer(11, d, n_h, d_h, t)
    out, conv = _mla_prefill(x, wq, wk, wv, xc, n_h, d_h, r, n_h * (2 * d_h - 2 * r))
    ref = _textbook_mha(x, wq, wk, wv, n_h, d_h, [list(p) for p in conv["pair_idx"]])
    np.testing.assert_allclose(out, ref, rtol=0, atol=1e-11 * np.abs(ref).max())


def test_full_rank_no_rope_is_nope_mha():
    d, n_h, d_h, t = 40, 2, 8, 9
    wq, wk, wv, x, xc = _layer(12, d, n_h, d_h, t)
    out, _ = _mla_prefill(x, wq, wk, wv, xc, n_h, d_h, 0, n_h * 2 * d_h)
    ref = _textbook_mha(x, wq, wk, wv, n_h, d_h, [[]] * n_h)
    np.testing.assert_allclose(out, ref, rtol=0, atol=1e-11 * np.abs(ref).max())


def _small_cache(seed=20, d=32, n_h=3, d_h=8, r=2, d_kv=6, t=17, positions=None):
    wq, wk, wv, x, xc = _layer(seed, d, n_h, d_h, t)
    conv = oracle.convert_layer(wq, wk, wv, xc, n_h, d_h, r, d_kv)
    pos = np.arange(t) if positions is None else positions
    c, kr = oracle.append_ref(x, conv["w_dkv"], conv["w_krope"], conv["pair_idx"], pos, d_h, 1e4)
    q = (x[-1] @ wq).reshape(n_h, d_h)
    return conv, c, kr, q


def test_absorbed_equals_unabsorbed():
    """Folding W_uk into the query and applying W_uv after the weighted latent sum is exact algebra."""
    for seed in (21, 22):
        conv, c, kr, q = _small_cache(seed)
        a = oracle.decode_ref(q, c, kr, conv["w_uk"], conv["w_uv"], conv["pair_idx"], 8, 1e4)
        b = oracle.absorbed_decode_ref(q, c, kr, conv["w_uk"], conv["w_uv"], conv["pair_idx"], 8, 1e4)
        np.testing.assert_allclose(a, b, rtol=0, atol=1e-12 * np.abs(a).max())


def test_decode_closed_forms():
    conv, c, kr, q = _small_cache(23)
    w_uv, w_uk, pidx = conv["w_uv"], conv["w_uk"], conv["pair_idx"]
    # one cached token: the output is that token's value
    one = oracle.decode_ref(q, c[:1], kr[:1], w_uk, w_uv, pidx, 8, 1e4)
    np.testing.assert_allclose(one, np.stack([c[0] @ w_uv[h] for h in range(3)]), atol=1e-14)
    # zero query: uniform weights, the output is the mean value
    zero = oracle.decode_ref(np.zeros_like(q), c, kr, w_uk, w_uv, pidx, 8, 1e4)
    np.testing.assert_allclose(zero, np.stack([(c @ w_uv[h]).mean(0) for h in range(3)]), atol=1e-14)


def test_decode_shift_invariance():
    """Shifting every position by a constant leaves the output unchanged (RoPE depends on n - m only)."""
    conv, c, kr, q = _small_cache(24)
    t = c.shape[0]
    base = oracle.attend_ref(q[None], [t - 1], c, kr, np.arange(t), conv["w_uk"], conv["w_uv"], conv["pair_idx"], 8, 1e4)
    conv2, c2, kr2, q2 = _small_cache(24, positions=np.arange(t) + 1000)
    shifted = oracle.attend_ref(q2[None], [t - 1 + 1000], c2, kr2, np.arange(t) + 1000, conv2["w_uk"], conv2["w_uv"],
                                conv2["pair_idx"], 8, 1e4)
    np.testing.assert_allclose(shifted, base, rtol=0, atol=1e-10 * np.abs(base).max())


def test_rope_rotation_properties():
    rng = np.random.default_rng(0)
    a, b = rng.standard_normal(50), rng.standard_normal(50)
    x, y = oracle.rope_rotate(a, b, np.zeros(50))
    np.testing.assert_array_equal(x, a)
    np.testing.assert_array_equal(y, b)
    phi = rng.uniform(-100, 100, 50)
    x, y = oracle.rope_rotate(a, b, phi)
    np.testing.assert_allclose(x * x + y * y, a * a + b * b, rtol=1e-13)
    z = (a + 1j * b) * np.exp(1j * phi)
    np.testing.assert_allclose(x, z.real, atol=1e-13)
    np.testing.assert_allclose(y, z.imag, atol=1e-13)


def test_latent_scale_sanity():
    """With iid N(0,1) activations and orthonormal W_dkv each latent component has unit variance."""
    conv, c, kr, q = _small_cache(25, d=64, t=4000, d_kv=6)
    assert np.mean(c ** 2) == pytest.approx(1.0, rel=0.1)
