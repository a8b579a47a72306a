"""Pins of oracle/paged.py: the page gather against an explicit position-by-position copy and the identity
table, and multi-query decode against single-query decodes over truncated caches."""

import numpy as np
import pytest

import oracle


def test_gather_pages_identity_and_permutation():
    rng = np.random.default_rng(1)
    P, pages_per_seq, B = 4, 5, 3
    logical = rng.standard_normal((B, P * pages_per_seq, 6))
    # identity table: the pool is the contiguous cache
    ident = np.arange(B * pages_per_seq).reshape(B, pages_per_seq)
    pool = logical.reshape(B * P * pages_per_seq, 6)
    for b in range(B):
        np.testing.assert_array_equal(oracle.gather_pages(pool, ident[b], 17, P), logical[b, :17])
    # a permuted table over a larger pool: write each logical page to its physical page, read it back
    perm = rng.permutation(40)[: B * pages_per_seq].reshape(B, pages_per_seq)
    pool2 = np.full((40 * P, 6), np.nan)
    for b in range(B):
        for j in range(pages_per_seq):
            pool2[perm[b, j] * P:(perm[b, j] + 1) * P] = logical[b, j * P:(j + 1) * P]
    for b in range(B):
        for L in (0, 1, 4, 5, 20):
            np.testing.assert_array_equal(oracle.gather_pages(pool2, perm[b], L, P), logical[b, :L])


def _small(seed=3, t=13, d=24, n_h=3, d_h=8, r=2, d_kv=6):
    rng = np.random.default_rng(seed)
    wq, wk, wv = (rng.standard_normal((d, n_h * d_h)) * 0.3 for _ in range(3))
    xc, x = rng.standard_normal((16, d)), rng.standard_normal((t, d))
    conv = oracle.convert_layer(wq, wk, wv, xc, n_h, d_h, r, d_kv)
    c, kr = oracle.append_ref(x, conv["w_dkv"], conv["w_krope"], conv["pair_idx"], np.arange(t), d_h, 1e4)
    q = (x @ wq).reshape(t, n_h, d_h)
    return conv, c, kr, q


@pytest.mark.parametrize("n_q", [1, 2, 4, 13, 15])
def test_multi_query_is_decodes_over_prefixes(n_q):
    """Query i of n_q equals a single-query decode over the cache truncated after its own position; queries at
    negative positions give zero rows."""
    conv, c, kr, q = _small()
    L = c.shape[0]
    qq = np.stack([q[max(L - n_q + i, 0)] for i in range(n_q)])
    got = oracle.multi_query_decode_ref(qq, c, kr, conv["w_uk"], conv["w_uv"], conv["pair_idx"], 8, 1e4)
    for i in range(n_q):
        pos = L - n_q + i
        if pos < 0:
            assert np.all(got[i] == 0)
            continue
        ref = oracle.decode_ref(qq[i], c[:pos + 1], kr[:pos + 1], conv["w_uk"], conv["w_uv"], conv["pair_idx"], 8, 1e4)
        np.testing.assert_allclose(got[i], ref, rtol=0, atol=1e-13)
