"""The library's offline converter (Gram-matrix eigen-decomposition) against the oracle's conversion
(explicit SVD): bit-exact pair selection, equal low-rank products and singular values."""

import numpy as np
import pytest

import oracle
from mla_latent_kv_cache_amd.convert import convert_layer
from synth import FAMILIES, layer_weights


@pytest.mark.parametrize("family,r,d_kv", [("tiny", 4, 32), ("mid", 4, 512), ("mid", 2, 256)])
def test_converter_matches_oracle(family, r, d_kv):
    d, n_h, d_h, _ = FAMILIES[family]
    wq, wk, wv, xc = layer_weights(family)
    ref = oracle.convert_layer(wq, wk, wv, xc, n_h, d_h, r, d_kv)
    got = convert_layer(wq, wk, wv, xc, n_h, d_h, r, d_kv)
    np.testing.assert_array_equal(got["pair_idx"], ref["pair_idx"])
    # ranking gaps: how far the selection is from a tie (reported, and large for these seeds)
    s = np.sort(ref["scores"], axis=1)[:, ::-1]
    assert np.all((s[:, r - 1] - s[:, r]) / s[:, r - 1] > 1e-9)
    np.testing.assert_array_equal(got["w_krope"], ref["w_krope"])
    np.testing.assert_allclose(got["sigma"][: d_kv + 1], ref["sigma"][: d_kv + 1], rtol=1e-10)
    # factors are unique up to an orthogonal change of latent basis: compare the products
    for key in ("w_uk", "w_uv"):
        a = np.einsum("dk,hke->hde", got["w_dkv"], got[key])
        b = np.einsum("dk,hke->hde", ref["w_dkv"], ref[key])
        assert np.linalg.norm(a - b) <= 1e-10 * np.linalg.norm(b)
    np.testing.assert_allclose(got["w_dkv"].T @ got["w_dkv"], np.eye(d_kv), atol=1e-10)


@pytest.mark.parametrize("strategy,svd", [("high", "joint"), ("low", "split"), ("uniform", "split"), ("2-norm", "split")])
def test_converter_variants_match_oracle(strategy, svd):
    """The ablation variants: the same kept subspaces bit for bit, and the same rank-truncated K_nope / V maps
    W_dkv W_uk,h and W_dkv W_uv,h (for SVD_split each half of the latent is unique up to a rotation within it)."""
    d, n_h, d_h, _ = FAMILIES["tiny"]
    r, d_kv = 4, 32
    wq, wk, wv, xc = layer_weights("tiny")
    ref = oracle.convert_layer(wq, wk, wv, xc, n_h, d_h, r, d_kv, strategy=strategy, svd=svd)
    got = convert_layer(wq, wk, wv, xc, n_h, d_h, r, d_kv, strategy=strategy, svd=svd)
    np.testing.assert_array_equal(got["pair_idx"], ref["pair_idx"])
    np.testing.assert_array_equal(got["w_krope"], ref["w_krope"])
    assert got["w_dkv"].shape == (d, d_kv) and got["w_uk"].shape == ref["w_uk"].shape
    for key in ("w_uk", "w_uv"):
        a = np.einsum("dk,hke->hde", got["w_dkv"], got[key])
        b = np.einsum("dk,hke->hde", ref["w_dkv"], ref[key])
        assert np.linalg.norm(a - b) <= 1e-10 * np.linalg.norm(b)
    if svd == "split":
        rk = d_kv // 2
        assert np.all(got["w_uk"][:, rk:] == 0) and np.all(got["w_uv"][:, :rk] == 0)
        np.testing.assert_allclose(got["sigma_k"][: rk + 1], ref["sigma_k"][: rk + 1], rtol=1e-10)
        np.testing.assert_allclose(got["sigma_v"][: rk + 1], ref["sigma_v"][: rk + 1], rtol=1e-10)


def test_converter_rejects_unknown_variants():
    d, n_h, d_h, _ = FAMILIES["tiny"]
    wq, wk, wv, xc = layer_weights("tiny")
    with pytest.raises(ValueError):
        convert_layer(wq, wk, wv, xc, n_h, d_h, 4, 32, strategy="middle")
    with pytest.raises(ValueError):
        convert_layer(wq, wk, wv, xc, n_h, d_h, 4, 32, svd="separate")
    with pytest.raises(ValueError):
        convert_layer(wq, wk, wv, xc, n_h, d_h, 4, 2 * d + 2, svd="split")
