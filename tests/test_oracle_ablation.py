"""Pins of the oracle's ablation variants (partial-RoPE strategies S_high / S_low / S_uniform, SVD_split at
the same latent width) and of the error measures of oracle.ablation.

Each check takes another route than the code it pins: RoPE angular speeds written out, planted singular
spectra (Eckart-Young closed forms), matrices with a known shared column space, torch's attention."""

import numpy as np
import pytest
import torch

import oracle
import synth
from oracle import ablation


def _speed(p, d_h, theta=1e4):
    # angular speed (radians per position) of RoPE subspace p in the RoFormer rotation
    return theta ** (-2.0 * p / d_h)


@pytest.mark.parametrize("n_pairs,r", [(8, 3), (32, 4), (64, 4), (64, 8), (64, 5), (16, 16), (16, 0)])
def test_fixed_strategies(n_pairs, r):
    """S_high keeps the r fastest-turning subspaces, S_low the r slowest, S_uniform r subspaces spaced evenly
    from the fastest (gaps differ by at most one); every head gets the same set; r = d_h/2 keeps all."""
    d_h = 2 * n_pairs
    scores = np.random.default_rng(n_pairs + r).random((3, n_pairs))
    speeds = np.array([_speed(p, d_h) for p in range(n_pairs)])
    hi = oracle.select_pairs_by("high", scores, r)
    lo = oracle.select_pairs_by("low", scores, r)
    un = oracle.select_pairs_by("uniform", scores, r)
    for sel in (hi, lo, un):
        assert sel.dtype == np.int32 and sel.shape == (3, r)
        assert all(list(row) == list(sel[0]) for row in sel)
        assert list(sel[0]) == sorted(set(sel[0].tolist()))
    order = np.argsort(-speeds, kind="stable")
    assert set(hi[0].tolist()) == set(order[:r].tolist())
    assert set(lo[0].tolist()) == set(order[n_pairs - r:].tolist())
    if r:
        assert un[0][0] == 0
        gaps = np.diff(np.append(un[0], n_pairs))
        assert gaps.max() - gaps.min() <= 1 and gaps.sum() == n_pairs
    if r == n_pairs:
        for sel in (hi, lo, un):
            assert list(sel[0]) == list(range(n_pairs))


def test_fixed_strategy_examples():
    s = np.zeros((2, 8))
    assert oracle.select_pairs_by("high", s, 3).tolist() == [[0, 1, 2]] * 2
    assert oracle.select_pairs_by("low", s, 3).tolist() == [[5, 6, 7]] * 2
    assert oracle.select_pairs_by("uniform", s, 3).tolist() == [[0, 2, 5]] * 2
    assert oracle.select_pairs_by("uniform", np.zeros((1, 64)), 4).tolist() == [[0, 16, 32, 48]]
    with pytest.raises(ValueError):
        oracle.select_pairs_by("random", s, 2)


def test_two_norm_drops_least_score():
    """S_2-norm keeps, per head, the largest possible score mass, so its dropped share is never above a fixed
    strategy's (equality only when the fixed set is also a top-r set)."""
    rng = np.random.default_rng(5)
    for _ in range(20):
        s = rng.lognormal(size=(4, 16))
        best = ablation.dropped_score(s, oracle.select_pairs_by("2-norm", s, 3))
        for strat in ("high", "low", "uniform"):
            assert best <= ablation.dropped_score(s, oracle.select_pairs_by(strat, s, 3)) + 1e-15


def test_dropped_score_hand_example():
    s = np.array([[4.0, 3.0, 2.0, 1.0], [1.0, 1.0, 1.0, 1.0]])
    idx = np.array([[0, 3], [1, 2]])
    assert ablation.dropped_score(s, idx) == pytest.approx(((3 + 2) / 10 + 2 / 4) / 2, rel=1e-15)


def _orthonormal(rng, n, k):
    q, _ = np.linalg.qr(rng.standard_normal((n, k)))
    return q


def _layer_with_nope(w_knope, w_rope_cols, pair_idx, n_h, d_h):
    """W_k whose NoPE columns (per head, ascending dims) are w_knope and RoPE columns w_rope_cols."""
    rope, nope = oracle.split_dims(pair_idx, d_h)
    d = w_knope.shape[0]
    w_k = np.zeros((d, n_h * d_h))
    dn = d_h - 2 * pair_idx.shape[1]
    for h in range(n_h):
        w_k[:, [h * d_h + i for i in nope[h]]] = w_knope[:, h * dn:(h + 1) * dn]
        w_k[:, [h * d_h + i for i in rope[h]]] = w_rope_cols[:, h * 2 * pair_idx.shape[1]:(h + 1) * 2 * pair_idx.shape[1]]
    return w_k


def test_split_layer_planted_spectra():
    """SVD_split with planted singular values: K and V errors are the tails of their own spectra
    (Eckart-Young), the latent has d_kv columns, each half orthonormal, up-projections zero on the other half."""
    rng = np.random.default_rng(11)
    d, n_h, d_h, r, d_kv = 40, 2, 8, 1, 10
    dn = d_h - 2 * r
    pidx = np.array([[1], [3]], dtype=np.int32)
    sk = np.array([9.0, 7.0, 5.0, 4.0, 3.0, 2.0, 1.0, 0.5, 0.25, 0.1, 0.05, 0.01])
    sv = np.array([8.0, 6.0, 4.5, 3.5, 2.5, 1.5, 1.25, 1.0, 0.75, 0.5, 0.3, 0.2, 0.1, 0.05, 0.02, 0.01])
    w_knope = _orthonormal(rng, d, n_h * dn) @ np.diag(sk) @ _orthonormal(rng, n_h * dn, n_h * dn).T
    w_v = _orthonormal(rng, d, n_h * d_h) @ np.diag(sv) @ _orthonormal(rng, n_h * d_h, n_h * d_h).T
    w_k = _layer_with_nope(w_knope, rng.standard_normal((d, n_h * 2 * r)), pidx, n_h, d_h)
    out = oracle.split_svd_layer(w_k, w_v, pidx, n_h, d_h, d_kv)
    rk, rv = d_kv // 2, d_kv - d_kv // 2
    assert out["w_dkv"].shape == (d, d_kv)
    np.testing.assert_allclose(out["w_dkv"][:, :rk].T @ out["w_dkv"][:, :rk], np.eye(rk), atol=1e-12)
    np.testing.assert_allclose(out["w_dkv"][:, rk:].T @ out["w_dkv"][:, rk:], np.eye(rv), atol=1e-12)
    assert np.all(out["w_uk"][:, rk:, :] == 0) and np.all(out["w_uv"][:, :rk, :] == 0)
    k_hat = np.concatenate([out["w_dkv"] @ out["w_uk"][h] for h in range(n_h)], axis=1)
    v_hat = np.concatenate([out["w_dkv"] @ out["w_uv"][h] for h in range(n_h)], axis=1)
    assert np.sum((w_knope - k_hat) ** 2) == pytest.approx(np.sum(sk[rk:] ** 2), rel=1e-9)
    assert np.sum((w_v - v_hat) ** 2) == pytest.approx(np.sum(sv[rv:] ** 2), rel=1e-9)
    np.testing.assert_allclose(out["sigma_k"], sk, rtol=1e-12)
    np.testing.assert_allclose(out["sigma_v"], sv, rtol=1e-12)
    np.testing.assert_array_equal(out["w_krope"], oracle.joint_svd(w_k, w_v, pidx, n_h, d_h, d_kv)["w_krope"])


def test_joint_uses_shared_latent_split_wastes_it():
    """K_nope and V drawing on one rank-6 column space: the joint SVD at d_kv = 6 is exact, SVD_split at the
    same width keeps 3 dims per side and cannot be (the pages' reason for the joint SVD)."""
    rng = np.random.default_rng(12)
    d, n_h, d_h, r, rho = 32, 2, 8, 1, 6
    dn = d_h - 2 * r
    a = rng.standard_normal((d, rho))
    w_knope = a @ rng.standard_normal((rho, n_h * dn))
    w_v = a @ rng.standard_normal((rho, n_h * d_h))
    pidx = np.array([[0], [2]], dtype=np.int32)
    w_k = _layer_with_nope(w_knope, rng.standard_normal((d, n_h * 2 * r)), pidx, n_h, d_h)
    j = oracle.joint_svd(w_k, w_v, pidx, n_h, d_h, rho)
    s = oracle.split_svd_layer(w_k, w_v, pidx, n_h, d_h, rho)
    assert ablation.kv_fit_error(j, n_h) < 1e-12
    assert ablation.kv_fit_error(s, n_h) > 1e-2
    # and with twice the width, the split one is exact too
    assert ablation.kv_fit_error(oracle.split_svd_layer(w_k, w_v, pidx, n_h, d_h, 2 * rho), n_h) < 1e-12


def test_kv_fit_error_eckart_young():
    """For the joint SVD the K/V fit error is the discarded singular-value tail, from an eigen-solver."""
    wq, wk, wv, xc = synth.structured_layer_weights("tiny")
    conv = oracle.convert_layer(wq, wk, wv, xc, 9, 64, 4, 32)
    g = conv["m"] @ conv["m"].T
    ev = np.sort(np.clip(np.linalg.eigvalsh(g), 0, None))[::-1]
    want = np.sqrt(ev[32:].sum() / ev.sum())
    assert ablation.kv_fit_error(conv, 9) == pytest.approx(want, rel=1e-8)


def test_mha_ref_is_textbook_attention():
    """mha_ref against torch's scaled_dot_product_attention on RoPE'd q, k written with complex numbers,
    for full RoPE and for per-head kept sets."""
    rng = np.random.default_rng(13)
    t, d, n_h, d_h = 21, 24, 3, 8
    wq, wk, wv = (rng.standard_normal((d, n_h * d_h)) * 0.3 for _ in range(3))
    x = rng.standard_normal((t, d))
    for kept in (None, [[0, 3], [1], []]):
        got = ablation.mha_ref(x, wq, wk, wv, n_h, d_h, 1e4, kept=kept)
        qs, ks = [], []
        for w in (wq, wk):
            z = (x @ w).reshape(t, n_h, d_h // 2, 2)
            zc = z[..., 0] + 1j * z[..., 1]
            for h in range(n_h):
                for p in (range(d_h // 2) if kept is None else kept[h]):
                    zc[:, h, p] *= np.exp(1j * np.arange(t) * _speed(p, d_h))
            (qs if w is wq else ks).append(np.stack([zc.real, zc.imag], axis=-1).reshape(t, n_h, d_h))
        v = (x @ wv).reshape(t, n_h, d_h)
        tq, tk, tv = (torch.from_numpy(np.ascontiguousarray(a.transpose(1, 0, 2)))[None] for a in (qs[0], ks[0], v))
        ref = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, is_causal=True)[0].numpy().transpose(1, 0, 2)
        np.testing.assert_allclose(got, ref, rtol=0, atol=1e-12 * np.abs(ref).max())


def test_converted_ref_full_rank_is_partial_rope_mha():
    """At full latent rank the converted layer (either SVD variant, any strategy) is MHA with RoPE on the
    kept subspaces, so end-to-end error = partial-RoPE error."""
    rng = np.random.default_rng(14)
    t, d, n_h, d_h, r = 17, 10, 2, 8, 1  # W_k,nope [10, 12] and W_v [10, 16] both have rank 10
    wq, wk, wv = (rng.standard_normal((d, n_h * d_h)) * 0.3 for _ in range(3))
    xc, x = rng.standard_normal((12, d)), rng.standard_normal((t, d))
    for strategy, svd in (("low", "joint"), ("uniform", "split"), ("2-norm", "split")):
        d_kv = d if svd == "joint" else 2 * d
        conv = oracle.convert_layer(wq, wk, wv, xc, n_h, d_h, r, d_kv, strategy=strategy, svd=svd)
        got = ablation.converted_ref(x, wq, conv, d_h, 1e4)
        ref = ablation.mha_ref(x, wq, wk, wv, n_h, d_h, 1e4, kept=conv["pair_idx"])
        np.testing.assert_allclose(got, ref, rtol=0, atol=1e-10 * np.abs(ref).max())


def test_ablation_ranking_on_structured_layer():
    """The guaranteed orderings, and the pages' qualitative ranking, on the seeded structured layer of the
    tiny family (heads with their own frequency bands, K and V on a shared input subspace):
    S_2-norm drops the least score and joint fits K/V no worse than split (both theorems); end to end,
    S_2-norm is best and S_low worst, and joint beats split for every strategy (measured on this workload)."""
    wq, wk, wv, xc = synth.structured_layer_weights("tiny")
    x = synth.eval_x("tiny", 192)
    rows = ablation.ablation_rows(wq, wk, wv, xc, x, 9, 64, 4, 32)
    by = {(row["strategy"], row["svd"]): row for row in rows}
    for strat in ("high", "uniform", "low"):
        assert by[("2-norm", "joint")]["dropped_score"] <= by[(strat, "joint")]["dropped_score"]
    for strat in ablation.STRATEGIES:
        assert by[(strat, "joint")]["kv_fit_err"] <= by[(strat, "split")]["kv_fit_err"] * (1 + 1e-12)
        assert by[(strat, "joint")]["end_to_end_err"] < by[(strat, "split")]["end_to_end_err"]
    e2e = {s: by[(s, "joint")]["end_to_end_err"] for s in ablation.STRATEGIES}
    assert e2e["2-norm"] == min(e2e.values()) and e2e["low"] == max(e2e.values())
