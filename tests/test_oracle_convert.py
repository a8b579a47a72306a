"""Pins of the oracle's conversion against facts fixed by the pages and by linear algebra.

Nothing here compares the oracle with itself: each check uses a different route (brute force,
exhaustive search, an independent eigen-solver, a theorem's closed form)."""

import itertools

import numpy as np
import pytest

import oracle
from synth import layer_weights


def _rand_layer(seed, d, n_h, d_h, t=24):
    rng = np.random.default_rng(seed)
    wq, wk, wv = (rng.standard_normal((d, n_h * d_h)) * 0.02 for _ in range(3))
    x = rng.standard_normal((t, d))
    return wq, wk, wv, x


def _complex_rot(z, pos, p, d_h, theta=1e4):
    # Rotation of subspace p written as multiplication by a unit complex number (independent of rope_rotate).
    return z * np.exp(1j * pos * theta ** (-2.0 * p / d_h))


def test_pair_score_is_mean_cauchy_schwarz_bound_bruteforce():
    """Score = average over all (query token m, key token n) of ||q_m^p|| ||k_n^p||, checked by an O(T^2) loop;
    every RoPE-rotated pair product is bounded by its Cauchy-Schwarz bound (page 2, key designs)."""
    wq, wk, wv, x = _rand_layer(1, 16, 2, 8, t=10)
    q, k = oracle.calibration_qk(x, wq, wk, 2, 8)
    s = oracle.pair_scores(q, k)
    t = x.shape[0]
    for h in range(2):
        for p in range(4):
            acc = 0.0
            for m in range(t):
                for n in range(t):
                    qz = complex(q[m, h, 2 * p], q[m, h, 2 * p + 1])
                    kz = complex(k[n, h, 2 * p], k[n, h, 2 * p + 1])
                    bound = abs(qz) * abs(kz)
                    acc += bound
                    # <R(m) q, R(n) k> = Re( conj(R(m) q) * R(n) k )
                    dot = (np.conj(_complex_rot(qz, m, p, 8)) * _complex_rot(kz, n, p, 8)).real
                    assert abs(dot) <= bound + 1e-12
            assert abs(acc / t ** 2 - s[h, p]) <= 1e-12 * max(1.0, abs(s[h, p]))


def test_scores_invariant_under_rope():
    """RoPE rotations at positions 0..T-1 leave every pair norm, hence every score, unchanged."""
    wq, wk, wv, x = _rand_layer(2, 32, 3, 8, t=64)
    q, k = oracle.calibration_qk(x, wq, wk, 3, 8)
    qr, kr = q.copy(), k.copy()
    for p in range(4):
        for arr, out in ((q, qr), (k, kr)):
            z = arr[:, :, 2 * p] + 1j * arr[:, :, 2 * p + 1]
            z = z * np.exp(1j * np.arange(64)[:, None] * 1e4 ** (-2.0 * p / 8))
            out[:, :, 2 * p], out[:, :, 2 * p + 1] = z.real, z.imag
    np.testing.assert_allclose(oracle.pair_scores(qr, kr), oracle.pair_scores(q, k), rtol=1e-13, atol=0)


def test_selection_exhaustive_tiny_config():
    """On the tiny config (9 heads x 32 pairs, r = 4, 64 calibration tokens) the chosen set of every head
    maximises the summed score over all C(32,4) = 35960 subsets."""
    wq, wk, wv, xc = layer_weights("tiny")
    q, k = oracle.calibration_qk(xc, wq, wk, 9, 64)
    s = oracle.pair_scores(q, k)
    idx = oracle.select_pairs(s, 4)
    combos = np.array(list(itertools.combinations(range(32), 4)))
    for h in range(9):
        sums = s[h][combos].sum(axis=1)
        assert s[h][idx[h]].sum() == pytest.approx(sums.max(), rel=1e-15, abs=0)
        assert list(idx[h]) == sorted(idx[h])
        # the optimum is unique unless there is a tie at the boundary
        srt = np.sort(s[h])[::-1]
        if srt[3] > srt[4] * (1 + 1e-9):
            assert np.count_nonzero(sums >= sums.max() * (1 - 1e-15)) == 1
    # page 2, key findings: different heads prefer different frequency subspaces
    assert len({tuple(r) for r in idx}) > 1


def test_selection_ties_and_full():
    s = np.array([[1.0, 3.0, 3.0, 0.5, 3.0]])
    assert oracle.select_pairs(s, 2).tolist() == [[1, 2]]  # tie among 1, 2, 4: lower indices win
    assert oracle.select_pairs(s, 5).tolist() == [[0, 1, 2, 3, 4]]  # r = d_h/2 keeps all pairs
    assert oracle.select_pairs(s, 0).shape == (1, 0)


def test_split_dims_is_partition():
    idx = np.array([[0, 3], [1, 2]], dtype=np.int32)
    rope, nope = oracle.split_dims(idx, 8)
    assert rope[0] == [0, 1, 6, 7] and nope[0] == [2, 3, 4, 5]
    assert rope[1] == [2, 3, 4, 5] and nope[1] == [0, 1, 6, 7]


def _eig_singular_values(a):
    # singular values via the symmetric eigen-solver on the smaller Gram matrix (not the SVD routine)
    g = a @ a.T if a.shape[0] <= a.shape[1] else a.T @ a
    w = np.linalg.eigvalsh(g)[::-1]
    return np.sqrt(np.clip(w, 0, None))


@pytest.mark.parametrize("d,n_h,d_h,r,d_kv", [(64, 4, 16, 2, 20), (48, 3, 8, 1, 7), (576, 9, 64, 4, 32)])
def test_joint_svd_eckart_young(d, n_h, d_h, r, d_kv):
    """Truncation error of the joint SVD equals the discarded singular values (Eckart-Young), in Frobenius
    and spectral norm, with singular values from an independent eigen-solver; W_dkv is orthonormal."""
    wq, wk, wv, x = _rand_layer(3, d, n_h, d_h)
    pidx = oracle.select_pairs(oracle.pair_scores(*oracle.calibration_qk(x, wq, wk, n_h, d_h)), r)
    out = oracle.joint_svd(wk, wv, pidx, n_h, d_h, d_kv)
    m = out["m"]
    assert m.shape == (d, n_h * (d_h - 2 * r) + n_h * d_h)
    z = np.concatenate([np.concatenate(list(out["w_uk"]), axis=1), np.concatenate(list(out["w_uv"]), axis=1)], axis=1)
    err = m - out["w_dkv"] @ z
    sig = _eig_singular_values(m)
    np.testing.assert_allclose(out["sigma"], sig[: len(out["sigma"])], rtol=1e-9)
    tail = np.sum(sig[d_kv:] ** 2)
    assert np.sum(err ** 2) == pytest.approx(tail, rel=1e-9)
    assert _eig_singular_values(err)[0] == pytest.approx(sig[d_kv], rel=1e-8)
    np.testing.assert_allclose(out["w_dkv"].T @ out["w_dkv"], np.eye(d_kv), atol=1e-12)
    # column order of M does not change the singular values
    perm = np.random.default_rng(0).permutation(m.shape[1])
    np.testing.assert_allclose(_eig_singular_values(m[:, perm])[:d_kv], sig[:d_kv], rtol=1e-9)


def test_joint_never_worse_than_split():
    """At equal total latent width the joint SVD error is never larger than SVD_split's (page 2, ablations)."""
    d, n_h, d_h, r = 96, 4, 16, 2
    wq, wk, wv, x = _rand_layer(4, d, n_h, d_h)
    pidx = oracle.select_pairs(oracle.pair_scores(*oracle.calibration_qk(x, wq, wk, n_h, d_h)), r)
    for d_kv in (8, 16, 32, 48):
        j = oracle.joint_svd(wk, wv, pidx, n_h, d_h, d_kv)
        zk = np.concatenate(list(j["w_uk"]), axis=1)
        zv = np.concatenate(list(j["w_uv"]), axis=1)
        sk, sv, wkn = oracle.split_svd(wk, wv, pidx, n_h, d_h, d_kv // 2, d_kv - d_kv // 2)
        ej = np.sum((wkn - j["w_dkv"] @ zk) ** 2) + np.sum((wv - j["w_dkv"] @ zv) ** 2)
        es = np.sum((wkn - sk) ** 2) + np.sum((wv - sv) ** 2)
        assert ej <= es * (1 + 1e-12)


def test_full_rank_reconstructs_exactly():
    d, n_h, d_h, r = 64, 2, 8, 1
    wq, wk, wv, x = _rand_layer(5, d, n_h, d_h)
    pidx = oracle.select_pairs(oracle.pair_scores(*oracle.calibration_qk(x, wq, wk, n_h, d_h)), r)
    rank = n_h * (2 * d_h - 2 * r)
    j = oracle.joint_svd(wk, wv, pidx, n_h, d_h, rank)
    z = np.concatenate([np.concatenate(list(j["w_uk"]), axis=1), np.concatenate(list(j["w_uv"]), axis=1)], axis=1)
    np.testing.assert_allclose(j["w_dkv"] @ z, j["m"], atol=1e-14)
    # [W_knope, W_krope] is a column permutation of W_k
    rope, nope = oracle.split_dims(pidx, d_h)
    cols = sorted([h * d_h + i for h in range(n_h) for i in nope[h]] + [h * d_h + i for h in range(n_h) for i in rope[h]])
    assert cols == list(range(n_h * d_h))
    np.testing.assert_array_equal(j["w_krope"][:, 0:2], wk[:, [rope[0][0], rope[0][1]]])
