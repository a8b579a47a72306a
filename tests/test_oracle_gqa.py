"""Pins of the oracle's grouped-query conversion (oracle.convert_gqa_layer) and the library converter's
n_kv_heads option against it.

Routes independent of the code pinned: an O(T^2) loop over token pairs and query heads for the group score,
exhaustive subset search, torch's scaled-dot-product attention over repeated KV heads at full rank, an
eigen-solver for the truncation error, and the one-query-head-per-group case against the MHA conversion."""

import itertools

import numpy as np
import pytest
import torch

import oracle
import synth
from mla_latent_kv_cache_amd.convert import convert_layer


def _rand_gqa(seed, d, n_h, n_kv, d_h, t=24, scale=0.3):
    rng = np.random.default_rng(seed)
    wq = rng.standard_normal((d, n_h * d_h)) * scale
    wk, wv = (rng.standard_normal((d, n_kv * d_h)) * scale for _ in range(2))
    return wq, wk, wv, rng.standard_normal((t, d)), rng.standard_normal((t + 5, d))


def test_group_score_is_mean_bound_bruteforce():
    """s[g, p] = average over the group's query heads and all (query token, key token) pairs of
    ||q_m,h^p|| ||k_n,g^p||, by a plain loop."""
    wq, wk, wv, xc, _ = _rand_gqa(1, 12, 4, 2, 8, t=7)
    q = (xc @ wq).reshape(7, 4, 8)
    k = (xc @ wk).reshape(7, 2, 8)
    s = oracle.gqa_pair_scores(q, k, 4, 2)
    for g in range(2):
        for p in range(4):
            acc, cnt = 0.0, 0
            for h in (2 * g, 2 * g + 1):  # heads 0, 1 read KV head 0; heads 2, 3 read KV head 1
                for m in range(7):
                    for n in range(7):
                        acc += np.hypot(q[m, h, 2 * p], q[m, h, 2 * p + 1]) * np.hypot(k[n, g, 2 * p], k[n, g, 2 * p + 1])
                        cnt += 1
            assert s[g, p] == pytest.approx(acc / cnt, rel=1e-12)
    assert [oracle.group_of(h, 32, 8) for h in (0, 3, 4, 31)] == [0, 0, 1, 7]


def test_group_selection_exhaustive():
    wq, wk, wv, xc = synth.gqa_layer_weights("gqa_mid")
    out = oracle.convert_gqa_layer(wq, wk, wv, xc, 32, 8, 128, 2, 64)
    s = out["scores"]
    combos = np.array(list(itertools.combinations(range(64), 2)))
    for g in range(8):
        sums = s[g][combos].sum(axis=1)
        assert s[g][out["group_pair_idx"][g]].sum() == pytest.approx(sums.max(), rel=1e-15)


def test_one_head_per_group_is_the_mha_conversion():
    """n_kv = n_heads: the grouped-query conversion is the MHA conversion (same subspaces, same maps)."""
    wq, wk, wv, xc = synth.layer_weights("tiny")
    a = oracle.convert_gqa_layer(wq, wk, wv, xc, 9, 9, 64, 4, 32)
    b = oracle.convert_layer(wq, wk, wv, xc, 9, 64, 4, 32)
    np.testing.assert_array_equal(a["pair_idx"], b["pair_idx"])
    np.testing.assert_array_equal(a["w_krope"], b["w_krope"])
    for key in ("w_uk", "w_uv"):
        pa = np.einsum("dk,hke->hde", a["w_dkv"], a[key])
        pb = np.einsum("dk,hke->hde", b["w_dkv"], b[key])
        assert np.linalg.norm(pa - pb) <= 1e-12 * np.linalg.norm(pb)


def test_heads_of_a_group_share_everything_of_the_group():
    wq, wk, wv, xc = synth.gqa_layer_weights("gqa_mid")
    out = oracle.convert_gqa_layer(wq, wk, wv, xc, 32, 8, 128, 4, 128)
    for h in range(32):
        g = h // 4
        assert list(out["pair_idx"][h]) == list(out["group_pair_idx"][g])
        np.testing.assert_array_equal(out["w_uk"][h], out["group_w_uk"][g])
        np.testing.assert_array_equal(out["w_uv"][h], out["group_w_uv"][g])
        np.testing.assert_array_equal(out["w_krope"][:, 8 * h:8 * h + 8], out["group_w_krope"][:, 8 * g:8 * g + 8])
    # the joint SVD runs over the 8 KV heads' columns only
    assert out["m"].shape == (1024, 8 * (128 - 8) + 8 * 128)


def test_gqa_truncation_is_eckart_young():
    wq, wk, wv, xc = synth.gqa_layer_weights("gqa_mid")
    out = oracle.convert_gqa_layer(wq, wk, wv, xc, 32, 8, 128, 4, 96)
    m = out["m"]
    z = np.concatenate([np.concatenate(list(out["group_w_uk"]), axis=1),
                        np.concatenate(list(out["group_w_uv"]), axis=1)], axis=1)
    ev = np.sort(np.clip(np.linalg.eigvalsh(m.T @ m if m.shape[0] > m.shape[1] else m @ m.T), 0, None))[::-1]
    assert np.sum((m - out["w_dkv"] @ z) ** 2) == pytest.approx(ev[96:].sum(), rel=1e-8)


def _rope_complex(a, kept, d_h, theta=1e4):
    """Rotate the kept subspaces of a [T, H, d_h] at positions 0..T-1, written with complex numbers."""
    t, n, _ = a.shape
    z = a.reshape(t, n, d_h // 2, 2)
    zc = z[..., 0] + 1j * z[..., 1]
    for hh in range(n):
        for p in kept[hh]:
            zc[:, hh, p] *= np.exp(1j * np.arange(t) * theta ** (-2.0 * p / d_h))
    return np.stack([zc.real, zc.imag], axis=-1).reshape(t, n, d_h)


@pytest.mark.parametrize("r", [1, 4])
def test_full_rank_gqa_conversion_is_textbook_gqa(r):
    """At full latent rank the converted layer is grouped-query attention (each query head against its group's
    K and V, repeated) with RoPE on the group's kept subspaces; r = d_h/2 is plain GQA with full RoPE."""
    d, n_h, n_kv, d_h = 10, 4, 2, 8
    wq, wk, wv, xc, x = _rand_gqa(7, d, n_h, n_kv, d_h)
    out = oracle.convert_gqa_layer(wq, wk, wv, xc, n_h, n_kv, d_h, r, d)
    t = x.shape[0]
    c, kr = oracle.append_ref(x, out["w_dkv"], out["w_krope"], out["pair_idx"], np.arange(t), d_h, 1e4)
    q = (x @ wq).reshape(t, n_h, d_h)
    got = oracle.prefill_ref(q, c, kr, out["w_uk"], out["w_uv"], out["pair_idx"], d_h, 1e4)
    kept_g = [list(p) for p in out["group_pair_idx"]]
    kept_h = [kept_g[h // 2] for h in range(n_h)]
    qr = _rope_complex(q, kept_h, d_h)
    kk = _rope_complex((x @ wk).reshape(t, n_kv, d_h), kept_g, d_h)
    vv = (x @ wv).reshape(t, n_kv, d_h)
    rep = [h // 2 for h in range(n_h)]
    tq, tk, tv = (torch.from_numpy(np.ascontiguousarray(a.transpose(1, 0, 2)))[None] for a in (qr, kk[:, rep], vv[:, rep]))
    ref = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, is_causal=True)[0].numpy().transpose(1, 0, 2)
    np.testing.assert_allclose(got, ref, rtol=0, atol=1e-10 * np.abs(ref).max())
    if r == d_h // 2:
        assert all(sorted(p) == list(range(d_h // 2)) for p in kept_g)


@pytest.mark.parametrize("strategy,svd", [("2-norm", "joint"), ("uniform", "split")])
def test_library_gqa_conversion_matches_oracle(strategy, svd):
    wq, wk, wv, xc = synth.gqa_layer_weights("gqa_mid")
    got = convert_layer(wq, wk, wv, xc, 32, 128, 4, 256, strategy=strategy, svd=svd, n_kv_heads=8)
    if strategy == "2-norm" and svd == "joint":
        ref = oracle.convert_gqa_layer(wq, wk, wv, xc, 32, 8, 128, 4, 256)
        np.testing.assert_allclose(got["scores"], ref["scores"], rtol=1e-12)
        np.testing.assert_array_equal(got["pair_idx"], ref["pair_idx"])
        np.testing.assert_array_equal(got["w_krope"], ref["w_krope"])
        np.testing.assert_allclose(got["sigma"][:257], ref["sigma"][:257], rtol=1e-10)
        for key in ("w_uk", "w_uv"):
            a = np.einsum("dk,hke->hde", got["w_dkv"], got[key])
            b = np.einsum("dk,hke->hde", ref["w_dkv"], ref[key])
            assert np.linalg.norm(a - b) <= 1e-10 * np.linalg.norm(b)
    # every variant: group-shared per-head outputs in the layouts of the MHA conversion
    assert got["pair_idx"].shape == (32, 4) and got["w_krope"].shape == (1024, 32 * 8)
    assert got["w_uk"].shape == (32, 256, 120) and got["w_uv"].shape == (32, 256, 128)
    for h in range(32):
        np.testing.assert_array_equal(got["w_uk"][h], got["group_w_uk"][h // 4])
    with pytest.raises(ValueError):
        convert_layer(wq, wk, wv, xc, 32, 128, 4, 256, n_kv_heads=5)


def test_gqa_reference_and_rows_at_full_rank():
    """oracle.ablation.gqa_ref is torch's attention over repeated KV heads (full RoPE); at full latent rank the
    measured end-to-end error of the grouped-query conversion equals its partial-RoPE error."""
    from oracle import ablation

    d, n_h, n_kv, d_h = 10, 4, 2, 8
    wq, wk, wv, xc, x = _rand_gqa(9, d, n_h, n_kv, d_h)
    t = x.shape[0]
    got = ablation.gqa_ref(x, wq, wk, wv, n_h, n_kv, d_h, 1e4)
    every = [list(range(d_h // 2))] * max(n_h, n_kv)
    qr = _rope_complex((x @ wq).reshape(t, n_h, d_h), every, d_h)
    kk = _rope_complex((x @ wk).reshape(t, n_kv, d_h), every, d_h)
    vv = (x @ wv).reshape(t, n_kv, d_h)
    rep = [h // 2 for h in range(n_h)]
    tq, tk, tv = (torch.from_numpy(np.ascontiguousarray(a.transpose(1, 0, 2)))[None] for a in (qr, kk[:, rep], vv[:, rep]))
    ref = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, is_causal=True)[0].numpy().transpose(1, 0, 2)
    np.testing.assert_allclose(got, ref, rtol=0, atol=1e-10 * np.abs(ref).max())
    row = ablation.gqa_rows(wq, wk, wv, xc, x, n_h, n_kv, d_h, 1, d)[0]
    assert row["kv_fit_err"] < 1e-12
    assert row["end_to_end_err"] == pytest.approx(row["partial_rope_err"], rel=1e-8, abs=1e-12)


def test_compact_rope_conversion_and_packing():
    """The converter's compact output keeps the RoPE part per KV head (the oracle's group pairs and key columns),
    and pack_weights forms the same compact device weights from the per-query-head expansion; a layer whose
    query heads of one key head differ is refused."""
    from mla_latent_kv_cache_amd import LayerShape, pack_weights

    wq, wk, wv, xc = synth.gqa_layer_weights("gqa_mid")
    ref = oracle.convert_gqa_layer(wq, wk, wv, xc, 32, 8, 128, 4, 256)
    comp = convert_layer(wq, wk, wv, xc, 32, 128, 4, 256, n_kv_heads=8, compact_rope=True)
    np.testing.assert_array_equal(comp["pair_idx"], ref["group_pair_idx"])
    assert comp["w_krope"].shape == (1024, 8 * 8)
    np.testing.assert_array_equal(comp["w_krope"].reshape(1024, 8, 8), ref["w_krope"].reshape(1024, 32, 8)[:, ::4])
    shape = LayerShape(1024, 32, 128, 4, 256, "f32", rope_heads=8)
    a = pack_weights(shape, comp, rope_len=16, device="cpu")
    b = pack_weights(shape, ref, rope_len=16, device="cpu")
    assert tuple(a.pair_idx.shape) == (8, 4) and tuple(a.w_krope.shape) == (64, 1024)
    assert torch.equal(a.pair_idx, b.pair_idx) and torch.equal(a.w_krope, b.w_krope)
    # 16 key heads (pairs of query heads) from the same expansion
    b16 = pack_weights(LayerShape(1024, 32, 128, 4, 256, "f32", rope_heads=16), ref, rope_len=16, device="cpu")
    assert torch.equal(b16.pair_idx[::2], a.pair_idx)
    bad = dict(ref)
    bad["pair_idx"] = ref["pair_idx"].copy()
    bad["pair_idx"][1] = (bad["pair_idx"][1] + 1) % 64
    with pytest.raises(ValueError):
        pack_weights(shape, bad, rope_len=16, device="cpu")
    with pytest.raises(ValueError):  # per-key-head tables of the wrong count
        pack_weights(LayerShape(1024, 32, 128, 4, 256, "f32", rope_heads=4), comp, rope_len=16, device="cpu")
